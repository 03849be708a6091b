// fp32-operand variants of the layer's kernels, for callers whose q..v' are
// float32 (small shapes and validation runs; the bf16 path is the fast one).
// Same mathematics as the bf16 path (ARL2, "Attend Locally, Remember
// Linearly", section 2.1 intra-frame branch, readout and update rule; section
// 2.2 frame-level access), computed with fp32 FMA and expf.
#include "ha_device.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

constexpr int QB = 64;   // queries per work-group (two threads per query)
constexpr int KB = 32;   // keys per LDS tile
constexpr int NT_A = 2 * QB;

// Each query is owned by a thread pair; each thread of the pair holds half of
// the d coordinates of q and of the output accumulator.
template <int D>
__global__ __launch_bounds__(NT_A) void attn_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ qp, const float* __restrict__ states, long long stride_bh,
    long long stride_frame, float* __restrict__ out, int H, int T, int L, int F, int qtiles,
    float scale) {
  constexpr int HD = D / 2;
  __shared__ __align__(16) float ks_[KB][D];
  __shared__ __align__(16) float vs_[KB][D];

  const int item = blockIdx.x;
  const int qt = item % qtiles;
  const int hf = item / qtiles;
  const int h = hf % H;
  const int n = (hf / H) % F;
  const int b = hf / (H * F);
  const int tid = threadIdx.x;
  const int qi = tid >> 1, part = tid & 1;
  const int my_q = qt * QB + qi;
  const bool valid = my_q < L;
  const long long rs = (long long)H * D;
  const long long fbase = ((long long)b * T + (long long)n * L) * rs + (long long)h * D;
  const int c0 = part * HD;

  float qr[HD], o[HD];
#pragma unroll
  for (int c = 0; c < HD; ++c) {
    qr[c] = valid ? q[fbase + my_q * rs + c0 + c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int key0 = 0; key0 < L; key0 += KB) {
    __syncthreads();
    for (int e = tid; e < KB * D / 4; e += NT_A) {
      const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
      const int key = key0 + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < L) {
        kv = *reinterpret_cast<const f32x4*>(k + fbase + key * rs + c4);
        vv = *reinterpret_cast<const f32x4*>(v + fbase + key * rs + c4);
      }
      *reinterpret_cast<f32x4*>(&ks_[row][c4]) = kv;
      *reinterpret_cast<f32x4*>(&vs_[row][c4]) = vv;
    }
    __syncthreads();
    const int nk = min(KB, L - key0);
    for (int kk = 0; kk < nk; ++kk) {
      float pd = 0.f;
#pragma unroll
      for (int c = 0; c < HD; ++c) pd = fmaf(qr[c], ks_[kk][c0 + c], pd);
      const float s = (pd + __shfl_xor(pd, 1)) * scale;
      const float mn = fmaxf(m, s);
      const float corr = expf(m - mn);
      const float p = expf(s - mn);
      l = fmaf(l, corr, p);
#pragma unroll
      for (int c = 0; c < HD; ++c) o[c] = fmaf(o[c], corr, p * vs_[kk][c0 + c]);
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = 1.f / l;
  const float* Sp = states + (long long)(b * H + h) * stride_bh + (long long)n * stride_frame;
  const float* qpr = qp + fbase + my_q * rs;
#pragma unroll
  for (int c = 0; c < HD; ++c) o[c] *= inv;
  for (int dk = 0; dk < D; ++dk) {
    const float a = qpr[dk];
#pragma unroll
    for (int c = 0; c < HD; ++c) o[c] = fmaf(a, Sp[dk * D + c0 + c], o[c]);
  }
  float* orow = out + fbase + my_q * rs + c0;
#pragma unroll
  for (int c = 0; c < HD; ++c) orow[c] = o[c];
}

constexpr int TCF = 32;   // tokens per LDS chunk
constexpr int NT_G = 256;

// [G | B] = K'^T diag(beta) [K' | V'] for one (b, h, frame, half), fp32 FMA.
template <int D>
__global__ __launch_bounds__(NT_G) void gram_fp32_kernel(const float* __restrict__ kp,
                                                         const float* __restrict__ vp,
                                                         const float* __restrict__ beta,
                                                         float* __restrict__ gram, int H, int T,
                                                         int L, int F) {
  constexpr int TPR = NT_G / D;   // threads per output row
  constexpr int OPT = D / TPR;    // outputs per thread
  __shared__ __align__(16) float as_[TCF][D];
  __shared__ __align__(16) float bs_[TCF][D];

  const int half = blockIdx.x & 1;
  const int hf = blockIdx.x >> 1;
  const int h = hf % H;
  const int n = (hf / H) % F;
  const int b = hf / (H * F);
  const int tid = threadIdx.x;
  const int i = tid / TPR, j0 = (tid % TPR) * OPT;
  const long long rs = (long long)H * D;
  const long long fbase = ((long long)b * T + (long long)n * L) * rs + (long long)h * D;
  const float* bbase = beta + ((long long)b * T + (long long)n * L) * H + h;
  const float* src = half ? vp : kp;

  float acc[OPT];
#pragma unroll
  for (int c = 0; c < OPT; ++c) acc[c] = 0.f;
  for (int t0 = 0; t0 < L; t0 += TCF) {
    __syncthreads();
    for (int e = tid; e < TCF * D; e += NT_G) {
      const int row = e / D, c = e % D;
      const int t = t0 + row;
      float a = 0.f, bv = 0.f;
      if (t < L) {
        a = bbase[(long long)t * H] * kp[fbase + t * rs + c];
        bv = src[fbase + t * rs + c];
      }
      as_[row][c] = a;
      bs_[row][c] = bv;
    }
    __syncthreads();
    for (int tt = 0; tt < TCF; ++tt) {
      const float a = as_[tt][i];
#pragma unroll
      for (int c = 0; c < OPT; ++c) acc[c] = fmaf(a, bs_[tt][j0 + c], acc[c]);
    }
  }
  float* g = gram + ((long long)(b * H + h) * F + n) * (long long)D * 2 * D + (long long)i * 2 * D +
             half * D + j0;
#pragma unroll
  for (int c = 0; c < OPT; ++c) g[c] = acc[c];
}

}  // namespace

hipError_t launch_attn_fp32(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            void* out, const Shape& s, float scale, hipStream_t st) {
  const int qtiles = (s.L + QB - 1) / QB;
  const long long items = (long long)s.B * s.H * s.F * qtiles;
  HA_LOG("launch attn_fp32_kernel<%d>: grid %lld x %d threads (query tiles of %d)", s.d, items, NT_A, QB);
  auto go = [&](auto kern) {
    kern<<<(int)items, NT_A, 0, st>>>((const float*)q, (const float*)k, (const float*)v,
                                      (const float*)qp, states, stride_bh, stride_frame,
                                      (float*)out, s.H, s.T, s.L, s.F, qtiles, scale);
  };
  if (s.d == 128) go(attn_fp32_kernel<128>);
  else go(attn_fp32_kernel<64>);
  return hipGetLastError();
}

hipError_t launch_gram_fp32(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st) {
  const long long groups = (long long)s.B * s.H * s.F * 2;
  HA_LOG("launch gram_fp32_kernel<%d>: grid %lld x %d threads", s.d, groups, NT_G);
  if (s.d == 128)
    gram_fp32_kernel<128><<<(int)groups, NT_G, 0, st>>>((const float*)kp, (const float*)vp, beta,
                                                        gram, s.H, s.T, s.L, s.F);
  else
    gram_fp32_kernel<64><<<(int)groups, NT_G, 0, st>>>((const float*)kp, (const float*)vp, beta,
                                                       gram, s.H, s.T, s.L, s.F);
  return hipGetLastError();
}

}  // namespace ha
