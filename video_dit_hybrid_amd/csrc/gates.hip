// Headwise gate projections (ARL2, "Attend Locally, Remember Linearly",
// section 2.1: the forget gate alpha and the step size beta are learned
// per-token projections; the ablations favour one gate per head). Per token t
// of stream b and head h, from the layer input x_t (C channels):
//   a_t = sigmoid(x_t . w_gate[0][h] + b_gate[0][h])
//   g_t = sigmoid(x_t . w_gate[1][h] + b_gate[1][h])
// The state is written once per frame, so frame N gets one forget gate, the
// mean of its tokens' a_t; beta_t = g_t / L.
//
// The projection is a [tokens x C] x [C x 2H] product: on MFMA, with the 2H
// gate rows as the A operand and 32 tokens as the B operand columns, both read
// straight from global memory (C contiguous in both). The pass is bound by the
// HBM read of x (2 bytes per token and channel); the weights (2H x C bf16)
// stay in L2.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {
namespace {

constexpr int GT = 64;  // tokens per work-group

// One work-group (4 waves) per (b, frame, 64-token chunk of the frame). Wave w
// takes the k-steps ks = w, w + 4, ... of the C / 16 for both 32-token column
// blocks, so each gate-weight fragment it loads serves 64 tokens; the four
// partial logit blocks are added through LDS in wave order. Outputs: beta for
// the chunk's tokens, and the chunk's sum of alpha gates per head (apart,
// added up per frame by alpha_kernel).
template <int NOB>
__global__ __launch_bounds__(256) void gates_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wg,
                                                    const float* __restrict__ bg, float* __restrict__ beta,
                                                    float* __restrict__ apart, int T, int C, int H, int L,
                                                    int F, int nch) {
  constexpr int UNR = NOB <= 2 ? 8 : 4;  // k-steps whose loads are issued together
  __shared__ float red[4][NOB][2][16][64];
  __shared__ float sa[16 * NOB][GT];
  const int blk = blockIdx.x;
  const int c = blk % nch, bn = blk / nch;
  const int n = bn % F, b = bn / F;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int O = 2 * H;

  // token rows of the two column blocks; the tail reads the frame's last token
  const uint16_t* xr[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tok = c * GT + 32 * tb + lr;
    xr[tb] = x + ((size_t)b * T + (size_t)n * L + (tok < L ? tok : L - 1)) * C + 8 * hh;
  }
  const uint16_t* wr[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) {
    const int o = 32 * ob + lr;  // rows past 2H repeat the last one; never stored
    wr[ob] = wg + (size_t)(o < O ? o : O - 1) * C + 8 * hh;
  }
  f32x16 acc[NOB][2];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) acc[ob][0] = acc[ob][1] = f32x16{};
  const int nks = C / 16;
  for (int ks0 = w; ks0 < nks; ks0 += 4 * UNR) {
    u32x4 xb[UNR][2], wa[UNR][NOB];
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int ks = ks0 + 4 * i;
      if (ks < nks) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) xb[i][tb] = ld_global_16B(xr[tb] + 16 * ks);
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) wa[i][ob] = ld_global_16B(wr[ob] + 16 * ks);
      } else {
        xb[i][0] = xb[i][1] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) wa[i][ob] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < UNR; ++i)
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[ob][tb] = mfma32x32x16(wa[i][ob], xb[i][tb], acc[ob][tb]);
  }
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[w][ob][tb][r][lane] = acc[ob][tb][r];
  __syncthreads();

  // logit (o, t) sits in register r = 4*(oo/8) + oo%4 of lane t%32 + 32*((oo/4)%2)
  // of block (o / 32, t / 32), oo = o % 32
  for (int idx = tid; idx < O * GT; idx += 256) {
    const int o = idx / GT, t = idx % GT;
    const int ob = o >> 5, oo = o & 31, tb = t >> 5;
    const int r = ((oo >> 3) << 2) | (oo & 3);
    const int ln = (t & 31) + 32 * ((oo >> 2) & 1);
    const float z = red[0][ob][tb][r][ln] + red[1][ob][tb][r][ln] + red[2][ob][tb][r][ln] +
                    red[3][ob][tb][r][ln] + bg[o];
    const float gsig = 1.0f / (1.0f + expf(-z));
    const bool valid = c * GT + t < L;
    if (o >= H) {
      if (valid) beta[((size_t)b * T + (size_t)n * L + c * GT + t) * H + (o - H)] = gsig / (float)L;
    } else {
      sa[o][t] = valid ? gsig : 0.0f;
    }
  }
  __syncthreads();
  for (int h = tid; h < H; h += 256) {
    float s = 0.0f;
#pragma unroll 16
    for (int t = 0; t < GT; ++t) s += sa[h][t];
    apart[((size_t)bn * nch + c) * H + h] = s;
  }
}

// alpha[b, n, h] = (sum of the frame's chunk sums) / L: one wave per (b, n, h),
// lane l adds chunks l, l + 64, ... and a butterfly over the 64 lanes adds
// those (an order fixed by the shape).
__global__ __launch_bounds__(256) void alpha_kernel(const float* __restrict__ apart, float* __restrict__ alpha,
                                                    int nch, int H, int total, int L) {
  const int wv = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wv >= total) return;
  const int bn = wv / H, h = wv % H;
  float s = 0.0f;
  for (int c = lane; c < nch; c += 64) s += apart[((size_t)bn * nch + c) * H + h];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) alpha[wv] = s / (float)L;
}

}  // namespace

int gates_chunks(const Shape& s) { return (s.L + GT - 1) / GT; }

size_t gates_partial_bytes(const Shape& s) {
  return (size_t)s.B * s.F * gates_chunks(s) * s.H * sizeof(float);
}

hipError_t launch_gates(const void* x, const void* wg, const float* bg, float* alpha, float* beta, float* apart,
                        int C, const Shape& s, hipStream_t st) {
  const int nch = gates_chunks(s);
  const int grid = s.B * s.F * nch;
  const int nob = (2 * s.H + 31) / 32;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)wg;
  switch (nob) {
    case 1: gates_kernel<1><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    case 2: gates_kernel<2><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    case 3: gates_kernel<3><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    case 4: gates_kernel<4><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = s.B * s.F * s.H;
  alpha_kernel<<<(total + 3) / 4, 256, 0, st>>>(apart, alpha, nch, s.H, total, s.L);
  return hipGetLastError();
}

}  // namespace ha
