// Sequential part of the clean-pass state write (ARL2, "Attend Locally,
// Remember Linearly", section 2.1 update rule in affine form, one step per
// frame as section 2.2 prescribes):
//   S_n = alpha_n S_{n-1} - G_n S_{n-1} + B_n,   G_n, B_n from the gram kernels.
// Column j of S_n depends only on column j of S_{n-1}, so a work-group owns a
// column block of one (b, h) state and walks the frames in order.
//
// bf16 path (state_scan_mfma_kernel): the block is 32 columns; wave w keeps
// rows [32w, 32w+32) of it in MFMA accumulators (fp32) for the whole walk.
// Per step: S_{n-1} is split into bf16 hi + lo and written transposed to LDS;
// the accumulators are set to alpha S_{n-1} + B_n; then
// acc += (-G)_hi S_hi + (-G)_hi S_lo + (-G)_lo S_hi on MFMA, which keeps the
// product fp32-accurate (~16 mantissa bits per operand). The operands of step
// n+1 (G rows, B block, alpha) are loaded while step n computes.
//
// fp32 path (state_scan_fp32_kernel): the block is 16 columns in LDS and the
// product is plain fp32 FMA, for callers whose inputs are fp32.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {
namespace {

// ---------------------------------------------------------------- bf16 path
constexpr int CWM = 32;   // state columns per work-group
constexpr int NTM = 256;  // 4 waves, one 32-row block each (D = 128); D = 64 uses 2 waves

__device__ __forceinline__ int sw8(int i) { return (i & 7) ^ ((i >> 3) & 1); }

template <int D>
__global__ __launch_bounds__(NTM) void state_scan_mfma_kernel(const unsigned char* __restrict__ ws,
                                                              const float* __restrict__ alpha,
                                                              float* __restrict__ state,
                                                              float* __restrict__ snaps, int H,
                                                              int F) {
  constexpr int NCB = D / CWM;
  constexpr int KS = D / 16;                        // k-steps over d_k
  constexpr size_t PER = (size_t)D * D * 8;         // workspace bytes per (b, h, frame)
  constexpr int SROW = D * 2;                       // bytes of one S^T row (D bf16)
  // S^T[j][k] hi and lo planes, double buffered: 2 * 2 * CWM * D * 2 bytes
  __shared__ __align__(16) unsigned char lds[2][2][CWM * SROW];

  const int cb = blockIdx.x % NCB;
  const int bh = blockIdx.x / NCB;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const bool active = wave < D / 32;
  const int row0 = wave * 32;
  const int col = cb * CWM + lr;

  // running state block in the 32x32 MFMA accumulator layout:
  // acc[r] = S[row0 + 8*(r/4) + 4*hh + r%4][col]
  f32x16 acc = f32x16{};
  float* sbase = state + (size_t)bh * D * D;
  if (active) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = sbase[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col];
  }

  // operands of one step: rows row0.. of -G (hi, lo) as A fragments, B block, alpha
  u32x4 gh[KS], gl[KS];
  float bv[16];
  float al = 0.f;
  auto fetch = [&](int n) {
    const unsigned char* base = ws + ((size_t)bh * F + n) * PER;
    const uint16_t* ghp = reinterpret_cast<const uint16_t*>(base);
    const uint16_t* glp = ghp + (size_t)D * D;
    const float* bp = reinterpret_cast<const float*>(base + (size_t)D * D * 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const size_t off = (size_t)(row0 + lr) * D + ks * 16 + hh * 8;
      gh[ks] = ld_global_16B(ghp + off);
      gl[ks] = ld_global_16B(glp + off);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) bv[r] = bp[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col];
    al = alpha[((size_t)b * F + n) * H + h];
  };
  if (active) fetch(0);

  for (int n = 0; n < F; ++n) {
    const int buf = n & 1;
    if (active) {
      // S_{n-1}: snapshot out, and hi/lo split into S^T in LDS
      if (snaps) {
        float* dst = snaps + ((size_t)bh * F + n) * D * D;
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col] = acc[r];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int k0 = row0 + 8 * g + 4 * hh;  // four consecutive rows of S = four k of S^T
        const uint32_t h01 = pack_bf16x2(acc[4 * g], acc[4 * g + 1]);
        const uint32_t h23 = pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3]);
        const uint32_t l01 = pack_bf16x2(acc[4 * g] - bf16_lo_to_f32(h01), acc[4 * g + 1] - bf16_hi_to_f32(h01));
        const uint32_t l23 = pack_bf16x2(acc[4 * g + 2] - bf16_lo_to_f32(h23), acc[4 * g + 3] - bf16_hi_to_f32(h23));
        const int off = lr * SROW + (((k0 >> 3) ^ sw8(lr)) << 4) + (k0 & 7) * 2;
        *reinterpret_cast<u32x2*>(&lds[buf][0][off]) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(&lds[buf][1][off]) = u32x2{l01, l23};
      }
    }
    __syncthreads();
    if (active) {
      f32x16 nacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) nacc[r] = fmaf(al, acc[r], bv[r]);
      u32x4 cgh[KS], cgl[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) { cgh[ks] = gh[ks]; cgl[ks] = gl[ks]; }
      if (n + 1 < F) fetch(n + 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kc = 2 * ks + hh;
        const int off = lr * SROW + ((kc ^ sw8(lr)) << 4);
        const u32x4 shi = *reinterpret_cast<const u32x4*>(&lds[buf][0][off]);
        const u32x4 slo = *reinterpret_cast<const u32x4*>(&lds[buf][1][off]);
        nacc = mfma32x32x16(cgh[ks], shi, nacc);
        nacc = mfma32x32x16(cgh[ks], slo, nacc);
        nacc = mfma32x32x16(cgl[ks], shi, nacc);
      }
      acc = nacc;
    }
  }
  if (active) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sbase[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col] = acc[r];
  }
}

// ---------------------------------------------------------------- fp32 path
constexpr int CW = 16;   // state columns per work-group
constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT) void state_scan_fp32_kernel(const float* __restrict__ gram,
                                                             const float* __restrict__ alpha,
                                                             float* __restrict__ state,
                                                             float* __restrict__ snaps, int H, int F) {
  constexpr int NCB = D / CW;
  constexpr int TPR = NT / D;    // threads per state row
  constexpr int CPT = CW / TPR;  // columns per thread
  __shared__ float sb[D][CW];

  const int cb = blockIdx.x % NCB;
  const int bh = blockIdx.x / NCB;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x;
  const int i = tid / TPR, jc = (tid % TPR) * CPT;
  const long long sbase = (long long)bh * D * D + cb * CW + jc;
  float* srow = state + sbase + (long long)i * D;

#pragma unroll
  for (int c = 0; c < CPT; ++c) sb[i][jc + c] = srow[c];
  __syncthreads();

  for (int n = 0; n < F; ++n) {
    if (snaps) {
      float* dst = snaps + ((long long)bh * F + n) * D * D + cb * CW + jc + (long long)i * D;
#pragma unroll
      for (int c = 0; c < CPT; ++c) dst[c] = sb[i][jc + c];
    }
    const float* G = gram + ((long long)bh * F + n) * (long long)D * 2 * D + (long long)i * 2 * D;
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
#pragma unroll 4
    for (int kk = 0; kk < D; kk += 4) {
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(G + kk);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = fmaf(g4[u], sb[kk + u][jc + c], acc[c]);
    }
    const float a = alpha[((long long)b * F + n) * H + h];
    float nb[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) nb[c] = G[D + cb * CW + jc + c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) sb[i][jc + c] = fmaf(a, sb[i][jc + c], nb[c] - acc[c]);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) srow[c] = sb[i][jc + c];
}

}  // namespace

hipError_t launch_state_scan_bf16(const void* ws, const float* alpha, float* state, float* snapshots,
                                  const Shape& s, hipStream_t st) {
  const int groups = s.B * s.H * (s.d / CWM);
  if (s.d == 128)
    state_scan_mfma_kernel<128><<<groups, NTM, 0, st>>>((const unsigned char*)ws, alpha, state,
                                                        snapshots, s.H, s.F);
  else
    state_scan_mfma_kernel<64><<<groups, NTM, 0, st>>>((const unsigned char*)ws, alpha, state,
                                                       snapshots, s.H, s.F);
  return hipGetLastError();
}

hipError_t launch_state_scan_fp32(const float* gram, const float* alpha, float* state, float* snapshots,
                                  const Shape& s, hipStream_t st) {
  const int groups = s.B * s.H * (s.d / CW);
  if (s.d == 128)
    state_scan_fp32_kernel<128><<<groups, NT, 0, st>>>(gram, alpha, state, snapshots, s.H, s.F);
  else
    state_scan_fp32_kernel<64><<<groups, NT, 0, st>>>(gram, alpha, state, snapshots, s.H, s.F);
  return hipGetLastError();
}

}  // namespace ha
