// Sequential part of the clean-pass state write (ARL2, "Attend Locally,
// Remember Linearly", section 2.1 update rule in affine form, one step per
// frame as section 2.2 prescribes):
//   S_n = alpha_n S_{n-1} - G_n S_{n-1} + B_n,   G_n, B_n from the gram kernels.
// Column j of S_n depends only on column j of S_{n-1}, so a work-group owns a
// column block of one (b, h) state and walks the frames in order.
//
// bf16 path (state_scan_mfma_kernel): the block is 32 columns; wave w keeps
// rows [32w, 32w+32) of it in MFMA accumulators (fp32) for the whole walk.
// Per step: S_{n-1} is split into bf16 hi + lo and shared through LDS as MFMA
// B fragments (the accumulator layout already is one, in the contraction order
// the gram kernel writes -G in); the accumulators are set to
// alpha S_{n-1} + B_n; then
// acc += (-G)_hi S_hi + (-G)_hi S_lo + (-G)_lo S_hi on MFMA, which keeps the
// product fp32-accurate (~16 mantissa bits per operand). The operands of step
// n+2 (G rows, B block, alpha) are loaded while step n computes.
//
// fp32 path (state_scan_fp32_kernel): the block is 16 columns in LDS and the
// product is plain fp32 FMA, for callers whose inputs are fp32.
#include <type_traits>

#include "ha_device.h"
#include "ha_launch.h"

namespace ha {
namespace {

// ---------------------------------------------------------------- bf16 path
constexpr int CWM = 32;   // state columns per work-group
constexpr int NTM = 256;  // 4 waves, one 32-row block each (D = 128); D = 64 uses 2 waves

template <int D>
__global__ __launch_bounds__(NTM) void state_scan_mfma_kernel(const unsigned char* __restrict__ ws,
                                                              const float* __restrict__ alpha,
                                                              float* __restrict__ state,
                                                              float* __restrict__ snaps,
                                                              u32x4* __restrict__ sfrag, int H,
                                                              int F) {
  constexpr int NRB = D / 32;                       // 32-row bands (= waves in use)
  constexpr int NCB = D / CWM;
  constexpr int KS = D / 16;                        // k-steps over d_k
  constexpr size_t PER = (size_t)D * D * 8;         // workspace bytes per (b, h, frame)
  // S operand fragments [k-step][lane] 16 bytes, hi and lo planes, double buffered
  __shared__ __align__(16) u32x4 lds[2][2][KS][64];

  const int cb = blockIdx.x % NCB;
  const int bh = blockIdx.x / NCB;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const bool active = wave < NRB;
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

  // operands of one step (-G hi and lo A fragments of this band, the B block,
  // alpha) in a two-slot ring: step n's operands are requested two steps
  // earlier. Each request is one contiguous 1 KB per wave (fragment order).
  u32x4 gh[2][KS], gl[2][KS];
  f32x4 bv[2][4];
  float al[2] = {0.f, 0.f};
  auto fetch = [&](int slot, int n) {
    const unsigned char* base = ws + ((size_t)bh * F + n) * PER;
    const u32x4* ghp = reinterpret_cast<const u32x4*>(base) + (size_t)wave * KS * 64 + lane;
    const u32x4* glp = reinterpret_cast<const u32x4*>(base + (size_t)D * D * 2) + (size_t)wave * KS * 64 + lane;
    const f32x4* bp = reinterpret_cast<const f32x4*>(base + (size_t)D * D * 4) + ((size_t)(cb * NRB + wave) * 64 + lane) * 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      gh[slot][ks] = ghp[ks * 64];
      gl[slot][ks] = glp[ks * 64];
    }
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) bv[slot][v4] = bp[v4];
    al[slot] = alpha[((size_t)b * F + n) * H + h];
  };
  if (active) {
    fetch(0, 0);
    if (F > 1) fetch(1, 1);
  }

  // one frame; slot == n % 2 (also the LDS buffer), fixed at compile time
  auto step = [&](auto slot_c, int n) {
    constexpr int SL = decltype(slot_c)::value;
    if (active) {
      if (snaps) {  // S_{n-1}, the state frame n's readout reads
        float* dst = snaps + ((size_t)bh * F + n) * D * D;
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col] = acc[r];
      }
      // this band's rows of S_{n-1} are the B fragments of k-steps 2*wave, 2*wave+1
      // (same contraction order as the -G fragments): registers [8s, 8s+8)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        u32x4 hi, lo;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float x0 = acc[8 * sh + 2 * w2], x1 = acc[8 * sh + 2 * w2 + 1];
          const uint32_t hp = pack_bf16x2(x0, x1);
          hi[w2] = hp;
          lo[w2] = pack_bf16x2(x0 - bf16_lo_to_f32(hp), x1 - bf16_hi_to_f32(hp));
        }
        lds[SL][0][2 * wave + sh][lane] = hi;
        lds[SL][1][2 * wave + sh][lane] = lo;
        // bf16(S_{n-1}) for the readout: the same fragment, one 16-byte store
        if (sfrag) sfrag[(((size_t)bh * F + n) * NCB + cb) * KS * 64 + (2 * wave + sh) * 64 + lane] = hi;
      }
    }
    lds_barrier();
    if (active) {
      f32x16 nacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) nacc[r] = fmaf(al[SL], acc[r], bv[SL][r >> 2][r & 3]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 shi = lds[SL][0][ks][lane];
        const u32x4 slo = lds[SL][1][ks][lane];
        nacc = mfma32x32x16(gh[SL][ks], shi, nacc);
        nacc = mfma32x32x16(gh[SL][ks], slo, nacc);
        nacc = mfma32x32x16(gl[SL][ks], shi, nacc);
      }
      if (n + 2 < F) fetch(SL, n + 2);
      acc = nacc;
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int n = 0;
  for (; n + 1 < F; n += 2) {
    step(S0{}, n);
    step(S1{}, n + 1);
  }
  if (n < F) step(S0{}, n);
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
                                  void* sfrag, const Shape& s, hipStream_t st) {
  const int groups = s.B * s.H * (s.d / CWM);
  if (s.d == 128)
    state_scan_mfma_kernel<128><<<groups, NTM, 0, st>>>((const unsigned char*)ws, alpha, state,
                                                        snapshots, (u32x4*)sfrag, s.H, s.F);
  else
    state_scan_mfma_kernel<64><<<groups, NTM, 0, st>>>((const unsigned char*)ws, alpha, state,
                                                       snapshots, (u32x4*)sfrag, s.H, s.F);
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
