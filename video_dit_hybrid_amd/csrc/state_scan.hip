// Sequential part of the clean-pass state write (ARL2, "Attend Locally,
// Remember Linearly", section 2.1 update rule in affine form, one step per
// frame as section 2.2 prescribes):
//   S_n = alpha_n S_{n-1} - G_n S_{n-1} + B_n,   G_n, B_n from the gram kernels.
// Column j of S_n depends only on column j of S_{n-1}, so a work-group owns a
// column block of one (b, h) state and walks the frames in order.
//
// bf16 path (state_scan_mfma_kernel): the block is 32 columns; compute wave w
// keeps rows [32w, 32w+32) of it in MFMA accumulators (fp32) for the whole
// walk. Per step: S_{n-1} is split into bf16 hi + lo and shared through LDS as
// MFMA B fragments (the accumulator layout already is one, in the contraction
// order the gram kernel writes -G in); the accumulators are set to
// alpha S_{n-1} + B_n; then
// acc += (-G)_hi S_hi + (-G)_hi S_lo + (-G)_lo S_hi on MFMA, which keeps the
// product fp32-accurate (~16 mantissa bits per operand). One more wave per
// work-group copies -G of the frames ahead into LDS (two frames buffered), so
// the compute waves never stall issuing those 64 KB per step.
//
// fp32 path (state_scan_fp32_kernel): the block is 16 columns in LDS and the
// product is plain fp32 FMA, for callers whose inputs are fp32.
#include <type_traits>

#include "ha_device.h"
#include "ha_dma.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

// ---------------------------------------------------------------- bf16 path
constexpr int CWM = 32;   // state columns per work-group

// Waves 0..NRB-1 compute (wave w: rows [32w, 32w+32) of the column block);
// wave NRB only copies -G of the frames ahead into LDS, so the compute waves
// never wait for those loads to issue. Two barriers per frame:
//   E_n: the S_{n-1} fragments and -G_n are in LDS;
//   F_n: the compute waves hold -G_n in registers (its buffer may be refilled).
template <int D>
__global__ __launch_bounds__((D / 32 + 1) * 64) void state_scan_mfma_kernel(
    const unsigned char* __restrict__ ws, const float* __restrict__ alpha, float* __restrict__ state,
    float* __restrict__ snaps, u32x4* __restrict__ sfrag, int H, int F, int n_items) {
  constexpr int NRB = D / 32;                       // 32-row bands (= compute waves)
  constexpr int NCB = D / CWM;
  constexpr int KS = D / 16;                        // k-steps over d_k
  constexpr size_t PER = (size_t)D * D * 8;         // workspace bytes per (b, h, frame)
  constexpr int GB = D * D * 4;                     // -G hi + lo bytes per frame
  constexpr int NSEG = GB / 1024;                   // 1 KB copies per frame
  static_assert(NSEG % 4 == 0, "copies go in groups of four");
  // -G hi and lo fragments of two frames, then the S exchange (hi, lo; two frames)
  __shared__ __align__(16) unsigned char gbuf[2][GB];
  __shared__ __align__(16) u32x4 lds[2][2][KS][64];

  // the column blocks of one (b, h) are consecutive items on one XCD (the
  // grid gives each XCD a multiple of NCB items), so the four work-groups
  // reading the same -G of a frame share that XCD's L2
  const int item = xcd_major_item(gridDim.x);
  if (item >= n_items) return;
  const int cb = item % NCB;
  const int bh = item / NCB;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  // debug bit 1: one work-group per (b, h, column block), a loader wave past
  // the compute waves
  HA_CHECK(cb >= 0 && cb < NCB && h >= 0 && h < H && b >= 0 && wave <= NRB, 1);

  if (wave == NRB) {
    // ---- loader: -G_n of frame n into gbuf[n % 2], lane-linear (fragment order kept)
    const unsigned char* wsb = ws + (size_t)bh * F * PER;
    const uint64_t a = (uint64_t)wsb;
    const u32x4 rs = u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)),
                           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((size_t)F * PER)),
                           (uint32_t)kRsrcWord3};
    const uint32_t lds_g = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(&gbuf[0][0]));
    auto load = [&](int n) {
#pragma unroll 4
      for (int i = 0; i < NSEG; i += 4)
        dma16x4_asm(rs, lds_g + (n & 1) * GB + i * 1024, lane * 16, (uint32_t)((size_t)n * PER) + i * 1024);
    };
    // s_waitcnt immediate for "at most N vector-memory operations outstanding"
    // (vmcnt is 6 bits: N is capped at 63; expcnt and lgkmcnt left at their maxima)
    constexpr int NW_ = NSEG < 63 ? NSEG : 63;
    constexpr int kWaitNewOnly = (NW_ & 0xF) | (0x7 << 4) | (0xF << 8) | (((NW_ >> 4) & 3) << 14);
    load(0);
    if (F > 1) load(1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // -G_0 and -G_1 in LDS
    for (int n = 0; n < F; ++n) {
      lds_barrier();  // E_n
      lds_barrier();  // F_n
      // -G_{n+2} into the buffer -G_n leaves; -G_{n+1} (issued earlier) must
      // have landed before E_{n+1}: wait until only the new copies (or fewer) remain
      if (n + 2 < F) {
        load(n + 2);
        __builtin_amdgcn_s_waitcnt(kWaitNewOnly);
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
    }
    return;
  }

  // ---- compute waves
  const int row0 = wave * 32;
  const int col = cb * CWM + lr;
  f32x16 acc = f32x16{};
  float* sbase = state + (size_t)bh * D * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = sbase[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col];

  // B block and alpha of a frame, two frames ahead (registers)
  f32x4 bv[2][4];
  float al[2] = {0.f, 0.f};
  auto fetch = [&](int slot, int n) {
    const unsigned char* base = ws + ((size_t)bh * F + n) * PER;
    const f32x4* bp = reinterpret_cast<const f32x4*>(base + (size_t)D * D * 4) + ((size_t)(cb * NRB + wave) * 64 + lane) * 4;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) bv[slot][v4] = bp[v4];
    al[slot] = alpha[((size_t)b * F + n) * H + h];
  };
  fetch(0, 0);
  if (F > 1) fetch(1, 1);

  // S_{n-1} -> exchange buffer SL as B fragments (k-steps 2*wave, 2*wave+1 of
  // this band: registers [8s, 8s+8)), plus the snapshots of frame n
  auto publish = [&](auto slot_c, int n) {
    constexpr int SL = decltype(slot_c)::value;
    if (snaps) {
      float* dst = snaps + ((size_t)bh * F + n) * D * D;
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col] = acc[r];
    }
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
      if (sfrag) sfrag[(((size_t)bh * F + n) * NCB + cb) * KS * 64 + (2 * wave + sh) * 64 + lane] = hi;
    }
  };

  auto step = [&](auto slot_c, int n) {
    constexpr int SL = decltype(slot_c)::value;
    HA_CHECK(n >= 0 && n < F && (n & 1) == SL, 2);  // debug bit 2: frame n in buffer n % 2
    lds_barrier();  // E_n
    u32x4 gh[KS], gl[KS];
    const u32x4* gp = reinterpret_cast<const u32x4*>(&gbuf[SL][0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      gh[ks] = gp[(wave * KS + ks) * 64 + lane];
      gl[ks] = gp[(NRB * KS + wave * KS + ks) * 64 + lane];
    }
    lds_barrier();  // F_n (waits for the reads above)
    f32x16 nacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) nacc[r] = fmaf(al[SL], acc[r], bv[SL][r >> 2][r & 3]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 shi = lds[SL][0][ks][lane];
      const u32x4 slo = lds[SL][1][ks][lane];
      nacc = mfma32x32x16(gh[ks], shi, nacc);
      nacc = mfma32x32x16(gh[ks], slo, nacc);
      nacc = mfma32x32x16(gl[ks], shi, nacc);
    }
    if (n + 2 < F) fetch(SL, n + 2);
    acc = nacc;
    if (n + 1 < F) publish(std::integral_constant<int, SL ^ 1>{}, n + 1);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  publish(S0{}, 0);
  int n = 0;
  for (; n + 1 < F; n += 2) {
    step(S0{}, n);
    step(S1{}, n + 1);
  }
  if (n < F) step(S0{}, n);
#pragma unroll
  for (int r = 0; r < 16; ++r) sbase[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col] = acc[r];
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

HA_DEBUG_READER(debug_take_scan)

hipError_t launch_state_scan_bf16(const void* ws, const float* alpha, float* state, float* snapshots,
                                  void* sfrag, const Shape& s, hipStream_t st) {
  const int ncb = s.d / CWM;
  const int items = s.B * s.H * ncb;
  const int per_xcd = (items + 8 * ncb - 1) / (8 * ncb) * ncb;  // whole (b, h) units per XCD
  const int grid = 8 * per_xcd;
  HA_LOG("launch state_scan_mfma_kernel<%d>: grid %d x %d threads (%d (b, h, column block) items, %d per XCD; %d "
         "frames in sequence; snapshots %s)", s.d, grid, (s.d / 32 + 1) * 64, items, per_xcd, s.F,
         sfrag ? "as bf16 readout fragments" : snapshots ? "fp32" : "none");
  if (s.d == 128)
    state_scan_mfma_kernel<128><<<grid, (128 / 32 + 1) * 64, 0, st>>>(
        (const unsigned char*)ws, alpha, state, snapshots, (u32x4*)sfrag, s.H, s.F, items);
  else
    state_scan_mfma_kernel<64><<<grid, (64 / 32 + 1) * 64, 0, st>>>(
        (const unsigned char*)ws, alpha, state, snapshots, (u32x4*)sfrag, s.H, s.F, items);
  return hipGetLastError();
}

hipError_t launch_state_scan_fp32(const float* gram, const float* alpha, float* state, float* snapshots,
                                  const Shape& s, hipStream_t st) {
  const int groups = s.B * s.H * (s.d / CW);
  HA_LOG("launch state_scan_fp32_kernel<%d>: grid %d x %d threads (%d frames in sequence)", s.d, groups, NT, s.F);
  if (s.d == 128)
    state_scan_fp32_kernel<128><<<groups, NT, 0, st>>>(gram, alpha, state, snapshots, s.H, s.F);
  else
    state_scan_fp32_kernel<64><<<groups, NT, 0, st>>>(gram, alpha, state, snapshots, s.H, s.F);
  return hipGetLastError();
}

}  // namespace ha
