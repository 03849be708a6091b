// Intra-frame bidirectional softmax attention with the fused inter-frame
// readout, bf16 operands on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Computes, per stream b, head h and frame n (ARL2, "Attend Locally, Remember
// Linearly", section 2.1 item 1 and the readout O_inter = Q'_N S_{N-1}; section
// 2.2 frame-level access: all tokens of a frame read the same state):
//   out[rows of frame n] = softmax(Q K^T * s) V + Q' S_n
// where the softmax runs over the keys of frame n only.
//
// Work decomposition: one work-group (4 waves, 256 threads) owns 128 queries
// of one (b, h, frame); each wave owns 32 queries. Key and value tiles of 64
// keys are copied global -> LDS by buffer loads that write LDS directly
// (no VGPR staging), two tiles in flight, and shared by the 4 waves. Rows past
// the end of the frame are outside the buffer descriptor's range and arrive as
// zeros, so no load is predicated.
//
// Orientation: a wave computes S^T = K Q^T (keys x queries) so that every lane
// holds 16 scores of ONE query (column l%32) per 32x32 block. Row max and row
// sum are in-lane reductions plus one permlane32 swap, and the output
// accumulator O^T (dv x queries) of a lane also belongs to one query, so the
// softmax rescale is a per-lane scalar.
//
// Key permutation: MFMA row i of the S^T block reads physical key pi(i), pi
// swapping bits 2 and 3 of i. Then lane half hh holds the eight CONSECUTIVE
// keys 16*(r/8) + 8*hh + r%8 in accumulator elements r, which is exactly the
// B-operand layout of O^T += V^T P^T, so P feeds the next MFMA from registers.
// V stays row-major in LDS; its A operand (8 consecutive keys of one dv column
// per lane) comes from two ds_read_b64_tr_b16, which hand each lane of a
// 16-lane group one column of a 4 x 16 block that the group reads row-wise.
//
// Per key tile: S^T = K Q^T (16 MFMAs), online softmax on the VALU, then
// O^T += V^T P^T (16 MFMAs); the next tile's K and V are already in flight to
// the other LDS buffer. Inside each MFMA phase the LDS operand of MFMA i+4 is
// read while MFMA i issues, so LDS latency is hidden within the wave; two waves
// per SIMD (two work-groups per CU) overlap one wave's softmax with the other's
// MFMA phases.
// Online softmax in the exp2 domain with the scale folded into one FMA; the
// running max only moves when a tile's max exceeds it by more than 8 (log2
// units), so exp2 arguments stay <= 8 and accumulator rescales are rare. The
// result does not depend on that choice: a reference point common to the
// numerator and the denominator cancels.
//
// Loader wave (LOADER): when the launch has at most one work-group per CU
// (one frame of few heads), a work-group runs alone and its waves would stall
// issuing their share of each step's 32 KB of tile copies (the address unit
// takes 64 bytes per clock). A fifth wave then issues every copy and the four
// compute waves only compute; the step barrier still orders the buffers.
//
// Short last query tile: when a work-group's query tile holds at most 32
// queries (1560 = 12 x 128 + 24), waves 0 and 1 both take them, each with one
// 32-key half of every key tile, and merge their (max, sum, O) through LDS
// before the readout, instead of one wave walking all keys while three idle.
//
// Fused scan (FUSED, forward calls over several frames): the first
// work-groups of the launch run the clean pass's state scan (scan_role below)
// and publish S_{n-1} of every frame as readout fragments; an attention
// work-group of frame n waits at its readout until all column blocks of its
// frame's state are published, so the scan runs beside the attention instead
// of before it.
//
// KV mode (the softmax teacher with a full KV cache that the hybrid layer
// replaces, ARL2 section 1): the same kernel with frame n's queries attending
// to the keys [0, kv_off + (n+1) L) of a key/value cache, no readout. The keys
// of one (b, h, frame) may be split over nsplit work-groups, each writing its
// unnormalised fp32 output and (max, sum) for a merge pass. Work units
// (b, h, frame, split) go round-robin over the 8 XCDs, heaviest (latest)
// frames first, and a unit's query tiles stay on one XCD so they share its L2.
#include <type_traits>

#include "ha_device.h"
#include "ha_dma.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

constexpr int KT = 64;          // keys per LDS tile
constexpr int QPW = 32;         // queries per wave
constexpr int NW = 4;           // waves per work-group
constexpr int QPB = QPW * NW;   // queries per work-group
constexpr int NT = NW * kWave;  // threads per work-group
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct Cfg {
  static constexpr int NCH = D / 8;          // 16-byte chunks in a row of D bf16
  static constexpr int TILE = KT * D * 2;    // bytes of one K or V tile
  static constexpr int SMEM = 4 * TILE;      // K[2] then V[2]; also holds S (D*D*2)
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps over d
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int NLD = TILE / 1024 / NW;  // 1 KB direct-to-LDS loads per wave per tile
  static_assert(SMEM >= D * D * 2, "S must fit in the tile buffers");
  static_assert(NLD >= 1, "tile too small for the load split");
};

__device__ __forceinline__ int pi32(int i) {  // swap bits 2 and 3
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// K tile [KT][D]: 32 lanes read one 16-byte chunk column of rows pi(0..31);
// the XOR puts 16 consecutive lanes on 16 distinct chunk slots.
template <int NCH>
__device__ __forceinline__ int k_swz(int row) {
  const int i = pi32(row & 31);
  if constexpr (NCH >= 16) return i & 15;
  else return (i & 7) ^ ((i >> 3) & 1);
}
// V tile [KT][D] and S [D][D] are read with ds_read_tr16 (see tr_swz).
template <int NCH>
__device__ __forceinline__ int v_swz(int row) { return tr_swz<NCH>(row); }

// Scheduling groups for the preceding code of the same basic block (mask: 0x8
// MFMA, 0x100 LDS read, 0x402 VALU incl. transcendental): PF*R reads first,
// then per MFMA R reads (while reads remain) and V VALU instructions, so the
// MFMA pipe, the LDS and the VALU work of one wave interleave.
template <int N, int PF, int R, int V>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, PF * R, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    if (V > 0) __builtin_amdgcn_sched_group_barrier(0x402, V, 0);
  }
}

constexpr int kDevice = 16;              // cache policy: sc1 (device scope)
constexpr int kSpinLimit = 1 << 22;      // polls of a frame counter (a guard: it cannot run out)

// The clean pass's state scan as work-group (bh, cb) of the fused launch:
// column block cb of the state of (stream, head) bh walks the frames in order,
// S_n = alpha_n S_{n-1} + (-G_n) S_{n-1} + B_n with the increments ws of the
// gram kernel, on MFMA with -G and S split into bf16 hi + lo (the product of
// state_scan_mfma_kernel, the same operations in the same order, so the same
// result). Wave w < d/32 keeps rows [32w, 32w+32) of the block in its
// accumulator and loads its band's -G fragments of the next frame into
// registers; the S exchange goes through LDS. Each S_{n-1} is stored as the
// readout fragments of frame n with device-scope stores; after the next
// barrier (each wave's stores acknowledged before it) one lane adds one to
// flags[bh*F + n]. The last state goes to state (fp32).
// FM (the layer with per-head feature maps, Q' = Q W_q): the readout
// fragments of frame n are those of M_n = W_q S_{n-1} instead (the readout
// then contracts Q with M_n): wave w computes row band w of M_n[:, cb] from
// the S exchange in LDS and its band of W_q (bf16 A fragments held in
// registers, in the exchange's contraction order), and the counter of frame
// n is raised at the step after, once those fragments are stored.
template <int D, bool FM = false>
__device__ __forceinline__ void scan_role(const unsigned char* __restrict__ ws, const float* __restrict__ alpha,
                                          float* __restrict__ state, unsigned char* __restrict__ sfrag,
                                          unsigned* __restrict__ flags, int bh, int cb, int H, int F,
                                          unsigned char* smem, int wave, int lane,
                                          const uint16_t* __restrict__ wq = nullptr) {
  constexpr int NRB = D / 32, NCB = D / 32, KS = D / 16;
  constexpr size_t PER = (size_t)D * D * 8;  // increment bytes per (b, h, frame)
  u32x4(*lds)[2][KS][64] = reinterpret_cast<u32x4(*)[2][KS][64]>(smem);  // [slot][hi, lo][k-step][lane]
  static_assert(2 * 2 * KS * 64 * 16 <= 4 * KT * D * 2, "the exchange must fit in the tile buffers");
  const bool comp = wave < NRB;
  const int w = comp ? wave : 0;
  const int lr = lane & 31, hh = lane >> 5;
  const int row0 = w * 32, col = cb * 32 + lr;
  const int b = bh / H, h = bh % H;
  f32x16 acc = f32x16{};
  float* sbase = state + (size_t)bh * D * D;
  if (comp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = sbase[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col];
  }
  // FM: row band w of W_q (head h) as A fragments: k-slot 8*hh + e of k-step
  // ks holds column 16*ks + 8*(e/4) + 4*hh + e%4
  u32x4 wqa[FM ? KS : 1];
  if constexpr (FM) {
    const uint16_t* W = wq + (size_t)h * D * D + (size_t)(row0 + lr) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(W + 16 * ks + 4 * hh);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(W + 16 * ks + 8 + 4 * hh);
      wqa[ks] = u32x4{a0[0], a0[1], a1[0], a1[1]};
    }
  }
  u32x4 gh[KS], gl[KS];
  f32x4 bv[2][4];
  float al[2] = {0.f, 0.f};
  auto fetch_g = [&](int n) {
    const u32x4* gp = reinterpret_cast<const u32x4*>(ws + ((size_t)bh * F + n) * PER);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      gh[ks] = gp[(w * KS + ks) * 64 + lane];
      gl[ks] = gp[(NRB * KS + w * KS + ks) * 64 + lane];
    }
  };
  auto fetch_b = [&](int slot, int n) {
    const unsigned char* base = ws + ((size_t)bh * F + n) * PER;
    const f32x4* bp = reinterpret_cast<const f32x4*>(base + (size_t)D * D * 4) + ((size_t)(cb * NRB + w) * 64 + lane) * 4;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) bv[slot][v4] = bp[v4];
    al[slot] = alpha[((size_t)b * F + n) * H + h];
  };
  const __amdgpu_buffer_rsrc_t rsf = make_rsrc(sfrag + (size_t)bh * F * D * D * 2, F * D * D * 2);
  // S_{n-1} (acc) -> exchange slot SL as B fragments (k-steps 2w, 2w+1: registers
  // [8s, 8s+8)) and, its hi part, the readout fragments of frame n
  auto publish = [&](auto slot_c, int n) {
    constexpr int SL = decltype(slot_c)::value;
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
      lds[SL][0][2 * w + sh][lane] = hi;
      lds[SL][1][2 * w + sh][lane] = lo;
      if constexpr (!FM)
        __builtin_amdgcn_raw_buffer_store_b128(hi, rsf, (uint32_t)((((n * NCB + cb) * KS) + 2 * w + sh) * 64 + lane) * 16,
                                               0, kDevice);
    }
  };
  if (comp) {
    fetch_g(0);
    fetch_b(0, 0);
    if (F > 1) fetch_b(1, 1);
    publish(std::integral_constant<int, 0>{}, 0);
  }
  auto step = [&](auto slot_c, int n) {
    constexpr int SL = decltype(slot_c)::value;
    // every wave's fragments of frame n are stored (acknowledged) and its S
    // exchange is in LDS
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (FM) {  // M_{n-1}'s fragments, computed in the step before, are stored
      if (n > 0 && wave == 0 && lane == 0)
        __hip_atomic_fetch_add(flags + (size_t)bh * F + n - 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (wave == 0 && lane == 0) __hip_atomic_fetch_add(flags + (size_t)bh * F + n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (comp) {
      if constexpr (FM) {  // M_n = W_q S_{n-1}, row band w, from the exchange
        f32x16 m = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          m = mfma32x32x16(wqa[ks], lds[SL][0][ks][lane], m);
          m = mfma32x32x16(wqa[ks], lds[SL][1][ks][lane], m);
        }
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          u32x4 hi;
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) hi[w2] = pack_bf16x2(m[8 * sh + 2 * w2], m[8 * sh + 2 * w2 + 1]);
          __builtin_amdgcn_raw_buffer_store_b128(hi, rsf, (uint32_t)((((n * NCB + cb) * KS) + 2 * w + sh) * 64 + lane) * 16,
                                                 0, kDevice);
        }
      }
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
      if (n + 1 < F) fetch_g(n + 1);
      if (n + 2 < F) fetch_b(SL, n + 2);
      acc = nacc;
      if (n + 1 < F) publish(std::integral_constant<int, SL ^ 1>{}, n + 1);
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
  if constexpr (FM) {  // the last frame's M fragments are stored
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (wave == 0 && lane == 0)
      __hip_atomic_fetch_add(flags + (size_t)bh * F + F - 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (comp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sbase[(size_t)(row0 + 8 * (r >> 2) + 4 * hh + (r & 3)) * D + col] = acc[r];
  }
}

template <int P_, bool NEXT_, bool TAIL_, bool LOADK_>
struct StepFlags {
  static constexpr int P = P_;
  static constexpr bool NEXT = NEXT_, TAIL = TAIL_, LOADK = LOADK_;
};

template <int D, bool KV, bool MIX = false, bool LOADER = false, bool FUSED = false>
__global__ __launch_bounds__(LOADER ? NT + kWave : NT, LOADER ? 1 : 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ qp,
    const float* __restrict__ states, long long stride_bh, long long stride_frame,
    const unsigned char* __restrict__ sfrag, uint16_t* __restrict__ out, int H, int T, int L, int F,
    int qtiles, int n_items, float c2 /* softmax scale * log2(e) */,
    int Tk, int kv_off, int nsplit, float* __restrict__ part_o, float2* __restrict__ part_ml,
    const float* __restrict__ add_o, const float* __restrict__ mix, const unsigned char* __restrict__ gws,
    const float* __restrict__ alpha, float* __restrict__ state, unsigned* __restrict__ flags, int n_scan,
    const uint16_t* __restrict__ wq) {
  using C = Cfg<D>;
  constexpr int NCH = C::NCH;
  __shared__ __align__(16) unsigned char smem[C::SMEM];
  unsigned char* const kbuf = smem;                 // two K tiles
  unsigned char* const vbuf = smem + 2 * C::TILE;   // two V tiles

  int qt, h, n, b, sp = 0;
  if constexpr (KV) {
    // unit rank r = (m * 8 + xcd); units ordered latest frame first
    const int g = blockIdx.x, m = (g >> 3) / qtiles;
    qt = (g >> 3) % qtiles;
    const int r = m * 8 + (g & 7);
    if (r >= n_items) return;
    sp = r % nsplit;
    const int r2 = r / nsplit;
    const int BH = n_items / (F * nsplit);  // n_items = B * H * F * nsplit units
    const int bh = r2 % BH;
    n = F - 1 - r2 / BH;
    b = bh / H;
    h = bh % H;
  } else {
    int item;
    if constexpr (FUSED) {
      const int g = blockIdx.x;
      if (g < n_scan) {
        // the scan's work-groups come first (they hold CU slots before any
        // attention work-group can wait for them), XCD-major with the column
        // blocks of one (b, h) on one XCD
        constexpr int NCB = D / 32;
        const int si = (g & 7) * (n_scan >> 3) + (g >> 3);
        if (si >= n_items / (F * qtiles) * NCB) return;
        // with per-head feature maps (wq) the readout fragments are those of W_q S
        const int sw = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), sl = (int)threadIdx.x & 63;
        if (wq)
          scan_role<D, true>(gws, alpha, state, const_cast<unsigned char*>(sfrag), flags, si / NCB, si % NCB, H, F, smem,
                             sw, sl, wq);
        else
          scan_role<D>(gws, alpha, state, const_cast<unsigned char*>(sfrag), flags, si / NCB, si % NCB, H, F, smem, sw, sl);
        return;
      }
      const int ga = g - n_scan;
      item = (ga & 7) * ((int)(gridDim.x - n_scan) >> 3) + (ga >> 3);
    } else {
      item = xcd_major_item(gridDim.x);
    }
    if (item >= n_items) return;
    qt = item % qtiles;
    const int hf = item / qtiles;
    h = hf % H;
    n = (hf / H) % F;
    b = hf / (H * F);
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int lr = lane & 31, hh = lane >> 5;
  static_assert(!(KV && LOADER), "the loader wave serves the readout kernel only");
  static_assert(!FUSED || (!KV && !LOADER && !MIX), "the fused scan serves the plain forward call only");
  const bool is_loader = LOADER && wave == NW;
  // debug bit 1: the work item decodes to a valid (b, h, frame, query tile, split)
  HA_CHECK(qt >= 0 && qt < qtiles && h >= 0 && h < H && n >= 0 && n < F && b >= 0 && sp >= 0 && sp < nsplit, 1);
  const uint32_t rsb = (uint32_t)H * D * 2;  // bytes between consecutive tokens
  const long long fbase = ((long long)b * T + (long long)n * L) * ((long long)H * D) + (long long)h * D;
  // bytes of this (b, h, frame) slab as one buffer: tokens >= L read as zero
  const int span = (int)((uint32_t)(L - 1) * rsb + D * 2);
  const u32x4 rk = rsrc_words(k + fbase, span);
  const u32x4 rv = rsrc_words(v + fbase, span);
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(smem));
  // KV mode: visible keys [0, nkeys) of the cache, this split's tiles
  // [t0, t0 + ntiles); each tile gets its own descriptor (32-bit offsets stay
  // inside one tile however long the cache)
  int nkeys = L, t0 = 0;
  long long kvbase = 0;
  if constexpr (KV) {
    // kv_off < 0: a one-frame window, keys [n L, (n+1) L) (intra-frame only)
    nkeys = kv_off < 0 ? L : kv_off + (n + 1) * L;
    const int nt_all = (nkeys + KT - 1) / KT;
    t0 = (int)((long long)sp * nt_all / nsplit);
    const int t1 = (int)((long long)(sp + 1) * nt_all / nsplit);
    kvbase = ((long long)b * Tk + (kv_off < 0 ? (long long)n * L : 0)) * ((long long)H * D) + (long long)h * D;
    nkeys = (t1 == nt_all ? nkeys : t1 * KT) - t0 * KT;  // keys of this split
  }
  auto tile_rsrc = [&](const uint16_t* base, int j) {
    const int rows = nkeys - j * KT < KT ? nkeys - j * KT : KT;
    return rsrc_words(base + kvbase + (long long)(t0 + j) * KT * H * D, (int)((uint32_t)(rows - 1) * rsb + D * 2));
  };

  // a frame's last query tile holding at most one wave's queries (1560 =
  // 12 x 128 + 24): waves 0 and 1 both take its queries, each with one 32-key
  // half of every key tile (tsplit below), instead of one wave with all keys
  const bool tsplit = !KV && L - qt * QPB <= QPW;
  const int q0 = qt * QPB + ((is_loader || tsplit) ? 0 : wave) * QPW;
  bool wave_active = !is_loader && (tsplit ? wave < 2 : q0 < L);
  const int my_q = q0 + lr;

  // ---- direct-to-LDS tile loads. Load i of wave w fills the 1 KB LDS segment
  // seg = i*NW + w of the tile (lane l: 16-byte slot seg*64 + l), i.e. rows
  // 16*i*(NCH/16)... of the tile. Segments of one wave are 16 rows apart for
  // D = 128 (8 rows apart for D = 64), which leaves both swizzles unchanged,
  // so the per-lane byte offset of load i is the offset of load 0 plus a
  // uniform step.
  constexpr int ROWS_PER_SEG = 64 / NCH;
  constexpr int SEG_ROW_STEP = NW * ROWS_PER_SEG;  // rows between a wave's segments
  static_assert(SEG_ROW_STEP % 8 == 0 || NCH < 16, "segment step must keep the swizzle");
  // the load sets a wave issues: its own (set w = wave), or with a loader
  // wave all NW sets, from the loader
  constexpr int NSETS = LOADER ? NW : 1;
  uint32_t koff[NSETS], voff[NSETS];
#pragma unroll
  for (int s2 = 0; s2 < NSETS; ++s2) {
    const int row = (LOADER ? s2 : wave) * ROWS_PER_SEG + lane / NCH, pc = lane % NCH;
    koff[s2] = row * rsb + ((pc ^ k_swz<NCH>(row)) << 4);
    voff[s2] = row * rsb + ((pc ^ v_swz<NCH>(row)) << 4);
  }
  // The copies are inline asm: the compiler cannot tell which LDS bytes a
  // builtin copy writes and would wait for every copy in flight before each
  // later LDS read; with these, a tile's copies stay in flight until the wait
  // at the end of the step.
  auto issue_k = [&](int j, int buf) {
    if (LOADER && !is_loader) return;
    const uint32_t toff = KV ? 0u : (uint32_t)j * KT * rsb;
    const u32x4 r = KV ? tile_rsrc(k, j) : rk;
#pragma unroll
    for (int i = 0; i < C::NLD; ++i)
#pragma unroll
      for (int s2 = 0; s2 < NSETS; ++s2)
        dma16_asm(r, lds0 + buf * C::TILE + (i * NW + (LOADER ? s2 : wave)) * 1024, koff[s2],
                  toff + i * SEG_ROW_STEP * rsb);
  };
  auto issue_v = [&](int j, int buf) {
    if (LOADER && !is_loader) return;
    const uint32_t toff = KV ? 0u : (uint32_t)j * KT * rsb;
    const u32x4 r = KV ? tile_rsrc(v, j) : rv;
#pragma unroll
    for (int i = 0; i < C::NLD; ++i)
#pragma unroll
      for (int s2 = 0; s2 < NSETS; ++s2)
        dma16_asm(r, lds0 + 2 * C::TILE + buf * C::TILE + (i * NW + (LOADER ? s2 : wave)) * 1024, voff[s2],
                  toff + i * SEG_ROW_STEP * rsb);
  };

  // ---- per-lane LDS read offsets
  // K (A operand of S^T = K Q^T): row kb*32 + pi(lr), chunk 2*ks + hh, stored at
  // chunk (2*ks + hh) ^ sw; as 2*ks + hh == 2*ks ^ hh that byte offset is
  // kaddr ^ (ks << 5) with one per-lane base.
  const int krow = pi32(lr);
  const int kaddr = krow * (D * 2) + ((hh ^ k_swz<NCH>(krow)) << 4);
  // V / S (A operand through transposed reads): a 16-lane group g = lane/16 reads
  // rows rb + 8*hh + (i/4) (+4 for the second read), columns 16*(g%2) + 4*(i%4)
  const int gi = lane & 15, g = lane >> 4;
  const int vrow = 8 * hh + (gi >> 2);
  const int vsw = v_swz<NCH>(vrow);
  const int vcol = 16 * (g & 1) + 4 * (gi & 3);  // + 32*db
  auto v_off = [&](int row_add, int db) {  // row_add multiple of 4 and of no bit-3 effect on the swizzle
    const int col = vcol + 32 * db;
    return (vrow + row_add) * (D * 2) + (((col >> 3) ^ vsw) << 4) + (col & 7) * 2;
  };

  u32x4 qf[C::KSTEPS];
  {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + fbase), 0, span, kRsrcWord3);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] = buf_load16(rq, my_q * rsb + (ks * 16 + hh * 8) * 2);
  }

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l0 = 0.f, l1 = 0.f;

  const int ntiles = (nkeys + KT - 1) / KT;
  const int last_valid = nkeys - (ntiles - 1) * KT;  // keys in the last tile
  // debug bit 2: a non-empty key range; bit 4: the last LDS operand reads of a
  // tile (K rows through ds_read_b128, V^T through transposed reads) stay
  // inside the tile
  HA_CHECK(nkeys > 0 && t0 >= 0 && last_valid >= 1 && last_valid <= KT, 2);
  HA_CHECK((kaddr ^ ((C::KSTEPS - 1) << 5)) + 32 * D * 2 + 16 <= C::TILE &&
               v_off(32 + 16 + 4, C::DB - 1) + 8 <= C::TILE,
           4);

  // S^T for one tile (two 32-key blocks) from K buffer kb_. MFMA i uses the K
  // operand (ks, kb) = (i/2, i%2); operands are read PF MFMAs ahead.
  constexpr int PF = 4;
  auto qk = [&](const unsigned char* kb_, f32x16& s0, f32x16& s1) {
    constexpr int N = 2 * C::KSTEPS;
    auto kload = [&](int i) {
      return *reinterpret_cast<const u32x4*>(kb_ + (kaddr ^ ((i >> 1) << 5)) + (i & 1) * 32 * D * 2);
    };
    u32x4 ring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ring[i] = kload(i);
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const u32x4 a = ring[i % PF];
      if (i + PF < N) ring[i % PF] = kload(i + PF);
      if (i & 1) s1 = mfma32x32x16(a, qf[i >> 1], s1);
      else s0 = mfma32x32x16(a, qf[i >> 1], s0);
    }
  };

  // Rare paths below hold an empty volatile asm: it cannot be speculated, so
  // the compiler keeps a real (uniform) branch instead of executing the path
  // on every tile with selects.
  auto mask_tail = [&](f32x16& s0, f32x16& s1) {
    asm volatile("");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 16 * (r >> 3) + 8 * hh + (r & 7);
      if (key >= last_valid) s0[r] = -INFINITY;
      if (key + 32 >= last_valid) s1[r] = -INFINITY;
    }
  };
  auto tile_max = [&](const f32x16& s0, const f32x16& s1) {
    float m = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, fmaxf(s0[r], s1[r]));
    return max_across_halves(m) * c2;
  };
  auto rescale = [&](float mt) {
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
      asm volatile("");
      const float mn = fmaxf(m_run, mt);
      const float f = __builtin_amdgcn_exp2f(m_run - mn);
      l0 *= f;
      l1 *= f;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) o[db] *= f;
      m_run = mn;
    }
  };
  auto softmax_p = [&](const f32x16& s0, const f32x16& s1, uint32_t* p0, uint32_t* p1) {
    const float nm = -m_run;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float x0 = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, nm));
      const float x1 = __builtin_amdgcn_exp2f(fmaf(s0[r + 1], c2, nm));
      const float y0 = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, nm));
      const float y1 = __builtin_amdgcn_exp2f(fmaf(s1[r + 1], c2, nm));
      a0 += x0; a1 += x1; a2 += y0; a3 += y1;
      p0[r >> 1] = pack_bf16x2(x0, x1);
      p1[r >> 1] = pack_bf16x2(y0, y1);
    }
    l0 += a0 + a1;
    l1 += a2 + a3;
  };
  // O^T += V^T P^T. MFMA i: 16-key step ks = i/DB (block ks/2, half ks%2) and
  // dv block db = i%DB; its V operand (two transposed reads) is read PF ahead.
  auto pv = [&](const unsigned char* vb_, const uint32_t* p0, const uint32_t* p1) {
    constexpr int N = 4 * C::DB;
    auto vload = [&](int i) {
      const int ks = i / C::DB, db = i % C::DB;
      const int ra = 32 * (ks >> 1) + 16 * (ks & 1);
      const u32x2 x0 = ds_read_tr16(vb_ + v_off(ra, db));
      const u32x2 x1 = ds_read_tr16(vb_ + v_off(ra + 4, db));
      return u32x4{x0[0], x0[1], x1[0], x1[1]};
    };
    u32x4 ring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ring[i] = vload(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ks = i / C::DB, db = i % C::DB;
      const u32x4 a = ring[i % PF];
      if (i + PF < N) ring[i % PF] = vload(i + PF);
      const uint32_t* p = (ks >> 1) ? p1 : p0;
      const int hb = 4 * (ks & 1);
      o[db] = mfma32x32x16(a, u32x4{p[hb], p[hb + 1], p[hb + 2], p[hb + 3]}, o[db]);
    }
  };

  // FUSED: the frame's counter, first read during the last key tile
  unsigned fl_seen = 0;
  if (tsplit) {
    // ---- the short last query tile: waves 0 and 1 take key half `wave` of
    // every tile (one tile of K and V in flight, copied by the same waves as
    // in the main loop); their (max, sum, O) are merged into wave 0 at the end
    auto qk1 = [&](const unsigned char* kb_, f32x16& s) {
      s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
        s = mfma32x32x16(*reinterpret_cast<const u32x4*>(kb_ + (kaddr ^ (ks << 5)) + wave * 32 * D * 2), qf[ks], s);
    };
    auto pv1 = [&](const unsigned char* vb_, const uint32_t* p) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int ra = 32 * wave + 16 * h2;
          const u32x2 x0 = ds_read_tr16(vb_ + v_off(ra, db));
          const u32x2 x1 = ds_read_tr16(vb_ + v_off(ra + 4, db));
          o[db] = mfma32x32x16(u32x4{x0[0], x0[1], x1[0], x1[1]},
                               u32x4{p[4 * h2], p[4 * h2 + 1], p[4 * h2 + 2], p[4 * h2 + 3]}, o[db]);
        }
    };
    issue_k(0, 0);
    issue_v(0, 0);
    for (int t = 0; t < ntiles; ++t) {
      const int pb = t & 1;
      // tile t has landed and every wave is done with tile t-1's buffers
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 1 < ntiles) {
        issue_k(t + 1, pb ^ 1);
        issue_v(t + 1, pb ^ 1);
      }
      if constexpr (FUSED) {
        if (t + 1 == ntiles && wave == 0 && lane == 0)
          fl_seen = __hip_atomic_load(flags + ((size_t)(b * H + h) * F + n), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const int valid = t + 1 == ntiles ? last_valid : KT;  // keys of this tile
      if (wave_active && 32 * wave < valid) {  // this half holds at least one key
        f32x16 s1;
        qk1(kbuf + pb * C::TILE, s1);
        if (valid < 32 * wave + 32) {
          asm volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * wave + 16 * (r >> 3) + 8 * hh + (r & 7) >= valid) s1[r] = -INFINITY;
        }
        float mt = s1[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s1[r]);
        rescale(max_across_halves(mt) * c2);
        uint32_t p1[8];
        const float nm = -m_run;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, nm));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(s1[r + 1], c2, nm));
          a0 += x0;
          a1 += x1;
          p1[r >> 1] = pack_bf16x2(x0, x1);
        }
        l0 += a0 + a1;
        pv1(vbuf + pb * C::TILE, p1);
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();  // every wave is done with the last tile
    asm volatile("" ::: "memory");
    // wave 1's (O, sum, max) through the V buffers, lane-major
    float* mrg = reinterpret_cast<float*>(vbuf);
    static_assert((C::DB * 16 + 2) * 64 * 4 <= 2 * C::TILE, "the merge must fit in the V buffers");
    if (wave == 1) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mrg[(db * 16 + r) * 64 + lane] = o[db][r];
      mrg[C::DB * 16 * 64 + lane] = l0;
      mrg[(C::DB * 16 + 1) * 64 + lane] = m_run;
    }
    __syncthreads();
    if (wave == 0) {
      const float l_1 = mrg[C::DB * 16 * 64 + lane], m_1 = mrg[(C::DB * 16 + 1) * 64 + lane];
      const float mn = fmaxf(m_run, m_1);  // wave 0's half always holds a key: finite
      const float f0 = __builtin_amdgcn_exp2f(m_run - mn), f1 = __builtin_amdgcn_exp2f(m_1 - mn);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = fmaf(o[db][r], f0, mrg[(db * 16 + r) * 64 + lane] * f1);
      l0 = fmaf(l0, f0, l_1 * f1);
      m_run = mn;
    }
    wave_active = wave_active && wave == 0;
  } else {
    // ---- prologue: K_0, V_0, K_1 in flight, then S_0
    issue_k(0, 0);
    issue_v(0, 0);
    if (ntiles > 1) issue_k(1, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sa0, sa1, sb0, sb1;
    float mt_a = 0.f, mt_b = 0.f;
    if (wave_active) {
      qk(kbuf, sa0, sa1);
      if (ntiles == 1 && last_valid < KT) mask_tail(sa0, sa1);
      mt_a = tile_max(sa0, sa1);
    }
    __syncthreads();  // every wave has read K_0 before step 0 refills its buffer with K_2

    // Step j (K runs one tile ahead of V): prefetch K_{j+2} and V_{j+1}; then
    //   [S_{j+1} = K_{j+1} Q^T on MFMA]  beside  [P_j = exp2(S_j - m) on the VALU]
    //   [O += V_j^T P_j^T on MFMA]       beside  [max of S_{j+1}]
    // The flags are compile-time so that the steady-state loop has no branch
    // between the two regions: P = j % 2 (LDS buffers), NEXT = tile j+1 exists,
    // TAIL = tile j+1 may be the ragged last tile, LOADK = tile j+2 exists.
    auto step = [&](auto flags, int j, f32x16& c0, f32x16& c1, float& mt_c, f32x16& n0, f32x16& n1,
                    float& mt_n) {
      using Fl = decltype(flags);
      constexpr int P = Fl::P;
      // debug bit 2: the tiles this step copies exist
      HA_CHECK((!Fl::LOADK || j + 2 < ntiles) && (!Fl::NEXT || j + 1 < ntiles), 2);
      if constexpr (Fl::LOADK) issue_k(j + 2, P);
      else if (j + 2 < ntiles) issue_k(j + 2, P);
      if constexpr (Fl::NEXT) issue_v(j + 1, P ^ 1);
      if (wave_active) {
        rescale(mt_c);
        uint32_t p0[8], p1[8];
        if constexpr (Fl::NEXT) {
          qk(kbuf + (P ^ 1) * C::TILE, n0, n1);
          softmax_p(c0, c1, p0, p1);
          interleave<2 * C::KSTEPS, PF, 1, 7>();
          if constexpr (Fl::TAIL) {
            if (j + 2 == ntiles && last_valid < KT) mask_tail(n0, n1);
          }
          pv(vbuf + P * C::TILE, p0, p1);
          mt_n = tile_max(n0, n1);
          interleave<4 * C::DB, PF, 2, 2>();
        } else {
          softmax_p(c0, c1, p0, p1);
          pv(vbuf + P * C::TILE, p0, p1);
        }
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // flags: <P, NEXT, TAIL, LOADK>
    using Main0 = StepFlags<0, true, false, true>;
    using Main1 = StepFlags<1, true, false, true>;

    int j = 0;
    for (; j + 3 < ntiles; j += 2) {
      step(Main0{}, j, sa0, sa1, mt_a, sb0, sb1, mt_b);
      step(Main1{}, j + 1, sb0, sb1, mt_b, sa0, sa1, mt_a);
    }
    // Remaining 1 to 3 tiles, without the software pipeline (one score tile
    // live): S_t is in sa, V_t in buffer t % 2, K_{t+1} in buffer (t+1) % 2.
    // FUSED: the frame's counter (below) is first read during the last tile,
    // so that the device-scope load's latency hides behind the tile's work
    for (int t = j; t < ntiles; ++t) {
      const int pb = t & 1;
      if constexpr (FUSED) {
        if (t + 1 == ntiles && wave == 0 && lane == 0)
          fl_seen = __hip_atomic_load(flags + ((size_t)(b * H + h) * F + n), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (t + 1 < ntiles) issue_v(t + 1, pb ^ 1);
      if (t + 2 < ntiles) issue_k(t + 2, pb);
      if (wave_active) {
        rescale(mt_a);
        uint32_t p0[8], p1[8];
        softmax_p(sa0, sa1, p0, p1);
        pv(vbuf + pb * C::TILE, p0, p1);
        if (t + 1 < ntiles) {
          qk(kbuf + (pb ^ 1) * C::TILE, sa0, sa1);
          if (t + 2 == ntiles && last_valid < KT) mask_tail(sa0, sa1);
          mt_a = tile_max(sa0, sa1);
        }
      }
      asm volatile("" ::: "memory");
      if constexpr (FUSED) {
        // the last tile copies nothing: wait for LDS only, the counter load may stay in flight
        if (t + 1 == ntiles) __builtin_amdgcn_s_waitcnt(0xC07F);
        else __builtin_amdgcn_s_waitcnt(0);
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }

  }

  if constexpr (KV) {  // ---- epilogue without readout
    const float lsum = sum_across_halves(l0 + l1);
    if (!wave_active || my_q >= L) return;
    if (nsplit > 1) {  // unnormalised partial output and (max, sum) of this split
      const size_t row = (((size_t)sp * (n_items / (H * F * nsplit)) + b) * T + (size_t)n * L + my_q) * H + h;
      float* po = part_o + row * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
          *reinterpret_cast<f32x4*>(po + db * 32 + 8 * gg + 4 * hh) =
              f32x4{o[db][4 * gg], o[db][4 * gg + 1], o[db][4 * gg + 2], o[db][4 * gg + 3]};
      if (hh == 0) part_ml[row] = float2{m_run, lsum};
      return;
    }
    const float inv = 1.f / lsum;
    uint16_t* op = out + fbase + (long long)my_q * H * D;
    const float* ap = add_o ? add_o + fbase + (long long)my_q * H * D : nullptr;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int dv = db * 32 + 8 * gg + 4 * hh;
        f32x4 y = f32x4{o[db][4 * gg] * inv, o[db][4 * gg + 1] * inv, o[db][4 * gg + 2] * inv,
                        o[db][4 * gg + 3] * inv};
        if (ap) y += *reinterpret_cast<const f32x4*>(ap + dv);  // the token-level inter-frame output
        st_global_8B(op + dv, u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])});
      }
    }
    return;
  } else {
  // The readout Q'S goes into rd: o itself (the plain sum O/l + Q'S), or, with
  // per-branch weights (MIX: mix[b, h] = (w_softmax, w_inter)), a separate
  // accumulator, added as w_softmax O/l + w_inter Q'S.
  f32x16 racc[MIX ? C::DB : 1];
  f32x16* const rd = MIX ? racc : o;
  float w_inter = 1.f;
  auto mix_scale = [&](f32x16* oo, float l) {
    float f = 1.f / l;
    if constexpr (MIX) {
      const float2 w = reinterpret_cast<const float2*>(mix)[b * H + h];
      f *= w.x;
      w_inter = w.y;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) racc[db] = f32x16{};
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oo[db] *= f;
  };
  auto mix_add = [&](f32x16* oo) {
    if constexpr (MIX) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oo[db][r] = fmaf(w_inter, racc[db][r], oo[db][r]);
    }
  };
  // ---- epilogue: O = O / l + Q' S_n. S_n reaches LDS either as the bf16
  // readout fragments the state scan wrote (copied as they are), or from the
  // fp32 row-major state, converted here to bf16 [dk][dv].
  const __amdgpu_buffer_rsrc_t rqp = __builtin_amdgcn_make_buffer_rsrc((void*)(qp + fbase), 0, span, kRsrcWord3);
  if (sfrag) {
    constexpr int NSEG = D * D * 2 / 1024;  // 1 KB fragments
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(sfrag + (size_t)(b * H + h) * stride_bh + (size_t)n * stride_frame, D * D * 2);
    if constexpr (FUSED) {
      // the frame's state: all column blocks published by the scan work-groups
      if (wave == 0 && lane == 0) {
        const unsigned* fl = flags + ((size_t)(b * H + h) * F + n);
        unsigned seen = fl_seen;
        int it = 0;
        while (seen < (unsigned)(D / 32) && ++it < kSpinLimit) {
          __builtin_amdgcn_s_sleep(2);
          seen = __hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        HA_CHECK(it < kSpinLimit, 16);  // debug bit 16: a frame counter never completed
      }
      __syncthreads();
    }
    if (!is_loader) {
#pragma unroll
      for (int i = wave; i < NSEG; i += NW) dma16_to_lds<FUSED ? kDevice : 0>(rs, smem + i * 1024, lane * 16, i * 1024);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (!wave_active) return;
    mix_scale(o, sum_across_halves(l0 + l1));
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      // contraction slot 8*hh + e holds dk = 16*ks + 8*(e/4) + 4*hh + e%4
      const u32x2 q0v = buf_load8(rqp, my_q * rsb + (ks * 16 + 4 * hh) * 2);
      const u32x2 q1v = buf_load8(rqp, my_q * rsb + (ks * 16 + 8 + 4 * hh) * 2);
      const u32x4 bq = u32x4{q0v[0], q0v[1], q1v[0], q1v[1]};
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(smem + (db * C::KSTEPS + ks) * 1024 + lane * 16);
        rd[db] = mfma32x32x16(a, bq, rd[db]);
      }
    }
    mix_add(o);
  } else {
    // all of a thread's loads are issued before the first conversion, so
    // their latencies overlap instead of adding up
    const float* Sp = states + (long long)(b * H + h) * stride_bh + (long long)n * stride_frame;
    constexpr int NPER = D * D / 4 / NT;  // 16-byte pieces of S per thread
    static_assert(NPER * NT * 4 == D * D, "S must split evenly over the threads");
    if (!is_loader) {  // the NT threads of the compute waves
      f32x4 sx[NPER];
#pragma unroll
      for (int i = 0; i < NPER; ++i) sx[i] = *reinterpret_cast<const f32x4*>(Sp + (tid + i * NT) * 4);
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const int p = tid + i * NT;
        const int dk = p / (D / 4), dv0 = (p % (D / 4)) * 4;
        const int off = dk * (D * 2) + (((dv0 >> 3) ^ v_swz<NCH>(dk)) << 4) + (dv0 & 7) * 2;
        *reinterpret_cast<u32x2*>(smem + off) = u32x2{pack_bf16x2(sx[i][0], sx[i][1]), pack_bf16x2(sx[i][2], sx[i][3])};
      }
    }
    __syncthreads();
    if (!wave_active) return;
    mix_scale(o, sum_across_halves(l0 + l1));
    // same contraction order as the fragment path (slot 8*hh + e <-> dk =
    // 16*ks + 8*(e/4) + 4*hh + e%4), so both paths give identical results:
    // the two transposed reads take rows 16*ks + 4*hh + i/4 and those + 8
    const int srow = 4 * hh + (gi >> 2);
    auto s_off = [&](int row, int db) {
      const int col = vcol + 32 * db;
      return row * (D * 2) + (((col >> 3) ^ v_swz<NCH>(row)) << 4) + (col & 7) * 2;
    };
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const u32x2 q0v = buf_load8(rqp, my_q * rsb + (ks * 16 + 4 * hh) * 2);
      const u32x2 q1v = buf_load8(rqp, my_q * rsb + (ks * 16 + 8 + 4 * hh) * 2);
      const u32x4 bq = u32x4{q0v[0], q0v[1], q1v[0], q1v[1]};
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x2 x0 = ds_read_tr16(smem + s_off(16 * ks + srow, db));
        const u32x2 x1 = ds_read_tr16(smem + s_off(16 * ks + 8 + srow, db));
        rd[db] = mfma32x32x16(u32x4{x0[0], x0[1], x1[0], x1[1]}, bq, rd[db]);
      }
    }
    mix_add(o);
  }
  if (my_q < L) {
    uint16_t* op = out + fbase + (long long)my_q * H * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int dv = db * 32 + 8 * gg + 4 * hh;
        st_global_8B(op + dv, u32x2{pack_bf16x2(o[db][4 * gg], o[db][4 * gg + 1]),
                                    pack_bf16x2(o[db][4 * gg + 2], o[db][4 * gg + 3])});
      }
    }
  }
  }
}

// Merge of the key splits: per (b, token, h) row, m = max_s m_s and
// out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s, splits in order.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         uint16_t* __restrict__ out, long long rows,
                                                         int nsplit) {
  constexpr int TPR = D / 8;  // threads per row, 8 outputs each
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / TPR;
  if (row >= rows) return;
  const int c0 = (int)(t % TPR) * 8;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_ml[s * rows + row].x);
  float den = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float2 ml = part_ml[s * rows + row];
    const float wgt = __builtin_amdgcn_exp2f(ml.x - m);
    den = fmaf(wgt, ml.y, den);
    const f32x4* po = reinterpret_cast<const f32x4*>(part_o + (s * rows + row) * D + c0);
    const f32x4 a = po[0], b = po[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(wgt, a[e], acc[e]);
      acc[4 + e] = fmaf(wgt, b[e], acc[4 + e]);
    }
  }
  const float inv = 1.f / den;
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<u32x4*>(out + row * D + c0) = r;
}

// Copy of the call's K, V rows into the cache at token offset `at` of each
// stream (16 bytes per thread).
__global__ __launch_bounds__(256) void kv_append_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                        u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                        long long per_b, long long cap_b, long long at,
                                                        long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long long b = i / per_b, r = i % per_b;
  kc[b * cap_b + at + r] = k[i];
  vc[b * cap_b + at + r] = v[i];
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            const void* sfrag, void* out, const Shape& s, float scale,
                            hipStream_t st, const float* mix) {
  const int qtiles = (s.L + QPB - 1) / QPB;
  const long long items = (long long)s.B * s.H * s.F * qtiles;
  const int grid = (int)((items + 7) / 8 * 8);
  const float c2 = scale * kLog2e;
  // at most one work-group per CU: a loader wave issues the tile copies
  const bool loader = items <= kAttnLoaderMaxGroups;
  const int nt = loader ? NT + kWave : NT;
  HA_LOG("launch attn_bf16_kernel<%d>: grid %d x %d threads (%lld items = %d streams x %d heads x %d frames x %d "
         "query tiles of %d; key tiles of %d, %d KiB LDS; readout from %s%s%s)",
         s.d, grid, nt, items, s.B, s.H, s.F, qtiles, QPB, KT, (s.d == 128 ? Cfg<128>::SMEM : Cfg<64>::SMEM) >> 10,
         sfrag ? "bf16 fragments" : "fp32 states", mix ? "; per-branch weights" : "",
         loader ? "; a loader wave issues the tile copies" : "");
  auto args = [&](auto kern) {
    kern<<<grid, nt, 0, st>>>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                              (const uint16_t*)qp, states, stride_bh, stride_frame,
                              (const unsigned char*)sfrag, (uint16_t*)out, s.H, s.T, s.L, s.F,
                              qtiles, (int)items, c2, s.T, 0, 1, nullptr, nullptr, nullptr, mix, nullptr, nullptr,
                              nullptr, nullptr, 0, nullptr);
  };
  if (mix) {
    if (s.d == 128) loader ? args(attn_bf16_kernel<128, false, true, true>) : args(attn_bf16_kernel<128, false, true>);
    else loader ? args(attn_bf16_kernel<64, false, true, true>) : args(attn_bf16_kernel<64, false, true>);
  } else {
    if (s.d == 128) loader ? args(attn_bf16_kernel<128, false, false, true>) : args(attn_bf16_kernel<128, false>);
    else loader ? args(attn_bf16_kernel<64, false, false, true>) : args(attn_bf16_kernel<64, false>);
  }
  return hipGetLastError();
}

hipError_t launch_attn_scan_bf16(const void* q, const void* k, const void* v, const void* qp, const void* ws,
                                 const float* alpha, float* state, void* sfrag, unsigned* flags, void* out,
                                 const Shape& s, float scale, hipStream_t st, const void* wq) {
  const int qtiles = (s.L + QPB - 1) / QPB;
  const long long items = (long long)s.B * s.H * s.F * qtiles;
  const int ncb = s.d / 32;
  const int units = s.B * s.H * ncb;
  const int n_scan = 8 * ((units + 8 * ncb - 1) / (8 * ncb) * ncb);  // whole (b, h) units per XCD
  const int grid = n_scan + (int)((items + 7) / 8 * 8);
  const float c2 = scale * kLog2e;
  const long long fb = (long long)s.d * s.d * 2;  // fragment bytes per frame
  HA_LOG("launch attn_bf16_kernel<%d> with the state scan: grid %d x %d threads (%d scan work-groups for %d (b, h, "
         "column block) units walking %d frames, then %lld attention items = %d streams x %d heads x %d frames x %d "
         "query tiles; each waits for its frame's state%s)",
         s.d, grid, NT, n_scan, units, s.F, items, s.B, s.H, s.F, qtiles,
         wq ? "; readout fragments of W_q S, contracted with Q" : "");
  auto args = [&](auto kern) {
    kern<<<grid, NT, 0, st>>>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)qp,
                              nullptr, s.F * fb, fb, (const unsigned char*)sfrag, (uint16_t*)out, s.H, s.T, s.L, s.F,
                              qtiles, (int)items, c2, s.T, 0, 1, nullptr, nullptr, nullptr, nullptr,
                              (const unsigned char*)ws, alpha, state, flags, n_scan, (const uint16_t*)wq);
  };
  if (s.d == 128) args(attn_bf16_kernel<128, false, false, false, true>);
  else args(attn_bf16_kernel<64, false, false, false, true>);
  return hipGetLastError();
}

int kv_splits(const Shape& s, int kv_off) {
  const int qtiles = (s.L + QPB - 1) / QPB;
  const long long items = (long long)s.B * s.H * s.F * qtiles;
  if (items >= 256) return 1;
  const int nt_min = (kv_off + s.L + KT - 1) / KT;  // tiles of the call's first frame
  int n = (int)((512 + items - 1) / items);
  if (n > nt_min / 16) n = nt_min / 16;  // at least 16 key tiles per split
  if (n > 32) n = 32;
  return n < 1 ? 1 : n;
}

hipError_t launch_attn_kv_bf16(const void* q, const void* k_cache, const void* v_cache, void* out, float* part_o,
                               void* part_ml, int nsplit, int Tk, int kv_off, const Shape& s, float scale,
                               hipStream_t st, const float* add_o) {
  const int qtiles = (s.L + QPB - 1) / QPB;
  const int units = s.B * s.H * s.F * nsplit;
  const int grid = ((units + 7) / 8) * 8 * qtiles;
  const float c2 = scale * kLog2e;
  HA_LOG("launch attn_bf16_kernel<%d, KV>: grid %d x %d threads (%d units x %d query tiles, %d key splits, keys "
         "%s)%s", s.d, grid, NT, units, qtiles, nsplit, kv_off < 0 ? "of the own frame" : "of the cache",
         nsplit > 1 ? " + attn_merge_kernel" : "");
  auto args = [&](auto kern) {
    kern<<<grid, NT, 0, st>>>((const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache, nullptr,
                              nullptr, 0, 0, nullptr, (uint16_t*)out, s.H, s.T, s.L, s.F, qtiles, units, c2, Tk,
                              kv_off, nsplit, part_o, (float2*)part_ml, add_o, nullptr, nullptr, nullptr, nullptr, nullptr,
                              0, nullptr);
  };
  if (s.d == 128) args(attn_bf16_kernel<128, true>);
  else args(attn_bf16_kernel<64, true>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const long long rows = (long long)s.B * s.T * s.H;
  const long long threads = rows * (s.d / 8);
  if (s.d == 128)
    attn_merge_kernel<128><<<(int)((threads + 255) / 256), 256, 0, st>>>(part_o, (const float2*)part_ml,
                                                                         (uint16_t*)out, rows, nsplit);
  else
    attn_merge_kernel<64><<<(int)((threads + 255) / 256), 256, 0, st>>>(part_o, (const float2*)part_ml,
                                                                        (uint16_t*)out, rows, nsplit);
  return hipGetLastError();
}

HA_DEBUG_READER(debug_take_attn)

hipError_t launch_kv_append(const void* k, const void* v, void* k_cache, void* v_cache, int cache_tokens,
                            int at_token, const Shape& s, hipStream_t st) {
  const long long per_b = (long long)s.T * s.H * s.d * 2 / 16;  // 16-byte pieces per stream
  const long long cap_b = (long long)cache_tokens * s.H * s.d * 2 / 16;
  const long long at = (long long)at_token * s.H * s.d * 2 / 16;
  const long long total = per_b * s.B;
  HA_LOG("launch kv_append_kernel: %lld 16-byte pieces of K and V into the cache at token %d", total, at_token);
  kv_append_kernel<<<(int)((total + 255) / 256), 256, 0, st>>>((const u32x4*)k, (const u32x4*)v, (u32x4*)k_cache,
                                                              (u32x4*)v_cache, per_b, cap_b, at, total);
  return hipGetLastError();
}

}  // namespace ha
