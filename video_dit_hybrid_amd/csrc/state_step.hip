// Clean-pass state write of a one-frame call in a single launch (ARL2,
// "Attend Locally, Remember Linearly", section 2.1 update rule; section 2.2:
// one write per clean frame, after the whole frame):
//   S_1 = alpha S_0 + K'^T diag(beta) (V' - K' S_0)
// taken as written: the residual R = V' - K' S_0 of every token, then the
// increment K'^T (beta . R), then the decay, all in one kernel. Over several
// frames the affine form (gram + scan kernels) lets the frames' O(L d^2) work
// run in parallel; with one frame there is nothing to overlap, and this form
// reads K', V' once and writes S once, with no intermediate in HBM.
//
// Work decomposition (d = 128): a unit is (b, h, 32-column block cb of S);
// column block cb of S_1 depends only on column block cb of S_0. The tokens
// of a unit are split over nsplit work-groups when units alone leave most of
// the chip idle (shape only). A work-group has 4 waves; wave w takes the
// 32-token blocks w, w + 4, ... of its split.
//
// Per 32-token block, on MFMA (v_mfma_f32_32x32x16_bf16):
//   R[tok][col] = V' + K' (-S_0): A = K' rows (exact bf16), B = -S_0 split into
//     bf16 hi + lo (~16 mantissa bits), accumulator initialised with V';
//   Y = beta . R in fp32, split hi + lo;
//   dS[dk][col] += K'^T Y: A = K'^T through transposed LDS reads, B = Y taken
//     straight from R's accumulator registers. The accumulator gives lane half
//     hh the tokens 4hh..4hh+3 and 8+4hh..8+4hh+3 of each 16; the contraction
//     order over tokens is free, so the A operand reads K' rows in that same
//     order.
// K' blocks, the block's V' columns and beta reach LDS by direct global ->
// LDS copies (three blocks in flight per wave, each wave its own slots, waits
// by explicit vmcnt counts); tokens >= L are outside the buffer descriptors'
// range and arrive as zeros, so they add nothing. R's accumulator takes V'
// through transposed reads (one column, four consecutive tokens per lane).
// The four waves' increments are added through LDS in wave order; with
// nsplit > 1 each work-group leaves its sum in the workspace and the last to
// take the unit's ticket adds them up in split order (the result does not
// depend on which finishes last) and writes S_1 = alpha S_0 + dS.
#include <atomic>

#include "ha_device.h"
#include "ha_dma.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

constexpr int SW = 4;               // waves per work-group
constexpr int TB = 32;              // tokens per block
constexpr int SD = 128;             // head dimension of this kernel
constexpr int NCB = SD / 32;        // 32-column blocks of S (units per (b, h))
constexpr int KS = SD / 16;         // k-steps of K' S over d_k
constexpr int NRB = SD / 32;        // 32-row blocks of the increment
constexpr int KBLK = TB * SD * 2;   // bytes of one K' block (8 KB)
constexpr int VBLK = TB * 32 * 2;   // bytes of the block's V' columns [32 tokens][32] (2 KB)
constexpr int BUF = KBLK + VBLK + 256;  // + beta of 64 tokens (one 4-byte copy)
constexpr int NSLOT = 3;            // blocks in flight per wave
constexpr int OPS = KBLK / 1024 + VBLK / 1024 + 1;  // copies per block
constexpr int kDevice = 16;         // cache policy: sc1 (device scope)
static_assert(SW == NRB, "the wave-sum assigns one row block per wave");

// K' blocks are [32 tokens][128] bf16 rows of 16 chunks of 16 bytes; chunk c of
// row r sits at chunk c ^ swz(r). Row reads (16 lanes: 16 rows, one chunk) and
// transposed reads (32 lanes: 4 rows x 4 chunks) both hit 16 distinct chunks.
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// s_waitcnt immediate: at most n vector-memory operations outstanding
// (vmcnt split over bits 3:0 and 15:14; expcnt and lgkmcnt left at maximum)
constexpr int vm_wait(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// The unit's ticket: a 64-bit word holding the call's tag (low 8 bits clear,
// never 0) and the number of splits that have arrived. A word holding another
// tag, whatever it is (a finished call leaves 0, a fresh workspace anything),
// counts as no arrival; the last arrival puts back 0, so HIP graph replays of
// one launch (same tag) start clean. Returns whether the caller arrived last.
// One lane per work-group; every failed exchange is another split's
// successful one, so the loop ends within nsplit rounds (the bound is only a
// guard). A device-scope atomic without fences: the sums it guards are
// written and read with device-scope (sc1) buffer accesses, coherent across
// the XCDs' L2s without flushing them.
__device__ __forceinline__ int take_ticket(unsigned long long* t, unsigned long long tag, int nsplit) {
  unsigned long long cur = __hip_atomic_load(t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; it < 1024; ++it) {
    const unsigned cnt = (cur & ~0xFFull) == tag ? (unsigned)(cur & 0xFF) : 0u;
    const bool last = cnt + 1 == (unsigned)nsplit;
    const unsigned long long nxt = last ? 0ull : (tag | (cnt + 1));
    unsigned long long seen = cur;
    if (__hip_atomic_compare_exchange_strong(t, &seen, nxt, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return last;
    cur = seen;
  }
  HA_CHECK(false, 8);  // debug bit 8: the exchange loop ran out (cannot happen with nsplit <= 16 splits)
  return 0;
}

__global__ __launch_bounds__(SW * 64, 1) void state_step_kernel(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp, const float* __restrict__ alpha,
    const float* __restrict__ beta, float* __restrict__ state, float* __restrict__ snap,
    float* __restrict__ part, unsigned long long* __restrict__ tickets, unsigned long long tag, int H, int L,
    int nsplit, int n_items) {
  __shared__ __align__(16) unsigned char smem[SW * NSLOT * BUF];
  __shared__ int s_last;
  const int item = xcd_major_item(gridDim.x);  // the splits of a unit share an XCD
  if (item >= n_items) return;
  const int unit = item / nsplit, sp = item % nsplit;
  const int cb = unit % NCB, bh = unit / NCB, h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hh = lane >> 5;

  // this frame's K', V' of (b, h): tokens [0, L) of stream b (T = L)
  const uint32_t rsb = (uint32_t)H * SD * 2;
  const long long fbase = (long long)b * L * H * SD + (long long)h * SD;
  const int span = (int)((uint32_t)(L - 1) * rsb + SD * 2);
  const u32x4 rk = rsrc_words(kp + fbase, span);
  const u32x4 rv = rsrc_words(vp + fbase, span);
  const u32x4 rbeta = rsrc_words(beta + (long long)b * L * H + h, (int)(((uint32_t)(L - 1) * H + 1) * 4));
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(smem));

  const int nblk = (L + TB - 1) / TB;
  const int k0 = (int)((long long)sp * nblk / nsplit), k1 = (int)((long long)(sp + 1) * nblk / nsplit);
  const int nb = (k1 - k0 - wave + SW - 1) / SW;  // this wave's blocks k0 + wave + SW m, m < nb
  const int gi = lane & 15, g = lane >> 4;

  // K' block (rows swizzled), V' columns [32 cb, 32 cb + 32) ([32][32] bf16,
  // 64-byte rows) and beta -> this wave's LDS slot
  auto issue = [&](int m, int slot) {
    const int kb = k0 + wave + SW * m;
    HA_CHECK(kb >= k0 && kb < k1 && slot >= 0 && slot < NSLOT, 2);  // debug bit 2: a block of this split
    const uint32_t base = lds0 + (wave * NSLOT + slot) * BUF;
    const uint32_t toff = (uint32_t)kb * TB * rsb;
#pragma unroll
    for (int i = 0; i < KBLK / 1024; ++i) {
      const int r = 4 * i + (lane >> 4);
      dma16_asm(rk, base + i * 1024, (uint32_t)r * rsb + (((lane & 15) ^ swz(r)) << 4), toff);
    }
#pragma unroll
    for (int i = 0; i < VBLK / 1024; ++i)
      dma16_asm(rv, base + KBLK + i * 1024, (uint32_t)(16 * i + (lane >> 2)) * rsb + cb * 64 + (lane & 3) * 16,
                toff);
    dma4_asm(rbeta, base + KBLK + VBLK, (uint32_t)lane * H * 4, (uint32_t)kb * TB * H * 4);
  };

  // the first blocks' copies go out before the loads of S_0, so the two
  // latencies overlap
  for (int m = 0; m < NSLOT && m < nb; ++m) issue(m, m);

  // -S_0[:, cb] as the B operand of K'(-S_0): lane (j, hh) holds rows
  // 16 ks + 8 hh + e of column 32 cb + j, split into bf16 hi + lo
  u32x4 shi[KS], slo[KS];
  {
    const float* scol = state + (size_t)bh * SD * SD + cb * 32 + j;
    float x[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[ks][e] = -scol[(size_t)(16 * ks + 8 * hh + e) * SD];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float x0 = x[ks][2 * w2], x1 = x[ks][2 * w2 + 1];
        const uint32_t hp = pack_bf16x2(x0, x1);
        shi[ks][w2] = hp;
        slo[ks][w2] = pack_bf16x2(x0 - bf16_lo_to_f32(hp), x1 - bf16_hi_to_f32(hp));
      }
  }

  // per-lane LDS offsets: row reads of K' (row j, chunk 2 ks + hh) and the
  // transposed reads of K'^T (group g = lane / 16 reads rows base + gi / 4,
  // columns 32 rb + 16 (g % 2) + 4 (gi % 4))
  const int ka = j * (SD * 2) + ((hh ^ swz(j)) << 4);
  // debug bit 1: a valid unit and split, block range inside the frame; bit 4:
  // the last row and transposed reads of a block stay inside its K' tile
  HA_CHECK(cb < NCB && h < H && b >= 0 && sp < nsplit && k0 >= 0 && k0 <= k1 && k1 <= nblk, 1);
  auto tr_off = [&](int row, int rb) {
    const int col = 32 * rb + 16 * (g & 1) + 4 * (gi & 3);
    return row * (SD * 2) + (((col >> 3) ^ swz(row)) << 4) + (col & 7) * 2;
  };
  HA_CHECK((ka ^ ((KS - 1) << 5)) + 16 <= KBLK && tr_off(TB - 1, NRB - 1) + 8 <= KBLK, 4);

  // the S_0 elements this thread writes S_1 of at the end (rows 32 wave +
  // 8 v4 + 4 hh + e of column 32 cb + j), loaded now so that their latency
  // overlaps the blocks instead of the end
  float s0v[4][4];
  const float al = alpha[(size_t)b * H + h];
  {
    const float* scol = state + (size_t)bh * SD * SD + cb * 32 + j;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
      for (int e = 0; e < 4; ++e) s0v[v4][e] = scol[(size_t)(32 * wave + 8 * v4 + 4 * hh + e) * SD];
  }

  f32x16 ds[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) ds[rb] = f32x16{};

  auto process = [&](int slot) {
    const unsigned char* kt = smem + (wave * NSLOT + slot) * BUF;
    const unsigned char* vt = kt + KBLK;
    const float* bt = reinterpret_cast<const float*>(kt + KBLK + VBLK);
    // every LDS operand of the block is read up front (one wave per SIMD: no
    // other wave hides the LDS latency): K' rows for K'(-S_0), V' for R's
    // start, beta, then the transposed K'^T operands of the increment, which
    // the schedule below interleaves with the K'(-S_0) MFMAs
    u32x4 ar[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ar[ks] = *reinterpret_cast<const u32x4*>(kt + (ka ^ (ks << 5)));
    // R starts as V': elements 4 q4 .. 4 q4 + 3 are tokens 8 q4 + 4 hh + 0..3 of
    // column j, one transposed read (group g reads rows 8 q4 + 4 hh + gi / 4,
    // columns 16 (g % 2) + 4 (gi % 4))
    u32x2 vx[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      vx[q4] = ds_read_tr16(vt + (8 * q4 + 4 * hh + (gi >> 2)) * 64 + (16 * (g & 1) + 4 * (gi & 3)) * 2);
    // element q of the accumulator is token 8 (q / 4) + 4 hh + q % 4
    f32x4 bq[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) bq[q4] = *reinterpret_cast<const f32x4*>(bt + 8 * q4 + 4 * hh);
    // K'^T operands: token k-slot (hh, e) of step t is 16 t + 4 hh + e (e < 4)
    // and 16 t + 8 + 4 hh + e - 4 (e >= 4)
    u32x4 at[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x2 x0 = ds_read_tr16(kt + tr_off(16 * t + 4 * hh + (gi >> 2), rb));
        const u32x2 x1 = ds_read_tr16(kt + tr_off(16 * t + 8 + 4 * hh + (gi >> 2), rb));
        at[rb][t] = u32x4{x0[0], x0[1], x1[0], x1[1]};
      }
    f32x16 r;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      r[4 * q4] = bf16_lo_to_f32(vx[q4][0]);
      r[4 * q4 + 1] = bf16_hi_to_f32(vx[q4][0]);
      r[4 * q4 + 2] = bf16_lo_to_f32(vx[q4][1]);
      r[4 * q4 + 3] = bf16_hi_to_f32(vx[q4][1]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      r = mfma32x32x16(ar[ks], shi[ks], r);
      r = mfma32x32x16(ar[ks], slo[ks], r);
    }
    // Y = beta . R, split hi + lo: the B operand of step t is elements 8t..8t+7
    u32x4 yhi[2], ylo[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int q = 8 * t + 2 * p;
        const float y0 = bq[q >> 2][q & 3] * r[q], y1 = bq[(q + 1) >> 2][(q + 1) & 3] * r[q + 1];
        const uint32_t hp = pack_bf16x2(y0, y1);
        yhi[t][p] = hp;
        ylo[t][p] = pack_bf16x2(y0 - bf16_lo_to_f32(hp), y1 - bf16_hi_to_f32(hp));
      }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        ds[rb] = mfma32x32x16(at[rb][t], yhi[t], ds[rb]);
        ds[rb] = mfma32x32x16(at[rb][t], ylo[t], ds[rb]);
      }
    // schedule: the 16 reads for K'(-S_0), R's start and beta; then each of
    // its 16 MFMAs followed by one of the 16 transposed K'^T reads
    __builtin_amdgcn_sched_group_barrier(0x100, KS + 8, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // NSLOT blocks in flight per wave: block m sits in slot m % NSLOT; the wait
  // before block m leaves the copies of the blocks issued after it in flight
  for (int m = 0; m < nb; ++m) {
    const int later = nb - 1 - m < NSLOT - 1 ? nb - 1 - m : NSLOT - 1;
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vm_wait(2 * OPS));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vm_wait(OPS));
    else __builtin_amdgcn_s_waitcnt(vm_wait(0));
    process(m % NSLOT);
    if (m + NSLOT < nb) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's reads of the slot are done
      issue(m + NSLOT, m % NSLOT);
    }
  }

  // ---- sum of the four waves' increments, in wave order: thread (w, lane)
  // ends with rows 32 w + 8 (q / 4) + 4 hh + q % 4, column 32 cb + j
  __syncthreads();  // every wave is done with its block buffers
  f32x4* wsum = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      wsum[((wave * NRB + rb) * 4 + v4) * 64 + lane] =
          f32x4{ds[rb][4 * v4], ds[rb][4 * v4 + 1], ds[rb][4 * v4 + 2], ds[rb][4 * v4 + 3]};
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    acc[v4] = wsum[((0 * NRB + wave) * 4 + v4) * 64 + lane];
#pragma unroll
    for (int w = 1; w < SW; ++w) acc[v4] += wsum[((w * NRB + wave) * 4 + v4) * 64 + lane];
  }

  if (nsplit > 1) {
    // every split leaves its sum (device-scope stores; the release fence makes
    // each wave wait for their acknowledgement before the barrier ahead of the
    // ticket); the last adds all of them in split order, loading the others'
    // only after the ticket exchange returned
    constexpr int SLOT_B = SW * 4 * 64 * 16;  // bytes of one split's sum (16 KB)
    auto prs = [&](int s2) {
      return make_rsrc((const char*)part + ((size_t)unit * nsplit + s2) * SLOT_B, SLOT_B);
    };
    const uint32_t off = (uint32_t)(wave * 4 * 64 + lane) * 16;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[v4]), prs(sp), off + v4 * 64 * 16, 0,
                                             kDevice);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) s_last = take_ticket(tickets + unit, tag, nsplit);
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    f32x4 tot[4];
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) tot[v4] = f32x4{};
    // the splits' sums come in groups of 8, all loads of a group in flight
    // at once, then added in split order
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      f32x4 x[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          // past the last split the load repeats the last one (every
          // address it touches is inside the workspace); its value is unused
          const int s2 = s0 + i, s2c = s2 < nsplit ? s2 : nsplit - 1;
          const f32x4 ld = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs(s2c), off + v4 * 64 * 16, 0, kDevice));
          x[i][v4] = s2 < nsplit && s2 != sp ? ld : acc[v4];
        }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (s0 + i < nsplit)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) tot[v4] += x[i][v4];
    }
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) acc[v4] = tot[v4];
  }

  // S_1 = alpha S_0 + dS (and S_0 to the snapshot)
  float* scol = state + (size_t)bh * SD * SD + cb * 32 + j;
  float* snp = snap ? snap + (size_t)bh * SD * SD + cb * 32 + j : nullptr;
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t row = (size_t)(32 * wave + 8 * v4 + 4 * hh + e);
      if (snp) snp[row * SD] = s0v[v4][e];
      scol[row * SD] = fmaf(al, s0v[v4][e], acc[v4][e]);
    }
}

unsigned long long next_tag() {
  static std::atomic<unsigned long long> counter{0};
  for (;;) {  // splitmix64 (Steele, Lea and Flood, 2014), low 8 bits cleared
    unsigned long long z = (counter.fetch_add(1) + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z = (z ^ (z >> 31)) & ~0xFFull;
    if (z) return z;
  }
}

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

HA_DEBUG_READER(debug_take_step)

int state_step_splits(const Shape& s) {
  // one work-group per CU (the kernel holds -S_0 and the increment in
  // registers: ~330 VGPRs + 80 AGPRs, one wave per SIMD) over 256 CUs, 8
  // token blocks or more per split
  const int units = s.B * s.H * NCB;
  const int nblk = (s.L + TB - 1) / TB;
  int n = 256 / units;
  if (n > nblk / 8) n = nblk / 8;
  if (n > 16) n = 16;
  return n < 1 ? 1 : n;
}

size_t state_step_bytes(const Shape& s) {
  if (s.d != SD || s.F != 1) return 0;
  const int n = state_step_splits(s);
  if (n == 1) return 0;
  const size_t units = (size_t)s.B * s.H * NCB;
  return al256(units * n * SD * 32 * 4) + al256(units * 8);
}

hipError_t launch_state_step_bf16(const void* kp, const void* vp, const float* alpha, const float* beta,
                                  float* state, float* snapshots, void* ws, const Shape& s, hipStream_t st) {
  if (s.d != SD || s.F != 1) return hipErrorInvalidValue;
  const int nsplit = state_step_splits(s);
  const long long units = (long long)s.B * s.H * NCB;
  const long long items = units * nsplit;
  const int grid = (int)((items + 7) / 8 * 8);
  float* part = nullptr;
  unsigned long long* tickets = nullptr;
  unsigned long long tag = 0;
  if (nsplit > 1) {
    part = (float*)ws;
    tickets = (unsigned long long*)((char*)ws + al256((size_t)items * SD * 32 * 4));
    tag = next_tag();
  }
  HA_LOG("launch state_step_kernel<%d>: grid %d x %d threads (%lld (b, h, 32-column) units x %d token splits; "
         "snapshot %s)", SD, grid, SW * 64, units, nsplit, snapshots ? "fp32" : "none");
  state_step_kernel<<<grid, SW * 64, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, alpha, beta, state,
                                               snapshots, part, tickets, tag, s.H, s.L, nsplit, (int)items);
  return hipGetLastError();
}

}  // namespace ha
