// Clean-pass state write of the ARL2 inter-frame branch ("Attend Locally,
// Remember Linearly", section 2.1 update rule; section 2.2: one write per
// clean frame, after the whole frame):
//   S_N = alpha_N S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1})
//       = (alpha_N I - G_N) S_{N-1} + B_N,
//   G_N = K'^T diag(beta) K',  B_N = K'^T diag(beta) V'.
// The affine form moves all the O(L d^2) work of a frame into G_N and B_N,
// which do not depend on the state and are computed for every frame in
// parallel (this file); only the O(d^3) recursion over frames stays
// sequential (state_scan.hip).
//
// Precision: the state must stay fp32-accurate. K' and V' are exact in bf16
// (they are the inputs), but beta*K' is not; it is split into hi + lo bf16
// parts (hi = bf16(x), lo = bf16(x - hi)), which carries ~16 mantissa bits,
// and both parts are accumulated on MFMA in fp32.
#include <type_traits>

#include "ha_device.h"
#include "ha_dma.h"
#include "ha_launch.h"
#include "ha_log.h"
#include "ha_gram_format.h"

namespace ha {
namespace {

constexpr int TC = 64;   // tokens per LDS chunk
constexpr int NW = 8;    // waves per work-group
constexpr int NT = NW * kWave;

// grid: one work-group per (b, h, frame). Each wave owns one 32-row band rb
// of both G = K'^T diag(beta) K' and B = K'^T diag(beta) V' (the two share
// their A operand (beta K')^T) and one share kh of the k-steps of every
// 64-token chunk; the token shares are summed through LDS at the end.
//
// G is symmetric. When the work-group writes the scan's format (not partial
// sums), band rb computes only the G blocks (rb, cb >= rb), 10 of 16 at d =
// 128, and the fragments of a lower block (cb, rb) come from the upper block
// (rb, cb), transposed through LDS inside the wave that holds it. The bands
// then carry unequal work (8, 7, 6, 5 blocks per k-step at d = 128), so the
// waves that share a SIMD (w and w + 4) take a heavy and a light band.
//
// The K', V' chunks arrive row-major ([token][d] bf16, as stored) by direct
// global -> LDS loads, three chunks in flight, and beta by a 4-byte-per-lane
// load; tokens >= L are outside the buffer descriptors' range and arrive as zeros.
// Both MFMA operands need 8 consecutive tokens per lane, which transposed LDS
// reads deliver without any transposing write. The A operand beta*K' is formed
// in fp32 in registers and split into bf16 hi + lo (two MFMAs), which keeps
// ~16 mantissa bits; K' and V' themselves are exact in bf16.
//
// Output, per (b, h, frame): -G as bf16 hi + lo and B as fp32, laid out in the
// scan's MFMA fragment order (store_g_half, store_b4). With nsplit > 1 the
// work-group (b, h, frame, split) covers only its share of the 64-token chunks.
// When `partial` is set the work-group writes its fp32 sums there instead
// (partial_block), to be added up in split order by gram_reduce_kernel or by
// the feature-map transform (fmap.hip).

// The increment format and the partial-sum layout: ha_gram_format.h.

template <int D, bool TWO>
__global__ __launch_bounds__(NT) void gram_bf16_kernel(const uint16_t* __restrict__ kp,
                                                       const uint16_t* __restrict__ vp,
                                                       const float* __restrict__ beta,
                                                       const float* __restrict__ beta2,
                                                       float* __restrict__ gram,
                                                       float* __restrict__ partial, int nsplit,
                                                       int H, int T, int L, int F, unsigned* __restrict__ flags) {
  constexpr int NCH = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = TC * D * 2;           // bytes of one K' or V' chunk
  constexpr int BUF = 2 * TILE + TC * 4 * (TWO ? 2 : 1);  // K', V', beta (and beta2)
  constexpr int SEGS = TILE / 1024;          // 1 KB direct-to-LDS segments per tile
  constexpr int RPS = 64 / NCH;              // rows per segment
  constexpr int NRB = D / 32;                // 32-row (and -column) blocks
  constexpr int KH = NW / NRB;               // waves sharing a row band (token split)
  constexpr int KSC = TC / 16;               // k-steps per chunk
  static_assert(KSC % KH == 0, "token split");
  static_assert(SEGS % NW == 0 || SEGS == NW, "segment split");
  constexpr int NBUF = 4;                    // chunks in flight
  constexpr int PART = NRB * 2 * 16 * 64 * 4;  // one wave's partial sums (G and B blocks)
  constexpr int SMEM = (KH - 1) * NRB * PART > NBUF * BUF ? (KH - 1) * NRB * PART : NBUF * BUF;
  __shared__ __align__(16) unsigned char smem[SMEM];

  const int hf = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int h = hf % H;
  const int n = (hf / H) % F;
  const int b = hf / (H * F);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  // row band of G and B, and which k-steps of each chunk: waves w and w + 4
  // (one SIMD) hold bands 0 and 3 or 1 and 2 at d = 128, bands 0 and 1 at 64
  static_assert(NRB == 4 || NRB == 2, "band pairing");
  const int rb = NRB == 4 ? ((wave & 1) ^ (3 * (wave >> 2))) : (wave >> 2);
  const int kh = NRB == 4 ? ((wave >> 1) & 1) : (wave & 3);
  // only the upper-triangle G blocks, when writing the scan's format
  const bool tri = !TWO && partial == nullptr;
  // the frame's counter of the fused scan and attention starts at zero
  if (flags && sp == 0 && tid == 0) flags[((size_t)b * H + h) * F + n] = 0u;

  const uint32_t rsb = (uint32_t)H * D * 2;
  const long long fbase = ((long long)b * T + (long long)n * L) * ((long long)H * D) + (long long)h * D;
  const int span = (int)((uint32_t)(L - 1) * rsb + D * 2);
  const u32x4 rk = rsrc_words(kp + fbase, span);
  const u32x4 rv = rsrc_words(vp + fbase, span);
  const long long bofs = ((long long)b * T + (long long)n * L) * H + h;
  const int bspan = (int)(((uint32_t)(L - 1) * H + 1) * 4);
  const u32x4 rbeta = rsrc_words(beta + bofs, bspan);
  const u32x4 rbeta2 = rsrc_words((TWO ? beta2 : beta) + bofs, bspan);
  // waves 0 (and 1 with two step-size vectors) also load the chunk's beta
  const bool has_beta = wave == 0 || (TWO && wave == 1);
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(smem));

  // direct-to-LDS: wave w fills segments w, w + NW, ... of each tile; those are
  // NW*RPS rows apart, which leaves the transposed-read swizzle unchanged.
  constexpr int MY_SEGS = SEGS / NW;
  const int srow = wave * RPS + lane / NCH, spc = lane % NCH;
  const uint32_t soff = srow * rsb + ((spc ^ tr_swz<NCH>(srow)) << 4);
  auto issue = [&](int c, int buf) {
    const uint32_t base = lds0 + buf * BUF;
    const uint32_t toff = (uint32_t)c * TC * rsb;
#pragma unroll
    for (int i = 0; i < MY_SEGS; ++i) {
      const uint32_t so = toff + (uint32_t)i * NW * RPS * rsb;
      dma16_asm(rk, base + (wave + NW * i) * 1024, soff, so);
      dma16_asm(rv, base + TILE + (wave + NW * i) * 1024, soff, so);
    }
    if (wave == 0) dma4_asm(rbeta, base + 2 * TILE, (uint32_t)lane * H * 4, (uint32_t)c * TC * H * 4);
    if (TWO && wave == 1)
      dma4_asm(rbeta2, base + 2 * TILE + TC * 4, (uint32_t)lane * H * 4, (uint32_t)c * TC * H * 4);
  };

  // transposed-read offsets: 16-lane group g reads rows 8*hh + gi/4 (+4) of a
  // 16-token step, columns 16*(g%2) + 4*(gi%4) of a 32-column block
  const int gi = lane & 15, g = lane >> 4;
  const int vrow = 8 * hh + (gi >> 2);
  const int vsw = tr_swz<NCH>(vrow);
  const int vcol = 16 * (g & 1) + 4 * (gi & 3);
  auto tr_off = [&](int row_add, int cblk) {
    const int col = vcol + 32 * cblk;
    return (vrow + row_add) * (D * 2) + (((col >> 3) ^ vsw) << 4) + (col & 7) * 2;
  };
  auto tr8 = [&](const unsigned char* tile, int ks, int cblk) {
    const u32x2 x0 = ds_read_tr16(tile + tr_off(16 * ks, cblk));
    const u32x2 x1 = ds_read_tr16(tile + tr_off(16 * ks + 4, cblk));
    return u32x4{x0[0], x0[1], x1[0], x1[1]};
  };

  f32x16 ag[NRB], ab[NRB];  // G and B blocks (rb, cb) of this wave's tokens
#pragma unroll
  for (int i = 0; i < NRB; ++i) ag[i] = ab[i] = f32x16{};

  // this split's chunks: [c0, c0 + nch) of the frame's chunks
  const int nch_all = (L + TC - 1) / TC;
  const int c0 = (int)((long long)sp * nch_all / nsplit);
  const int nch = (int)((long long)(sp + 1) * nch_all / nsplit) - c0;
  // debug bit 1: a valid (b, h, frame, split) and chunk range; bit 2: the last
  // transposed operand read of a chunk stays inside its tile
  HA_CHECK(h >= 0 && h < H && n >= 0 && n < F && b >= 0 && sp < nsplit && c0 >= 0 && nch >= 0 &&
               c0 + nch <= nch_all,
           1);
  HA_CHECK(tr_off(16 * (KSC - 1) + 4, NRB - 1) + 8 <= TILE, 2);
  for (int c = 0; c < NBUF - 1 && c < nch; ++c) issue(c0 + c, c);
  // this wave's copies per chunk (K' and V' segments, and beta)
  constexpr int PER = 2 * MY_SEGS;
  static_assert(2 * (PER + 1) <= 15, "vmcnt field");
  // wait until at most `later` chunks after the awaited one are in flight
  auto wait_chunks = [&](int later) {
    if (has_beta) {
      if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (PER + 1)));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (PER + 1));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
      if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * PER));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | PER);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  };
  constexpr int KPW = KSC / KH;  // k-steps of a chunk per wave
  // TB < 0: every G block; TB >= 0: this wave's band is TB, G blocks cb >= TB.
  // The A operands of a chunk, (beta K')^T rows 32*band.., tokens 16*ks +
  // 8*hh + e split into bf16 hi + lo, are formed while the MFMAs of the chunk
  // before it run: the barrier at the top of step c makes chunk c + 1
  // visible, so no wave starts a chunk with its operand arithmetic.
  auto chunks = [&](auto tb_c) {
    constexpr int TB = decltype(tb_c)::value;
    const int band = TB >= 0 ? TB : rb;
    // A operands of k-step kk of the chunk in buffer buf (shared by the G
    // blocks, B operand K', and the B blocks, B operand V'; with two step-size
    // vectors the B blocks take their own (beta2 K')^T)
    auto prep = [&](int buf, int kk, u32x4& ahi, u32x4& alo, u32x4& bhi, u32x4& blo) {
      const unsigned char* kt = smem + buf * BUF;
      const float* be = reinterpret_cast<const float*>(kt + 2 * TILE);
      const int ks = kh * KPW + kk;
      const u32x4 kraw = tr8(kt, ks, band);
      auto scaled_split = [&](const float* bp, u32x4& hi4, u32x4& lo4) {
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(bp + 16 * ks + 8 * hh);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(bp + 16 * ks + 8 * hh + 4);
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float bl = w2 < 2 ? b0[2 * w2] : b1[2 * w2 - 4];
          const float bu = w2 < 2 ? b0[2 * w2 + 1] : b1[2 * w2 - 3];
          const float x0 = bl * bf16_lo_to_f32(kraw[w2]);
          const float x1 = bu * bf16_hi_to_f32(kraw[w2]);
          const uint32_t hi = pack_bf16x2(x0, x1);
          hi4[w2] = hi;
          lo4[w2] = pack_bf16x2(x0 - bf16_lo_to_f32(hi), x1 - bf16_hi_to_f32(hi));
        }
      };
      scaled_split(be, ahi, alo);
      if constexpr (TWO) scaled_split(be + TC, bhi, blo);
      else { bhi = ahi; blo = alo; }
    };
    u32x4 ahi[KPW], alo[KPW], bhi[KPW], blo[KPW];
    if (nch > 0) {
      // chunk 0 landed (chunks 1 and 2 may be in flight) and is visible
      wait_chunks(nch - 1 < NBUF - 2 ? nch - 1 : NBUF - 2);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < KPW; ++kk) prep(0, kk, ahi[kk], alo[kk], bhi[kk], blo[kk]);
    }
    for (int c = 0; c < nch; ++c) {
      const int buf = c % NBUF;
      const bool more = c + 1 < nch;
      if (more) {
        // chunk c+1 landed (chunk c+2 may be in flight), and every wave is
        // done with chunk c-1, whose buffer takes chunk c+NBUF-1
        wait_chunks(nch - 2 - c < 1 ? nch - 2 - c : 1);
        __syncthreads();
        if (c + NBUF - 1 < nch) issue(c0 + c + NBUF - 1, (c + NBUF - 1) % NBUF);
      }
      const unsigned char* kt = smem + buf * BUF;
      const unsigned char* vt = kt + TILE;
#pragma unroll
      for (int kk = 0; kk < KPW; ++kk) {
        const int ks = kh * KPW + kk;
#pragma unroll
        for (int cb = 0; cb < NRB; ++cb) {
          const u32x4 bv = tr8(vt, ks, cb);
          if (TB < 0 || cb >= TB) {
            const u32x4 bk = tr8(kt, ks, cb);
            ag[cb] = mfma32x32x16(ahi[kk], bk, ag[cb]);
            ab[cb] = mfma32x32x16(bhi[kk], bv, ab[cb]);
            ag[cb] = mfma32x32x16(alo[kk], bk, ag[cb]);
            ab[cb] = mfma32x32x16(blo[kk], bv, ab[cb]);
          } else {
            ab[cb] = mfma32x32x16(bhi[kk], bv, ab[cb]);
            ab[cb] = mfma32x32x16(blo[kk], bv, ab[cb]);
          }
        }
        // this k-step's operands are consumed: form chunk c+1's (after the
        // last chunk from a stale buffer, unused; no branch keeps the
        // arithmetic free to interleave with the MFMAs above)
        prep((c + 1) % NBUF, kk, ahi[kk], alo[kk], bhi[kk], blo[kk]);
      }
    }
  };
  // the band as a compile-time constant, so that each band's loop holds
  // exactly its MFMAs
  if (!tri) chunks(std::integral_constant<int, -1>{});
  else if (rb == 0) chunks(std::integral_constant<int, 0>{});
  else if (rb == 1) chunks(std::integral_constant<int, 1>{});
  else if constexpr (NRB > 2) {
    if (rb == 2) chunks(std::integral_constant<int, 2>{});
    else chunks(std::integral_constant<int, 3>{});
  }

  // sum the token halves: waves with kh > 0 hand their partial blocks to the
  // kh = 0 wave of the same row band through LDS (lane-linear, conflict-free)
  if constexpr (KH > 1) {
    __syncthreads();  // every wave is done with the chunk buffers
    f32x4* part = reinterpret_cast<f32x4*>(smem);
    if (kh > 0) {  // (with tri, the lower G blocks are zero and not read)
      f32x4* my = part + ((size_t)((kh - 1) * NRB + rb) * NRB * 2 * 4) * 64;
#pragma unroll
      for (int cb = 0; cb < NRB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          my[((cb * 2 + 0) * 4 + v4) * 64 + lane] = f32x4{ag[cb][4 * v4], ag[cb][4 * v4 + 1], ag[cb][4 * v4 + 2], ag[cb][4 * v4 + 3]};
          my[((cb * 2 + 1) * 4 + v4) * 64 + lane] = f32x4{ab[cb][4 * v4], ab[cb][4 * v4 + 1], ab[cb][4 * v4 + 2], ab[cb][4 * v4 + 3]};
        }
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int j = 1; j < KH; ++j) {
      const f32x4* src = part + ((size_t)((j - 1) * NRB + rb) * NRB * 2 * 4) * 64;
#pragma unroll
      for (int cb = 0; cb < NRB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 xg = src[((cb * 2 + 0) * 4 + v4) * 64 + lane];
          const f32x4 xb = src[((cb * 2 + 1) * 4 + v4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ag[cb][4 * v4 + e] += xg[e];
            ab[cb][4 * v4 + e] += xb[e];
          }
        }
    }
  }

  if (partial) {  // fp32 partial sums of this split, summed by a later pass
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb) {
      f32x4* dst = partial_block<D>(partial, (size_t)hf * nsplit + sp, rb, cb);
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        dst[(0 * 4 + v4) * 64 + lane] = f32x4{ag[cb][4 * v4], ag[cb][4 * v4 + 1], ag[cb][4 * v4 + 2], ag[cb][4 * v4 + 3]};
        dst[(1 * 4 + v4) * 64 + lane] = f32x4{ab[cb][4 * v4], ab[cb][4 * v4 + 1], ab[cb][4 * v4 + 2], ab[cb][4 * v4 + 3]};
      }
    }
    return;
  }
  // workspace order [b][h][frame] (the grid runs heads fastest)
  unsigned char* base = reinterpret_cast<unsigned char*>(gram) +
                        ((size_t)(b * H + h) * F + n) * (size_t)D * D * 8;
  // the lower block (cb, rb) of G is the transpose of the upper block (rb,
  // cb): it goes through 32 x 36 floats of LDS (rows padded to keep the
  // 16-byte reads aligned), the region whose partial sums this wave has read
  float* tp = reinterpret_cast<float*>(smem) + (size_t)rb * NRB * 2 * 4 * 64 * 4;
  const int lr = lane & 31;
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      store_b4<D>(base, rb, cb, v4, lane, f32x4{ab[cb][4 * v4], ab[cb][4 * v4 + 1], ab[cb][4 * v4 + 2], ab[cb][4 * v4 + 3]});
    if (tri && cb < rb) continue;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      float g8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g8[e] = ag[cb][8 * sh + e];
      store_g_half<D>(base, rb, cb, sh, lane, g8);
    }
    if (tri && cb > rb) {
      // element r of lane l is G(rb, cb)[x_r][l % 32], x_r = 8(r/4) + 4hh + r%4;
      // the lower block wants element r of lane l = G(rb, cb)[l % 32][x_r]
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // earlier reads of the region returned
      asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 16; ++r) tp[(8 * (r >> 2) + 4 * hh + (r & 3)) * 36 + lr] = ag[cb][r];
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);
      asm volatile("" ::: "memory");
      float t16[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(tp + lr * 36 + 8 * q4 + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) t16[4 * q4 + e] = x[e];
      }
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) store_g_half<D>(base, cb, rb, sh, lane, t16 + 8 * sh);
    }
  }
}

// Sum of the nsplit partial increments of one (b, h, frame), in split order,
// stored in the scan's format. Work-group (hf, rb, cb) with hf the gram grid's
// (b, frame, head) index, 256 threads: thread
// part p = tid / 64 handles, for lane tid % 64, the G accumulator elements
// [8p, 8p + 8) (p < 2) or the B elements [8(p-2), 8(p-2) + 8) (p >= 2).
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ partial,
                                                          float* __restrict__ gram, int nsplit,
                                                          int H, int F) {
  constexpr int NRB = D / 32;
  const int blk = blockIdx.x;
  const int cb = blk % NRB, rb = (blk / NRB) % NRB;
  const int hf = blk / (NRB * NRB);
  const int h = hf % H, n = (hf / H) % F, b = hf / (H * F);
  const int lane = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int gb = p >> 1, v0 = 2 * (p & 1);  // G or B, first of two 4-element pieces
  f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll 8
  for (int sp = 0; sp < nsplit; ++sp) {
    const f32x4* src = partial_block<D>(const_cast<float*>(partial), (size_t)hf * nsplit + sp, rb, cb);
    s0 += src[(gb * 4 + v0) * 64 + lane];
    s1 += src[(gb * 4 + v0 + 1) * 64 + lane];
  }
  unsigned char* base = reinterpret_cast<unsigned char*>(gram) +
                        ((size_t)(b * H + h) * F + n) * (size_t)D * D * 8;
  if (gb == 0) {
    const float g8[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    store_g_half<D>(base, rb, cb, p & 1, lane, g8);
  } else {
    store_b4<D>(base, rb, cb, v0, lane, s0);
    store_b4<D>(base, rb, cb, v0 + 1, lane, s1);
  }
}

}  // namespace

HA_DEBUG_READER(debug_take_gram)

hipError_t launch_gram_partials_bf16(const void* kp, const void* vp, const float* beta, const float* beta2,
                                     float* partial, int nsplit, const Shape& s, hipStream_t st) {
  const int grid = (int)((long long)s.B * s.H * s.F * nsplit);
  HA_LOG("launch gram_bf16_kernel<%d> (partial sums): grid %d x %d threads (%d token splits per frame%s)", s.d, grid,
         NT, nsplit, beta2 ? ", two step-size vectors" : "");
  auto run = [&](auto gk) {
    gk<<<grid, NT, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, beta, beta2, nullptr, partial, nsplit, s.H,
                            s.T, s.L, s.F, nullptr);
  };
  if (s.d == 128) {
    if (beta2) run(gram_bf16_kernel<128, true>);
    else run(gram_bf16_kernel<128, false>);
  } else {
    if (beta2) run(gram_bf16_kernel<64, true>);
    else run(gram_bf16_kernel<64, false>);
  }
  return hipGetLastError();
}

hipError_t launch_gram_bf16(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st, unsigned* flags) {
  const long long groups = (long long)s.B * s.H * s.F;
  const int nsplit = gram_splits(s);
  // partial sums after the increments (gram_bytes reserves both)
  float* partial = nsplit > 1 ? gram + gram_final_bytes(s) / sizeof(float) : nullptr;
  const int grid = (int)(groups * nsplit);
  HA_LOG("launch gram_bf16_kernel<%d>: grid %d x %d threads (%lld (b,h,frame) x %d token splits)%s", s.d, grid, NT,
         groups, nsplit, nsplit > 1 ? " + gram_reduce_kernel" : "");
  auto run = [&](auto gk, auto rk, int nrb) {
    gk<<<grid, NT, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, beta, nullptr, gram, partial, nsplit,
                            s.H, s.T, s.L, s.F, flags);
    if (nsplit > 1) rk<<<(int)(groups * nrb * nrb), 256, 0, st>>>(partial, gram, nsplit, s.H, s.F);
  };
  if (s.d == 128) run(gram_bf16_kernel<128, false>, gram_reduce_kernel<128>, 4);
  else run(gram_bf16_kernel<64, false>, gram_reduce_kernel<64>, 2);
  return hipGetLastError();
}

}  // namespace ha
