// The grouped per-head 1x1 feature maps of the inter-frame branch (ARL2,
// "Attend Locally, Remember Linearly", section 2.1 "adaptation": phi_q, phi_k,
// phi_v adapt the frozen projections' Q, K, V to the linear recurrence), read
// as one d x d linear map per head: Q' = Q W_q, K' = K W_k, V' = V W_v.
//
// The maps are folded into the work the layer already does instead of
// materialising Q', K', V':
//   readout   Q' S_{N-1} = Q (W_q S_{N-1})          -> mfrag_kernel writes the
//             readout fragments of M = W_q S; the attention kernel reads Q.
//   update    K'^T diag(beta) K' = W_k^T G0 W_k,
//             K'^T diag(beta) V' = W_k^T B0 W_v,
//             G0, B0 the increments of the unmapped K, V  -> gram_fmap_kernel
//             turns the gram pass's fp32 G0, B0 into the scan's format.
//
// Operands: every fp32 matrix entering an MFMA is split into bf16 hi + lo (two
// MFMAs), the maps are bf16 (exact); accumulation in fp32. All MFMA operands
// use the contraction order of the scan's fragments: k-slot 8*hh + e of k-step
// ks holds k = 16*ks + 8*(e/4) + 4*hh + e%4 (hh = lane / 32), in which the
// accumulator registers [8s, 8s+8) of a 32x32 block are the operand of k-step
// 2*(row band) + s.
#include "ha_device.h"
#include "ha_dma.h"
#include "ha_gram_format.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

// eight fp32 -> bf16 hi + lo (hi = bf16(x), lo = bf16(x - hi))
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const uint32_t hp = pack_bf16x2(x[2 * w2], x[2 * w2 + 1]);
    hi[w2] = hp;
    lo[w2] = pack_bf16x2(x[2 * w2] - bf16_lo_to_f32(hp), x[2 * w2 + 1] - bf16_hi_to_f32(hp));
  }
}

// W (bf16 [D][D] row-major) staged in LDS with the transposed-read swizzle;
// wtr returns the MFMA operand of k-step ks and 32-column block cb:
// lane l gets W[k][32*cb + l%32] for the eight k of its slots (two transposed
// 4 x 16 reads, rows 16*ks + 4*hh + i/4 and those + 8).
template <int D>
__device__ __forceinline__ void stage_w(unsigned char* lds, const uint16_t* w, int tid, int nthreads) {
  constexpr int NCH = D / 8;
  for (int i = tid; i < D * NCH; i += nthreads) {
    const int row = i / NCH, c = i % NCH;
    const u32x4 x = ld_global_16B(w + (size_t)row * D + c * 8);
    *reinterpret_cast<u32x4*>(lds + row * D * 2 + ((c ^ tr_swz<NCH>(row)) << 4)) = x;
  }
}
template <int D>
__device__ __forceinline__ u32x4 wtr(const unsigned char* lds, int ks, int cb, int lane) {
  constexpr int NCH = D / 8;
  const int gi = lane & 15, g = lane >> 4, hh = lane >> 5;
  const int col = 32 * cb + 16 * (g & 1) + 4 * (gi & 3);
  auto off = [&](int row) { return row * D * 2 + (((col >> 3) ^ tr_swz<NCH>(row)) << 4) + (col & 7) * 2; };
  const int r0 = 16 * ks + 4 * hh + (gi >> 2);
  const u32x2 x0 = ds_read_tr16(lds + off(r0));
  const u32x2 x1 = ds_read_tr16(lds + off(r0 + 8));
  return u32x4{x0[0], x0[1], x1[0], x1[1]};
}

// fp32 [D][D] row-major in LDS, 16-byte chunks XOR-swizzled by the row, so
// that 32 lanes reading 16 bytes of 32 different rows hit distinct banks
template <int D>
__device__ __forceinline__ int xrow(int row, int col) {
  constexpr int NC4 = D / 4;
  return row * D + ((((col >> 2) ^ (row & (NC4 - 1)))) << 2) + (col & 3);
}

// One work-group (D/32 waves) per (b, h, frame), in the gram grid's order
// hf = (b*F + n)*H + h. Wave w computes row band w of every product.
//   T_G = G0 W_k : A = G0's column block w (G0 is symmetric), B = W_k
//   G   = W_k^T T_G : A = W_k^T band w (= W_k column block w), B = T_G via LDS
//   T_B = B0 W_v : A = B0 band w (rows from LDS), B = W_v
//   B   = W_k^T T_B
template <int D>
__global__ __launch_bounds__(D / 32 * 64) void gram_fmap_kernel(const float* __restrict__ partial,
                                                                int nsplit,
                                                                const uint16_t* __restrict__ wk,
                                                                const uint16_t* __restrict__ wv,
                                                                float* __restrict__ gram, int H, int F,
                                                                unsigned* __restrict__ flags) {
  constexpr int NRB = D / 32, KS = D / 16, NTH = NRB * 64;
  __shared__ __align__(16) unsigned char smem[2 * D * D * 2 + D * D * 4];
  unsigned char* const wkl = smem;
  unsigned char* const wvl = smem + D * D * 2;
  float* const X = reinterpret_cast<float*>(smem + 2 * D * D * 2);
  f32x4* const Xf = reinterpret_cast<f32x4*>(X);  // fragment layout [band][cb][v4][lane]

  const int hf = blockIdx.x;
  const int h = hf % H, n = (hf / H) % F, b = hf / (H * F);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the frame's counter of a scan fused into the attention launch starts at zero
  if (flags && tid == 0) flags[((size_t)b * H + h) * F + n] = 0u;

  stage_w<D>(wkl, wk + (size_t)h * D * D, tid, NTH);
  stage_w<D>(wvl, wv + (size_t)h * D * D, tid, NTH);

  auto sum_partial = [&](int rb, int cb, int gb) {  // sum over splits, split order
    f32x16 r = f32x16{};
    for (int sp = 0; sp < nsplit; ++sp) {
      const f32x4* src = partial_block<D>(const_cast<float*>(partial), (size_t)hf * nsplit + sp, rb, cb);
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x4 x = src[(gb * 4 + v4) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 * v4 + e] += x[e];
      }
    }
    return r;
  };
  auto frags_to_lds = [&](const f32x16* t) {
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        Xf[((w * NRB + cb) * 4 + v4) * 64 + lane] =
            f32x4{t[cb][4 * v4], t[cb][4 * v4 + 1], t[cb][4 * v4 + 2], t[cb][4 * v4 + 3]};
  };
  // acc[cb] += W_k^T (band w) * Y, Y (fp32) in fragment layout in LDS
  auto left_wkt = [&](f32x16* acc) {
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb) acc[cb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 a = wtr<D>(wkl, ks, w, lane);
      const int rb = ks >> 1, s = ks & 1;
#pragma unroll
      for (int cb = 0; cb < NRB; ++cb) {
        const f32x4 y0 = Xf[((rb * NRB + cb) * 4 + 2 * s) * 64 + lane];
        const f32x4 y1 = Xf[((rb * NRB + cb) * 4 + 2 * s + 1) * 64 + lane];
        const float y8[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        u32x4 bhi, blo;
        split8(y8, bhi, blo);
        acc[cb] = mfma32x32x16(a, bhi, acc[cb]);
        acc[cb] = mfma32x32x16(a, blo, acc[cb]);
      }
    }
  };
  unsigned char* const base = reinterpret_cast<unsigned char*>(gram) +
                              ((size_t)(b * H + h) * F + n) * (size_t)D * D * 8;

  // ---- G = W_k^T (G0 W_k)
  f32x16 t[NRB];
  {
    f32x16 g0[NRB];  // G0 blocks (rb, column block w) = G0 band w, transposed
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) g0[rb] = sum_partial(rb, w, 0);
    __syncthreads();  // the maps are staged
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb) t[cb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float a8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] = g0[ks >> 1][8 * (ks & 1) + e];
      u32x4 ahi, alo;
      split8(a8, ahi, alo);
#pragma unroll
      for (int cb = 0; cb < NRB; ++cb) {
        const u32x4 bk = wtr<D>(wkl, ks, cb, lane);
        t[cb] = mfma32x32x16(ahi, bk, t[cb]);
        t[cb] = mfma32x32x16(alo, bk, t[cb]);
      }
    }
  }
  frags_to_lds(t);
  __syncthreads();
  left_wkt(t);
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb)
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      float g8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g8[e] = t[cb][8 * sh + e];
      store_g_half<D>(base, w, cb, sh, lane, g8);
    }
  __syncthreads();  // X is reused

  // ---- B = W_k^T (B0 W_v); B0 row-major in LDS (its band w is not a
  // column block of anything in registers)
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb) {
    const f32x16 x = sum_partial(w, cb, 1);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      X[xrow<D>(32 * w + 8 * (r >> 2) + 4 * hh + (r & 3), 32 * cb + lr)] = x[r];
  }
  __syncthreads();
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb) t[cb] = f32x16{};
  const int arow = 32 * w + lr;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = 16 * ks + 4 * hh;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(X + xrow<D>(arow, c0));
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(X + xrow<D>(arow, c0 + 8));
    const float a8[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    u32x4 ahi, alo;
    split8(a8, ahi, alo);
#pragma unroll
    for (int cb = 0; cb < NRB; ++cb) {
      const u32x4 bv = wtr<D>(wvl, ks, cb, lane);
      t[cb] = mfma32x32x16(ahi, bv, t[cb]);
      t[cb] = mfma32x32x16(alo, bv, t[cb]);
    }
  }
  __syncthreads();  // every wave has read B0
  frags_to_lds(t);
  __syncthreads();
  left_wkt(t);
#pragma unroll
  for (int cb = 0; cb < NRB; ++cb)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      store_b4<D>(base, w, cb, v4, lane, f32x4{t[cb][4 * v4], t[cb][4 * v4 + 1], t[cb][4 * v4 + 2], t[cb][4 * v4 + 3]});
}

// Readout fragments of M = W_q S for one (b, h, frame, 32-column block cb):
// wave w computes row band w of M[:, cb]; the fragment layout is the scan's
// ([b*H + h][frame][cb][k-step][lane] x 16 bytes, bf16 of the band's
// accumulator registers [8s, 8s+8) as k-step 2*w + s). S is fp32 row-major at
// states + (b*H + h)*sbh + n*sfr (floats).
template <int D>
__global__ __launch_bounds__(D / 32 * 64) void mfrag_kernel(const float* __restrict__ states, long long sbh,
                                                            long long sfr, const uint16_t* __restrict__ wq,
                                                            u32x4* __restrict__ mfrag, int H, int Fe) {
  constexpr int NCB = D / 32, KS = D / 16;
  const int blk = blockIdx.x;
  const int cb = blk % NCB, bhn = blk / NCB;
  const int n = bhn % Fe, bh = bhn / Fe, h = bh % H;
  const int lane = threadIdx.x & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const float* S = states + (size_t)bh * sbh + (size_t)n * sfr;
  const uint16_t* W = wq + (size_t)h * D * D + (size_t)(32 * w + lr) * D;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = 16 * ks + 4 * hh;
    const u32x2 a0 = *reinterpret_cast<const u32x2*>(W + c0);
    const u32x2 a1 = *reinterpret_cast<const u32x2*>(W + c0 + 8);
    const u32x4 a = u32x4{a0[0], a0[1], a1[0], a1[1]};
    float b8[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b8[e] = S[(size_t)(c0 + e) * D + 32 * cb + lr];
      b8[4 + e] = S[(size_t)(c0 + 8 + e) * D + 32 * cb + lr];
    }
    u32x4 bhi, blo;
    split8(b8, bhi, blo);
    acc = mfma32x32x16(a, bhi, acc);
    acc = mfma32x32x16(a, blo, acc);
  }
#pragma unroll
  for (int sh = 0; sh < 2; ++sh) {
    u32x4 hi;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) hi[w2] = pack_bf16x2(acc[8 * sh + 2 * w2], acc[8 * sh + 2 * w2 + 1]);
    mfrag[(((size_t)bhn * NCB + cb) * KS + 2 * w + sh) * 64 + lane] = hi;
  }
}

// Step sizes for L2-normalised keys K'_t = K_t W_k / max(||K_t W_k||, 1e-12):
// with n_t that norm, K'^T diag(beta) K' = W_k^T (K^T diag(beta / n^2) K) W_k
// and K'^T diag(beta) V' = W_k^T (K^T diag(beta / n) V) W_v, so the increment
// pass keeps the unmapped K, V and takes two step-size vectors. This kernel
// writes them: beta_g = beta / n^2, beta_b = beta / n.
// One work-group (4 waves) per (b, 512-token chunk, head h). Wave w owns the
// output features [32 eb, 32 eb + 32) with eb = w % (D/32) and holds that
// block of W_k^T as MFMA A fragments in registers for the whole chunk (read
// once from a staging copy of W_k in LDS). The chunk's K rows stream through
// LDS in slices of 64 tokens: direct global -> LDS copies of 1 KB per wave
// instruction, each covering whole rows (4 x 256 bytes at d = 128), two
// slices in flight while a third is read (deeper pipelines measured no
// faster), chunk c of row r stored at position
// c ^ kswz(r) so that the B operand reads (16 bytes of 16 consecutive rows per
// LDS cycle) hit distinct banks. Per 32-token column block a wave forms its
// 32 rows of Y^T = W_k^T K^T and their column sums of squares; the D/32 waves
// sharing a column block add theirs through LDS in wave order.
template <int NCH>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (NCH >= 16) return row & 15;
  else return (row >> 1) & 7;
}

template <int D>
__global__ __launch_bounds__(256) void keyscale_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ wk,
                                                       const float* __restrict__ beta,
                                                       float* __restrict__ beta_g, float* __restrict__ beta_b,
                                                       int H, int T, int nchunk) {
  constexpr int RB = D * 2;              // bytes of one token's row of a head
  constexpr int NCH = D / 8;             // 16-byte chunks per row
  constexpr int KS = D / 16;             // MFMA k-steps over d
  constexpr int NEB = D / 32;            // 32-feature blocks of Y^T
  constexpr int TS = 64;                 // tokens per slice
  constexpr int CT = 512;                // tokens per work-group
  constexpr int SLICE = TS * RB;
  constexpr int RPC = 1024 / RB;         // rows per 1 KB copy
  constexpr int CPW = SLICE / 1024 / 4;  // copies per wave per slice
  constexpr int NBUF = 3;                // slices in flight + 1
  constexpr int TBW = 2 * NEB / 4;       // 32-token column blocks per wave and slice
  static_assert(NBUF * SLICE >= D * D * 2, "W_k staging fits the slice buffers");
  static_assert((NBUF - 2) * CPW <= 15, "vmcnt immediate");
  __shared__ __align__(16) unsigned char smem[NBUF * SLICE];
  __shared__ float part[2][NEB][TS];
  const int blk = blockIdx.x;
  const int h = blk % H, rest = blk / H;
  const int ch = rest % nchunk, b = rest / nchunk;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eb = w % NEB, tb0 = (w / NEB) * TBW;
  const int ct0 = ch * CT;
  const int ns = (T - ct0 < CT ? T - ct0 + TS - 1 : CT) / TS;  // slices of this chunk
  const uint32_t rsb = (uint32_t)H * D * 2;  // bytes between consecutive tokens
  // this chunk's rows of head h (at most CT tokens: 32-bit offsets for any T);
  // rows past T are outside the range and arrive as zeros
  const int crows = T - ct0 < CT ? T - ct0 : CT;
  const u32x4 rk = rsrc_words(k + (((size_t)b * T + ct0) * H + h) * D, (int)((uint32_t)(crows - 1) * rsb + RB));
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(smem));

  // W_k^T rows 32 eb + lr, contraction d = 16 ks + 8 hh + j, into registers
  {
    const uint16_t* wh = wk + (size_t)h * D * D;
    for (int i = tid; i < D * NCH; i += 256)
      *reinterpret_cast<u32x4*>(smem + i * 16) = ld_global_16B(wh + (size_t)i * 8);
  }
  __syncthreads();
  u32x4 wf[KS];
  {
    const uint16_t* wl = reinterpret_cast<const uint16_t*>(smem);
    const int col = 32 * eb + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 16 * ks + 8 * hh + 2 * i;
        wf[ks][i] = (uint32_t)wl[d0 * D + col] | ((uint32_t)wl[(d0 + 1) * D + col] << 16);
      }
  }
  __syncthreads();  // the staging copy is consumed: the slices reuse its LDS

  // copy s of a slice covers rows RPC s .. RPC s + RPC - 1: lane l fills
  // position l % NCH of row RPC s + l / NCH; wave w issues copies w, w + 4, ...,
  // whose rows have the same kswz for a given lane
  const int crow = RPC * (w % (16 / RPC)) + lane / NCH;
  const uint32_t voff = (uint32_t)(lane / NCH) * rsb + (uint32_t)(((lane % NCH) ^ kswz<NCH>(crow)) << 4);
  auto issue = [&](int sl, int buf) {
    const uint32_t base = lds0 + buf * SLICE;
    const uint32_t t0 = (uint32_t)(sl * TS);  // relative to the chunk
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int sg = w + 4 * i;
      dma16_asm(rk, base + sg * 1024, voff, (t0 + RPC * sg) * rsb);
    }
  };
  // n_t^2 of the slice's tokens from the partial sums; token j by thread j
  auto finish = [&](int sl) {
    if (tid < TS) {
      const int t = ct0 + sl * TS + tid;
      float ss = part[sl & 1][0][tid];
#pragma unroll
      for (int e = 1; e < NEB; ++e) ss += part[sl & 1][e][tid];
      if (t < T) {
        const float n2 = fmaxf(ss, 1e-24f);
        const size_t i = ((size_t)b * T + t) * H + h;
        const float be = beta[i];
        beta_g[i] = be / n2;
        beta_b[i] = be / sqrtf(n2);
      }
    }
  };

  const int rd = (hh ^ kswz<NCH>(lr)) << 4;  // chunk 2 ks + hh of row 32 tb + lr: rd ^ (ks << 5)
  for (int sl = 0; sl < NBUF - 1 && sl < ns; ++sl) issue(sl, sl);
  for (int sl = 0; sl < ns; ++sl) {
    // slice sl landed: at most the copies of the slices after it are outstanding
    wait_later_copies<NBUF - 2, CPW>(ns - 1 - sl);
    lds_barrier();  // all copies of slice sl are in LDS; slice sl-1 and its partial sums are consumed
    if (sl + NBUF - 1 < ns) issue(sl + NBUF - 1, (sl + NBUF - 1) % NBUF);
    if (sl > 0) finish(sl - 1);
    const unsigned char* kt = smem + (sl % NBUF) * SLICE;
#pragma unroll
    for (int i = 0; i < TBW; ++i) {
      const int tb = tb0 + i;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = mfma32x32x16(wf[ks], *reinterpret_cast<const u32x4*>(kt + (32 * tb + lr) * RB + (rd ^ (ks << 5))),
                           acc);
      float ss = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ss = fmaf(acc[r], acc[r], ss);
      ss += __shfl_xor(ss, 32);
      if (hh == 0) part[sl & 1][eb][32 * tb + lr] = ss;
    }
  }
  lds_barrier();
  if (ns > 0) finish(ns - 1);
}

}  // namespace

hipError_t launch_gram_fmap(const float* partial, int nsplit, const void* wk, const void* wv, float* gram,
                            const Shape& s, hipStream_t st, unsigned* flags) {
  const int groups = s.B * s.H * s.F;
  HA_LOG("launch gram_fmap_kernel<%d>: grid %d (sums of %d token splits, then the maps)", s.d, groups, nsplit);
  if (s.d == 128)
    gram_fmap_kernel<128><<<groups, 256, 0, st>>>(partial, nsplit, (const uint16_t*)wk, (const uint16_t*)wv,
                                                  gram, s.H, s.F, flags);
  else
    gram_fmap_kernel<64><<<groups, 128, 0, st>>>(partial, nsplit, (const uint16_t*)wk, (const uint16_t*)wv,
                                                 gram, s.H, s.F, flags);
  return hipGetLastError();
}

hipError_t launch_mfrag(const float* states, long long sbh, long long sfr, const void* wq, void* mfrag, int frames,
                        const Shape& s, hipStream_t st) {
  const int ncb = s.d / 32;
  const int groups = s.B * s.H * frames * ncb;
  HA_LOG("launch mfrag_kernel<%d>: grid %d (%d states per (b, h))", s.d, groups, frames);
  if (s.d == 128)
    mfrag_kernel<128><<<groups, 256, 0, st>>>(states, sbh, sfr, (const uint16_t*)wq, (u32x4*)mfrag, s.H, frames);
  else
    mfrag_kernel<64><<<groups, 128, 0, st>>>(states, sbh, sfr, (const uint16_t*)wq, (u32x4*)mfrag, s.H, frames);
  return hipGetLastError();
}

hipError_t launch_keyscale(const void* k, const void* wk, const float* beta, float* beta_g, float* beta_b,
                           const Shape& s, hipStream_t st) {
  const int nchunk = (s.T + 511) / 512;
  const int grid = s.B * nchunk * s.H;
  HA_LOG("launch keyscale_kernel<%d>: grid %d (512-token chunks)", s.d, grid);
  if (s.d == 128)
    keyscale_kernel<128><<<grid, 256, 0, st>>>((const uint16_t*)k, (const uint16_t*)wk, beta, beta_g, beta_b, s.H,
                                               s.T, nchunk);
  else
    keyscale_kernel<64><<<grid, 256, 0, st>>>((const uint16_t*)k, (const uint16_t*)wk, beta, beta_g, beta_b, s.H,
                                              s.T, nchunk);
  return hipGetLastError();
}

}  // namespace ha
