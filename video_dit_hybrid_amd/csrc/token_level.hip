// Token-level access: the ablated alternative to frame-level access (ARL2,
// "Attend Locally, Remember Linearly", section 4 ablations; the canonical
// per-token gated delta rule). Per stream b and head h, tokens in order:
// token t reads S_{t-1}, the state after every earlier token, then
//   S_t = a_t S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1}),
// a_t = alpha_N at the first token of frame N, 1 elsewhere. The inter-frame
// output of token t is q'_t S_{t-1}; the intra-frame softmax is unchanged.
//
// Chunked (WY) form, chunks of 64 tokens that never cross a frame: for a chunk
// with entry state S and decay a (alpha of the frame for its first chunk,
// else 1), D = diag(1, a, .., a), c = (1, a, .., a),
//   T = (I + strict_lower(diag(beta) K K^T))^-1
//   X = T diag(beta) V - T diag(beta) D K S          (= U - W S)
//   tokens read      c_i (Q S)_i + sum_{j<i} (q_i . k_j) X_j
//   exit state       a S + K^T X
// tl_prep_kernel builds, for every chunk in parallel, the MFMA fragments of
// -W, U, P = strict_lower(Q K^T) and K^T; tl_scan_kernel walks the chunks of
// one (b, h, 32-column block of S) in order. Every fp32 operand of an MFMA is
// split into bf16 hi + lo; K, Q, V are the bf16 inputs (exact).
//
// Contraction orders: where an accumulator feeds the next MFMA as an operand,
// k-step ks of block rb uses the permuted slots 8*hh + e <-> k = 16*ks +
// 8*(e/4) + 4*hh + e%4 (hh = lane / 32), in which accumulator registers
// [8s, 8s + 8) of 32-row block rb are the operand of k-step 2*rb + s.
#include "ha_device.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

constexpr int TLD = 128;                 // head size of this path
constexpr int TLC = 64;                  // tokens per chunk
constexpr int NCH_D = TLD / 8;           // 16-byte pieces in a row of d bf16
constexpr int TILE_B = TLC * TLD * 2;    // one bf16 [64][128] tile
// per-chunk fragment block in the workspace (bytes)
constexpr int WF_B = 2 * 8 * 2 * 64 * 16;   // -W as A fragments [tb][ks over d][hi/lo][lane]
constexpr int UC_B = 2 * 4 * 64 * 64;       // U in C layout [tb][cb][lane][16 floats]
constexpr int PF_B = 2 * 4 * 2 * 64 * 16;   // P as A fragments [ib][ks over tokens][hi/lo][lane]
constexpr int KF_B = 4 * 4 * 64 * 16;       // K^T as A fragments [d block][ks over tokens][lane]
constexpr int CHUNK_B = WF_B + UC_B + PF_B + KF_B;

__device__ __forceinline__ void split8f(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const uint32_t hp = pack_bf16x2(x[2 * w2], x[2 * w2 + 1]);
    hi[w2] = hp;
    lo[w2] = pack_bf16x2(x[2 * w2] - bf16_lo_to_f32(hp), x[2 * w2 + 1] - bf16_hi_to_f32(hp));
  }
}

// bf16 tile [64][128] in LDS, 16-byte piece p of row r at r*256 + ((p ^ swz(r)) << 4)
__device__ __forceinline__ int toff(int r, int col) {
  return r * TLD * 2 + ((((col >> 3) ^ tr_swz<NCH_D>(r))) << 4) + (col & 7) * 2;
}
// natural-order transposed read: lane l gets X[16*ks + 8*hh + e][32*cb + l%32]
__device__ __forceinline__ u32x4 trn(const unsigned char* t, int ks, int cb, int lane) {
  const int gi = lane & 15, g = lane >> 4, hh = lane >> 5;
  const int r0 = 16 * ks + 8 * hh + (gi >> 2);
  const int col = 32 * cb + 16 * (g & 1) + 4 * (gi & 3);
  const u32x2 x0 = ds_read_tr16(t + toff(r0, col));
  const u32x2 x1 = ds_read_tr16(t + toff(r0 + 4, col));
  return u32x4{x0[0], x0[1], x1[0], x1[1]};
}
// natural-order row read: lane l gets X[32*tb + l%32][16*ks + 8*hh + e]
__device__ __forceinline__ u32x4 rown(const unsigned char* t, int ks, int tb, int lane) {
  const int r = 32 * tb + (lane & 31);
  return *reinterpret_cast<const u32x4*>(t + r * TLD * 2 + (((2 * ks + (lane >> 5)) ^ tr_swz<NCH_D>(r)) << 4));
}
// fp32 [64][64] in LDS, 16-byte pieces XOR-swizzled by the row
__device__ __forceinline__ int m64(int r, int c) { return r * 64 + ((((c >> 2) ^ (r & 15))) << 2) + (c & 3); }

// One work-group (4 waves) per chunk g = ((b*H + h)*F + n)*nchf + i of the
// frames' 64-token chunks.
__global__ __launch_bounds__(256) void tl_prep_kernel(const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
                                                      const uint16_t* __restrict__ vp, const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, unsigned char* __restrict__ frag,
                                                      int H, int T, int L, int F, int nchf) {
  __shared__ __align__(16) unsigned char kt[TILE_B];
  __shared__ __align__(16) unsigned char vt[TILE_B];
  __shared__ __align__(16) float am[TLC * TLC];  // strict_lower(diag(beta) K K^T), then T
  __shared__ float bs[TLC], ds[TLC];             // beta_j, beta_j * D_j
  const int g = blockIdx.x;
  const int ci = g % nchf, bhn = g / nchf;
  const int n = bhn % F, bh = bhn / F, h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = n * L + ci * TLC;                       // first token of the chunk
  const int m = L - ci * TLC < TLC ? L - ci * TLC : TLC; // tokens in the chunk
  const float dec = ci == 0 ? alpha[((size_t)b * F + n) * H + h] : 1.0f;
  const size_t rs = (size_t)H * TLD;                     // elements between tokens
  const uint16_t* kb = kp + ((size_t)b * T + t0) * rs + (size_t)h * TLD;
  const uint16_t* vb = vp + ((size_t)b * T + t0) * rs + (size_t)h * TLD;
  const uint16_t* qb = qp + ((size_t)b * T + t0) * rs + (size_t)h * TLD;

  // K, V rows into LDS (rows >= m zero); beta and beta * D
  for (int p = tid; p < TLC * NCH_D; p += 256) {
    const int r = p / NCH_D, c = p % NCH_D;
    u32x4 xk = u32x4{0, 0, 0, 0}, xv = u32x4{0, 0, 0, 0};
    if (r < m) {
      xk = ld_global_16B(kb + r * rs + c * 8);
      xv = ld_global_16B(vb + r * rs + c * 8);
    }
    *reinterpret_cast<u32x4*>(kt + r * TLD * 2 + ((c ^ tr_swz<NCH_D>(r)) << 4)) = xk;
    *reinterpret_cast<u32x4*>(vt + r * TLD * 2 + ((c ^ tr_swz<NCH_D>(r)) << 4)) = xv;
  }
  if (tid < TLC) {
    const float be = tid < m ? beta[((size_t)b * T + t0 + tid) * H + h] : 0.0f;
    bs[tid] = be;
    ds[tid] = tid == 0 ? be : be * dec;
  }
  __syncthreads();

  unsigned char* fr = frag + (size_t)g * CHUNK_B;
  u32x4* wf = reinterpret_cast<u32x4*>(fr);
  f32x4* uc = reinterpret_cast<f32x4*>(fr + WF_B);
  u32x4* pf = reinterpret_cast<u32x4*>(fr + WF_B + UC_B);
  u32x4* kf = reinterpret_cast<u32x4*>(fr + WF_B + UC_B + PF_B);

  // G = K K^T block (w/2, w%2) -> A = beta_i G_ij (j < i) into am;
  // P^T = K Q^T block (jb, ib) = (w/2, w%2), masked to j < i -> P fragments
  {
    const int rb = w >> 1, cb = w & 1;
    f32x16 gacc = f32x16{}, pacc = f32x16{};
    const int qi = 32 * cb + lr;
    const uint16_t* qrow = qb + (size_t)qi * rs;
#pragma unroll
    for (int ks = 0; ks < TLD / 16; ++ks) {
      const u32x4 ka = rown(kt, ks, rb, lane);
      const u32x4 kbb = rown(kt, ks, cb, lane);
      const u32x4 qq = qi < m ? ld_global_16B(qrow + 16 * ks + 8 * hh) : u32x4{0, 0, 0, 0};
      gacc = mfma32x32x16(ka, kbb, gacc);
      pacc = mfma32x32x16(ka, qq, pacc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);  // row of G (token i)
      const int j = 32 * cb + lr;                               // column (token j)
      am[m64(i, j)] = j < i ? bs[i] * gacc[r] : 0.0f;
      // P^T rows are key tokens j' = i, columns query tokens i' = j: keep j' < i'
      if (!(i < j)) pacc[r] = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x8[e] = pacc[8 * s + e];
      u32x4 hi, lo;
      split8f(x8, hi, lo);
      pf[((cb * 4 + 2 * rb + s) * 2 + 0) * 64 + lane] = hi;
      pf[((cb * 4 + 2 * rb + s) * 2 + 1) * 64 + lane] = lo;
    }
  }
  // K^T fragments for S += K^T X: d block w, tokens in the permuted order
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const int e0 = 2 * w2, e1 = 2 * w2 + 1;
      const int r0 = 16 * ks + 8 * (e0 >> 2) + 4 * hh + (e0 & 3);
      const int r1 = 16 * ks + 8 * (e1 >> 2) + 4 * hh + (e1 & 3);
      const int col = 32 * w + lr;
      const uint32_t lo16 = *reinterpret_cast<const uint16_t*>(kt + toff(r0, col));
      const uint32_t hi16 = *reinterpret_cast<const uint16_t*>(kt + toff(r1, col));
      f[w2] = lo16 | (hi16 << 16);
    }
    kf[(w * 4 + ks) * 64 + lane] = f;
  }
  __syncthreads();

  // T = (I + A)^-1, lower unit triangular: wave 0, lane j forward-substitutes
  // column j (four partial sums per row); then am holds T
  if (w == 0) {
    const int j = lane;
    float t[TLC];
#pragma unroll
    for (int i = 0; i < TLC; ++i) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int k = 0; k + 3 < i; k += 4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(am + m64(i, k));
        a0 = fmaf(av[0], t[k], a0);
        a1 = fmaf(av[1], t[k + 1], a1);
        a2 = fmaf(av[2], t[k + 2], a2);
        a3 = fmaf(av[3], t[k + 3], a3);
      }
#pragma unroll
      for (int k = i & ~3; k < i; ++k) a0 = fmaf(am[m64(i, k)], t[k], a0);
      t[i] = i < j ? 0.0f : (i == j ? 1.0f : -((a0 + a1) + (a2 + a3)));
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // every read of A is done before T overwrites it
#pragma unroll
    for (int i = 0; i < TLC; ++i) am[m64(i, j)] = t[i];
  }
  __syncthreads();

  // U = T diag(beta) V: wave w computes d block w for both token blocks.
  // -W^T = -(K^T (T diag(beta D))^T): wave w computes d block w.
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    f32x16 ua = f32x16{}, wa = f32x16{};
    const int i = 32 * tb + lr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int j0 = 16 * ks + 8 * hh;
      const f32x4 t0v = *reinterpret_cast<const f32x4*>(am + m64(i, j0));
      const f32x4 t1v = *reinterpret_cast<const f32x4*>(am + m64(i, j0 + 4));
      float tb8[8], td8[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tb8[e] = t0v[e] * bs[j0 + e];
        tb8[4 + e] = t1v[e] * bs[j0 + 4 + e];
        td8[e] = t0v[e] * ds[j0 + e];
        td8[4 + e] = t1v[e] * ds[j0 + 4 + e];
      }
      u32x4 bh_, bl_, dh_, dl_;
      split8f(tb8, bh_, bl_);
      split8f(td8, dh_, dl_);
      const u32x4 vv = trn(vt, ks, w, lane);  // V[j][32w + l%32]
      const u32x4 kk = trn(kt, ks, w, lane);  // K[j][32w + l%32] = K^T as A
      ua = mfma32x32x16(bh_, vv, ua);         // rows i (tokens), columns d
      ua = mfma32x32x16(bl_, vv, ua);
      wa = mfma32x32x16(kk, dh_, wa);         // rows d, columns i (tokens)
      wa = mfma32x32x16(kk, dl_, wa);
    }
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      uc[((tb * 4 + w) * 64 + lane) * 4 + v4] = f32x4{ua[4 * v4], ua[4 * v4 + 1], ua[4 * v4 + 2], ua[4 * v4 + 3]};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x8[e] = -wa[8 * s + e];
      u32x4 hi, lo;
      split8f(x8, hi, lo);
      wf[((tb * 8 + 2 * w + s) * 2 + 0) * 64 + lane] = hi;
      wf[((tb * 8 + 2 * w + s) * 2 + 1) * 64 + lane] = lo;
    }
  }
}

// One work-group (4 waves) per (b, h, 32-column block cb of S); wave w keeps
// rows [32w, 32w + 32) of the block in its accumulators over all chunks.
// Per chunk: S to LDS as split B fragments; waves 0, 1 form X = U - W S for
// token block w, waves 2, 3 Q S for token block w - 2; X to LDS as split B
// fragments; waves 2, 3 write the inter-frame output c (Q S) + P X (fp32);
// every wave advances its rows S = a S + K^T X. Two register sets of operands
// alternate between the chunks: each part of a set is reloaded with the
// operands of the chunk two ahead as soon as its chunk has used it (the
// barriers order LDS only, so those loads stay in flight).
struct TlOps {
  u32x4 big[16];  // waves 0, 1: -W fragments [ks][hi/lo]; waves 2, 3: Q [ks] then P [ks][hi/lo]
  f32x16 u;       // waves 0, 1: U block
  u32x4 kk[4];    // K^T fragments of the wave's rows
};

__global__ __launch_bounds__(256) void tl_scan_kernel(const unsigned char* __restrict__ frag,
                                                      const uint16_t* __restrict__ qp, const float* __restrict__ alpha,
                                                      float* __restrict__ state, float* __restrict__ o_inter,
                                                      int H, int T, int L, int F, int nchf, int update_state) {
  __shared__ u32x4 sfr[8][2][64];  // S[:, cb] as B fragments, k-step over d
  __shared__ u32x4 xfr[4][2][64];  // X[:, cb] as B fragments, k-step over tokens
  const int cb = blockIdx.x % 4, bh = blockIdx.x / 4;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* Sg = state + (size_t)bh * TLD * TLD;
  f32x16 S;
#pragma unroll
  for (int r = 0; r < 16; ++r) S[r] = Sg[(32 * w + 8 * (r >> 2) + 4 * hh + (r & 3)) * TLD + 32 * cb + lr];
  const size_t rs = (size_t)H * TLD;
  const int nc = F * nchf;
  const int tb = w & 1;

  // the operands of chunk c, in three parts, each loaded into a register set
  // as soon as the chunk that set serves no longer reads that part:
  // part 0, the X or Q S phase (waves 0, 1: -W and U; waves 2, 3: Q rows);
  // part 1, the output phase (waves 2, 3: P); part 2, the state advance (K^T)
  auto load = [&](int c, TlOps& o, int part) {
    const int n = c / nchf, ci = c % nchf;
    const int t0 = n * L + ci * TLC;
    const int m = L - ci * TLC < TLC ? L - ci * TLC : TLC;
    const unsigned char* fr = frag + ((size_t)bh * nc + c) * CHUNK_B;
    const u32x4* wf = reinterpret_cast<const u32x4*>(fr);
    const f32x4* uc = reinterpret_cast<const f32x4*>(fr + WF_B);
    const u32x4* pf = reinterpret_cast<const u32x4*>(fr + WF_B + UC_B);
    const u32x4* kf = reinterpret_cast<const u32x4*>(fr + WF_B + UC_B + PF_B);
    if (part == 0 && w < 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) o.big[i] = wf[((tb * 8 + (i >> 1)) * 2 + (i & 1)) * 64 + lane];
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x4 x = uc[((tb * 4 + cb) * 64 + lane) * 4 + v4];
        o.u[4 * v4] = x[0]; o.u[4 * v4 + 1] = x[1]; o.u[4 * v4 + 2] = x[2]; o.u[4 * v4 + 3] = x[3];
      }
    } else if (part == 0) {
      const int i = 32 * tb + lr;
      const uint16_t* qrow = qp + ((size_t)b * T + t0 + (i < m ? i : m - 1)) * rs + (size_t)h * TLD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {  // Q rows, d in the permuted order of the S fragments
        const int c0 = 16 * ks + 4 * hh;
        const u32x2 q0 = *reinterpret_cast<const u32x2*>(qrow + c0);
        const u32x2 q1 = *reinterpret_cast<const u32x2*>(qrow + c0 + 8);
        o.big[ks] = u32x4{q0[0], q0[1], q1[0], q1[1]};
      }
    } else if (part == 1 && w >= 2) {
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) o.big[8 + i2] = pf[((tb * 4 + (i2 >> 1)) * 2 + (i2 & 1)) * 64 + lane];
    } else if (part == 2) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) o.kk[ks] = kf[(w * 4 + ks) * 64 + lane];
    }
  };

  // chunk c on register set cur, which then takes chunk pf (pf < nc)
  auto chunk = [&](int c, TlOps& cur, int pf) {
    const int n = c / nchf, ci = c % nchf;
    const int t0 = n * L + ci * TLC;
    const int m = L - ci * TLC < TLC ? L - ci * TLC : TLC;
    const float dec = ci == 0 ? alpha[((size_t)b * F + n) * H + h] : 1.0f;

    // S -> LDS: registers [8s, 8s + 8) are the B operand of k-step 2w + s
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float x8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x8[e] = S[8 * s + e];
      u32x4 hi, lo;
      split8f(x8, hi, lo);
      sfr[2 * w + s][0][lane] = hi;
      sfr[2 * w + s][1][lane] = lo;
    }
    lds_barrier();
    f32x16 acc;
    if (w < 2) {  // X = U - W S, token block tb
      acc = cur.u;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 sh = sfr[ks][0][lane], sl = sfr[ks][1][lane];
        acc = mfma32x32x16(cur.big[2 * ks], sh, acc);
        acc = mfma32x32x16(cur.big[2 * ks], sl, acc);
        acc = mfma32x32x16(cur.big[2 * ks + 1], sh, acc);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x8[e] = acc[8 * s + e];
        u32x4 hi, lo;
        split8f(x8, hi, lo);
        xfr[2 * tb + s][0][lane] = hi;
        xfr[2 * tb + s][1][lane] = lo;
      }
    } else {  // Q S, token block tb
      acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        acc = mfma32x32x16(cur.big[ks], sfr[ks][0][lane], acc);
        acc = mfma32x32x16(cur.big[ks], sfr[ks][1][lane], acc);
      }
    }
    if (pf < nc) load(pf, cur, 0);
    lds_barrier();
    if (w >= 2) {  // out_i = c_i (Q S)_i + sum_{j<i} P_ij X_j
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * tb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (i != 0) acc[r] *= dec;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xh = xfr[ks][0][lane], xl = xfr[ks][1][lane];
        acc = mfma32x32x16(cur.big[8 + 2 * ks], xh, acc);
        acc = mfma32x32x16(cur.big[8 + 2 * ks], xl, acc);
        acc = mfma32x32x16(cur.big[8 + 2 * ks + 1], xh, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * tb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (i < m) o_inter[((size_t)b * T + t0 + i) * rs + (size_t)h * TLD + 32 * cb + lr] = acc[r];
      }
    }
    if (pf < nc) load(pf, cur, 1);
    // S rows of wave w: a S + K^T X
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] *= dec;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      S = mfma32x32x16(cur.kk[ks], xfr[ks][0][lane], S);
      S = mfma32x32x16(cur.kk[ks], xfr[ks][1][lane], S);
    }
    if (pf < nc) load(pf, cur, 2);
    lds_barrier();
  };
  TlOps o0, o1;
#pragma unroll
  for (int part = 0; part < 3; ++part) {
    load(0, o0, part);
    if (nc > 1) load(1, o1, part);
  }
  for (int c = 0; c < nc; c += 2) {
    chunk(c, o0, c + 2);
    if (c + 1 < nc) chunk(c + 1, o1, c + 3);
  }
  if (update_state) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Sg[(32 * w + 8 * (r >> 2) + 4 * hh + (r & 3)) * TLD + 32 * cb + lr] = S[r];
  }
}

}  // namespace

size_t token_level_frag_bytes(const Shape& s) {
  const int nchf = (s.L + TLC - 1) / TLC;
  return (size_t)s.B * s.H * s.F * nchf * CHUNK_B;
}

hipError_t launch_token_level(const void* qp, const void* kp, const void* vp, const float* alpha, const float* beta,
                              float* state, void* frag, float* o_inter, int update_state, const Shape& s,
                              hipStream_t st) {
  const int nchf = (s.L + TLC - 1) / TLC;
  const int nchunks = s.B * s.H * s.F * nchf;
  HA_LOG("launch tl_prep_kernel: grid %d chunks of %d tokens; tl_scan_kernel: grid %d", nchunks, TLC, s.B * s.H * 4);
  tl_prep_kernel<<<nchunks, 256, 0, st>>>((const uint16_t*)qp, (const uint16_t*)kp, (const uint16_t*)vp, alpha, beta,
                                          (unsigned char*)frag, s.H, s.T, s.L, s.F, nchf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tl_scan_kernel<<<s.B * s.H * 4, 256, 0, st>>>((const unsigned char*)frag, (const uint16_t*)qp, alpha, state,
                                                o_inter, s.H, s.T, s.L, s.F, nchf, update_state);
  return hipGetLastError();
}

}  // namespace ha
