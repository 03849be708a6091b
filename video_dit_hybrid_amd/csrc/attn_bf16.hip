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
// of one (b, h, frame); each wave owns 32 queries. Key/value tiles of 64 keys
// are staged in LDS (double buffered) and shared by the 4 waves.
//
// Orientation: the wave computes S^T = K Q^T (keys x queries) so that every
// lane holds 16 scores of ONE query (column l%32) per 32x32 block. The row
// max and row sum are then in-lane reductions plus one permlane32 swap, and
// the output accumulator O^T (dv x queries) of a lane also belongs to one
// query, so the softmax rescale is a per-lane scalar.
//
// Key permutation: MFMA row i of the S^T block reads physical key pi(i), pi
// swapping bits 2 and 3 of i. With it, lane half hh holds physical keys
// [16*(r/8) + 8*hh + r%8] in accumulator element r, i.e. eight CONSECUTIVE keys
// per k-step of the P V product, so P feeds the B operand of O^T += V^T P^T
// straight from registers and V^T is read from LDS as one 16-byte chunk.
//
// Online softmax in the exp2 domain with the scale folded into one FMA; the
// running max is only moved when a tile's max exceeds it by more than 8
// (log2 units), so exp2 arguments stay <= 8 and rescales of the accumulator
// are rare after the first tiles (the result is exact either way: any
// reference point common to numerator and denominator cancels).
#include "ha_device.h"
#include "ha_launch.h"

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
  static constexpr int K_TILE = KT * D * 2;  // bytes of the K tile
  static constexpr int V_TILE = D * KT * 2;  // bytes of the V^T tile
  static constexpr int BUF = K_TILE + V_TILE;
  static constexpr int SMEM = 2 * BUF;       // double buffer; also holds S^T (D*D*2)
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps over d
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int K_LD = KT * NCH / NT; // K chunks loaded per thread per tile
  static constexpr int KPT = NCH / 4;        // keys per thread in the V transpose
  static constexpr int KQN = NT / NCH;       // key groups in the V transpose
  static_assert(SMEM >= D * D * 2, "S^T must fit in the tile buffers");
  static_assert(KQN * KPT == KT, "V transpose must cover the tile");
};

__device__ __forceinline__ int pi32(int i) {  // swap bits 2 and 3
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// XOR swizzles of 16-byte chunks: rows read by 16 consecutive lanes land on
// 16 distinct chunk slots (and 8 consecutive lanes on 8), so ds_read_b128 of
// a column of chunks is free of bank conflicts for 128- and 256-byte banks.
template <int NCH>
__device__ __forceinline__ int swz_row(int i) {
  if constexpr (NCH >= 16) return i & 15;
  else return (i & 7) ^ ((i >> 3) & 1);
}

template <int D>
__device__ __forceinline__ int k_off(int row, int ch) {  // K tile [KT][D]
  return row * (D * 2) + ((ch ^ swz_row<D / 8>(pi32(row & 31))) << 4);
}
__device__ __forceinline__ int vt_off(int dv, int kc) {  // V^T tile [D][KT]
  return dv * (KT * 2) + ((kc ^ swz_row<8>(dv)) << 4);
}
template <int D>
__device__ __forceinline__ int st_off(int dv, int ch) {  // S^T [D][D]
  return dv * (D * 2) + ((ch ^ swz_row<D / 8>(dv)) << 4);
}

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ qp,
    const float* __restrict__ states, long long stride_bh, long long stride_frame,
    uint16_t* __restrict__ out, int H, int T, int L, int F, int qtiles, int n_items,
    float c2 /* softmax scale * log2(e) */) {
  using C = Cfg<D>;
  __shared__ __align__(16) unsigned char smem[C::SMEM];

  const int item = xcd_major_item(gridDim.x);
  if (item >= n_items) return;
  const int qt = item % qtiles;
  const int hf = item / qtiles;
  const int h = hf % H;
  const int n = (hf / H) % F;
  const int b = hf / (H * F);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const long long rs = (long long)H * D;  // elements between consecutive tokens
  const long long fbase = ((long long)b * T + (long long)n * L) * rs + (long long)h * D;

  const int q0 = qt * QPB + wave * QPW;
  const bool wave_active = q0 < L;
  const int my_q = q0 + lr;
  const bool q_valid = my_q < L;

  u32x4 qf[C::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks)
    qf[ks] = q_valid ? ld_global_16B(q + fbase + my_q * rs + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0};

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (L + KT - 1) / KT;
  const int vkq = tid % C::KQN, vch = tid / C::KQN;

  u32x4 kreg[C::K_LD];
  u32x4 vreg[C::KPT];
  auto load_tile = [&](int j) {
    const int key0 = j * KT;
#pragma unroll
    for (int i = 0; i < C::K_LD; ++i) {
      const int id = i * NT + tid, row = id / C::NCH, ch = id % C::NCH;
      const int key = key0 + row;
      kreg[i] = key < L ? ld_global_16B(k + fbase + key * rs + ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int key = key0 + vkq * C::KPT + i;
      vreg[i] = key < L ? ld_global_16B(v + fbase + key * rs + vch * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* kb = smem + buf * C::BUF;
    unsigned char* vb = kb + C::K_TILE;
#pragma unroll
    for (int i = 0; i < C::K_LD; ++i) {
      const int id = i * NT + tid, row = id / C::NCH, ch = id % C::NCH;
      *reinterpret_cast<u32x4*>(kb + k_off<D>(row, ch)) = kreg[i];
    }
    const int key_in = vkq * C::KPT;
    const int kc = key_in >> 3, within = (key_in & 7) * 2;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const int dv = vch * 8 + jd;
      unsigned char* dst = vb + vt_off(dv, kc) + within;
      if constexpr (C::KPT == 4) {
        const uint32_t lo = bf16_elem(vreg[0], jd) | (bf16_elem(vreg[1], jd) << 16);
        const uint32_t hi = bf16_elem(vreg[2], jd) | (bf16_elem(vreg[3], jd) << 16);
        *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = bf16_elem(vreg[0], jd) | (bf16_elem(vreg[1], jd) << 16);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int r0 = pi32(lr), r1 = 32 + pi32(lr);
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    if (wave_active) {
      const unsigned char* kb = smem + buf * C::BUF;
      const unsigned char* vb = kb + C::K_TILE;
      // S^T = K Q^T for 64 keys x 32 queries
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        const int ch = 2 * ks + hh;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(kb + k_off<D>(r0, ch));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(kb + k_off<D>(r1, ch));
        s0 = mfma32x32x16(a0, qf[ks], s0);
        s1 = mfma32x32x16(a1, qf[ks], s1);
      }
      const int nvalid = L - j * KT;
      if (nvalid < KT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 16 * (r >> 3) + 8 * hh + (r & 7);
          if (key >= nvalid) s0[r] = -INFINITY;
          if (key + 32 >= nvalid) s1[r] = -INFINITY;
        }
      }
      float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
      mt = max_across_halves(mt) * c2;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
        const float mn = fmaxf(m_run, mt);
        const float f = __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= f;
        m_run = mn;
      }
      const float nm = -m_run;
      uint32_t p0[8], p1[8];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float a = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, nm));
        const float bb = __builtin_amdgcn_exp2f(fmaf(s0[r + 1], c2, nm));
        const float cc = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, nm));
        const float dd = __builtin_amdgcn_exp2f(fmaf(s1[r + 1], c2, nm));
        ls += (a + bb) + (cc + dd);
        p0[r >> 1] = pack_bf16x2(a, bb);
        p1[r >> 1] = pack_bf16x2(cc, dd);
      }
      l_run += ls;
      // O^T += V^T P^T
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4 pb0 = {p0[4 * half], p0[4 * half + 1], p0[4 * half + 2], p0[4 * half + 3]};
        const u32x4 pb1 = {p1[4 * half], p1[4 * half + 1], p1[4 * half + 2], p1[4 * half + 3]};
        const int kc0 = 2 * half + hh, kc1 = 4 + 2 * half + hh;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int dv = db * 32 + lr;
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(vb + vt_off(dv, kc0));
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(vb + vt_off(dv, kc1));
          o[db] = mfma32x32x16(a0, pb0, o[db]);
          o[db] = mfma32x32x16(a1, pb1, o[db]);
        }
      }
    }
    if (j + 1 < ntiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: S_n -> LDS as bf16 S^T[dv][dk]; O = O / l + Q' S_n.
  const float* Sp = states + (long long)(b * H + h) * stride_bh + (long long)n * stride_frame;
  for (int p = tid; p < D * D / 8; p += NT) {
    const int dv4 = p % (D / 4), dkp = p / (D / 4);
    const int dk = 2 * dkp, dv0 = 4 * dv4;
    const f32x4 ra = *reinterpret_cast<const f32x4*>(Sp + dk * D + dv0);
    const f32x4 rb = *reinterpret_cast<const f32x4*>(Sp + (dk + 1) * D + dv0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dv = dv0 + i;
      *reinterpret_cast<uint32_t*>(smem + st_off<D>(dv, dk >> 3) + (dk & 7) * 2) = pack_bf16x2(ra[i], rb[i]);
    }
  }
  __syncthreads();
  if (!wave_active) return;

  const float inv = 1.f / sum_across_halves(l_run);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] *= inv;
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) {
    const u32x4 bq = q_valid ? ld_global_16B(qp + fbase + my_q * rs + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0};
    const int ch = 2 * ks + hh;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(smem + st_off<D>(db * 32 + lr, ch));
      o[db] = mfma32x32x16(a, bq, o[db]);
    }
  }
  if (q_valid) {
    uint16_t* op = out + fbase + my_q * rs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dv = db * 32 + 8 * g + 4 * hh;
        st_global_8B(op + dv, u32x2{pack_bf16x2(o[db][4 * g], o[db][4 * g + 1]),
                                    pack_bf16x2(o[db][4 * g + 2], o[db][4 * g + 3])});
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            void* out, const Shape& s, float scale, hipStream_t st) {
  const int qtiles = (s.L + QPB - 1) / QPB;
  const long long items = (long long)s.B * s.H * s.F * qtiles;
  const int grid = (int)((items + 7) / 8 * 8);
  const float c2 = scale * kLog2e;
  auto args = [&](auto kern) {
    kern<<<grid, NT, 0, st>>>((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                              (const uint16_t*)qp, states, stride_bh, stride_frame, (uint16_t*)out,
                              s.H, s.T, s.L, s.F, qtiles, (int)items, c2);
  };
  if (s.d == 128) args(attn_bf16_kernel<128>);
  else args(attn_bf16_kernel<64>);
  return hipGetLastError();
}

}  // namespace ha
