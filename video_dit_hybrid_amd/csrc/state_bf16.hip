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
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {
namespace {

constexpr int TC = 64;   // tokens per LDS chunk
constexpr int NT = 256;  // threads per work-group

__device__ __forceinline__ int swz8(int i) { return (i & 7) ^ ((i >> 3) & 1); }
// [D rows][TC tokens] bf16, 16-byte chunks of 8 tokens, XOR-swizzled by row.
__device__ __forceinline__ int tt_off(int row, int kc) { return row * (TC * 2) + ((kc ^ swz8(row)) << 4); }

// grid: B*H*F*2 work-groups; work-group (hf, half) computes G (half 0) or B
// (half 1) for one (b, h, frame), contracting over the frame's tokens. G is
// stored negated and split into bf16 hi + lo planes, ready to be the A
// operand of the scan's MFMA; B is stored in fp32.
template <int D>
__global__ __launch_bounds__(NT, 2) void gram_bf16_kernel(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const float* __restrict__ beta, float* __restrict__ gram, int H, int T, int L, int F) {
  constexpr int NCH = D / 8;        // 16-byte chunks in a row of D bf16
  constexpr int KPT = NCH / 4;      // tokens per thread in the transposing load
  constexpr int KQN = NT / NCH;     // token groups
  constexpr int RB = D / 32;        // 32-row blocks of the output
  constexpr int NBLK = RB * RB / 4; // output blocks per wave
  constexpr int TILE = D * TC * 2;  // bytes of one transposed operand tile
  static_assert(KQN * KPT == TC, "transpose must cover the chunk");
  __shared__ __align__(16) unsigned char smem[3 * TILE];
  unsigned char* a_hi = smem;
  unsigned char* a_lo = smem + TILE;
  unsigned char* b_t = smem + 2 * TILE;

  const int half = blockIdx.x & 1;
  const int hf = blockIdx.x >> 1;
  const int h = hf % H;
  const int n = (hf / H) % F;
  const int b = hf / (H * F);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;
  const long long rs = (long long)H * D;
  const long long fbase = ((long long)b * T + (long long)n * L) * rs + (long long)h * D;
  const float* bbase = beta + ((long long)b * T + (long long)n * L) * H + h;
  const uint16_t* src_b = half ? vp : kp;

  const int tq = tid % KQN, tch = tid / KQN;

  f32x16 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i) acc[i] = f32x16{};

  for (int t0 = 0; t0 < L; t0 += TC) {
    u32x4 kr[KPT], br[KPT];
    float be[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int t = t0 + tq * KPT + i;
      const bool ok = t < L;
      kr[i] = ok ? ld_global_16B(kp + fbase + t * rs + tch * 8) : u32x4{0, 0, 0, 0};
      br[i] = ok ? (half ? ld_global_16B(src_b + fbase + t * rs + tch * 8) : kr[i]) : u32x4{0, 0, 0, 0};
      be[i] = ok ? bbase[(long long)t * H] : 0.f;
    }
    __syncthreads();  // previous chunk's operand reads are done
    const int tin = tq * KPT, kc = tin >> 3, within = (tin & 7) * 2;
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const int row = tch * 8 + jd;
      uint32_t wb[KPT / 2], wh[KPT / 2], wl[KPT / 2];
#pragma unroll
      for (int i = 0; i < KPT; i += 2) {
        wb[i / 2] = bf16_elem(br[i], jd) | (bf16_elem(br[i + 1], jd) << 16);
        const float x0 = be[i] * __uint_as_float(bf16_elem(kr[i], jd) << 16);
        const float x1 = be[i + 1] * __uint_as_float(bf16_elem(kr[i + 1], jd) << 16);
        const uint32_t hi = pack_bf16x2(x0, x1);
        wh[i / 2] = hi;
        wl[i / 2] = pack_bf16x2(x0 - bf16_lo_to_f32(hi), x1 - bf16_hi_to_f32(hi));
      }
      const int off = tt_off(row, kc) + within;
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2*>(b_t + off) = u32x2{wb[0], wb[1]};
        *reinterpret_cast<u32x2*>(a_hi + off) = u32x2{wh[0], wh[1]};
        *reinterpret_cast<u32x2*>(a_lo + off) = u32x2{wl[0], wl[1]};
      } else {
        *reinterpret_cast<uint32_t*>(b_t + off) = wb[0];
        *reinterpret_cast<uint32_t*>(a_hi + off) = wh[0];
        *reinterpret_cast<uint32_t*>(a_lo + off) = wl[0];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TC / 16; ++ks) {
      const int kcr = 2 * ks + hh;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const int id = wave * NBLK + blk;
        const int rb = id / RB, cb = id % RB;
        const int ra = rb * 32 + lr, rbt = cb * 32 + lr;
        const u32x4 ah = *reinterpret_cast<const u32x4*>(a_hi + tt_off(ra, kcr));
        const u32x4 al = *reinterpret_cast<const u32x4*>(a_lo + tt_off(ra, kcr));
        const u32x4 bt = *reinterpret_cast<const u32x4*>(b_t + tt_off(rbt, kcr));
        acc[blk] = mfma32x32x16(ah, bt, acc[blk]);
        acc[blk] = mfma32x32x16(al, bt, acc[blk]);
      }
    }
  }

  // workspace per (b, h, frame): [-G hi: D x D bf16][-G lo: D x D bf16][B: D x D fp32]
  unsigned char* base = reinterpret_cast<unsigned char*>(gram) +
                        ((size_t)(b * H + h) * F + n) * (size_t)D * D * 8;
  uint16_t* gh = reinterpret_cast<uint16_t*>(base);
  uint16_t* gl = gh + (size_t)D * D;
  float* bo = reinterpret_cast<float*>(base + (size_t)D * D * 4);
#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
    const int id = wave * NBLK + blk;
    const int rb = id / RB, cb = id % RB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = rb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const size_t o = (size_t)i * D + cb * 32 + lr;
      if (half) {
        bo[o] = acc[blk][r];
      } else {
        const float x = -acc[blk][r];
        const uint32_t hi = pack_bf16x2(x, 0.f) & 0xffffu;
        gh[o] = (uint16_t)hi;
        gl[o] = (uint16_t)(pack_bf16x2(x - __uint_as_float(hi << 16), 0.f) & 0xffffu);
      }
    }
  }
}

}  // namespace

hipError_t launch_gram_bf16(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st) {
  const long long groups = (long long)s.B * s.H * s.F * 2;
  if (s.d == 128)
    gram_bf16_kernel<128><<<(int)groups, NT, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, beta,
                                                      gram, s.H, s.T, s.L, s.F);
  else
    gram_bf16_kernel<64><<<(int)groups, NT, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, beta,
                                                     gram, s.H, s.T, s.L, s.F);
  return hipGetLastError();
}

}  // namespace ha
