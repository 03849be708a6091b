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
constexpr int NW = 8;    // waves per work-group
constexpr int NT = NW * kWave;

// grid: one work-group per (b, h, frame). Waves 0-3 compute G = K'^T diag(beta)
// K', waves 4-7 compute B = K'^T diag(beta) V', each wave a 32-row band of the
// d x d result, contracting over the frame's tokens in chunks of 64.
//
// The K', V' chunks arrive row-major ([token][d] bf16, as stored) by direct
// global -> LDS loads, two chunks in flight, and beta by a 4-byte-per-lane load;
// tokens >= L are outside the buffer descriptors' range and arrive as zeros.
// Both MFMA operands need 8 consecutive tokens per lane, which transposed LDS
// reads deliver without any transposing write. The A operand beta*K' is formed
// in fp32 in registers and split into bf16 hi + lo (two MFMAs), which keeps
// ~16 mantissa bits; K' and V' themselves are exact in bf16.
//
// Output, per (b, h, frame): -G as bf16 hi + lo and B as fp32, laid out in the
// scan's MFMA fragment order (see the stores at the end).
template <int D>
__global__ __launch_bounds__(NT) void gram_bf16_kernel(const uint16_t* __restrict__ kp,
                                                       const uint16_t* __restrict__ vp,
                                                       const float* __restrict__ beta,
                                                       float* __restrict__ gram, int H, int T, int L,
                                                       int F) {
  constexpr int NCH = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = TC * D * 2;           // bytes of one K' or V' chunk
  constexpr int BUF = 2 * TILE + TC * 4;     // K', V', beta
  constexpr int SEGS = TILE / 1024;          // 1 KB direct-to-LDS segments per tile
  constexpr int RPS = 64 / NCH;              // rows per segment
  constexpr int NRB = D / 32;                // 32-row (and -column) blocks
  constexpr int NB = NRB * NRB / 4;          // output blocks per wave
  static_assert(SEGS % NW == 0 || SEGS == NW, "segment split");
  static_assert(NB == NRB || NB == 1, "a wave's blocks share one row band");
  __shared__ __align__(16) unsigned char smem[2 * BUF];

  const int hf = blockIdx.x;
  const int h = hf % H;
  const int n = (hf / H) % F;
  const int b = hf / (H * F);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int half = wave >> 2;                 // 0: G, 1: B
  const int q0 = (wave & 3) * NB;             // first block index within the half
  const int rb = q0 / NRB;                    // row band (shared by the wave's blocks)

  const uint32_t rsb = (uint32_t)H * D * 2;
  const long long fbase = ((long long)b * T + (long long)n * L) * ((long long)H * D) + (long long)h * D;
  const int span = (int)((uint32_t)(L - 1) * rsb + D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + fbase, span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + fbase, span);
  const __amdgpu_buffer_rsrc_t rbeta =
      make_rsrc(beta + ((long long)b * T + (long long)n * L) * H + h, (int)(((uint32_t)(L - 1) * H + 1) * 4));

  // direct-to-LDS: wave w fills segments w, w + NW, ... of each tile; those are
  // NW*RPS rows apart, which leaves the transposed-read swizzle unchanged.
  constexpr int MY_SEGS = SEGS / NW;
  const int srow = wave * RPS + lane / NCH, spc = lane % NCH;
  const uint32_t soff = srow * rsb + ((spc ^ tr_swz<NCH>(srow)) << 4);
  auto issue = [&](int c, int buf) {
    unsigned char* base = smem + buf * BUF;
    const uint32_t toff = (uint32_t)c * TC * rsb;
#pragma unroll
    for (int i = 0; i < MY_SEGS; ++i) {
      const uint32_t so = toff + (uint32_t)i * NW * RPS * rsb;
      dma16_to_lds(rk, base + (wave + NW * i) * 1024, soff, so);
      dma16_to_lds(rv, base + TILE + (wave + NW * i) * 1024, soff, so);
    }
    if (wave == 0) dma4_to_lds(rbeta, base + 2 * TILE, (uint32_t)lane * H * 4, (uint32_t)c * TC * H * 4);
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

  f32x16 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x16{};

  const int nch = (L + TC - 1) / TC;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) issue(c + 1, buf ^ 1);
    const unsigned char* kt = smem + buf * BUF;
    const unsigned char* bt = half ? kt + TILE : kt;
    const float* be = reinterpret_cast<const float*>(kt + 2 * TILE);
#pragma unroll
    for (int ks = 0; ks < TC / 16; ++ks) {
      // A = (beta K')^T rows 32*rb.., tokens 16*ks + 8*hh + e: split hi + lo
      const u32x4 kraw = tr8(kt, ks, rb);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(be + 16 * ks + 8 * hh);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(be + 16 * ks + 8 * hh + 4);
      u32x4 ahi, alo;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float bl = w2 < 2 ? b0[2 * w2] : b1[2 * w2 - 4];
        const float bu = w2 < 2 ? b0[2 * w2 + 1] : b1[2 * w2 - 3];
        const float x0 = bl * bf16_lo_to_f32(kraw[w2]);
        const float x1 = bu * bf16_hi_to_f32(kraw[w2]);
        const uint32_t hi = pack_bf16x2(x0, x1);
        ahi[w2] = hi;
        alo[w2] = pack_bf16x2(x0 - bf16_lo_to_f32(hi), x1 - bf16_hi_to_f32(hi));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const u32x4 bop = tr8(bt, ks, (q0 + i) % NRB);
        acc[i] = mfma32x32x16(ahi, bop, acc[i]);
        acc[i] = mfma32x32x16(alo, bop, acc[i]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Workspace per (b, h, frame), in the scan's MFMA fragment order:
  //   G hi : [band i (NRB)][k-step (D/16)][lane] 16 bytes  (8 bf16 of -G)
  //   G lo : the same for the low halves
  //   B    : [col block (NRB)][row band (NRB)][lane] 64 bytes (16 fp32)
  // G is symmetric, so the accumulator registers [8s, 8s+8) of the block
  // (row band kb, column block rb) are the scan's A fragment of -G for output
  // band rb and k-step 2*kb + s, under the contraction order in which k-slot
  // 8*hh + e of that step is k = 32*kb + 16*s + 8*(e/4) + 4*hh + e%4.
  unsigned char* base = reinterpret_cast<unsigned char*>(gram) +
                        ((size_t)(b * H + h) * F + n) * (size_t)D * D * 8;
  constexpr int KS = D / 16;
  u32x4* ghi = reinterpret_cast<u32x4*>(base);
  u32x4* glo = reinterpret_cast<u32x4*>(base + (size_t)D * D * 2);
  f32x4* bfr = reinterpret_cast<f32x4*>(base + (size_t)D * D * 4);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int cb = (q0 + i) % NRB;
    if (half) {
      f32x4* dst = bfr + ((size_t)(cb * NRB + rb) * 64 + lane) * 4;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        dst[v4] = f32x4{acc[i][4 * v4], acc[i][4 * v4 + 1], acc[i][4 * v4 + 2], acc[i][4 * v4 + 3]};
    } else {
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        u32x4 hi, lo;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float x0 = -acc[i][8 * sh + 2 * w2], x1 = -acc[i][8 * sh + 2 * w2 + 1];
          const uint32_t hp = pack_bf16x2(x0, x1);
          hi[w2] = hp;
          lo[w2] = pack_bf16x2(x0 - bf16_lo_to_f32(hp), x1 - bf16_hi_to_f32(hp));
        }
        const size_t fo = (size_t)(cb * KS + 2 * rb + sh) * 64 + lane;
        ghi[fo] = hi;
        glo[fo] = lo;
      }
    }
  }
}

}  // namespace

hipError_t launch_gram_bf16(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st) {
  const long long groups = (long long)s.B * s.H * s.F;
  if (s.d == 128)
    gram_bf16_kernel<128><<<(int)groups, NT, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, beta,
                                                      gram, s.H, s.T, s.L, s.F);
  else
    gram_bf16_kernel<64><<<(int)groups, NT, 0, st>>>((const uint16_t*)kp, (const uint16_t*)vp, beta,
                                                     gram, s.H, s.T, s.L, s.F);
  return hipGetLastError();
}

}  // namespace ha
