// Headwise gate projections (ARL2, "Attend Locally, Remember Linearly",
// section 2.1: the forget gate alpha and the step size beta are learned
// per-token projections; the ablations favour one gate per head). Per token t
// of stream b and head h, from the layer input x_t (C channels):
//   a_t = sigmoid(x_t . w_gate[0][h] + b_gate[0][h])
//   g_t = sigmoid(x_t . w_gate[1][h] + b_gate[1][h])
// The state is written once per frame, so frame N gets one forget gate, the
// mean of its tokens' a_t; beta_t = g_t / L.
//
// The projection is a [tokens x C] x [C x 2H] product on MFMA, the 2H gate
// rows as the A operand and 32 tokens as the B operand columns. The pass is
// bound by the HBM read of x (2 bytes per token and channel); the weights
// (2H x C bf16) stay in L2.
#include "ha_device.h"
#include "ha_dma.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {
namespace {

constexpr int GT = 64;          // tokens per work-group
constexpr int SC = 64;          // channels per LDS slice
constexpr int ROWB = SC * 2;    // bytes of one row's slice (8 chunks of 16 bytes)
constexpr int RPC = 1024 / ROWB;  // rows per 1 KB copy

// LDS position of chunk c of slice row r: c ^ gswz(r). Sixteen consecutive rows
// (one LDS cycle of 16-byte reads) then cover all 64 banks: rows of equal
// parity share bank lines and get distinct positions.
__device__ __forceinline__ int gswz(int row) { return (row >> 1) & 7; }

// One work-group (4 waves) per (b, frame, 64-token chunk of the frame). The
// chunk's x rows and the gate rows are streamed through LDS in slices of 64
// channels: direct global -> LDS copies of 1 KB per wave instruction, each
// covering 8 rows x 128 contiguous bytes (whole cache lines), two slices in
// flight while a third is read (deeper pipelines measured no faster); the
// small slices keep the LDS footprint at four work-groups per CU, so a 480p
// launch (525 work-groups) runs in one round. In LDS a slice
// is [row][8 chunks of 16 bytes] with chunk c of row r at position
// c ^ gswz(r). Wave w takes k-step w of every slice for both 32-token column
// blocks and all gate-row blocks; the four partial logit blocks are added through LDS
// in wave order. x rows past the frame end and gate rows past 2H lie outside
// their buffer descriptors and arrive as zeros. Outputs: beta for the chunk's
// tokens, and the chunk's sum of alpha gates per head (apart, added up per
// frame by alpha_kernel).
template <int NOB>
__global__ __launch_bounds__(256) void gates_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wg,
                                                    const float* __restrict__ bg, float* __restrict__ beta,
                                                    float* __restrict__ apart, int T, int C, int H, int L,
                                                    int F, int nch) {
  constexpr int NBUF = 3;                     // slices in flight + 1
  constexpr int XT = GT * ROWB;               // x bytes of a slice
  constexpr int WT = 32 * NOB * ROWB;         // gate-row bytes of a slice
  constexpr int BUF = XT + WT;
  constexpr int XSEG = XT / 1024 / 4;         // 1 KB copies per wave per slice: x
  constexpr int WSEG = WT / 1024 / 4;         // and gate rows
  constexpr int PER = XSEG + WSEG;
  static_assert((NBUF - 2) * PER <= 15, "vmcnt immediate");
  static_assert(SC / 16 == 4, "one k-step per wave and slice");
  constexpr int RED = 4 * NOB * 2 * 16 * 64 * 4;  // partial logits of the 4 waves
  constexpr int SMEM = NBUF * BUF > RED ? NBUF * BUF : RED;
  __shared__ __align__(16) unsigned char smem[SMEM];
  __shared__ float sa[16 * NOB][GT];
  const int blk = blockIdx.x;
  const int c = blk % nch, bn = blk / nch;
  const int n = bn % F, b = bn / F;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int O = 2 * H;
  const int rows = L - c * GT < GT ? L - c * GT : GT;
  const u32x4 rx = rsrc_words(x + ((size_t)b * T + (size_t)n * L + (size_t)c * GT) * C, rows * C * 2);
  const u32x4 rw = rsrc_words(wg, O * C * 2);
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_ptr(smem));

  // copy s (rows 8s .. 8s + 7) of a slice: lane l fills position l % 8 of
  // row 8s + l / 8; wave w issues copies w, w + 4, ..., whose rows have the
  // same gswz for a given lane, so the per-lane offset is fixed
  const int crow = RPC * (w & 1) + (lane >> 3);
  const uint32_t voff = (uint32_t)(lane >> 3) * C * 2 + (uint32_t)(((lane & 7) ^ gswz(crow)) << 4);
  auto issue = [&](int k, int buf) {
    const uint32_t base = lds0 + buf * BUF;
    const uint32_t ko = (uint32_t)k * ROWB;
#pragma unroll
    for (int i = 0; i < XSEG; ++i) {
      const int sg = w + 4 * i;
      dma16_asm(rx, base + sg * 1024, voff, (uint32_t)(RPC * sg) * C * 2 + ko);
    }
#pragma unroll
    for (int i = 0; i < WSEG; ++i) {
      const int sg = w + 4 * i;
      dma16_asm(rw, base + XT + sg * 1024, voff, (uint32_t)(RPC * sg) * C * 2 + ko);
    }
  };

  f32x16 acc[NOB][2];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) acc[ob][0] = acc[ob][1] = f32x16{};
  const int ns = (C + SC - 1) / SC;
  const int rd = (hh ^ gswz(lr)) << 4;  // chunk 2ks + hh of row 32tb + lr: rd ^ (ks << 5)
  for (int k = 0; k < NBUF - 1 && k < ns; ++k) issue(k, k);
  for (int k = 0; k < ns; ++k) {
    // slice k landed: at most the copies of the slices after it are outstanding
    wait_later_copies<NBUF - 2, PER>(ns - 1 - k);
    lds_barrier();  // every wave's copies of slice k are in LDS; slice k-1 is consumed
    if (k + NBUF - 1 < ns) issue(k + NBUF - 1, (k + NBUF - 1) % NBUF);
    const unsigned char* xs = smem + (k % NBUF) * BUF;
    const unsigned char* wsl = xs + XT;
    const int kv = (C - k * SC < SC ? C - k * SC : SC) / 16;  // k-steps of this slice
    {
      const int ks = w;
      if (ks < kv) {
        const int off = rd ^ (ks << 5);
        u32x4 bx[2], aw[NOB];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) bx[tb] = *reinterpret_cast<const u32x4*>(xs + (32 * tb + lr) * ROWB + off);
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) aw[ob] = *reinterpret_cast<const u32x4*>(wsl + (32 * ob + lr) * ROWB + off);
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) acc[ob][tb] = mfma32x32x16(aw[ob], bx[tb], acc[ob][tb]);
      }
    }
  }
  lds_barrier();  // the slice buffers are free: they hold the partial logits next
  float* red = reinterpret_cast<float*>(smem);
  auto ridx = [&](int wv, int ob, int tb, int r, int ln) { return (((wv * NOB + ob) * 2 + tb) * 16 + r) * 64 + ln; };
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[ridx(w, ob, tb, r, lane)] = acc[ob][tb][r];
  lds_barrier();

  // logit (o, t) sits in register r = 4*(oo/8) + oo%4 of lane t%32 + 32*((oo/4)%2)
  // of block (o / 32, t / 32), oo = o % 32
  for (int idx = tid; idx < O * GT; idx += 256) {
    const int o = idx / GT, t = idx % GT;
    const int ob = o >> 5, oo = o & 31, tb = t >> 5;
    const int r = ((oo >> 3) << 2) | (oo & 3);
    const int ln = (t & 31) + 32 * ((oo >> 2) & 1);
    const float z = red[ridx(0, ob, tb, r, ln)] + red[ridx(1, ob, tb, r, ln)] + red[ridx(2, ob, tb, r, ln)] +
                    red[ridx(3, ob, tb, r, ln)] + bg[o];
    const float gsig = 1.0f / (1.0f + expf(-z));
    const bool valid = t < rows;
    if (o >= H) {
      if (valid) beta[((size_t)b * T + (size_t)n * L + c * GT + t) * H + (o - H)] = gsig / (float)L;
    } else {
      sa[o][t] = valid ? gsig : 0.0f;
    }
  }
  __syncthreads();
  for (int h = tid; h < H; h += 256) {
    float s = 0.0f;
#pragma unroll 16
    for (int t = 0; t < GT; ++t) s += sa[h][t];
    apart[((size_t)bn * nch + c) * H + h] = s;
  }
}

// alpha[b, n, h] = (sum of the frame's chunk sums) / L: one wave per (b, n, h),
// lane l adds chunks l, l + 64, ... and a butterfly over the 64 lanes adds
// those (an order fixed by the shape).
__global__ __launch_bounds__(256) void alpha_kernel(const float* __restrict__ apart, float* __restrict__ alpha,
                                                    int nch, int H, int total, int L) {
  const int wv = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wv >= total) return;
  const int bn = wv / H, h = wv % H;
  float s = 0.0f;
  for (int c = lane; c < nch; c += 64) s += apart[((size_t)bn * nch + c) * H + h];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) alpha[wv] = s / (float)L;
}

}  // namespace

int gates_chunks(const Shape& s) { return (s.L + GT - 1) / GT; }

size_t gates_partial_bytes(const Shape& s) {
  return (size_t)s.B * s.F * gates_chunks(s) * s.H * sizeof(float);
}

hipError_t launch_gates(const void* x, const void* wg, const float* bg, float* alpha, float* beta, float* apart,
                        int C, const Shape& s, hipStream_t st) {
  const int nch = gates_chunks(s);
  const int grid = s.B * s.F * nch;
  const int nob = (2 * s.H + 31) / 32;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)wg;
  HA_LOG("launch gates_kernel<%d>: grid %d (%d 64-token chunks per frame, C = %d) + alpha_kernel", nob, grid, nch, C);
  switch (nob) {
    case 1: gates_kernel<1><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    case 2: gates_kernel<2><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    case 3: gates_kernel<3><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    case 4: gates_kernel<4><<<grid, 256, 0, st>>>(xp, wp, bg, beta, apart, s.T, C, s.H, s.L, s.F, nch); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = s.B * s.F * s.H;
  alpha_kernel<<<(total + 3) / 4, 256, 0, st>>>(apart, alpha, nch, s.H, total, s.L);
  return hipGetLastError();
}

}  // namespace ha
