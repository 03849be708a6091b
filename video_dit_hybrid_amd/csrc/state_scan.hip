// Sequential part of the clean-pass state write (ARL2 section 2.1 update rule
// in affine form, one step per frame as section 2.2 prescribes):
//   S_n = alpha_n S_{n-1} - G_n S_{n-1} + B_n,   [G_n | B_n] from the gram kernel.
// Column j of S_n depends only on column j of S_{n-1}, so one work-group owns
// a 16-column block of one (b, h) state and walks the frames in order, keeping
// its block in LDS in fp32. Before step n it can copy S_{n-1} out as the
// snapshot that frame n's readout reads.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {
namespace {

constexpr int CW = 16;   // state columns per work-group
constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT) void state_scan_kernel(const float* __restrict__ gram,
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

hipError_t launch_state_scan(const float* gram, const float* alpha, float* state, float* snapshots,
                             const Shape& s, hipStream_t st) {
  const int groups = s.B * s.H * (s.d / CW);
  if (s.d == 128)
    state_scan_kernel<128><<<groups, NT, 0, st>>>(gram, alpha, state, snapshots, s.H, s.F);
  else
    state_scan_kernel<64><<<groups, NT, 0, st>>>(gram, alpha, state, snapshots, s.H, s.F);
  return hipGetLastError();
}

}  // namespace ha
