// Host-side launch interface between the C ABI (hybrid_attn.hip) and the
// kernel translation units. Shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ha {

struct Shape {
  int B, H, T, d, L, F;  // F = T / L
};

// Intra-frame softmax + Q'S readout, bf16 operands on MFMA.
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            void* out, const Shape& s, float scale, hipStream_t st);

// The same on fp32 operands (fp32 FMA).
hipError_t launch_attn_fp32(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            void* out, const Shape& s, float scale, hipStream_t st);

// Per-frame increments G_n = K'^T diag(beta) K', B_n = K'^T diag(beta) V'.
// bf16 path workspace, per (b, h, frame): [-G hi bf16 d x d][-G lo bf16 d x d][B fp32 d x d].
hipError_t launch_gram_bf16(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st);
// fp32 path workspace, per (b, h, frame): [G | B] fp32 d x 2d.
hipError_t launch_gram_fp32(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st);

// Sequential state advance S_n = alpha_n S_{n-1} - G_n S_{n-1} + B_n over the
// frames; writes S_{n-1} to snapshots[b,h,n] when snapshots is not null.
hipError_t launch_state_scan_bf16(const void* ws, const float* alpha, float* state,
                                  float* snapshots, const Shape& s, hipStream_t st);
hipError_t launch_state_scan_fp32(const float* gram, const float* alpha, float* state,
                                  float* snapshots, const Shape& s, hipStream_t st);

inline size_t gram_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * 2 * s.d * sizeof(float);
}
inline size_t snapshot_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * s.d * sizeof(float);
}

}  // namespace ha
