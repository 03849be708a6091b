// Host-side launch interface between the C ABI (hybrid_attn.hip) and the
// kernel translation units. Shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ha {

struct Shape {
  int B, H, T, d, L, F;  // F = T / L
};

// Intra-frame softmax + Q'S readout, bf16 operands on MFMA. The state of
// (b, h, frame n) is either fp32 row-major at states + b*H*stride_bh... (see
// hybrid_attn.h), or, when sfrag is not null, bf16 readout fragments at
// sfrag + ((b*H + h)*F + n) * d*d (the layout state_scan writes, below).
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            const void* sfrag, void* out, const Shape& s, float scale,
                            hipStream_t st);

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
// frames; writes S_{n-1} to snapshots[b,h,n] (fp32 row-major) when snapshots
// is not null, and as bf16 readout fragments to sfrag when that is not null:
// per (b, h, frame) [column block (d/32)][k-step (d/16)][lane] 16 bytes, the
// MFMA A operand of O^T += S^T Q'^T for output rows 32*cb + lane%32 and
// contraction slots 8*(lane/32) + e <-> dk = 16*ks + 8*(e/4) + 4*(lane/32) + e%4.
hipError_t launch_state_scan_bf16(const void* ws, const float* alpha, float* state,
                                  float* snapshots, void* sfrag, const Shape& s, hipStream_t st);
hipError_t launch_state_scan_fp32(const float* gram, const float* alpha, float* state,
                                  float* snapshots, const Shape& s, hipStream_t st);

inline size_t gram_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * 2 * s.d * sizeof(float);
}
inline size_t snapshot_frag_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * s.d * 2;
}
inline size_t snapshot_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * s.d * sizeof(float);
}

}  // namespace ha
