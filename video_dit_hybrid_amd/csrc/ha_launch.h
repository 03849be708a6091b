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
// hybrid_attn.h), or, when sfrag is not null, d x d bf16 readout fragments
// (the layout state_scan writes, below) at sfrag + (b*H + h)*stride_bh +
// n*stride_frame, the two strides then counted in bytes.
// mix, if not null: fp32 [B, H, 2] weights (w_softmax, w_inter) per (stream,
// head); the output is then w_softmax O/l + w_inter Q'S instead of the sum.
// Attention work-groups of a call: one per (stream, head, frame, 128-query
// tile). Launches of at most kAttnLoaderMaxGroups (one per CU) take the
// kernel with a loader wave; larger ones the kernel without it, and of those
// the forward call over several frames runs its state scan in the same launch.
constexpr int kAttnLoaderMaxGroups = 256;
inline long long attn_groups(const Shape& s) { return (long long)s.B * s.H * s.F * ((s.L + 127) / 128); }
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            const void* sfrag, void* out, const Shape& s, float scale,
                            hipStream_t st, const float* mix = nullptr);
// The forward call's state scan and its attention in one launch (bf16, F > 1):
// the first work-groups walk the frames as state_scan_mfma_kernel does (from
// the increments ws written by launch_gram_bf16, advancing state to S_F),
// publishing each S_{n-1} as readout fragments to sfrag (strides F*d*d*2 and
// d*d*2 bytes) and counting each frame's published column blocks in
// flags[(b*H + h)*F + n], which launch_gram_bf16 (or launch_gram_fmap)
// zeroed; the attention work-groups of frame n wait for that count before
// their readout. With wq (per-head maps [H][d][d] bf16) the fragments are
// those of W_q S_{n-1}, and qp is the unmapped Q.
hipError_t launch_attn_scan_bf16(const void* q, const void* k, const void* v, const void* qp, const void* ws,
                                 const float* alpha, float* state, void* sfrag, unsigned* flags, void* out,
                                 const Shape& s, float scale, hipStream_t st, const void* wq = nullptr);

// KV mode of the same kernel (the softmax teacher with a full KV cache): the
// queries of call frame n (q, out [B, T, H, d], T = F * L) attend to the keys
// [0, kv_off + (n+1) L) of k_cache, v_cache [B, Tk, H, d]; no readout. With
// nsplit > 1 the keys of each (b, h, frame) are split over nsplit work-groups
// whose partial outputs (part_o: nsplit * B * T * H * d fp32, part_ml:
// nsplit * B * T * H float2) a merge pass adds up. kv_splits gives the split
// count (shape only: equal shapes give bitwise equal results).
int kv_splits(const Shape& s, int kv_off);
// kv_off < 0 selects a one-frame window instead (keys of the query's own
// frame: the intra-frame softmax without readout); with nsplit == 1, add_o
// (fp32 [B, T, H, d], or null) is added to the output before it is rounded.
hipError_t launch_attn_kv_bf16(const void* q, const void* k_cache, const void* v_cache, void* out, float* part_o,
                               void* part_ml, int nsplit, int Tk, int kv_off, const Shape& s, float scale,
                               hipStream_t st, const float* add_o = nullptr);
// Token-level access (token_level.hip): the per-token gated delta rule in
// chunked form; writes the inter-frame output q'_t S_{t-1} (fp32 [B, T, H, d])
// to o_inter and, with update_state, the final state. d = 128 only. frag holds
// token_level_frag_bytes of per-chunk operands.
size_t token_level_frag_bytes(const Shape& s);
hipError_t launch_token_level(const void* qp, const void* kp, const void* vp, const float* alpha, const float* beta,
                              float* state, void* frag, float* o_inter, int update_state, const Shape& s,
                              hipStream_t st);
// k, v [B, T, H, d] bf16 -> the cache [B, cache_tokens, H, d] at token at_token.
hipError_t launch_kv_append(const void* k, const void* v, void* k_cache, void* v_cache, int cache_tokens,
                            int at_token, const Shape& s, hipStream_t st);

// The same on fp32 operands (fp32 FMA).
hipError_t launch_attn_fp32(const void* q, const void* k, const void* v, const void* qp,
                            const float* states, long long stride_bh, long long stride_frame,
                            void* out, const Shape& s, float scale, hipStream_t st);

// Per-frame increments G_n = K'^T diag(beta) K', B_n = K'^T diag(beta) V'.
// bf16 path workspace, per (b, h, frame): [-G hi bf16 d x d][-G lo bf16 d x d][B fp32 d x d].
// flags, if not null: B*H*F words set to zero (the counters of
// launch_attn_scan_bf16).
hipError_t launch_gram_bf16(const void* kp, const void* vp, const float* beta, float* gram,
                            const Shape& s, hipStream_t st, unsigned* flags = nullptr);
// fp32 path workspace, per (b, h, frame): [G | B] fp32 d x 2d.
// The same pass writing only fp32 partial sums (partial_block layout of
// ha_gram_format.h), nsplit token splits per (b, h, frame). With beta2 not
// null the B increments use it: G = K'^T diag(beta) K', B = K'^T diag(beta2) V'.
hipError_t launch_gram_partials_bf16(const void* kp, const void* vp, const float* beta, const float* beta2,
                                     float* partial, int nsplit, const Shape& s, hipStream_t st);
// Feature maps (fmap.hip): the increments under K' = K W_k, V' = V W_v from the
// partial sums of the unmapped K, V, written in the scan's format to gram;
// and the readout fragments of M = W_q S for `frames` states per (b, h)
// (fp32 row-major at states + (b*H + h)*sbh + n*sfr, in floats).
hipError_t launch_gram_fmap(const float* partial, int nsplit, const void* wk, const void* wv, float* gram,
                            const Shape& s, hipStream_t st, unsigned* flags = nullptr);
hipError_t launch_mfrag(const float* states, long long sbh, long long sfr, const void* wq, void* mfrag,
                        int frames, const Shape& s, hipStream_t st);
// Step sizes for L2-normalised keys (fmap.hip): with n_t = ||K_t W_k||,
// beta_g = beta / n^2 and beta_b = beta / n per (b, token, h), [B, T, H] fp32.
hipError_t launch_keyscale(const void* k, const void* wk, const float* beta, float* beta_g, float* beta_b,
                           const Shape& s, hipStream_t st);
// Headwise gate projections (gates.hip) from x [B, T, C] bf16, w_gate [2, H, C]
// bf16, b_gate [2, H] fp32: alpha [B, F, H], beta [B, T, H]; apart holds
// gates_partial_bytes of per-chunk alpha sums.
int gates_chunks(const Shape& s);
size_t gates_partial_bytes(const Shape& s);
hipError_t launch_gates(const void* x, const void* wg, const float* bg, float* alpha, float* beta, float* apart,
                        int C, const Shape& s, hipStream_t st);
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

// Token splits of the state-increment (gram) pass: one work-group per
// (stream, head, frame) leaves most of the GPU idle when there are few frames
// (one frame per call while streaming), so those calls split each frame's
// tokens over several work-groups, whose fp32 partial sums are added in split
// order by a second pass. The count depends on the shape only, so equal shapes
// always take the same path and give bitwise equal results.
constexpr int kGramTargetGroups = 256;  // about one work-group per CU
constexpr int kGramMaxSplits = 16;
inline int gram_splits(const Shape& s) {
  const long long groups = (long long)s.B * s.H * s.F;
  if (groups * 2 >= kGramTargetGroups) return 1;
  const int chunks = (s.L + 63) / 64;  // 64-token chunks per frame
  int n = (int)((kGramTargetGroups + groups - 1) / groups);
  if (n > kGramMaxSplits) n = kGramMaxSplits;
  if (n > chunks) n = chunks;
  return n < 1 ? 1 : n;
}
// per (stream, head, frame): the increments in the scan's format (d x 2d fp32
// worth of bytes), then, when split, one d x 2d fp32 partial sum per split
inline size_t gram_final_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * 2 * s.d * sizeof(float);
}
inline size_t gram_bytes(const Shape& s) {
  const int n = gram_splits(s);
  return gram_final_bytes(s) * (n > 1 ? 1 + n : 1);
}
// One-frame state write in a single kernel (state_step.hip, d = 128, F = 1):
// S_1 = alpha S_0 + K'^T diag(beta) (V' - K' S_0), the tokens of each (b, h,
// 32-column block) split over state_step_splits(s) work-groups (shape only)
// whose sums the last to finish adds up; ws holds state_step_bytes(s) bytes
// (0 when not split). snapshots, if not null, receives S_0.
int state_step_splits(const Shape& s);
size_t state_step_bytes(const Shape& s);
hipError_t launch_state_step_bf16(const void* kp, const void* vp, const float* alpha, const float* beta,
                                  float* state, float* snapshots, void* ws, const Shape& s, hipStream_t st);
// Workspace of the state update: the gram kernels' increments, or what the
// one-frame kernel needs, whichever is larger (the size query has no dtype).
inline size_t update_bytes(const Shape& s) {
  const size_t a = gram_bytes(s), b = state_step_bytes(s);
  return a > b ? a : b;
}
inline size_t snapshot_frag_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * s.d * 2;
}
inline size_t snapshot_bytes(const Shape& s) {
  return (size_t)s.B * s.H * s.F * (size_t)s.d * s.d * sizeof(float);
}

#if defined(HA_DEBUG)
// Debug words of the kernel files (bit set = an index check failed), read and
// cleared: attention, gram (state increments), scan, one-frame state write.
unsigned debug_take_attn();
unsigned debug_take_gram();
unsigned debug_take_scan();
unsigned debug_take_step();
#endif

}  // namespace ha
