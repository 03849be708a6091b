/*
 * hybrid_attn.h - C ABI of the MI355X (gfx950) hybrid attention layer.
 *
 * The layer is the ARL2 hybrid attention of an autoregressive video diffusion
 * transformer ("Attend Locally, Remember Linearly", arXiv 2605.16579,
 * section 2.1 "hybrid attention decomposition" and section 2.2 "state
 * management"). Per stream b and head h, frame N (tokens [N*L, (N+1)*L)):
 *
 *   O_N   = softmax(Q_N K_N^T * s) V_N  +  Q'_N S_{N-1}           (2.1)
 *   S_N   = alpha_N S_{N-1} + K'_N^T diag(beta_N) (V'_N - K'_N S_{N-1})  (2.1)
 *
 * The softmax runs among the L tokens of the frame only, in both directions
 * (2.1 item 1); the two branches are summed; every token of frame N reads the
 * same pre-update state S_{N-1} and the state is written only after the whole
 * frame, and only on the clean pass (2.2).
 *
 * Layouts (all row-major, last index contiguous):
 *   q, k, v, qp, kp, vp, out : [B, T, H, d]   T = F * frame_len
 *   alpha                    : [B, F, H]      fp32
 *   beta                     : [B, T, H]      fp32
 *   state                    : [B, H, d, d]   fp32, state[b][h][dk][dv]
 * q..vp and out are bf16 (HA_BF16) or fp32 (HA_FP32); state is always fp32.
 *
 * Ownership: every pointer is device memory owned by the caller (for example
 * allocated through PyTorch). The library allocates nothing and keeps no
 * state between calls; scratch space is the caller's workspace argument.
 *
 * Execution: calls are asynchronous on the given HIP stream (a hipStream_t
 * passed as void*; NULL is the default stream). A call returns after
 * enqueueing its kernels. Argument errors are returned before any device
 * work is enqueued and leave every buffer untouched; a failed launch returns
 * HA_ERR_DEVICE; a fault inside a kernel surfaces at the caller's next
 * synchronisation. Calls are reentrant: there is no global mutable state.
 * Two calls that share a state or workspace buffer must be ordered by the
 * caller (for example by issuing them on one stream).
 */
#ifndef HYBRID_ATTN_H
#define HYBRID_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums below have int as their fixed underlying type, so every
 * int a C caller passes is a valid value (C enums are ints already). */
#ifdef __cplusplus
#define HA_ENUM_INT : int
#else
#define HA_ENUM_INT
#endif

typedef enum HA_ENUM_INT {
  HA_BF16 = 0, /* q..vp and out are bfloat16 */
  HA_FP32 = 1  /* q..vp and out are float32 */
} ha_dtype;

typedef enum HA_ENUM_INT {
  HA_OK = 0,
  HA_ERR_NULL = 1,        /* a required pointer is NULL */
  HA_ERR_SHAPE = 2,       /* a size <= 0, T % frame_len != 0, or a size too large to index */
  HA_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, or an unknown dtype */
  HA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned (alpha, beta: 4-byte) */
  HA_ERR_WORKSPACE = 5,   /* workspace is NULL or smaller than the size the query returns */
  HA_ERR_DEVICE = 6,      /* a kernel launch failed */
  HA_ERR_ALIAS = 7,       /* a buffer the call writes (out, state, snapshots, workspace)
                             overlaps another buffer of the call */
  HA_ERR_SCRATCH = 8,     /* the call needs more workspace than hybrid_attn_forward_noalloc's
                             fixed scratch holds (hybrid_attn_noalloc_scratch_bytes) */
  HA_ERR_NONFINITE = 9    /* only with HA_CHECK_FINITE set: the state holds Inf or NaN after
                             the call */
} ha_status;

/*
 * Diagnostics, read from the environment at every call (any value other than
 * empty or "0" switches one on):
 *   HA_LOG           one line on stderr per call (sizes, workspace) and per
 *                    kernel launch (grid, block, tiling).
 *   HA_CHECK_FINITE  after every call that writes the state, a scan of it for
 *                    Inf or NaN; the call then synchronises its stream and
 *                    returns HA_ERR_NONFINITE if it finds one. This makes the
 *                    call synchronous; not for use under HIP graph capture.
 */

/*
 * Bytes of workspace hybrid_attn_forward needs for these sizes: 0 when
 * update_state is 0; otherwise the per-frame state increments (d x 2d fp32 per
 * stream, head and frame) plus, when T / frame_len > 1, the per-frame
 * pre-update states S_{N-1} (d x d fp32 each). A call with fewer than 128
 * (stream, head, frame) groups computes each frame's increments in
 * n = min(ceil(256 / groups), 16, ceil(frame_len / 64)) token splits and needs n
 * more d x 2d fp32 blocks per group for their partial sums. A bf16 call with
 * one frame and d = 128 writes the state in one kernel instead, whose u =
 * B * H * 4 (stream, head, 32-column) units split their tokens over
 * m = min(floor(256 / u), floor(ceil(frame_len / 32) / 8), 16) work-groups and,
 * when m > 1, need u * m * 16 KiB of partial sums plus 8 bytes per unit (each
 * rounded up to 256 bytes); the size returned is the larger of the two (the
 * query has no dtype). The size depends on the arguments only. Returns 0 for
 * invalid sizes.
 */
size_t hybrid_attn_workspace_bytes(int B, int H, int T, int frame_len, int d,
                                   int update_state);

/*
 * The whole layer call (ARL2 2.1 and 2.2).
 *   q, k, v      intra-frame branch inputs (the frozen softmax projections)
 *   qp, kp, vp   inter-frame branch inputs Q', K', V' (after the feature maps)
 *   alpha        forget gate per (stream, frame, head), read if update_state
 *   beta         step size per (stream, token, head), read if update_state
 *   state        S in/out: frame 0 reads it; with update_state != 0 it is
 *                overwritten with S_F after the last frame, otherwise it is
 *                left bitwise unchanged and every frame reads it
 *   out          O, written in full
 *   workspace    caller scratch of at least hybrid_attn_workspace_bytes(...)
 *   softmax_scale  s; a value <= 0 selects 1/sqrt(d)
 * When update_state is 0, kp, vp, alpha, beta and workspace may be NULL.
 * HA_ERR_ALIAS: out overlaps an input, the state or the workspace; or, with
 * update_state != 0, the state or the workspace overlaps an input or each
 * other (the workspace counted for the bytes the size query returns).
 */
ha_status hybrid_attn_forward(const void* q, const void* k, const void* v,
                              const void* qp, const void* kp, const void* vp,
                              const float* alpha, const float* beta,
                              float* state, void* out,
                              void* workspace, size_t workspace_bytes,
                              int B, int H, int T, int d, int frame_len,
                              ha_dtype dtype, int update_state,
                              float softmax_scale, void* stream);

/*
 * hybrid_attn_forward with a weight on each branch's output: for stream b and
 * head h, O = w_softmax O_intra + w_inter O_inter with (w_softmax, w_inter) =
 * (mix[2 (b H + h)], mix[2 (b H + h) + 1]) for every frame of the call. The
 * pages' mixtures of a softmax and a linear branch are such pairs: LinVideo's
 * selective transfer ("LinVideo" page: o = r SoftmaxAttn + (1 - r) LinearAttn,
 * a learned r in [0, 1] per layer) is (r, 1 - r); SALAD's input- and
 * timestep-aware scale on the linear branch ("SALAD" page, ITADS: s in (0, 1)
 * through a sigmoid) is (1, s). The weights touch the output only; the state
 * update is that of hybrid_attn_forward.
 *   mix   fp32 [B, H, 2], device memory, 8-byte aligned; required (NULL gives
 *         HA_ERR_NULL). Read only.
 * Other arguments, workspace and errors as hybrid_attn_forward; bf16 only
 * (HA_ERR_UNSUPPORTED for fp32); HA_ERR_ALIAS also when out overlaps mix.
 */
ha_status hybrid_attn_forward_mix(const void* q, const void* k, const void* v,
                                  const void* qp, const void* kp, const void* vp,
                                  const float* alpha, const float* beta,
                                  float* state, void* out, const float* mix,
                                  void* workspace, size_t workspace_bytes,
                                  int B, int H, int T, int d, int frame_len,
                                  ha_dtype dtype, int update_state,
                                  float softmax_scale, void* stream);

/*
 * hybrid_attn_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Arguments,
 * results and errors are those of hybrid_attn_forward without the workspace:
 * the call uses a fixed scratch array inside this library instead, of
 * hybrid_attn_noalloc_scratch_bytes() bytes (64 MiB) on each GPU it runs on,
 * held until the process ends. Calls whose workspace (the size
 * hybrid_attn_workspace_bytes returns) exceeds it fail with HA_ERR_SCRATCH
 * before any device work. The call allocates nothing and clears nothing (every
 * scratch byte a call reads it has written first). All calls on one GPU share
 * that GPU's scratch: two calls that overlap in time on one GPU (different
 * streams, or different host threads without ordering) race and give wrong
 * results; issue them on one stream. The stream must belong to the current
 * device. HA_ERR_DEVICE also when the scratch address cannot be obtained.
 */
ha_status hybrid_attn_forward_noalloc(const void* q, const void* k, const void* v,
                                      const void* qp, const void* kp, const void* vp,
                                      const float* alpha, const float* beta,
                                      float* state, void* out,
                                      int B, int H, int T, int d, int frame_len,
                                      ha_dtype dtype, int update_state,
                                      float softmax_scale, void* stream);

/* Bytes of scratch hybrid_attn_forward_noalloc holds per GPU. */
size_t hybrid_attn_noalloc_scratch_bytes(void);

/*
 * The read side alone (ARL2 2.1 intra-frame branch plus the Q'S readout,
 * 2.2 frame-level access): out = softmax-within-frame(Q K^T s) V + Q' S_n for
 * every frame n, where S_n of stream b and head h is the fp32 d x d matrix at
 *   states + (b*H + h)*state_stride_bh + n*state_stride_frame   (in floats).
 * With state_stride_frame = 0 every frame reads the same state (a denoising
 * pass). Both strides are multiples of 4 floats (HA_ERR_ALIGN otherwise).
 * Nothing but out is written; out must not overlap q, k, v, qp or the
 * states (HA_ERR_ALIAS).
 */
ha_status hybrid_attn_intra_readout(const void* q, const void* k,
                                    const void* v, const void* qp,
                                    const float* states,
                                    long long state_stride_bh,
                                    long long state_stride_frame, void* out,
                                    int B, int H, int T, int d, int frame_len,
                                    ha_dtype dtype, float softmax_scale,
                                    void* stream);

/*
 * Bytes of workspace hybrid_attn_state_update needs: the per-frame state
 * increments, B*H*F*d*2d fp32, plus the token-split partial sums under the
 * same rule as hybrid_attn_workspace_bytes. Returns 0 for invalid sizes.
 */
size_t hybrid_attn_state_workspace_bytes(int B, int H, int T, int frame_len,
                                         int d);

/*
 * The write side alone (ARL2 2.1 update rule, applied once per clean frame as
 * 2.2 prescribes): state <- S_F after frames 0..F-1 of kp, vp, alpha, beta.
 * If snapshots is not NULL it receives S_{n-1} for every frame n, laid out
 * [B, H, F, d, d] fp32 (snapshot n of frame 0 is the input state).
 * HA_ERR_ALIAS: state, snapshots or the workspace (counted for the bytes the
 * size query returns) overlaps kp, vp, alpha, beta or one another.
 */
ha_status hybrid_attn_state_update(const void* kp, const void* vp,
                                   const float* alpha, const float* beta,
                                   float* state, float* snapshots,
                                   void* workspace, size_t workspace_bytes,
                                   int B, int H, int T, int d, int frame_len,
                                   ha_dtype dtype, void* stream);

/*
 * Bytes of workspace hybrid_attn_forward_fmap needs (always at least the
 * readout fragments): with update_state = 0, d x d bf16 per (stream, head);
 * otherwise per (stream, head, frame) the state increments (d x 2d fp32), the
 * fp32 partial sums of n token splits (n as for hybrid_attn_workspace_bytes,
 * at least 1; d x 2d fp32 each), the pre-update state S_{N-1} (d x d fp32),
 * its readout fragments (d x d bf16) and a 4-byte frame counter, each region
 * 256-byte aligned. Returns 0 for invalid sizes.
 */
size_t hybrid_attn_fmap_workspace_bytes(int B, int H, int T, int frame_len, int d,
                                        int update_state);

/*
 * The layer with the inter-frame branch's feature maps applied inside the
 * call (ARL2 2.1, "adaptation": grouped per-head 1x1 maps phi_q, phi_k, phi_v
 * of the frozen projections' Q, K, V), taken as one d x d linear map per head:
 *   Q' = Q W_q, K' = K W_k, V' = V W_v  (row vectors; no bias, no nonlinearity)
 * and otherwise exactly hybrid_attn_forward with those Q', K', V'. Q', K', V'
 * are never formed: the readout uses Q (W_q S_{N-1}) and the state update the
 * increments W_k^T G0 W_k and W_k^T B0 W_v of the unmapped K, V.
 *   wq, wk, wv   [H, d, d] bf16, map of head h at w + h*d*d, row-major
 *                (entry [j][e] multiplies input channel j into output e)
 *   workspace    at least hybrid_attn_fmap_workspace_bytes(...); required
 *                also when update_state is 0
 * bf16 only (HA_ERR_UNSUPPORTED for HA_FP32). When update_state is 0, wk, wv,
 * alpha and beta may be NULL. Other arguments, errors and stream behaviour
 * as for hybrid_attn_forward.
 */
ha_status hybrid_attn_forward_fmap(const void* q, const void* k, const void* v,
                                   const void* wq, const void* wk, const void* wv,
                                   const float* alpha, const float* beta,
                                   float* state, void* out,
                                   void* workspace, size_t workspace_bytes,
                                   int B, int H, int T, int d, int frame_len,
                                   ha_dtype dtype, int update_state,
                                   float softmax_scale, void* stream);

/*
 * Bytes of workspace hybrid_attn_forward_gated needs: with update_state 0 the
 * same as hybrid_attn_fmap_workspace_bytes; with update_state 1 that layout
 * followed by beta, beta / n^2 and beta / n ([B, T, H] fp32 each), the
 * per-chunk alpha sums of the gate pass and alpha ([B, F, H] fp32), each
 * region 256-byte aligned. Returns 0 for invalid sizes.
 */
size_t hybrid_attn_gated_workspace_bytes(int B, int H, int T, int frame_len, int d,
                                         int update_state);

/*
 * The layer from the inputs a transformer block holds: the gates come from
 * the layer input x and the feature maps are applied inside the call.
 * ARL2 2.1: alpha (forget gate) and beta (step size) are learned per-token
 * projections, one per head (headwise gating, ablations of section 4); read
 * here, per token t and head h, as
 *   a_t = sigmoid(x_t . w_gate[0][h] + b_gate[0][h]),
 *   g_t = sigmoid(x_t . w_gate[1][h] + b_gate[1][h]),
 * alpha_N = the mean of a_t over the L tokens of frame N (the state is written
 * once per frame), beta_t = g_t / L. Then, as hybrid_attn_forward_fmap,
 * Q' = Q W_q, K' = K W_k, V' = V W_v, and with normalize_k != 0 each K' row
 * divided by max(||K'_t||_2, 1e-12) (no normalisation is named on the page;
 * unit keys are the delta rule's usual convention).
 *   x        [B, T, C] bf16, C channels per token (C % 16 == 0, C < 2^23)
 *   w_gate   [2, H, C] bf16: row 0 the alpha projections, row 1 beta's
 *   b_gate   [2, H] fp32
 *   wq, wk, wv, q, k, v, state, out: as hybrid_attn_forward_fmap
 *   workspace at least hybrid_attn_gated_workspace_bytes(...)
 * bf16 only; H <= 64 when update_state is 1 (HA_ERR_UNSUPPORTED beyond).
 * When update_state is 0 only the readout runs (M = W_q S); x, wk, wv,
 * w_gate and b_gate may then be NULL and C is ignored. Errors and stream
 * behaviour as for hybrid_attn_forward.
 */
ha_status hybrid_attn_forward_gated(const void* x, const void* q, const void* k, const void* v,
                                    const void* wq, const void* wk, const void* wv,
                                    const void* w_gate, const float* b_gate,
                                    float* state, void* out,
                                    void* workspace, size_t workspace_bytes,
                                    int B, int H, int T, int d, int C, int frame_len,
                                    ha_dtype dtype, int update_state, int normalize_k,
                                    float softmax_scale, void* stream);

/*
 * Bytes of workspace hybrid_attn_gates needs (the per-chunk alpha sums,
 * B * F * ceil(L / 64) * H floats, 256-byte aligned). 0 for invalid sizes.
 */
size_t hybrid_attn_gates_workspace_bytes(int B, int H, int T, int frame_len);

/*
 * The gate projections of hybrid_attn_forward_gated alone: writes
 * alpha [B, F, H] and beta [B, T, H] (fp32) from x [B, T, C] bf16,
 * w_gate [2, H, C] bf16 and b_gate [2, H] fp32. alpha is the frame mean of
 * the per-token gates, summed in a fixed order (equal inputs give bitwise
 * equal results). bf16 only; C % 16 == 0, C < 2^23 (else HA_ERR_SHAPE); H <= 64. Outputs must not overlap
 * the inputs or the workspace (HA_ERR_ALIAS). Asynchronous on `stream`.
 */
ha_status hybrid_attn_gates(const void* x, const void* w_gate, const float* b_gate,
                            float* alpha, float* beta, void* workspace, size_t workspace_bytes,
                            int B, int H, int T, int C, int frame_len, ha_dtype dtype,
                            void* stream);

/*
 * Bytes of workspace hybrid_attn_kvcache_forward needs for these sizes and
 * frame_index: 0 when every (b, h, frame) runs in one work-group set;
 * otherwise room for the key splits' fp32 partial outputs (nsplit x B x T x
 * H x d floats) and their (max, sum) pairs (nsplit x B x T x H x 8 bytes),
 * 256-byte aligned. The split count depends on the sizes only (few query
 * work-groups, long caches). Returns 0 also for invalid sizes.
 */
size_t hybrid_attn_kvcache_workspace_bytes(int B, int H, int T, int frame_len, int d, int frame_index);

/*
 * The softmax attention the hybrid layer replaces, with a full KV cache
 * (ARL2 section 1: chunk-wise causal generation; every generated chunk keeps
 * its keys and values for all later chunks, so memory and time grow with the
 * video). For the call's F = T / frame_len frames, which are frames
 * frame_index .. frame_index + F - 1 of the video:
 *   1. k, v are written into the cache at frames frame_index .. + F - 1
 *      (a later call for the same frames overwrites them: denoising passes
 *      leave their own K, V there until the clean pass replaces them);
 *   2. the queries of call frame n attend, with one softmax, to the cache's
 *      keys of frames 0 .. frame_index + n (bidirectional inside their frame,
 *      no later frame); out = softmax(Q K^T * s) V, no readout, no state.
 *   q, k, v, out   [B, T, H, d] bf16
 *   k_cache, v_cache [B, cache_frames * frame_len, H, d] bf16, caller-owned;
 *                  frames < frame_index must hold the earlier frames' K, V
 *   workspace      hybrid_attn_kvcache_workspace_bytes(...) bytes (may be
 *                  NULL when that is 0)
 * bf16 only. HA_ERR_SHAPE if frame_index + F > cache_frames; HA_ERR_ALIAS if
 * out overlaps an input, the caches or the workspace, or k, v, q overlap a
 * cache. Other errors and stream behaviour as for hybrid_attn_forward.
 */
ha_status hybrid_attn_kvcache_forward(const void* q, const void* k, const void* v,
                                      void* k_cache, void* v_cache, void* out,
                                      void* workspace, size_t workspace_bytes,
                                      int B, int H, int T, int d, int frame_len,
                                      int cache_frames, int frame_index, ha_dtype dtype,
                                      float softmax_scale, void* stream);

/*
 * Bytes of workspace hybrid_attn_forward_token_level needs: 96 KiB of
 * operands per 64-token chunk (B * H * F * ceil(frame_len / 64) chunks) and
 * the fp32 inter-frame output (B * T * H * d floats), 256-byte aligned.
 * Returns 0 for invalid sizes or d != 128.
 */
size_t hybrid_attn_token_level_workspace_bytes(int B, int H, int T, int frame_len, int d);

/*
 * The layer with token-level instead of frame-level access (the alternative
 * the ARL2 ablations compare against, section 4; the canonical per-token
 * gated delta rule): tokens in order, token t of frame N reads S_{t-1}, the
 * state after every earlier token, and then writes
 *   S_t = a_t S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1}),
 * a_t = alpha_N for the frame's first token and 1 for the others;
 * out = intra-frame softmax (as hybrid_attn_forward) + q'_t S_{t-1}.
 * Arguments and layouts as hybrid_attn_forward. With update_state 0 the
 * tokens still read the states their predecessors in the call leave (a
 * transient copy) and `state` is left unchanged; kp, vp, alpha and beta are
 * required either way. bf16 and d = 128 only (HA_ERR_UNSUPPORTED otherwise);
 * the workspace is required.
 */
ha_status hybrid_attn_forward_token_level(const void* q, const void* k, const void* v,
                                          const void* qp, const void* kp, const void* vp,
                                          const float* alpha, const float* beta,
                                          float* state, void* out,
                                          void* workspace, size_t workspace_bytes,
                                          int B, int H, int T, int d, int frame_len,
                                          ha_dtype dtype, int update_state,
                                          float softmax_scale, void* stream);

/* A static, human-readable description of a status code ("unknown status"
 * for a value that is not one). */
const char* hybrid_attn_status_string(ha_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int hybrid_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_ATTN_H */
