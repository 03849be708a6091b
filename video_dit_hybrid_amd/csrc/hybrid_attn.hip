// C ABI of the hybrid attention layer: argument validation, workspace layout
// and launch order. The kernels live in attn_bf16.hip, state_bf16.hip,
// state_scan.hip, fp32_path.hip, fmap.hip, gates.hip and token_level.hip.
//
// Launch order of a call (ARL2 section 2.2: every token of frame N reads
// S_{N-1}; the state is written once per clean frame, after the frame):
//   update_state = 0      : readout kernel on `state` for every frame.
//   update_state = 1, F=1 : readout on `state`, then gram, then the scan
//                           writes S_1 into `state` (same stream, so the
//                           readout has read S_0 before it is overwritten).
//   update_state = 1, F>1 : gram, scan (writes S_{n-1} snapshots to the
//                           workspace and S_F to `state`), then the readout
//                           on the snapshots (bf16 readout fragments on the
//                           bf16 path, fp32 row-major on the fp32 path).
#include <math.h>
#include <stdint.h>

#include "../../include/hybrid_attn.h"
#include "ha_launch.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Largest element count the kernels index with 32-bit work decomposition.
constexpr long long kMaxItems = 0x7fffffffLL;

ha_status check_shape(int B, int H, int T, int d, int L, int dtype, ha::Shape* s) {
  if (B <= 0 || H <= 0 || T <= 0 || L <= 0 || d <= 0) return HA_ERR_SHAPE;
  if (T % L != 0) return HA_ERR_SHAPE;
  if (d != 64 && d != 128) return HA_ERR_UNSUPPORTED;
  if (dtype != HA_BF16 && dtype != HA_FP32) return HA_ERR_UNSUPPORTED;
  // work items of the widest launch (fp32 readout: 64 queries per item)
  const long long items = (long long)B * H * (T / L) * ((L + 63) / 64);
  if (items > kMaxItems) return HA_ERR_SHAPE;
  if ((long long)B * H * (T / L) * 2 > kMaxItems) return HA_ERR_SHAPE;
  // one (stream, head, frame) slab is addressed with 32-bit byte offsets, and
  // so are the per-frame state increments of one (stream, head)
  if (((long long)L * H * d + d) * 4 > kMaxItems) return HA_ERR_SHAPE;
  if ((long long)(T / L) * d * d * 8 > kMaxItems) return HA_ERR_SHAPE;
  *s = ha::Shape{B, H, T, d, L, T / L};
  return HA_OK;
}

size_t tensor_bytes(const ha::Shape& s, int dtype) {
  return (size_t)s.B * s.T * s.H * (size_t)s.d * (dtype == HA_BF16 ? 2 : 4);
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

float resolve_scale(float s, int d) { return s > 0.f ? s : 1.0f / sqrtf((float)d); }

ha_status launched(hipError_t e) { return e == hipSuccess ? HA_OK : HA_ERR_DEVICE; }

ha_status run_readout(const void* q, const void* k, const void* v, const void* qp,
                      const float* states, long long sbh, long long sfr, void* out,
                      const ha::Shape& s, int dtype, float scale, hipStream_t st,
                      const void* sfrag = nullptr) {
  if (dtype == HA_BF16)
    return launched(ha::launch_attn_bf16(q, k, v, qp, states, sbh, sfr, sfrag, out, s, scale, st));
  return launched(ha::launch_attn_fp32(q, k, v, qp, states, sbh, sfr, out, s, scale, st));
}

ha_status run_update(const void* kp, const void* vp, const float* alpha, const float* beta,
                     float* state, float* snaps, float* gram, const ha::Shape& s, int dtype,
                     hipStream_t st, void* sfrag = nullptr) {
  if (dtype == HA_BF16) {
    if (ha::launch_gram_bf16(kp, vp, beta, gram, s, st) != hipSuccess) return HA_ERR_DEVICE;
    return launched(ha::launch_state_scan_bf16(gram, alpha, state, snaps, sfrag, s, st));
  }
  if (ha::launch_gram_fp32(kp, vp, beta, gram, s, st) != hipSuccess) return HA_ERR_DEVICE;
  return launched(ha::launch_state_scan_fp32(gram, alpha, state, snaps, s, st));
}

}  // namespace

extern "C" {

int hybrid_attn_version(void) { return 100; }

const char* hybrid_attn_status_string(int status) {
  switch (status) {
    case HA_OK: return "ok";
    case HA_ERR_NULL: return "a required pointer is NULL";
    case HA_ERR_SHAPE: return "invalid sizes (non-positive, T not a multiple of frame_len, or too large)";
    case HA_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64 or 128) or dtype";
    case HA_ERR_ALIGN: return "a tensor pointer is misaligned (16 bytes; alpha and beta 4 bytes)";
    case HA_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case HA_ERR_DEVICE: return "a kernel launch failed";
    case HA_ERR_ALIAS: return "out overlaps an input, the state or the workspace";
    default: return "unknown status";
  }
}

size_t hybrid_attn_state_workspace_bytes(int B, int H, int T, int frame_len, int d) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK) return 0;
  return align_up(ha::gram_bytes(s));
}

size_t hybrid_attn_workspace_bytes(int B, int H, int T, int frame_len, int d, int update_state) {
  ha::Shape s;
  if (!update_state) return 0;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK) return 0;
  size_t n = align_up(ha::gram_bytes(s));
  if (s.F > 1) n += align_up(ha::snapshot_bytes(s));
  return n;
}

ha_status hybrid_attn_intra_readout(const void* q, const void* k, const void* v, const void* qp,
                                    const float* states, long long state_stride_bh,
                                    long long state_stride_frame, void* out, int B, int H, int T,
                                    int d, int frame_len, ha_dtype dtype, float softmax_scale,
                                    void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (!q || !k || !v || !qp || !states || !out) return HA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qp, 16) ||
      !aligned(states, 16) || !aligned(out, 16))
    return HA_ERR_ALIGN;
  if (state_stride_bh < 0 || state_stride_frame < 0 || state_stride_bh % 4 || state_stride_frame % 4)
    return HA_ERR_ALIGN;
  const size_t tb = tensor_bytes(s, dtype);
  const size_t sb = (size_t)((B * (long long)H - 1) * state_stride_bh +
                             (s.F - 1) * state_stride_frame + (long long)d * d) * sizeof(float);
  if (overlap(out, tb, q, tb) || overlap(out, tb, k, tb) || overlap(out, tb, v, tb) ||
      overlap(out, tb, qp, tb) || overlap(out, tb, states, sb))
    return HA_ERR_ALIAS;
  return run_readout(q, k, v, qp, states, state_stride_bh, state_stride_frame, out, s, dtype,
                     resolve_scale(softmax_scale, d), (hipStream_t)stream);
}

ha_status hybrid_attn_state_update(const void* kp, const void* vp, const float* alpha,
                                   const float* beta, float* state, float* snapshots,
                                   void* workspace, size_t workspace_bytes, int B, int H, int T,
                                   int d, int frame_len, ha_dtype dtype, void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (!kp || !vp || !alpha || !beta || !state || !workspace) return HA_ERR_NULL;
  if (!aligned(kp, 16) || !aligned(vp, 16) || !aligned(state, 16) || !aligned(workspace, 16) ||
      !aligned(alpha, 4) || !aligned(beta, 4) || (snapshots && !aligned(snapshots, 16)))
    return HA_ERR_ALIGN;
  if (workspace_bytes < hybrid_attn_state_workspace_bytes(B, H, T, frame_len, d))
    return HA_ERR_WORKSPACE;
  return run_update(kp, vp, alpha, beta, state, snapshots, (float*)workspace, s, dtype,
                    (hipStream_t)stream);
}

ha_status hybrid_attn_forward(const void* q, const void* k, const void* v, const void* qp,
                              const void* kp, const void* vp, const float* alpha,
                              const float* beta, float* state, void* out, void* workspace,
                              size_t workspace_bytes, int B, int H, int T, int d, int frame_len,
                              ha_dtype dtype, int update_state, float softmax_scale,
                              void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (!q || !k || !v || !qp || !state || !out) return HA_ERR_NULL;
  if (update_state && (!kp || !vp || !alpha || !beta)) return HA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qp, 16) ||
      !aligned(state, 16) || !aligned(out, 16))
    return HA_ERR_ALIGN;
  if (update_state && (!aligned(kp, 16) || !aligned(vp, 16) || !aligned(alpha, 4) ||
                       !aligned(beta, 4) || !aligned(workspace, 16)))
    return HA_ERR_ALIGN;
  const size_t need = hybrid_attn_workspace_bytes(B, H, T, frame_len, d, update_state);
  if (need > 0 && (!workspace || workspace_bytes < need)) return HA_ERR_WORKSPACE;

  const size_t tb = tensor_bytes(s, dtype);
  const size_t stb = (size_t)B * H * (size_t)d * d * sizeof(float);
  if (overlap(out, tb, q, tb) || overlap(out, tb, k, tb) || overlap(out, tb, v, tb) ||
      overlap(out, tb, qp, tb) || overlap(out, tb, state, stb) ||
      (update_state && (overlap(out, tb, kp, tb) || overlap(out, tb, vp, tb) ||
                        overlap(out, tb, workspace, need))))
    return HA_ERR_ALIAS;

  const float scale = resolve_scale(softmax_scale, d);
  hipStream_t st = (hipStream_t)stream;
  const long long dd = (long long)d * d;
  if (!update_state)
    return run_readout(q, k, v, qp, state, dd, 0, out, s, dtype, scale, st);

  float* gram = (float*)workspace;
  if (s.F == 1) {
    r = run_readout(q, k, v, qp, state, dd, 0, out, s, dtype, scale, st);
    if (r != HA_OK) return r;
    return run_update(kp, vp, alpha, beta, state, nullptr, gram, s, dtype, st);
  }
  void* snap_area = (char*)workspace + align_up(ha::gram_bytes(s));
  if (dtype == HA_BF16) {
    // S_{n-1} of every frame as bf16 readout fragments (the readout rounds the
    // state to bf16 either way)
    r = run_update(kp, vp, alpha, beta, state, nullptr, gram, s, dtype, st, snap_area);
    if (r != HA_OK) return r;
    const long long fb = (long long)s.d * s.d * 2;  // fragment bytes per frame
    return run_readout(q, k, v, qp, nullptr, (long long)s.F * fb, fb, out, s, dtype, scale, st, snap_area);
  }
  float* snaps = (float*)snap_area;
  r = run_update(kp, vp, alpha, beta, state, snaps, gram, s, dtype, st);
  if (r != HA_OK) return r;
  return run_readout(q, k, v, qp, snaps, (long long)s.F * dd, dd, out, s, dtype, scale, st);
}

}  // extern "C"

// ---- feature-map variant (fmap.hip): the layer with Q' = Q W_q, K' = K W_k,
// V' = V W_v folded into the kernels instead of materialised.
//   update_state = 0 : M = W_q S once per (b, h), then the readout kernel on
//                      Q and the fragments of M for every frame.
//   update_state = 1 : gram pass on K, V (fp32 partial sums), the transform to
//                      the increments under the maps, the scan (fp32
//                      snapshots S_{n-1}, S_F into `state`), M_n = W_q S_{n-1}
//                      for every frame, then the readout on Q and M_n.
// The gated variant (gates.hip) first computes alpha and beta from the layer
// input x and, for normalised keys, the two step-size vectors beta / n^2 and
// beta / n (keyscale), then runs the same passes.
namespace {
struct FmapWs {
  size_t gram, partial, snaps, mfrag;
  size_t beta, beta_g, beta_b, apart, alpha;  // gated variant only
  size_t total;
};
FmapWs fmap_layout(const ha::Shape& s, int update_state, bool gated) {
  FmapWs w{};
  const size_t dd = (size_t)s.d * s.d;
  if (!update_state) {
    w.mfrag = 0;
    w.total = align_up((size_t)s.B * s.H * dd * 2);
    return w;
  }
  const size_t gf = ha::gram_final_bytes(s);
  w.gram = 0;
  w.partial = align_up(gf);
  w.snaps = w.partial + align_up(gf * ha::gram_splits(s));
  w.mfrag = w.snaps + align_up((size_t)s.B * s.H * s.F * dd * 4);
  w.total = w.mfrag + align_up((size_t)s.B * s.H * s.F * dd * 2);
  if (gated) {
    const size_t tok = (size_t)s.B * s.T * s.H * sizeof(float);
    w.beta = w.total;
    w.beta_g = w.beta + align_up(tok);
    w.beta_b = w.beta_g + align_up(tok);
    w.apart = w.beta_b + align_up(tok);
    w.alpha = w.apart + align_up(ha::gates_partial_bytes(s));
    w.total = w.alpha + align_up((size_t)s.B * s.F * s.H * sizeof(float));
  }
  return w;
}

// The passes shared by the two variants; arguments already validated.
ha_status fmap_run(const void* q, const void* k, const void* v, const void* wq, const void* wk, const void* wv,
                   const float* alpha, const float* beta, const float* beta2, float* state, void* out,
                   char* ws, const FmapWs& lay, const ha::Shape& s, int update_state, float scale,
                   hipStream_t st) {
  const long long dd = (long long)s.d * s.d, fb = dd * 2;
  if (!update_state) {
    void* mf = ws + lay.mfrag;
    if (ha::launch_mfrag(state, dd, 0, wq, mf, 1, s, st) != hipSuccess) return HA_ERR_DEVICE;
    return run_readout(q, k, v, q, nullptr, fb, 0, out, s, HA_BF16, scale, st, mf);
  }
  float* gram = (float*)(ws + lay.gram);
  float* partial = (float*)(ws + lay.partial);
  float* snaps = (float*)(ws + lay.snaps);
  void* mf = ws + lay.mfrag;
  const int nsplit = ha::gram_splits(s);
  if (ha::launch_gram_partials_bf16(k, v, beta, beta2, partial, nsplit, s, st) != hipSuccess) return HA_ERR_DEVICE;
  if (ha::launch_gram_fmap(partial, nsplit, wk, wv, gram, s, st) != hipSuccess) return HA_ERR_DEVICE;
  if (ha::launch_state_scan_bf16(gram, alpha, state, snaps, nullptr, s, st) != hipSuccess) return HA_ERR_DEVICE;
  if (ha::launch_mfrag(snaps, (long long)s.F * dd, dd, wq, mf, s.F, s, st) != hipSuccess) return HA_ERR_DEVICE;
  return run_readout(q, k, v, q, nullptr, (long long)s.F * fb, fb, out, s, HA_BF16, scale, st, mf);
}

// Shape checks of the gate projection: C channels in 16-element k-steps, at
// most 64 heads (2H gate rows in four 32-row MFMA blocks).
ha_status check_gate_shape(const ha::Shape& s, int C) {
  if (C <= 0 || C % 16 != 0) return HA_ERR_SHAPE;
  // 64 tokens (or 2H <= 128 gate rows) of C channels are addressed with
  // 32-bit byte offsets
  if ((long long)C * 2 * 128 > kMaxItems) return HA_ERR_SHAPE;
  if (s.H > 64) return HA_ERR_UNSUPPORTED;
  if ((long long)s.B * s.F * ha::gates_chunks(s) > kMaxItems) return HA_ERR_SHAPE;
  return HA_OK;
}
}  // namespace

extern "C" {

size_t hybrid_attn_fmap_workspace_bytes(int B, int H, int T, int frame_len, int d, int update_state) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK) return 0;
  return fmap_layout(s, update_state, false).total;
}

ha_status hybrid_attn_forward_fmap(const void* q, const void* k, const void* v, const void* wq,
                                   const void* wk, const void* wv, const float* alpha,
                                   const float* beta, float* state, void* out, void* workspace,
                                   size_t workspace_bytes, int B, int H, int T, int d,
                                   int frame_len, ha_dtype dtype, int update_state,
                                   float softmax_scale, void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (dtype != HA_BF16) return HA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !wq || !state || !out || !workspace) return HA_ERR_NULL;
  if (update_state && (!wk || !wv || !alpha || !beta)) return HA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(wq, 16) ||
      !aligned(state, 16) || !aligned(out, 16) || !aligned(workspace, 16))
    return HA_ERR_ALIGN;
  if (update_state && (!aligned(wk, 16) || !aligned(wv, 16) || !aligned(alpha, 4) || !aligned(beta, 4)))
    return HA_ERR_ALIGN;
  const FmapWs lay = fmap_layout(s, update_state, false);
  if (workspace_bytes < lay.total) return HA_ERR_WORKSPACE;

  const size_t tb = tensor_bytes(s, dtype);
  const size_t stb = (size_t)B * H * (size_t)d * d * sizeof(float);
  const size_t wb = (size_t)H * d * d * 2;
  if (overlap(out, tb, q, tb) || overlap(out, tb, k, tb) || overlap(out, tb, v, tb) ||
      overlap(out, tb, wq, wb) || overlap(out, tb, state, stb) || overlap(out, tb, workspace, lay.total) ||
      (update_state && (overlap(out, tb, wk, wb) || overlap(out, tb, wv, wb))))
    return HA_ERR_ALIAS;
  return fmap_run(q, k, v, wq, wk, wv, alpha, beta, nullptr, state, out, (char*)workspace, lay, s, update_state,
                  resolve_scale(softmax_scale, d), (hipStream_t)stream);
}

size_t hybrid_attn_gated_workspace_bytes(int B, int H, int T, int frame_len, int d, int update_state) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK) return 0;
  return fmap_layout(s, update_state, true).total;
}

ha_status hybrid_attn_forward_gated(const void* x, const void* q, const void* k, const void* v,
                                    const void* wq, const void* wk, const void* wv, const void* w_gate,
                                    const float* b_gate, float* state, void* out, void* workspace,
                                    size_t workspace_bytes, int B, int H, int T, int d, int C,
                                    int frame_len, ha_dtype dtype, int update_state, int normalize_k,
                                    float softmax_scale, void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (dtype != HA_BF16) return HA_ERR_UNSUPPORTED;
  if (update_state && (r = check_gate_shape(s, C)) != HA_OK) return r;
  if (!q || !k || !v || !wq || !state || !out || !workspace) return HA_ERR_NULL;
  if (update_state && (!x || !wk || !wv || !w_gate || !b_gate)) return HA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(wq, 16) ||
      !aligned(state, 16) || !aligned(out, 16) || !aligned(workspace, 16))
    return HA_ERR_ALIGN;
  if (update_state && (!aligned(x, 16) || !aligned(wk, 16) || !aligned(wv, 16) || !aligned(w_gate, 16) ||
                       !aligned(b_gate, 4)))
    return HA_ERR_ALIGN;
  const FmapWs lay = fmap_layout(s, update_state, true);
  if (workspace_bytes < lay.total) return HA_ERR_WORKSPACE;

  const size_t tb = tensor_bytes(s, dtype);
  const size_t stb = (size_t)B * H * (size_t)d * d * sizeof(float);
  const size_t wb = (size_t)H * d * d * 2;
  const size_t xb = (size_t)B * T * (size_t)(update_state ? C : 0) * 2;
  const size_t gb = (size_t)2 * H * (size_t)(update_state ? C : 0) * 2;
  if (overlap(out, tb, q, tb) || overlap(out, tb, k, tb) || overlap(out, tb, v, tb) ||
      overlap(out, tb, wq, wb) || overlap(out, tb, state, stb) || overlap(out, tb, workspace, lay.total) ||
      (update_state && (overlap(out, tb, wk, wb) || overlap(out, tb, wv, wb) || overlap(out, tb, x, xb) ||
                        overlap(out, tb, w_gate, gb) || overlap(out, tb, b_gate, (size_t)2 * H * 4))))
    return HA_ERR_ALIAS;

  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  const float scale = resolve_scale(softmax_scale, d);
  if (!update_state)
    return fmap_run(q, k, v, wq, wk, wv, nullptr, nullptr, nullptr, state, out, ws, lay, s, 0, scale, st);
  float* alpha = (float*)(ws + lay.alpha);
  float* beta = (float*)(ws + lay.beta);
  if (ha::launch_gates(x, w_gate, b_gate, alpha, beta, (float*)(ws + lay.apart), C, s, st) != hipSuccess)
    return HA_ERR_DEVICE;
  if (!normalize_k)
    return fmap_run(q, k, v, wq, wk, wv, alpha, beta, nullptr, state, out, ws, lay, s, 1, scale, st);
  float* bgv = (float*)(ws + lay.beta_g);
  float* bbv = (float*)(ws + lay.beta_b);
  if (ha::launch_keyscale(k, wk, beta, bgv, bbv, s, st) != hipSuccess) return HA_ERR_DEVICE;
  return fmap_run(q, k, v, wq, wk, wv, alpha, bgv, bbv, state, out, ws, lay, s, 1, scale, st);
}

size_t hybrid_attn_gates_workspace_bytes(int B, int H, int T, int frame_len) {
  ha::Shape s;
  if (check_shape(B, H, T, 64, frame_len, HA_BF16, &s) != HA_OK) return 0;
  return align_up(ha::gates_partial_bytes(s));
}

ha_status hybrid_attn_gates(const void* x, const void* w_gate, const float* b_gate, float* alpha, float* beta,
                            void* workspace, size_t workspace_bytes, int B, int H, int T, int C,
                            int frame_len, ha_dtype dtype, void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, 64, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (dtype != HA_BF16) return HA_ERR_UNSUPPORTED;
  if ((r = check_gate_shape(s, C)) != HA_OK) return r;
  if (!x || !w_gate || !b_gate || !alpha || !beta || !workspace) return HA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(b_gate, 4) || !aligned(alpha, 4) ||
      !aligned(beta, 4) || !aligned(workspace, 16))
    return HA_ERR_ALIGN;
  if (workspace_bytes < align_up(ha::gates_partial_bytes(s))) return HA_ERR_WORKSPACE;
  const size_t ab = (size_t)B * s.F * H * 4, bb = (size_t)B * T * H * 4;
  const size_t xb = (size_t)B * T * (size_t)C * 2, gb = (size_t)2 * H * (size_t)C * 2;
  const size_t wsb = align_up(ha::gates_partial_bytes(s));
  if (overlap(alpha, ab, beta, bb) || overlap(alpha, ab, x, xb) || overlap(beta, bb, x, xb) ||
      overlap(alpha, ab, w_gate, gb) || overlap(beta, bb, w_gate, gb) || overlap(alpha, ab, workspace, wsb) ||
      overlap(beta, bb, workspace, wsb) || overlap(alpha, ab, b_gate, (size_t)2 * H * 4) ||
      overlap(beta, bb, b_gate, (size_t)2 * H * 4))
    return HA_ERR_ALIAS;
  return launched(ha::launch_gates(x, w_gate, b_gate, alpha, beta, (float*)workspace, C, s, (hipStream_t)stream));
}

}  // extern "C"

// ---- the softmax teacher with a full KV cache (attn_bf16.hip, KV mode): the
// call's K, V rows are appended to the cache at frame frame_index, then frame
// n of the call attends to the cache's first (frame_index + n + 1) * L keys.
namespace {
struct KvWs {
  size_t part_o, part_ml, total;
  int nsplit;
};
KvWs kv_layout(const ha::Shape& s, int frame_index) {
  KvWs w{0, 0, 0, 1};
  w.nsplit = ha::kv_splits(s, frame_index * s.L);
  if (w.nsplit == 1) return w;
  const size_t rows = (size_t)s.B * s.T * s.H;
  w.part_o = 0;
  w.part_ml = align_up((size_t)w.nsplit * rows * s.d * 4);
  w.total = w.part_ml + align_up((size_t)w.nsplit * rows * 8);
  return w;
}
}  // namespace

extern "C" {

size_t hybrid_attn_kvcache_workspace_bytes(int B, int H, int T, int frame_len, int d, int frame_index) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK || frame_index < 0) return 0;
  return kv_layout(s, frame_index).total;
}

ha_status hybrid_attn_kvcache_forward(const void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                                      void* out, void* workspace, size_t workspace_bytes, int B, int H, int T,
                                      int d, int frame_len, int cache_frames, int frame_index, ha_dtype dtype,
                                      float softmax_scale, void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (dtype != HA_BF16) return HA_ERR_UNSUPPORTED;
  if (frame_index < 0 || cache_frames <= 0 || (long long)frame_index + s.F > cache_frames) return HA_ERR_SHAPE;
  if ((long long)cache_frames * frame_len > kMaxItems) return HA_ERR_SHAPE;
  if (!q || !k || !v || !k_cache || !v_cache || !out) return HA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 16) || (workspace && !aligned(workspace, 16)))
    return HA_ERR_ALIGN;
  const KvWs lay = kv_layout(s, frame_index);
  if (lay.total && (!workspace || workspace_bytes < lay.total)) return HA_ERR_WORKSPACE;
  const size_t tb = tensor_bytes(s, dtype);
  const size_t cb = (size_t)B * cache_frames * frame_len * H * (size_t)d * 2;
  if (overlap(out, tb, q, tb) || overlap(out, tb, k, tb) || overlap(out, tb, v, tb) ||
      overlap(out, tb, k_cache, cb) || overlap(out, tb, v_cache, cb) || overlap(out, tb, workspace, lay.total) ||
      overlap(k_cache, cb, v_cache, cb) || overlap(k, tb, k_cache, cb) || overlap(v, tb, k_cache, cb) ||
      overlap(k, tb, v_cache, cb) || overlap(v, tb, v_cache, cb) || overlap(q, tb, k_cache, cb) ||
      overlap(q, tb, v_cache, cb) || overlap(workspace, lay.total, k_cache, cb) ||
      overlap(workspace, lay.total, v_cache, cb))
    return HA_ERR_ALIAS;
  hipStream_t st = (hipStream_t)stream;
  const int cap = cache_frames * frame_len;
  if (ha::launch_kv_append(k, v, k_cache, v_cache, cap, frame_index * frame_len, s, st) != hipSuccess)
    return HA_ERR_DEVICE;
  char* ws = (char*)workspace;
  return launched(ha::launch_attn_kv_bf16(q, k_cache, v_cache, out, lay.total ? (float*)(ws + lay.part_o) : nullptr,
                                          lay.total ? (void*)(ws + lay.part_ml) : nullptr, lay.nsplit, cap,
                                          frame_index * frame_len, s, resolve_scale(softmax_scale, d), st));
}

}  // extern "C"

// ---- token-level access (token_level.hip): the per-token gated delta rule
// (prep + sequential chunk pass, writing the fp32 inter-frame output), then
// the intra-frame softmax in its one-frame window, which adds that output
// before rounding.
namespace {
size_t tl_frag_offset(const ha::Shape&) { return 0; }
size_t tl_oint_offset(const ha::Shape& s) { return align_up(ha::token_level_frag_bytes(s)); }
size_t tl_total(const ha::Shape& s) {
  return tl_oint_offset(s) + align_up((size_t)s.B * s.T * s.H * (size_t)s.d * sizeof(float));
}
}  // namespace

extern "C" {

size_t hybrid_attn_token_level_workspace_bytes(int B, int H, int T, int frame_len, int d) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK || d != 128) return 0;
  return tl_total(s);
}

ha_status hybrid_attn_forward_token_level(const void* q, const void* k, const void* v, const void* qp,
                                          const void* kp, const void* vp, const float* alpha,
                                          const float* beta, float* state, void* out, void* workspace,
                                          size_t workspace_bytes, int B, int H, int T, int d, int frame_len,
                                          ha_dtype dtype, int update_state, float softmax_scale, void* stream) {
  ha::Shape s;
  ha_status r = check_shape(B, H, T, d, frame_len, dtype, &s);
  if (r != HA_OK) return r;
  if (dtype != HA_BF16 || d != 128) return HA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !qp || !kp || !vp || !alpha || !beta || !state || !out || !workspace) return HA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qp, 16) || !aligned(kp, 16) ||
      !aligned(vp, 16) || !aligned(state, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return HA_ERR_ALIGN;
  const size_t total = tl_total(s);
  if (workspace_bytes < total) return HA_ERR_WORKSPACE;
  const size_t tb = tensor_bytes(s, dtype);
  const size_t stb = (size_t)B * H * (size_t)d * d * sizeof(float);
  if (overlap(out, tb, q, tb) || overlap(out, tb, k, tb) || overlap(out, tb, v, tb) || overlap(out, tb, qp, tb) ||
      overlap(out, tb, kp, tb) || overlap(out, tb, vp, tb) || overlap(out, tb, state, stb) ||
      overlap(out, tb, workspace, total) || overlap(state, stb, workspace, total))
    return HA_ERR_ALIAS;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* oint = (float*)(ws + tl_oint_offset(s));
  if (ha::launch_token_level(qp, kp, vp, alpha, beta, state, ws + tl_frag_offset(s), oint, update_state, s, st) !=
      hipSuccess)
    return HA_ERR_DEVICE;
  return launched(ha::launch_attn_kv_bf16(q, k, v, out, nullptr, nullptr, 1, T, -1, s,
                                          resolve_scale(softmax_scale, d), st, oint));
}

}  // extern "C"
