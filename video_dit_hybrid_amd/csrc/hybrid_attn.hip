// C ABI of the hybrid attention layer: argument validation, workspace layout
// and launch order. The kernels live in attn_bf16.hip, state_bf16.hip,
// state_scan.hip, fp32_path.hip, fmap.hip, gates.hip and token_level.hip.
//
// Launch order of a call (ARL2 section 2.2: every token of frame N reads
// S_{N-1}; the state is written once per clean frame, after the frame):
//   update_state = 0      : readout kernel on `state` for every frame.
//   update_state = 1, F=1 : readout on `state`, then the state write into
//                           `state` (one kernel at d = 128 in bf16, else gram
//                           and scan; same stream, so the readout has read
//                           S_0 before it is overwritten).
//   update_state = 1, F>1 : gram, scan (writes S_{n-1} snapshots to the
//                           workspace and S_F to `state`), then the readout
//                           on the snapshots (bf16 readout fragments on the
//                           bf16 path, fp32 row-major on the fp32 path). In
//                           bf16 with more than 256 attention work-groups the
//                           scan runs as the first work-groups of the readout's
//                           launch, which wait frame by frame for it.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/hybrid_attn.h"
#include "ha_launch.h"
#include "ha_log.h"

namespace ha {

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && strcmp(v, "0") != 0;
}

void log_line(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[hybrid_attn] %s\n", buf);
}

}  // namespace ha

namespace {

// ---- HA_CHECK_FINITE: a scan of a written state for Inf / NaN. The test is on
// the exponent bits, which stays valid under -fno-honor-nans.
__device__ unsigned int g_nonfinite;

__global__ __launch_bounds__(256) void nonfinite_reset_kernel() { g_nonfinite = 0u; }

__global__ __launch_bounds__(256) void nonfinite_scan_kernel(const float* __restrict__ x, long long n) {
  bool bad = false;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    bad |= (__float_as_uint(x[i]) & 0x7f800000u) == 0x7f800000u;
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(&g_nonfinite, 1u);
}

// With HA_CHECK_FINITE set: scans nfloats floats at x after the work already on
// st, synchronises st and reports what it found.
ha_status check_finite(const char* what, const float* x, size_t nfloats, hipStream_t st) {
  if (!ha::env_flag("HA_CHECK_FINITE") || nfloats == 0) return HA_OK;
  const long long n = (long long)nfloats;
  const int grid = (int)(n / 256 + 1 < 1024 ? n / 256 + 1 : 1024);
  nonfinite_reset_kernel<<<1, 1, 0, st>>>();
  nonfinite_scan_kernel<<<grid, 256, 0, st>>>(x, n);
  unsigned int found = 0;
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpyFromSymbol(&found, HIP_SYMBOL(g_nonfinite), sizeof found, 0, hipMemcpyDeviceToHost) != hipSuccess)
    return HA_ERR_DEVICE;
  HA_LOG("HA_CHECK_FINITE: %s (%zu floats) %s", what, nfloats, found ? "holds Inf or NaN" : "finite");
  return found ? HA_ERR_NONFINITE : HA_OK;
}

const char* dtype_name(int dtype) { return dtype == HA_BF16 ? "bf16" : dtype == HA_FP32 ? "fp32" : "?"; }

void log_call(const char* entry, const ha::Shape& s, int dtype, int update_state, size_t workspace) {
  HA_LOG("%s: B=%d H=%d T=%d (%d frames x %d tokens) d=%d %s update_state=%d workspace %zu bytes", entry, s.B, s.H,
         s.T, s.F, s.L, s.d, dtype_name(dtype), update_state, workspace);
}

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
  // Each product below is bounded before the next factor joins it, so no
  // intermediate overflows (every factor is < 2^31).
  const long long F = T / L;
  const long long bh = (long long)B * H;
  if (bh > kMaxItems || bh * F * 2 > kMaxItems) return HA_ERR_SHAPE;
  // work items of the widest launch (fp32 readout: 64 queries per item)
  if (bh * F * (((long long)L + 63) / 64) > kMaxItems) return HA_ERR_SHAPE;
  // one (stream, head, frame) slab is addressed with 32-bit byte offsets, and
  // so are the per-frame state increments of one (stream, head)
  if ((long long)L * H > kMaxItems || ((long long)L * H * d + d) * 4 > kMaxItems) return HA_ERR_SHAPE;
  if (F * d * d * 8 > kMaxItems) return HA_ERR_SHAPE;
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

// A buffer of a call: base pointer and the bytes the call may touch.
struct Span {
  const void* p;
  size_t n;
};

// True when a buffer the call writes overlaps any other buffer of the call
// (an input it reads, or another buffer it writes). NULL or empty spans are
// absent arguments.
bool written_overlaps(std::initializer_list<Span> written, std::initializer_list<Span> read) {
  for (const Span* w = written.begin(); w != written.end(); ++w) {
    for (const Span* o = written.begin(); o != written.end(); ++o)
      if (o != w && overlap(w->p, w->n, o->p, o->n)) return true;
    for (const Span& r : read)
      if (overlap(w->p, w->n, r.p, r.n)) return true;
  }
  return false;
}

float resolve_scale(float s, int d) { return s > 0.f ? s : 1.0f / sqrtf((float)d); }

ha_status launched(hipError_t e) { return e == hipSuccess ? HA_OK : HA_ERR_DEVICE; }

ha_status run_readout(const void* q, const void* k, const void* v, const void* qp,
                      const float* states, long long sbh, long long sfr, void* out,
                      const ha::Shape& s, int dtype, float scale, hipStream_t st,
                      const void* sfrag = nullptr, const float* mix = nullptr) {
  if (dtype == HA_BF16)
    return launched(ha::launch_attn_bf16(q, k, v, qp, states, sbh, sfr, sfrag, out, s, scale, st, mix));
  return launched(ha::launch_attn_fp32(q, k, v, qp, states, sbh, sfr, out, s, scale, st));
}

ha_status run_update(const void* kp, const void* vp, const float* alpha, const float* beta,
                     float* state, float* snaps, float* gram, const ha::Shape& s, int dtype,
                     hipStream_t st, void* sfrag = nullptr) {
  if (dtype == HA_BF16) {
    // one frame, d = 128: the residual, the increment and the decay in one kernel
    if (s.F == 1 && s.d == 128 && !sfrag)
      return launched(ha::launch_state_step_bf16(kp, vp, alpha, beta, state, snaps, gram, s, st));
    if (ha::launch_gram_bf16(kp, vp, beta, gram, s, st) != hipSuccess) return HA_ERR_DEVICE;
    return launched(ha::launch_state_scan_bf16(gram, alpha, state, snaps, sfrag, s, st));
  }
  if (ha::launch_gram_fp32(kp, vp, beta, gram, s, st) != hipSuccess) return HA_ERR_DEVICE;
  return launched(ha::launch_state_scan_fp32(gram, alpha, state, snaps, s, st));
}

// The arguments of a forward call other than its workspace and stream.
struct ForwardArgs {
  const void *q, *k, *v, *qp, *kp, *vp;
  const float *alpha, *beta;
  float* state;
  void* out;
  int B, H, T, d, frame_len;
  ha_dtype dtype;
  int update_state;
  float softmax_scale;
  const float* mix;  // per-branch output weights [B, H, 2], or null (the plain sum)
};

// Checks of a forward call that do not involve the workspace; on success
// fills the shape and the workspace bytes the call needs.
ha_status validate_forward(const ForwardArgs& a, ha::Shape* s, size_t* need) {
  ha_status r = check_shape(a.B, a.H, a.T, a.d, a.frame_len, a.dtype, s);
  if (r != HA_OK) return r;
  if (!a.q || !a.k || !a.v || !a.qp || !a.state || !a.out) return HA_ERR_NULL;
  if (a.update_state && (!a.kp || !a.vp || !a.alpha || !a.beta)) return HA_ERR_NULL;
  if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(a.qp, 16) ||
      !aligned(a.state, 16) || !aligned(a.out, 16))
    return HA_ERR_ALIGN;
  if (a.update_state &&
      (!aligned(a.kp, 16) || !aligned(a.vp, 16) || !aligned(a.alpha, 4) || !aligned(a.beta, 4)))
    return HA_ERR_ALIGN;
  if (a.mix && a.dtype != HA_BF16) return HA_ERR_UNSUPPORTED;
  if (a.mix && !aligned(a.mix, 8)) return HA_ERR_ALIGN;
  *need = hybrid_attn_workspace_bytes(a.B, a.H, a.T, a.frame_len, a.d, a.update_state);
  return HA_OK;
}

// The aliasing rules of a forward call, with the workspace of `need` bytes.
bool workspace_overlaps(const ForwardArgs& a, const ha::Shape& s, const void* ws, size_t need) {
  const size_t tb = tensor_bytes(s, a.dtype);
  const size_t stb = (size_t)a.B * a.H * (size_t)a.d * a.d * sizeof(float);
  const size_t ab = (size_t)a.B * s.F * a.H * sizeof(float), bb = (size_t)a.B * a.T * a.H * sizeof(float);
  const size_t mb = a.mix ? (size_t)a.B * a.H * 2 * sizeof(float) : 0;
  if (a.update_state)
    return written_overlaps({{a.out, tb}, {a.state, stb}, {ws, need}},
                            {{a.q, tb}, {a.k, tb}, {a.v, tb}, {a.qp, tb}, {a.kp, tb}, {a.vp, tb}, {a.alpha, ab},
                             {a.beta, bb}, {a.mix, mb}});
  return written_overlaps({{a.out, tb}},
                          {{a.q, tb}, {a.k, tb}, {a.v, tb}, {a.qp, tb}, {a.state, stb}, {a.mix, mb}});
}

// Workspace of a forward call: the state update's increments and, over
// several frames, the per-frame states.
size_t forward_base_bytes(const ha::Shape& s, int update_state) {
  if (!update_state) return 0;
  size_t n = align_up(ha::update_bytes(s));
  if (s.F > 1) n += align_up(ha::snapshot_bytes(s));
  return n;
}

// Launch order of a validated forward call (see the top of this file).
ha_status launch_forward(const ForwardArgs& a, const ha::Shape& s, void* workspace, hipStream_t st) {
  const float scale = resolve_scale(a.softmax_scale, a.d);
  const long long dd = (long long)a.d * a.d;
  if (!a.update_state)
    return run_readout(a.q, a.k, a.v, a.qp, a.state, dd, 0, a.out, s, a.dtype, scale, st, nullptr, a.mix);
  float* gram = (float*)workspace;
  const size_t nstate = (size_t)s.B * s.H * (size_t)dd;
  if (s.F == 1) {
    ha_status r = run_readout(a.q, a.k, a.v, a.qp, a.state, dd, 0, a.out, s, a.dtype, scale, st, nullptr, a.mix);
    if (r != HA_OK) return r;
    r = run_update(a.kp, a.vp, a.alpha, a.beta, a.state, nullptr, gram, s, a.dtype, st);
    return r != HA_OK ? r : check_finite("state", a.state, nstate, st);
  }
  void* snap_area = (char*)workspace + align_up(ha::update_bytes(s));
  if (a.dtype == HA_BF16 && !a.mix && ha::attn_groups(s) > ha::kAttnLoaderMaxGroups) {
    // the scan runs in the attention launch: its work-groups publish each
    // frame's S_{n-1} as readout fragments and count them per frame (the
    // counters follow the fragments in the snapshot area, which is sized for
    // fp32 snapshots; the gram kernel zeroes them)
    unsigned* flags = (unsigned*)((char*)snap_area + align_up(ha::snapshot_frag_bytes(s)));
    if (ha::launch_gram_bf16(a.kp, a.vp, a.beta, gram, s, st, flags) != hipSuccess) return HA_ERR_DEVICE;
    const ha_status r = launched(ha::launch_attn_scan_bf16(a.q, a.k, a.v, a.qp, gram, a.alpha, a.state, snap_area,
                                                           flags, a.out, s, scale, st));
    return r != HA_OK ? r : check_finite("state", a.state, nstate, st);
  }
  if (a.dtype == HA_BF16) {
    // S_{n-1} of every frame as bf16 readout fragments (the readout rounds the
    // state to bf16 either way)
    ha_status r = run_update(a.kp, a.vp, a.alpha, a.beta, a.state, nullptr, gram, s, a.dtype, st, snap_area);
    if (r != HA_OK) return r;
    const long long fb = (long long)s.d * s.d * 2;  // fragment bytes per frame
    r = run_readout(a.q, a.k, a.v, a.qp, nullptr, (long long)s.F * fb, fb, a.out, s, a.dtype, scale, st, snap_area,
                    a.mix);
    return r != HA_OK ? r : check_finite("state", a.state, nstate, st);
  }
  float* snaps = (float*)snap_area;
  ha_status r = run_update(a.kp, a.vp, a.alpha, a.beta, a.state, snaps, gram, s, a.dtype, st);
  if (r != HA_OK) return r;
  r = run_readout(a.q, a.k, a.v, a.qp, snaps, (long long)s.F * dd, dd, a.out, s, a.dtype, scale, st);
  return r != HA_OK ? r : check_finite("state", a.state, nstate, st);
}

// Debug build (-DHA_DEBUG): after an entry point's launches, wait for them and
// report every failed index check of the kernels (the kernel files' debug
// words) on stderr, as HA_ERR_DEVICE. Other builds return r as it is.
ha_status debug_finish(const char* entry, ha_status r, hipStream_t st) {
#if defined(HA_DEBUG)
  if (r != HA_OK) return r;
  if (hipStreamSynchronize(st) != hipSuccess) return HA_ERR_DEVICE;
  const struct {
    const char* name;
    unsigned (*take)();
  } files[] = {{"attention", ha::debug_take_attn}, {"gram", ha::debug_take_gram},
               {"state scan", ha::debug_take_scan}, {"one-frame state write", ha::debug_take_step}};
  for (const auto& f : files) {
    const unsigned w = f.take();
    if (w) {
      fprintf(stderr, "[hybrid_attn debug] %s: index check bits 0x%x failed in the %s kernel\n", entry, w, f.name);
      r = HA_ERR_DEVICE;
    }
  }
  return r;
#else
  (void)entry;
  (void)st;
  return r;
#endif
}

}  // namespace

extern "C" {

int hybrid_attn_version(void) { return 100; }

const char* hybrid_attn_status_string(ha_status status) {
  switch (status) {
    case HA_OK: return "ok";
    case HA_ERR_NULL: return "a required pointer is NULL";
    case HA_ERR_SHAPE: return "invalid sizes (non-positive, T not a multiple of frame_len, or too large)";
    case HA_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64 or 128) or dtype";
    case HA_ERR_ALIGN: return "a tensor pointer is misaligned (16 bytes; alpha and beta 4 bytes)";
    case HA_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case HA_ERR_DEVICE: return "a kernel launch failed";
    case HA_ERR_ALIAS: return "a buffer the call writes overlaps another buffer of the call";
    case HA_ERR_SCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
    case HA_ERR_NONFINITE: return "the state holds Inf or NaN after the call (HA_CHECK_FINITE)";
    default: return "unknown status";
  }
}

size_t hybrid_attn_state_workspace_bytes(int B, int H, int T, int frame_len, int d) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK) return 0;
  return align_up(ha::update_bytes(s));
}

size_t hybrid_attn_workspace_bytes(int B, int H, int T, int frame_len, int d, int update_state) {
  ha::Shape s;
  if (check_shape(B, H, T, d, frame_len, HA_BF16, &s) != HA_OK) return 0;
  return forward_base_bytes(s, update_state);
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
  log_call("hybrid_attn_intra_readout", s, dtype, 0, 0);
  return debug_finish("hybrid_attn_intra_readout",
                      run_readout(q, k, v, qp, states, state_stride_bh, state_stride_frame, out, s, dtype,
                     resolve_scale(softmax_scale, d), (hipStream_t)stream), (hipStream_t)stream);
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
  const size_t need = hybrid_attn_state_workspace_bytes(B, H, T, frame_len, d);
  if (workspace_bytes < need) return HA_ERR_WORKSPACE;
  const size_t tb = tensor_bytes(s, dtype);
  const size_t stb = (size_t)B * H * (size_t)d * d * sizeof(float);
  const size_t snb = snapshots ? stb * s.F : 0;
  const size_t ab = (size_t)B * s.F * H * sizeof(float), bb = (size_t)B * T * H * sizeof(float);
  if (written_overlaps({{state, stb}, {snapshots, snb}, {workspace, need}},
                       {{kp, tb}, {vp, tb}, {alpha, ab}, {beta, bb}}))
    return HA_ERR_ALIAS;
  log_call("hybrid_attn_state_update", s, dtype, 1, need);
  r = run_update(kp, vp, alpha, beta, state, snapshots, (float*)workspace, s, dtype, (hipStream_t)stream);
  if (r == HA_OK) r = check_finite("state", state, stb / sizeof(float), (hipStream_t)stream);
  return debug_finish("hybrid_attn_state_update", r, (hipStream_t)stream);
}

ha_status hybrid_attn_forward(const void* q, const void* k, const void* v, const void* qp,
                              const void* kp, const void* vp, const float* alpha,
                              const float* beta, float* state, void* out, void* workspace,
                              size_t workspace_bytes, int B, int H, int T, int d, int frame_len,
                              ha_dtype dtype, int update_state, float softmax_scale,
                              void* stream) {
  const ForwardArgs a{q, k, v, qp, kp, vp, alpha, beta, state, out, B, H, T, d, frame_len, dtype, update_state,
                      softmax_scale};
  ha::Shape s;
  size_t need = 0;
  ha_status r = validate_forward(a, &s, &need);
  if (r != HA_OK) return r;
  if (update_state && !aligned(workspace, 16)) return HA_ERR_ALIGN;
  if (need > 0 && (!workspace || workspace_bytes < need)) return HA_ERR_WORKSPACE;
  if (workspace_overlaps(a, s, workspace, need)) return HA_ERR_ALIAS;
  log_call("hybrid_attn_forward", s, dtype, update_state, need);
  return debug_finish("hybrid_attn_forward",
                      launch_forward(a, s, workspace, (hipStream_t)stream), (hipStream_t)stream);
}

ha_status hybrid_attn_forward_mix(const void* q, const void* k, const void* v, const void* qp,
                                  const void* kp, const void* vp, const float* alpha,
                                  const float* beta, float* state, void* out, const float* mix,
                                  void* workspace, size_t workspace_bytes, int B, int H, int T, int d,
                                  int frame_len, ha_dtype dtype, int update_state, float softmax_scale,
                                  void* stream) {
  const ForwardArgs a{q, k, v, qp, kp, vp, alpha, beta, state, out, B, H, T, d, frame_len, dtype, update_state,
                      softmax_scale, mix};
  ha::Shape s;
  size_t need = 0;
  if (!mix) return check_shape(B, H, T, d, frame_len, dtype, &s) != HA_OK ? HA_ERR_SHAPE : HA_ERR_NULL;
  ha_status r = validate_forward(a, &s, &need);
  if (r != HA_OK) return r;
  if (update_state && !aligned(workspace, 16)) return HA_ERR_ALIGN;
  if (need > 0 && (!workspace || workspace_bytes < need)) return HA_ERR_WORKSPACE;
  if (workspace_overlaps(a, s, workspace, need)) return HA_ERR_ALIAS;
  log_call("hybrid_attn_forward_mix", s, dtype, update_state, need);
  return debug_finish("hybrid_attn_forward_mix", launch_forward(a, s, workspace, (hipStream_t)stream),
                      (hipStream_t)stream);
}

}  // extern "C"

// ---- feature-map variant (fmap.hip): the layer with Q' = Q W_q, K' = K W_k,
// V' = V W_v folded into the kernels instead of materialised.
//   update_state = 0 : M = W_q S once per (b, h), then the readout kernel on
//                      Q and the fragments of M for every frame.
//   update_state = 1 : gram pass on K, V (fp32 partial sums), the transform to
//                      the increments under the maps, the scan (fp32
//                      snapshots S_{n-1}, S_F into `state`), M_n = W_q S_{n-1}
//                      for every frame, then the readout on Q and M_n; with
//                      more than 256 attention work-groups the scan runs in
//                      the readout's launch and publishes M_n itself.
// The gated variant (gates.hip) first computes alpha and beta from the layer
// input x and, for normalised keys, the two step-size vectors beta / n^2 and
// beta / n (keyscale), then runs the same passes.
namespace {
struct FmapWs {
  size_t gram, partial, snaps, mfrag, flags;
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
  w.flags = w.mfrag + align_up((size_t)s.B * s.H * s.F * dd * 2);  // counters of the fused scan
  w.total = w.flags + align_up((size_t)s.B * s.H * s.F * sizeof(unsigned));
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
  if (ha::attn_groups(s) > ha::kAttnLoaderMaxGroups) {
    // the scan runs in the readout's launch and publishes M_n = W_q S_{n-1}
    // of every frame as its readout fragments (as the plain forward call does
    // with S_{n-1}); the map transform zeroes the frame counters
    unsigned* flags = (unsigned*)(ws + lay.flags);
    if (ha::launch_gram_fmap(partial, nsplit, wk, wv, gram, s, st, flags) != hipSuccess) return HA_ERR_DEVICE;
    const ha_status r =
        launched(ha::launch_attn_scan_bf16(q, k, v, q, gram, alpha, state, mf, flags, out, s, scale, st, wq));
    return r != HA_OK ? r : check_finite("state", state, (size_t)s.B * s.H * (size_t)dd, st);
  }
  if (ha::launch_gram_fmap(partial, nsplit, wk, wv, gram, s, st) != hipSuccess) return HA_ERR_DEVICE;
  if (ha::launch_state_scan_bf16(gram, alpha, state, snaps, nullptr, s, st) != hipSuccess) return HA_ERR_DEVICE;
  if (ha::launch_mfrag(snaps, (long long)s.F * dd, dd, wq, mf, s.F, s, st) != hipSuccess) return HA_ERR_DEVICE;
  const ha_status r = run_readout(q, k, v, q, nullptr, (long long)s.F * fb, fb, out, s, HA_BF16, scale, st, mf);
  return r != HA_OK ? r : check_finite("state", state, (size_t)s.B * s.H * (size_t)dd, st);
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
  const size_t ab = update_state ? (size_t)B * s.F * H * sizeof(float) : 0;
  const size_t bb = update_state ? (size_t)B * T * H * sizeof(float) : 0;
  const size_t uwb = update_state ? wb : 0;
  if (update_state ? written_overlaps({{out, tb}, {state, stb}, {workspace, lay.total}},
                                      {{q, tb}, {k, tb}, {v, tb}, {wq, wb}, {wk, uwb}, {wv, uwb}, {alpha, ab},
                                       {beta, bb}})
                   : written_overlaps({{out, tb}, {workspace, lay.total}},
                                      {{q, tb}, {k, tb}, {v, tb}, {wq, wb}, {state, stb}}))
    return HA_ERR_ALIAS;
  log_call("hybrid_attn_forward_fmap", s, dtype, update_state, lay.total);
  r = fmap_run(q, k, v, wq, wk, wv, alpha, beta, nullptr, state, out, (char*)workspace, lay, s, update_state,
               resolve_scale(softmax_scale, d), (hipStream_t)stream);
  return debug_finish("hybrid_attn_forward_fmap", r, (hipStream_t)stream);
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
  const size_t uwb = update_state ? wb : 0, bgb = update_state ? (size_t)2 * H * 4 : 0;
  if (update_state ? written_overlaps({{out, tb}, {state, stb}, {workspace, lay.total}},
                                      {{q, tb}, {k, tb}, {v, tb}, {wq, wb}, {wk, uwb}, {wv, uwb}, {x, xb},
                                       {w_gate, gb}, {b_gate, bgb}})
                   : written_overlaps({{out, tb}, {workspace, lay.total}},
                                      {{q, tb}, {k, tb}, {v, tb}, {wq, wb}, {state, stb}}))
    return HA_ERR_ALIAS;

  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  const float scale = resolve_scale(softmax_scale, d);
  log_call("hybrid_attn_forward_gated", s, dtype, update_state, lay.total);
  if (!update_state)
    return debug_finish("hybrid_attn_forward_gated",
                        fmap_run(q, k, v, wq, wk, wv, nullptr, nullptr, nullptr, state, out, ws, lay, s, 0, scale, st),
                        st);
  float* alpha = (float*)(ws + lay.alpha);
  float* beta = (float*)(ws + lay.beta);
  if (ha::launch_gates(x, w_gate, b_gate, alpha, beta, (float*)(ws + lay.apart), C, s, st) != hipSuccess)
    return HA_ERR_DEVICE;
  if (!normalize_k)
    return debug_finish("hybrid_attn_forward_gated",
                        fmap_run(q, k, v, wq, wk, wv, alpha, beta, nullptr, state, out, ws, lay, s, 1, scale, st), st);
  float* bgv = (float*)(ws + lay.beta_g);
  float* bbv = (float*)(ws + lay.beta_b);
  if (ha::launch_keyscale(k, wk, beta, bgv, bbv, s, st) != hipSuccess) return HA_ERR_DEVICE;
  return debug_finish("hybrid_attn_forward_gated",
                      fmap_run(q, k, v, wq, wk, wv, alpha, bgv, bbv, state, out, ws, lay, s, 1, scale, st), st);
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
  log_call("hybrid_attn_gates", s, dtype, 0, wsb);
  hipStream_t st = (hipStream_t)stream;
  return debug_finish("hybrid_attn_gates",
                      launched(ha::launch_gates(x, w_gate, b_gate, alpha, beta, (float*)workspace, C, s, st)), st);
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
  if (((long long)frame_index + s.F) * frame_len > kMaxItems) return 0;  // cache tokens in 32 bits
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
  log_call("hybrid_attn_kvcache_forward", s, dtype, 0, lay.total);
  if (ha::launch_kv_append(k, v, k_cache, v_cache, cap, frame_index * frame_len, s, st) != hipSuccess)
    return HA_ERR_DEVICE;
  char* ws = (char*)workspace;
  const ha_status r2 = launched(ha::launch_attn_kv_bf16(
      q, k_cache, v_cache, out, lay.total ? (float*)(ws + lay.part_o) : nullptr,
      lay.total ? (void*)(ws + lay.part_ml) : nullptr, lay.nsplit, cap, frame_index * frame_len, s,
      resolve_scale(softmax_scale, d), st));
  return debug_finish("hybrid_attn_kvcache_forward", r2, st);
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
  const size_t ab = (size_t)B * s.F * H * sizeof(float), bb = (size_t)B * T * H * sizeof(float);
  // the state is written only with update_state; it is read either way
  if (update_state ? written_overlaps({{out, tb}, {state, stb}, {workspace, total}},
                                      {{q, tb}, {k, tb}, {v, tb}, {qp, tb}, {kp, tb}, {vp, tb}, {alpha, ab},
                                       {beta, bb}})
                   : written_overlaps({{out, tb}, {workspace, total}},
                                      {{q, tb}, {k, tb}, {v, tb}, {qp, tb}, {kp, tb}, {vp, tb}, {alpha, ab},
                                       {beta, bb}, {state, stb}}))
    return HA_ERR_ALIAS;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* oint = (float*)(ws + tl_oint_offset(s));
  log_call("hybrid_attn_forward_token_level", s, dtype, update_state, total);
  if (ha::launch_token_level(qp, kp, vp, alpha, beta, state, ws + tl_frag_offset(s), oint, update_state, s, st) !=
      hipSuccess)
    return HA_ERR_DEVICE;
  r = launched(ha::launch_attn_kv_bf16(q, k, v, out, nullptr, nullptr, 1, T, -1, s, resolve_scale(softmax_scale, d),
                                       st, oint));
  return debug_finish("hybrid_attn_forward_token_level",
                      r != HA_OK || !update_state ? r : check_finite("state", state, stb / sizeof(float), st), st);
}

}  // extern "C"

// ---- allocation-free variant of hybrid_attn_forward, for callers that cannot
// allocate (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc): the workspace is a fixed device array of this library instead of
// a caller buffer. Every call on one GPU shares that GPU's copy.
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per GPU
// The array's name is a host-side stand-in in host code: kernels get the
// per-device address that hipGetSymbolAddress returns, never `scratch`.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device with
// that device current.
ha_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return HA_ERR_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HA_OK;
}

}  // namespace

extern "C" {

size_t hybrid_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

ha_status hybrid_attn_forward_noalloc(const void* q, const void* k, const void* v, const void* qp,
                                      const void* kp, const void* vp, const float* alpha,
                                      const float* beta, float* state, void* out, int B, int H, int T,
                                      int d, int frame_len, ha_dtype dtype, int update_state,
                                      float softmax_scale, void* stream) {
  const ForwardArgs a{q, k, v, qp, kp, vp, alpha, beta, state, out, B, H, T, d, frame_len, dtype, update_state,
                      softmax_scale};
  ha::Shape s;
  size_t need = 0;
  ha_status r = validate_forward(a, &s, &need);
  if (r != HA_OK) return r;
  if (need > kScratchBytes) return HA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && (r = scratch_of_current_device(&ws)) != HA_OK) return r;
  if (workspace_overlaps(a, s, ws, need)) return HA_ERR_ALIAS;
  log_call("hybrid_attn_forward_noalloc", s, dtype, update_state, need);
  return debug_finish("hybrid_attn_forward_noalloc",
                      launch_forward(a, s, ws, (hipStream_t)stream), (hipStream_t)stream);
}

}  // extern "C"
