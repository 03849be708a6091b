"""Thin ctypes binding of libhybrid_attn.so (the C ABI in include/hybrid_attn.h).

Only argument marshalling lives here: checks of device, dtype, shape and
contiguity, allocation of the output and the workspace through PyTorch, and
the current HIP stream. Every step of the layer runs in the HIP kernels.
There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HA_BF16, HA_FP32 = 0, 1
STATUS = {0: "HA_OK", 1: "HA_ERR_NULL", 2: "HA_ERR_SHAPE", 3: "HA_ERR_UNSUPPORTED",
          4: "HA_ERR_ALIGN", 5: "HA_ERR_WORKSPACE", 6: "HA_ERR_DEVICE", 7: "HA_ERR_ALIAS", 8: "HA_ERR_SCRATCH",
          9: "HA_ERR_NONFINITE"}
EXPORTS = ("hybrid_attn_forward", "hybrid_attn_workspace_bytes", "hybrid_attn_intra_readout",
           "hybrid_attn_state_update", "hybrid_attn_state_workspace_bytes",
           "hybrid_attn_status_string", "hybrid_attn_version", "hybrid_attn_forward_fmap",
           "hybrid_attn_fmap_workspace_bytes", "hybrid_attn_forward_gated",
           "hybrid_attn_gated_workspace_bytes", "hybrid_attn_gates", "hybrid_attn_gates_workspace_bytes",
           "hybrid_attn_kvcache_forward", "hybrid_attn_kvcache_workspace_bytes",
           "hybrid_attn_forward_token_level", "hybrid_attn_token_level_workspace_bytes",
           "hybrid_attn_forward_noalloc", "hybrid_attn_noalloc_scratch_bytes", "hybrid_attn_forward_mix")

_PKG = os.path.dirname(os.path.abspath(__file__))
# HYBRID_ATTN_LIBRARY=debug selects the build with device index checks
# (libhybrid_attn_debug.so, built beside the release library)
LIB_PATH = os.path.join(_PKG, "libhybrid_attn_debug.so" if os.environ.get("HYBRID_ATTN_LIBRARY") == "debug"
                        else "libhybrid_attn.so")
_lib = None


class HybridAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load the HIP library once; raise if it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m video_dit_hybrid_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz, f, ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_longlong
    L.hybrid_attn_forward.argtypes = [vp] * 10 + [vp, sz, i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_forward.restype = i
    L.hybrid_attn_forward_mix.argtypes = [vp] * 11 + [vp, sz, i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_forward_mix.restype = i
    L.hybrid_attn_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.hybrid_attn_workspace_bytes.restype = sz
    L.hybrid_attn_intra_readout.argtypes = [vp, vp, vp, vp, vp, ll, ll, vp, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_intra_readout.restype = i
    L.hybrid_attn_state_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, vp]
    L.hybrid_attn_state_update.restype = i
    L.hybrid_attn_state_workspace_bytes.argtypes = [i, i, i, i, i]
    L.hybrid_attn_state_workspace_bytes.restype = sz
    L.hybrid_attn_forward_fmap.argtypes = [vp] * 10 + [vp, sz, i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_forward_fmap.restype = i
    L.hybrid_attn_fmap_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.hybrid_attn_fmap_workspace_bytes.restype = sz
    L.hybrid_attn_forward_gated.argtypes = [vp] * 11 + [vp, sz, i, i, i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_forward_gated.restype = i
    L.hybrid_attn_gated_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.hybrid_attn_gated_workspace_bytes.restype = sz
    L.hybrid_attn_gates.argtypes = [vp] * 5 + [vp, sz, i, i, i, i, i, i, vp]
    L.hybrid_attn_gates.restype = i
    L.hybrid_attn_gates_workspace_bytes.argtypes = [i, i, i, i]
    L.hybrid_attn_gates_workspace_bytes.restype = sz
    L.hybrid_attn_kvcache_forward.argtypes = [vp] * 7 + [sz, i, i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_kvcache_forward.restype = i
    L.hybrid_attn_kvcache_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.hybrid_attn_kvcache_workspace_bytes.restype = sz
    L.hybrid_attn_forward_token_level.argtypes = [vp] * 11 + [sz, i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_forward_token_level.restype = i
    L.hybrid_attn_token_level_workspace_bytes.argtypes = [i, i, i, i, i]
    L.hybrid_attn_token_level_workspace_bytes.restype = sz
    L.hybrid_attn_forward_noalloc.argtypes = [vp] * 10 + [i, i, i, i, i, i, i, f, vp]
    L.hybrid_attn_forward_noalloc.restype = i
    L.hybrid_attn_noalloc_scratch_bytes.argtypes = []
    L.hybrid_attn_noalloc_scratch_bytes.restype = sz
    L.hybrid_attn_status_string.argtypes = [i]
    L.hybrid_attn_status_string.restype = ctypes.c_char_p
    L.hybrid_attn_version.argtypes = []
    L.hybrid_attn_version.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().hybrid_attn_status_string(int(status)).decode()


def workspace_bytes(B, H, T, frame_len, d, update_state) -> int:
    return int(lib().hybrid_attn_workspace_bytes(B, H, T, frame_len, d, int(bool(update_state))))


def state_workspace_bytes(B, H, T, frame_len, d) -> int:
    return int(lib().hybrid_attn_state_workspace_bytes(B, H, T, frame_len, d))


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HA_BF16
    if t.dtype == torch.float32:
        return HA_FP32
    raise TypeError(f"q..v' must be bfloat16 or float32, got {t.dtype}")


def _check(name, t, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _forward_args(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, out):
    """Checks of the forward call's tensors; returns (B, T, H, d, dtype code, out)."""
    torch = _torch()
    if q.device.type != "cuda":
        raise ValueError("hybrid_attn_forward runs on a GPU; tensors must be on a cuda device")
    B, T, H, d = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    F = T // frame_len if frame_len > 0 and T % frame_len == 0 else -1
    if F <= 0:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    for name, t in (("k", k), ("v", v), ("qp", qp)):
        _check(name, t, (B, T, H, d), dt, dev)
    _check("state", state, (B, H, d, d), torch.float32, dev)
    if update_state:
        for name, t in (("kp", kp), ("vp", vp)):
            _check(name, t, (B, T, H, d), dt, dev)
        _check("alpha", alpha, (B, F, H), torch.float32, dev)
        _check("beta", beta, (B, T, H), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, T, H, d), dt, dev)
    return B, T, H, d, code, out


def noalloc_scratch_bytes() -> int:
    return int(lib().hybrid_attn_noalloc_scratch_bytes())


def hybrid_attn_forward_noalloc(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, out,
                                softmax_scale: float = 0.0):
    """hybrid_attn_forward without a workspace argument: the library's fixed
    per-GPU scratch is used instead, and nothing is allocated (out must be
    given). Calls that overlap in time on one GPU race on that scratch."""
    B, T, H, d, code, out = _forward_args(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, out)
    st = lib().hybrid_attn_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(qp), _ptr(kp if update_state else None),
        _ptr(vp if update_state else None), _ptr(alpha if update_state else None),
        _ptr(beta if update_state else None), _ptr(state), _ptr(out), B, H, T, d, frame_len, code,
        int(bool(update_state)), float(softmax_scale), _stream(q.device))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_forward_noalloc")
    return out


def hybrid_attn_forward(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state,
                        softmax_scale: float = 0.0, out=None, workspace=None):
    """The layer call: returns out [B,T,H,d]; with update_state the fp32 state
    [B,H,d,d] is advanced in place to S_F, otherwise it is left unchanged.
    Layouts as in include/hybrid_attn.h. Asynchronous on the current stream."""
    return _forward_call(lib().hybrid_attn_forward, "hybrid_attn_forward", q, k, v, qp, kp, vp, alpha, beta, state,
                         frame_len, update_state, softmax_scale, out, workspace)


def _forward_call(fn, name, q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, softmax_scale, out,
                  workspace, mix=None):
    """Checks, output and workspace allocation of a forward call, then the
    call of fn (hybrid_attn_forward, or hybrid_attn_forward_mix with mix)."""
    torch = _torch()
    if q.device.type != "cuda":
        raise ValueError(f"{name} runs on a GPU; tensors must be on a cuda device")
    B, T, H, d = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    F = T // frame_len if frame_len > 0 and T % frame_len == 0 else -1
    if F <= 0:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    for nm, t in (("k", k), ("v", v), ("qp", qp)):
        _check(nm, t, (B, T, H, d), dt, dev)
    _check("state", state, (B, H, d, d), torch.float32, dev)
    if update_state:
        for nm, t in (("kp", kp), ("vp", vp)):
            _check(nm, t, (B, T, H, d), dt, dev)
        _check("alpha", alpha, (B, F, H), torch.float32, dev)
        _check("beta", beta, (B, T, H), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, T, H, d), dt, dev)
    need = workspace_bytes(B, H, T, frame_len, d, update_state)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = [_ptr(q), _ptr(k), _ptr(v), _ptr(qp), _ptr(kp if update_state else None),
            _ptr(vp if update_state else None), _ptr(alpha if update_state else None),
            _ptr(beta if update_state else None), _ptr(state), _ptr(out)]
    if mix is not None:
        head.append(_ptr(mix))
    st = fn(*head, _ptr(workspace), ws_bytes, B, H, T, d, frame_len, code, int(bool(update_state)),
            float(softmax_scale), _stream(dev))
    if st != 0:
        raise HybridAttnError(st, name)
    return out


def hybrid_attn_forward_mix(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, mix,
                            softmax_scale: float = 0.0, out=None, workspace=None):
    """hybrid_attn_forward with per-branch output weights: mix fp32 [B, H, 2]
    holds (w_softmax, w_inter) per (stream, head); out = w_softmax O_intra +
    w_inter O_inter. bf16 only."""
    torch = _torch()
    B, T, H, d = q.shape
    _check("mix", mix, (B, H, 2), torch.float32, q.device)
    return _forward_call(lib().hybrid_attn_forward_mix, "hybrid_attn_forward_mix", q, k, v, qp, kp, vp, alpha, beta,
                         state, frame_len, update_state, softmax_scale, out, workspace, mix)


def fmap_workspace_bytes(B, H, T, frame_len, d, update_state) -> int:
    return int(lib().hybrid_attn_fmap_workspace_bytes(B, H, T, frame_len, d, int(bool(update_state))))


def hybrid_attn_forward_fmap(q, k, v, wq, wk, wv, alpha, beta, state, frame_len, update_state,
                             softmax_scale: float = 0.0, out=None, workspace=None):
    """The layer with the per-head feature maps W_q, W_k, W_v ([H, d, d], same
    dtype as q) applied inside the call: as hybrid_attn_forward with
    Q' = Q W_q, K' = K W_k, V' = V W_v, none of which is materialised."""
    torch = _torch()
    if q.device.type != "cuda":
        raise ValueError("hybrid_attn_forward_fmap runs on a GPU; tensors must be on a cuda device")
    B, T, H, d = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    F = T // frame_len if frame_len > 0 and T % frame_len == 0 else -1
    if F <= 0:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, T, H, d), dt, dev)
    _check("wq", wq, (H, d, d), dt, dev)
    _check("state", state, (B, H, d, d), torch.float32, dev)
    if update_state:
        for name, t in (("wk", wk), ("wv", wv)):
            _check(name, t, (H, d, d), dt, dev)
        _check("alpha", alpha, (B, F, H), torch.float32, dev)
        _check("beta", beta, (B, T, H), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, T, H, d), dt, dev)
    need = fmap_workspace_bytes(B, H, T, frame_len, d, update_state)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().hybrid_attn_forward_fmap(
        _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk if update_state else None),
        _ptr(wv if update_state else None), _ptr(alpha if update_state else None),
        _ptr(beta if update_state else None), _ptr(state), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, T, d, frame_len, code,
        int(bool(update_state)), float(softmax_scale), _stream(dev))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_forward_fmap")
    return out



def gated_workspace_bytes(B, H, T, frame_len, d, update_state) -> int:
    return int(lib().hybrid_attn_gated_workspace_bytes(B, H, T, frame_len, d, int(bool(update_state))))


def gates_workspace_bytes(B, H, T, frame_len) -> int:
    return int(lib().hybrid_attn_gates_workspace_bytes(B, H, T, frame_len))


def hybrid_attn_gates(x, w_gate, b_gate, H, frame_len, alpha=None, beta=None, workspace=None):
    """alpha [B, F, H] and beta [B, T, H] (fp32) from the layer input x
    [B, T, C] and the headwise gate projections w_gate [2, H, C] (x's dtype),
    b_gate [2, H] fp32."""
    torch = _torch()
    if x.device.type != "cuda":
        raise ValueError("hybrid_attn_gates runs on a GPU; tensors must be on a cuda device")
    B, T, C = x.shape
    dev = x.device
    code = _dtype_code(x)
    F = T // frame_len if frame_len > 0 and T % frame_len == 0 else -1
    if F <= 0:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    _check("w_gate", w_gate, (2, H, C), x.dtype, dev)
    _check("b_gate", b_gate, (2, H), torch.float32, dev)
    if alpha is None:
        alpha = torch.empty((B, F, H), dtype=torch.float32, device=dev)
    if beta is None:
        beta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _check("alpha", alpha, (B, F, H), torch.float32, dev)
    _check("beta", beta, (B, T, H), torch.float32, dev)
    need = gates_workspace_bytes(B, H, T, frame_len)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().hybrid_attn_gates(_ptr(x), _ptr(w_gate), _ptr(b_gate), _ptr(alpha), _ptr(beta), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), B, H, T, C, frame_len, code,
                                 _stream(dev))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_gates")
    return alpha, beta


def hybrid_attn_forward_gated(x, q, k, v, wq, wk, wv, w_gate, b_gate, state, frame_len, update_state,
                              normalize_k=True, softmax_scale: float = 0.0, out=None, workspace=None):
    """The layer with its gates projected from x [B, T, C] (w_gate [2, H, C],
    b_gate [2, H] fp32) and the per-head feature maps applied inside the call
    (K' L2-normalised per token when normalize_k); on a denoising pass
    (update_state 0) x, wk, wv and the gate weights are not read."""
    torch = _torch()
    if q.device.type != "cuda":
        raise ValueError("hybrid_attn_forward_gated runs on a GPU; tensors must be on a cuda device")
    B, T, H, d = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    F = T // frame_len if frame_len > 0 and T % frame_len == 0 else -1
    if F <= 0:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, T, H, d), dt, dev)
    _check("wq", wq, (H, d, d), dt, dev)
    _check("state", state, (B, H, d, d), torch.float32, dev)
    C = 0
    if update_state:
        C = x.shape[-1]
        _check("x", x, (B, T, C), dt, dev)
        for name, t in (("wk", wk), ("wv", wv)):
            _check(name, t, (H, d, d), dt, dev)
        _check("w_gate", w_gate, (2, H, C), dt, dev)
        _check("b_gate", b_gate, (2, H), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, T, H, d), dt, dev)
    need = gated_workspace_bytes(B, H, T, frame_len, d, update_state)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    u = bool(update_state)
    st = lib().hybrid_attn_forward_gated(
        _ptr(x if u else None), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk if u else None),
        _ptr(wv if u else None), _ptr(w_gate if u else None), _ptr(b_gate if u else None), _ptr(state),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, T, d, C, frame_len,
        code, int(u), int(bool(normalize_k)), float(softmax_scale), _stream(dev))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_forward_gated")
    return out


def kvcache_workspace_bytes(B, H, T, frame_len, d, frame_index) -> int:
    return int(lib().hybrid_attn_kvcache_workspace_bytes(B, H, T, frame_len, d, frame_index))


def hybrid_attn_kvcache_forward(q, k, v, k_cache, v_cache, frame_len, frame_index, softmax_scale: float = 0.0,
                                out=None, workspace=None):
    """Softmax attention with a full KV cache: k, v ([B, T, H, d]) are written
    into the caches ([B, cache_frames * frame_len, H, d]) at frame
    frame_index, then frame n of the call attends to the cache's first
    (frame_index + n + 1) * frame_len keys."""
    torch = _torch()
    if q.device.type != "cuda":
        raise ValueError("hybrid_attn_kvcache_forward runs on a GPU; tensors must be on a cuda device")
    B, T, H, d = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    if frame_len <= 0 or T % frame_len:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    cap_t = k_cache.shape[1]
    if cap_t % frame_len:
        raise ValueError("the cache length must be a multiple of frame_len")
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, T, H, d), dt, dev)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check(name, t, (B, cap_t, H, d), dt, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, T, H, d), dt, dev)
    need = kvcache_workspace_bytes(B, H, T, frame_len, d, frame_index)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().hybrid_attn_kvcache_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                           _ptr(workspace), wsb, B, H, T, d, frame_len, cap_t // frame_len,
                                           frame_index, code, float(softmax_scale), _stream(dev))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_kvcache_forward")
    return out


def token_level_workspace_bytes(B, H, T, frame_len, d) -> int:
    return int(lib().hybrid_attn_token_level_workspace_bytes(B, H, T, frame_len, d))


def hybrid_attn_forward_token_level(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state,
                                    softmax_scale: float = 0.0, out=None, workspace=None):
    """The layer with token-level access (per-token gated delta rule; the
    alternative to frame-level access), same arguments as hybrid_attn_forward;
    kp, vp, alpha, beta are required also when update_state is 0."""
    torch = _torch()
    if q.device.type != "cuda":
        raise ValueError("hybrid_attn_forward_token_level runs on a GPU; tensors must be on a cuda device")
    B, T, H, d = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    F = T // frame_len if frame_len > 0 and T % frame_len == 0 else -1
    if F <= 0:
        raise ValueError(f"T={T} must be a positive multiple of frame_len={frame_len}")
    for name, t in (("k", k), ("v", v), ("qp", qp), ("kp", kp), ("vp", vp)):
        _check(name, t, (B, T, H, d), dt, dev)
    _check("alpha", alpha, (B, F, H), torch.float32, dev)
    _check("beta", beta, (B, T, H), torch.float32, dev)
    _check("state", state, (B, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, T, H, d), dt, dev)
    need = token_level_workspace_bytes(B, H, T, frame_len, d)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().hybrid_attn_forward_token_level(
        _ptr(q), _ptr(k), _ptr(v), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, T, d, frame_len, code,
        int(bool(update_state)), float(softmax_scale), _stream(dev))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_forward_token_level")
    return out

def hybrid_attn_intra_readout(q, k, v, qp, states, state_stride_bh, state_stride_frame,
                              frame_len, softmax_scale: float = 0.0, out=None):
    """Read side only: out = softmax-within-frame(QK^T s)V + Q' S_n, with S_n the
    fp32 d x d block at states + b*stride_bh + n*stride_frame (in floats)."""
    B, T, H, d = q.shape
    code = _dtype_code(q)
    if out is None:
        out = _torch().empty_like(q)
    st = lib().hybrid_attn_intra_readout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(qp), _ptr(states), int(state_stride_bh),
        int(state_stride_frame), _ptr(out), B, H, T, d, frame_len, code, float(softmax_scale),
        _stream(q.device))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_intra_readout")
    return out


def hybrid_attn_state_update(kp, vp, alpha, beta, state, frame_len, snapshots=None, workspace=None):
    """Write side only: advance the fp32 state in place over the frames of
    kp, vp, alpha, beta; optionally write S_{n-1} of every frame to snapshots
    [B,H,F,d,d]."""
    torch = _torch()
    B, T, H, d = kp.shape
    code = _dtype_code(kp)
    need = state_workspace_bytes(B, H, T, frame_len, d)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=kp.device)
    st = lib().hybrid_attn_state_update(
        _ptr(kp), _ptr(vp), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(snapshots),
        _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, T, d, frame_len,
        code, _stream(kp.device))
    if st != 0:
        raise HybridAttnError(st, "hybrid_attn_state_update")
    return state
