"""Seeded synthetic workloads for the hybrid attention layer.

This module holds the workload shapes and the seeded input generator that both
the GPU path's tests/bench and the CPU oracle consume. It contains none of the
layer's arithmetic: it only draws random tensors, L2-normalises the K' rows
(the inputs are defined as unit rows), squashes the gates through a sigmoid
(the gates are defined as sigmoid outputs), and rounds to the storage dtype.

Layouts (token-major, as a fused QKV projection of a DiT emits them):
  q, k, v, qp, kp, vp : [B, T, H, d]   T = F * L, frame n = tokens [nL, (n+1)L)
  alpha               : [B, F, H]      fp32, one forget gate per (stream, frame, head)
  beta                : [B, T, H]      fp32, one step size per (stream, token, head)
  state               : [B, H, d, d]   fp32, S[dk, dv] with dv contiguous
  x                   : [B, T, C]      the tokens' layer input (C = H * d), for the gates

Every slab is drawn from numpy PCG64 seeded with
SeedSequence([cfg_id, tensor_id, b, frame, pass]) so that any (stream, frame,
pass) can be regenerated alone, bit for bit, without drawing the rest.
bf16 tensors are returned as their raw uint16 bit patterns (round to nearest
even from the fp32 draw); fp32 tensors as float32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

# tensor ids used in the seed sequence
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "qp": 3, "kp": 4, "vp": 5,
              "alpha": 6, "beta": 7, "state": 8, "wq": 9, "wk": 10, "wv": 11,
              "x": 12, "wgate": 13, "bgate": 14}
QKV_NAMES = ("q", "k", "v", "qp", "kp", "vp")


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value distributions, pass schedule."""
    name: str
    cfg_id: int
    B: int
    H: int
    d: int
    frames: int          # frames in the whole run
    L: int               # tokens per frame
    dtype: str           # "bf16" or "fp32" for q,k,v,q',k',v'
    alpha_mu: float = 2.0
    alpha_sigma: float = 0.5
    beta_mu: float = 0.0
    beta_sigma: float = 1.0
    state0_sigma: float = 0.0   # 0 => S_0 = 0
    denoise_passes: int = 0     # query-only passes before the clean pass
    frames_per_call: int = 0    # 0 => all frames in one call

    @property
    def T(self) -> int:
        return self.frames * self.L

    @property
    def call_frames(self) -> int:
        return self.frames_per_call or self.frames


# The five workloads: a tiny fp32 case, a Wan-1.3B-shaped 480p layer (21 latent
# frames of a 30x52 patch grid), a 120-frame autoregressive stream, a
# Wan-14B-shaped 720p layer (45x80 grid) and an 8-stream single-frame step.
WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, H=2, d=64, frames=4, L=256, dtype="fp32"),
    "480p": Workload("480p", 1, B=1, H=12, d=128, frames=21, L=1560, dtype="bf16"),
    "stream": Workload("stream", 2, B=1, H=12, d=128, frames=120, L=1560, dtype="bf16",
                       denoise_passes=4, frames_per_call=1),
    "720p": Workload("720p", 3, B=1, H=40, d=128, frames=21, L=3600, dtype="bf16",
                     alpha_mu=3.0, beta_mu=-1.0),
    "batched": Workload("batched", 4, B=8, H=12, d=128, frames=1, L=1560, dtype="bf16",
                        state0_sigma=0.05, denoise_passes=4, frames_per_call=1),
}


def _rng(cfg_id: int, tensor: str, b: int, frame: int, pass_: int) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg_id, TENSOR_IDS[tensor], b, frame, pass_])
    return np.random.Generator(np.random.PCG64(ss))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (uint16 bf16 bits or float32) -> float64, exactly."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def draw_slab(w: Workload, tensor: str, b: int, frame: int, pass_: int) -> np.ndarray:
    """One (stream, frame, pass) slab of one tensor, in fp32 before rounding.

    q,k,v,qp,vp ~ N(0,1) [L,H,d]; kp the same then each (token, head) row
    scaled to unit L2 norm; beta = sigmoid(N(mu,sigma))/L [L,H];
    alpha = sigmoid(N(mu,sigma)) [H].
    """
    g = _rng(w.cfg_id, tensor, b, frame, pass_)
    if tensor in QKV_NAMES:
        x = g.standard_normal((w.L, w.H, w.d), dtype=np.float32)
        if tensor == "kp":
            n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
            x = (x / n).astype(np.float32)
        return x
    if tensor == "beta":
        z = g.normal(w.beta_mu, w.beta_sigma, size=(w.L, w.H)).astype(np.float32)
        return (_sigmoid(z) / np.float32(w.L)).astype(np.float32)
    if tensor == "alpha":
        z = g.normal(w.alpha_mu, w.alpha_sigma, size=(w.H,)).astype(np.float32)
        return _sigmoid(z)
    raise KeyError(tensor)


def make_state0(w: Workload) -> np.ndarray:
    """Initial state [B,H,d,d] fp32: zeros, or N(0, state0_sigma) per stream."""
    s = np.zeros((w.B, w.H, w.d, w.d), dtype=np.float32)
    if w.state0_sigma > 0:
        for b in range(w.B):
            g = _rng(w.cfg_id, "state", b, 0, 0)
            s[b] = g.normal(0.0, w.state0_sigma, size=(w.H, w.d, w.d)).astype(np.float32)
    return s


def make_fmap_weights(w: Workload) -> dict:
    """Per-head feature maps wq, wk, wv [H, d, d] for the feature-map variant,
    N(0, 1) entries scaled so that the mapped tensors keep the statistics of
    the plain workload's inputs when the unmapped ones are N(0, 1): wq and wv
    by 1/sqrt(d) (Q', V' entries about N(0, 1)), wk by 1/d (K' rows of about
    unit norm). Encoded like the other tensors (bf16 bits or fp32)."""
    out = {}
    for name, sc in (("wq", 1.0 / np.sqrt(w.d)), ("wk", 1.0 / w.d), ("wv", 1.0 / np.sqrt(w.d))):
        g = _rng(w.cfg_id, name, 0, 0, 0)
        x = (g.standard_normal((w.H, w.d, w.d)) * sc).astype(np.float32)
        out[name] = _encode(x, w.dtype)
    return out



def make_gate_weights(w: Workload) -> dict:
    """Headwise gate projections for the gated variant: wgate [2, H, C]
    (row 0 alpha, row 1 beta; N(0, 1/sqrt(C)) entries, so that a logit over an
    N(0, 1) input has unit variance), encoded like the other tensors; bgate
    [2, H] fp32 = the workload's alpha and beta logit means, so the gates have
    the plain workload's centres."""
    C = w.H * w.d
    g = _rng(w.cfg_id, "wgate", 0, 0, 0)
    wg = (g.standard_normal((2, w.H, C)) / np.sqrt(C)).astype(np.float32)
    bg = np.empty((2, w.H), dtype=np.float32)
    bg[0] = w.alpha_mu
    bg[1] = w.beta_mu
    return {"wgate": _encode(wg, w.dtype), "bgate": bg}


def make_layer_input(w: Workload, frame0: int, nframes: int, pass_: int, streams=None) -> np.ndarray:
    """x [nb, nframes * L, C] (C = H * d), N(0, 1) per (stream, frame) slab,
    encoded to the workload dtype."""
    streams = list(range(w.B)) if streams is None else list(streams)
    C = w.H * w.d
    out = np.empty((len(streams), nframes * w.L, C), dtype=np.uint16 if w.dtype == "bf16" else np.float32)

    def job(args):
        bi, b, fi = args
        g = _rng(w.cfg_id, "x", b, frame0 + fi, pass_)
        out[bi, fi * w.L:(fi + 1) * w.L] = _encode(g.standard_normal((w.L, C), dtype=np.float32), w.dtype)

    jobs = [(bi, b, fi) for bi, b in enumerate(streams) for fi in range(nframes)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, jobs))
    return out

def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_call_inputs(w: Workload, frame0: int, nframes: int, pass_: int,
                     clean: bool = True, streams=None, tensors=None) -> dict:
    """Inputs of one layer call covering frames [frame0, frame0+nframes).

    pass_ is the pass index within the frame (denoise passes 0..P-1, the clean
    pass P); single-pass workloads use pass 0. A denoise pass (clean=False)
    draws only q,k,v,q'; a clean pass also draws k',v',alpha,beta.
    Returns storage arrays in the layouts of the module docstring.
    """
    streams = list(range(w.B)) if streams is None else list(streams)
    names = list(tensors) if tensors is not None else (
        list(QKV_NAMES) + ["alpha", "beta"] if clean else ["q", "k", "v", "qp"])
    nb, L, H, d = len(streams), w.L, w.H, w.d
    out = {}
    for t in names:
        if t in QKV_NAMES:
            out[t] = np.empty((nb, nframes * L, H, d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
        elif t == "beta":
            out[t] = np.empty((nb, nframes * L, H), dtype=np.float32)
        elif t == "alpha":
            out[t] = np.empty((nb, nframes, H), dtype=np.float32)

    def job(args):
        t, bi, b, fi = args
        x = draw_slab(w, t, b, frame0 + fi, pass_)
        if t in QKV_NAMES:
            out[t][bi, fi * L:(fi + 1) * L] = _encode(x, w.dtype)
        elif t == "beta":
            out[t][bi, fi * L:(fi + 1) * L] = x
        else:
            out[t][bi, fi] = x

    jobs = [(t, bi, b, fi) for t in names for bi, b in enumerate(streams) for fi in range(nframes)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, jobs))
    return out


def call_schedule(w: Workload):
    """The sequence of layer calls of a whole run: (frame0, nframes, pass, clean)."""
    if w.frames_per_call == 0:
        return [(0, w.frames, 0, True)]
    sched = []
    for f in range(0, w.frames, w.frames_per_call):
        for p in range(w.denoise_passes):
            sched.append((f, w.frames_per_call, p, False))
        sched.append((f, w.frames_per_call, w.denoise_passes, True))
    return sched


def as_torch(x: np.ndarray, dtype: str, device="cuda"):
    """Storage array -> torch tensor on device, same bytes (bf16 bits are viewed, not converted)."""
    import torch
    if dtype == "bf16" and x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    """Device tensor -> storage array (bf16 as uint16 bits, fp32 as float32)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
