"""Helpers of the GPU parity tests: upload generator bytes, run the HIP path,
slice the fp64 oracle per (stream, head), and the error metric."""
from __future__ import annotations

import numpy as np

import oracle.hybrid_oracle as O
from video_dit_hybrid_amd import api
from video_dit_hybrid_amd import workloads as W

# Tolerances: max|x - r| / max|r| over a tensor (or over a sampled slab of it).
TOL_OUT = 2e-2
TOL_STATE = 1e-3


def rel_err(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(x - r)) / (den if den > 0 else 1.0))


def upload(inp: dict, dtype: str, device="cuda"):
    return {k: W.as_torch(v, dtype if k not in ("alpha", "beta") else "fp32", device)
            for k, v in inp.items()}


def run_gpu(inp_dev: dict, state_dev, frame_len: int, update: bool, scale=0.0, **kw):
    return api.hybrid_attn_forward(inp_dev["q"], inp_dev["k"], inp_dev["v"], inp_dev["qp"],
                                   inp_dev.get("kp"), inp_dev.get("vp"), inp_dev.get("alpha"),
                                   inp_dev.get("beta"), state_dev, frame_len, int(update),
                                   softmax_scale=scale, **kw)


def f64(inp: dict, dtype: str) -> dict:
    return {k: (W.to_f64(v, dtype) if k not in ("alpha", "beta") else v.astype(np.float64))
            for k, v in inp.items()}


def oracle_head(x: dict, state0, b: int, h: int, L: int, update: bool, frames=None, scale=None):
    """fp64 oracle for one (stream, head): (out [T, d], final state [d, d])."""
    g = lambda k: x[k][b, :, h] if k in x else None
    a = x["alpha"][b, :, h] if "alpha" in x else None
    bt = x["beta"][b, :, h] if "beta" in x else None
    return O.hybrid_layer_head(g("q"), g("k"), g("v"), g("qp"), g("kp"), g("vp"), a, bt,
                               np.asarray(state0[b, h], dtype=np.float64), L, update,
                               scale=scale, frames=frames)
