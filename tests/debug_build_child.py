"""Child process of test_gpu_debug_build: every main-path entry point of the
debug library (device index checks on, HYBRID_ATTN_LIBRARY=debug) on the edge
shapes. Each call synchronises and raises if an index check failed; the
results of one case are compared with the fp64 oracle."""
import dataclasses
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle.hybrid_oracle as O  # noqa: E402
from video_dit_hybrid_amd import api  # noqa: E402
from video_dit_hybrid_amd import workloads as W  # noqa: E402

assert api.LIB_PATH.endswith("libhybrid_attn_debug.so"), api.LIB_PATH


def case(name, **kw):
    w = dataclasses.replace(W.WORKLOADS["480p"], **kw)
    print(f"debug case {name}: {kw}", flush=True)
    return w


def upload(inp):
    return {k: W.as_torch(v, "bf16" if k in W.QKV_NAMES else "fp32", "cuda") for k, v in inp.items()}


worst = 0.0
shapes = [("multi-frame", dict(H=2, L=200, frames=3)), ("ragged 129, d=64", dict(H=1, L=129, frames=2, d=64)),
          ("one token", dict(H=2, L=1, frames=3)), ("one frame, token splits", dict(H=12, L=1560, frames=1)),
          ("one frame, 513", dict(H=1, L=513, frames=1)), ("two streams", dict(B=2, H=3, L=300, frames=2))]
for name, kw in shapes:
    w = case(name, state0_sigma=0.05, **kw)
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    dev = upload(inp)
    s0 = W.make_state0(w)
    st = torch.from_numpy(s0.copy()).cuda()
    for update in (0, 1):
        out = api.hybrid_attn_forward(dev["q"], dev["k"], dev["v"], dev["qp"], dev["kp"], dev["vp"], dev["alpha"],
                                      dev["beta"], st, w.L, update)
    torch.cuda.synchronize()
    if name == "multi-frame":
        x = {k: (W.to_f64(v, "bf16") if k in W.QKV_NAMES else v.astype(np.float64)) for k, v in inp.items()}
        ref, sref = O.hybrid_layer(x["q"], x["k"], x["v"], x["qp"], x["kp"], x["vp"], x["alpha"], x["beta"],
                                   s0.astype(np.float64), w.L, 1)
        got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
        worst = max(worst, float(np.abs(got - ref).max() / np.abs(ref).max()))
    snaps = torch.empty((w.B, w.H, w.frames, w.d, w.d), device="cuda")
    api.hybrid_attn_state_update(dev["kp"], dev["vp"], dev["alpha"], dev["beta"], st, w.L, snapshots=snaps)
    api.hybrid_attn_intra_readout(dev["q"], dev["k"], dev["v"], dev["qp"], snaps, w.frames * w.d * w.d, w.d * w.d,
                                  w.L)
    torch.cuda.synchronize()
print(f"multi-frame rel_err out {worst:.3e}", flush=True)
assert worst < 2e-2
print("debug build: all index checks passed", flush=True)
