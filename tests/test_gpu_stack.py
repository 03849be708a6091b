"""The attention stack on an MI355X: its layers do exactly what the standalone
entry points do (bitwise), and the softmax layers' output matches the oracle."""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.hybrid_oracle as O
from tests.gpu_util import TOL_OUT, rel_err
from video_dit_hybrid_amd import api
from video_dit_hybrid_amd import workloads as W
from video_dit_hybrid_amd.stack import AttentionStack, layer_kinds

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_stack_layers_match_standalone_calls():
    w = dataclasses.replace(W.WORKLOADS["stream"], L=200, H=2, frames=3, denoise_passes=1)
    kinds = layer_kinds(4, 0.5)
    say(f"case stack {kinds}")
    B, H, d, L, F = w.B, w.H, w.d, w.L, w.frames
    stack = AttentionStack(kinds, B, H, d, L, F)
    frames = []
    for n in range(F):
        passes = []
        for p in range(2):
            inp = W.make_call_inputs(w, n, 1, p, clean=(p == 1))
            passes.append({k: W.as_torch(v, "bf16" if k in W.QKV_NAMES else "fp32") for k, v in inp.items()})
        frames.append(passes)
        out = torch.empty_like(passes[0]["q"])
        stack.run_frame(n, passes, out)
    torch.cuda.synchronize()
    # standalone: one hybrid layer and one softmax layer over the same frames
    st = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    kc = torch.empty((B, F * L, H, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    for n, passes in enumerate(frames):
        for p, t in enumerate(passes):
            if p == 1:
                o_h = api.hybrid_attn_forward(t["q"], t["k"], t["v"], t["qp"], t["kp"], t["vp"], t["alpha"],
                                              t["beta"], st, L, 1)
            else:
                api.hybrid_attn_forward(t["q"], t["k"], t["v"], t["qp"], None, None, None, None, st, L, 0)
            o_s = api.hybrid_attn_kvcache_forward(t["q"], t["k"], t["v"], kc, vc, L, n)
    torch.cuda.synchronize()
    for kind, s, c in zip(stack.kinds, stack.states, stack.caches):
        if kind == "hybrid":
            assert torch.equal(s, st)
        else:
            assert torch.equal(c[0], kc) and torch.equal(c[1], vc)
    assert torch.equal(out, o_h)  # the last layer is hybrid
    # the softmax layer's last output against the oracle (clean past + this frame)
    got = W.to_f64(W.from_torch(o_s, "bf16"), "bf16")
    K = W.to_f64(W.from_torch(kc, "bf16"), "bf16")
    V = W.to_f64(W.from_torch(vc, "bf16"), "bf16")
    q = W.to_f64(W.from_torch(frames[-1][1]["q"], "bf16"), "bf16")
    err = max(rel_err(got[0, :, h], O.intra_frame_attention(q[0, :, h], K[0, :, h], V[0, :, h])) for h in range(H))
    say(f"stack softmax layer: rel_err {err:.3e}; state bytes {stack.state_bytes()}, cache bytes {stack.cache_bytes(F)}")
    assert err < TOL_OUT
    assert stack.state_bytes() == 2 * B * H * d * d * 4 and stack.cache_bytes(F) == 2 * 2 * B * F * L * H * d * 2
