"""Per-branch output weights (hybrid_attn_forward_mix) on the GPU against the
fp64 oracle (hybrid_layer_mixed): random weights per (stream, head), the
LinVideo and SALAD pairs, ragged frames, d = 64, and the stack harness."""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.hybrid_oracle as O
from tests.gpu_util import TOL_OUT, TOL_STATE, f64, rel_err, run_gpu, upload
from video_dit_hybrid_amd import api
from video_dit_hybrid_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def mixed_call(w, mix, update=True, seed_pass=0):
    inp = W.make_call_inputs(w, 0, w.frames, seed_pass, clean=True)
    dev = upload(inp, "bf16")
    s0 = W.make_state0(w)
    st = torch.from_numpy(s0.copy()).cuda()
    m = torch.from_numpy(np.ascontiguousarray(mix, dtype=np.float32)).cuda()
    out = api.hybrid_attn_forward_mix(dev["q"], dev["k"], dev["v"], dev["qp"], dev["kp"], dev["vp"], dev["alpha"],
                                      dev["beta"], st, w.L, int(update), m)
    torch.cuda.synchronize()
    x = f64(inp, "bf16")
    ref, sref = O.hybrid_layer_mixed(x["q"], x["k"], x["v"], x["qp"], x["kp"], x["vp"], x["alpha"], x["beta"],
                                     s0.astype(np.float64), w.L, int(update), np.asarray(mix, dtype=np.float64))
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    return got, ref, st.cpu().numpy().astype(np.float64), sref, dev, s0


@pytest.mark.parametrize("L,F,B,H,d", [(200, 3, 2, 3, 128), (129, 2, 1, 2, 64), (1560, 1, 1, 12, 128),
                                       (1, 3, 1, 2, 128)])
def test_mix_random_weights(L, F, B, H, d):
    w = dataclasses.replace(W.WORKLOADS["480p"], B=B, H=H, d=d, L=L, frames=F, state0_sigma=0.05)
    mix = np.random.default_rng(L + F).uniform(-0.5, 1.5, size=(B, H, 2))
    say(f"case mix L={L} F={F} B={B} H={H} d={d}")
    got, ref, S, sref, *_ = mixed_call(w, mix)
    eo = rel_err(got, ref)
    es = rel_err(S, sref)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


@pytest.mark.parametrize("kind", ["linvideo", "salad"])
def test_mix_pages_pairs(kind):
    # LinVideo (r, 1 - r) with r per layer (one value for every head); SALAD
    # (1, s) with s in (0, 1) per stream
    w = dataclasses.replace(W.WORKLOADS["480p"], B=2, H=4, L=300, frames=2, state0_sigma=0.05)
    if kind == "linvideo":
        r = 0.3
        mix = np.tile([r, 1.0 - r], (w.B, w.H, 1))
    else:
        s = 1.0 / (1.0 + np.exp(-np.array([0.4, -1.2])))
        mix = np.stack([np.ones((w.B, w.H)), np.repeat(s[:, None], w.H, axis=1)], axis=-1)
    say(f"case mix {kind}")
    got, ref, S, sref, *_ = mixed_call(w, mix)
    assert rel_err(got, ref) < TOL_OUT and rel_err(S, sref) < TOL_STATE


def test_mix_leaves_the_state_path_and_unit_weights_give_the_plain_layer():
    # the weights only touch the output: the state equals the plain forward's
    # bitwise; weights (1, 1) give the plain output to the output tolerance
    # (the readout is summed in a separate accumulator, so rounding differs)
    w = dataclasses.replace(W.WORKLOADS["480p"], H=3, L=520, frames=3, state0_sigma=0.05)
    say("case mix state path")
    mix = np.ones((w.B, w.H, 2))
    got, ref, S, sref, dev, s0 = mixed_call(w, mix)
    st = torch.from_numpy(s0.copy()).cuda()
    plain = run_gpu(dev, st, w.L, True)
    torch.cuda.synchronize()
    assert np.array_equal(S, st.cpu().numpy().astype(np.float64))
    p = W.to_f64(W.from_torch(plain, "bf16"), "bf16")
    assert rel_err(got, p) < TOL_OUT and rel_err(got, ref) < TOL_OUT


def test_stack_with_mixed_layers():
    from video_dit_hybrid_amd.stack import AttentionStack, layer_kinds
    w = dataclasses.replace(W.WORKLOADS["stream"], L=200, H=2, frames=2, denoise_passes=1)
    kinds = layer_kinds(4, 0.5)
    say(f"case stack with per-layer LinVideo weights {kinds}")
    rs = [0.25, 0.5, 0.75, 1.0]
    mixes = [torch.tensor(np.tile([r, 1 - r], (w.B, w.H, 1)), dtype=torch.float32, device="cuda") for r in rs]
    stack = AttentionStack(kinds, w.B, w.H, w.d, w.L, w.frames, mix_weights=mixes)
    st = torch.zeros((w.B, w.H, w.d, w.d), dtype=torch.float32, device="cuda")
    last_h = max(i for i, k in enumerate(kinds) if k == "hybrid")
    for n in range(w.frames):
        passes = []
        for p in range(2):
            inp = W.make_call_inputs(w, n, 1, p, clean=(p == 1))
            passes.append({k: W.as_torch(v, "bf16" if k in W.QKV_NAMES else "fp32") for k, v in inp.items()})
        out = torch.empty_like(passes[0]["q"])
        stack.run_frame(n, passes, out)
        for p, t in enumerate(passes):  # the last hybrid layer on its own
            upd = (t["kp"], t["vp"], t["alpha"], t["beta"]) if p == 1 else (None, None, None, None)
            o_h = api.hybrid_attn_forward_mix(t["q"], t["k"], t["v"], t["qp"], *upd, st, w.L, int(p == 1),
                                              mixes[last_h])
    torch.cuda.synchronize()
    assert torch.equal(stack.states[last_h], st)
    if kinds[-1] == "hybrid":
        assert torch.equal(out, o_h)
