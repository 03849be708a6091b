"""Token-level access (hybrid_attn_forward_token_level) against the fp64
oracle (oracle.hybrid_oracle.hybrid_layer_token_level) on an MI355X, through
the C ABI. Bars as the other parity tests: 2e-2 on the output, 1e-3 on the
fp32 state."""
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


def run_tl(dev, st, L, update):
    return api.hybrid_attn_forward_token_level(dev["q"], dev["k"], dev["v"], dev["qp"], dev["kp"], dev["vp"],
                                               dev["alpha"], dev["beta"], st, L, int(update))


@pytest.mark.parametrize("L,F,B,H", [(300, 3, 1, 2), (64, 4, 2, 1), (17, 3, 1, 2), (130, 2, 1, 3)])
@pytest.mark.parametrize("update", [1, 0])
def test_token_level_parity(L, F, B, H, update):
    """Whole calls: full and partial 64-token chunks, frames of one partial
    chunk, two streams; clean and denoise."""
    w = dataclasses.replace(W.WORKLOADS["480p"], L=L, frames=F, B=B, H=H, state0_sigma=0.05)
    say(f"case token-level L={L} F={F} B={B} H={H} update={update}")
    inp = W.make_call_inputs(w, 0, F, 0)
    s0 = W.make_state0(w)
    dev = upload(inp, "bf16")
    st = torch.from_numpy(s0.copy()).cuda()
    out = run_tl(dev, st, L, update)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    S = st.cpu().numpy().astype(np.float64)
    x = f64(inp, "bf16")
    eo = es = 0.0
    for b in range(B):
        for h in range(H):
            ref, Sref = O.hybrid_layer_token_level(x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h],
                                                   x["qp"][b, :, h], x["kp"][b, :, h], x["vp"][b, :, h],
                                                   x["alpha"][b, :, h], x["beta"][b, :, h],
                                                   s0[b, h].astype(np.float64), L, update)
            eo = max(eo, rel_err(got[b, :, h], ref))
            es = max(es, rel_err(S[b, h], Sref))
    say(f"token-level: rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE
    if not update:
        assert np.array_equal(S, s0.astype(np.float64))


def test_token_level_one_token_frames_equal_frame_level():
    """frame_len = 1: token-level and frame-level access are the same layer;
    the two GPU paths agree closely (different arithmetic)."""
    w = dataclasses.replace(W.WORKLOADS["480p"], L=1, frames=40, B=1, H=2, state0_sigma=0.05)
    say("case token-level L=1")
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    dev = upload(inp, "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st1, st2 = s0.clone(), s0.clone()
    o1 = run_tl(dev, st1, 1, 1)
    o2 = run_gpu(dev, st2, 1, True)
    torch.cuda.synchronize()
    eo = rel_err(o1.float().cpu().numpy(), o2.float().cpu().numpy())
    es = rel_err(st1.cpu().numpy(), st2.cpu().numpy())
    say(f"token-level vs frame-level at L=1: out {eo:.3e} state {es:.3e}")
    assert eo < 1e-2 and es < 1e-4


def test_token_level_denoise_output_equals_clean_output():
    w = dataclasses.replace(W.WORKLOADS["480p"], L=200, frames=2, B=1, H=2, state0_sigma=0.05)
    say("case token-level denoise vs clean")
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    dev = upload(inp, "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st = s0.clone()
    o0 = run_tl(dev, st, w.L, 0)
    torch.cuda.synchronize()
    assert torch.equal(st, s0)
    o1 = run_tl(dev, st, w.L, 1)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and not torch.equal(st, s0)


def test_token_level_480p_sampled():
    """The 480p shape (B1 H12, 21 frames x 1560): the state of three heads and
    sampled output frames of two of them against the oracle."""
    w = W.WORKLOADS["480p"]
    say("case token-level 480p")
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    s0 = W.make_state0(w)
    dev = upload(inp, "bf16")
    st = torch.from_numpy(s0.copy()).cuda()
    out = run_tl(dev, st, w.L, 1)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    S = st.cpu().numpy().astype(np.float64)
    x = f64(inp, "bf16")
    eo = es = 0.0
    for h in (0, 5, 11):
        ref, Sref = O.hybrid_layer_token_level(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h], x["qp"][0, :, h],
                                               x["kp"][0, :, h], x["vp"][0, :, h], x["alpha"][0, :, h],
                                               x["beta"][0, :, h], s0[0, h].astype(np.float64), w.L, 1)
        es = max(es, rel_err(S[0, h], Sref))
        if h != 5:
            for n in (0, 10, 20):
                r = slice(n * w.L, (n + 1) * w.L)
                eo = max(eo, rel_err(got[0, r, h], ref[r]))
    say(f"token-level 480p: rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE
