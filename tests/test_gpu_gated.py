"""The gated entry points (hybrid_attn_gates, hybrid_attn_forward_gated)
against the fp64 oracle (oracle.hybrid_oracle.gate_projections,
hybrid_layer_gated) on an MI355X, through the C ABI.

Gate bar: the logits are fp32 sums of C exact bf16 products, so their error
is at most about C * 2^-24 of the sum of |x_c w_c| (about 1e-4 of a unit
logit at C = 1536, far less in practice), and sigmoid' <= 1/4; alpha and beta
are compared at 1e-4 of their largest value. Layer bars as the other parity
tests: 2e-2 on the output, 1e-3 on the fp32 state.
"""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.hybrid_oracle as O
from tests.gpu_util import TOL_OUT, TOL_STATE, f64, rel_err, upload
from video_dit_hybrid_amd import api
from video_dit_hybrid_amd import workloads as W

pytestmark = pytest.mark.gpu
TOL_GATE = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    api.lib()
    yield
    torch.cuda.synchronize()


def small(name, **kw):
    return dataclasses.replace(W.WORKLOADS[name], **kw)


def gate_case(w, C=None):
    """x [B, T, C] and the gate weights, device tensors and their fp64 values."""
    x = W.make_layer_input(w, 0, w.frames, 0)
    g = W.make_gate_weights(w)
    if C is not None and C != x.shape[-1]:  # a narrower input: keep the first C channels
        x = np.ascontiguousarray(x[..., :C])
        g["wgate"] = np.ascontiguousarray(g["wgate"][..., :C])
    dev = {"x": W.as_torch(x, "bf16"), "wgate": W.as_torch(g["wgate"], "bf16"),
           "bgate": W.as_torch(g["bgate"], "fp32")}
    ref = {"x": W.to_f64(x, "bf16"), "wgate": W.to_f64(g["wgate"], "bf16"),
           "bgate": g["bgate"].astype(np.float64)}
    return dev, ref


def maps(w):
    wts = W.make_fmap_weights(w)
    return ({k: W.as_torch(v, "bf16") for k, v in wts.items()},
            {k: W.to_f64(v, "bf16") for k, v in wts.items()})


@pytest.mark.parametrize("B,H,L,F,C", [(2, 12, 300, 3, 1536), (1, 3, 17, 3, 64), (1, 40, 100, 2, 256),
                                       (1, 64, 64, 1, 128), (1, 12, 1560, 2, 1536), (2, 3, 50, 2, 16),
                                       (1, 20, 100, 2, 80), (1, 13, 130, 2, 1552)])
def test_gates_parity(B, H, L, F, C):
    """alpha (frame means) and beta against the oracle: one to four 32-row gate
    blocks (H up to 64), ragged 64-token chunks, C from 16 to 1552 (channel
    counts that leave a partial last 64-channel slice: 16, 80, 1552)."""
    w = small("480p", B=B, H=H, L=L, frames=F, d=128)
    say(f"case gates B={B} H={H} L={L} F={F} C={C}")
    dev, ref = gate_case(w, C)
    a, b = api.hybrid_attn_gates(dev["x"], dev["wgate"], dev["bgate"], H, L)
    torch.cuda.synchronize()
    wa, wb = O.gate_projections(ref["x"], ref["wgate"], ref["bgate"], L)
    ea = rel_err(a.cpu().numpy(), wa)
    eb = rel_err(b.cpu().numpy(), wb)
    say(f"gates: rel_err alpha {ea:.3e} beta {eb:.3e}")
    assert ea < TOL_GATE and eb < TOL_GATE
    # repeatable bit for bit (fixed summation order)
    a2, b2 = api.hybrid_attn_gates(dev["x"], dev["wgate"], dev["bgate"], H, L)
    torch.cuda.synchronize()
    assert torch.equal(a, a2) and torch.equal(b, b2)


def run_gated(w, norm, update, dev=None):
    inp = W.make_call_inputs(w, 0, w.frames, 0, tensors=["q", "k", "v"])
    s0 = W.make_state0(w)
    d = upload(inp, "bf16")
    gdev, gref = gate_case(w)
    wdev, wref = maps(w)
    st = torch.from_numpy(s0.copy()).cuda()
    out = api.hybrid_attn_forward_gated(gdev["x"], d["q"], d["k"], d["v"], wdev["wq"], wdev["wk"], wdev["wv"],
                                        gdev["wgate"], gdev["bgate"], st, w.L, update, normalize_k=norm)
    torch.cuda.synchronize()
    return inp, s0, d, gdev, gref, wdev, wref, st, out


@pytest.mark.parametrize("d,L,F,B,H", [(128, 300, 3, 1, 2), (64, 130, 2, 2, 1), (128, 64, 4, 1, 1),
                                       (128, 1560, 1, 1, 12), (64, 17, 3, 2, 2)])
@pytest.mark.parametrize("norm", [1, 0])
def test_gated_layer_parity(d, L, F, B, H, norm):
    """Whole small clean calls: gates from x, maps, K' normalised or not; both
    head sizes, ragged frames, a one-frame call on the token-split path."""
    w = small("480p", d=d, L=L, frames=F, B=B, H=H, state0_sigma=0.05)
    say(f"case gated d={d} L={L} F={F} B={B} H={H} norm={norm}")
    inp, s0, _, _, gref, _, wref, st, out = run_gated(w, norm, 1)
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    x = f64(inp, "bf16")
    ref, Sref, _, _ = O.hybrid_layer_gated(gref["x"], x["q"], x["k"], x["v"], wref["wq"], wref["wk"], wref["wv"],
                                           gref["wgate"], gref["bgate"], s0.astype(np.float64), w.L, 1, bool(norm))
    eo = rel_err(got, ref)
    es = rel_err(st.cpu().numpy(), Sref)
    say(f"gated: rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


def test_gated_without_normalisation_is_fmap_on_projected_gates():
    """normalize_k = 0: the call is hybrid_attn_forward_fmap fed the alpha and
    beta of hybrid_attn_gates: the same kernels on the same bytes, so the
    outputs and states are bitwise equal."""
    w = small("480p", H=3, L=400, frames=3, state0_sigma=0.05)
    say("case gated(norm 0) vs gates + fmap")
    inp, s0, d, gdev, _, wdev, _, st, out = run_gated(w, 0, 1)
    a, b = api.hybrid_attn_gates(gdev["x"], gdev["wgate"], gdev["bgate"], w.H, w.L)
    st2 = torch.from_numpy(s0.copy()).cuda()
    out2 = api.hybrid_attn_forward_fmap(d["q"], d["k"], d["v"], wdev["wq"], wdev["wk"], wdev["wv"], a, b, st2,
                                        w.L, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(st, st2)


def test_gated_state_ignores_key_scale():
    """With normalised keys, doubling K leaves K' and hence the state: on the
    GPU the step sizes scale by exact powers of two, so the state is bitwise
    equal (the output moves: the intra-frame branch reads K)."""
    w = small("480p", H=2, L=300, frames=2, state0_sigma=0.05)
    say("case gated key scale")
    _, s0, d, gdev, _, wdev, _, st, _ = run_gated(w, 1, 1)
    st2 = torch.from_numpy(s0.copy()).cuda()
    api.hybrid_attn_forward_gated(gdev["x"], d["q"], (d["k"].float() * 2).to(torch.bfloat16), d["v"], wdev["wq"],
                                  wdev["wk"], wdev["wv"], gdev["wgate"], gdev["bgate"], st2, w.L, 1)
    torch.cuda.synchronize()
    assert torch.equal(st, st2)


def test_gated_denoise_pass():
    """update_state = 0 reads only q, k, v, W_q and the state: the output
    equals the feature-map entry point's, bitwise, and S is left unchanged."""
    w = small("480p", H=3, L=520, frames=1, state0_sigma=0.05)
    say("case gated denoise")
    inp = W.make_call_inputs(w, 0, 1, 0, tensors=["q", "k", "v"])
    d = upload(inp, "bf16")
    wdev, _ = maps(w)
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st = s0.clone()
    o1 = api.hybrid_attn_forward_gated(None, d["q"], d["k"], d["v"], wdev["wq"], None, None, None, None, st, w.L, 0)
    o2 = api.hybrid_attn_forward_fmap(d["q"], d["k"], d["v"], wdev["wq"], None, None, None, None, st, w.L, 0)
    torch.cuda.synchronize()
    assert torch.equal(st, s0) and torch.equal(o1, o2)


def test_gated_480p_sampled_heads():
    """The 480p shape (B1 H12, 21 frames x 1560, C = 1536) in the launch
    configuration of the bench: gates of all heads, the full state of every
    head and the output of two heads on three frames against the oracle."""
    w = W.WORKLOADS["480p"]
    say("case gated 480p")
    inp, s0, _, gdev, gref, _, wref, st, out = run_gated(w, 1, 1)
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    S = st.cpu().numpy().astype(np.float64)
    x = f64(inp, "bf16")
    alpha, beta = O.gate_projections(gref["x"], gref["wgate"], gref["bgate"], w.L)
    frames = {0, 10, 20}
    worst_o, worst_s = 0.0, 0.0
    for h in range(w.H):
        qp = x["q"][0, :, h] @ wref["wq"][h]
        kp = O.l2_normalize_rows(x["k"][0, :, h] @ wref["wk"][h])
        vp = x["v"][0, :, h] @ wref["wv"][h]
        want_out = h in (0, w.H - 1)
        ref, Sref = O.hybrid_layer_head(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h], qp, kp, vp,
                                        alpha[0, :, h], beta[0, :, h], s0[0, h].astype(np.float64), w.L, True,
                                        frames=(frames if want_out else set()))
        worst_s = max(worst_s, rel_err(S[0, h], Sref))
        if want_out:
            for n in frames:
                r = slice(n * w.L, (n + 1) * w.L)
                worst_o = max(worst_o, rel_err(got[0, r, h], ref[r]))
    say(f"gated 480p: rel_err out {worst_o:.3e} state {worst_s:.3e}")
    assert worst_o < TOL_OUT and worst_s < TOL_STATE
