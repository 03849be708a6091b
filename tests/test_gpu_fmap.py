"""The feature-map entry point (hybrid_attn_forward_fmap) against the fp64
oracle (oracle.hybrid_oracle.hybrid_layer_fmap) on an MI355X, through the C ABI.

The oracle materialises Q' = Q W_q, K' = K W_k, V' = V W_v per head from the
exact bytes the GPU consumed; the GPU path never forms them (it folds the maps
into the state increments and the readout). Same error metric and bars as the
other parity tests: 2e-2 on the output, 1e-3 on the fp32 state.
"""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    api.lib()
    yield
    torch.cuda.synchronize()


def small(name, **kw):
    return dataclasses.replace(W.WORKLOADS[name], **kw)


def maps(w):
    wts = W.make_fmap_weights(w)
    dev = {k: W.as_torch(v, w.dtype) for k, v in wts.items()}
    x = {k: W.to_f64(v, w.dtype) for k, v in wts.items()}
    return dev, x


def run_fmap(dev, wdev, st, L, update, **kw):
    return api.hybrid_attn_forward_fmap(dev["q"], dev["k"], dev["v"], wdev["wq"], wdev["wk"], wdev["wv"],
                                        dev.get("alpha"), dev.get("beta"), st, L, int(update), **kw)


def compare(w, update):
    inp = W.make_call_inputs(w, 0, w.frames, 0, clean=True)
    s0 = W.make_state0(w)
    dev = upload(inp, w.dtype)
    wdev, wx = maps(w)
    st = torch.from_numpy(s0.copy()).cuda()
    out = run_fmap(dev, wdev, st, w.L, update)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, w.dtype), w.dtype)
    x = f64(inp, w.dtype)
    ref, Sref = O.hybrid_layer_fmap(x["q"], x["k"], x["v"], wx["wq"], wx["wk"], wx["wv"], x["alpha"],
                                    x["beta"], s0.astype(np.float64), w.L, int(update))
    S = st.cpu().numpy().astype(np.float64)
    return rel_err(got, ref), rel_err(S, Sref), S, s0


@pytest.mark.parametrize("d,L,F,B,H", [(128, 300, 3, 1, 2), (64, 130, 2, 2, 1), (128, 64, 4, 1, 1),
                                       (128, 1560, 1, 1, 12), (64, 17, 3, 2, 2)])
@pytest.mark.parametrize("update", [1, 0])
def test_fmap_parity(d, L, F, B, H, update):
    """Whole small calls, both head sizes, ragged frames, one-frame calls whose
    increments take the token-split path (B*H*F = 12), denoise and clean."""
    w = small("480p", d=d, L=L, frames=F, B=B, H=H, state0_sigma=0.05)
    say(f"case fmap d={d} L={L} F={F} B={B} H={H} update={update}")
    eo, es, S, s0 = compare(w, update)
    say(f"fmap: rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE
    if not update:
        assert np.array_equal(S, s0.astype(np.float64))  # the state is left bitwise unchanged


def test_fmap_identity_maps_match_plain_forward():
    """With identity maps the layer is hybrid_attn_forward with Q' = Q, K' = K,
    V' = V (different arithmetic on the GPU: close, not bitwise)."""
    w = small("480p", H=2, L=400, frames=3, state0_sigma=0.05)
    say("case fmap identity maps")
    inp = W.make_call_inputs(w, 0, w.frames, 0, clean=True)
    dev = upload(inp, "bf16")
    eye = torch.eye(w.d, dtype=torch.bfloat16, device="cuda").expand(w.H, w.d, w.d).contiguous()
    wdev = {"wq": eye, "wk": eye, "wv": eye}
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st1 = s0.clone()
    out1 = run_fmap(dev, wdev, st1, w.L, 1)
    plain = dict(dev, qp=dev["q"], kp=dev["k"], vp=dev["v"])
    st2 = s0.clone()
    out2 = run_gpu(plain, st2, w.L, True)
    torch.cuda.synchronize()
    eo = rel_err(out1.float().cpu().numpy(), out2.float().cpu().numpy())
    es = rel_err(st1.cpu().numpy(), st2.cpu().numpy())
    say(f"identity maps vs plain: out {eo:.3e} state {es:.3e}")
    assert eo < 1e-2 and es < 1e-4


def test_fmap_denoise_output_equals_clean_output():
    """One frame: the denoise pass (update_state = 0) and the clean pass read
    the same S_{N-1}, so their outputs are bitwise equal; only the clean pass
    moves the state."""
    w = small("480p", H=3, L=520, frames=1, state0_sigma=0.05)
    say("case fmap denoise vs clean")
    inp = W.make_call_inputs(w, 0, 1, 0, clean=True)
    dev = upload(inp, "bf16")
    wdev, _ = maps(w)
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st = s0.clone()
    o_d = run_fmap(dev, wdev, st, w.L, 0)
    torch.cuda.synchronize()
    assert torch.equal(st, s0)
    o_c = run_fmap(dev, wdev, st, w.L, 1)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_c)
    assert not torch.equal(st, s0)


def test_fmap_480p_sampled_heads():
    """The 480p shape (B1 H12, 21 frames x 1560), launch configuration of the
    bench: the full state of every head and the output of two heads on three
    frames against the oracle (per head, maps materialised in fp64)."""
    w = W.WORKLOADS["480p"]
    say("case fmap 480p")
    inp = W.make_call_inputs(w, 0, w.frames, 0, clean=True)
    s0 = W.make_state0(w)
    dev = upload(inp, "bf16")
    wdev, wx = maps(w)
    st = torch.from_numpy(s0.copy()).cuda()
    out = run_fmap(dev, wdev, st, w.L, 1)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    S = st.cpu().numpy().astype(np.float64)
    x = f64(inp, "bf16")
    frames = {0, 10, 20}
    worst_o, worst_s = 0.0, 0.0
    for h in range(w.H):
        qp = x["q"][0, :, h] @ wx["wq"][h]
        kp = x["k"][0, :, h] @ wx["wk"][h]
        vp = x["v"][0, :, h] @ wx["wv"][h]
        want_out = h in (0, w.H - 1)
        ref, Sref = O.hybrid_layer_head(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h], qp, kp, vp,
                                        x["alpha"][0, :, h], x["beta"][0, :, h], s0[0, h].astype(np.float64),
                                        w.L, True, frames=(frames if want_out else set()))
        worst_s = max(worst_s, rel_err(S[0, h], Sref))
        if want_out:
            for n in frames:
                r = slice(n * w.L, (n + 1) * w.L)
                worst_o = max(worst_o, rel_err(got[0, r, h], ref[r]))
    say(f"fmap 480p: rel_err out {worst_o:.3e} state {worst_s:.3e}")
    assert worst_o < TOL_OUT and worst_s < TOL_STATE


@pytest.mark.parametrize("d,B,H,L,F", [(64, 1, 8, 200, 17), (128, 1, 8, 200, 17), (128, 2, 12, 1560, 1)])
def test_fmap_fused_scan_parity_and_graph_replay(d, B, H, L, F):
    """More than 256 attention work-groups: the scan runs in the readout's
    launch and publishes the fragments of W_q S_{n-1} itself. Against the
    oracle, then HIP-graph replays of the captured call (the map transform
    zeroes the frame counters, so every replay starts clean) bitwise equal to
    eager calls."""
    w = small("480p", B=B, H=H, d=d, L=L, frames=F, state0_sigma=0.05)
    assert w.B * w.H * w.frames * ((w.L + 127) // 128) > 256
    say(f"case fmap, scan in the readout launch, d={d} B={B} H={H} L={L} F={F}")
    eo, es, *_ = compare(w, 1)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE
    inp = W.make_call_inputs(w, 0, w.frames, 0, clean=True)
    dev = upload(inp, w.dtype)
    wdev, _ = maps(w)
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    out = torch.empty_like(dev["q"])
    ws = torch.empty(api.fmap_workspace_bytes(w.B, w.H, w.T, w.L, w.d, 1), dtype=torch.uint8, device="cuda")

    def call(state):
        run_fmap(dev, wdev, state, w.L, 1, out=out, workspace=ws)

    st = s0.clone()
    ref = []
    for _ in range(3):
        call(st)
        torch.cuda.synchronize()
        ref.append((out.clone(), st.clone()))
    gst = s0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(gst)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(gst)
    torch.cuda.synchronize()
    gst.copy_(s0)
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[i][0]) and torch.equal(gst, ref[i][1])
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
