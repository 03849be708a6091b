"""HIP path against the fp64 oracle on an MI355X, through the C ABI.

Every comparison feeds the oracle the exact bytes the GPU consumed (bf16 or
fp32, upcast to fp64). Error metric: max|x - r| / max|r| over the tensor or
the sampled slab; bars: 2e-2 on the output, 1e-3 on the fp32 state.
"""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.hybrid_oracle as O
from tests.gpu_util import TOL_OUT, TOL_STATE, f64, oracle_head, rel_err, run_gpu, upload
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


def full_compare(w, update=True, seed_pass=0, scale=0.0, state0=None):
    """Run one call over the whole (small) workload and compare everything."""
    inp = W.make_call_inputs(w, 0, w.frames, seed_pass, clean=True)
    s0 = W.make_state0(w) if state0 is None else state0
    dev = upload(inp, w.dtype)
    st = torch.from_numpy(s0.copy()).cuda()
    out = run_gpu(dev, st, w.L, update, scale=scale)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, w.dtype), w.dtype)
    S = st.cpu().numpy().astype(np.float64)
    x = f64(inp, w.dtype)
    ref, Sref = O.hybrid_layer(x["q"], x["k"], x["v"], x["qp"], x["kp"], x["vp"], x["alpha"],
                               x["beta"], s0.astype(np.float64), w.L, int(update),
                               scale=(scale if scale > 0 else None))
    return rel_err(got, ref), rel_err(S, Sref), got, ref, S, Sref


# --- the tiny fp32 workload, whole --------------------------------------------

def test_tiny_config_fp32():
    w = W.WORKLOADS["tiny"]
    say("case tiny fp32", w)
    eo, es, *_ = full_compare(w)
    say(f"tiny: rel_err out {eo:.3e} state {es:.3e}")
    assert eo < 1e-5 and es < 1e-5   # fp32 path: fp32-accurate
    assert eo < TOL_OUT and es < TOL_STATE


def test_tiny_shape_bf16_path():
    w = small("tiny", dtype="bf16")
    say("case tiny shape on the bf16 path")
    eo, es, *_ = full_compare(w)
    say(f"tiny bf16: rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


# --- ragged and edge frame lengths, both head sizes, both dtypes --------------

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,F,B,H", [(1, 3, 1, 2), (17, 3, 2, 1), (64, 2, 1, 2), (100, 3, 1, 3),
                                     (129, 2, 1, 1), (256, 2, 1, 2), (160, 3, 1, 1), (24, 1, 1, 3)])
def test_edge_frame_lengths(dtype, d, L, F, B, H):
    w = small("480p", B=B, H=H, d=d, L=L, frames=F, dtype=dtype, state0_sigma=0.05)
    say(f"case edge dtype={dtype} d={d} L={L} F={F} B={B} H={H}")
    eo, es, *_ = full_compare(w)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE
    if dtype == "fp32":
        assert eo < 1e-5 and es < 1e-5


# --- ragged lengths with more than 256 attention work-groups ------------------
# (launches of up to 256 work-groups, as in every test above, take the
# attention kernel with a loader wave; these take the one without)

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,F,H", [(1, 33, 8), (17, 33, 8), (129, 17, 8), (200, 17, 8)])
def test_edge_lengths_without_loader_wave(d, L, F, H):
    w = small("480p", B=1, H=H, d=d, L=L, frames=F, state0_sigma=0.05)
    qtiles = (L + 127) // 128
    assert w.B * w.H * w.frames * qtiles > 256
    say(f"case edge, no loader wave, d={d} L={L} F={F} H={H}")
    eo, es, *_ = full_compare(w)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


# --- the short last query tile: two waves, one 32-key half each ------------
# A query tile of at most 32 queries (L - 128 qt <= 32) splits its keys over
# waves 0 and 1 and merges their (max, sum, O); 33 queries or more take the
# usual loop. Both sides of the boundary, with and without the loader wave
# (up to 256 work-groups), ragged and full last key tiles.

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,F,H", [(32, 2, 2), (33, 2, 2), (160, 2, 2), (161, 2, 2), (192, 3, 2),
                                   (160, 17, 8), (161, 17, 8), (1560, 2, 2)])
def test_short_last_query_tile(d, L, F, H):
    w = small("480p", B=1, H=H, d=d, L=L, frames=F, state0_sigma=0.05)
    tail = L - (L - 1) // 128 * 128
    say(f"case short last query tile d={d} L={L} (tail {tail} queries) F={F} H={H}")
    eo, es, *_ = full_compare(w)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


# --- many frames: one gram work-group per (stream, head, frame) ----------------

@pytest.mark.parametrize("d", [64, 128])
def test_many_frames_unsplit_gram(d):
    # 8 heads x 16 frames = 128 units: each frame's increments come from one
    # work-group computing the upper-triangle blocks of G (4 chunks of 64
    # tokens per frame, the last ragged), not from split partial sums
    w = small("480p", B=1, H=8, d=d, L=200, frames=16, state0_sigma=0.05)
    say(f"case many frames, unsplit gram, d={d}")
    eo, es, *_ = full_compare(w)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


# --- one frame per call: the state write as one kernel (d = 128) -------------

@pytest.mark.parametrize("L,B,H,d", [(1560, 1, 12, 128), (1560, 1, 2, 128), (1000, 1, 1, 128), (513, 1, 1, 128),
                                     (513, 2, 1, 128), (300, 1, 3, 128), (33, 2, 2, 128), (1, 1, 2, 128),
                                     (520, 1, 2, 64)])
def test_one_frame_state_write(L, B, H, d):
    # token splits per (b, h, 32-column block), shape only: (1560, H=12) 6,
    # (1560, H=2) 6, (1000) 4, (513) 2, the others 1; the last block of a
    # split may hold 1 to 31 tokens (1560 = 48 x 32 + 24, 1000 = 31 x 32 + 8,
    # 513 = 16 x 32 + 1); d = 64 takes the gram + scan kernels
    w = small("480p", B=B, H=H, L=L, d=d, frames=1, state0_sigma=0.05)
    say(f"case one-frame state write L={L} B={B} H={H} d={d}")
    eo, es, *_ = full_compare(w, update=True)
    say(f"  rel_err out {eo:.3e} state {es:.3e}")
    assert eo < TOL_OUT and es < TOL_STATE


def test_one_frame_state_write_snapshot_and_determinism():
    # the write-only entry point: the snapshot holds S_0 bitwise, and two
    # calls from the same S_0 give bitwise equal states whichever split of a
    # column block finishes last
    w = small("480p", H=12, L=1560, frames=1, state0_sigma=0.05)
    say("case one-frame state write: snapshot, determinism")
    inp = W.make_call_inputs(w, 0, 1, 0, clean=True)
    dev = upload(inp, "bf16")
    s0 = W.make_state0(w)
    res = []
    for _ in range(3):
        st = torch.from_numpy(s0.copy()).cuda()
        snap = torch.full((1, w.H, 1, w.d, w.d), float("nan"), device="cuda")
        api.hybrid_attn_state_update(dev["kp"], dev["vp"], dev["alpha"], dev["beta"], st, w.L, snapshots=snap)
        torch.cuda.synchronize()
        res.append((st.cpu().numpy(), snap.cpu().numpy()))
    assert np.array_equal(res[0][1][0, :, 0], s0[0])
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][0], res[2][0])


def test_one_frame_state_write_workspace_reuse():
    # one workspace for calls on different inputs: a partial sum left by an
    # earlier call (or garbage in a fresh workspace) must never reach a later
    # call's sum
    w = small("480p", H=12, L=1560, frames=1, state0_sigma=0.05)
    say("case one-frame state write: workspace reuse")
    s0 = W.make_state0(w)
    ws = torch.full((api.workspace_bytes(1, w.H, w.L, w.L, w.d, 1),), 0x3F, dtype=torch.uint8, device="cuda")
    inps = [W.make_call_inputs(w, 0, 1, p, clean=True) for p in (0, 1)]
    got = []
    for i in (0, 1, 0):
        st = torch.from_numpy(s0.copy()).cuda()
        run_gpu(upload(inps[i], "bf16"), st, w.L, True, workspace=ws)
        torch.cuda.synchronize()
        got.append(st.cpu().numpy().astype(np.float64))
    assert np.array_equal(got[0], got[2])
    for i, S in ((0, got[0]), (1, got[1])):
        x = f64(inps[i], "bf16")
        worst = 0.0
        for h in range(w.H):
            S1 = O.delta_update(s0[0, h].astype(np.float64), x["kp"][0, :, h], x["vp"][0, :, h],
                                float(x["alpha"][0, 0, h]), x["beta"][0, :, h])
            worst = max(worst, rel_err(S[0, h], S1))
        say(f"  inputs {i}: rel_err state {worst:.3e} (all heads)")
        assert worst < TOL_STATE


def test_softmax_scale_argument():
    w = small("480p", H=2, L=200, frames=2)
    say("case explicit softmax scale")
    eo, es, *_ = full_compare(w, scale=0.05)
    assert eo < TOL_OUT and es < TOL_STATE


# --- the method's special cases, on the GPU -----------------------------------

def _gates(inp, alpha, beta):
    inp["alpha"][:] = alpha
    inp["beta"][:] = beta
    return inp


@pytest.mark.parametrize("F", [1, 3])
def test_alpha1_beta0_keeps_state_bitwise(F):
    w = small("480p", H=3, L=300, frames=F, state0_sigma=0.05)
    say(f"case alpha=1 beta=0 F={F}")
    inp = _gates(W.make_call_inputs(w, 0, F, 0), 1.0, 0.0)
    s0 = W.make_state0(w)
    st = torch.from_numpy(s0.copy()).cuda()
    run_gpu(upload(inp, "bf16"), st, w.L, True)
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), s0)


def test_alpha0_beta0_clears_state():
    w = small("480p", H=2, L=300, frames=3, state0_sigma=0.05)
    say("case alpha=0 beta=0")
    inp = _gates(W.make_call_inputs(w, 0, 3, 0), 0.0, 0.0)
    st = torch.from_numpy(W.make_state0(w)).cuda()
    out = run_gpu(upload(inp, "bf16"), st, w.L, True)
    torch.cuda.synchronize()
    assert not st.cpu().numpy().any()
    # frames >= 1 read S = 0: equal to a call with zero state and no update
    out0 = run_gpu(upload(inp, "bf16"), torch.zeros_like(st), w.L, False)
    torch.cuda.synchronize()
    assert torch.equal(out[:, w.L:], out0[:, w.L:])


def test_denoise_pass_leaves_state_and_matches_clean_output():
    w = small("batched", B=2, H=3)
    say("case denoise vs clean pass")
    inp = W.make_call_inputs(w, 0, 1, 0)
    dev = upload(inp, "bf16")
    s0 = W.make_state0(w)
    st = torch.from_numpy(s0.copy()).cuda()
    o_den = [run_gpu(dev, st, w.L, False) for _ in range(3)]
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), s0)
    o_clean = run_gpu(dev, st, w.L, True)
    torch.cuda.synchronize()
    for o in o_den:
        assert torch.equal(o, o_clean)
    assert not np.array_equal(st.cpu().numpy(), s0)


def test_orthonormal_keys_recall_values_fp32():
    """beta = 1, alpha = 1, orthonormal K' rows: K' S_1 = V' (delta-rule recall)."""
    say("case delta-rule recall fp32")
    rng = np.random.default_rng(5)
    L, d, H = 32, 64, 2
    kp = np.stack([np.linalg.qr(rng.standard_normal((d, L)))[0].T for _ in range(H)], axis=1)
    inp = {n: rng.standard_normal((1, L, H, d)).astype(np.float32) for n in ("q", "k", "v", "qp", "vp")}
    inp["kp"] = kp[None].astype(np.float32)
    inp["alpha"] = np.ones((1, 1, H), np.float32)
    inp["beta"] = np.ones((1, L, H), np.float32)
    s0 = (0.3 * rng.standard_normal((1, H, d, d))).astype(np.float32)
    st = torch.from_numpy(s0.copy()).cuda()
    run_gpu(upload(inp, "fp32"), st, L, True)
    torch.cuda.synchronize()
    S = st.cpu().numpy().astype(np.float64)
    for h in range(H):
        k64 = inp["kp"][0, :, h].astype(np.float64)
        assert rel_err(k64 @ S[0, h], inp["vp"][0, :, h]) < 1e-5


def test_multi_frame_call_equals_single_frame_calls():
    w = small("480p", H=2, L=520, frames=4, state0_sigma=0.05)
    say("case call splitting")
    inp = W.make_call_inputs(w, 0, 4, 0)
    dev = upload(inp, "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st1 = s0.clone()
    out1 = run_gpu(dev, st1, w.L, True)
    st2 = s0.clone()
    outs = []
    for n in range(4):
        r = slice(n * w.L, (n + 1) * w.L)
        sub = {k: (v[:, n:n + 1].contiguous() if k == "alpha" else v[:, r].contiguous()) for k, v in dev.items()}
        outs.append(run_gpu(sub, st2, w.L, True))
    torch.cuda.synchronize()
    out2 = torch.cat(outs, dim=1)
    assert rel_err(out2.float().cpu().numpy(), out1.float().cpu().numpy()) < 1e-2
    assert rel_err(st2.cpu().numpy(), st1.cpu().numpy()) < 1e-5


def test_batch_permutation_permutes_outputs():
    w = small("batched", B=4, H=2, L=300)
    say("case batch permutation")
    inp = W.make_call_inputs(w, 0, 1, 0)
    s0 = W.make_state0(w)
    perm = [2, 0, 3, 1]
    dev = upload(inp, "bf16")
    st = torch.from_numpy(s0.copy()).cuda()
    out = run_gpu(dev, st, w.L, True)
    devp = {k: v[perm].contiguous() for k, v in dev.items()}
    stp = torch.from_numpy(s0[perm].copy()).cuda()
    outp = run_gpu(devp, stp, w.L, True)
    torch.cuda.synchronize()
    assert torch.equal(outp, out[perm])
    assert torch.equal(stp, st[perm])


def test_readout_with_frame_major_state_layout():
    # states laid out [F, B, H, d, d]: S_n of (b, h) at (b*H + h)*d*d + n*B*H*d*d
    w = small("480p", B=2, H=3, L=200, frames=3, state0_sigma=0.05)
    say("case readout, frame-major state layout, B=2 H=3")
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    dev = upload(inp, "bf16")
    g = np.random.default_rng(7)
    Sfb = (0.05 * g.standard_normal((w.frames, w.B, w.H, w.d, w.d))).astype(np.float32)
    states = torch.from_numpy(Sfb).cuda()
    out = api.hybrid_attn_intra_readout(dev["q"], dev["k"], dev["v"], dev["qp"], states,
                                        w.d * w.d, w.B * w.H * w.d * w.d, w.L)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    x = f64(inp, "bf16")
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            for n in range(w.frames):
                r = slice(n * w.L, (n + 1) * w.L)
                ref = O.intra_frame_attention(x["q"][b, r, h], x["k"][b, r, h], x["v"][b, r, h]) + \
                    O.inter_frame_readout(x["qp"][b, r, h], Sfb[n, b, h].astype(np.float64))
                worst = max(worst, rel_err(got[b, r, h], ref))
    say(f"frame-major states: rel_err out {worst:.3e}")
    assert worst < TOL_OUT


def test_sub_entry_points_compose_to_forward():
    w = small("480p", H=2, L=400, frames=3, state0_sigma=0.05)
    say("case sub entry points")
    inp = W.make_call_inputs(w, 0, 3, 0)
    dev = upload(inp, "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st = s0.clone()
    out = run_gpu(dev, st, w.L, True)
    st2 = s0.clone()
    snaps = torch.empty(1, 2, 3, 128, 128, device="cuda")
    api.hybrid_attn_state_update(dev["kp"], dev["vp"], dev["alpha"], dev["beta"], st2, w.L, snapshots=snaps)
    out2 = api.hybrid_attn_intra_readout(dev["q"], dev["k"], dev["v"], dev["qp"], snaps,
                                         3 * 128 * 128, 128 * 128, w.L)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(st, st2)
    assert torch.equal(snaps[:, :, 0], s0)


# --- the full workloads (sampled comparisons where the oracle is slow) ---------

def _state_chain_check(x, s0, w, heads, S_gpu, streams=(0,)):
    worst = 0.0
    chains = {}
    for b in streams:
        for h in heads:
            ch = O.state_chain(x["kp"][b, :, h], x["vp"][b, :, h], x["alpha"][b, :, h],
                               x["beta"][b, :, h], s0[b, h].astype(np.float64), w.L)
            chains[(b, h)] = ch
            worst = max(worst, rel_err(S_gpu[b, h], ch[-1]))
    return worst, chains


def _sampled_out_check(x, got, chains, w, samples, b=0):
    worst = 0.0
    for n, h in samples:
        r = slice(n * w.L, (n + 1) * w.L)
        ref = O.intra_frame_attention(x["q"][b, r, h], x["k"][b, r, h], x["v"][b, r, h]) + \
            O.inter_frame_readout(x["qp"][b, r, h], chains[(b, h)][n])
        worst = max(worst, rel_err(got[b, r, h], ref))
    return worst


@pytest.mark.parametrize("name,heads,samples", [
    # every head's final state; one output frame per head (frames spread over
    # the call), plus the first and last frame of head 0
    ("480p", list(range(12)), [((7 * h) % 21, h) for h in range(12)] + [(0, 0), (20, 0)]),
    ("720p", list(range(40)), [((5 * h) % 21, h) for h in range(40)] + [(20, 0)]),
])
def test_full_clean_pass_workloads(name, heads, samples):
    w = W.WORKLOADS[name]
    say(f"case {name} full clean pass: generating inputs")
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    s0 = W.make_state0(w)
    dev = upload(inp, "bf16")
    st = torch.from_numpy(s0.copy()).cuda()
    say(f"case {name}: running the layer")
    out = run_gpu(dev, st, w.L, True)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    S = st.cpu().numpy().astype(np.float64)
    del dev, out
    say(f"case {name}: oracle")
    x = f64({k: inp[k] for k in ("q", "k", "v", "qp", "kp", "vp", "alpha", "beta")}, "bf16")
    es, chains = _state_chain_check(x, s0, w, heads, S)
    eo = _sampled_out_check(x, got, chains, w, samples)
    say(f"{name}: rel_err state {es:.3e} (heads {heads}), out {eo:.3e} (samples {samples})")
    assert np.isfinite(got).all()
    assert es < TOL_STATE and eo < TOL_OUT


def test_batched_streaming_step():
    w = W.WORKLOADS["batched"]
    say("case batched: 4 denoise passes + 1 clean pass, 8 streams")
    s0 = W.make_state0(w)
    st = torch.from_numpy(s0.copy()).cuda()
    outs, inps = [], []
    for (f0, nf, p, clean) in W.call_schedule(w):
        inp = W.make_call_inputs(w, f0, nf, p, clean=clean)
        outs.append(W.to_f64(W.from_torch(run_gpu(upload(inp, "bf16"), st, w.L, clean), "bf16"), "bf16"))
        inps.append(f64(inp, "bf16"))
    torch.cuda.synchronize()
    S = st.cpu().numpy().astype(np.float64)
    worst_s = 0.0
    for b in range(w.B):
        x = inps[-1]
        for h in range(w.H):
            S1 = O.delta_update(s0[b, h].astype(np.float64), x["kp"][b, :, h], x["vp"][b, :, h],
                                float(x["alpha"][b, 0, h]), x["beta"][b, :, h])
            worst_s = max(worst_s, rel_err(S[b, h], S1))
    worst_o = 0.0
    for p, b, h in [(0, 0, 0), (1, 3, 7), (3, 7, 11), (4, 5, 2), (4, 0, 0)]:
        x = inps[p]
        ref = O.intra_frame_attention(x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]) + \
            x["qp"][b, :, h] @ s0[b, h].astype(np.float64)
        worst_o = max(worst_o, rel_err(outs[p][b, :, h], ref))
    say(f"batched: rel_err state {worst_s:.3e} (all 96 heads), out {worst_o:.3e} (5 samples)")
    assert worst_s < TOL_STATE and worst_o < TOL_OUT


def test_long_stream_constant_memory_and_parity():
    w = W.WORKLOADS["stream"]
    say("case stream: 120 frames x (4 denoise + 1 clean)")
    s0 = W.make_state0(w)
    st = torch.from_numpy(s0.copy()).cuda()
    shape = (w.B, w.L, w.H, w.d)
    bufs = {k: torch.empty(shape, dtype=torch.bfloat16, device="cuda") for k in W.QKV_NAMES}
    bufs["alpha"] = torch.empty((w.B, 1, w.H), device="cuda")
    bufs["beta"] = torch.empty((w.B, w.L, w.H), device="cuda")
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(api.workspace_bytes(w.B, w.H, w.L, w.L, w.d, 1), dtype=torch.uint8, device="cuda")
    keep = {0: {}, 59: {}, 119: {}}
    clean_inputs = []
    mem = {}
    for (f0, nf, p, clean) in W.call_schedule(w):
        inp = W.make_call_inputs(w, f0, nf, p, clean=clean)
        for k, a in inp.items():
            bufs[k].copy_(W.as_torch(a, "bf16" if k in W.QKV_NAMES else "fp32", "cpu"))
        run_gpu(bufs, st, w.L, clean, out=out, workspace=ws)
        if clean:
            clean_inputs.append({k: inp[k] for k in ("kp", "vp", "alpha", "beta")})
        if f0 in keep and p in (0, w.denoise_passes):
            keep[f0][p] = (inp, W.from_torch(out, "bf16"))
        if clean and f0 in (0, 59, 119):
            torch.cuda.synchronize()
            mem[f0] = torch.cuda.memory_allocated()
            say(f"  frame {f0} done, allocated {mem[f0]}")
    torch.cuda.synchronize()
    assert mem[0] == mem[59] == mem[119]
    S = st.cpu().numpy().astype(np.float64)
    worst_s, worst_o = 0.0, 0.0
    for h in range(w.H):
        Sh = s0[0, h].astype(np.float64)
        hist = [Sh]
        for ci in clean_inputs:
            Sh = O.delta_update(Sh, W.to_f64(ci["kp"][0, :, h], "bf16"), W.to_f64(ci["vp"][0, :, h], "bf16"),
                                float(ci["alpha"][0, 0, h]), ci["beta"][0, :, h].astype(np.float64))
            hist.append(Sh)
        worst_s = max(worst_s, rel_err(S[0, h], Sh))
        # every head: the first denoise pass and the clean pass of frames 0, 59, 119
        for f0, passes in keep.items():
            for p, (inp, o) in passes.items():
                x = f64(inp, "bf16")
                ref = O.intra_frame_attention(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h]) + \
                    x["qp"][0, :, h] @ hist[f0]
                worst_o = max(worst_o, rel_err(W.to_f64(o[0, :, h], "bf16"), ref))
    say(f"stream: rel_err state {worst_s:.3e} after 120 frames (all heads), out {worst_o:.3e}")
    assert worst_s < TOL_STATE and worst_o < TOL_OUT


@pytest.mark.parametrize("L", [200, 1560])
def test_graph_replay_matches_eager(L):
    # One frame of a streaming run (a denoise call, then the clean call) captured
    # in a HIP graph and replayed: every replay must equal the eager calls
    # bitwise, with eager work and synchronisations between the replays.
    # L = 1560 splits the tokens of the one-frame state write over 6
    # work-groups per column block (ticket words in the workspace, put back
    # to 0 by every call).
    w = small("stream", H=2, L=L, frames=1)
    say(f"case graph replay L={L}")
    d_in = upload(W.make_call_inputs(w, 0, 1, 0, clean=False), "bf16")
    c_in = upload(W.make_call_inputs(w, 0, 1, w.denoise_passes, clean=True), "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    out_d = torch.empty_like(d_in["q"])
    out_c = torch.empty_like(c_in["q"])
    ws = torch.empty(api.workspace_bytes(1, w.H, w.L, w.L, w.d, 1), dtype=torch.uint8, device="cuda")

    def frame(state):
        api.hybrid_attn_forward(d_in["q"], d_in["k"], d_in["v"], d_in["qp"], None, None, None, None,
                                state, w.L, 0, out=out_d, workspace=ws)
        api.hybrid_attn_forward(c_in["q"], c_in["k"], c_in["v"], c_in["qp"], c_in["kp"], c_in["vp"],
                                c_in["alpha"], c_in["beta"], state, w.L, 1, out=out_c, workspace=ws)

    # eager reference for three frames
    st = s0.clone()
    ref = []
    for _ in range(3):
        frame(st)
        torch.cuda.synchronize()
        ref.append((out_d.clone(), out_c.clone(), st.clone()))
    # graph of one frame on its own state tensor
    gst = s0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        frame(gst)          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gst.copy_(s0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        frame(gst)
    torch.cuda.synchronize()
    gst.copy_(s0)           # capture does not run the kernels; start from S_0
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, ref[i][0]) and torch.equal(out_c, ref[i][1])
        assert torch.equal(gst, ref[i][2])
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)


# --- the forward call's scan inside the attention launch -----------------------
# (calls over several frames with more than 256 attention work-groups: the
# scan's work-groups publish each frame's state as readout fragments and the
# attention work-groups wait for them; the same operations as the separate
# state update and readout, so the results must be bitwise equal)

@pytest.mark.parametrize("d,B,H,L,F", [(128, 1, 8, 200, 17), (128, 1, 4, 300, 24), (64, 1, 8, 129, 17),
                                       (128, 1, 12, 1560, 3), (128, 2, 4, 200, 17), (128, 1, 12, 1560, 2),
                                       (128, 1, 8, 24, 40)])
def test_fused_scan_matches_sub_entry_points(d, B, H, L, F):
    w = small("480p", B=B, H=H, d=d, L=L, frames=F, state0_sigma=0.05)
    assert w.B * w.H * w.frames * ((L + 127) // 128) > 256
    say(f"case fused scan d={d} B={B} H={H} L={L} F={F}")
    inp = W.make_call_inputs(w, 0, F, 0)
    dev = upload(inp, "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    st = s0.clone()
    out = run_gpu(dev, st, w.L, True)
    st2 = s0.clone()
    snaps = torch.empty(B, H, F, d, d, device="cuda")
    api.hybrid_attn_state_update(dev["kp"], dev["vp"], dev["alpha"], dev["beta"], st2, w.L, snapshots=snaps)
    out2 = api.hybrid_attn_intra_readout(dev["q"], dev["k"], dev["v"], dev["qp"], snaps, F * d * d, d * d, w.L)
    torch.cuda.synchronize()
    assert torch.equal(st, st2)
    assert torch.equal(out, out2)


def test_fused_scan_graph_replay_matches_eager():
    # the frame counters are zeroed by each call's gram kernel, so replays of
    # a captured call start clean
    w = small("480p", B=1, H=8, L=200, frames=17, state0_sigma=0.05)
    say("case fused scan, graph replay")
    dev = upload(W.make_call_inputs(w, 0, w.frames, 0), "bf16")
    s0 = torch.from_numpy(W.make_state0(w)).cuda()
    out = torch.empty_like(dev["q"])
    ws = torch.empty(api.workspace_bytes(1, w.H, w.T, w.L, w.d, 1), dtype=torch.uint8, device="cuda")

    def call(state):
        api.hybrid_attn_forward(dev["q"], dev["k"], dev["v"], dev["qp"], dev["kp"], dev["vp"], dev["alpha"],
                                dev["beta"], state, w.L, 1, out=out, workspace=ws)

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
