"""The seeded input generator (CPU only)."""
import dataclasses

import numpy as np
import torch

from video_dit_hybrid_amd import workloads as W


def small(name, **kw):
    base = W.WORKLOADS[name]
    return dataclasses.replace(base, **kw)


def test_deterministic_and_slab_addressable():
    w = small("480p", H=3, L=40, frames=3)
    a = W.make_call_inputs(w, 0, 3, 0)
    b = W.make_call_inputs(w, 0, 3, 0)
    for key in a:
        assert np.array_equal(a[key], b[key])
    one = W.make_call_inputs(w, 1, 1, 0)
    for key in ("q", "kp", "vp", "beta"):
        assert np.array_equal(one[key][:, :, ...], a[key][:, 40:80, ...])
    assert np.array_equal(one["alpha"][:, 0], a["alpha"][:, 1])


def test_passes_and_streams_are_independent_draws():
    w = small("batched", L=16, H=2)
    p0 = W.make_call_inputs(w, 0, 1, 0, clean=False)
    p1 = W.make_call_inputs(w, 0, 1, 1, clean=False)
    assert set(p0) == {"q", "k", "v", "qp"}
    assert not np.array_equal(p0["q"], p1["q"])
    assert not np.array_equal(p0["q"][0], p0["q"][1])
    sub = W.make_call_inputs(w, 0, 1, 0, clean=False, streams=[3])
    assert np.array_equal(sub["q"][0], p0["q"][3])


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100_000).astype(np.float32) * 3.0
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_distributions_match_the_workload_definition():
    w = small("720p", H=4, L=64, frames=2)
    x = W.make_call_inputs(w, 0, 2, 0)
    kp = W.to_f64(x["kp"], "bf16")
    n = np.linalg.norm(kp, axis=-1)
    assert np.max(np.abs(n - 1.0)) < 2e-2            # unit rows up to bf16 rounding
    assert np.all(x["beta"] > 0) and np.all(x["beta"] < 1.0 / w.L)
    assert np.all(x["alpha"] > 0) and np.all(x["alpha"] < 1.0)
    # 720p gates: alpha = sigmoid(N(3, 0.5)) has mean ~0.95
    assert 0.9 < float(x["alpha"].mean()) < 0.99
    q = W.to_f64(x["q"], "bf16")
    assert abs(q.mean()) < 0.05 and abs(q.std() - 1.0) < 0.05
    t = W.make_call_inputs(W.WORKLOADS["tiny"], 0, 1, 0)
    assert t["q"].dtype == np.float32 and t["q"].shape == (1, 256, 2, 64)


def test_state0_and_schedules():
    assert not W.make_state0(W.WORKLOADS["480p"]).any()
    s = W.make_state0(W.WORKLOADS["batched"])
    assert s.shape == (8, 12, 128, 128) and abs(s.std() - 0.05) < 1e-3
    st = W.call_schedule(W.WORKLOADS["stream"])
    assert len(st) == 600 and sum(c for *_, c in st) == 120
    assert st[:5] == [(0, 1, 0, False), (0, 1, 1, False), (0, 1, 2, False), (0, 1, 3, False), (0, 1, 4, True)]
    assert W.call_schedule(W.WORKLOADS["480p"]) == [(0, 21, 0, True)]
    assert W.WORKLOADS["480p"].T == 32760 and W.WORKLOADS["720p"].T == 75600
