"""The HA_LOG and HA_CHECK_FINITE diagnostics of the library, on the GPU."""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.gpu_util import run_gpu, upload
from video_dit_hybrid_amd import api
from video_dit_hybrid_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture()
def env():
    saved = {k: os.environ.get(k) for k in ("HA_LOG", "HA_CHECK_FINITE")}
    yield os.environ
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def small_call(update=True, nan_state=False, nan_vp=False):
    w = dataclasses.replace(W.WORKLOADS["480p"], H=2, L=200, frames=3, state0_sigma=0.05)
    inp = W.make_call_inputs(w, 0, w.frames, 0)
    dev = upload(inp, "bf16")
    s0 = W.make_state0(w)
    if nan_state:
        s0[0, 1, 5, 7] = np.nan
    if nan_vp:
        dev["vp"][0, 250, 0, 3] = float("inf")
    st = torch.from_numpy(s0.copy()).cuda()
    return w, dev, st


def test_check_finite_passes_clean_calls_unchanged(env):
    w, dev, st = small_call()
    ref_st = st.clone()
    ref = run_gpu(dev, ref_st, w.L, True)
    env["HA_CHECK_FINITE"] = "1"
    out = run_gpu(dev, st, w.L, True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(st, ref_st)


@pytest.mark.parametrize("where", ["state", "vp"])
def test_check_finite_reports_nonfinite_state(env, where):
    w, dev, st = small_call(nan_state=where == "state", nan_vp=where == "vp")
    # without the flag the call goes through (the state just holds the NaN / Inf)
    env.pop("HA_CHECK_FINITE", None)
    run_gpu(dev, st.clone(), w.L, True)
    torch.cuda.synchronize()
    env["HA_CHECK_FINITE"] = "1"
    with pytest.raises(api.HybridAttnError) as e:
        run_gpu(dev, st, w.L, True)
    assert e.value.status == 9
    assert not torch.isfinite(st).all()


def test_log_prints_calls_and_launches(env, capfd):
    w, dev, st = small_call()
    env["HA_LOG"] = "1"
    run_gpu(dev, st, w.L, True)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "hybrid_attn_forward: B=1 H=2 T=600 (3 frames x 200 tokens) d=128 bf16 update_state=1" in err
    assert "launch gram_bf16_kernel<128>" in err
    assert "launch state_scan_mfma_kernel<128>" in err
    assert "launch attn_bf16_kernel<128>: grid" in err and "readout from bf16 fragments" in err
    env["HA_LOG"] = "0"
    run_gpu(dev, st, w.L, True)
    torch.cuda.synchronize()
    assert "[hybrid_attn]" not in capfd.readouterr().err
