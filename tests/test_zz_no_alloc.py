"""The allocation-free entry point against hybrid_attn_forward, through the C ABI.

hybrid_attn_forward_noalloc runs the same kernels as hybrid_attn_forward with
the library's fixed per-GPU scratch in place of a caller workspace, so its
output and state must equal the workspace call's bitwise. Two calls in a row,
the second with smaller sizes (the scratch keeps the first call's bytes), each
as a clean pass (state written) and as a denoising pass; the larger one is also
checked against the fp64 oracle on sampled heads.
"""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.gpu_util import TOL_OUT, TOL_STATE, f64, oracle_head, rel_err, upload
from video_dit_hybrid_amd import api
from video_dit_hybrid_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_pair(w, update, check_oracle=False):
    inp = W.make_call_inputs(w, 0, w.frames, 0, clean=True)
    s0 = W.make_state0(w)
    dev = upload(inp, w.dtype)
    args = [dev["q"], dev["k"], dev["v"], dev["qp"], dev.get("kp"), dev.get("vp"), dev.get("alpha"), dev.get("beta")]
    st_ref = torch.from_numpy(s0.copy()).cuda()
    out_ref = api.hybrid_attn_forward(*args, st_ref, w.L, int(update))
    st = torch.from_numpy(s0.copy()).cuda()
    out = torch.empty_like(dev["q"])
    api.hybrid_attn_forward_noalloc(*args, st, w.L, int(update), out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       out_ref.view(torch.int16) if out_ref.dtype == torch.bfloat16 else out_ref)
    assert torch.equal(st, st_ref)
    if not update:
        assert torch.equal(st, torch.from_numpy(s0).cuda())
    if check_oracle:
        x = f64(inp, w.dtype)
        got = W.to_f64(W.from_torch(out, w.dtype), w.dtype)
        S = st.cpu().numpy().astype(np.float64)
        for h in (0, w.H - 1):
            ref, Sref = oracle_head(x, s0, 0, h, w.L, update)
            eo = rel_err(got[0, :, h], ref)
            es = rel_err(S[0, h], Sref) if update else 0.0
            say(f"  head {h}: out {eo:.3e} state {es:.3e}")
            assert eo < TOL_OUT and es < TOL_STATE


@pytest.mark.parametrize("update", [1, 0])
def test_noalloc_matches_workspace_call_twice_second_smaller(update):
    big = dataclasses.replace(W.WORKLOADS["480p"], frames=4, state0_sigma=0.05)
    small = dataclasses.replace(W.WORKLOADS["480p"], H=3, L=200, frames=2, state0_sigma=0.05)
    for w, check in ((big, True), (small, False)):
        need = api.workspace_bytes(w.B, w.H, w.frames * w.L, w.L, w.d, update)
        say(f"case noalloc update={update} B={w.B} H={w.H} F={w.frames} L={w.L} workspace {need} B "
            f"(scratch {api.noalloc_scratch_bytes()} B)")
        assert need <= api.noalloc_scratch_bytes()
        run_pair(w, update, check_oracle=check)


def test_noalloc_one_frame_stream_step():
    # the streaming shape: one frame, clean pass (token-split increments in the scratch)
    w = dataclasses.replace(W.WORKLOADS["480p"], frames=1, H=12, state0_sigma=0.05)
    say("case noalloc one frame, 12 heads")
    run_pair(w, 1)
