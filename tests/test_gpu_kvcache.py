"""The KV-cache softmax teacher (hybrid_attn_kvcache_forward) against the fp64
oracle (oracle.hybrid_oracle.chunk_causal_attention) on an MI355X, through the
C ABI. Output bar as the layer's: 2e-2 of max|O| (bf16 operands, fp32
accumulation; reached about 4e-3)."""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.hybrid_oracle as O
from tests.gpu_util import TOL_OUT, rel_err
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


def small(**kw):
    return dataclasses.replace(W.WORKLOADS["480p"], **kw)


def qkv(w, frames, pass_=0, frame0=0):
    inp = W.make_call_inputs(w, frame0, frames, pass_, tensors=["q", "k", "v"])
    return ({k: W.as_torch(x, "bf16") for k, x in inp.items()},
            {k: W.to_f64(x, "bf16") for k, x in inp.items()})


def cache(w, frames):
    shape = (w.B, frames * w.L, w.H, w.d)
    return (torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
            torch.zeros(shape, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("d,L,F,B,H", [(128, 300, 3, 1, 2), (64, 130, 2, 2, 1), (128, 17, 4, 1, 2),
                                       (128, 1560, 2, 1, 12), (64, 64, 5, 1, 3)])
def test_whole_video_call(d, L, F, B, H):
    """One call over F frames from an empty cache: frame n attends to frames
    0..n (the teacher-forcing form); partial tiles, both head sizes."""
    w = small(d=d, L=L, frames=F, B=B, H=H)
    say(f"case kv whole d={d} L={L} F={F} B={B} H={H}")
    dev, x = qkv(w, F)
    kc, vc = cache(w, F + 1)
    out = api.hybrid_attn_kvcache_forward(dev["q"], dev["k"], dev["v"], kc, vc, L, 0)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = O.chunk_causal_attention(x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h], L)
            worst = max(worst, rel_err(got[b, :, h], ref))
    say(f"kv whole: rel_err out {worst:.3e}")
    assert worst < TOL_OUT
    assert torch.equal(kc[:, :F * L], dev["k"]) and torch.equal(vc[:, :F * L], dev["v"])


@pytest.mark.parametrize("d,L,H,n_frames", [(128, 1560, 12, 6), (128, 200, 2, 4), (64, 100, 3, 5)])
def test_streaming_denoise_then_clean(d, L, H, n_frames):
    """Frame by frame (F = 1 per call, key splits once the cache is long):
    per frame two denoising passes, whose K, V are overwritten, then the clean
    pass; the clean outputs match the oracle on the clean K, V of all frames so
    far, and each denoising output matches attention over the clean past plus
    the pass's own frame."""
    w = small(d=d, L=L, H=H, frames=n_frames, B=1)
    say(f"case kv stream d={d} L={L} H={H} frames={n_frames}")
    kc, vc = cache(w, n_frames)
    ks, vs = [], []
    worst = 0.0
    splits = set()
    for n in range(n_frames):
        splits.add(api.kvcache_workspace_bytes(1, H, L, L, d, n) > 0)
        for p in range(3):  # passes 0, 1 denoise, 2 clean
            dev, x = qkv(w, 1, pass_=p, frame0=n)
            out = api.hybrid_attn_kvcache_forward(dev["q"], dev["k"], dev["v"], kc, vc, L, n)
            torch.cuda.synchronize()
            got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
            K = np.concatenate(ks + [x["k"][0]], axis=0)
            V = np.concatenate(vs + [x["v"][0]], axis=0)
            for h in range(H):
                ref = O.intra_frame_attention(x["q"][0, :, h], K[:, h], V[:, h])
                worst = max(worst, rel_err(got[0, :, h], ref))
        ks.append(x["k"][0])
        vs.append(x["v"][0])
    say(f"kv stream: rel_err out {worst:.3e}; split paths taken: {sorted(splits)}")
    assert worst < TOL_OUT
    full_k = torch.from_numpy(np.concatenate([W.bf16_bits(k.astype(np.float32)) for k in ks]).view(np.int16))
    assert torch.equal(kc[0].cpu().view(torch.int16), full_k)


def test_streaming_equals_whole_video_reads():
    """The cache after F streaming clean calls holds the same bytes as after
    one F-frame call, and a final frame read against either cache is bitwise
    equal (same shape, same split count)."""
    w = small(L=300, H=2, frames=4, B=1)
    say("case kv stream vs whole cache")
    dev, _ = qkv(w, 4)
    kc1, vc1 = cache(w, 5)
    api.hybrid_attn_kvcache_forward(dev["q"], dev["k"], dev["v"], kc1, vc1, w.L, 0)
    kc2, vc2 = cache(w, 5)
    for n in range(4):
        r = slice(n * w.L, (n + 1) * w.L)
        api.hybrid_attn_kvcache_forward(dev["q"][:, r].contiguous(), dev["k"][:, r].contiguous(),
                                        dev["v"][:, r].contiguous(), kc2, vc2, w.L, n)
    torch.cuda.synchronize()
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    nxt, _ = qkv(w, 1, frame0=4)
    o1 = api.hybrid_attn_kvcache_forward(nxt["q"], nxt["k"], nxt["v"], kc1, vc1, w.L, 4)
    o2 = api.hybrid_attn_kvcache_forward(nxt["q"], nxt["k"], nxt["v"], kc2, vc2, w.L, 4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_480p_late_frame_sampled():
    """The 480p shape at frame 20 (21 frames of keys, 32,760 per head) as the
    bench streams it: two heads against the oracle."""
    w = W.WORKLOADS["480p"]
    say("case kv 480p frame 20")
    kc, vc = cache(w, 21)
    dev, x = qkv(w, 21)
    api.hybrid_attn_kvcache_forward(dev["q"][:, :20 * w.L].contiguous(), dev["k"][:, :20 * w.L].contiguous(),
                                    dev["v"][:, :20 * w.L].contiguous(), kc, vc, w.L, 0)
    r = slice(20 * w.L, 21 * w.L)
    out = api.hybrid_attn_kvcache_forward(dev["q"][:, r].contiguous(), dev["k"][:, r].contiguous(),
                                          dev["v"][:, r].contiguous(), kc, vc, w.L, 20)
    torch.cuda.synchronize()
    got = W.to_f64(W.from_torch(out, "bf16"), "bf16")
    worst = 0.0
    for h in (0, 11):
        ref = O.intra_frame_attention(x["q"][0, r, h], x["k"][0, :, h], x["v"][0, :, h])
        worst = max(worst, rel_err(got[0, :, h], ref))
    say(f"kv 480p frame 20: rel_err out {worst:.3e} (split: {api.kvcache_workspace_bytes(1, 12, w.L, w.L, 128, 20) > 0})")
    assert worst < TOL_OUT
