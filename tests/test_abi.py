"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments before any device work (no GPU needed)."""
import ctypes
import os
import re

import pytest

from video_dit_hybrid_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hybrid_attn.h")

P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hybrid_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 7
    L = api.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(api.EXPORTS) == set(names)


def test_debug_library_exports_every_declared_symbol():
    # the build with device index checks (__graft_entry__.build() makes both)
    from video_dit_hybrid_amd import build as B
    if not os.path.exists(B.DEBUG_LIB_PATH):
        pytest.skip("the debug library is not built")
    L = ctypes.CDLL(B.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert api.lib().hybrid_attn_version() >= 100
    for code in range(10):
        s = api.status_string(code)
        assert s and s != "unknown status"
    assert api.status_string(99) == "unknown status"


def test_workspace_sizes():
    d, H, L, F = 128, 12, 1560, 21
    gram = H * F * d * 2 * d * 4
    snaps = H * F * d * d * 4
    up = lambda x: (x + 255) // 256 * 256
    assert api.workspace_bytes(1, H, F * L, L, d, 0) == 0
    assert api.workspace_bytes(1, H, F * L, L, d, 1) == up(gram) + up(snaps)
    # F = 1: no snapshots; only 12 (stream, head, frame) groups, so the
    # increments are computed in min(ceil(256 / 12), 16, 25 chunks) = 16 token
    # splits whose fp32 partial sums (d x 2d each) follow the increments
    assert api.workspace_bytes(1, H, L, L, d, 1) == up(H * d * 2 * d * 4 * (1 + 16))
    # 96 groups: 3 splits; 128 or more groups: no split
    assert api.workspace_bytes(8, H, L, L, d, 1) == up(8 * H * d * 2 * d * 4 * (1 + 3))
    assert api.workspace_bytes(1, 128, L, L, d, 1) == up(128 * d * 2 * d * 4)
    # never more splits than 64-token chunks: L = 100 has 2
    assert api.workspace_bytes(1, 1, 100, 100, d, 1) == up(d * 2 * d * 4 * (1 + 2))
    assert api.state_workspace_bytes(1, H, F * L, L, d) == up(gram)
    assert api.workspace_bytes(1, H, F * L + 1, L, d, 1) == 0                # invalid sizes


def fwd(**kw):
    a = dict(q=4096, k=8192, v=12288, qp=16384, kp=20480, vp=24576, alpha=28672, beta=32768,
             state=36864, out=1 << 40, ws=1 << 41, ws_bytes=1 << 40, B=1, H=2, T=64, d=64, L=32,
             dtype=0, update=1, scale=0.0)
    a.update(kw)
    ptr = lambda x: None if x is None else P(x)
    return api.lib().hybrid_attn_forward(
        ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["qp"]), ptr(a["kp"]), ptr(a["vp"]),
        ptr(a["alpha"]), ptr(a["beta"]), ptr(a["state"]), ptr(a["out"]), ptr(a["ws"]),
        a["ws_bytes"], a["B"], a["H"], a["T"], a["d"], a["L"], a["dtype"], a["update"],
        a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(state=None), 1), (dict(out=None), 1),
    (dict(kp=None), 1), (dict(alpha=None), 1), (dict(beta=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(T=0), 2), (dict(L=0), 2), (dict(T=65), 2),
    (dict(B=1 << 20, H=1 << 12, T=1 << 20, L=1), 2),
    (dict(T=40000, L=1, d=128), 2),   # per-(stream, head) state increments past 32-bit offsets
    (dict(d=96), 3), (dict(d=256), 3), (dict(dtype=2), 3),
    (dict(q=4097), 4), (dict(out=(1 << 40) + 8), 4), (dict(alpha=28673), 4), (dict(state=36868), 4),
    (dict(ws=None), 5), (dict(ws_bytes=100), 5),
    (dict(out=8192), 7), (dict(out=36864 - 64), 7),
])
def test_validation_codes(kw, code):
    assert fwd(**kw) == code


def test_denoise_pass_needs_no_update_inputs():
    # update_state = 0: kp, vp, alpha, beta, workspace may be NULL. A valid call
    # would launch, so only check that the NULLs are not what gets rejected:
    # give it an invalid d to stop before any device work.
    assert fwd(kp=None, vp=None, alpha=None, beta=None, ws=None, ws_bytes=0, update=0, d=96) == 3
    assert fwd(kp=None, vp=None, alpha=None, beta=None, ws=None, ws_bytes=0, update=0, q=4097) == 4


def test_sub_entry_points_validate():
    L = api.lib()
    r = L.hybrid_attn_intra_readout(P(4096), P(8192), P(12288), P(16384), P(20480), 64 * 64, 0,
                                    P(1 << 40), 1, 2, 64, 64, 33, 0, 0.0, None)
    assert r == 2
    r = L.hybrid_attn_intra_readout(P(4096), P(8192), P(12288), P(16384), P(20480), 64 * 64 + 2, 0,
                                    P(1 << 40), 1, 2, 64, 64, 32, 0, 0.0, None)
    assert r == 4
    r = L.hybrid_attn_state_update(P(4096), P(8192), P(12288), P(16384), P(20480), None, P(1 << 40),
                                   10, 1, 2, 64, 64, 32, 0, None)
    assert r == 5
    r = L.hybrid_attn_state_update(P(4096), None, P(12288), P(16384), P(20480), None, P(1 << 40),
                                   1 << 30, 1, 2, 64, 64, 32, 0, None)
    assert r == 1


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 32, 2, 64, dtype=torch.bfloat16)
    s = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError):
        api.hybrid_attn_forward(x, x, x, x, x, x, None, None, s, 32, 0)


def test_feature_map_and_gated_workspace_sizes():
    d, H, L, F = 128, 12, 1560, 21
    T = F * L
    up = lambda x: (x + 255) // 256 * 256
    gf = H * F * d * 2 * d * 4
    # increments, partial sums, fp32 snapshots, readout fragments, frame counters
    fmap1 = up(gf) + up(gf) + up(H * F * d * d * 4) + up(H * F * d * d * 2) + up(H * F * 4)
    assert api.fmap_workspace_bytes(1, H, T, L, d, 0) == up(H * d * d * 2)
    assert api.fmap_workspace_bytes(1, H, T, L, d, 1) == fmap1
    # gated: beta, beta / n^2, beta / n, per-64-token-chunk alpha sums (25 chunks
    # of a 1560-token frame), alpha
    tok = up(T * H * 4)
    assert api.gated_workspace_bytes(1, H, T, L, d, 1) == fmap1 + 3 * tok + up(F * 25 * H * 4) + up(F * H * 4)
    assert api.gated_workspace_bytes(1, H, T, L, d, 0) == api.fmap_workspace_bytes(1, H, T, L, d, 0)
    assert api.gates_workspace_bytes(1, H, T, L) == up(F * 25 * H * 4)
    assert api.gated_workspace_bytes(1, H, T + 1, L, d, 1) == 0


def gated(**kw):
    a = dict(x=4096, q=8192, k=12288, v=16384, wq=20480, wk=24576, wv=28672, wg=32768, bg=36864,
             state=40960, out=1 << 40, ws=1 << 41, ws_bytes=1 << 40, B=1, H=2, T=64, d=64, C=128, L=32,
             dtype=0, update=1, norm=1, scale=0.0)
    a.update(kw)
    ptr = lambda x: None if x is None else P(x)
    return api.lib().hybrid_attn_forward_gated(
        ptr(a["x"]), ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["wq"]), ptr(a["wk"]), ptr(a["wv"]),
        ptr(a["wg"]), ptr(a["bg"]), ptr(a["state"]), ptr(a["out"]), ptr(a["ws"]), a["ws_bytes"], a["B"],
        a["H"], a["T"], a["d"], a["C"], a["L"], a["dtype"], a["update"], a["norm"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(wg=None), 1), (dict(bg=None), 1), (dict(wk=None), 1), (dict(q=None), 1),
    (dict(C=0), 2), (dict(C=24), 2), (dict(T=65), 2), (dict(C=1 << 23), 2),
    (dict(H=65), 3), (dict(dtype=1), 3), (dict(d=96), 3),
    (dict(x=4100), 4), (dict(wg=32772), 4), (dict(bg=36866), 4),
    (dict(ws_bytes=100), 5),
    (dict(out=4096), 7), (dict(out=32768), 7),
])
def test_gated_validation_codes(kw, code):
    assert gated(**kw) == code


def test_gated_denoise_pass_needs_no_gate_inputs():
    # update_state = 0 reads neither x nor the gate weights nor wk, wv (and C
    # is ignored); stop before device work with an invalid d
    assert gated(x=None, wk=None, wv=None, wg=None, bg=None, C=0, update=0, d=96) == 3
    assert gated(x=None, wk=None, wv=None, wg=None, bg=None, C=0, update=0, q=8196) == 4


def test_gates_entry_validates():
    L = api.lib()

    def g(x=4096, wg=8192, bg=12288, al=16384, be=20480, ws=1 << 41, wsb=1 << 40, B=1, H=2, T=64, C=64,
          Lf=32, dtype=0):
        p = lambda v: None if v is None else P(v)
        return L.hybrid_attn_gates(p(x), p(wg), p(bg), p(al), p(be), p(ws), wsb, B, H, T, C, Lf, dtype, None)
    assert g(C=8) == 2 and g(T=65) == 2
    assert g(C=1 << 23) == 2  # 64 tokens of C channels past 32-bit byte offsets
    assert g(al=None) == 1 and g(ws=None) == 1
    assert g(H=65) == 3 and g(dtype=1) == 3
    assert g(x=4097) == 4
    assert g(wsb=4) == 5
    assert g(be=16384 + 8) == 7


def test_kvcache_workspace_and_validation():
    up = lambda x: (x + 255) // 256 * 256
    L, H, d = 1560, 12, 128
    # one frame against a cache of 1 frame: 156 query work-groups, 25 key tiles: no split
    assert api.kvcache_workspace_bytes(1, H, L, L, d, 0) == 0
    # at frame 20: 512 key tiles, ceil(512 / 156) = 4 splits
    rows = L * H
    assert api.kvcache_workspace_bytes(1, H, L, L, d, 20) == up(4 * rows * d * 4) + up(4 * rows * 8)
    # a 21-frame call has 3276 query work-groups: no split
    assert api.kvcache_workspace_bytes(1, H, 21 * L, L, d, 0) == 0
    assert api.kvcache_workspace_bytes(1, H, L + 1, L, d, 0) == 0

    def kv(q=4096, k=8192, v=12288, kc=1 << 30, vc=1 << 31, out=1 << 32, ws=None, wsb=0, B=1, H=2, T=64, d=64,
           L=32, cap=4, fi=0, dtype=0):
        p = lambda x: None if x is None else P(x)
        return api.lib().hybrid_attn_kvcache_forward(p(q), p(k), p(v), p(kc), p(vc), p(out), p(ws), wsb, B, H, T,
                                                     d, L, cap, fi, dtype, 0.0, None)
    assert kv(fi=3) == 2 and kv(cap=1) == 2 and kv(fi=-1) == 2
    assert kv(q=None) == 1 and kv(kc=None) == 1
    assert kv(dtype=1) == 3 and kv(d=96) == 3
    assert kv(k=8200) == 4
    assert kv(out=(1 << 30) + 64) == 7 and kv(k=(1 << 31) + 64) == 7
    # a long cache with one frame of queries needs split workspace
    assert kv(T=1560, L=1560, H=12, d=128, cap=40, fi=30, q=1 << 33, k=1 << 34, v=1 << 35, kc=1 << 36,
              vc=1 << 37, out=1 << 38) == 5


def test_token_level_workspace_and_validation():
    up = lambda x: (x + 255) // 256 * 256
    L, H, d, F = 1560, 12, 128, 21
    chunks = H * F * 25
    assert api.token_level_workspace_bytes(1, H, F * L, L, d) == up(chunks * 96 * 1024) + up(F * L * H * d * 4)
    assert api.token_level_workspace_bytes(1, H, F * L, L, 64) == 0

    def tl(d=128, dtype=0, q=4096, kp=8192, ws=1 << 40, wsb=1 << 40, out=1 << 41):
        p = lambda x: None if x is None else P(x)
        return api.lib().hybrid_attn_forward_token_level(p(q), P(12288), P(16384), P(20480), p(kp), P(24576),
                                                         P(28672), P(32768), P(36864), p(out), p(ws), wsb, 1, 2, 64,
                                                         d, 32, dtype, 1, 0.0, None)
    assert tl(d=64) == 3 and tl(dtype=1) == 3
    assert tl(kp=None) == 1 and tl(ws=None) == 1
    assert tl(q=4100) == 4
    assert tl(wsb=64) == 5
    assert tl(out=8192) == 7


# Buffers 4 GiB apart, so no two overlap unless a case moves one onto another.
SEP = dict(q=1 << 32, k=2 << 32, v=3 << 32, qp=4 << 32, kp=5 << 32, vp=6 << 32, alpha=7 << 32, beta=8 << 32,
           state=9 << 32, out=10 << 32, ws=11 << 32, ws_bytes=1 << 40, d=96)


@pytest.mark.parametrize("kw", [
    dict(ws=SEP["q"] + 64), dict(ws=SEP["kp"]), dict(ws=SEP["beta"] + 16), dict(ws=SEP["state"] - 256),
    dict(state=SEP["kp"] + 1024), dict(state=SEP["alpha"]), dict(state=SEP["q"]),
    dict(out=SEP["state"] + 512), dict(out=SEP["ws"] + 4096),
])
def test_forward_rejects_written_buffers_that_overlap(kw):
    # d = 96 would be HA_ERR_UNSUPPORTED; use d = 64 so the alias check is what
    # decides (a call that passes every check would launch: none here does)
    a = dict(SEP, d=64)
    a.update(kw)
    assert fwd(**a) == 7


def test_forward_written_state_must_not_share_inputs():
    # with update_state = 1 the state is written: overlapping q is rejected
    # (a call that passed every check would launch, so the read-only case of
    # update_state = 0 is covered by the GPU tests instead)
    assert fwd(**dict(SEP, state=SEP["q"], update=1, d=64)) == 7


def state_update(kp=1 << 32, vp=2 << 32, alpha=3 << 32, beta=4 << 32, state=5 << 32, snaps=6 << 32, ws=7 << 32,
                 wsb=1 << 40, B=1, H=2, T=64, d=64, L=32):
    p = lambda x: None if x is None else P(x)
    return api.lib().hybrid_attn_state_update(p(kp), p(vp), p(alpha), p(beta), p(state), p(snaps), p(ws), wsb, B,
                                              H, T, d, L, 0, None)


@pytest.mark.parametrize("kw", [
    dict(snaps=1 << 32), dict(snaps=(2 << 32) + 4096), dict(snaps=(5 << 32) + 1024), dict(snaps=(7 << 32) + 256),
    dict(ws=(1 << 32) + 16), dict(ws=(4 << 32)), dict(ws=(5 << 32) + 16384),
    dict(state=(2 << 32) + 64), dict(state=3 << 32),
])
def test_state_update_rejects_written_buffers_that_overlap(kw):
    assert state_update(**kw) == 7


def test_state_update_snapshots_optional_and_sized_by_frames():
    # snapshots [B, H, F, d, d] fp32: 2 frames x 2 heads x 16 KiB = 64 KiB, so
    # a workspace 256 bytes before their end overlaps them
    snap = 1 << 36
    assert state_update(snaps=snap, ws=snap + 65536 - 256) == 7
    # without snapshots: a state (2 heads x 16 KiB) reaching 256 bytes into the
    # workspace
    assert state_update(snaps=None, ws=5 << 32, state=(5 << 32) - 32768 + 256) == 7


def test_feature_map_entry_rejects_workspace_over_inputs():
    def fm(ws=9 << 32, update=1, state=7 << 32, d=64):
        return api.lib().hybrid_attn_forward_fmap(P(1 << 32), P(2 << 32), P(3 << 32), P(4 << 32), P(5 << 32),
                                                  P(6 << 32), P(10 << 32), P(11 << 32), P(state), P(8 << 32), P(ws),
                                                  1 << 40, 1, 2, 64, d, 32, 0, update, 0.0, None)
    assert fm(ws=(5 << 32) + 64) == 7           # workspace over wk
    assert fm(ws=(11 << 32)) == 7               # workspace over beta
    assert fm(state=2 << 32) == 7               # written state over k


def test_status_string_of_every_status():
    for code in range(10):
        assert api.status_string(code) != "unknown status"
    for code in (10, 99, -1, 2**31 - 1):
        assert api.status_string(code) == "unknown status"


def noalloc(**kw):
    a = dict(SEP, d=64, B=1, H=2, T=64, L=32, dtype=0, update=1, scale=0.0)
    a.update(kw)
    ptr = lambda x: None if x is None else P(x)
    return api.lib().hybrid_attn_forward_noalloc(
        ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["qp"]), ptr(a["kp"]), ptr(a["vp"]), ptr(a["alpha"]),
        ptr(a["beta"]), ptr(a["state"]), ptr(a["out"]), a["B"], a["H"], a["T"], a["d"], a["L"], a["dtype"],
        a["update"], a["scale"], None)


def test_noalloc_entry_validates_before_touching_its_scratch():
    assert api.noalloc_scratch_bytes() == 64 << 20
    assert noalloc(q=None) == 1 and noalloc(alpha=None) == 1
    assert noalloc(T=65) == 2 and noalloc(d=96) == 3 and noalloc(dtype=2) == 3
    assert noalloc(q=SEP["q"] + 4) == 4
    # a denoise pass needs no workspace, so the alias rules are checked without
    # a scratch lookup
    assert noalloc(update=0, out=SEP["k"] + 64) == 7
    # the 720p 14B-shaped clean call needs 165 MiB of workspace: more than the
    # fixed scratch holds
    need = api.workspace_bytes(1, 40, 21 * 3600, 3600, 128, 1)
    assert need > api.noalloc_scratch_bytes()
    assert noalloc(H=40, T=21 * 3600, L=3600, d=128) == 8
    # the 480p clean call fits
    assert api.workspace_bytes(1, 12, 21 * 1560, 1560, 128, 1) <= api.noalloc_scratch_bytes()
