"""Pins of the fp64 oracle against what the ARL2 page and the mathematics fix.

Each check_* function raises AssertionError when the oracle it is handed
disagrees with a property that does not depend on the oracle itself: a
closed form worked out by hand, a textbook routine, brute force written with
scalar loops, or an invariant of the method ("Attend Locally, Remember
Linearly", section 2.1 update rule and readout, section 2.2 access rules).
The checks take the oracle module as an argument so that
tests/test_oracle_mutants.py can hand them deliberately broken copies.
"""
from __future__ import annotations

import math

import numpy as np


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, B=1, T=12, H=2, d=4, L=4, alpha=None, beta=None, S0=None):
    F = T // L
    q, k, v, qp, kp, vp = (_rand(rng, B, T, H, d) for _ in range(6))
    kp = _unit_rows(kp)
    a = rng.uniform(0.6, 0.99, (B, F, H)) if alpha is None else np.full((B, F, H), float(alpha))
    b = rng.uniform(0.01, 0.3, (B, T, H)) if beta is None else np.full((B, T, H), float(beta))
    s = 0.3 * _rand(rng, B, H, d, d) if S0 is None else S0
    return q, k, v, qp, kp, vp, a, b, s


# --- brute force with scalar loops (independent of numpy linear algebra) ------

def brute_layer_head(q, k, v, qp, kp, vp, alpha, beta, S, L, update, scale):
    """The layer for one head, written with Python scalar loops only."""
    T, d = len(q), len(q[0])
    S = [[float(S[i][j]) for j in range(d)] for i in range(d)]
    out = [[0.0] * d for _ in range(T)]
    for n in range(T // L):
        rows = range(n * L, (n + 1) * L)
        for i in rows:
            scores = [sum(q[i][c] * k[j][c] for c in range(d)) * scale for j in rows]
            m = max(scores)
            w = [math.exp(z - m) for z in scores]
            tot = sum(w)
            for c in range(d):
                intra = sum(w[jj] * v[j][c] for jj, j in enumerate(rows)) / tot
                inter = sum(qp[i][r] * S[r][c] for r in range(d))
                out[i][c] = intra + inter
        if update:
            a = float(alpha[n])
            newS = [[a * S[r][c] for c in range(d)] for r in range(d)]
            for t in rows:
                for c in range(d):
                    resid = vp[t][c] - sum(kp[t][r] * S[r][c] for r in range(d))
                    for r in range(d):
                        newS[r][c] += kp[t][r] * beta[t] * resid
            S = newS
    return np.array(out), np.array(S)


# --- the checks ---------------------------------------------------------------

def check_softmax_rows_sum_to_one(o):
    rng = np.random.default_rng(1)
    z = 4.0 * _rand(rng, 37, 53)
    p = o.softmax_rows(z)
    assert np.all(p > 0) and np.all(p <= 1)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    # two-element closed form: softmax([a, b]) = [1/(1+e^(b-a)), 1/(1+e^(a-b))]
    p2 = o.softmax_rows(np.array([[0.3, -1.2]]))
    assert abs(p2[0, 0] - 1.0 / (1.0 + math.exp(-1.5))) < 1e-15
    assert abs(p2[0, 1] - 1.0 / (1.0 + math.exp(1.5))) < 1e-15


def check_hand_worked_example(o):
    """Two frames of two tokens, d = 2, every value worked out by hand."""
    e = math.e
    I = np.eye(2)
    q = np.zeros((1, 4, 1, 2)); k = np.zeros_like(q); v = np.zeros_like(q)
    qp = np.zeros_like(q); kp = np.zeros_like(q); vp = np.zeros_like(q)
    # frame 0: Q = K = I, V = [[1,2],[3,4]], Q' = [[1,1],[0,2]], K' = I,
    #          V' = [[2,3],[4,5]], beta = (0.5, 0.25), alpha = 0.5, S0 = I
    q[0, 0:2, 0] = I; k[0, 0:2, 0] = I; v[0, 0:2, 0] = [[1, 2], [3, 4]]
    qp[0, 0:2, 0] = [[1, 1], [0, 2]]; kp[0, 0:2, 0] = I; vp[0, 0:2, 0] = [[2, 3], [4, 5]]
    # frame 1: Q = K = 0 (uniform softmax), V = [[2,0],[0,2]], Q' = I
    v[0, 2:4, 0] = [[2, 0], [0, 2]]; qp[0, 2:4, 0] = I; kp[0, 2:4, 0] = I
    alpha = np.array([[[0.5], [1.0]]])
    beta = np.zeros((1, 4, 1)); beta[0, 0:2, 0] = [0.5, 0.25]
    S0 = I.reshape(1, 1, 2, 2).copy()
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, alpha, beta, S0, 2, 1, scale=1.0)
    # frame 0 intra: softmax of the identity score matrix
    w0 = np.array([[e / (e + 1), 1 / (e + 1)], [1 / (e + 1), e / (e + 1)]])
    intra0 = w0 @ np.array([[1.0, 2.0], [3.0, 4.0]])
    want0 = intra0 + np.array([[1.0, 1.0], [0.0, 2.0]])          # + Q' S0
    # S1 = 0.5 I + diag(0.5, 0.25) ([[2,3],[4,5]] - I) = [[1, 1.5], [1, 1.5]]
    S1 = np.array([[1.0, 1.5], [1.0, 1.5]])
    want1 = np.array([[1.0, 1.0], [1.0, 1.0]]) + S1                 # uniform avg of V + I S1
    assert np.max(np.abs(out[0, 0:2, 0] - want0)) < 1e-14
    assert np.max(np.abs(out[0, 2:4, 0] - want1)) < 1e-14
    # frame 1 has beta = 0 and alpha = 1: S2 = S1
    assert np.max(np.abs(S[0, 0] - S1)) < 1e-14


def check_single_frame_is_textbook_attention(o):
    """F = 1, S0 = 0: the layer is plain softmax(QK^T/sqrt(d))V (2.1 item 1)."""
    import torch
    rng = np.random.default_rng(2)
    B, L, H, d = 2, 9, 3, 5
    q, k, v, qp, kp, vp, a, b, _ = _inputs(rng, B, L, H, d, L)
    S0 = np.zeros((B, H, d, d))
    out, _ = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, S0, L, 0)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def check_brute_force_tiny(o):
    """The whole layer against scalar-loop brute force, 3 frames, update on."""
    rng = np.random.default_rng(3)
    B, H, d, L, F = 1, 2, 3, 3, 3
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, B, F * L, H, d, L)
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, L, 1, scale=0.7)
    for h in range(H):
        ro, rs = brute_layer_head(q[0, :, h].tolist(), k[0, :, h].tolist(), v[0, :, h].tolist(),
                                  qp[0, :, h].tolist(), kp[0, :, h].tolist(), vp[0, :, h].tolist(),
                                  a[0, :, h], b[0, :, h], s[0, h], L, True, 0.7)
        assert np.max(np.abs(out[0, :, h] - ro)) < 1e-12
        assert np.max(np.abs(S[0, h] - rs)) < 1e-12


def check_alpha1_beta0_keeps_state(o):
    """alpha = 1, beta = 0: S_N = S_{N-1} exactly and O_inter = Q' S_0 always."""
    rng = np.random.default_rng(4)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 12, 2, 4, 4, alpha=1.0, beta=0.0)
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    assert np.array_equal(S, s)
    out0, _ = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 0)
    assert np.max(np.abs(out - out0)) == 0.0


def check_alpha0_beta0_clears_state(o):
    """alpha = 0, beta = 0: S_1 = 0, so frames >= 1 get no inter-frame term."""
    rng = np.random.default_rng(5)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 12, 2, 4, 4, alpha=0.0, beta=0.0)
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    assert np.all(S == 0.0)
    zero = np.zeros_like(s)
    out_z, _ = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, zero, 4, 0)
    assert np.max(np.abs(out[:, 4:] - out_z[:, 4:])) < 1e-14
    # frame 0 still reads S_0: its output differs from the S_0 = 0 output by Q' S_0
    diff = out[0, 0:4, 0] - out_z[0, 0:4, 0]
    assert np.max(np.abs(diff - qp[0, 0:4, 0] @ s[0, 0])) < 1e-13


def check_beta0_geometric_decay(o):
    """beta = 0: S_F = (prod alpha_n) S_0 (closed form)."""
    rng = np.random.default_rng(6)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 20, 2, 4, 4, beta=0.0)
    _, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    for h in range(2):
        want = np.prod(a[0, :, h]) * s[0, h]
        assert np.max(np.abs(S[0, h] - want)) < 1e-14


def check_delta_rule_recall(o):
    """Orthonormal K' rows, beta = 1: with alpha = 1 the written state recalls
    V' exactly (K' S_N = V'); with alpha < 1 the printed rule gives
    K' S_N = V' - (1 - alpha) K' S_{N-1} (residual against the undecayed state)."""
    rng = np.random.default_rng(7)
    L, d = 32, 64
    Qm, _ = np.linalg.qr(rng.standard_normal((d, L)))
    kp = Qm.T                                   # [L, d], orthonormal rows
    vp = rng.standard_normal((L, d))
    S_prev = rng.standard_normal((d, d))
    beta = np.ones(L)
    S1 = o.delta_update(S_prev, kp, vp, 1.0, beta)
    assert np.max(np.abs(kp @ S1 - vp)) < 1e-12
    S2 = o.delta_update(S_prev, kp, vp, 0.6, beta)
    assert np.max(np.abs(kp @ S2 - (vp - 0.4 * kp @ S_prev))) < 1e-12
    # directions orthogonal to the written keys only decay
    null = np.linalg.qr(np.concatenate([kp.T, rng.standard_normal((d, d - L))], axis=1))[0][:, L:]
    assert np.max(np.abs(null.T @ S2 - 0.6 * null.T @ S_prev)) < 1e-12


def check_affine_form(o):
    """S_N = (alpha I - K'^T diag(beta) K') S_{N-1} + K'^T diag(beta) V'."""
    rng = np.random.default_rng(8)
    L, d = 40, 16
    kp = _unit_rows(rng.standard_normal((L, d))); vp = rng.standard_normal((L, d))
    S = rng.standard_normal((d, d)); beta = rng.uniform(0, 1, L)
    A = 0.8 * np.eye(d) - kp.T @ np.diag(beta) @ kp
    Bm = kp.T @ np.diag(beta) @ vp
    assert np.max(np.abs(o.delta_update(S, kp, vp, 0.8, beta) - (A @ S + Bm))) < 1e-12


def check_column_separability(o):
    """Column j of V' only moves column j of S and of later O_inter."""
    rng = np.random.default_rng(9)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 12, 1, 4, 4)
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    vp2 = vp.copy(); vp2[0, :, 0, 2] += 1.0
    out2, S2 = o.hybrid_layer(q, k, v, qp, kp, vp2, a, b, s, 4, 1)
    other = [0, 1, 3]
    assert np.max(np.abs(S2[0, 0][:, other] - S[0, 0][:, other])) < 1e-14
    assert np.max(np.abs(S2[0, 0][:, 2] - S[0, 0][:, 2])) > 1e-3
    assert np.max(np.abs(out2[..., other] - out[..., other])) < 1e-14
    assert np.max(np.abs(out2[0, 4:, 0, 2] - out[0, 4:, 0, 2])) > 1e-4


def check_token_permutation(o):
    """Permuting the tokens of a frame permutes its output rows; S is invariant."""
    rng = np.random.default_rng(10)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 12, 2, 4, 4)
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    perm = np.arange(12); perm[4:8] = [6, 4, 7, 5]
    P = lambda x: x[:, perm]
    out2, S2 = o.hybrid_layer(P(q), P(k), P(v), P(qp), P(kp), P(vp), a, P(b), s, 4, 1)
    assert np.max(np.abs(out2 - out[:, perm])) < 1e-12
    assert np.max(np.abs(S2 - S)) < 1e-12


def check_frame_isolation(o):
    """Changing frame m leaves earlier outputs untouched and the intra branch of
    every other frame untouched (2.1 item 1, 2.2 frame-level access)."""
    rng = np.random.default_rng(11)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 16, 2, 4, 4)
    out, _ = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    k2 = k.copy(); k2[0, 8:12] += 0.5 * rng.standard_normal(k2[0, 8:12].shape)
    vp2 = vp.copy(); vp2[0, 8:12] += 0.5
    out2, _ = o.hybrid_layer(q, k2, v, qp, kp, vp2, a, b, s, 4, 1)
    assert np.max(np.abs(out2[:, :8] - out[:, :8])) == 0.0
    assert np.max(np.abs(out2[:, 8:12] - out[:, 8:12])) > 1e-6
    # frame 3 changes only through O_inter (vp of frame 2 moved the state)
    zero_s = np.zeros_like(s)
    i1, _ = o.hybrid_layer(q, k, v, 0 * qp, kp, vp, a, b, zero_s, 4, 0)
    i2, _ = o.hybrid_layer(q, k2, v, 0 * qp, kp, vp2, a, b, zero_s, 4, 0)
    assert np.max(np.abs(i1[:, 12:] - i2[:, 12:])) == 0.0


def check_call_splitting(o):
    """One F-frame clean call equals F single-frame clean calls."""
    rng = np.random.default_rng(12)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 2, 15, 2, 4, 5)
    out, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 5, 1)
    St = s.copy()
    for n in range(3):
        r = slice(5 * n, 5 * n + 5)
        on, St = o.hybrid_layer(q[:, r], k[:, r], v[:, r], qp[:, r], kp[:, r], vp[:, r],
                                a[:, n:n + 1], b[:, r], St, 5, 1)
        assert np.max(np.abs(on - out[:, r])) < 1e-12
    assert np.max(np.abs(St - S)) < 1e-12


def check_denoise_pass_leaves_state(o):
    """update_state = 0 never writes S; a denoise pass and the clean pass over
    the same inputs give the same output (2.2 clean-pass updates)."""
    rng = np.random.default_rng(13)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 4, 2, 4, 4)
    o0, S0 = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 0)
    assert np.array_equal(S0, s)
    o1, S1 = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    assert np.array_equal(o0, o1)
    assert not np.allclose(S1, s)
    # with update_state = 0 every frame of a multi-frame call reads the input S
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 8, 1, 4, 4)
    o2, _ = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 0)
    for n in range(2):
        r = slice(4 * n, 4 * n + 4)
        want = o.intra_frame_attention(q[0, r, 0], k[0, r, 0], v[0, r, 0]) + qp[0, r, 0] @ s[0, 0]
        assert np.max(np.abs(o2[0, r, 0] - want)) < 1e-13


def check_state_chain_matches_layer(o):
    """state_chain's last state equals the layer's final state, per head."""
    rng = np.random.default_rng(14)
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, 1, 12, 2, 4, 4)
    _, S = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, 4, 1)
    for h in range(2):
        ch = o.state_chain(kp[0, :, h], vp[0, :, h], a[0, :, h], b[0, :, h], s[0, h], 4)
        assert len(ch) == 4
        assert np.max(np.abs(ch[-1] - S[0, h])) < 1e-14


def _fmap_inputs(rng, B=1, T=8, H=3, d=4, L=4):
    q, k, v, _, _, _, a, b, S0 = _inputs(rng, B=B, T=T, H=H, d=d, L=L)
    w = [rng.standard_normal((H, d, d)) / math.sqrt(d) for _ in range(3)]
    return q, k, v, w, a, b, S0


def check_fmap_brute_force(o):
    """Feature maps by scalar loops: Q'[b,t,h,e] = sum_j Q[b,t,h,j] W[h][j,e]
    (a 1x1 map per head, grouped by head), then the layer on them."""
    rng = np.random.default_rng(21)
    q, k, v, (wq, wk, wv), a, b, S0 = _fmap_inputs(rng, B=2, T=8, H=2, d=3)
    B, T, H, d = q.shape
    maps = []
    for x, w in ((q, wq), (k, wk), (v, wv)):
        y = np.zeros_like(x)
        for bb in range(B):
            for t in range(T):
                for h in range(H):
                    for e in range(d):
                        acc = 0.0
                        for j in range(d):
                            acc += x[bb, t, h, j] * w[h][j, e]
                        y[bb, t, h, e] = acc
        maps.append(y)
    got = o.feature_maps(q, k, v, wq, wk, wv)
    for g, want in zip(got, maps):
        assert np.allclose(g, want, rtol=1e-12, atol=1e-12)
    out, st = o.hybrid_layer_fmap(q, k, v, wq, wk, wv, a, b, S0, 4, 1)
    out2, st2 = o.hybrid_layer(q, k, v, *maps, a, b, S0, 4, 1)
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-12) and np.allclose(st, st2, rtol=1e-12, atol=1e-12)


def check_fmap_permutation(o):
    """A permutation matrix as every map: Q' is Q with its channels reordered
    (a cyclic shift, which a transposed map would shift the other way)."""
    rng = np.random.default_rng(22)
    q, k, v, _, a, b, S0 = _fmap_inputs(rng, H=2, d=4)
    d = q.shape[3]
    P = np.zeros((d, d))
    for j in range(d):
        P[j, (j + 1) % d] = 1.0  # e = j + 1: Q'[..., e] = Q[..., e - 1]
    W = np.stack([P, P])
    qp, kp, vp = o.feature_maps(q, k, v, W, W, W)
    assert np.array_equal(qp, np.roll(q, 1, axis=3))
    assert np.array_equal(kp, np.roll(k, 1, axis=3)) and np.array_equal(vp, np.roll(v, 1, axis=3))


def check_fmap_grouped_by_head(o):
    """Each head uses its own maps: changing head 1's maps leaves head 0's
    outputs and state unchanged and changes head 1's."""
    rng = np.random.default_rng(23)
    q, k, v, (wq, wk, wv), a, b, S0 = _fmap_inputs(rng, H=2)
    out, st = o.hybrid_layer_fmap(q, k, v, wq, wk, wv, a, b, S0, 4, 1)
    for i in range(3):
        w2 = [wq.copy(), wk.copy(), wv.copy()]
        w2[i][1] = rng.standard_normal(w2[i][1].shape)
        out2, st2 = o.hybrid_layer_fmap(q, k, v, *w2, a, b, S0, 4, 1)
        assert np.array_equal(out2[:, :, 0], out[:, :, 0]) and np.array_equal(st2[:, 0], st[:, 0])
        assert not np.allclose(out2[:, :, 1], out[:, :, 1])


def check_fmap_fold(o):
    """The identities the GPU path folds the maps with (exact algebra):
    Q'S = Q (W_q S), and one clean frame gives
    S_N = (alpha I - W_k^T G0 W_k) S + W_k^T B0 W_v with G0 = K^T diag(beta) K,
    B0 = K^T diag(beta) V of the unmapped K, V."""
    rng = np.random.default_rng(24)
    q, k, v, (wq, wk, wv), a, b, S0 = _fmap_inputs(rng, B=1, T=4, H=1, d=4, L=4)
    S = S0[0, 0] + 0.3 * rng.standard_normal(S0[0, 0].shape)
    S0 = S[None, None]
    out, st = o.hybrid_layer_fmap(q, k, v, wq, wk, wv, a, b, S0, 4, 1)
    K, V, Q = k[0, :, 0], v[0, :, 0], q[0, :, 0]
    G0 = K.T @ (b[0, :, 0][:, None] * K)
    B0 = K.T @ (b[0, :, 0][:, None] * V)
    Wq, Wk, Wv = wq[0], wk[0], wv[0]
    want_S = (a[0, 0, 0] * np.eye(4) - Wk.T @ G0 @ Wk) @ S + Wk.T @ B0 @ Wv
    assert np.allclose(st[0, 0], want_S, rtol=1e-10, atol=1e-12)
    intra = o.intra_frame_attention(Q, K, V)
    assert np.allclose(out[0, :, 0], intra + Q @ (Wq @ S), rtol=1e-10, atol=1e-12)



# --- gates and K' normalisation ---------------------------------------------

def _gate_inputs(rng, B=2, T=8, C=5, H=2):
    x = rng.standard_normal((B, T, C))
    wg = rng.standard_normal((2, H, C)) / math.sqrt(C)
    bg = rng.standard_normal((2, H))
    return x, wg, bg


def _brute_gates(x, wg, bg, L):
    """alpha and beta by scalar loops and math.exp."""
    B, T, C = x.shape
    H = wg.shape[1]
    F = T // L
    alpha = np.zeros((B, F, H))
    beta = np.zeros((B, T, H))
    for bb in range(B):
        for h in range(H):
            for n in range(F):
                acc = 0.0
                for t in range(n * L, (n + 1) * L):
                    za = bg[0, h]
                    zb = bg[1, h]
                    for c in range(C):
                        za += x[bb, t, c] * wg[0, h, c]
                        zb += x[bb, t, c] * wg[1, h, c]
                    acc += 1.0 / (1.0 + math.exp(-za))
                    beta[bb, t, h] = (1.0 / (1.0 + math.exp(-zb))) / L
                alpha[bb, n, h] = acc / L
    return alpha, beta


def _brute_normalize(x):
    y = np.zeros_like(x)
    for idx in np.ndindex(*x.shape[:-1]):
        row = [float(e) for e in x[idx]]
        nrm = math.sqrt(sum(e * e for e in row))
        y[idx] = [e / max(nrm, 1e-12) for e in row]
    return y


def check_gates_brute_force(o):
    """alpha = frame mean of sigmoid(x.w_alpha + b), beta = sigmoid(x.w_beta + b) / L,
    per head, against scalar loops."""
    rng = np.random.default_rng(31)
    x, wg, bg = _gate_inputs(rng)
    a, b = o.gate_projections(x, wg, bg, 4)
    wa, wb = _brute_gates(x, wg, bg, 4)
    assert a.shape == (2, 2, 2) and b.shape == (2, 8, 2)
    assert np.allclose(a, wa, rtol=1e-13, atol=1e-15) and np.allclose(b, wb, rtol=1e-13, atol=1e-15)


def check_gates_zero_projection(o):
    """Zero weights and biases: every gate is sigmoid(0) = 1/2 exactly, so
    alpha = 1/2 and beta = 1/(2L)."""
    rng = np.random.default_rng(32)
    x, wg, bg = _gate_inputs(rng, T=12)
    a, b = o.gate_projections(x, 0 * wg, 0 * bg, 4)
    assert np.all(a == 0.5) and np.all(b == 0.125)


def check_gates_constant_frame(o):
    """A frame whose tokens are all equal has alpha equal to that token's
    gate (the mean of equal values): sigmoid(x.w + b) by hand."""
    rng = np.random.default_rng(33)
    x, wg, bg = _gate_inputs(rng, B=1, T=8, C=3, H=2)
    x[0, 4:8] = x[0, 5]
    a, _ = o.gate_projections(x, wg, bg, 4)
    for h in range(2):
        z = bg[0, h] + sum(x[0, 5, c] * wg[0, h, c] for c in range(3))
        assert abs(a[0, 1, h] - 1.0 / (1.0 + math.exp(-z))) < 1e-15


def check_gates_token_permutation(o):
    """Permuting the tokens inside a frame leaves alpha (a frame mean) and
    permutes beta; gates of one head ignore the other heads' weights."""
    rng = np.random.default_rng(34)
    x, wg, bg = _gate_inputs(rng, B=1, T=8, C=6, H=3)
    a, b = o.gate_projections(x, wg, bg, 4)
    perm = np.array([2, 0, 3, 1, 4, 5, 6, 7])
    a2, b2 = o.gate_projections(x[:, perm], wg, bg, 4)
    assert np.allclose(a2, a, rtol=1e-14, atol=0) and np.array_equal(b2, b[:, perm])
    wg2 = wg.copy()
    wg2[:, 1] = rng.standard_normal(wg2[:, 1].shape)
    a3, b3 = o.gate_projections(x, wg2, bg, 4)
    for h in (0, 2):
        assert np.array_equal(a3[..., h], a[..., h]) and np.array_equal(b3[..., h], b[..., h])
    assert not np.allclose(a3[..., 1], a[..., 1]) and not np.allclose(b3[..., 1], b[..., 1])


def check_key_normalisation(o):
    """Normalised K' rows: scalar-loop division by the row's L2 norm; unit
    norms; a zero row stays zero; scaling a token's K by c > 0 leaves K'."""
    rng = np.random.default_rng(35)
    q, k, v, (wq, wk, wv), _, _, _ = _fmap_inputs(rng, B=1, T=8, H=2, d=3)
    k[0, 3, 1] = 0.0
    _, kp, _ = o.feature_maps(q, k, v, wq, wk, wv, True)
    _, raw, _ = o.feature_maps(q, k, v, wq, wk, wv)
    assert np.allclose(kp, _brute_normalize(raw), rtol=1e-13, atol=1e-15)
    nrm = np.sqrt((kp ** 2).sum(-1))
    assert np.all(kp[0, 3, 1] == 0.0)
    nrm[0, 3, 1] = 1.0
    assert np.allclose(nrm, 1.0, rtol=0, atol=1e-14)
    c = rng.uniform(0.1, 10.0, (1, 8, 2, 1))
    qp2, kp2, vp2 = o.feature_maps(q, k * c, v, wq, wk, wv, True)
    assert np.allclose(kp2, kp, rtol=1e-13, atol=1e-15)


def check_gated_layer_wiring(o):
    """hybrid_layer_gated = hybrid_layer on brute-force gates and brute-force
    maps with K' (and only K') normalised; without the flag, K' is the plain map."""
    rng = np.random.default_rng(36)
    B, T, H, d, C, L = 1, 8, 2, 3, 5, 4
    q, k, v, (wq, wk, wv), _, _, S0 = _fmap_inputs(rng, B=B, T=T, H=H, d=d, L=L)
    x, wg, bg = _gate_inputs(rng, B=B, T=T, C=C, H=H)
    wa, wb = _brute_gates(x, wg, bg, L)
    maps = []
    for xx, w in ((q, wq), (k, wk), (v, wv)):
        y = np.zeros_like(xx)
        for t in range(T):
            for h in range(H):
                for e in range(d):
                    y[0, t, h, e] = sum(xx[0, t, h, j] * w[h][j, e] for j in range(d))
        maps.append(y)
    for norm in (True, False):
        kk = _brute_normalize(maps[1]) if norm else maps[1]
        out, st, a, b = o.hybrid_layer_gated(x, q, k, v, wq, wk, wv, wg, bg, S0, L, 1, norm)
        out2, st2 = o.hybrid_layer(q, k, v, maps[0], kk, maps[2], wa, wb, S0, L, 1)
        assert np.allclose(a, wa, rtol=1e-13, atol=1e-15) and np.allclose(b, wb, rtol=1e-13, atol=1e-15)
        assert np.allclose(out, out2, rtol=1e-11, atol=1e-12) and np.allclose(st, st2, rtol=1e-11, atol=1e-12)


def check_gated_fold_normalised(o):
    """The identity the GPU path uses for normalised keys (exact algebra):
    with n_t = ||K_t W_k||, one clean frame gives
    S_N = (alpha I - W_k^T K^T diag(beta/n^2) K W_k) S + W_k^T K^T diag(beta/n) V W_v;
    and the final state does not change when a token's K is scaled by c > 0."""
    rng = np.random.default_rng(37)
    L, d, C = 4, 4, 6
    q, k, v, (wq, wk, wv), _, _, S0 = _fmap_inputs(rng, B=1, T=4, H=1, d=d, L=L)
    x, wg, bg = _gate_inputs(rng, B=1, T=4, C=C, H=1)
    S = S0[0, 0] + 0.3 * rng.standard_normal((d, d))
    _, st, a, b = o.hybrid_layer_gated(x, q, k, v, wq, wk, wv, wg, bg, S[None, None], L, 1, True)
    K, V, Wk, Wv = k[0, :, 0], v[0, :, 0], wk[0], wv[0]
    n = np.sqrt(((K @ Wk) ** 2).sum(1))
    bt = b[0, :, 0]
    G0 = K.T @ ((bt / n ** 2)[:, None] * K)
    B0 = K.T @ ((bt / n)[:, None] * V)
    want = (a[0, 0, 0] * np.eye(d) - Wk.T @ G0 @ Wk) @ S + Wk.T @ B0 @ Wv
    assert np.allclose(st[0, 0], want, rtol=1e-10, atol=1e-12)
    c = rng.uniform(0.2, 5.0, (1, 4, 1, 1))
    _, st2, _, _ = o.hybrid_layer_gated(x, q, k * c, v, wq, wk, wv, wg, bg, S[None, None], L, 1, True)
    assert np.allclose(st2, st, rtol=1e-11, atol=1e-13)



# --- the KV-cache softmax teacher ---------------------------------------------

def check_chunk_causal_single_frame(o):
    """One frame: chunk-causal attention is the frame's own softmax attention."""
    rng = np.random.default_rng(41)
    q, k, v = (rng.standard_normal((8, 4)) for _ in range(3))
    assert np.allclose(o.chunk_causal_attention(q, k, v, 8), o.intra_frame_attention(q, k, v),
                       rtol=1e-14, atol=1e-15)


def check_chunk_causal_is_block_masked_sdpa(o):
    """Against torch's fp64 scaled_dot_product_attention with an explicit
    block mask: key j is visible to query i iff frame(j) <= frame(i); and the
    last frame sees every key (the unmasked routine)."""
    import torch
    rng = np.random.default_rng(42)
    T, d, L = 12, 5, 4
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    got = o.chunk_causal_attention(q, k, v, L)
    fr = np.arange(T) // L
    mask = torch.from_numpy(fr[None, :] <= fr[:, None])
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)[0, 0].numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
    full = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
    assert np.allclose(got[8:], full[8:], rtol=1e-12, atol=1e-13)


def check_chunk_causal_brute_force(o):
    """Scalar loops: softmax over keys of frames <= the query's frame."""
    rng = np.random.default_rng(43)
    T, d, L = 6, 3, 2
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    sc = 0.7
    got = o.chunk_causal_attention(q, k, v, L, sc)
    for i in range(T):
        vis = range(0, (i // L + 1) * L)
        z = [sum(q[i, c] * k[j, c] for c in range(d)) * sc for j in vis]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        den = sum(e)
        for c in range(d):
            want = sum(e[t] * v[j, c] for t, j in enumerate(vis)) / den
            assert abs(got[i, c] - want) < 1e-13


def check_chunk_causal_causality_and_streaming(o):
    """Perturbing frame m leaves the outputs of frames < m and changes those of
    frames >= m; frame by frame over a growing cache (each frame's queries on
    the keys of the frames so far) equals the whole call; the order of the
    visible past tokens does not matter (attention over a set)."""
    rng = np.random.default_rng(44)
    T, d, L = 16, 4, 4
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    out = o.chunk_causal_attention(q, k, v, L)
    k2, v2 = k.copy(), v.copy()
    k2[8:12] += 1.0
    v2[8:12] -= 0.5
    out2 = o.chunk_causal_attention(q, k2, v2, L)
    assert np.array_equal(out2[:8], out[:8]) and not np.allclose(out2[8:], out[8:])
    for n in range(4):
        step = o.intra_frame_attention(q[n * L:(n + 1) * L], k[:(n + 1) * L], v[:(n + 1) * L])
        assert np.allclose(step, out[n * L:(n + 1) * L], rtol=1e-14, atol=1e-15)
    perm = np.concatenate([rng.permutation(12), np.arange(12, 16)])
    last = o.intra_frame_attention(q[12:], k[perm], v[perm])
    assert np.allclose(last, out[12:], rtol=1e-13, atol=1e-14)



# --- token-level access ----------------------------------------------------------

def _tok_inputs(rng, T=12, d=4, L=4):
    q, k, v, qp, kp, vp = (rng.standard_normal((T, d)) for _ in range(6))
    kp = kp / np.linalg.norm(kp, axis=1, keepdims=True)
    a = rng.uniform(0.5, 0.95, T // L)
    b = rng.uniform(0.05, 0.4, T)
    S0 = 0.3 * rng.standard_normal((d, d))
    return q, k, v, qp, kp, vp, a, b, S0


def check_token_level_one_token_frames(o):
    """L = 1: every frame is one token, so token-level and frame-level access
    coincide; the same layer through hybrid_layer_head."""
    rng = np.random.default_rng(51)
    q, k, v, qp, kp, vp, a, b, S0 = _tok_inputs(rng, T=6, L=1)
    out, S = o.hybrid_layer_token_level(q, k, v, qp, kp, vp, a, b, S0, 1, 1)
    out2, S2 = o.hybrid_layer_head(q, k, v, qp, kp, vp, a, b, S0, 1, 1)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-14) and np.allclose(S, S2, rtol=1e-13, atol=1e-14)


def check_token_level_beta0_closed_form(o):
    """beta = 0: the first token of frame N reads (prod_{m<N} alpha_m) S_0, the
    others (prod_{m<=N} alpha_m) S_0; the final state is (prod alpha) S_0."""
    rng = np.random.default_rng(52)
    q, k, v, qp, kp, vp, a, b, S0 = _tok_inputs(rng)
    out, S = o.hybrid_layer_token_level(q, k, v, qp, kp, vp, a, 0 * b, S0, 4, 1)
    intra = np.concatenate([o.intra_frame_attention(q[i:i + 4], k[i:i + 4], v[i:i + 4]) for i in (0, 4, 8)])
    for t in range(12):
        n = t // 4
        f = np.prod(a[:n]) * (1.0 if t % 4 == 0 else a[n])
        assert np.allclose(out[t] - intra[t], f * (qp[t] @ S0), rtol=1e-12, atol=1e-13)
    assert np.allclose(S, np.prod(a) * S0, rtol=1e-13, atol=1e-15)


def check_token_level_brute_force_and_recall(o):
    """Scalar loops over tokens; with beta = 1, alpha = 1 and unit keys each
    token's write is recalled exactly: k'_t S_t = v'_t (the delta rule)."""
    rng = np.random.default_rng(53)
    q, k, v, qp, kp, vp, a, b, S0 = _tok_inputs(rng, T=6, d=3, L=3)
    out, S = o.hybrid_layer_token_level(q, k, v, qp, kp, vp, a, b, S0, 3, 1)
    d = 3
    St = [[S0[i][j] for j in range(d)] for i in range(d)]
    for t in range(6):
        inter = [sum(qp[t][i] * St[i][j] for i in range(d)) for j in range(d)]
        n = t // 3
        want = o.intra_frame_attention(q[n * 3:(n + 1) * 3], k[n * 3:(n + 1) * 3], v[n * 3:(n + 1) * 3])[t % 3]
        for j in range(d):
            assert abs(out[t][j] - (want[j] + inter[j])) < 1e-12
        aa = a[n] if t % 3 == 0 else 1.0
        ks = [sum(kp[t][i] * St[i][j] for i in range(d)) for j in range(d)]
        St = [[aa * St[i][j] + b[t] * kp[t][i] * (vp[t][j] - ks[j]) for j in range(d)] for i in range(d)]
    assert np.allclose(S, np.array(St), rtol=1e-12, atol=1e-13)
    # recall
    _, S1 = o.hybrid_layer_token_level(q[:1], k[:1], v[:1], qp[:1], kp[:1], vp[:1], np.ones(1), np.ones(1), S0, 1, 1)
    assert np.allclose(kp[0] @ S1, vp[0], rtol=1e-12, atol=1e-12)


def check_token_level_chunked_wy_form(o):
    """The chunked form the GPU path evaluates (exact algebra): for a chunk of
    tokens inside one frame with entry state S and decay a (alpha of the frame
    for its first chunk, else 1), D = diag(1, a, .., a), T = (I + strict_lower(
    diag(beta) K K^T))^-1, X = T diag(beta) V - T diag(beta) D K S; then
    S_end = a S + K^T X and the tokens read c_t S + sum_{j<t} (q_t.k_j) X_j,
    c = (1, a, .., a). Chunks of 3 tokens over frames of 6."""
    rng = np.random.default_rng(54)
    q, k, v, qp, kp, vp, a, b, S0 = _tok_inputs(rng, T=12, d=4, L=6)
    out, Sf = o.hybrid_layer_token_level(q, k, v, qp, kp, vp, a, b, S0, 6, 1)
    intra = np.concatenate([o.intra_frame_attention(q[i:i + 6], k[i:i + 6], v[i:i + 6]) for i in (0, 6)])
    S = S0.copy()
    for c0 in range(0, 12, 3):
        r = slice(c0, c0 + 3)
        dec = a[c0 // 6] if c0 % 6 == 0 else 1.0
        K, V, Q, bt = kp[r], vp[r], qp[r], b[r]
        Dv = np.array([1.0, dec, dec])
        Tm = np.linalg.inv(np.eye(3) + np.tril(bt[:, None] * (K @ K.T), -1))
        X = Tm @ (bt[:, None] * V) - Tm @ ((bt * Dv)[:, None] * K) @ S
        inter = Dv[:, None] * (Q @ S) + np.tril(Q @ K.T, -1) @ X
        assert np.allclose(out[r] - intra[r], inter, rtol=1e-11, atol=1e-12)
        S = dec * S + K.T @ X
    assert np.allclose(S, Sf, rtol=1e-11, atol=1e-12)


def check_token_level_denoise_and_causality(o):
    """update_state = 0 returns the input state and the same outputs; perturbing
    token j moves the inter-frame outputs of later tokens only."""
    rng = np.random.default_rng(55)
    q, k, v, qp, kp, vp, a, b, S0 = _tok_inputs(rng)
    out, S = o.hybrid_layer_token_level(q, k, v, qp, kp, vp, a, b, S0, 4, 1)
    out0, S_0 = o.hybrid_layer_token_level(q, k, v, qp, kp, vp, a, b, S0, 4, 0)
    assert np.array_equal(out0, out) and np.array_equal(S_0, S0)
    vp2 = vp.copy()
    vp2[5] += 1.0
    out2, _ = o.hybrid_layer_token_level(q, k, v, qp, kp, vp2, a, b, S0, 4, 1)
    assert np.array_equal(out2[:6], out[:6]) and not np.allclose(out2[6], out[6])


def _mix_inputs(rng, B=2, H=3, d=4, L=4, F=3):
    q, k, v, qp, kp, vp, a, b, s = _inputs(rng, B, F * L, H, d, L)
    mix = rng.uniform(-1.0, 2.0, size=(B, H, 2))
    return q, k, v, qp, kp, vp, a, b, s, mix, L


def check_mix_unit_weights_is_the_plain_layer(o):
    """Weights (1, 1) give the plain sum O_intra + O_inter exactly, and the
    state never depends on the weights."""
    rng = np.random.default_rng(41)
    q, k, v, qp, kp, vp, a, b, s, mix, L = _mix_inputs(rng)
    ref, Sref = o.hybrid_layer(q, k, v, qp, kp, vp, a, b, s, L, 1)
    out, S = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, np.ones_like(mix))
    assert np.array_equal(out, ref) and np.array_equal(S, Sref)
    _, S2 = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, mix)
    assert np.array_equal(S2, Sref)


def check_mix_softmax_only_is_textbook_attention(o):
    """LinVideo r = 1 (weights (1, 0)): every frame is plain per-frame softmax
    attention whatever the state; r = 0 (weights (0, 1)): Q'_N S_{N-1} by scalar
    loops over a state chain computed token by token."""
    import torch
    rng = np.random.default_rng(42)
    q, k, v, qp, kp, vp, a, b, s, mix, L = _mix_inputs(rng, B=1, H=2, d=3, L=3, F=2)
    B, T, H, d = q.shape
    out, _ = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, np.tile([1.0, 0.0], (B, H, 1)))
    for n in range(T // L):
        r = slice(n * L, (n + 1) * L)
        tq, tk, tv = (torch.from_numpy(x[:, r]).permute(0, 2, 1, 3) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).numpy()
        assert np.max(np.abs(out[:, r] - ref)) < 1e-12
    out, _ = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, np.tile([0.0, 1.0], (B, H, 1)))
    for h in range(H):
        S = [[float(s[0, h, i, j]) for j in range(d)] for i in range(d)]
        for n in range(T // L):
            for t in range(n * L, (n + 1) * L):
                for j in range(d):
                    want = sum(qp[0, t, h, i] * S[i][j] for i in range(d))
                    assert abs(out[0, t, h, j] - want) < 1e-12
            an = float(a[0, n, h])
            new = [[an * S[i][j] for j in range(d)] for i in range(d)]
            for t in range(n * L, (n + 1) * L):
                resid = [vp[0, t, h, j] - sum(kp[0, t, h, i] * S[i][j] for i in range(d)) for j in range(d)]
                for i in range(d):
                    for j in range(d):
                        new[i][j] += kp[0, t, h, i] * float(b[0, t, h]) * resid[j]
            S = new


def check_mix_weights_per_stream_and_head(o):
    """Each (stream, head) takes its own pair: the output is linear in the two
    weights, with the branches of weights (1, 0) and (0, 1)."""
    rng = np.random.default_rng(43)
    q, k, v, qp, kp, vp, a, b, s, mix, L = _mix_inputs(rng, B=2, H=3)
    B, _, H, _ = q.shape
    o10, _ = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, np.tile([1.0, 0.0], (B, H, 1)))
    o01, _ = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, np.tile([0.0, 1.0], (B, H, 1)))
    out, _ = o.hybrid_layer_mixed(q, k, v, qp, kp, vp, a, b, s, L, 1, mix)
    for bb in range(B):
        for h in range(H):
            want = mix[bb, h, 0] * o10[bb, :, h] + mix[bb, h, 1] * o01[bb, :, h]
            assert np.max(np.abs(out[bb, :, h] - want)) < 1e-12


ALL_CHECKS = [
    check_mix_unit_weights_is_the_plain_layer,
    check_mix_softmax_only_is_textbook_attention,
    check_mix_weights_per_stream_and_head,
    check_token_level_one_token_frames,
    check_token_level_beta0_closed_form,
    check_token_level_brute_force_and_recall,
    check_token_level_chunked_wy_form,
    check_token_level_denoise_and_causality,
    check_chunk_causal_single_frame,
    check_chunk_causal_is_block_masked_sdpa,
    check_chunk_causal_brute_force,
    check_chunk_causal_causality_and_streaming,
    check_gates_brute_force,
    check_gates_zero_projection,
    check_gates_constant_frame,
    check_gates_token_permutation,
    check_key_normalisation,
    check_gated_layer_wiring,
    check_gated_fold_normalised,
    check_fmap_brute_force,
    check_fmap_permutation,
    check_fmap_grouped_by_head,
    check_fmap_fold,
    check_softmax_rows_sum_to_one,
    check_hand_worked_example,
    check_single_frame_is_textbook_attention,
    check_brute_force_tiny,
    check_alpha1_beta0_keeps_state,
    check_alpha0_beta0_clears_state,
    check_beta0_geometric_decay,
    check_delta_rule_recall,
    check_affine_form,
    check_column_separability,
    check_token_permutation,
    check_frame_isolation,
    check_call_splitting,
    check_denoise_pass_leaves_state,
    check_state_chain_matches_layer,
]
