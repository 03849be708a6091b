"""Plant plausible mistakes in a private copy of the oracle (CPU only) and check
that at least one pin catches each: the pins are only worth something if a
dropped term, a wrong sign or index, or a transposed operand fails them."""
import importlib.util
import os

import numpy as np
import pytest

from tests.oracle_pins import ALL_CHECKS

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "hybrid_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant_copy", ORACLE_FILE)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def m_no_transpose(m):
    def f(state, kp, vp, alpha, beta):
        return alpha * state + kp @ (beta[:, None] * (vp - kp @ state))
    m.delta_update = f


def m_decayed_residual(m):
    def f(state, kp, vp, alpha, beta):
        return alpha * state + kp.T @ (beta[:, None] * (vp - kp @ (alpha * state)))
    m.delta_update = f


def m_sign(m):
    def f(state, kp, vp, alpha, beta):
        return alpha * state - kp.T @ (beta[:, None] * (vp - kp @ state))
    m.delta_update = f


def m_drop_alpha(m):
    def f(state, kp, vp, alpha, beta):
        return state + kp.T @ (beta[:, None] * (vp - kp @ state))
    m.delta_update = f


def m_drop_beta(m):
    def f(state, kp, vp, alpha, beta):
        return alpha * state + kp.T @ (vp - kp @ state)
    m.delta_update = f


def m_drop_residual_term(m):
    def f(state, kp, vp, alpha, beta):
        return alpha * state + kp.T @ (beta[:, None] * vp)
    m.delta_update = f


def m_readout_transposed(m):
    m.inter_frame_readout = lambda qp, state: qp @ state.T


def m_softmax_columns(m):
    def f(z):
        z = np.asarray(z, dtype=np.float64)
        e = np.exp(z - z.max(axis=0, keepdims=True))
        return e / e.sum(axis=0, keepdims=True)
    m.softmax_rows = f


def m_no_scale(m):
    orig = m.intra_frame_attention

    def f(q, k, v, scale=None):
        return orig(q, k, v, 1.0 if scale is None else scale)
    m.intra_frame_attention = f


def m_pv_transposed_keys(m):
    def f(q, k, v, scale=None):
        s = 1.0 / np.sqrt(q.shape[1]) if scale is None else scale
        return m.softmax_rows((k @ q.T) * s) @ v
    m.intra_frame_attention = f


def _layer_head_variant(m, read_after_update=False, global_attention=False,
                        always_update=False, alpha_index_shift=False):
    def f(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, scale=None, frames=None):
        T = q.shape[0]; L = int(frame_len); F = T // L
        S = np.array(state, dtype=np.float64, copy=True)
        out = np.full((T, v.shape[1]), np.nan)
        for n in range(F):
            r = slice(n * L, (n + 1) * L)
            kk = slice(0, T) if global_attention else r
            Snew = S
            if update_state or always_update:
                an = float(alpha[min(n + 1, F - 1)] if alpha_index_shift else alpha[n])
                Snew = m.delta_update(S, kp[r], vp[r], an, beta[r])
            Sread = Snew if read_after_update else S
            out[r] = m.intra_frame_attention(q[r], k[kk], v[kk], scale) + m.inter_frame_readout(qp[r], Sread)
            S = Snew
        return out, S
    m.hybrid_layer_head = f


def m_fmap_transposed(m):
    def f(q, k, v, wq, wk, wv):
        out = []
        for x, w in ((q, wq), (k, wk), (v, wv)):
            y = np.empty_like(x)
            for h in range(x.shape[2]):
                y[:, :, h, :] = x[:, :, h, :] @ w[h].T
            out.append(y)
        return tuple(out)
    m.feature_maps = f


def m_fmap_head0(m):
    def f(q, k, v, wq, wk, wv):
        return tuple(np.einsum("bthd,de->bthe", x, w[0]) for x, w in ((q, wq), (k, wk), (v, wv)))
    m.feature_maps = f


def m_fmap_wk_for_v(m):
    orig = m.feature_maps
    m.feature_maps = lambda q, k, v, wq, wk, wv: orig(q, k, v, wq, wk, wk)


def m_fmap_maps_intra_branch(m):
    def f(q, k, v, wq, wk, wv, alpha, beta, state, frame_len, update_state, scale=None):
        qp, kp, vp = m.feature_maps(q, k, v, wq, wk, wv)
        return m.hybrid_layer(qp, kp, vp, qp, kp, vp, alpha, beta, state, frame_len, update_state, scale)
    m.hybrid_layer_fmap = f



def m_gates_swapped(m):
    orig = m.gate_projections
    m.gate_projections = lambda x, wg, bg, L: orig(x, wg[::-1], bg[::-1], L)


def m_beta_not_over_frame_len(m):
    orig = m.gate_projections
    def f(x, wg, bg, L):
        a, b = orig(x, wg, bg, L)
        return a, b * L
    m.gate_projections = f


def m_alpha_first_token(m):
    def f(x, wg, bg, L):
        B, T, _ = x.shape
        a = m.sigmoid(x @ wg[0].T + bg[0])
        g = m.sigmoid(x @ wg[1].T + bg[1])
        return a[:, ::L], g / L
    m.gate_projections = f


def m_alpha_sigmoid_of_mean_logit(m):
    def f(x, wg, bg, L):
        B, T, _ = x.shape
        z = x @ wg[0].T + bg[0]
        g = m.sigmoid(x @ wg[1].T + bg[1])
        return m.sigmoid(z.reshape(B, T // L, L, -1).mean(axis=2)), g / L
    m.gate_projections = f


def m_gates_no_bias(m):
    orig = m.gate_projections
    m.gate_projections = lambda x, wg, bg, L: orig(x, wg, 0 * bg, L)


def m_normalise_wrong_axis(m):
    def f(x, eps=1e-12):
        n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
        return x / np.maximum(n, eps)
    m.l2_normalize_rows = f


def m_normalise_before_map(m):
    orig = m.feature_maps
    def f(q, k, v, wq, wk, wv, normalize_k=False):
        kk = m.l2_normalize_rows(k) if normalize_k else k
        return orig(q, kk, v, wq, wk, wv, False)
    m.feature_maps = f


def m_normalise_q_too(m):
    orig = m.feature_maps
    def f(q, k, v, wq, wk, wv, normalize_k=False):
        qp, kp, vp = orig(q, k, v, wq, wk, wv, normalize_k)
        return (m.l2_normalize_rows(qp) if normalize_k else qp), kp, vp
    m.feature_maps = f



def _causal_variant(m, lo=None, hi=None, token_causal=False):
    def f(q, k, v, frame_len, scale=None):
        T, L = q.shape[0], int(frame_len)
        out = np.empty_like(v, dtype=np.float64)
        for n in range(T // L):
            r = slice(n * L, (n + 1) * L)
            a = 0 if lo is None else lo(n, L)
            b = (n + 1) * L if hi is None else min(T, hi(n, L))
            if token_causal:
                for i in range(n * L, (n + 1) * L):
                    out[i] = m.intra_frame_attention(q[i:i + 1], k[a:i + 1], v[a:i + 1], scale)[0]
            else:
                out[r] = m.intra_frame_attention(q[r], k[a:b], v[a:b], scale)
        return out
    m.chunk_causal_attention = f



def _token_variant(m, decay_every_token=False, read_after=False, decayed_residual=False):
    def f(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, scale=None):
        T, L = q.shape[0], int(frame_len)
        S = np.array(state, dtype=np.float64, copy=True)
        out = np.empty_like(vp, dtype=np.float64)
        for n in range(T // L):
            r = slice(n * L, (n + 1) * L)
            out[r] = m.intra_frame_attention(q[r], k[r], v[r], scale)
        for t in range(T):
            a = float(alpha[t // L]) if (t % L == 0 or decay_every_token) else 1.0
            base = a * S if decayed_residual else S
            Sn = a * S + float(beta[t]) * np.outer(kp[t], vp[t] - kp[t] @ base)
            out[t] += qp[t] @ (Sn if read_after else S)
            S = Sn
        return out, (S if update_state else np.array(state, dtype=np.float64, copy=True))
    m.hybrid_layer_token_level = f


def _mix_variant(m, swap=False, transpose=False, scale_update=False):
    base = m.hybrid_layer_mixed

    def f(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, mix, scale=None):
        mx = np.array(mix, dtype=np.float64, copy=True)
        if swap:
            mx = mx[:, :, ::-1]
        if transpose:  # an off-by-one head index: head h takes head h - 1's pair
            mx = np.roll(mx, 1, axis=1)
        out, st = base(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, mx, scale)
        if scale_update and update_state:
            st = st * mx[:, :, 1][:, :, None, None]
        return out, st
    m.hybrid_layer_mixed = f


MUTANTS = {
    "mix_weights_swapped": lambda m: _mix_variant(m, swap=True),
    "mix_head_index_shifted": lambda m: _mix_variant(m, transpose=True),
    "mix_scales_the_state": lambda m: _mix_variant(m, scale_update=True),
    "token_decay_every_token": lambda m: _token_variant(m, decay_every_token=True),
    "token_reads_own_write": lambda m: _token_variant(m, read_after=True),
    "token_decayed_residual": lambda m: _token_variant(m, decayed_residual=True),
    "causal_sees_next_frame": lambda m: _causal_variant(m, hi=lambda n, L: (n + 2) * L),
    "causal_misses_own_frame": lambda m: _causal_variant(m, hi=lambda n, L: max(n, 1) * L),
    "causal_own_frame_only": lambda m: _causal_variant(m, lo=lambda n, L: n * L),
    "causal_token_mask_in_frame": lambda m: _causal_variant(m, token_causal=True),
    "gates_swapped": m_gates_swapped,
    "beta_not_over_frame_len": m_beta_not_over_frame_len,
    "alpha_first_token": m_alpha_first_token,
    "alpha_sigmoid_of_mean_logit": m_alpha_sigmoid_of_mean_logit,
    "gates_no_bias": m_gates_no_bias,
    "normalise_wrong_axis": m_normalise_wrong_axis,
    "normalise_before_map": m_normalise_before_map,
    "normalise_q_too": m_normalise_q_too,
    "fmap_transposed": m_fmap_transposed,
    "fmap_head0_for_all": m_fmap_head0,
    "fmap_wk_for_v": m_fmap_wk_for_v,
    "fmap_maps_intra_branch": m_fmap_maps_intra_branch,
    "no_transpose": m_no_transpose,
    "decayed_residual": m_decayed_residual,
    "update_sign": m_sign,
    "drop_alpha": m_drop_alpha,
    "drop_beta": m_drop_beta,
    "drop_residual_term": m_drop_residual_term,
    "readout_transposed": m_readout_transposed,
    "softmax_over_columns": m_softmax_columns,
    "no_softmax_scale": m_no_scale,
    "scores_transposed": m_pv_transposed_keys,
    "read_after_update": lambda m: _layer_head_variant(m, read_after_update=True),
    "attend_across_frames": lambda m: _layer_head_variant(m, global_attention=True),
    "update_on_denoise": lambda m: _layer_head_variant(m, always_update=True),
    "alpha_off_by_one": lambda m: _layer_head_variant(m, alpha_index_shift=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    m = fresh_oracle()
    MUTANTS[name](m)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(m)
        except Exception as e:  # noqa: BLE001 - any failure (assert or shape error) is a catch
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    m = fresh_oracle()
    for check in ALL_CHECKS:
        check(m)
