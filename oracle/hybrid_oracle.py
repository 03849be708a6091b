"""Plain fp64 CPU oracle of the ARL2 hybrid attention layer.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import this module. The product path never calls
it and shares no code with it (it does not import the GPU package; it takes
float64 numpy arrays and nothing else).

Source: "Attend Locally, Remember Linearly" (ARL2, arXiv 2605.16579; the
gist.science technical summary), section 2.1 (hybrid attention decomposition)
and section 2.2 (state management). What the layer computes, per stream b and
head h, for frame N with rows r = [N*L, (N+1)*L):

  intra-frame branch (2.1, item 1): bidirectional softmax attention among the
      tokens of frame N only, with the frozen Q, K, V;
  inter-frame branch (2.1, "outputs"): O_inter = Q'_N S_{N-1};
  state update (2.1, gated update rule):
      S_N = alpha_N S_{N-1} + K'_N^T diag(beta_N) (V'_N - K'_N S_{N-1});
  frame-level access (2.2): every token of frame N reads the same S_{N-1};
      S is written only after the whole frame;
  clean-pass updates (2.2): denoising passes read S and never write it; only
      the clean pass writes it (update_state = 1).

Readings where the page is silent or garbled:
  * the printed update rule has no transpose and no diag; the only
    dimensionally valid reading is K'^T diag(beta) (V' - K' S_{N-1}), with the
    residual taken against the undecayed S_{N-1} exactly as printed;
  * alpha is one scalar per (stream, frame, head); beta one scalar per
    (stream, token, head);
  * the branches combine by a plain sum, O = O_intra + O_inter;
  * the softmax scale is 1/sqrt(d) unless given; no mask inside a frame;
  * with update_state = 0 every frame reads the input state.
  * the feature maps phi_q, phi_k, phi_v (2.1, "adaptation": grouped per-head
    1x1 maps) are one d x d linear map per head, no bias, no nonlinearity,
    applied to the inter-frame branch's inputs only;
  * K' may be L2-normalised per (token, head) after its map (a flag; the page
    names no normalisation; a zero row stays zero);
  * the gates (2.1: alpha the forget gate, beta the step size, learned
    per-token projections; ablations: headwise gating) are one projection per
    head of the token's input x [C channels] plus a bias, through a sigmoid;
    the frame's alpha_N is the mean of its tokens' alpha gates (one write per
    frame), and beta_t is the token's gate divided by the frame length L.

The softmax teacher the hybrid layer replaces (ARL2 section 1: chunk-wise
causal attention with a KV cache that grows with every generated chunk;
section 4: the baselines' memory and time grow with video length) is here too
(chunk_causal_attention): the queries of frame N attend to the keys of frames
0..N, bidirectionally inside frame N.

The token-level access variant (ARL2 section 4 ablations: token-level
instead of frame-level access degrades quality; it is the canonical,
per-token gated delta rule) is here as hybrid_layer_token_level: every token
reads the state left by all earlier tokens, and every token of a clean pass
writes it; the frame's forget gate applies once, at its first token.

A per-branch output weight (hybrid_layer_mixed) covers the mixtures of
softmax and linear branches that the LinVideo and SALAD pages describe.

Every function here is pinned by tests/test_oracle_pins.py against
properties the page and the mathematics fix (row sums, closed forms, the
delta-rule recall property, brute force on tiny inputs, textbook attention).
"""
from __future__ import annotations

import math

import numpy as np


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row-wise softmax of a 2-D fp64 array: exp(z - max) / sum (2.1, item 1)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def intra_frame_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          scale: float | None = None) -> np.ndarray:
    """Bidirectional softmax attention among the L tokens of one frame.

    q, k: [L, d_k], v: [L, d_v] fp64. Returns softmax(q k^T * scale) v, [L, d_v].
    ARL2 section 2.1 item 1 (the branch keeps the pretrained softmax attention
    inside each frame, no causal mask).
    """
    d = q.shape[1]
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    p = softmax_rows((q @ k.T) * s)
    return p @ v


def inter_frame_readout(qp: np.ndarray, state: np.ndarray) -> np.ndarray:
    """O_inter = Q'_N S_{N-1}; qp [L, d_k], state [d_k, d_v]. ARL2 2.1 outputs."""
    return qp @ state


def delta_update(state: np.ndarray, kp: np.ndarray, vp: np.ndarray,
                 alpha: float, beta: np.ndarray) -> np.ndarray:
    """One gated-delta write of the state after a clean frame (ARL2 2.1).

    S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}).
    state [d_k, d_v], kp [L, d_k], vp [L, d_v], beta [L], alpha scalar.
    """
    resid = vp - kp @ state
    return alpha * state + kp.T @ (beta[:, None] * resid)


def hybrid_layer_head(q, k, v, qp, kp, vp, alpha, beta, state, frame_len,
                      update_state, scale=None, frames=None):
    """The layer for one (stream, head): all frames in order.

    q..vp: [T, d] fp64; alpha: [F]; beta: [T]; state: [d_k, d_v].
    frames: optional set of frame indices whose output is wanted (others are
    returned as NaN); the state chain always runs over every frame.
    Returns (out [T, d_v], state_after [d_k, d_v]).
    Frame N reads S_{N-1} (section 2.2, frame-level access); with
    update_state the state advances after each frame, otherwise it is left
    as given (section 2.2, clean-pass updates).
    """
    T = q.shape[0]
    L = int(frame_len)
    F = T // L
    S = np.array(state, dtype=np.float64, copy=True)
    out = np.full((T, v.shape[1]), np.nan)
    for n in range(F):
        r = slice(n * L, (n + 1) * L)
        if frames is None or n in frames:
            out[r] = intra_frame_attention(q[r], k[r], v[r], scale) + inter_frame_readout(qp[r], S)
        if update_state:
            S = delta_update(S, kp[r], vp[r], float(alpha[n]), beta[r])
    return out, S


def hybrid_layer(q, k, v, qp, kp, vp, alpha, beta, state, frame_len,
                 update_state, scale=None):
    """The whole layer call, all streams and heads.

    q..vp: [B, T, H, d] fp64; alpha: [B, F, H]; beta: [B, T, H];
    state: [B, H, d_k, d_v]. Returns (out [B, T, H, d_v], state_out).
    state_out equals state when update_state is 0.
    """
    B, T, H, _ = q.shape
    out = np.empty((B, T, H, v.shape[3]), dtype=np.float64)
    st = np.array(state, dtype=np.float64, copy=True)
    for b in range(B):
        for h in range(H):
            a = alpha[b, :, h] if alpha is not None else None
            bt = beta[b, :, h] if beta is not None else None
            kk = kp[b, :, h] if kp is not None else None
            vv = vp[b, :, h] if vp is not None else None
            out[b, :, h], st[b, h] = hybrid_layer_head(
                q[b, :, h], k[b, :, h], v[b, :, h], qp[b, :, h], kk, vv, a, bt,
                st[b, h], frame_len, update_state, scale)
    return out, st


def hybrid_layer_mixed(q, k, v, qp, kp, vp, alpha, beta, state, frame_len,
                       update_state, mix, scale=None):
    """The layer with a weight on each branch's output:
        O = w_softmax * O_intra + w_inter * O_inter,
    mix [B, H, 2] = (w_softmax, w_inter) per (stream, head), the same for every
    frame of the call. This covers the mixtures the pages describe for
    swapping softmax layers to linear ones: LinVideo's selective transfer,
    o = r SoftmaxAttn + (1 - r) LinearAttn with a learned r in [0, 1] per
    layer (weights (r, 1 - r)), and SALAD's input- and timestep-dependent
    scale s in (0, 1) on the linear branch (weights (1, s)). The weights touch
    the output only; the state recursion is that of hybrid_layer.
    Returns (out [B, T, H, d_v], state_out).
    """
    B, T, H, _ = q.shape
    L = int(frame_len)
    F = T // L
    out = np.empty((B, T, H, v.shape[3]), dtype=np.float64)
    st = np.array(state, dtype=np.float64, copy=True)
    for b in range(B):
        for h in range(H):
            w_soft, w_inter = float(mix[b, h, 0]), float(mix[b, h, 1])
            S = st[b, h]
            for n in range(F):
                r = slice(n * L, (n + 1) * L)
                o_intra = intra_frame_attention(q[b, r, h], k[b, r, h], v[b, r, h], scale)
                o_inter = inter_frame_readout(qp[b, r, h], S)
                out[b, r, h] = w_soft * o_intra + w_inter * o_inter
                if update_state:
                    S = delta_update(S, kp[b, r, h], vp[b, r, h], float(alpha[b, n, h]), beta[b, r, h])
            st[b, h] = S
    return out, st


def state_chain(kp, vp, alpha, beta, state, frame_len):
    """Only the state recursion for one (stream, head): S after every frame.

    kp, vp: [T, d]; alpha: [F]; beta: [T]; state: [d, d].
    Returns the list [S_0 (input), S_1, ..., S_F]. ARL2 2.1 update rule.
    """
    L = int(frame_len)
    F = kp.shape[0] // L
    S = np.array(state, dtype=np.float64, copy=True)
    chain = [S]
    for n in range(F):
        r = slice(n * L, (n + 1) * L)
        S = delta_update(S, kp[r], vp[r], float(alpha[n]), beta[r])
        chain.append(S)
    return chain


def feature_maps(q, k, v, wq, wk, wv, normalize_k=False):
    """The grouped per-head 1x1 feature maps of the inter-frame branch
    (ARL2 2.1, "adaptation": phi_q, phi_k, phi_v adapt the frozen projections'
    Q, K, V to the linear recurrence). Read here as one d x d linear map per
    head over that head's channels, no bias and no nonlinearity (a 1x1
    convolution grouped by head):
        Q'[b, t, h, :] = Q[b, t, h, :] @ wq[h]   (likewise K' with wk, V' with wv)
    q, k, v: [B, T, H, d] fp64; wq, wk, wv: [H, d, d] fp64.
    With normalize_k, each row K'[b, t, h, :] is then divided by its L2 norm
    (l2_normalize_rows).
    Returns (qp, kp, vp), each [B, T, H, d].
    """
    maps = []
    for x, w in ((q, wq), (k, wk), (v, wv)):
        y = np.empty_like(x, dtype=np.float64)
        for h in range(x.shape[2]):
            y[:, :, h, :] = x[:, :, h, :] @ w[h]
        maps.append(y)
    if normalize_k:
        maps[1] = l2_normalize_rows(maps[1])
    return tuple(maps)


def l2_normalize_rows(x, eps=1e-12):
    """x / max(||x||_2, eps) over the last axis (one key vector per token and
    head); a zero row stays zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def sigmoid(z):
    """1 / (1 + exp(-z)), fp64."""
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def gate_projections(x, w_gate, b_gate, frame_len):
    """The forget gate alpha and step size beta from the layer input (ARL2
    2.1: learned per-token projections; headwise gating).

    x: [B, T, C] fp64 (the tokens' input to the layer); w_gate: [2, H, C]
    (row 0: alpha projections, row 1: beta projections, one per head);
    b_gate: [2, H]. Per token t and head h:
        a_t = sigmoid(x_t . w_gate[0, h] + b_gate[0, h])
        g_t = sigmoid(x_t . w_gate[1, h] + b_gate[1, h])
    alpha[b, N, h] = mean of a_t over the L tokens of frame N (the state is
    written once per frame); beta[b, t, h] = g_t / L.
    Returns (alpha [B, F, H], beta [B, T, H]).
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    L = int(frame_len)
    F = T // L
    a = sigmoid(x @ np.asarray(w_gate[0], dtype=np.float64).T + np.asarray(b_gate[0], dtype=np.float64))
    g = sigmoid(x @ np.asarray(w_gate[1], dtype=np.float64).T + np.asarray(b_gate[1], dtype=np.float64))
    alpha = a.reshape(B, F, L, -1).mean(axis=2)
    beta = g / L
    return alpha, beta


def hybrid_layer_fmap(q, k, v, wq, wk, wv, alpha, beta, state, frame_len,
                      update_state, scale=None):
    """The layer with the feature maps applied in front of the inter-frame
    branch (ARL2 2.1): Q', K', V' = phi(Q, K, V), then hybrid_layer. The
    intra-frame branch keeps the unmapped Q, K, V (2.1 item 1: the frozen
    projections). Returns (out, state_out) as hybrid_layer."""
    qp, kp, vp = feature_maps(q, k, v, wq, wk, wv)
    return hybrid_layer(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, scale)


def hybrid_layer_gated(x, q, k, v, wq, wk, wv, w_gate, b_gate, state, frame_len,
                       update_state, normalize_k=True, scale=None):
    """The layer from its inputs as a transformer block holds them: the gates
    from x (gate_projections), the feature maps (feature_maps, K' optionally
    L2-normalised), then hybrid_layer. Returns (out, state_out, alpha, beta)."""
    alpha, beta = gate_projections(x, w_gate, b_gate, frame_len)
    qp, kp, vp = feature_maps(q, k, v, wq, wk, wv, normalize_k)
    out, st = hybrid_layer(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, scale)
    return out, st, alpha, beta


def chunk_causal_attention(q, k, v, frame_len, scale=None):
    """Softmax attention with a full KV cache, one head (the teacher of ARL2
    section 1: chunk-wise causal generation, every chunk attending to the keys
    and values of all chunks generated so far and to its own).

    q, k, v: [T, d] fp64, T = F * L. Frame N's queries (rows [N L, (N+1) L))
    attend to keys [0, (N+1) L): no mask inside the frame, none of the later
    frames. Returns [T, d].
    """
    T = q.shape[0]
    L = int(frame_len)
    out = np.empty((T, v.shape[1]), dtype=np.float64)
    for n in range(T // L):
        r = slice(n * L, (n + 1) * L)
        vis = slice(0, (n + 1) * L)
        out[r] = intra_frame_attention(q[r], k[vis], v[vis], scale)
    return out


def hybrid_layer_token_level(q, k, v, qp, kp, vp, alpha, beta, state, frame_len, update_state, scale=None):
    """The layer with token-level access (the ablated alternative to ARL2
    2.2's frame-level access), one (stream, head): tokens in order, token t of
    frame N reads S_{t-1}, the state after every earlier token, then
        S_t = a_t S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1}),
    a_t = alpha_N for the first token of frame N and 1 for the others (the
    frame's decay applied once, the residual against the undecayed state as in
    the frame-level rule). out = intra-frame softmax (unchanged) + q'_t S_{t-1}.
    With update_state = 0 the per-token states are still what the tokens read
    (the pass's own tokens update a transient copy) and the input state is
    returned unchanged.

    q..vp: [T, d]; alpha: [F]; beta: [T]; state: [d, d]. Returns (out, state).
    """
    T, d = q.shape
    L = int(frame_len)
    S = np.array(state, dtype=np.float64, copy=True)
    out = np.empty((T, vp.shape[1]), dtype=np.float64)
    for n in range(T // L):
        r = slice(n * L, (n + 1) * L)
        out[r] = intra_frame_attention(q[r], k[r], v[r], scale)
    for t in range(T):
        out[t] += qp[t] @ S
        a = float(alpha[t // L]) if t % L == 0 else 1.0
        S = a * S + float(beta[t]) * np.outer(kp[t], vp[t] - kp[t] @ S)
    return out, (S if update_state else np.array(state, dtype=np.float64, copy=True))
