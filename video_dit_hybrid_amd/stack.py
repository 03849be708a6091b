"""A stack of attention layers for streaming video generation, for timing and
memory: each layer is either the hybrid layer (a fixed-size state per stream
and head) or the softmax teacher with a full KV cache (keys and values of every
generated frame). ARL2 ("Attend Locally, Remember Linearly") replaces part of
the 30 attention layers of its 1.3B model (50 % or 75 %, section 4) and keeps
softmax attention in the others; its memory and wall-clock claims are about
such a mixed stack.

Which layers are replaced comes from a learned per-layer score in the pages
(section 2.3, stage 1); without trained weights the stack spreads the hybrid
layers evenly (layer_kinds). There are no projection weights either, so every
layer of a pass reads the same q, k, v (and q', k', v', alpha, beta): the work
of each layer is that of a real layer of this shape, the values are not.

Optionally every hybrid layer weights its two branches (mix_weights): LinVideo
trains a per-layer r with o = r SoftmaxAttn + (1 - r) LinearAttn, SALAD scales
the linear branch by a sigmoid s computed from the input and the timestep. A
layer's weights are one fp32 [B, H, 2] tensor of (w_softmax, w_inter) per
(stream, head); without trained models they are synthetic.

All the arithmetic runs in the HIP library through the C ABI (api.py); this
module only owns the per-layer buffers and the call order.
"""
from __future__ import annotations

from . import api


def layer_kinds(n_layers: int, hybrid_fraction: float) -> list[str]:
    """'hybrid' or 'softmax' per layer: round(fraction * n_layers) hybrid
    layers (halves rounded up), spread evenly: layer i is hybrid when
    floor((i + 1) * n_h / n_layers) > floor(i * n_h / n_layers)."""
    if not 0.0 <= hybrid_fraction <= 1.0:
        raise ValueError("hybrid_fraction must be in [0, 1]")
    n_h = int(hybrid_fraction * n_layers + 0.5)
    return ["hybrid" if (i + 1) * n_h // n_layers > i * n_h // n_layers else "softmax" for i in range(n_layers)]


class AttentionStack:
    """Per-layer states (hybrid layers) and KV caches (softmax layers) for B
    streams of frames of frame_len tokens, H heads of size d, up to max_frames
    frames. run_frame(n, passes) runs one frame's passes (denoising passes,
    then the clean pass, the last of `passes`) through every layer."""

    def __init__(self, kinds, B, H, d, frame_len, max_frames, device="cuda", mix_weights=None):
        """mix_weights: None (hybrid layers output the plain sum of the two
        branches) or one fp32 [B, H, 2] tensor per layer (entries of softmax
        layers are ignored): (w_softmax, w_inter) for hybrid_attn_forward_mix."""
        import torch
        self.kinds = list(kinds)
        if mix_weights is not None and len(mix_weights) != len(self.kinds):
            raise ValueError("mix_weights needs one entry per layer")
        self.mix = list(mix_weights) if mix_weights is not None else [None] * len(self.kinds)
        self.B, self.H, self.d, self.L, self.max_frames = B, H, d, frame_len, max_frames
        self.states, self.caches = [], []
        for kind in self.kinds:
            if kind == "hybrid":
                self.states.append(torch.zeros((B, H, d, d), dtype=torch.float32, device=device))
                self.caches.append(None)
            elif kind == "softmax":
                shape = (B, max_frames * frame_len, H, d)
                self.states.append(None)
                self.caches.append((torch.empty(shape, dtype=torch.bfloat16, device=device),
                                    torch.empty(shape, dtype=torch.bfloat16, device=device)))
            else:
                raise ValueError(f"unknown layer kind {kind!r}")
        hws = api.workspace_bytes(B, H, frame_len, frame_len, d, 1)
        kws = api.kvcache_workspace_bytes(B, H, frame_len, frame_len, d, max_frames - 1)
        self.hws = torch.empty(max(hws, 1), dtype=torch.uint8, device=device)
        self.kws = torch.empty(max(kws, 1), dtype=torch.uint8, device=device)

    def run_frame(self, n: int, passes, out):
        """Frame n (0-based): every pass through every layer, in pass order;
        hybrid layers write their state on the clean (last) pass only, softmax
        layers append the pass's K, V at frame n (the clean pass's stay)."""
        if not 0 <= n < self.max_frames:
            raise ValueError(f"frame {n} outside the stack's {self.max_frames} frames")
        last = len(passes) - 1
        for p, t in enumerate(passes):
            clean = p == last
            for kind, st, cache, mix in zip(self.kinds, self.states, self.caches, self.mix):
                if kind == "hybrid":
                    upd = (t["kp"], t["vp"], t["alpha"], t["beta"]) if clean else (None, None, None, None)
                    if mix is None:
                        api.hybrid_attn_forward(t["q"], t["k"], t["v"], t["qp"], *upd, st, self.L, int(clean),
                                                out=out, workspace=self.hws)
                    else:
                        api.hybrid_attn_forward_mix(t["q"], t["k"], t["v"], t["qp"], *upd, st, self.L, int(clean),
                                                    mix, out=out, workspace=self.hws)
                else:
                    api.hybrid_attn_kvcache_forward(t["q"], t["k"], t["v"], cache[0], cache[1], self.L, n, out=out,
                                                    workspace=self.kws)
        return out

    def state_bytes(self) -> int:
        """Bytes of the hybrid layers' states (constant in the frame count)."""
        return sum(s.numel() * 4 for s in self.states if s is not None)

    def cache_bytes(self, frames: int) -> int:
        """Bytes of the softmax layers' KV caches once `frames` frames are in
        them (linear in the frame count)."""
        n_soft = sum(1 for c in self.caches if c is not None)
        return n_soft * 2 * self.B * frames * self.L * self.H * self.d * 2
