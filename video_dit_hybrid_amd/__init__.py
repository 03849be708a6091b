"""MI355X (gfx950) hybrid attention layer: intra-frame softmax + inter-frame gated-delta state.

The compute path is the HIP library ``libhybrid_attn.so`` behind a C ABI
(``include/hybrid_attn.h``); ``video_dit_hybrid_amd.api`` is a thin ctypes
binding over it. Importing this package does not load the library; the first
call into ``api`` does, and fails loudly if it is not built.
"""
__all__ = ["api", "workloads"]
