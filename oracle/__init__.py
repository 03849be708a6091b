"""fp64 CPU oracle of the ARL2 hybrid attention layer (test infrastructure only)."""
from .hybrid_oracle import (  # noqa: F401
    softmax_rows, intra_frame_attention, inter_frame_readout, delta_update,
    hybrid_layer_head, hybrid_layer, state_chain,
)
