"""Layer assignment of the attention stack (CPU)."""
import pytest

from video_dit_hybrid_amd.stack import layer_kinds


def test_layer_kinds_counts_and_spread():
    k = layer_kinds(30, 0.5)
    assert k.count("hybrid") == 15 and all((x == "hybrid") == (i % 2 == 1) for i, x in enumerate(k))
    k = layer_kinds(30, 0.75)
    assert k.count("hybrid") == 23
    # evenly spread: no run of more than two hybrid layers between softmax ones... and never two softmax in a row
    assert "softmax,softmax" not in ",".join(k)
    assert layer_kinds(30, 0.0) == ["softmax"] * 30 and layer_kinds(30, 1.0) == ["hybrid"] * 30
    assert layer_kinds(4, 0.5) == ["softmax", "hybrid", "softmax", "hybrid"]
    with pytest.raises(ValueError):
        layer_kinds(30, 1.5)
