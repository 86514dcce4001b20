"""The attention block's argument checks, on the CPU (no kernel runs)."""
import pytest


def test_block_head_dimensions():
    torch = pytest.importorskip("torch")
    from linear_lsh_sketch_amd import mha
    for hd in (32, 64, 128):
        blk = mha.RaceMHA(2 * hd, head_dim=hd)
        assert blk.heads == 2 and tuple(blk.planes.shape) == (16, 4, hd)
        x = torch.zeros(1, 3, 2 * hd)
        assert tuple(blk.split(x).shape) == (1, 2, 3, hd)
    with pytest.raises(ValueError):
        mha.RaceMHA(96, head_dim=48)      # head dimensions other than 32, 64, 128
    with pytest.raises(ValueError):
        mha.RaceMHA(100, head_dim=64)     # d_model not a multiple of the head dimension
