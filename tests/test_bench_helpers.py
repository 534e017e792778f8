"""CPU checks of the benchmark's own arithmetic: the counted FLOP it divides
by, on whole-tile and padded latents, against counts made from the oracle's
window mask and padding mask."""
import os
import sys

import numpy as np
import pytest

import oracle as O

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("latent,tile,wins", [
    ((6, 16, 16), (2, 4, 4), [(3, 3, 3), (1, 2, 5)]),
    ((5, 15, 13), (2, 4, 4), [(3, 1, 3), (2, 2, 2)]),     # padded to (6, 16, 16)
    ((3, 5, 6), (2, 2, 4), [(9, 9, 9)]),                  # padded, full window
])
def test_counted_flops_match_mask_counts(latent, tile, wins):
    D, B = 8, 2
    grid = O.padded_latent(latent, tile)
    valid = O.valid_positions(latent, tile)
    padded = real = 0
    for w in wins:
        m = O.window_mask(grid, tile, w)
        padded += int(m.sum())
        real += int((m & valid[:, None] & valid[None, :]).sum())
    assert bench.fwd_flops(latent, tile, wins, B, D) == B * 4 * D * padded
    assert bench.real_token_flops(latent, tile, wins, B, D) == B * 4 * D * real


def test_headline_count():
    # (30,48,80), tile (6,8,8), 24 heads of (3,3,3): 194,400 pairs of 384 x 384 x 128
    f = bench.fwd_flops((30, 48, 80), (6, 8, 8), [(3, 3, 3)] * 24, 1, 128)
    assert f == 24 * 300 * 27 * 4 * 384 * 384 * 128 == 14676708556800
    assert bench.real_token_flops((30, 48, 80), (6, 8, 8), [(3, 3, 3)] * 24, 1, 128) == f
