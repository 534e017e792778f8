"""Seeded random small configurations through the C-ABI against the fp64 oracle.

The fixed cases elsewhere pick shapes by hand; these draw the tile (t in 1..3,
h and w in {4, 8}, L a multiple of 32), the tile grid, an optional padding
of each dimension, head dim, batch, heads and one window per head (possibly
larger than the grid, so clamped) from a fixed seed, and check the bf16
forward (tile-major, and raster order where that instance applies) and the
backward to the same tolerance as the fixed cases.
"""
import numpy as np
import pytest

import oracle as O
from _helpers import err_report, to64
from sparse_sliding_tile_amd import inputs as I

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
BF16_REL_RMS = 1e-2
MAX_TOKENS = 3072      # tile-major rows per sequence, so the oracle stays quick
MAX_SEQS = 4           # batch x heads


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        tile = (int(rng.integers(1, 4)), int(rng.choice([4, 8])), int(rng.choice([4, 8])))
        L = tile[0] * tile[1] * tile[2]
        if L % 32:
            continue
        grid = (int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 5)))
        if L * grid[0] * grid[1] * grid[2] > MAX_TOKENS:
            continue
        padded = bool(rng.random() < 0.5)
        # padding keeps the grid: drop fewer than a tile's worth of tokens
        latent = tuple(g * s - (int(rng.integers(0, s)) if padded else 0) for g, s in zip(grid, tile))
        B, Hh = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        if B * Hh > MAX_SEQS:
            continue
        D = int(rng.choice([64, 128]))
        wins = [tuple(int(rng.integers(1, g + 2)) for g in grid) for _ in range(Hh)]
        cases.append((latent, tile, B, wins, D))
    return cases


FWD_CASES = _draw(32, seed=2024)
BWD_CASES = _draw(16, seed=77)


@pytest.fixture(scope="module")
def sta():
    import sparse_sliding_tile_amd as s
    s.lib()
    return s


def _tm(sta, t, latent, tile):
    return sta.tile_reorder(t.to("cuda").contiguous(), latent, tile)


@pytest.mark.parametrize("latent,tile,B,wins,D", FWD_CASES)
def test_random_forward(sta, latent, tile, B, wins, D):
    print("case", latent, tile, B, wins, D, flush=True)
    S = int(np.prod(latent))
    x = I.make_inputs(B, len(wins), S, D, "bf16", seed=11)
    scale = D ** -0.5
    q, k, v = (_tm(sta, x[n], latent, tile) for n in ("q", "k", "v"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    rq, rk, rv = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v"))
    ro, rl = O.forward(rq, rk, rv, latent, tile, wins, scale)
    eo, el = err_report(to64(o), ro), err_report(to64(lse), rl)
    print("O", eo, "LSE", el)
    assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
    assert el["max_abs"] < BF16_TOL
    # raster order: whole-tile latents with a tile width that fills the copy segments
    whole = all(a % t == 0 for a, t in zip(latent, tile))
    if whole and tile[2] % (512 // D) == 0:
        qr, kr, vr = (x[n].to("cuda").contiguous() for n in ("q", "k", "v"))
        orr, lr = sta.forward_raster(qr, kr, vr, latent, tile, wins, scale=scale)
        er = err_report(to64(orr), O.unreorder(ro, latent, tile))
        elr = err_report(to64(lr)[..., None], O.unreorder(rl[..., None], latent, tile))
        print("raster O", er, "LSE", elr)
        assert er["max_abs"] < BF16_TOL and er["rel_rms"] < BF16_REL_RMS
        assert elr["max_abs"] < BF16_TOL


@pytest.mark.parametrize("latent,tile,B,wins,D", BWD_CASES)
def test_random_backward(sta, latent, tile, B, wins, D):
    print("case", latent, tile, B, wins, D, flush=True)
    S = int(np.prod(latent))
    x = I.make_inputs(B, len(wins), S, D, "bf16", seed=13, with_do=True)
    scale = D ** -0.5
    q, k, v, do = (_tm(sta, x[n], latent, tile) for n in ("q", "k", "v", "do"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=scale)
    ref = O.backward(*(O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v", "do")),
                     latent, tile, wins, scale)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e = err_report(to64(got), r)
        print(name, e)
        assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS, name
