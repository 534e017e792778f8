"""Pins for the CPU oracle: brute force, closed forms, invariants and library
routines that fix what Sliding Tile Attention computes, so that the oracle is
not trusted on its own say-so.  CPU only."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O


# ---------------------------------------------------------------- reorder / pi

def _pi_by_enumeration(latent, tile):
    """Tile-major order written as an enumeration: walk tiles in raster order
    over the tile grid and, inside each, tokens in raster order; hand out
    consecutive sequence positions."""
    T, H, W = latent
    t, h, w = tile
    pi = np.full(T * H * W, -1, dtype=np.int64)
    pos = 0
    for a0, a1, a2 in itertools.product(range(T // t), range(H // h), range(W // w)):
        for i0, i1, i2 in itertools.product(range(t), range(h), range(w)):
            r = ((a0 * t + i0) * H + (a1 * h + i1)) * W + (a2 * w + i2)
            pi[r] = pos
            pos += 1
    return pi


SHAPES = [((6, 16, 16), (2, 4, 4)), ((4, 8, 8), (2, 4, 4)), ((5, 6, 10), (5, 3, 2)),
          ((1, 8, 16), (1, 8, 8)), ((3, 4, 5), (1, 1, 1)), ((3, 4, 5), (3, 4, 5)),
          ((30, 48, 80), (6, 8, 8))]


@pytest.mark.parametrize("latent,tile", SHAPES)
def test_pi_matches_enumeration(latent, tile):
    assert np.array_equal(O.tile_major_index(latent, tile), _pi_by_enumeration(latent, tile))


@pytest.mark.parametrize("latent,tile", SHAPES)
def test_pi_is_bijection_and_roundtrip_exact(latent, tile):
    S = int(np.prod(latent))
    pi = O.tile_major_index(latent, tile)
    assert np.array_equal(np.sort(pi), np.arange(S))
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, S, 4)).astype(np.float32)
    y = O.reorder(x, latent, tile)
    assert np.array_equal(O.unreorder(y, latent, tile), x)
    assert not np.array_equal(y, x) or np.array_equal(pi, np.arange(S))


@pytest.mark.parametrize("latent,tile", SHAPES[:5])
def test_reorder_matches_reshape_transpose(latent, tile):
    """Tile-major as a 6-D reshape/transpose of the (T,H,W) volume."""
    T, H, W = latent
    t, h, w = tile
    x = np.arange(T * H * W * 2, dtype=np.float64).reshape(T * H * W, 2)
    ref = (x.reshape(T // t, t, H // h, h, W // w, w, 2)
           .transpose(0, 2, 4, 1, 3, 5, 6).reshape(-1, 2))
    assert np.array_equal(O.reorder(x, latent, tile), ref)


def test_non_tile_multiple_rejected():
    with pytest.raises(ValueError):
        O.tile_grid((29, 45, 76), (6, 8, 8))
    with pytest.raises(ValueError):
        O.window_start(0, 0, 4)


# ---------------------------------------------------------------- windows

@pytest.mark.parametrize("n,w,starts", [
    (4, 3, [0, 0, 1, 1]),
    (6, 3, [0, 0, 1, 2, 3, 3]),
    (10, 5, [0, 0, 0, 1, 2, 3, 4, 5, 5, 5]),
    (5, 1, [0, 1, 2, 3, 4]),
    (3, 7, [0, 0, 0]),
    (6, 6, [0, 0, 0, 0, 0, 0]),
    (5, 2, [0, 0, 1, 2, 3]),   # even window: extra tile on the low side
])
def test_window_start_worked_sequences(n, w, starts):
    assert [O.window_start(q, w, n)[0] for q in range(n)] == starts


@pytest.mark.parametrize("n,w,counts", [(10, 5, [3, 4, 5, 6, 7, 7, 6, 5, 4, 3]),
                                        (4, 3, [2, 4, 4, 2]),
                                        (8, 5, [3, 4, 5, 8, 8, 5, 4, 3])])
def test_transposed_window_counts(n, w, counts):
    got = [sum(1 for q in range(n) if O.window_contains((q, 0, 0), (k, 0, 0), (w, 1, 1), (n, 1, 1)))
           for k in range(n)]
    assert got == counts


def _window_by_sliding(q, w, n):
    """Second formulation: put the window around q (floor(w'/2) tiles below),
    then slide it back inside the grid by however far it overflows."""
    wp = min(w, n)
    lo = q - wp // 2
    hi = lo + wp - 1
    if lo < 0:
        lo, hi = 0, hi - lo
    if hi > n - 1:
        lo, hi = lo - (hi - (n - 1)), n - 1
    return set(range(lo, hi + 1))


def test_window_matches_sliding_formulation():
    for n in range(1, 13):
        for w in range(1, 15):
            for q in range(n):
                s, wp = O.window_start(q, w, n)
                assert set(range(s, s + wp)) == _window_by_sliding(q, w, n)


def test_odd_window_is_symmetric_in_interior():
    for n in range(1, 14):
        for w in range(1, n + 1, 2):
            r = w // 2
            for q in range(r, n - r):
                s, wp = O.window_start(q, w, n)
                assert (s, s + wp - 1) == (q - r, q + r)


PAIR_CASES = [((6, 16, 16), (2, 4, 4), [(3, 3, 3), (1, 2, 5)]),
              ((30, 48, 80), (6, 8, 8), [(3, 3, 3), (5, 6, 10), (1, 6, 10), (3, 3, 5), (5, 3, 3)]),
              ((24, 64, 64), (6, 8, 8), [(3, 5, 5)]),
              ((4, 8, 8), (2, 4, 4), [(9, 9, 9), (1, 1, 1)])]


@pytest.mark.parametrize("latent,tile,wins", PAIR_CASES)
def test_pair_count_invariant_and_own_tile(latent, tile, wins):
    n, _ = O.tile_grid(latent, tile)
    pairs, off = O.tile_pairs(latent, tile, wins)
    nt = int(np.prod(n))
    for h, win in enumerate(wins):
        kh = int(np.prod([min(a, b) for a, b in zip(win, n)]))
        p = pairs[off[h]:off[h + 1]]
        assert p.shape[0] == nt * kh
        counts = np.bincount(p[:, 0], minlength=nt)
        assert np.all(counts == kh)
        own = {(a, a) for a in range(nt)}
        assert own <= {tuple(x) for x in p}
        # canonical order: query tile, then key tile, increasing
        key = p[:, 0].astype(np.int64) * nt + p[:, 1]
        assert np.all(np.diff(key) > 0)
        if all(a >= b for a, b in zip(win, n)):
            assert p.shape[0] == nt * nt


@pytest.mark.parametrize("latent,tile,wins", PAIR_CASES[:1] + PAIR_CASES[2:])
def test_transposed_pairs_same_set(latent, tile, wins):
    n, _ = O.tile_grid(latent, tile)
    nt = int(np.prod(n))
    f, fo = O.tile_pairs(latent, tile, wins)
    t, to = O.tile_pairs(latent, tile, wins, transpose=True)
    assert np.array_equal(fo, to)
    for h in range(len(wins)):
        a, b = f[fo[h]:fo[h + 1]], t[to[h]:to[h + 1]]
        assert {tuple(x) for x in a} == {tuple(x) for x in b}
        key = b[:, 1].astype(np.int64) * nt + b[:, 0]
        assert np.all(np.diff(key) > 0)


def test_mask_blocks_are_whole_tiles():
    latent, tile = (6, 16, 16), (2, 4, 4)
    _, L = O.tile_grid(latent, tile)
    m = O.window_mask(latent, tile, (3, 1, 3))
    blocks = m.reshape(m.shape[0] // L, L, m.shape[1] // L, L)
    assert np.all(blocks.all(axis=(1, 3)) == blocks.any(axis=(1, 3)))


# ---------------------------------------------------------------- forward

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute_force_raster(q, k, v, latent, tile, wins, scale):
    """Per-token softmax in raster order with scalar loops and math.exp."""
    T, H, W = latent
    t, h, w = tile
    n = (T // t, H // h, W // w)
    B, Hh, S, D = q.shape
    coords = [(tau, y, x) for tau in range(T) for y in range(H) for x in range(W)]
    tc = [(tau // t, y // h, x // w) for tau, y, x in coords]
    out = np.zeros_like(q)
    lse = np.zeros((B, Hh, S))
    for hh in range(Hh):
        wins_d = [[_window_by_sliding(qq, wins[hh][d], n[d]) for qq in range(n[d])] for d in range(3)]
        for b in range(B):
            for i in range(S):
                vis = [j for j in range(S) if all(tc[j][d] in wins_d[d][tc[i][d]] for d in range(3))]
                s = [scale * sum(q[b, hh, i, c] * k[b, hh, j, c] for c in range(D)) for j in vis]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                for c in range(D):
                    out[b, hh, i, c] = sum(e[a] * v[b, hh, j, c] for a, j in enumerate(vis)) / tot
                lse[b, hh, i] = mx + math.log(tot)
    return out, lse


def test_forward_matches_brute_force():
    latent, tile = (4, 8, 8), (2, 4, 4)     # tile grid 2x2x2, 256 tokens
    wins = [(1, 1, 1), (2, 1, 2), (9, 2, 1)]
    B, Hh, D, S = 2, 3, 6, 256
    q, k, v = (_rand((B, Hh, S, D), s) for s in (1, 2, 3))
    scale = 0.7
    ref_o, ref_l = _brute_force_raster(q, k, v, latent, tile, wins, scale)
    o, l = O.forward(q, k, v, latent, tile, wins, scale, order="raster")
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)
    # the same through the tile-major order
    qt, kt, vt = (O.reorder(a, latent, tile) for a in (q, k, v))
    o2, l2 = O.forward(qt, kt, vt, latent, tile, wins, scale)
    np.testing.assert_allclose(O.unreorder(o2, latent, tile), ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.unreorder(l2[..., None], latent, tile)[..., 0], ref_l, rtol=0, atol=1e-12)


def test_forward_brute_force_uneven_grid():
    latent, tile = (6, 8, 12), (2, 4, 4)    # tile grid 3x2x3, 576 tokens
    wins = [(2, 1, 2), (3, 3, 1)]
    q, k, v = (_rand((1, 2, 576, 4), s) for s in (4, 5, 6))
    ref_o, ref_l = _brute_force_raster(q, k, v, latent, tile, wins, 0.5)
    o, l = O.forward(q, k, v, latent, tile, wins, 0.5, order="raster")
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


def _sdpa(q, k, v, scale, mask=None):
    t = [torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m, scale=scale).numpy()


def test_full_window_equals_full_attention():
    latent, tile = (6, 16, 16), (2, 4, 4)
    q, k, v = (_rand((1, 2, 1536, 64), s) for s in (7, 8, 9))
    scale = 1 / 8
    o, l = O.forward(q, k, v, latent, tile, [(3, 4, 4), (99, 99, 99)], scale)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale), rtol=0, atol=1e-12)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    ref_lse = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    np.testing.assert_allclose(l, ref_lse, rtol=0, atol=1e-10)
    o2, l2 = O.dense_forward(q, k, v, scale)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l, rtol=0, atol=1e-12)


def test_unit_window_is_per_tile_attention():
    latent, tile = (6, 16, 16), (2, 4, 4)
    _, L = O.tile_grid(latent, tile)
    q, k, v = (_rand((1, 2, 1536, 16), s) for s in (10, 11, 12))
    o, _ = O.forward(q, k, v, latent, tile, [(1, 1, 1)] * 2, 0.3)
    for a in range(1536 // L):
        sl = slice(a * L, (a + 1) * L)
        np.testing.assert_allclose(o[:, :, sl], _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.3),
                                   rtol=0, atol=1e-12)


def test_zero_query_gives_window_mean_and_log_count():
    """Q = 0 makes every visible score 0: O_i is the plain mean of V over the
    window's K_h*L tokens and LSE_i = ln(K_h*L)."""
    latent, tile = (6, 16, 16), (2, 4, 4)
    n, L = O.tile_grid(latent, tile)
    win = (3, 1, 2)
    v = _rand((1, 1, 1536, 5), 13)
    q = np.zeros_like(v)
    k = _rand(v.shape, 14)
    o, l = O.forward(q, k, v, latent, tile, [win], 0.125)
    kh = int(np.prod([min(a, b) for a, b in zip(win, n)]))
    coords = list(itertools.product(range(n[0]), range(n[1]), range(n[2])))
    vt = v[0, 0].reshape(len(coords), L, 5)
    for a, ca in enumerate(coords):
        sets = [_window_by_sliding(ca[d], win[d], n[d]) for d in range(3)]
        keys = [b for b, cb in enumerate(coords) if all(cb[d] in sets[d] for d in range(3))]
        assert len(keys) == kh
        ref = vt[keys].reshape(-1, 5).mean(axis=0)
        np.testing.assert_allclose(o[0, 0, a * L:(a + 1) * L], np.broadcast_to(ref, (L, 5)),
                                   rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.log(kh * L), rtol=0, atol=1e-12)


def test_constant_values_pass_through():
    latent, tile = (6, 16, 16), (2, 4, 4)
    q, k = _rand((1, 2, 1536, 8), 15), _rand((1, 2, 1536, 8), 16)
    c = _rand((1, 2, 1, 8), 17)
    v = np.broadcast_to(c, q.shape).copy()
    o, _ = O.forward(q, k, v, latent, tile, [(3, 3, 3), (1, 4, 2)], 0.125)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-12)


def test_forward_rows_subset():
    latent, tile = (6, 16, 16), (2, 4, 4)
    q, k, v = (_rand((2, 2, 1536, 8), s) for s in (18, 19, 20))
    wins = [(3, 3, 3), (1, 2, 4)]
    o, l = O.forward(q, k, v, latent, tile, wins, 0.3)
    rows = np.array([0, 31, 32, 700, 1535])
    o2, l2 = O.forward(q, k, v, latent, tile, wins, 0.3, rows=rows)
    np.testing.assert_allclose(o2, o[:, :, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l[:, :, rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- backward

def _autograd_ref(q, k, v, do, latent, tile, wins, scale):
    """Gradients by torch autograd through masked SDPA, float64 on the CPU."""
    qt, kt, vt = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    masks = torch.stack([torch.from_numpy(O.window_mask(latent, tile, w)) for w in wins])
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=masks[None], scale=scale)
    out.backward(torch.from_numpy(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_backward_matches_autograd():
    latent, tile = (6, 16, 16), (2, 4, 4)
    wins = [(3, 3, 3), (1, 2, 5)]
    q, k, v, do = (_rand((2, 2, 1536, 16), s) for s in (21, 22, 23, 24))
    got = O.backward(q, k, v, do, latent, tile, wins, 0.25)
    ref = _autograd_ref(q, k, v, do, latent, tile, wins, 0.25)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11)


def test_backward_finite_differences():
    latent, tile = (2, 4, 8), (1, 2, 4)      # 64 tokens, grid 2x2x2
    wins = [(1, 2, 1)]
    q, k, v, do = (_rand((1, 1, 64, 3), s) for s in (25, 26, 27, 28))
    scale = 0.9
    dq, dk, dv = O.backward(q, k, v, do, latent, tile, wins, scale)

    def loss(qq, kk, vv):
        return float((O.forward(qq, kk, vv, latent, tile, wins, scale)[0] * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        for _ in range(6):
            idx = (0, 0, int(rng.integers(64)), int(rng.integers(3)))
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7


def test_backward_invariants():
    """Rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    sum_j dV_j = sum_i dO_i."""
    latent, tile = (6, 16, 16), (2, 4, 4)
    q, k, v, do = (_rand((1, 2, 1536, 8), s) for s in (29, 30, 31, 32))
    _, dk, dv = O.backward(q, k, v, do, latent, tile, [(3, 3, 3), (2, 1, 3)], 0.4)
    np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-10)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-10)


def test_backward_zero_query_closed_form():
    """Q = 0: P_ij = 1/(K_h L) on visible pairs, so dV_j = sum over the queries
    that see j of dO_i / (K_h L)."""
    latent, tile = (6, 16, 16), (2, 4, 4)
    n, L = O.tile_grid(latent, tile)
    win = (1, 3, 2)
    kh = int(np.prod([min(a, b) for a, b in zip(win, n)]))
    k, v, do = (_rand((1, 1, 1536, 4), s) for s in (33, 34, 35))
    q = np.zeros_like(k)
    _, _, dv = O.backward(q, k, v, do, latent, tile, [win], 0.3)
    coords = list(itertools.product(range(n[0]), range(n[1]), range(n[2])))
    dot = do[0, 0].reshape(len(coords), L, 4)
    for b, cb in enumerate(coords):
        seers = [a for a, ca in enumerate(coords)
                 if all(cb[d] in _window_by_sliding(ca[d], win[d], n[d]) for d in range(3))]
        ref = dot[seers].sum(axis=(0, 1)) / (kh * L)
        np.testing.assert_allclose(dv[0, 0, b * L:(b + 1) * L], np.broadcast_to(ref, (L, 4)), atol=1e-12)


def test_backward_key_rows_matches_full():
    latent, tile = (6, 16, 16), (2, 4, 4)
    wins = [(3, 3, 3)]
    q, k, v, do = (_rand((1, 1, 1536, 8), s) for s in (36, 37, 38, 39))
    _, dk, dv = O.backward(q, k, v, do, latent, tile, wins, 0.3)
    rows = np.array([0, 5, 33, 1000, 1535])
    dk2, dv2 = O.backward_key_rows(q, k, v, do, latent, tile, wins[0], 0.3, 0, 0, rows)
    np.testing.assert_allclose(dk2, dk[0, 0, rows], atol=1e-12)
    np.testing.assert_allclose(dv2, dv[0, 0, rows], atol=1e-12)


def test_backward_query_rows_matches_full():
    latent, tile = (6, 16, 16), (2, 4, 4)
    wins = [(1, 3, 3)]
    q, k, v, do = (_rand((1, 1, 1536, 8), s) for s in (43, 44, 45, 46))
    dq, _, _ = O.backward(q, k, v, do, latent, tile, wins, 0.3)
    rows = np.array([0, 7, 31, 32, 900, 1535])
    dq2 = O.backward_query_rows(q, k, v, do, latent, tile, wins[0], 0.3, 0, 0, rows)
    np.testing.assert_allclose(dq2, dq[0, 0, rows], atol=1e-12)


# ---------------------------------------------------------------- planted mistakes
#
# Every window decision of the oracle (pairs, masks, forward, backward, mass)
# goes through window_start.  A mistake planted there must make the pins above
# fail: the worked start sequences and the scalar brute-force forward, which
# builds its windows with its own sliding rule and so does not see the plant.

WORKED_STARTS = [(4, 3, [0, 0, 1, 1]), (6, 3, [0, 0, 1, 2, 3, 3]),
                 (10, 5, [0, 0, 0, 1, 2, 3, 4, 5, 5, 5])]


def _pin_worked_sequences():
    for n, w, starts in WORKED_STARTS:
        assert [O.sta_oracle.window_start(q, w, n)[0] for q in range(n)] == starts


def _pin_forward_brute_force():
    latent, tile = (4, 8, 12), (2, 4, 4)    # tile grid 2x2x3, 384 tokens
    wins = [(1, 1, 3), (2, 1, 1)]
    q, k, v = (_rand((1, 2, 384, 3), s) for s in (70, 71, 72))
    ref_o, ref_l = _brute_force_raster(q, k, v, latent, tile, wins, 0.6)
    o, l = O.sta_oracle.forward(q, k, v, latent, tile, wins, 0.6, order="raster")
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


def test_pins_hold_unplanted():
    _pin_worked_sequences()
    _pin_forward_brute_force()


@pytest.mark.parametrize("plant", ["shift_low", "shift_high", "truncate"])
def test_pins_catch_planted_window_mistake(monkeypatch, plant):
    """Each planted window mistake fails the worked-sequence pin and the
    brute-force forward pin."""
    real = O.sta_oracle.window_start

    def planted(q, w, n):
        s, wp = real(q, w, n)
        if plant == "shift_low":       # window one tile too low (clamped at 0)
            return max(s - 1, 0), wp
        if plant == "shift_high":      # window one tile too high (clamped at the edge)
            return min(s + 1, int(n) - wp), wp
        # truncate at the grid edge instead of clamping the centre: the
        # window is cut short where it would leave the grid
        lo = int(q) - wp // 2
        hi = lo + wp
        return max(lo, 0), min(hi, int(n)) - max(lo, 0)
    monkeypatch.setattr(O.sta_oracle, "window_start", planted)
    with pytest.raises(AssertionError):
        _pin_worked_sequences() if plant != "truncate" else _pin_count_invariant()
    with pytest.raises(AssertionError):
        _pin_forward_brute_force()


def _pin_count_invariant():
    """Every query tile sees prod w' key tiles (the pair-count pin)."""
    latent, tile, wins = (6, 16, 16), (2, 4, 4), [(3, 3, 3)]
    n, _ = O.tile_grid(latent, tile)
    pairs, _ = O.sta_oracle.tile_pairs(latent, tile, wins)
    counts = np.bincount(pairs[:, 0], minlength=int(np.prod(n)))
    assert np.all(counts == 27)


# ---------------------------------------------------------------- padding with masking

PAD_LATENT, PAD_TILE = (3, 5, 6), (2, 2, 4)     # padded to (4, 6, 8): tile grid 2x3x2, 90 real of 192


def test_padded_latent_and_valid_positions():
    assert O.padded_latent((29, 45, 76), (6, 8, 8)) == (30, 48, 80)    # the pages' example
    assert O.padded_latent((30, 48, 80), (6, 8, 8)) == (30, 48, 80)
    v = O.valid_positions(PAD_LATENT, PAD_TILE)
    assert v.size == 4 * 6 * 8 and v.sum() == 3 * 5 * 6
    # tile-major: position a*L + i holds a real token iff its padded coordinates are inside
    L = 2 * 2 * 4
    for pos in range(v.size):
        a, i = divmod(pos, L)
        a0, a1, a2 = a // 6, (a // 2) % 3, a % 2
        i0, i1, i2 = i // 8, (i // 4) % 2, i % 4
        tau, y, x = a0 * 2 + i0, a1 * 2 + i1, a2 * 4 + i2
        assert v[pos] == (tau < 3 and y < 5 and x < 6)
    assert O.valid_positions((4, 6, 8), PAD_TILE).all()


def test_pad_reorder_brute_force_and_round_trip():
    T, H, W = PAD_LATENT
    x = _rand((2, T * H * W, 3), 60)
    y = O.pad_reorder(x, PAD_LATENT, PAD_TILE)
    assert y.shape == (2, 192, 3)
    for tau in range(T):
        for yy in range(H):
            for xx in range(W):
                a = ((tau // 2) * 3 + yy // 2) * 2 + xx // 4
                i = ((tau % 2) * 2 + yy % 2) * 4 + xx % 4
                assert np.array_equal(y[:, a * 16 + i], x[:, (tau * H + yy) * W + xx])
    assert not y[:, ~O.valid_positions(PAD_LATENT, PAD_TILE)].any()    # padding rows are zero
    assert np.array_equal(O.pad_unreorder(y, PAD_LATENT, PAD_TILE), x)
    # a whole-tile latent: the same as the plain reorder
    z = _rand((1, 192, 2), 61)
    assert np.array_equal(O.pad_reorder(z, (4, 6, 8), PAD_TILE), O.reorder(z, (4, 6, 8), PAD_TILE))


def _brute_force_padded(q, k, v, latent, tile, wins, scale):
    """Raster tokens of a latent that is not a whole number of tiles: the tile
    grid is the padded one (ceil), windows slide on it, and only real tokens
    are keys.  Scalar loops and math.exp."""
    T, H, W = latent
    t, h, w = tile
    n = (-(-T // t), -(-H // h), -(-W // w))
    B, Hh, S, D = q.shape
    coords = [(tau, y, x) for tau in range(T) for y in range(H) for x in range(W)]
    tc = [(tau // t, y // h, x // w) for tau, y, x in coords]
    out = np.zeros_like(q)
    lse = np.zeros((B, Hh, S))
    for hh in range(Hh):
        wins_d = [[_window_by_sliding(qq, wins[hh][d], n[d]) for qq in range(n[d])] for d in range(3)]
        for b in range(B):
            for i in range(S):
                vis = [j for j in range(S) if all(tc[j][d] in wins_d[d][tc[i][d]] for d in range(3))]
                s = [scale * sum(q[b, hh, i, c] * k[b, hh, j, c] for c in range(D)) for j in vis]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                for c in range(D):
                    out[b, hh, i, c] = sum(e[a] * v[b, hh, j, c] for a, j in enumerate(vis)) / tot
                lse[b, hh, i] = mx + math.log(tot)
    return out, lse


def test_padded_forward_matches_brute_force():
    wins = [(1, 2, 1), (2, 3, 2), (1, 1, 2)]
    S = 90
    q, k, v = (_rand((1, 3, S, 5), s) for s in (62, 63, 64))
    ref_o, ref_l = _brute_force_padded(q, k, v, PAD_LATENT, PAD_TILE, wins, 0.6)
    qt, kt, vt = (O.pad_reorder(a, PAD_LATENT, PAD_TILE) for a in (q, k, v))
    o, l = O.forward(qt, kt, vt, PAD_LATENT, PAD_TILE, wins, 0.6)
    np.testing.assert_allclose(O.pad_unreorder(o, PAD_LATENT, PAD_TILE), ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.pad_unreorder(l[..., None], PAD_LATENT, PAD_TILE)[..., 0], ref_l,
                               rtol=0, atol=1e-12)
    pad = ~O.valid_positions(PAD_LATENT, PAD_TILE)
    assert not o[:, :, pad].any() and not l[:, :, pad].any()


def test_padded_forward_ignores_padding_values():
    """Whatever the padding rows hold, no real row changes."""
    wins = [(2, 2, 2)]
    q, k, v = (_rand((1, 1, 90, 4), s) for s in (65, 66, 67))
    qt, kt, vt = (O.pad_reorder(a, PAD_LATENT, PAD_TILE) for a in (q, k, v))
    o, l = O.forward(qt, kt, vt, PAD_LATENT, PAD_TILE, wins, 0.5)
    pad = ~O.valid_positions(PAD_LATENT, PAD_TILE)
    for a in (qt, kt, vt):
        a[:, :, pad] = 7.0
    o2, l2 = O.forward(qt, kt, vt, PAD_LATENT, PAD_TILE, wins, 0.5)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(l2, l)


def test_padded_full_window_is_dense_over_real_tokens():
    """A window covering the padded grid: attention over every real token."""
    latent, tile = (29, 5, 7), (6, 2, 4)
    S = 29 * 5 * 7
    q, k, v = (_rand((1, 2, S, 8), s) for s in (68, 69, 70))
    qt, kt, vt = (O.pad_reorder(a, latent, tile) for a in (q, k, v))
    o, l = O.forward(qt, kt, vt, latent, tile, [(9, 9, 9), (5, 3, 2)], 0.35)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a) for a in (q, k, v)), scale=0.35).numpy()
    np.testing.assert_allclose(O.pad_unreorder(o, latent, tile), ref, rtol=0, atol=1e-12)
    lse_ref = torch.logsumexp(0.35 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2), -1).numpy()
    np.testing.assert_allclose(O.pad_unreorder(l[..., None], latent, tile)[..., 0], lse_ref, rtol=0, atol=1e-12)


def test_padded_backward_matches_autograd():
    """Autograd through SDPA over the real tokens (raster order) with the mask
    of the padded tile grid built by the test's own sliding-window rule."""
    latent, tile, wins, scale = PAD_LATENT, PAD_TILE, [(1, 2, 1), (2, 3, 2)], 0.45
    T, H, W = latent
    n = (2, 3, 2)
    coords = [(tau // 2, y // 2, x // 4) for tau in range(T) for y in range(H) for x in range(W)]
    masks = []
    for win in wins:
        wd = [[_window_by_sliding(qq, win[d], n[d]) for qq in range(n[d])] for d in range(3)]
        masks.append([[all(cj[d] in wd[d][ci[d]] for d in range(3)) for cj in coords] for ci in coords])
    q, k, v, do = (_rand((2, 2, 90, 6), s) for s in (71, 72, 73, 74))
    qt, kt, vt = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.tensor(masks)[None], scale=scale)
    out.backward(torch.from_numpy(do))
    ref = (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy())
    args = [O.pad_reorder(a, latent, tile) for a in (q, k, v, do)]
    got = O.backward(*args, latent, tile, wins, scale)
    pad = ~O.valid_positions(latent, tile)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(O.pad_unreorder(g, latent, tile), r, rtol=0, atol=1e-11)
        assert not g[:, :, pad].any()
    # the sampled-row helpers agree with the whole-tensor gradients
    rows = np.arange(192)
    dq_rows = O.backward_query_rows(*args, latent, tile, wins[1], scale, 1, 1, rows)
    np.testing.assert_allclose(dq_rows, got[0][1, 1], rtol=0, atol=1e-12)
    dk_rows, dv_rows = O.backward_key_rows(*args, latent, tile, wins[1], scale, 1, 1, rows)
    np.testing.assert_allclose(dk_rows, got[1][1, 1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_rows, got[2][1, 1], rtol=0, atol=1e-12)


# --- attention mass of candidate windows (per-head window search) ---------

def _brute_force_mass(q, k, latent, tile, cands, scale):
    """Mass by scalar loops: full softmax of each real query over every real
    key with math.exp, then the probabilities of keys in the window summed.
    Raster order; padded latents slide windows on the ceil grid."""
    T, H, W = latent
    t, h, w = tile
    n = (-(-T // t), -(-H // h), -(-W // w))
    B, Hh, S, D = q.shape
    tc = [(tau // t, y // h, x // w) for tau in range(T) for y in range(H) for x in range(W)]
    out = np.zeros((len(cands), B, Hh))
    for c, win in enumerate(cands):
        wins_d = [[_window_by_sliding(qq, win[d], n[d]) for qq in range(n[d])] for d in range(3)]
        for b in range(B):
            for hh in range(Hh):
                tot = 0.0
                for i in range(S):
                    s = [scale * sum(q[b, hh, i, x] * k[b, hh, j, x] for x in range(D)) for j in range(S)]
                    mx = max(s)
                    e = [math.exp(x - mx) for x in s]
                    inside = sum(e[j] for j in range(S)
                                 if all(tc[j][d] in wins_d[d][tc[i][d]] for d in range(3)))
                    tot += inside / sum(e)
                out[c, b, hh] = tot / S
    return out


def test_window_mass_matches_brute_force():
    latent, tile = (4, 8, 8), (2, 4, 4)     # tile grid 2x2x2, 256 tokens
    cands = [(1, 1, 1), (2, 1, 2), (1, 2, 1), (9, 9, 9)]
    q, k = (_rand((2, 2, 256, 3), s) for s in (71, 72))
    ref = _brute_force_mass(q, k, latent, tile, cands, 0.8)
    got = O.window_mass(q, k, latent, tile, cands, 0.8, order="raster")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    qt, kt = (O.reorder(a, latent, tile) for a in (q, k))
    np.testing.assert_allclose(O.window_mass(qt, kt, latent, tile, cands, 0.8), ref, rtol=0, atol=1e-12)


def test_window_mass_padded_matches_brute_force():
    cands = [(1, 1, 1), (1, 2, 1), (2, 3, 2)]
    q, k = (_rand((1, 2, 90, 4), s) for s in (73, 74))
    ref = _brute_force_mass(q, k, PAD_LATENT, PAD_TILE, cands, 0.6)
    qt, kt = (O.pad_reorder(a, PAD_LATENT, PAD_TILE) for a in (q, k))
    got = O.window_mass(qt, kt, PAD_LATENT, PAD_TILE, cands, 0.6)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_mass_full_window_is_one():
    latent, tile = (6, 8, 12), (2, 4, 4)    # grid 3x2x3
    q, k = (_rand((1, 3, 576, 8), s) for s in (75, 76))
    got = O.window_mass(q, k, latent, tile, [(3, 2, 3), (7, 7, 7)], 0.4)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-12)


def test_window_mass_uniform_attention_counts_keys():
    # Q = 0: attention is uniform over the real keys, so a window keeps the
    # fraction of real keys lying in it.
    latent, tile = (6, 8, 12), (2, 4, 4)    # grid 3x2x3, L = 32
    k = _rand((1, 1, 576, 4), 77)
    got = O.window_mass(np.zeros_like(k), k, latent, tile, [(1, 1, 1), (3, 1, 2), (2, 2, 2)], 1.0)
    np.testing.assert_allclose(got[:, 0, 0], [1 / 18, 6 / 18, 8 / 18], rtol=0, atol=1e-12)
    # padded: count real keys per window tile by tile
    kp = O.pad_reorder(_rand((1, 1, 90, 4), 78), PAD_LATENT, PAD_TILE)
    cands = [(1, 1, 1), (1, 2, 1)]
    got = O.window_mass(np.zeros_like(kp), kp, PAD_LATENT, PAD_TILE, cands, 1.0)
    grid = O.padded_latent(PAD_LATENT, PAD_TILE)
    n, L = O.tile_grid(grid, PAD_TILE)
    real = O.valid_positions(PAD_LATENT, PAD_TILE).reshape(-1, L)
    tiles = list(itertools.product(*(range(x) for x in n)))
    for c, win in enumerate(cands):
        num = 0.0
        for qi, qt in enumerate(tiles):
            keys = sum(real[ki].sum() for ki, kt in enumerate(tiles) if O.window_contains(qt, kt, win, n))
            num += real[qi].sum() * keys / real.sum()
        assert got[c, 0, 0] == pytest.approx(num / real.sum(), abs=1e-12)


def test_window_mass_is_exp_of_lse_difference():
    # The window's softmax normaliser against the full one: mass_i = exp(LSE_w - LSE_full).
    latent, tile = (6, 8, 12), (2, 4, 4)
    q, k, v = (_rand((2, 2, 576, 8), s) for s in (79, 80, 81))
    win = (2, 1, 2)
    _, lw = O.forward(q, k, v, latent, tile, [win] * 2, 0.5)
    _, lf = O.dense_forward(q, k, v, 0.5)
    ref = np.exp(lw - lf).mean(axis=2)
    np.testing.assert_allclose(O.window_mass(q, k, latent, tile, [win], 0.5)[0], ref, rtol=0, atol=1e-12)


def test_window_mass_grows_with_nested_windows():
    latent, tile = (10, 8, 12), (2, 4, 4)   # grid 5x2x3
    q, k = (_rand((1, 2, 960, 4), s) for s in (82, 83))
    m = O.window_mass(q, k, latent, tile, [(1, 1, 1), (3, 1, 1), (3, 1, 3), (5, 2, 3)], 1.0)
    assert np.all(np.diff(m[:, 0, :], axis=0) > 0)
    np.testing.assert_allclose(m[-1], 1.0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pair-by-pair key rows

@pytest.mark.parametrize("latent,tile,win", [
    ((6, 16, 16), (2, 4, 4), (3, 3, 3)),
    ((6, 16, 16), (2, 4, 4), (2, 1, 4)),          # even windows, one of them clamped
    ((6, 16, 16), (2, 4, 4), (9, 9, 9)),          # full window
    ((5, 15, 13), (2, 4, 4), (3, 1, 3)),          # padded to (6, 16, 16)
])
def test_backward_key_rows_by_pairs_matches_full(latent, tile, win):
    """The pair-by-pair formulation equals the masked dense backward at every
    sampled key row, heaviest and padding rows included."""
    S = O.tile_grid(O.padded_latent(latent, tile), tile)[1] * int(np.prod(
        [-(-a // b) for a, b in zip(latent, tile)]))
    q, k, v, do = (_rand((1, 2, S, 8), s) for s in (80, 81, 82, 83))
    valid = O.valid_positions(latent, tile)
    for a in (q, k, v, do):
        a[:, :, ~valid] = 0.0
    _, dk, dv = O.backward(q, k, v, do, latent, tile, [win, win], 0.4)
    rows = np.array([0, 1, 31, 32, 300, 777, 1000, S - 33, S - 1])
    dk2, dv2 = O.backward_key_rows_by_pairs(q, k, v, do, latent, tile, win, 0.4, 0, 1, rows)
    np.testing.assert_allclose(dk2, dk[0, 1, rows], atol=1e-12)
    np.testing.assert_allclose(dv2, dv[0, 1, rows], atol=1e-12)
    # and the masked dense helper agrees too
    dk3, dv3 = O.backward_key_rows(q, k, v, do, latent, tile, win, 0.4, 0, 1, rows)
    np.testing.assert_allclose(dk2, dk3, atol=1e-12)
    np.testing.assert_allclose(dv2, dv3, atol=1e-12)
