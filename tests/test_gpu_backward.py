"""GPU parity of sta_backward (bf16 MFMA and fp32 debug) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from _helpers import err_report, to64
from sparse_sliding_tile_amd import inputs as I

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
BF16_REL_RMS = 1e-2


@pytest.fixture(scope="module")
def sta():
    import sparse_sliding_tile_amd as s
    s.lib()
    return s


def _tm(sta, t, latent, tile):
    return sta.tile_reorder(t.to("cuda").contiguous(), latent, tile)


BWD_SMALL = [  # latent, tile, B, windows, D
    ((6, 16, 16), (2, 4, 4), 2, [(3, 3, 3), (1, 2, 5)], 128),      # L = 32
    ((6, 16, 16), (2, 4, 4), 1, [(2, 3, 1), (9, 9, 9)], 64),
    ((6, 32, 32), (2, 8, 8), 2, [(3, 3, 3), (1, 4, 2)], 128),      # L = 128
    ((12, 16, 24), (6, 8, 8), 1, [(1, 3, 3), (2, 2, 2)], 128),     # L = 384
    ((6, 32, 32), (2, 8, 8), 1, [(3, 1, 3)], 64),
    ((1, 32, 40), (1, 8, 8), 2, [(1, 3, 3), (1, 2, 4)], 128),     # 2D, L = 64
    ((5, 15, 13), (2, 4, 4), 1, [(3, 3, 3), (2, 1, 4)], 128),     # padded to (6, 16, 16)
    ((11, 30, 29), (2, 8, 8), 1, [(3, 3, 3)], 128),               # padded, L = 128
]


@pytest.mark.parametrize("latent,tile,B,wins,D", BWD_SMALL)
def test_backward_bf16_small(sta, latent, tile, B, wins, D):
    S = int(np.prod(latent))
    x = I.make_inputs(B, len(wins), S, D, "bf16", seed=9, with_do=True)
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


@pytest.mark.parametrize("magnitude", ["moderate", "edge"])
@pytest.mark.parametrize("latent,tile", [((11, 30, 29), (2, 8, 8)), ((5, 15, 13), (2, 4, 4))])
def test_padding_contents_any_finite(sta, latent, tile, magnitude):
    """Padding rows of q, k, v and dout may hold any finite values (the
    header's contract).  'moderate' fills them with values in +-30; 'edge'
    with +-3e38, whose products overflow fp32 to +-inf (and their sums to
    NaN) inside the kernels.  Forward and backward outputs of real rows match
    the oracle on zero-padded inputs, and every output at a padding row is
    exactly zero.  Tile widths 8 and 4, partial tiles along every axis: the
    kernels stage only real rows of partial tiles (compacted), so padding
    contents must never reach a result."""
    wins = [(3, 3, 3), (2, 1, 3)]
    S = int(np.prod(latent))
    print(f"[padding contents] {latent} {tile} {magnitude}", flush=True)
    x = I.make_inputs(1, len(wins), S, 128, "bf16", seed=21, with_do=True)
    scale = 128 ** -0.5
    pad = torch.from_numpy(~O.valid_positions(latent, tile)).to("cuda")
    g = torch.Generator(device="cpu").manual_seed(5)
    t = {}
    for n in ("q", "k", "v", "do"):
        y = _tm(sta, x[n], latent, tile).clone()
        if magnitude == "moderate":
            junk = torch.rand(y.shape, generator=g) * 60 - 30
        else:
            junk = torch.where(torch.rand(y.shape, generator=g) < 0.5, -3.0e38, 3.0e38)
        junk = junk.to(torch.bfloat16).to("cuda")
        assert bool(torch.isfinite(junk.float()).all())
        y[:, :, pad] = junk[:, :, pad]
        t[n] = y
    o, lse = sta.forward(t["q"], t["k"], t["v"], latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(t["q"], t["k"], t["v"], o, t["do"], lse, latent, tile, wins, scale=scale)
    xs = [O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v", "do")]
    ro, rl = O.forward(*xs[:3], latent, tile, wins, scale)
    ref = O.backward(*xs, latent, tile, wins, scale)
    for name, got, r in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), (ro, rl) + tuple(ref)):
        assert bool(torch.isfinite(got.float()).all()), name
        assert float(got[:, :, pad].float().abs().max()) == 0.0, name
        e = err_report(to64(got), r)
        print(name, e)
        assert e["max_abs"] < BF16_TOL, name
        if name != "lse":
            assert e["rel_rms"] < BF16_REL_RMS, name


def test_backward_bf16_zero_query(sta):
    """Q = 0: P is uniform over each window, so dV_j is the mean-weighted sum of
    dO over the queries that see key j; pins the transposed window walk."""
    latent, tile, wins = (6, 32, 32), (2, 8, 8), [(3, 3, 3), (1, 2, 4)]
    S = int(np.prod(latent))
    x = I.make_inputs(1, 2, S, 128, "bf16", seed=10, with_do=True)
    q = torch.zeros((1, 2, S, 128), dtype=torch.bfloat16, device="cuda")
    k, v, do = (_tm(sta, x[n], latent, tile) for n in ("k", "v", "do"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=0.088)
    _, _, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=0.088)
    rk, rv, rdo = (O.reorder(to64(x[n]), latent, tile) for n in ("k", "v", "do"))
    _, _, rdv = O.backward(np.zeros((1, 2, S, 128)), rk, rv, rdo, latent, tile, wins, 0.088)
    e = err_report(to64(dv), rdv)
    print(e)
    assert e["max_abs"] < 4e-3 and e["rel_rms"] < BF16_REL_RMS


def _full_size_backward(sta, name, seed):
    w = I.WORKLOADS[name]
    latent, tile, wins, D = w["latent"], w["tile"], w["windows"], w["head_dim"]
    print(f"[full-size backward] {name} seed {seed}", flush=True)
    x = I.workload_inputs(name, seed=seed, with_do=True)
    q, k, v, do = (_tm(sta, x[nm], latent, tile) for nm in ("q", "k", "v", "do"))
    scale = D ** -0.5
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=scale)
    torch.cuda.synchronize()
    del q, k, v, o, lse
    return {"x": x, "do": do, "dq": dq, "dk": dk, "dv": dv, "latent": latent, "tile": tile, "wins": wins,
            "scale": scale, "grid": O.tile_grid(latent, tile)}


@pytest.fixture(scope="module")
def finetune(sta):
    """Fine-tuning shape: latent (24,64,64), tile (6,8,8), 24 heads, D=128,
    window (3,5,5); the backward runs once on the GPU for every test below."""
    r = _full_size_backward(sta, "finetune_24x64x64_w355", 0)
    yield r
    r.clear()


@pytest.fixture(scope="module")
def mixed(sta):
    """HunyuanVideo shape (30,48,80) with the mixed per-head windows."""
    r = _full_size_backward(sta, "hunyuan_30x48x80_mixed", 2)
    yield r
    r.clear()


def _invariants(r):
    # rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    # sum_j dV_j = sum_i dO_i.  The bound allows bf16 rounding (2^-8
    # relative) of every summed element.
    dkf, dvf, dof = r["dk"].float(), r["dv"].float(), r["do"].float()
    assert bool((dkf.sum(2).abs() <= 2.0 ** -7 * dkf.abs().sum(2) + 1e-3).all())
    assert bool(((dvf.sum(2) - dof.sum(2)).abs()
                 <= 2.0 ** -7 * (dvf.abs().sum(2) + dof.abs().sum(2)) + 1e-3).all())


def _head(r, h):
    lt = (r["latent"], r["tile"])
    return [O.pad_reorder(to64(r["x"][nm][:, h:h + 1]), *lt) for nm in ("q", "k", "v", "do")]


def _check_dq(r, h, qrows):
    hq, hk, hv, hdo = _head(r, h)
    rdq = O.backward_query_rows(hq, hk, hv, hdo, r["latent"], r["tile"], r["wins"][h], r["scale"], 0, 0, qrows)
    e = err_report(to64(r["dq"][0, h, torch.from_numpy(qrows).cuda()]), rdq)
    print("head", h, r["wins"][h], "dq", e)
    assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS


def _check_dkdv(r, h, ktiles, per_tile=8):
    """dK/dV on the first and last per_tile rows of each key tile in ktiles
    (pair-by-pair oracle: its cost follows the window)."""
    L = r["grid"][1]
    krows = np.concatenate([np.r_[t * L:t * L + per_tile, (t + 1) * L - per_tile:(t + 1) * L] for t in ktiles])
    hq, hk, hv, hdo = _head(r, h)
    rdk, rdv = O.backward_key_rows_by_pairs(hq, hk, hv, hdo, r["latent"], r["tile"], r["wins"][h], r["scale"],
                                            0, 0, krows)
    kr = torch.from_numpy(krows).cuda()
    for nm, got, ref in (("dk", r["dk"], rdk), ("dv", r["dv"], rdv)):
        e = err_report(to64(got[0, h, kr]), ref)
        print("head", h, r["wins"][h], "key tiles", ktiles, nm, e)
        assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS


def _transposed_count(t, n, win):
    """Query tiles whose window holds key tile t (oracle window rule)."""
    coords = np.stack(np.meshgrid(*(np.arange(a) for a in n), indexing="ij"), -1).reshape(-1, 3)
    return sum(O.window_contains(c, coords[t], win, n) for c in coords)


def test_backward_finetune_invariants(finetune):
    _invariants(finetune)


def test_backward_finetune_dq_sampled(finetune):
    n, L = finetune["grid"]
    nt = n[0] * n[1] * n[2]
    qrows = np.r_[0:16, L - 16:L + 16, (nt - 1) * L:(nt - 1) * L + 16]
    for h in (0, 23):
        _check_dq(finetune, h, qrows)


def test_backward_finetune_dkdv_light_tile(finetune):
    """Key tile 0, seen by 2*3*3 = 18 query tiles."""
    assert _transposed_count(0, finetune["grid"][0], finetune["wins"][0]) == 18
    _check_dkdv(finetune, 0, [0], per_tile=16)


def test_backward_finetune_dkdv_heavy_tiles(finetune):
    """The heaviest key tile (seen by all 4*8*8 = 256 query tiles: the first
    key-major workgroups to run) and a mid-count one (4*5*5 = 100)."""
    n, win = finetune["grid"][0], finetune["wins"][0]
    heavy = ((1 * n[1]) + 3) * n[2] + 3        # tile (1, 3, 3)
    mid = ((1 * n[1]) + 2) * n[2] + 2          # tile (1, 2, 2)
    assert _transposed_count(heavy, n, win) == 256 and _transposed_count(mid, n, win) == 100
    _check_dkdv(finetune, 0, [heavy, mid])
    _check_dkdv(finetune, 17, [heavy])


def test_backward_mixed_invariants(mixed):
    _invariants(mixed)


def test_backward_mixed_dq_sampled(mixed):
    n, L = mixed["grid"]
    nt = n[0] * n[1] * n[2]
    wins = mixed["wins"]
    qrows = np.r_[0:8, 150 * L - 8:150 * L + 8, (nt - 1) * L:(nt - 1) * L + 8]
    for h in sorted({wins.index(wd) for wd in set(wins)}):   # one head of every window kind
        _check_dq(mixed, h, qrows)


def _mixed_head(mixed, win):
    return mixed["wins"].index(win)


def test_backward_mixed_dkdv_333(mixed):
    """A (3,3,3) head: corner key tile 0 and interior tile (2,3,5)."""
    n = mixed["grid"][0]
    _check_dkdv(mixed, _mixed_head(mixed, (3, 3, 3)), [0, ((2 * n[1]) + 3) * n[2] + 5])


def test_backward_mixed_dkdv_1_6_10(mixed):
    """A (1,6,10) head (the whole H x W plane of one T slice): tile 0 and an
    interior tile."""
    n = mixed["grid"][0]
    _check_dkdv(mixed, _mixed_head(mixed, (1, 6, 10)), [0, ((2 * n[1]) + 3) * n[2] + 5])


def test_backward_mixed_dkdv_full_window(mixed):
    """A (5,6,10) head (every key tile seen by all 300 query tiles: the
    heaviest key-major work of the launch): tile 0 and an interior tile."""
    n, win = mixed["grid"][0], (5, 6, 10)
    interior = ((2 * n[1]) + 3) * n[2] + 5
    assert _transposed_count(interior, n, win) == 300
    _check_dkdv(mixed, _mixed_head(mixed, win), [0, interior], per_tile=4)
