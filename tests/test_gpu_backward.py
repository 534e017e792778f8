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


@pytest.mark.parametrize("latent,tile", [((11, 30, 29), (2, 8, 8)), ((5, 15, 13), (2, 4, 4))])
def test_backward_bf16_padding_contents(sta, latent, tile):
    """Padding rows of q, k, v and dout filled with large finite values (the
    header asks only for finite contents there): the gradients of real rows
    match the oracle on zero-padded inputs and padding rows stay zero.  Covers
    both key-mask modes of the dQ pass (tile width 8 and 4) and the dK/dV
    pass, which relies on the +inf statistics of padding queries."""
    wins = [(3, 3, 3), (2, 1, 3)]
    S = int(np.prod(latent))
    x = I.make_inputs(1, len(wins), S, 128, "bf16", seed=21, with_do=True)
    scale = 128 ** -0.5
    pad = torch.from_numpy(~O.valid_positions(latent, tile)).to("cuda")
    g = torch.Generator(device="cpu").manual_seed(5)
    t = {}
    for n in ("q", "k", "v", "do"):
        y = _tm(sta, x[n], latent, tile).clone()
        junk = (torch.rand(y.shape, generator=g) * 60 - 30).to(torch.bfloat16).to("cuda")
        y[:, :, pad] = junk[:, :, pad]
        t[n] = y
    o, lse = sta.forward(t["q"], t["k"], t["v"], latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(t["q"], t["k"], t["v"], o, t["do"], lse, latent, tile, wins, scale=scale)
    ref = O.backward(*(O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v", "do")),
                     latent, tile, wins, scale)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert bool(torch.isfinite(got.float()).all()), name
        assert float(got[:, :, pad].float().abs().max()) == 0.0, name
        e = err_report(to64(got), r)
        print(name, e)
        assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS, name


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


def test_backward_bf16_finetune_sampled(sta):
    """Fine-tuning shape: latent (24,64,64), tile (6,8,8), 24 heads, D=128,
    window (3,5,5).  dQ on sampled query rows and dK/dV on the rows of a corner
    key tile (few query tiles see it) against the oracle; at full size, the
    invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i."""
    name = "finetune_24x64x64_w355"
    w = I.WORKLOADS[name]
    latent, tile, wins, D = w["latent"], w["tile"], w["windows"], w["head_dim"]
    n, L = O.tile_grid(latent, tile)
    scale = D ** -0.5
    x = I.workload_inputs(name, with_do=True)
    q, k, v, do = (_tm(sta, x[nm], latent, tile) for nm in ("q", "k", "v", "do"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=scale)
    torch.cuda.synchronize()
    # Invariants over whole sequences (every head): rows of dS sum to zero, so
    # sum_j dK_j = 0; rows of P sum to one, so sum_j dV_j = sum_i dO_i.  The
    # bound allows bf16 rounding (2^-8 relative) of every summed element.
    dkf, dvf, dof = dk.float(), dv.float(), do.float()
    assert bool((dkf.sum(2).abs() <= 2.0 ** -7 * dkf.abs().sum(2) + 1e-3).all())
    assert bool(((dvf.sum(2) - dof.sum(2)).abs()
                 <= 2.0 ** -7 * (dvf.abs().sum(2) + dof.abs().sum(2)) + 1e-3).all())
    del dkf, dvf, dof
    heads = [0, 23]
    qrows = np.r_[0:16, L - 16:L + 16, (n[0] * n[1] * n[2] - 1) * L:(n[0] * n[1] * n[2] - 1) * L + 16]
    krows = np.r_[0:16, L - 16:L]           # tile 0: seen by 2*3*3 query tiles
    for h in heads:
        hq, hk, hv, hdo = (O.pad_reorder(to64(x[nm][:, h:h + 1]), latent, tile)
                           for nm in ("q", "k", "v", "do"))
        rdq = O.backward_query_rows(hq, hk, hv, hdo, latent, tile, wins[h], scale, 0, 0, qrows)
        e = err_report(to64(dq[0, h, torch.from_numpy(qrows).cuda()]), rdq)
        print("head", h, "dq", e)
        assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS
        if h != heads[0]:
            continue   # the key-row oracle is the slow one: one head suffices
        rdk, rdv = O.backward_key_rows(hq, hk, hv, hdo, latent, tile, wins[h], scale, 0, 0, krows)
        kr = torch.from_numpy(krows).cuda()
        for nm, got, r in (("dk", dk, rdk), ("dv", dv, rdv)):
            e = err_report(to64(got[0, h, kr]), r)
            print("head", h, nm, e)
            assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS


def test_backward_bf16_hunyuan_mixed_sampled(sta):
    """HunyuanVideo shape (30,48,80) with the mixed per-head windows (full,
    (1,6,10), (3,3,3), ...): dQ on sampled query rows of one head per window
    kind, dK/dV on a corner key tile of a (3,3,3) head, and the full-size
    invariants.  Exercises non-uniform transposed windows and the key-tile
    ordering across heads of different weight."""
    name = "hunyuan_30x48x80_mixed"
    w = I.WORKLOADS[name]
    latent, tile, wins, D = w["latent"], w["tile"], w["windows"], w["head_dim"]
    n, L = O.tile_grid(latent, tile)
    scale = D ** -0.5
    x = I.workload_inputs(name, seed=2, with_do=True)
    q, k, v, do = (_tm(sta, x[nm], latent, tile) for nm in ("q", "k", "v", "do"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=scale)
    torch.cuda.synchronize()
    dkf, dvf, dof = dk.float(), dv.float(), do.float()
    assert bool((dkf.sum(2).abs() <= 2.0 ** -7 * dkf.abs().sum(2) + 1e-3).all())
    assert bool(((dvf.sum(2) - dof.sum(2)).abs()
                 <= 2.0 ** -7 * (dvf.abs().sum(2) + dof.abs().sum(2)) + 1e-3).all())
    del dkf, dvf, dof
    heads = sorted({wins.index(wd) for wd in set(wins)})   # one head of every window kind
    qrows = np.r_[0:8, 150 * L - 8:150 * L + 8, (n[0] * n[1] * n[2] - 1) * L:(n[0] * n[1] * n[2] - 1) * L + 8]
    krows = np.r_[0:8, L - 8:L]           # key tile 0
    for h in heads:
        hq, hk, hv, hdo = (O.pad_reorder(to64(x[nm][:, h:h + 1]), latent, tile)
                           for nm in ("q", "k", "v", "do"))
        rdq = O.backward_query_rows(hq, hk, hv, hdo, latent, tile, wins[h], scale, 0, 0, qrows)
        e = err_report(to64(dq[0, h, torch.from_numpy(qrows).cuda()]), rdq)
        print("head", h, wins[h], "dq", e)
        assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS
        if tuple(wins[h]) != (3, 3, 3):
            continue   # the key-row oracle's cost grows with the window: one kind suffices
        rdk, rdv = O.backward_key_rows(hq, hk, hv, hdo, latent, tile, wins[h], scale, 0, 0, krows)
        kr = torch.from_numpy(krows).cuda()
        for nm, got, r in (("dk", dk, rdk), ("dv", dv, rdv)):
            e = err_report(to64(got[0, h, kr]), r)
            print("head", h, wins[h], nm, e)
            assert e["max_abs"] < BF16_TOL and e["rel_rms"] < BF16_REL_RMS
