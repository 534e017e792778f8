"""GPU parity of the libsta kernels against the fp64 CPU oracle (through the C-ABI)."""
import numpy as np
import pytest
import torch

import oracle as O
from _helpers import bits, err_report, sample_query_tiles, to64
from sparse_sliding_tile_amd import inputs as I

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2     # max-abs, bf16 I/O with fp32 accumulation
F32_TOL = 1e-5      # max-abs, fp32 debug instance
BF16_REL_RMS = 1e-2


@pytest.fixture(scope="module")
def sta():
    import sparse_sliding_tile_amd as s
    s.lib()
    return s


def _dev(x):
    return x.to("cuda").contiguous()


# ------------------------------------------------------------------ reorder

REORDER_CASES = [((6, 16, 16), (2, 4, 4), 1, 2, 64, torch.float32),
                 ((6, 16, 16), (2, 4, 4), 2, 3, 128, torch.bfloat16),
                 ((5, 6, 10), (5, 3, 2), 1, 2, 24, torch.bfloat16),     # ragged rows: 48-byte tokens
                 ((3, 4, 5), (1, 1, 1), 2, 1, 7, torch.float32),       # 28-byte rows, identity order
                 ((30, 48, 80), (6, 8, 8), 1, 2, 128, torch.bfloat16),
                 ((5, 15, 13), (2, 4, 4), 2, 2, 64, torch.bfloat16),    # padded to (6, 16, 16)
                 ((5, 6, 9), (5, 3, 2), 1, 2, 24, torch.float32),      # padded, ragged rows
                 ((29, 45, 76), (6, 8, 8), 1, 1, 128, torch.bfloat16)]  # the pages' padding example


@pytest.mark.parametrize("latent,tile,B,Hh,D,dtype", REORDER_CASES)
def test_reorder_bit_exact(sta, latent, tile, B, Hh, D, dtype):
    S = int(np.prod(latent))
    g = torch.Generator().manual_seed(3)
    x = torch.randn((B, Hh, S, D), generator=g).to(dtype)
    y = sta.tile_reorder(_dev(x), latent, tile)
    ref = O.pad_reorder(bits(x), latent, tile)     # padding rows zero
    assert np.array_equal(bits(y), ref)
    back = sta.tile_unreorder(y, latent, tile)
    assert np.array_equal(bits(back), bits(x))


def test_reorder_full_size_sampled(sta):
    """Wan-sized tensor [1, 40, 92160, 128] bf16: every sampled raster row lands
    at its oracle position, and the round trip is the identity."""
    latent, tile = (24, 48, 80), (6, 8, 8)
    S = int(np.prod(latent))
    g = torch.Generator().manual_seed(4)
    x = torch.randn((1, 40, S, 128), generator=g).to(torch.bfloat16)
    xd = _dev(x)
    y = sta.tile_reorder(xd, latent, tile)
    pi = O.tile_major_index(latent, tile)
    rows = np.random.default_rng(0).choice(S, 4096, replace=False)
    got = bits(y[:, :, torch.from_numpy(pi[rows]).cuda()])
    assert np.array_equal(got, bits(x[:, :, torch.from_numpy(rows)]))
    back = sta.tile_unreorder(y, latent, tile)
    assert torch.equal(back.view(torch.int16), xd.view(torch.int16))


# ------------------------------------------------------------------ pairs

PAIR_CASES = [((6, 16, 16), (2, 4, 4), [(3, 3, 3), (1, 2, 5)]),
              ((30, 48, 80), (6, 8, 8), I.mixed_windows(24, 0)),
              ((24, 48, 80), (6, 8, 8), [(3, 3, 5)] * 3),
              ((24, 64, 64), (6, 8, 8), [(3, 5, 5)] * 2)]


@pytest.mark.parametrize("latent,tile,wins", PAIR_CASES)
@pytest.mark.parametrize("transpose", [False, True])
def test_tile_pairs_bit_exact(sta, latent, tile, wins, transpose):
    p, off = sta.tile_pairs(latent, tile, wins, transpose=transpose)
    rp, roff = O.tile_pairs(latent, tile, wins, transpose=transpose)
    assert np.array_equal(off, roff)
    assert np.array_equal(p.cpu().numpy(), rp)


# ------------------------------------------------------------------ forward, fp32 debug

def _tile_major(sta, t, latent, tile):
    return sta.tile_reorder(_dev(t), latent, tile)


def test_forward_f32_tiny(sta):
    w = I.WORKLOADS["tiny_f32"]
    x = I.workload_inputs("tiny_f32")
    latent, tile, wins = w["latent"], w["tile"], w["windows"]
    q, k, v = (_tile_major(sta, x[n], latent, tile) for n in ("q", "k", "v"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=64 ** -0.5)
    rq, rk, rv = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v"))
    ro, rl = O.forward(rq, rk, rv, latent, tile, wins, 64 ** -0.5)
    assert err_report(to64(o), ro)["max_abs"] < F32_TOL
    assert err_report(to64(lse), rl)["max_abs"] < F32_TOL
    # the same result in raster order after unreorder
    ro_r, _ = O.forward(to64(x["q"]), to64(x["k"]), to64(x["v"]), latent, tile, wins, 64 ** -0.5,
                        order="raster")
    assert err_report(to64(sta.tile_unreorder(o, latent, tile)), ro_r)["max_abs"] < F32_TOL


def test_backward_f32_tiny(sta):
    w = I.WORKLOADS["tiny_f32"]
    x = I.workload_inputs("tiny_f32", with_do=True)
    latent, tile = w["latent"], w["tile"]
    wins = [(3, 3, 3), (1, 2, 4)]
    scale = 64 ** -0.5
    q, k, v, do = (_tile_major(sta, x[n], latent, tile) for n in ("q", "k", "v", "do"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=scale)
    rq, rk, rv, rdo = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v", "do"))
    ref = O.backward(rq, rk, rv, rdo, latent, tile, wins, scale)
    for got, r in zip((dq, dk, dv), ref):
        assert err_report(to64(got), r)["max_abs"] < F32_TOL


# ------------------------------------------------------------------ forward, bf16 MFMA

RASTER_CASES = [  # latent, tile, B, windows, D: every workgroup shape of the raster instance
    ((6, 32, 32), (2, 8, 8), 2, [(3, 3, 3), (1, 4, 2)], 128),     # L = 128: four waves
    ((6, 16, 32), (2, 4, 8), 1, [(3, 3, 3), (1, 2, 3)], 128),     # L = 64: two waves
    ((12, 16, 24), (3, 4, 8), 1, [(3, 3, 3), (2, 1, 2)], 128),    # L = 96: one wave
    ((6, 32, 32), (2, 8, 8), 1, [(3, 3, 3), (2, 2, 2)], 64),      # D = 64 (8-row copy segments)
    ((1, 32, 40), (1, 8, 8), 2, [(1, 3, 3), (1, 1, 5)], 128),     # 2D
]


@pytest.mark.parametrize("latent,tile,B,wins,D", RASTER_CASES)
def test_forward_raster_matches_oracle_and_reorder_path(sta, latent, tile, B, wins, D):
    """Raster-order forward: within tolerance of the oracle in raster order, and
    bit-identical to reorder -> sta_forward -> unreorder."""
    S = int(np.prod(latent))
    x = I.make_inputs(B, len(wins), S, D, "bf16", seed=9)
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = sta.forward_raster(q, k, v, latent, tile, wins)
    ro, rl = O.forward(to64(x["q"]), to64(x["k"]), to64(x["v"]), latent, tile, wins, D ** -0.5,
                       order="raster")
    eo, el = err_report(to64(o), ro), err_report(to64(lse), rl)
    print("O", eo, "LSE", el)
    assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
    assert el["max_abs"] < BF16_TOL
    qt, kt, vt = (sta.tile_reorder(a, latent, tile) for a in (q, k, v))
    ot, lt = sta.forward(qt, kt, vt, latent, tile, wins)
    assert torch.equal(sta.tile_unreorder(ot, latent, tile).view(torch.int16), o.view(torch.int16))
    lr = sta.tile_unreorder(lt.unsqueeze(-1), latent, tile).squeeze(-1)
    assert torch.equal(lr.view(torch.int32), lse.view(torch.int32))


RASTER_PADDED_CASES = [  # latent, tile, B, windows, D: padded latents in one launch
    ((5, 15, 13), (2, 4, 4), 2, [(3, 3, 3), (2, 1, 4)], 128),    # -> (6, 16, 16), L = 32, one wave
    # -> (12, 32, 32), L = 128, four waves; last-t tiles: 64 real keys in 2 of 4 key blocks and 64 real
    # query rows in 2 of 4 waves (2 idle); the corner tile's 30 real tokens (1 x 6 x 5) compacted into
    # one masked key block and one wave
    ((11, 30, 29), (2, 8, 8), 1, [(3, 3, 3), (1, 2, 2)], 128),
    ((3, 14, 29), (1, 8, 8), 1, [(1, 3, 3), (3, 1, 5)], 128),    # -> (3, 16, 32), L = 64, two waves
    ((5, 16, 20), (1, 8, 8), 1, [(3, 3, 3)], 64),                # D = 64 (8-row copy segments)
    # L = 96, one-wave workgroups, partial in every dim; the corner tile's 7 real tokens (1 x 1 x 7) in
    # one masked key block and one workgroup (the tile's other two find no real row)
    ((7, 9, 23), (3, 4, 8), 1, [(3, 3, 3), (1, 2, 2)], 128),
]


@pytest.mark.parametrize("latent,tile,B,wins,D", RASTER_PADDED_CASES)
def test_forward_raster_padded_matches_oracle_and_reorder_path(sta, latent, tile, B, wins, D):
    """Padded latents on the one-launch raster path: the raster tensors hold
    only the real tokens; O and LSE are within tolerance of the oracle (padded
    tile-major, then cropped back to raster) and bit-identical to tile_reorder
    (zero padding) -> sta_forward -> tile_unreorder."""
    S = int(np.prod(latent))
    x = I.make_inputs(B, len(wins), S, D, "bf16", seed=12)
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = sta.forward_raster(q, k, v, latent, tile, wins)
    rq, rk, rv = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v"))
    ro, rl = O.forward(rq, rk, rv, latent, tile, wins, D ** -0.5)
    ro_r = O.pad_unreorder(ro, latent, tile)
    rl_r = O.pad_unreorder(rl[..., None], latent, tile)[..., 0]
    eo, el = err_report(to64(o), ro_r), err_report(to64(lse), rl_r)
    print("O", eo, "LSE", el)
    assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
    assert el["max_abs"] < BF16_TOL
    qt, kt, vt = (sta.tile_reorder(a, latent, tile) for a in (q, k, v))
    ot, lt = sta.forward(qt, kt, vt, latent, tile, wins)
    assert torch.equal(sta.tile_unreorder(ot, latent, tile).view(torch.int16), o.view(torch.int16))
    lr = sta.tile_unreorder(lt.unsqueeze(-1), latent, tile).squeeze(-1)
    assert torch.equal(lr.view(torch.int32), lse.view(torch.int32))


def test_forward_raster_padded_29x45x76(sta):
    """The pages' padding example in one launch: (29,45,76) -> (30,48,80) with
    tile (6,8,8), 24 heads, window (3,3,3).  Bit-identical to the reorder path
    over the whole tensor, and sampled raster rows against the oracle."""
    name = "hunyuan_29x45x76_w333_padded"
    w = I.WORKLOADS[name]
    latent, tile, wins, D = w["latent"], w["tile"], w["windows"], w["head_dim"]
    print(f"[raster padded] {name}", flush=True)
    x = I.workload_inputs(name)
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = sta.forward_raster(q, k, v, latent, tile, wins)
    qt, kt, vt = (sta.tile_reorder(a, latent, tile) for a in (q, k, v))
    ot, lt = sta.forward(qt, kt, vt, latent, tile, wins)
    assert torch.equal(sta.tile_unreorder(ot, latent, tile).view(torch.int16), o.view(torch.int16))
    lr = sta.tile_unreorder(lt.unsqueeze(-1), latent, tile).squeeze(-1)
    assert torch.equal(lr.view(torch.int32), lse.view(torch.int32))
    del qt, kt, vt, ot, lt
    # sampled raster rows: the oracle's tile-major rows of those tokens
    T, H, W = latent
    grid = O.padded_latent(latent, tile)
    pi = O.tile_major_index(grid, tile)
    rng = np.random.default_rng(3)
    rr = np.unique(np.concatenate([[0, T * H * W - 1, (T - 1) * H * W, H * W - 1], rng.integers(0, T * H * W, 60)]))
    tau, y, xx = rr // (H * W), (rr // W) % H, rr % W
    tm_rows = pi[(tau * grid[1] + y) * grid[2] + xx]
    rt = torch.from_numpy(rr).cuda()
    for h in (0, 23):
        hq, hk, hv = (O.pad_reorder(to64(x[nm][:, h:h + 1]), latent, tile) for nm in ("q", "k", "v"))
        ro, rl = O.forward(hq, hk, hv, latent, tile, [wins[h]], D ** -0.5, rows=tm_rows)
        eo, el = err_report(to64(o[:, h:h + 1, rt]), ro), err_report(to64(lse[:, h:h + 1, rt]), rl)
        print("head", h, "O", eo, "LSE", el)
        assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
        assert el["max_abs"] < BF16_TOL


def test_forward_raster_hunyuan_bit_identical(sta):
    """(30,48,80), tile (6,8,8), 24 heads, mixed windows: the raster instance
    equals reorder -> sta_forward -> unreorder bit for bit."""
    w = I.WORKLOADS["hunyuan_30x48x80_mixed"]
    latent, tile, wins = w["latent"], w["tile"], w["windows"]
    S = int(np.prod(latent))
    g = torch.Generator(device="cuda").manual_seed(21)
    q, k, v = (torch.randn((1, 24, S, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    o, lse = sta.forward_raster(q, k, v, latent, tile, wins)
    qt, kt, vt = (sta.tile_reorder(a, latent, tile) for a in (q, k, v))
    ot, lt = sta.forward(qt, kt, vt, latent, tile, wins)
    assert torch.equal(sta.tile_unreorder(ot, latent, tile).view(torch.int16), o.view(torch.int16))
    lr = sta.tile_unreorder(lt.unsqueeze(-1), latent, tile).squeeze(-1)
    assert torch.equal(lr.view(torch.int32), lse.view(torch.int32))


def test_forward_raster_bench_config_sampled(sta):
    """The benchmark's step itself, in its launch configuration:
    sta_forward_raster on the (30,48,80) latent, tile (6,8,8), 24 heads,
    D = 128, window (3,3,3), on the benchmark's seeded inputs.  Sampled raster
    rows (corners of the latent, tile-boundary rows and seeded random rows) of
    three heads against the oracle in raster order."""
    name = "hunyuan_30x48x80_w333"
    w = I.WORKLOADS[name]
    latent, tile, wins, D = w["latent"], w["tile"], w["windows"], w["head_dim"]
    T, H, W = latent
    S = T * H * W
    print(f"[raster bench config] {name}", flush=True)
    x = I.workload_inputs(name)
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = sta.forward_raster(q, k, v, latent, tile, wins)
    torch.cuda.synchronize()
    corners = [((a * H) + b) * W + c for a in (0, T - 1) for b in (0, H - 1) for c in (0, W - 1)]
    edges = [((5 * H) + 7) * W + 8, ((6 * H) + 8) * W + 7, ((17 * H) + 23) * W + 40]   # tile borders
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([corners, edges, rng.integers(0, S, 120)]))
    rt = torch.from_numpy(rows).cuda()
    for h in (0, 12, 23):
        ro, rl = O.forward(*(to64(x[nm][:, h:h + 1]) for nm in ("q", "k", "v")), latent, tile, [wins[h]],
                           D ** -0.5, order="raster", rows=rows)
        eo, el = err_report(to64(o[:, h:h + 1, rt]), ro), err_report(to64(lse[:, h:h + 1, rt]), rl)
        print("head", h, "O", eo, "LSE", el)
        assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
        assert el["max_abs"] < BF16_TOL


BF16_SMALL = [  # latent, tile, B, windows, D   (tile volume 32 and 128; several tiles; batch 2)
    ((6, 16, 16), (2, 4, 4), 2, [(3, 3, 3), (1, 2, 5), (9, 9, 9)], 128),
    ((6, 16, 16), (2, 4, 4), 1, [(2, 3, 1), (3, 1, 3)], 64),
    ((6, 32, 32), (2, 8, 8), 2, [(3, 3, 3), (1, 1, 1), (3, 2, 4)], 128),
    ((12, 16, 24), (6, 8, 8), 1, [(1, 3, 3), (2, 2, 2)], 128),        # L = 384
    ((6, 32, 32), (2, 8, 8), 1, [(3, 3, 3), (1, 4, 2)], 64),
    ((1, 32, 40), (1, 8, 8), 2, [(1, 3, 3), (1, 1, 5), (1, 9, 9)], 128),   # 2D, L = 64
    ((1, 24, 40), (1, 8, 8), 1, [(1, 3, 3), (2, 2, 2)], 64),               # 2D, L = 64, D = 64
    ((5, 15, 13), (2, 4, 4), 2, [(3, 3, 3), (2, 1, 4)], 128),              # padded to (6, 16, 16)
    ((11, 30, 29), (2, 8, 8), 1, [(3, 3, 3), (1, 2, 4)], 128),             # padded, L = 128
    ((5, 16, 20), (1, 8, 8), 1, [(3, 3, 3)], 64),                          # padded, L = 64
]


@pytest.mark.parametrize("latent,tile,B,wins,D", BF16_SMALL)
def test_forward_bf16_small(sta, latent, tile, B, wins, D):
    S = int(np.prod(latent))
    x = I.make_inputs(B, len(wins), S, D, "bf16", seed=5)
    scale = D ** -0.5
    q, k, v = (_tile_major(sta, x[n], latent, tile) for n in ("q", "k", "v"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    rq, rk, rv = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v"))
    ro, rl = O.forward(rq, rk, rv, latent, tile, wins, scale)
    eo, el = err_report(to64(o), ro), err_report(to64(lse), rl)
    print("O", eo, "LSE", el)
    assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
    assert el["max_abs"] < BF16_TOL


def test_forward_bf16_zero_query_window_mean(sta):
    """Q = 0: every output row is the plain mean of V over its window, which
    pins window membership far more tightly than the 2e-2 tolerance."""
    latent, tile, wins = (6, 32, 32), (2, 8, 8), [(3, 3, 3), (1, 2, 4)]
    S = int(np.prod(latent))
    x = I.make_inputs(1, 2, S, 128, "bf16", seed=6)
    q = torch.zeros((1, 2, S, 128), dtype=torch.bfloat16, device="cuda")
    k, v = (_tile_major(sta, x[n], latent, tile) for n in ("k", "v"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=0.088)
    rk, rv = (O.reorder(to64(x[n]), latent, tile) for n in ("k", "v"))
    ro, rl = O.forward(np.zeros((1, 2, S, 128)), rk, rv, latent, tile, wins, 0.088)
    e = err_report(to64(o), ro)
    print(e)
    assert e["max_abs"] < 4e-3
    assert err_report(to64(lse), rl)["max_abs"] < 1e-4


def _check_sampled(sta, name, heads, rows_per_tile=32, seed=0):
    w = I.WORKLOADS[name]
    latent, tile, wins, D = w["latent"], w["tile"], w["windows"], w["head_dim"]
    n, L = O.tile_grid(O.padded_latent(latent, tile), tile)
    x = I.workload_inputs(name)
    scale = D ** -0.5
    q, k, v = (_tile_major(sta, x[nm], latent, tile) for nm in ("q", "k", "v"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    torch.cuda.synchronize()
    tiles = sample_query_tiles(n, 1, seed)
    rows = np.concatenate([np.r_[a * L:a * L + rows_per_tile // 2, (a + 1) * L - rows_per_tile // 2:(a + 1) * L]
                           for a in tiles])
    rt = torch.from_numpy(rows).cuda()
    worst = {}
    for h in heads:
        hq, hk, hv = (O.pad_reorder(to64(x[nm][:, h:h + 1]), latent, tile) for nm in ("q", "k", "v"))
        ro, rl = O.forward(hq, hk, hv, latent, tile, [wins[h]], scale, rows=rows)
        eo = err_report(to64(o[:, h:h + 1, rt]), ro)
        el = err_report(to64(lse[:, h:h + 1, rt]), rl)
        print(name, "head", h, wins[h], "O", eo, "LSE", el)
        assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
        assert el["max_abs"] < BF16_TOL
        worst[h] = eo
    return worst


def test_forward_bf16_hunyuan_uniform_sampled(sta):
    _check_sampled(sta, "hunyuan_30x48x80_w333", heads=[0, 11, 23])


def test_forward_bf16_hunyuan_mixed_sampled(sta):
    wins = I.WORKLOADS["hunyuan_30x48x80_mixed"]["windows"]
    heads = sorted({wins.index(wd) for wd in set(wins)})   # one head of every window kind drawn
    _check_sampled(sta, "hunyuan_30x48x80_mixed", heads=heads, rows_per_tile=16)


def test_forward_bf16_wan_sampled(sta):
    _check_sampled(sta, "wan_24x48x80_w335", heads=[0, 39])


def test_forward_bf16_image_2d_sampled(sta):
    _check_sampled(sta, "image_2d_1x128x128_w155", heads=[0, 23])


def test_forward_bf16_padded_29x45x76_sampled(sta):
    """The pages' padding example: a (29,45,76) latent padded to (30,48,80).
    The sampled tiles include the last tile, whose tail rows are padding."""
    _check_sampled(sta, "hunyuan_29x45x76_w333_padded", heads=[0, 23])


def test_forward_backward_f32_padded(sta):
    """fp32 debug instance on a padded latent at 1e-5, forward and backward."""
    latent, tile, wins, scale = (5, 15, 13), (2, 4, 4), [(3, 3, 3), (2, 1, 4)], 0.2
    x = I.make_inputs(1, 2, 5 * 15 * 13, 32, "f32", seed=11, with_do=True)
    q, k, v, do = (_tile_major(sta, x[n], latent, tile) for n in ("q", "k", "v", "do"))
    o, lse = sta.forward(q, k, v, latent, tile, wins, scale=scale)
    dq, dk, dv = sta.backward(q, k, v, o, do, lse, latent, tile, wins, scale=scale)
    rq, rk, rv, rdo = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v", "do"))
    ro, rl = O.forward(rq, rk, rv, latent, tile, wins, scale)
    assert err_report(to64(o), ro)["max_abs"] < F32_TOL
    assert err_report(to64(lse), rl)["max_abs"] < F32_TOL
    for got, r in zip((dq, dk, dv), O.backward(rq, rk, rv, rdo, latent, tile, wins, scale)):
        assert err_report(to64(got), r)["max_abs"] < F32_TOL
    back = sta.tile_unreorder(o, latent, tile)
    assert np.array_equal(bits(back), O.pad_unreorder(bits(o), latent, tile))


# ------------------------------------------------------------------ dense

def test_dense_bf16_small(sta):
    x = I.make_inputs(1, 2, 1536, 128, "bf16", seed=7)
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = sta.dense_forward(q, k, v, scale=128 ** -0.5)
    ro, rl = O.dense_forward(to64(x["q"]), to64(x["k"]), to64(x["v"]), 128 ** -0.5)
    eo = err_report(to64(o), ro)
    assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
    assert err_report(to64(lse), rl)["max_abs"] < BF16_TOL


def test_dense_f32_small(sta):
    x = I.make_inputs(1, 2, 640, 64, "f32", seed=8)
    q, k, v = (_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = sta.dense_forward(q, k, v, scale=0.125)
    ro, rl = O.dense_forward(to64(x["q"]), to64(x["k"]), to64(x["v"]), 0.125)
    assert err_report(to64(o), ro)["max_abs"] < F32_TOL
    assert err_report(to64(lse), rl)["max_abs"] < F32_TOL


def test_forward_bf16_finetune_sampled(sta):
    """The fine-tuning shape (24,64,64), tile (6,8,8), window (3,5,5): forward
    O and LSE on sampled query tiles (its backward is checked elsewhere)."""
    _check_sampled(sta, "finetune_24x64x64_w355", heads=[0, 23])


def test_dense_bf16_hunyuan_sampled(sta):
    """Dense attention (the speedup denominator) at the HunyuanVideo sequence
    length S = 115200, 2 heads, on sampled rows against all keys."""
    S = 30 * 48 * 80
    g = torch.Generator(device="cuda").manual_seed(31)
    q, k, v = (torch.randn((1, 2, S, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    o, lse = sta.dense_forward(q, k, v, scale=128 ** -0.5)
    rows = np.concatenate([np.arange(0, 48), np.arange(S // 2, S // 2 + 48), np.arange(S - 48, S)])
    rt = torch.from_numpy(rows).cuda()
    ro, rl = O.dense_forward(to64(q), to64(k), to64(v), 128 ** -0.5, rows=rows)
    eo, el = err_report(to64(o[:, :, rt]), ro), err_report(to64(lse[:, :, rt]), rl)
    print("dense O", eo, "LSE", el)
    assert eo["max_abs"] < BF16_TOL and eo["rel_rms"] < BF16_REL_RMS
    assert el["max_abs"] < BF16_TOL
