"""GPU parity of the window-mass measurement (the measurement side of the
per-head window search) against the fp64 CPU oracle, through the C-ABI."""
import numpy as np
import pytest
import torch

import oracle as O
from _helpers import sample_query_tiles, to64
from sparse_sliding_tile_amd import inputs as I

pytestmark = pytest.mark.gpu

# Tolerances (max-abs on masses in [0, 1], and on natural-log LSE values).
# Both sides see the same bf16 (or fp32) inputs exactly.  The GPU forms each
# score with fp32 accumulation over D products (relative error ~ D * 2^-24 of
# sum |q_d k_d|, below 1e-5 in the exponent here) and sums fp32 exponentials,
# so per-row LSE errors stay near 1e-5 and masses, exp of an LSE difference,
# near 1e-5 relative.  The bounds leave a factor of ten.
F32_TOL = 1e-5
BF16_TOL = 1e-4
LSE_TOL = 1e-4


@pytest.fixture(scope="module")
def sta():
    import sparse_sliding_tile_amd as s
    s.lib()
    return s


CASES = [
    ((6, 16, 16), (2, 4, 4), 1, 2, 64, "f32", [(1, 1, 1), (3, 3, 3), (1, 2, 3), (9, 9, 9)]),
    ((6, 16, 32), (2, 4, 8), 2, 2, 128, "bf16", [(1, 1, 1), (3, 3, 3), (1, 2, 3), (3, 4, 4)]),
    ((6, 16, 16), (2, 4, 4), 1, 3, 64, "bf16", [(3, 3, 3), (2, 1, 4), (3, 4, 4)]),
    ((5, 13, 14), (2, 4, 4), 1, 2, 128, "bf16", [(1, 1, 1), (2, 2, 2), (3, 4, 4)]),   # padded to (6, 16, 16)
    ((5, 13, 14), (2, 4, 4), 1, 2, 64, "f32", [(1, 2, 1), (3, 4, 4)]),                # padded, fp32
    ((3, 12, 13), (2, 8, 8), 1, 2, 128, "bf16", [(1, 1, 1), (2, 2, 2), (1, 2, 2)]),   # padded, 8-wide tiles
    ((1, 40, 48), (1, 8, 8), 1, 2, 128, "bf16", [(1, 3, 3), (1, 5, 5), (1, 1, 1)]),   # 2D, 64-token tiles
]


@pytest.mark.parametrize("latent,tile,B,Hh,D,dt,cands", CASES)
def test_window_mass_matches_oracle(sta, latent, tile, B, Hh, D, dt, cands):
    S = int(np.prod(latent))
    x = I.make_inputs(B, Hh, S, D, dt, seed=11)
    q, k = (sta.tile_reorder(x[n].to("cuda"), latent, tile) for n in ("q", "k"))
    got = to64(sta.window_mass(q, k, latent, tile, cands))
    rq, rk = (O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k"))
    ref = O.window_mass(rq, rk, latent, tile, cands, D ** -0.5)
    assert got.shape == ref.shape
    err = float(np.abs(got - ref).max())
    print(f"{latent} {dt}: max-abs {err:.2e}")
    assert err < (F32_TOL if dt == "f32" else BF16_TOL)


def test_window_mass_hunyuan_shape_sampled_and_closed_forms(sta):
    """HunyuanVideo latent (30, 48, 80), tile (6, 8, 8), 4 heads, bf16, the five
    candidate windows of the mixed-window workload plus (1, 1, 1).
    - Per-row statistics left in the workspace (full and last-candidate LSE)
      match the oracle on sampled query tiles;
    - the full-grid candidate keeps mass 1; nested windows keep more mass;
    - with Q = 0 every window keeps exactly its share of keys, K L / S."""
    latent, tile, Hh, D = (30, 48, 80), (6, 8, 8), 4, 128
    cands = [(5, 6, 10), (3, 3, 3), (3, 3, 5), (5, 3, 3), (1, 6, 10), (1, 1, 1)]
    S = int(np.prod(latent))
    x = I.make_inputs(1, Hh, S, D, "bf16", seed=12)
    q, k = (sta.tile_reorder(x[n].to("cuda"), latent, tile) for n in ("q", "k"))
    ws = torch.empty(sta.window_mass_workspace_bytes(1, Hh, latent, tile, len(cands)), dtype=torch.uint8,
                     device="cuda")
    mass = to64(sta.window_mass(q, k, latent, tile, cands, workspace=ws))[:, 0, :]
    torch.cuda.synchronize()
    lse = ws.view(torch.float32)[:2 * Hh * S].view(2, 1, Hh, S)
    lse_full, lse_last = to64(lse[0]), to64(lse[1])
    assert np.abs(mass[0] - 1.0).max() < 1e-6
    assert np.all(mass[5] < mass[1]) and np.all(mass[1] < mass[2]) and np.all(mass[1] < mass[3])
    assert np.all(mass[2] < mass[0]) and np.all(mass[4] < mass[0])
    n, L = O.tile_grid(latent, tile)
    rows = np.concatenate([np.arange(t * L, t * L + L, 37) for t in sample_query_tiles(n, 2, seed=5)])
    scale = D ** -0.5
    for h in range(Hh):
        rq, rk = (O.reorder(to64(x[nm][:, h:h + 1]), latent, tile) for nm in ("q", "k"))
        _, lf = O.dense_forward(rq, rk, rk, scale, rows=rows)
        _, lw = O.forward(rq, rk, rk, latent, tile, [cands[-1]], scale, rows=rows)
        e_full = np.abs(lse_full[0, h, rows] - lf[0, 0]).max()
        e_last = np.abs(lse_last[0, h, rows] - lw[0, 0]).max()
        e_mass = np.abs(np.exp(lse_last[0, h, rows] - lse_full[0, h, rows]) - np.exp(lw[0, 0] - lf[0, 0])).max()
        print(f"head {h}: LSE full {e_full:.2e}, LSE (1,1,1) {e_last:.2e}, row mass {e_mass:.2e}")
        assert e_full < LSE_TOL and e_last < LSE_TOL and e_mass < BF16_TOL
    # Q = 0: uniform attention over all keys, the window keeps K * L / S.
    z = torch.zeros_like(q)
    m0 = to64(sta.window_mass(z, k, latent, tile, cands, workspace=ws))[:, 0, :]
    share = np.array([np.prod([min(w, m) for w, m in zip(c, n)]) * L / S for c in cands])
    assert np.abs(m0 - share[:, None]).max() < 1e-5


def test_calibration_loop_closed_form(sta):
    """The matrix-core calibration loop (libsta_calib.so, benchmark support) on
    all-ones bf16 operands: each of the four accumulator chains takes 4 MFMAs
    of 16 ones per iteration, so every thread's sum over its 4 x 16
    accumulator elements is 4096 * iters."""
    from sparse_sliding_tile_amd import calib
    ops = torch.ones(1 << 12, dtype=torch.bfloat16, device="cuda")
    out, flop = calib.calib_mfma_bf16(ops, 10, 8)
    torch.cuda.synchronize()
    assert flop == 8 * 4 * 10 * 16 * 32768
    assert torch.equal(out, torch.full_like(out, 4096.0 * 10))
    zeros = torch.zeros(1 << 12, dtype=torch.bfloat16, device="cuda")
    out0, _ = calib.calib_mfma_bf16(zeros, 10, 8)
    torch.cuda.synchronize()
    assert not out0.any()
