"""sta_backward_noalloc (static scratch, no allocation) against sta_backward
(caller workspace) through the C-ABI: the same kernels on the same inputs, so
the gradients must be bit-identical; and within the bf16 tolerance of the fp64
oracle.  Two calls in a row, the second on a smaller input, so the second
call runs on scratch the first one filled."""
import numpy as np
import pytest
import torch

import oracle as O
from _helpers import err_report, to64
from sparse_sliding_tile_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = [  # latent, tile, B, windows, D: a larger case, then a smaller padded one
    ((6, 32, 32), (2, 8, 8), 2, [(3, 3, 3), (1, 2, 4)], 128),
    ((5, 15, 13), (2, 4, 4), 1, [(3, 3, 3), (2, 1, 3)], 64),
]


def test_backward_noalloc_matches_workspace_entry_point():
    import sparse_sliding_tile_amd as sta
    sta.lib()
    for latent, tile, B, wins, D in CASES:
        print(f"[noalloc] {latent} {tile} B={B} D={D}", flush=True)
        S = int(np.prod(latent))
        x = I.make_inputs(B, len(wins), S, D, "bf16", seed=31, with_do=True)
        q, k, v, do = (sta.tile_reorder(x[n].to("cuda").contiguous(), latent, tile) for n in ("q", "k", "v", "do"))
        o, lse = sta.forward(q, k, v, latent, tile, wins)
        ref = sta.backward(q, k, v, o, do, lse, latent, tile, wins)
        got = sta.backward_noalloc(q, k, v, o, do, lse, latent, tile, wins)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        oref = O.backward(*(O.pad_reorder(to64(x[n]), latent, tile) for n in ("q", "k", "v", "do")),
                          latent, tile, wins, D ** -0.5)
        for name, a, r in zip(("dq", "dk", "dv"), got, oref):
            e = err_report(to64(a), r)
            print(name, e)
            assert e["max_abs"] < 2e-2 and e["rel_rms"] < 1e-2, name
