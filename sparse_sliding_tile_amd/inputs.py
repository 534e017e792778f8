"""Seeded synthetic inputs for Sliding Tile Attention workloads.

This module only draws random numbers and names workload shapes; it holds none
of the attention arithmetic, so both the HIP path's tests/benchmark and the CPU
oracle can take their inputs from it.

Recipe: one ``torch.Generator('cpu')`` seeded with ``seed`` draws Q, K, V and
then dO, each ``randn`` in float32 shaped [B, Hh, S, D] in raster token order
(T, H, W with W fastest).  Tensors of bfloat16 workloads are then rounded to
nearest-even bfloat16; the oracle consumes those rounded values.
"""

import numpy as np
import torch

# Window choices for the mixed per-head workload, in tiles (T, H, W).
MIXED_WINDOW_SET = ((5, 6, 10), (3, 3, 3), (3, 3, 5), (5, 3, 3), (1, 6, 10))


def mixed_windows(heads, seed=0):
    """Per-head windows drawn from MIXED_WINDOW_SET by numpy's default_rng(seed)."""
    idx = np.random.default_rng(seed).integers(0, len(MIXED_WINDOW_SET), size=heads)
    return [MIXED_WINDOW_SET[i] for i in idx]


# Named workloads.  Shapes follow the pages: HunyuanVideo 720P 5 s latent
# (30,48,80), Wan-sized latents, tile (6,8,8).
WORKLOADS = {
    "tiny_f32": dict(latent=(6, 16, 16), tile=(2, 4, 4), batch=1, heads=2, head_dim=64,
                     dtype="f32", windows=[(3, 3, 3)] * 2),
    "hunyuan_30x48x80_w333": dict(latent=(30, 48, 80), tile=(6, 8, 8), batch=1, heads=24,
                                  head_dim=128, dtype="bf16", windows=[(3, 3, 3)] * 24),
    "hunyuan_30x48x80_mixed": dict(latent=(30, 48, 80), tile=(6, 8, 8), batch=1, heads=24,
                                   head_dim=128, dtype="bf16", windows=mixed_windows(24, 0)),
    "wan_24x48x80_w335": dict(latent=(24, 48, 80), tile=(6, 8, 8), batch=1, heads=40,
                              head_dim=128, dtype="bf16", windows=[(3, 3, 5)] * 40),
    "finetune_24x64x64_w355": dict(latent=(24, 64, 64), tile=(6, 8, 8), batch=1, heads=24,
                                   head_dim=128, dtype="bf16", windows=[(3, 5, 5)] * 24),
    # Padding with masking, the pages' example: (29, 45, 76) padded to (30, 48, 80).
    "hunyuan_29x45x76_w333_padded": dict(latent=(29, 45, 76), tile=(6, 8, 8), batch=1, heads=24,
                                         head_dim=128, dtype="bf16", windows=[(3, 3, 3)] * 24),
    # 2D STA (T = 1, an image latent): 128 x 128 tokens, tile (1, 8, 8) = 64
    # tokens, window 5 x 5 tiles.
    "image_2d_1x128x128_w155": dict(latent=(1, 128, 128), tile=(1, 8, 8), batch=1, heads=24,
                                    head_dim=128, dtype="bf16", windows=[(1, 5, 5)] * 24),
}


def make_inputs(batch, heads, seq, head_dim, dtype="bf16", seed=0, with_do=False):
    """Q, K, V (and dO) as CPU tensors [B, Hh, S, D], drawn in that order."""
    g = torch.Generator("cpu").manual_seed(seed)
    names = ("q", "k", "v", "do") if with_do else ("q", "k", "v")
    out = {}
    for n in names:
        x = torch.randn((batch, heads, seq, head_dim), generator=g, dtype=torch.float32)
        out[n] = x.to(torch.bfloat16) if dtype == "bf16" else x
    return out


def workload_inputs(name, seed=0, with_do=False):
    w = WORKLOADS[name]
    T, H, W = w["latent"]
    return make_inputs(w["batch"], w["heads"], T * H * W, w["head_dim"], w["dtype"], seed, with_do)
