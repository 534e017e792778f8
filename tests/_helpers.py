"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""
import numpy as np
import torch


def to64(t):
    """Device or host tensor -> float64 numpy array (exact for bf16 and fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t):
    """Raw bit pattern of a bf16 or fp32 tensor as a numpy integer array."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def err_report(got, ref):
    """Max-abs error, relative RMS error and max-abs relative to max |ref|."""
    d = got - ref
    mx = float(np.abs(d).max()) if d.size else 0.0
    rms = float(np.sqrt((d ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    return {"max_abs": mx, "rel_rms": rms, "max_rel_to_max": mx / max(float(np.abs(ref).max()), 1e-300)}


def sample_query_tiles(n, count_interior=1, seed=0):
    """The 8 corner tiles of an n0 x n1 x n2 tile grid plus seeded interior tiles
    (raster tile numbers)."""
    n0, n1, n2 = n
    corners = {((a * n1) + b) * n2 + c for a in (0, n0 - 1) for b in (0, n1 - 1) for c in (0, n2 - 1)}
    rng = np.random.default_rng(seed)
    extra = set()
    while len(extra) < count_interior:
        t = int(rng.integers(n0 * n1 * n2))
        if t not in corners:
            extra.add(t)
    return sorted(corners | extra)
