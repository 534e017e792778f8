"""Plain CPU oracle for Sliding Tile Attention (STA), in float64 numpy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library; the two meet only through the seeded input
generators, which hold none of the method's arithmetic.

Sources (web pages, cited by title and section):
  [STA-abs]  "Sliding Tile Attention" (arXiv 2502.04507), abstract as printed on
             the gptget.net summary page: attention over a local 3D window,
             taken tile by tile instead of token by token.
  [STA-meth] same page, sections on the core innovation and method details:
             the latent is cut into non-overlapping space-time tiles, each
             (query tile, key tile) block is fully dense (no mixed blocks),
             and every head has its own window size.
  [STA-rebut] "Fast Video Generation with Sliding Tile Attention", OpenReview
             rebuttal, answer on input resolution: tile (6,8,8); the latent must
             be a whole number of tiles in every dimension.

What the oracle computes is the plain definition the method reaches exactly:
full softmax attention whose mask admits key token j for query token i iff the
tile holding j lies in the window of the tile holding i.  Readings taken where
the pages are silent:
  * raster order of the latent is (T, H, W) with W fastest;
  * tile-major order: tiles in raster order over the tile grid, tokens in raster
    order inside a tile;
  * window per dimension: w' = min(w, n); the window of query tile q starts at
    clamp(q - floor(w'/2), 0, n - w') and spans w' tiles (the centre is clamped
    so the window stays inside the tile grid; for even w' the extra tile falls
    on the low side);
  * windows are counted in tiles; a window < 1 is an error;
  * the log-sum-exp uses the natural logarithm;
  * the per-head window search ([STA-meth]: each head gets its own window,
    chosen automatically) is measured by the attention mass a candidate window
    keeps: the share of a head's full (unmasked) softmax probability whose keys
    lie in the window, averaged over the real queries.  How a window is then
    picked from these numbers needs the model and is not part of the oracle;
  * a latent that is not a whole number of tiles is handled as [STA-rebut]'s
    "padding with masking": it is padded up to the next tile multiple in each
    dimension, windows live on the padded tile grid, padding tokens are never
    keys, and the rows of padding tokens are outputs of no real token (O, LSE
    and all gradients are zero there).
Every function here is pinned by ``tests/test_oracle.py`` against brute force,
closed forms, invariants and library routines.  One case is parity unpinned by
the pages: an even window narrower than the tile grid, where the pages do not
say on which side the extra tile falls; the tests pin only the reading above.
"""

import numpy as np

__all__ = [
    "tile_grid", "tile_major_index", "reorder", "unreorder", "padded_latent", "valid_positions",
    "pad_reorder", "pad_unreorder", "window_start",
    "window_contains", "tile_pairs", "token_tile_coords", "window_mask",
    "forward", "backward", "backward_key_rows", "backward_query_rows", "backward_key_rows_by_pairs",
    "dense_forward", "window_mass",
]


def tile_grid(latent, tile):
    """Tile grid n = (T/t, H/h, W/w) and tile volume L = t*h*w.

    [STA-rebut]: the latent must be an integer multiple of the tile in each of
    its three dimensions; anything else is rejected here.
    """
    latent = tuple(int(v) for v in latent)
    tile = tuple(int(v) for v in tile)
    if len(latent) != 3 or len(tile) != 3:
        raise ValueError("latent and tile are (T, H, W) triples")
    if min(latent) < 1 or min(tile) < 1:
        raise ValueError("latent and tile sizes must be positive")
    if any(a % b for a, b in zip(latent, tile)):
        raise ValueError(f"latent {latent} is not a multiple of tile {tile}")
    n = tuple(a // b for a, b in zip(latent, tile))
    return n, tile[0] * tile[1] * tile[2]


def tile_major_index(latent, tile):
    """pi[r]: position in the tile-major sequence of the raster token r.

    [STA-meth] tiling step: every tile becomes one contiguous run of the
    sequence.  Raster token r = (tau*H + y)*W + x sits in tile a = (tau//t,
    y//h, x//w) at intra-tile coordinate i = (tau%t, y%h, x%w), and goes to
    ((a0*n1 + a1)*n2 + a2)*L + (i0*h + i1)*w + i2.
    """
    (n0, n1, n2), L = tile_grid(latent, tile)
    T, H, W = latent
    t, h, w = tile
    tau, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    tile_id = ((tau // t) * n1 + (y // h)) * n2 + (x // w)
    intra = ((tau % t) * h + (y % h)) * w + (x % w)
    return (tile_id * L + intra).reshape(-1).astype(np.int64)


def reorder(x, latent, tile):
    """Raster -> tile-major along axis -2: Y[..., pi(r), :] = X[..., r, :]."""
    pi = tile_major_index(latent, tile)
    if x.shape[-2] != pi.size:
        raise ValueError("sequence axis does not match the latent")
    y = np.empty_like(x)
    y[..., pi, :] = x
    return y


def unreorder(y, latent, tile):
    """Tile-major -> raster along axis -2: X[..., r, :] = Y[..., pi(r), :]."""
    pi = tile_major_index(latent, tile)
    if y.shape[-2] != pi.size:
        raise ValueError("sequence axis does not match the latent")
    return y[..., pi, :].copy()


def padded_latent(latent, tile):
    """The smallest whole-tile latent holding ``latent``.

    [STA-rebut], answer on input resolution, "padding with masking": a latent
    such as (29, 45, 76) is padded to the tile-aligned (30, 48, 80) and the
    padding tokens are masked out of the attention.
    """
    latent = tuple(int(v) for v in latent)
    tile = tuple(int(v) for v in tile)
    if len(latent) != 3 or len(tile) != 3 or min(latent) < 1 or min(tile) < 1:
        raise ValueError("latent and tile are positive (T, H, W) triples")
    return tuple(-(-a // b) * b for a, b in zip(latent, tile))


def _raster_in_padded(latent, tile):
    """Raster index inside the padded latent of every raster token of ``latent``."""
    T, H, W = (int(v) for v in latent)
    _, P1, P2 = padded_latent(latent, tile)
    tau, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return ((tau * P1 + y) * P2 + x).reshape(-1).astype(np.int64)


def valid_positions(latent, tile, order="tile"):
    """Boolean [S_pad]: the position of the padded latent holds a real token.

    ``order`` is the order of the padded sequence: "tile" (tile-major) or
    "raster".  All true when the latent is a whole number of tiles.
    """
    P = padded_latent(latent, tile)
    v = np.zeros(P[0] * P[1] * P[2], dtype=bool)
    v[_raster_in_padded(latent, tile)] = True
    if order == "raster":
        return v
    if order != "tile":
        raise ValueError("order is 'tile' or 'raster'")
    out = np.empty_like(v)
    out[tile_major_index(P, tile)] = v
    return out


def pad_reorder(x, latent, tile):
    """Raster tokens of ``latent`` (axis -2) -> tile-major sequence of the
    padded latent; rows of padding tokens are zero."""
    P = padded_latent(latent, tile)
    idx = _raster_in_padded(latent, tile)
    if x.shape[-2] != idx.size:
        raise ValueError("sequence axis does not match the latent")
    xp = np.zeros(x.shape[:-2] + (P[0] * P[1] * P[2], x.shape[-1]), dtype=x.dtype)
    xp[..., idx, :] = x
    return reorder(xp, P, tile)


def pad_unreorder(y, latent, tile):
    """Inverse of ``pad_reorder``: the raster tokens of ``latent`` (crop)."""
    P = padded_latent(latent, tile)
    return unreorder(y, P, tile)[..., _raster_in_padded(latent, tile), :].copy()


def window_start(q, w, n):
    """First tile of the window of query tile q along one dimension, and w'.

    [STA-abs]/[STA-meth]: a query tile attends to a local window of tiles.  The
    window keeps its full size w' = min(w, n) at the grid edges: its start is
    q - floor(w'/2) clamped into [0, n - w'].
    """
    if w < 1:
        raise ValueError("window must be at least one tile")
    wp = min(int(w), int(n))
    return min(max(int(q) - wp // 2, 0), int(n) - wp), wp


def window_contains(qt, kt, win, n):
    """True iff key tile kt lies in the window of query tile qt (3D coords)."""
    for d in range(3):
        s, wp = window_start(qt[d], win[d], n[d])
        if not (s <= kt[d] < s + wp):
            return False
    return True


def _tile_coords(n):
    """Tile-grid coordinates in raster order over the grid, shape [N_t, 3]."""
    return np.stack(np.meshgrid(np.arange(n[0]), np.arange(n[1]), np.arange(n[2]),
                                indexing="ij"), axis=-1).reshape(-1, 3)


def tile_pairs(latent, tile, windows, transpose=False):
    """Canonical (query tile, key tile) list per head.

    Tiles are numbered in raster order over the tile grid.  Forward order is
    head, then query tile, then key tile; the transposed order (used by the
    backward pass, where a key tile collects the query tiles whose window holds
    it) is head, then key tile, then query tile.  Returns (pairs [P, 2] int32
    holding (q, k), offsets [Hh + 1] int64).
    """
    n, _ = tile_grid(latent, tile)
    coords = _tile_coords(n)
    out, offsets = [], [0]
    for win in np.asarray(windows).reshape(-1, 3):
        head = []
        for a, ca in enumerate(coords):
            for b, cb in enumerate(coords):
                if transpose:
                    if window_contains(cb, ca, win, n):
                        head.append((b, a))
                elif window_contains(ca, cb, win, n):
                    head.append((a, b))
        out.extend(head)
        offsets.append(offsets[-1] + len(head))
    return np.asarray(out, dtype=np.int32).reshape(-1, 2), np.asarray(offsets, dtype=np.int64)


def token_tile_coords(latent, tile, order="tile"):
    """Tile-grid coordinates [S, 3] of the tile holding each sequence position."""
    n, L = tile_grid(latent, tile)
    T, H, W = latent
    t, h, w = tile
    if order == "tile":
        return np.repeat(_tile_coords(n), L, axis=0)
    if order == "raster":
        tau, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
        return np.stack([tau // t, y // h, x // w], axis=-1).reshape(-1, 3)
    raise ValueError("order is 'tile' or 'raster'")


def window_mask(latent, tile, win, order="tile", rows=None, cols=None):
    """Boolean mask M[i, j]: key position j is visible to query position i.

    [STA-meth]: visibility is decided per tile pair, so every block of the mask
    is all-true or all-false.  ``rows`` / ``cols`` restrict the query / key
    positions.
    """
    n, _ = tile_grid(latent, tile)
    tc = token_tile_coords(latent, tile, order)
    qc = tc if rows is None else tc[np.asarray(rows)]
    kc = tc if cols is None else tc[np.asarray(cols)]
    m = np.ones((qc.shape[0], kc.shape[0]), dtype=bool)
    for d in range(3):
        # the window of every query tile coordinate along d, from window_start
        table = np.array([window_start(c, win[d], n[d]) for c in range(n[d])], dtype=np.int64)
        start, width = table[qc[:, d], 0], table[qc[:, d], 1]
        m &= (kc[None, :, d] >= start[:, None]) & (kc[None, :, d] < (start + width)[:, None])
    return m


def _check_qkv(q, k, v, windows):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, Hh, S, D] shape")
    windows = np.asarray(windows).reshape(-1, 3)
    if windows.shape[0] != q.shape[1]:
        raise ValueError("one window per head")
    return windows


def forward(q, k, v, latent, tile, windows, scale, order="tile", rows=None, chunk=256):
    """STA forward: O and LSE of masked softmax attention, float64.

    [STA-abs]: each query attends, with softmax, to every key in its tile's
    window.  For query row i: s_j = scale * <q_i, k_j> on visible j, m = max s,
    l = sum exp(s - m), O_i = sum_j exp(s_j - m) v_j / l, LSE_i = m + ln l.
    ``rows`` (query positions) limits the work to a sample of rows; the result
    then has shape [B, Hh, len(rows), D].
    """
    windows = _check_qkv(q, k, v, windows)
    grid, valid = _padding(latent, tile, order)
    B, Hh, S, D = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    o = np.zeros((B, Hh, rows.size, D))
    lse = np.zeros((B, Hh, rows.size))
    for h in range(Hh):
        for c0 in range(0, rows.size, chunk):
            r = rows[c0:c0 + chunk]
            m = window_mask(grid, tile, windows[h], order, rows=r)
            if valid is not None:
                m &= valid[None, :]
            for b in range(B):
                s = scale * (q[b, h, r] @ k[b, h].T)
                s[~m] = -np.inf
                mx = s.max(axis=1, keepdims=True)
                e = np.exp(s - mx)
                l = e.sum(axis=1, keepdims=True)
                o[b, h, c0:c0 + r.size] = (e @ v[b, h]) / l
                lse[b, h, c0:c0 + r.size] = (mx + np.log(l))[:, 0]
    if valid is not None:
        o[:, :, ~valid[rows]] = 0.0
        lse[:, :, ~valid[rows]] = 0.0
    return o, lse


def _padding(latent, tile, order):
    """The whole-tile grid latent to build windows on, and the key validity
    mask over it (None when the latent is already a whole number of tiles)."""
    grid = padded_latent(latent, tile)
    if grid == tuple(int(v) for v in latent):
        return grid, None
    if order != "tile":
        raise ValueError("a padded latent is only defined in tile-major order")
    return grid, valid_positions(latent, tile)


def backward(q, k, v, do, latent, tile, windows, scale, order="tile"):
    """Gradients (dQ, dK, dV) of the STA forward, float64, whole tensors.

    The pages give no backward formulas; this is the exact gradient of the
    forward above (softmax attention restricted to the window mask):
    P = softmax(masked S), O = P V, Dl_i = sum_d dO_id O_id,
    dP = dO V^T, dS = P * (dP - Dl), dQ = scale dS K, dK = scale dS^T Q,
    dV = P^T dO.  Meant for small grids (it forms the S x S matrices).
    """
    windows = _check_qkv(q, k, v, windows)
    grid, valid = _padding(latent, tile, order)
    B, Hh, S, D = q.shape
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(Hh):
        m = window_mask(grid, tile, windows[h], order)
        if valid is not None:
            m &= valid[None, :]
        for b in range(B):
            s = scale * (q[b, h] @ k[b, h].T)
            s[~m] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            if valid is not None:
                p[~valid] = 0.0     # rows of padding tokens belong to no real query
            o = p @ v[b, h]
            dl = (do[b, h] * o).sum(axis=1, keepdims=True)
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - dl)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
            dv[b, h] = p.T @ do[b, h]
    return dq, dk, dv


def backward_key_rows(q, k, v, do, latent, tile, win, scale, b, h, key_rows, order="tile"):
    """dK and dV of one (batch b, head h) at the key positions ``key_rows``.

    Same formulas as ``backward``, evaluated only where needed: the query rows
    that can see any of the sampled keys are found from the mask, their full
    softmax rows (over every visible key) give P, and the sampled columns of
    dS give dK_j = scale sum_i dS_ij q_i and dV_j = sum_i P_ij dO_i.
    """
    key_rows = np.asarray(key_rows)
    grid, valid = _padding(latent, tile, order)
    qf, kf, vf, dof = (np.asarray(a[b, h], dtype=np.float64) for a in (q, k, v, do))
    qi = np.nonzero(window_mask(grid, tile, win, order, cols=key_rows).any(axis=1))[0]
    if valid is not None:
        qi = qi[valid[qi]]              # padding rows are no query
    dk = np.zeros((key_rows.size, qf.shape[1]))
    dv = np.zeros_like(dk)
    for c0 in range(0, qi.size, 512):
        r = qi[c0:c0 + 512]
        m = window_mask(grid, tile, win, order, rows=r)
        if valid is not None:
            m &= valid[None, :]
        s = scale * (qf[r] @ kf.T)
        s[~m] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ vf
        dl = (dof[r] * o).sum(axis=1, keepdims=True)
        pj = p[:, key_rows]
        ds = pj * (dof[r] @ vf[key_rows].T - dl)
        dk += scale * (ds.T @ qf[r])
        dv += pj.T @ dof[r]
    if valid is not None:
        dk[~valid[key_rows]] = 0.0
        dv[~valid[key_rows]] = 0.0
    return dk, dv


def backward_key_rows_by_pairs(q, k, v, do, latent, tile, win, scale, b, h, key_rows):
    """dK and dV of one (batch b, head h) at tile-major key positions
    ``key_rows``, written tile pair by tile pair.

    [STA-meth]: each query tile attends densely to the key tiles of its
    window.  This is the same gradient as ``backward``, organised the way the
    method states it instead of as a masked dense matrix: for every query tile
    a whose window holds a tile of the sampled keys, the keys of a's window
    (its tiles, real positions only) give P = softmax(scale Q_a K_win^T),
    O = P V_win and Dl = rowsum(dO_a * O); the sampled key columns j then get
    dS_ij = P_ij (<dO_i, v_j> - Dl_i), dK_j += scale sum_i dS_ij q_i and
    dV_j += sum_i P_ij dO_i.  Only the keys a query sees enter its softmax, so
    the cost follows the window instead of the sequence (full-size samples of
    the heaviest key tiles stay cheap).  fp64 torch CPU ops (multi-threaded).
    """
    import torch
    grid = padded_latent(latent, tile)
    n, L = tile_grid(grid, tile)
    nt = n[0] * n[1] * n[2]
    valid = valid_positions(latent, tile)
    key_rows = np.asarray(key_rows, dtype=np.int64)
    coords = _tile_coords(n)
    win = tuple(int(x) for x in win)
    # per query tile: the key tiles of its window
    windows = [[t for t in range(nt) if window_contains(coords[a], coords[t], win, n)] for a in range(nt)]
    ktiles = set(int(t) for t in np.unique(key_rows // L))
    qf, kf, vf, dof = (torch.from_numpy(np.ascontiguousarray(a[b, h], dtype=np.float64)) for a in (q, k, v, do))
    dk = torch.zeros((key_rows.size, qf.shape[1]), dtype=torch.float64)
    dv = torch.zeros_like(dk)
    pos = np.full(grid[0] * grid[1] * grid[2], -1, dtype=np.int64)
    for a in range(nt):
        if not ktiles.intersection(windows[a]):
            continue
        rows = np.arange(a * L, (a + 1) * L)
        rows = rows[valid[rows]]                  # padding positions are no query
        if rows.size == 0:
            continue
        cols = np.concatenate([np.arange(t * L, (t + 1) * L) for t in windows[a]])
        cols = cols[valid[cols]]                  # ... and no key
        pos[:] = -1
        pos[cols] = np.arange(cols.size)
        sel = np.flatnonzero(pos[key_rows] >= 0)  # sampled keys this query tile sees
        if sel.size == 0:
            continue
        rt, ct = torch.from_numpy(rows), torch.from_numpy(cols)
        qa, doa = qf[rt], dof[rt]
        p = torch.softmax(scale * (qa @ kf[ct].T), dim=1)
        o = p @ vf[ct]
        dl = (doa * o).sum(dim=1, keepdim=True)
        jt = torch.from_numpy(key_rows[sel])
        pj = p[:, torch.from_numpy(pos[key_rows[sel]])]
        ds = pj * (doa @ vf[jt].T - dl)
        st = torch.from_numpy(sel)
        dk[st] += scale * (ds.T @ qa)
        dv[st] += pj.T @ doa
    out_dk, out_dv = dk.numpy(), dv.numpy()
    out_dk[~valid[key_rows]] = 0.0
    out_dv[~valid[key_rows]] = 0.0
    return out_dk, out_dv


def backward_query_rows(q, k, v, do, latent, tile, win, scale, b, h, rows, order="tile"):
    """dQ of one (batch b, head h) at the query positions ``rows``.

    Same formulas as ``backward``, row by row: each sampled query's softmax row
    over its visible keys gives P_i and O_i, then Dl_i = <dO_i, O_i>,
    dS_ij = P_ij (<dO_i, v_j> - Dl_i) and dQ_i = scale sum_j dS_ij k_j.
    """
    rows = np.asarray(rows)
    grid, valid = _padding(latent, tile, order)
    qf, kf, vf, dof = (np.asarray(a[b, h], dtype=np.float64) for a in (q, k, v, do))
    out = np.zeros((rows.size, qf.shape[1]))
    for c0 in range(0, rows.size, 256):
        r = rows[c0:c0 + 256]
        m = window_mask(grid, tile, win, order, rows=r)
        if valid is not None:
            m &= valid[None, :]
        s = scale * (qf[r] @ kf.T)
        s[~m] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ vf
        dl = (dof[r] * o).sum(axis=1, keepdims=True)
        ds = p * (dof[r] @ vf.T - dl)
        out[c0:c0 + r.size] = scale * (ds @ kf)
    if valid is not None:
        out[~valid[rows]] = 0.0
    return out


def dense_forward(q, k, v, scale, rows=None, chunk=256):
    """Full (unmasked) softmax attention, O and LSE, float64: the denominator
    the method is compared with ([STA-abs] compares against FlashAttention)."""
    B, Hh, S, D = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    o = np.zeros((B, Hh, rows.size, D))
    lse = np.zeros((B, Hh, rows.size))
    for b in range(B):
        for h in range(Hh):
            for c0 in range(0, rows.size, chunk):
                r = rows[c0:c0 + chunk]
                s = scale * (q[b, h, r] @ k[b, h].T)
                mx = s.max(axis=1, keepdims=True)
                e = np.exp(s - mx)
                l = e.sum(axis=1, keepdims=True)
                o[b, h, c0:c0 + r.size] = (e @ v[b, h]) / l
                lse[b, h, c0:c0 + r.size] = (mx + np.log(l))[:, 0]
    return o, lse


def window_mass(q, k, latent, tile, candidates, scale, order="tile", chunk=256):
    """Attention mass of candidate windows, per head, float64.

    [STA-abs]: attention in pretrained video models concentrates in local 3D
    windows; [STA-meth]: the window is configured per head.  The quantity that
    compares candidate windows of one head is the share of its full attention
    that a window keeps.  For query row i of (batch b, head h):
      P_ij = exp(s_ij) / sum_j' exp(s_ij'),  s_ij = scale * <q_i, k_j>,
    over every real key j (no window), and
      mass_i(w) = sum of P_ij over the keys j whose tile lies in window w of
                  the tile of i.
    Returns mass[c, b, h] = mean of mass_i(candidates[c]) over the real query
    rows of (b, h).  On a padded latent, padding positions are neither keys nor
    queries.
    """
    grid, valid = _padding(latent, tile, order)
    B, Hh, S, D = q.shape
    if k.shape != q.shape:
        raise ValueError("q and k must share one [B, Hh, S, D] shape")
    cands = np.asarray(candidates).reshape(-1, 3)
    if cands.shape[0] < 1:
        raise ValueError("at least one candidate window")
    q, k = (np.asarray(a, dtype=np.float64) for a in (q, k))
    real = np.ones(S, dtype=bool) if valid is None else valid
    rows_all = np.flatnonzero(real)
    total = np.zeros((cands.shape[0], B, Hh))
    for c0 in range(0, rows_all.size, chunk):
        r = rows_all[c0:c0 + chunk]
        masks = [window_mask(grid, tile, cands[c], order, rows=r) & real[None, :]
                 for c in range(cands.shape[0])]
        for b in range(B):
            for h in range(Hh):
                s = scale * (q[b, h, r] @ k[b, h].T)
                s[:, ~real] = -np.inf
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                for c, m in enumerate(masks):
                    total[c, b, h] += p[m].sum()
    return total / rows_all.size
