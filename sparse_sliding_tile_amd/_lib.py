"""ctypes binding of libsta (include/sta.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libsta.so.  torch supplies device memory and the current stream.
There is no fallback: without the built library every call raises.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsta.so")

STA_BF16 = 0
STA_F32 = 1
STA_MAX_HEADS = 256

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class Dim3(ctypes.Structure):
    _fields_ = [("t", c_i32), ("h", c_i32), ("w", c_i32)]


# name -> (restype, argtypes); mirrors include/sta.h
SIGNATURES = {
    "sta_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "sta_tile_reorder": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, Dim3, Dim3, ctypes.c_int, c_vp]),
    "sta_tile_unreorder": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, Dim3, Dim3, ctypes.c_int, c_vp]),
    "sta_tile_pairs_count": (c_i64, [Dim3, Dim3, c_vp, c_i64, ctypes.c_int]),
    "sta_tile_pairs": (ctypes.c_int, [c_vp, c_vp, Dim3, Dim3, c_vp, c_i64, ctypes.c_int, c_vp]),
    "sta_tile_pairs_host": (ctypes.c_int, [c_vp, c_vp, Dim3, Dim3, c_vp, c_i64, ctypes.c_int]),
    "sta_forward": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, Dim3, Dim3, c_vp,
                                   c_f32, ctypes.c_int, c_vp]),
    "sta_forward_raster": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, Dim3, Dim3,
                                          c_vp, c_f32, ctypes.c_int, c_vp]),
    "sta_backward_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, Dim3, Dim3, ctypes.c_int]),
    "sta_backward": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                    c_i64, c_i64, c_i64, Dim3, Dim3, c_vp, c_f32, ctypes.c_int, c_vp]),
    "sta_backward_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                            c_i64, c_i64, c_i64, Dim3, Dim3, c_vp, c_f32, ctypes.c_int, c_vp]),
    "sta_dense_forward": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64,
                                         c_f32, ctypes.c_int, c_vp]),
    "sta_window_mass_workspace_bytes": (c_sz, [c_i64, c_i64, Dim3, Dim3, c_i64]),
    "sta_window_mass": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_sz, c_i64, c_i64, c_i64, Dim3, Dim3, c_vp,
                                       c_i64, c_f32, ctypes.c_int, c_vp]),
}

_lib = None


class StaError(RuntimeError):
    def __init__(self, code, fn):
        self.code = code
        super().__init__(f"{fn}: {strerror(code)} (code {code})")


def lib():
    """The loaded libsta.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_sliding_tile_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(code):
    return lib().sta_strerror(int(code)).decode()


def _check(code, fn):
    if code != 0:
        raise StaError(int(code), fn)


def _dim3(x):
    t, h, w = (int(a) for a in x)
    return Dim3(t, h, w)


def _windows(windows, heads):
    arr = np.ascontiguousarray(np.asarray(windows, dtype=np.int32).reshape(-1, 3))
    if arr.shape[0] == 1 and heads > 1:
        arr = np.ascontiguousarray(np.repeat(arr, heads, axis=0))
    if arr.shape[0] != heads:
        raise ValueError(f"need one window per head ({heads}), got {arr.shape[0]}")
    return arr


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return STA_BF16
    if t.dtype == torch.float32:
        return STA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape4(x, name):
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, Hh, S, D]")
    return x.shape


def raster_len(latent):
    """Tokens of the latent (rows of a raster-order tensor)."""
    t, h, w = (int(a) for a in latent)
    return t * h * w


def tile_major_len(latent, tile):
    """Rows of a tile-major tensor: the latent padded up to whole tiles."""
    return int(np.prod([-(-int(a) // int(b)) * int(b) for a, b in zip(latent, tile)]))


def _same(ref, name, *tensors):
    for n, t in tensors:
        if tuple(t.shape) != tuple(ref) or t.dtype != tensors[0][1].dtype:
            raise ValueError(f"{n} must match {name}: shape {tuple(ref)}, dtype {tensors[0][1].dtype}")


def tile_reorder(x, latent, tile, out=None):
    """Raster [B, Hh, T*H*W, D] -> tile-major [B, Hh, S', D] (S' padded up to
    whole tiles; padding rows are zero)."""
    B, Hh, S, D = _shape4(x, "x")
    if S != raster_len(latent):
        raise ValueError(f"x has {S} rows, the latent {latent} has {raster_len(latent)} tokens")
    shape = (B, Hh, tile_major_len(latent, tile), D)
    out = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    _same(shape, "the tile-major shape", ("out", out))
    if out.dtype != x.dtype:
        raise ValueError("out must have the dtype of x")
    _check(lib().sta_tile_reorder(_dev(x, "x"), _dev(out, "out"), B, Hh, D, _dim3(latent), _dim3(tile),
                                  _dtype(x), _stream(x)), "sta_tile_reorder")
    return out


def tile_unreorder(y, latent, tile, out=None):
    """Tile-major [B, Hh, S', D] -> raster [B, Hh, T*H*W, D] (padding dropped)."""
    B, Hh, S, D = _shape4(y, "y")
    if S != tile_major_len(latent, tile):
        raise ValueError(f"y has {S} rows, tile-major {latent}/{tile} has {tile_major_len(latent, tile)}")
    shape = (B, Hh, raster_len(latent), D)
    out = torch.empty(shape, dtype=y.dtype, device=y.device) if out is None else out
    _same(shape, "the raster shape", ("out", out))
    if out.dtype != y.dtype:
        raise ValueError("out must have the dtype of y")
    _check(lib().sta_tile_unreorder(_dev(y, "y"), _dev(out, "out"), B, Hh, D, _dim3(latent), _dim3(tile),
                                    _dtype(y), _stream(y)), "sta_tile_unreorder")
    return out


def tile_pairs_count(latent, tile, windows, transpose=False):
    w = _windows(windows, len(np.asarray(windows).reshape(-1, 3)))
    n = lib().sta_tile_pairs_count(_dim3(latent), _dim3(tile), w.ctypes.data_as(c_vp), w.shape[0],
                                   1 if transpose else 0)
    if n < 0:
        raise StaError(int(n), "sta_tile_pairs_count")
    return int(n)


def tile_pairs(latent, tile, windows, transpose=False, device="cuda"):
    """Pair list computed on the GPU: (int32 [P, 2] tensor, int64 offsets [Hh+1])."""
    w = _windows(windows, len(np.asarray(windows).reshape(-1, 3)))
    n = tile_pairs_count(latent, tile, w, transpose)
    out = torch.empty((max(n, 1), 2), dtype=torch.int32, device=device)
    off = np.zeros(w.shape[0] + 1, dtype=np.int64)
    _check(lib().sta_tile_pairs(_dev(out, "pairs"), off.ctypes.data_as(c_vp), _dim3(latent), _dim3(tile),
                                w.ctypes.data_as(c_vp), w.shape[0], int(bool(transpose)), _stream(out)),
           "sta_tile_pairs")
    return out[:n], off


def tile_pairs_host(latent, tile, windows, transpose=False):
    """Same list computed by the library on the host: (int32 [P, 2], int64 [Hh+1])."""
    w = _windows(windows, len(np.asarray(windows).reshape(-1, 3)))
    n = tile_pairs_count(latent, tile, w, transpose)
    out = np.zeros((max(n, 1), 2), dtype=np.int32)
    off = np.zeros(w.shape[0] + 1, dtype=np.int64)
    _check(lib().sta_tile_pairs_host(out.ctypes.data_as(c_vp), off.ctypes.data_as(c_vp), _dim3(latent),
                                     _dim3(tile), w.ctypes.data_as(c_vp), w.shape[0], int(bool(transpose))),
           "sta_tile_pairs_host")
    return out[:n], off


def forward(q, k, v, latent, tile, windows, scale=None, out=None, lse=None, want_lse=True):
    """STA forward on tile-major [B, Hh, S, D] tensors: returns (O, LSE or None)."""
    B, Hh, S, D = _shape4(q, "q")
    if S != tile_major_len(latent, tile):
        raise ValueError(f"q has {S} rows, tile-major {latent}/{tile} has {tile_major_len(latent, tile)}")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    w = _windows(windows, Hh)
    out = torch.empty_like(q) if out is None else out
    _same(q.shape, "q", ("q", q), ("k", k), ("v", v), ("out", out))
    if lse is None and want_lse:
        lse = torch.empty((B, Hh, S), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, Hh, S) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, Hh, S]")
    lp = _dev(lse, "lse") if lse is not None else c_vp(None)
    _check(lib().sta_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "o"), lp, B, Hh, D,
                             _dim3(latent), _dim3(tile), w.ctypes.data_as(c_vp), scale, _dtype(q),
                             _stream(q)), "sta_forward")
    return out, lse


def forward_raster(q, k, v, latent, tile, windows, scale=None, out=None, lse=None, want_lse=True):
    """STA forward on raster-order [B, Hh, T*H*W, D] tensors (reorder and
    unreorder inside the kernel): returns (O, LSE or None), both raster."""
    B, Hh, S, D = _shape4(q, "q")
    if S != raster_len(latent):
        raise ValueError(f"q has {S} rows, the latent {latent} has {raster_len(latent)} tokens")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    w = _windows(windows, Hh)
    out = torch.empty_like(q) if out is None else out
    _same(q.shape, "q", ("q", q), ("k", k), ("v", v), ("out", out))
    if lse is None and want_lse:
        lse = torch.empty((B, Hh, S), dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != (B, Hh, S) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, Hh, S]")
    lp = _dev(lse, "lse") if lse is not None else c_vp(None)
    _check(lib().sta_forward_raster(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "o"), lp, B, Hh, D,
                                    _dim3(latent), _dim3(tile), w.ctypes.data_as(c_vp), scale, _dtype(q),
                                    _stream(q)), "sta_forward_raster")
    return out, lse


def backward_workspace_bytes(B, Hh, D, latent, tile, dtype=torch.bfloat16):
    dt = STA_BF16 if dtype == torch.bfloat16 else STA_F32
    return int(lib().sta_backward_workspace_bytes(B, Hh, D, _dim3(latent), _dim3(tile), dt))


def backward(q, k, v, o, do, lse, latent, tile, windows, scale=None, workspace=None):
    """STA backward on tile-major tensors: returns (dQ, dK, dV)."""
    B, Hh, S, D = _shape4(q, "q")
    if S != tile_major_len(latent, tile):
        raise ValueError(f"q has {S} rows, tile-major {latent}/{tile} has {tile_major_len(latent, tile)}")
    _same(q.shape, "q", ("q", q), ("k", k), ("v", v), ("o", o), ("do", do))
    if tuple(lse.shape) != (B, Hh, S) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hh, S]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    w = _windows(windows, Hh)
    nbytes = backward_workspace_bytes(B, Hh, D, latent, tile, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib().sta_backward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(do, "do"),
                              _dev(lse, "lse"), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"),
                              _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                              B, Hh, D, _dim3(latent), _dim3(tile), w.ctypes.data_as(c_vp), scale,
                              _dtype(q), _stream(q)), "sta_backward")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, latent, tile, windows, scale=None, out=None):
    """STA backward through sta_backward_noalloc (the library's static scratch
    instead of a workspace): returns (dQ, dK, dV).  ``out`` may pass the three
    output tensors, so the call itself allocates nothing."""
    B, Hh, S, D = _shape4(q, "q")
    if S != tile_major_len(latent, tile):
        raise ValueError(f"q has {S} rows, tile-major {latent}/{tile} has {tile_major_len(latent, tile)}")
    _same(q.shape, "q", ("q", q), ("k", k), ("v", v), ("o", o), ("do", do))
    if tuple(lse.shape) != (B, Hh, S) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hh, S]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    w = _windows(windows, Hh)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None else out
    _same(q.shape, "q", ("dq", dq), ("dk", dk), ("dv", dv))
    _check(lib().sta_backward_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(do, "do"),
                                      _dev(lse, "lse"), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"),
                                      B, Hh, D, _dim3(latent), _dim3(tile), w.ctypes.data_as(c_vp), scale,
                                      _dtype(q), _stream(q)), "sta_backward_noalloc")
    return dq, dk, dv


def dense_forward(q, k, v, scale=None, out=None, want_lse=True):
    """Full softmax attention over all S keys: returns (O, LSE or None)."""
    B, Hh, S, D = _shape4(q, "q")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    _same(q.shape, "q", ("q", q), ("k", k), ("v", v), ("out", out))
    lse = torch.empty((B, Hh, S), dtype=torch.float32, device=q.device) if want_lse else None
    lp = _dev(lse, "lse") if lse is not None else c_vp(None)
    _check(lib().sta_dense_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "o"), lp, B, Hh, S, D,
                                   scale, _dtype(q), _stream(q)), "sta_dense_forward")
    return out, lse


def window_mass_workspace_bytes(B, Hh, latent, tile, n_cand):
    return int(lib().sta_window_mass_workspace_bytes(B, Hh, _dim3(latent), _dim3(tile), int(n_cand)))


def window_mass(q, k, latent, tile, candidates, scale=None, workspace=None, out=None):
    """Attention mass of each candidate window (one window for all heads at a
    time) on tile-major q, k: float32 [C, B, Hh] on the device, the mean over
    real query rows of the share of the full softmax the window keeps."""
    B, Hh, S, D = _shape4(q, "q")
    if S != tile_major_len(latent, tile):
        raise ValueError(f"q has {S} rows, tile-major {latent}/{tile} has {tile_major_len(latent, tile)}")
    _same(q.shape, "q", ("q", q), ("k", k))
    scale = float(D) ** -0.5 if scale is None else float(scale)
    c = np.ascontiguousarray(np.asarray(candidates, dtype=np.int32).reshape(-1, 3))
    nbytes = window_mass_workspace_bytes(B, Hh, latent, tile, c.shape[0])
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    shape = (c.shape[0], B, Hh)
    out = torch.empty(shape, dtype=torch.float32, device=q.device) if out is None else out
    if tuple(out.shape) != shape or out.dtype != torch.float32:
        raise ValueError(f"out must be float32 {shape}")
    _check(lib().sta_window_mass(_dev(q, "q"), _dev(k, "k"), _dev(out, "mass"), _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), B, Hh, D, _dim3(latent),
                                 _dim3(tile), c.ctypes.data_as(c_vp), c.shape[0], scale, _dtype(q), _stream(q)),
           "sta_window_mass")
    return out
