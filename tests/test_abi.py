"""The C-ABI library on the CPU: it loads, exports every function include/sta.h
declares, rejects bad arguments with the documented codes before launching
anything, and its host-side tile-pair list equals the oracle's bit for bit.

Every call here fails validation (or is host-only), so no kernel is launched
and no device memory is touched: the fake device pointers are never used.
"""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import torch
import pytest

import oracle as O
import sparse_sliding_tile_amd._lib as L
from sparse_sliding_tile_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sta.h")

OK, ARG, NOT_MULT, WINDOW, UNSUP, ALIGN, HIP, WS, TOO_LARGE = 0, -1, -2, -3, -4, -5, -6, -7, -8
P = ctypes.c_void_p(0x10000)      # aligned stand-in, never dereferenced
MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only
NUL = ctypes.c_void_p(None)


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|size_t|const char\*)\s+(sta_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"binding lacks {n}"


def test_exports_nothing_else(lib):
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"]})
    assert exported == header_functions()


def test_strerror_covers_codes(lib):
    for c in (OK, ARG, NOT_MULT, WINDOW, UNSUP, ALIGN, HIP, WS, TOO_LARGE):
        s = lib.sta_strerror(c).decode()
        assert s and s != "unknown error code"
    assert lib.sta_strerror(12345).decode() == "unknown error code"


def d3(*a):
    return L.Dim3(*a)


def win(rows):
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))


def fwd(lib, q=P, k=P, v=P, o=P, lse=NUL, B=1, Hh=2, D=128, latent=(6, 16, 16), tile=(2, 4, 4),
        windows=((3, 3, 3), (3, 3, 3)), scale=0.1, dt=L.STA_BF16):
    w = win(windows)
    return lib.sta_forward(q, k, v, o, lse, B, Hh, D, d3(*latent), d3(*tile), w.ctypes.data_as(ctypes.c_void_p),
                           scale, dt, NUL)


def test_forward_argument_errors(lib):
    assert fwd(lib, q=NUL) == ARG
    assert fwd(lib, o=NUL) == ARG
    assert fwd(lib, scale=0.0) == ARG
    assert fwd(lib, scale=-1.0) == ARG
    assert fwd(lib, scale=float("nan")) == ARG
    assert fwd(lib, B=0) == ARG
    assert fwd(lib, latent=(0, 16, 16)) == ARG
    assert fwd(lib, latent=(5, 16, 16), windows=((3, 0, 3), (3, 3, 3))) == WINDOW   # padded latent, bad window
    assert fwd(lib, latent=(2000, 2000, 2000), tile=(6, 8, 8)) == TOO_LARGE
    assert fwd(lib, windows=((3, 0, 3), (3, 3, 3))) == WINDOW
    assert fwd(lib, windows=((3, 3, 3), (3, 3, -1))) == WINDOW
    assert fwd(lib, D=96) == UNSUP                             # bf16 needs D in {64, 128}
    assert fwd(lib, D=96, dt=L.STA_F32) == UNSUP
    assert fwd(lib, dt=7) == UNSUP
    assert fwd(lib, tile=(1, 4, 4), latent=(6, 16, 16)) == UNSUP   # L = 16 is not a multiple of 32
    # a padded latent's compacted key index is split in fp32: L <= 2^20 (here 1024 * 1032)
    assert fwd(lib, tile=(1, 1024, 1032), latent=(1, 1025, 1025)) == UNSUP
    assert fwd(lib, q=MIS) == ALIGN
    assert fwd(lib, lse=MIS) == ALIGN
    many = [(3, 3, 3)] * 257
    assert fwd(lib, Hh=257, windows=many) == UNSUP
    assert lib.sta_forward(P, P, P, P, NUL, 1, 2, 128, d3(6, 16, 16), d3(2, 4, 4), NUL, 0.1, 0, NUL) == ARG


def test_forward_raster_argument_errors(lib):
    w = win([(3, 3, 3), (3, 3, 3)])

    def fr(latent=(6, 16, 32), tile=(2, 4, 8), D=128, dt=L.STA_BF16, q=P, lse=NUL):
        return lib.sta_forward_raster(q, P, P, P, lse, 1, 2, D, d3(*latent), d3(*tile),
                                      w.ctypes.data_as(ctypes.c_void_p), 0.1, dt, NUL)
    assert fr(q=NUL) == ARG
    assert fr(dt=L.STA_F32) == UNSUP
    assert fr(tile=(2, 8, 2), latent=(6, 16, 32)) == UNSUP    # copy segments of 4 rows span x-runs
    assert fr(D=64, tile=(2, 8, 4)) == UNSUP                   # D = 64: 8-row segments, width 4 too narrow
    assert fr(D=96) == UNSUP
    # the raster instance tabulates at most 1024 copy segments per tile: L <= 4096 for D = 128
    assert fr(latent=(8, 64, 64), tile=(8, 32, 32)) == UNSUP
    assert fr(q=MIS) == ALIGN
    assert fr(lse=MIS) == ALIGN


def test_reorder_argument_errors(lib):
    f = lib.sta_tile_reorder
    assert f(NUL, P, 1, 2, 64, d3(6, 16, 16), d3(2, 4, 4), 0, NUL) == ARG
    assert f(P, P, 1, 2, 64, d3(1, 2, 1 << 30), d3(1, 1, 3), 0, NUL) == TOO_LARGE
    assert f(MIS, P, 1, 2, 64, d3(6, 16, 16), d3(2, 4, 4), 0, NUL) == ALIGN
    assert f(P, P, 1, 2, 64, d3(6, 16, 16), d3(2, 4, 4), 9, NUL) == UNSUP
    assert lib.sta_tile_unreorder(P, NUL, 1, 2, 64, d3(6, 16, 16), d3(2, 4, 4), 0, NUL) == ARG
    assert f(P, P, 1, 2, 0, d3(6, 16, 16), d3(2, 4, 4), 0, NUL) == ARG


def test_backward_argument_errors(lib):
    w = win([(3, 3, 3)] * 2)
    wp = w.ctypes.data_as(ctypes.c_void_p)
    need = lib.sta_backward_workspace_bytes(1, 2, 128, d3(6, 16, 16), d3(2, 4, 4), 0)
    assert need == 2 * 1 * 2 * 1536 * 4 + 2 * 48 * 4   # row statistics + key-tile order (48 tiles)
    assert lib.sta_backward_workspace_bytes(1, 2, 128, d3(6, 16, 16), d3(2, 4, 4), 1) == 2 * 1 * 2 * 1536 * 4
    # padded latent (5, 15, 16) -> (6, 16, 16): sizes follow the padded sequence
    assert lib.sta_backward_workspace_bytes(1, 2, 128, d3(5, 15, 16), d3(2, 4, 4), 0) == need
    assert lib.sta_backward_workspace_bytes(1, 2, 128, d3(0, 15, 16), d3(2, 4, 4), 0) == 0

    def bwd(ws=P, nbytes=need, lse=P, dq=P, D=128, dt=0, windows=wp):
        return lib.sta_backward(P, P, P, P, P, lse, dq, P, P, ws, nbytes, 1, 2, D, d3(6, 16, 16), d3(2, 4, 4),
                                windows, 0.1, dt, NUL)
    assert bwd(ws=NUL) == WS
    assert bwd(nbytes=need - 1) == WS
    assert bwd(lse=NUL) == ARG
    assert bwd(dq=NUL) == ARG
    assert bwd(dq=MIS) == ALIGN
    assert bwd(D=80) == UNSUP
    assert bwd(windows=NUL) == ARG
    # a padded latent's compacted row index is split in fp32: L <= 2^20 (here 1024 * 1032)
    big = (L.Dim3(1, 1025, 1025), L.Dim3(1, 1024, 1032))
    nbig = lib.sta_backward_workspace_bytes(1, 2, 128, *big, 0)
    assert lib.sta_backward(P, P, P, P, P, P, P, P, P, P, nbig, 1, 2, 128, *big, wp, 0.1, 0, NUL) == UNSUP


def test_backward_noalloc_argument_errors(lib):
    """The static-scratch backward validates everything before it touches a
    device: bad arguments and sizes whose workspace exceeds the 32 MiB array."""
    w = win([(3, 3, 3)] * 2)
    wp = w.ctypes.data_as(ctypes.c_void_p)

    def bn(lse=P, dq=P, B=1, Hh=2, D=128, latent=(6, 16, 16), tile=(2, 4, 4), windows=wp, scale=0.1, dt=0):
        return lib.sta_backward_noalloc(P, P, P, P, P, lse, dq, P, P, B, Hh, D, d3(*latent), d3(*tile), windows,
                                        scale, dt, NUL)
    assert bn(lse=NUL) == ARG
    assert bn(dq=NUL) == ARG
    assert bn(scale=0.0) == ARG
    assert bn(windows=NUL) == ARG
    assert bn(latent=(0, 16, 16)) == ARG
    # 40 heads at (30, 48, 80): 8 bytes of row statistics per row, 4.6 M rows > 32 MiB
    forty = win([(3, 3, 3)] * 40)
    assert bn(Hh=40, latent=(30, 48, 80), tile=(6, 8, 8), windows=forty.ctypes.data_as(ctypes.c_void_p)) == TOO_LARGE
    need = lib.sta_backward_workspace_bytes(1, 40, 128, d3(30, 48, 80), d3(6, 8, 8), 0)
    assert need > (32 << 20)
    # the fine-tuning and HunyuanVideo shapes at 24 heads fit
    assert lib.sta_backward_workspace_bytes(1, 24, 128, d3(24, 64, 64), d3(6, 8, 8), 0) <= (32 << 20)
    assert lib.sta_backward_workspace_bytes(1, 24, 128, d3(30, 48, 80), d3(6, 8, 8), 0) <= (32 << 20)


def test_dense_argument_errors(lib):
    f = lib.sta_dense_forward
    assert f(P, P, P, P, NUL, 1, 2, 1000, 128, 0.1, 0, NUL) == UNSUP    # bf16 needs S % 32 == 0
    assert f(P, P, P, P, NUL, 1, 2, 0, 128, 0.1, 0, NUL) == ARG
    assert f(NUL, P, P, P, NUL, 1, 2, 1024, 128, 0.1, 0, NUL) == ARG
    assert f(P, P, P, P, NUL, 1, 2, 1024, 128, 0.0, 0, NUL) == ARG


def test_window_mass_argument_errors(lib):
    need = lib.sta_window_mass_workspace_bytes(1, 2, d3(6, 16, 16), d3(2, 4, 4), 2)
    assert need == 2 * 1 * 2 * 1536 * 4 + 2 * 1 * 2 * 48 * 4    # two fp32 LSE vectors + partials
    assert lib.sta_window_mass_workspace_bytes(1, 2, d3(5, 15, 16), d3(2, 4, 4), 2) == need   # padded
    assert lib.sta_window_mass_workspace_bytes(0, 2, d3(6, 16, 16), d3(2, 4, 4), 2) == 0
    assert lib.sta_window_mass_workspace_bytes(1, 2, d3(6, 16, 16), d3(2, 4, 4), 0) == 0
    good = win([(3, 3, 3), (1, 1, 1)])
    bad = win([(3, 3, 3), (1, 0, 1)])

    def wm(q=P, k=P, mass=P, ws=P, nbytes=need, Hh=2, D=128, cands=good, n=2, scale=0.1, dt=0):
        cp = cands.ctypes.data_as(ctypes.c_void_p) if cands is not None else NUL
        return lib.sta_window_mass(q, k, mass, ws, nbytes, 1, Hh, D, d3(6, 16, 16), d3(2, 4, 4), cp, n,
                                   scale, dt, NUL)
    assert wm(q=NUL) == ARG
    assert wm(mass=NUL) == ARG
    assert wm(cands=None) == ARG
    assert wm(n=0) == ARG
    assert wm(scale=0.0) == ARG
    assert wm(ws=NUL) == WS
    assert wm(nbytes=need - 1) == WS
    assert wm(D=96) == UNSUP
    assert wm(dt=5) == UNSUP
    assert wm(q=MIS) == ALIGN
    assert wm(cands=bad) == WINDOW          # every candidate is checked before the first launch
    assert wm(Hh=257) == UNSUP
    nine = win([(1, 1, 1)] * 9)
    assert wm(cands=nine, n=9, nbytes=1 << 30) == UNSUP     # more than STA_MAX_CANDIDATES


def test_calib_library_argument_errors():
    """The calibration loop lives in its own library (benchmark support, not
    libsta's interface) and validates before launching."""
    from sparse_sliding_tile_amd import calib
    f = calib.lib().sta_calib_mfma_bf16
    assert f(NUL, 1 << 20, 10, 4, P, NUL) == ARG
    assert f(P, 1 << 20, 10, 4, NUL, NUL) == ARG
    assert f(P, 3 << 16, 10, 4, P, NUL) == ARG        # not a power of two
    assert f(P, 128, 10, 4, P, NUL) == ARG            # fewer than 16 vectors
    assert f(P, 1 << 20, 0, 4, P, NUL) == ARG
    assert f(P, 1 << 20, 10, 1 << 40, P, NUL) == ARG
    assert f(MIS, 1 << 20, 10, 4, P, NUL) == ALIGN


def test_grid_dimension_limit(lib):
    """Clamped windows reach the kernels as 16-bit widths: a tile grid with
    more than 65535 tiles along a dimension is refused, never wrapped."""
    full = win([(1, 1, 65536)])
    fp = full.ctypes.data_as(ctypes.c_void_p)
    assert lib.sta_tile_pairs_count(d3(1, 1, 65535 * 32), d3(1, 1, 32), fp, 1, 0) == 65535 * 65535
    assert lib.sta_tile_pairs_count(d3(1, 1, 65536 * 32), d3(1, 1, 32), fp, 1, 0) == TOO_LARGE
    assert lib.sta_tile_pairs_count(d3(65536, 1, 1), d3(1, 1, 1), fp, 1, 0) == TOO_LARGE
    # dense attention over 2^23 tokens picks 128-token tiles: 65536 of them
    assert lib.sta_dense_forward(P, P, P, P, NUL, 1, 2, 1 << 23, 128, 0.1, 0, NUL) == TOO_LARGE
    assert fwd(lib, latent=(1, 1, 65536 * 32), tile=(1, 1, 32), windows=((1, 1, 3), (1, 1, 3))) == TOO_LARGE


def test_pairs_argument_errors(lib):
    w = win([(3, 3, 3)])
    wp = w.ctypes.data_as(ctypes.c_void_p)
    assert lib.sta_tile_pairs_count(d3(0, 16, 16), d3(4, 4, 4), wp, 1, 0) == ARG
    assert lib.sta_tile_pairs_count(d3(6, 16, 16), d3(2, 4, 4), NUL, 1, 0) == ARG
    bad = win([(0, 3, 3)])
    assert lib.sta_tile_pairs_count(d3(6, 16, 16), d3(2, 4, 4), bad.ctypes.data_as(ctypes.c_void_p), 1, 0) == WINDOW
    assert lib.sta_tile_pairs(NUL, NUL, d3(6, 16, 16), d3(2, 4, 4), wp, 1, 0, NUL) == ARG
    # the count takes the list's transpose flag: 0 or 1, the same count for both
    n0 = lib.sta_tile_pairs_count(d3(6, 16, 16), d3(2, 4, 4), wp, 1, 0)
    assert n0 == 48 * 27 and lib.sta_tile_pairs_count(d3(6, 16, 16), d3(2, 4, 4), wp, 1, 1) == n0
    assert lib.sta_tile_pairs_count(d3(6, 16, 16), d3(2, 4, 4), wp, 1, 2) == ARG
    assert lib.sta_tile_pairs_count(d3(6, 16, 16), d3(2, 4, 4), wp, 1, -1) == ARG


PAIR_CASES = [((6, 16, 16), (2, 4, 4), [(3, 3, 3), (1, 2, 5)]),
              ((30, 48, 80), (6, 8, 8), I.mixed_windows(24, 0)),
              ((30, 48, 80), (6, 8, 8), [(3, 3, 3)] * 2),
              ((24, 48, 80), (6, 8, 8), [(3, 3, 5)]),
              ((24, 64, 64), (6, 8, 8), [(3, 5, 5)]),
              ((5, 6, 10), (5, 3, 2), [(2, 2, 4), (9, 1, 1)]),
              ((1, 8, 16), (1, 8, 8), [(1, 1, 1), (1, 1, 2)]),
              ((29, 45, 76), (6, 8, 8), [(3, 3, 3), (1, 6, 10)]),     # padded to (30, 48, 80)
              ((5, 15, 13), (2, 4, 4), [(3, 3, 3), (2, 1, 4)])]       # padded to (6, 16, 16)


@pytest.mark.parametrize("latent,tile,wins", PAIR_CASES)
def test_pair_count_matches_oracle(latent, tile, wins):
    _, off = O.tile_pairs(O.padded_latent(latent, tile), tile, wins)
    assert L.tile_pairs_count(latent, tile, wins) == off[-1]
    assert L.tile_pairs_count(latent, tile, wins, transpose=True) == off[-1]


@pytest.mark.parametrize("latent,tile,wins", PAIR_CASES)
@pytest.mark.parametrize("transpose", [False, True])
def test_host_pairs_bit_exact(latent, tile, wins, transpose):
    p, off = L.tile_pairs_host(latent, tile, wins, transpose=transpose)
    rp, roff = O.tile_pairs(O.padded_latent(latent, tile), tile, wins, transpose=transpose)
    assert np.array_equal(off, roff)
    assert np.array_equal(p, rp)


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        L.lib()


def test_product_never_imports_oracle():
    pkg = os.path.join(ROOT, "sparse_sliding_tile_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), errors="replace").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f


def test_binding_validates_shapes():
    """The binding checks tensor rows against the latent before any call (the
    C entry points take sizes, not tensors)."""
    x = torch.zeros((1, 1, 10, 8))
    with pytest.raises((ValueError, TypeError)):
        L.tile_reorder(x, (2, 2, 3), (1, 2, 2))        # 12 tokens expected
    assert L.raster_len((29, 45, 76)) == 29 * 45 * 76
    assert L.tile_major_len((29, 45, 76), (6, 8, 8)) == 30 * 48 * 80
    assert L.tile_major_len((30, 48, 80), (6, 8, 8)) == 30 * 48 * 80
