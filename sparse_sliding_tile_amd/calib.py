"""ctypes binding of libsta_calib.so: the matrix-core calibration loop the
benchmark times next to the attention kernels (not part of libsta).

It launches blocks x 256 threads; each wave runs iters iterations of 16 bf16
32x32x16 MFMAs on operands taken from the caller's buffer, so its rate shows
what the matrix cores sustain on data drawn like the attention inputs.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsta_calib.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_sliding_tile_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sta_calib_mfma_bf16.restype = ctypes.c_int
        L.sta_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def calib_mfma_bf16(operands, iters, blocks, out=None):
    """Launch the loop on ``operands`` (a contiguous device tensor of a
    power-of-two byte size); returns (out, FLOP of the launch)."""
    if not operands.is_cuda or not operands.is_contiguous():
        raise ValueError("operands must be a contiguous GPU tensor")
    nbytes = operands.numel() * operands.element_size()
    out = torch.empty(blocks * 256, dtype=torch.float32, device=operands.device) if out is None else out
    stream = torch.cuda.current_stream(operands.device).cuda_stream
    rc = lib().sta_calib_mfma_bf16(ctypes.c_void_p(operands.data_ptr()), nbytes, int(iters), int(blocks),
                                   ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"sta_calib_mfma_bf16 failed with code {rc}")
    return out, blocks * 4 * int(iters) * 16 * 32768
