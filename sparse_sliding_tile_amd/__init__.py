"""Sliding Tile Attention for AMD MI355X: a thin Python face over libsta.so.

The library is loaded on first use; without it every call raises.
"""
from ._lib import (STA_BF16, STA_F32, StaError, backward, backward_noalloc, backward_workspace_bytes,  # noqa: F401
                   dense_forward, forward, forward_raster, lib, raster_len, strerror, tile_major_len, tile_pairs,
                   tile_pairs_count, tile_pairs_host, tile_reorder, tile_unreorder, window_mass,
                   window_mass_workspace_bytes)
