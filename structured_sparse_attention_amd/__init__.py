"""Structured-sparse (Sparse VideoGen) video attention for AMD MI355X.

The compute path is the HIP library ``libsvgattn.so`` (C ABI declared in
``include/svg_attn.h``); this package only binds it with ctypes.
"""
from ._lib import (  # noqa: F401
    ATTN_MASK_ALL_TILES, ERR_ALIGNMENT, ERR_HIP, ERR_INVALID_ARG, ERR_OOM,
    ERR_SHAPE_MISMATCH, ERR_UNSUPPORTED, EXPORTED, HEAD_DENSE, HEAD_SPATIAL,
    HEAD_TEMPORAL, LIB_PATH, OK, ROUND_EXACT, ROUND_TILE, TILE_BOUNDARY,
    TILE_FULL, TILE_SKIP, TO_KERNEL_LAYOUT, TO_ORIGINAL_LAYOUT, MaskSpec,
    SvgError, TileMap, abi_version, load, svg_attn_fwd, svg_autotune_tiles,
    svg_build_tile_map, svg_permute_tokens, svg_route_heads,
)
