"""Block-sparse tiled attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libbsa.so`` (hand-written HIP kernels behind the C
ABI in ``include/bsa.h``); this package only marshals arguments.
"""
from .api import (  # noqa: F401
    COARSE_MAX_TILES,
    BsaError,
    bwd,
    bwd_k2q,
    coarse,
    coarse_combine,
    coarse_pooled,
    coarse_workspace_size,
    cube_tile_map,
    fwd,
    fwd_lse,
    fwd_noalloc,
    fwd_out_shape,
    load,
    status_string,
    tile_layout,
    tile_layout_pool,
    tile_unlayout,
    tile_unlayout_combine,
    within_launch_limits,
    within_launch_limits_py,
    workspace_size,
)
