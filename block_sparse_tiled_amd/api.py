"""Python binding of libbsa: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(``include/bsa.h``); this module checks torch tensors, passes their device
pointers and sizes, and turns status codes into exceptions.  There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsa.so")

# Launch limits, mirrored from include/bsa.h (FastVideo fastvideo-kernel commit
# list, page 3, hardening commit: batch*heads <= 65535, rows < 2^31, tiles < 2^22).
MAX_BATCH_HEADS = 65535
ROWS_LIMIT = 1 << 31
TILES_LIMIT = 1 << 22
TILES = (64, 128, 256)
HEAD_DIMS = (64, 128)

STATUS = {
    0: "BSA_OK",
    1: "BSA_ERR_INVALID_ARGUMENT",
    2: "BSA_ERR_UNSUPPORTED_SHAPE",
    3: "BSA_ERR_LAUNCH_LIMITS",
    4: "BSA_ERR_NO_DEVICE",
    5: "BSA_ERR_UNSUPPORTED_DEVICE",
    6: "BSA_ERR_HIP",
    7: "BSA_ERR_SCRATCH_LIMIT",
}


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load():
    """Load libbsa.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_tiled_amd.build` "
            "(the HIP library is required; there is no other implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.bsa_within_launch_limits.argtypes = [i64, i64, i64, i64]
    lib.bsa_within_launch_limits.restype = ctypes.c_int
    lib.bsa_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, i32, i32, vp, i64, vp]
    lib.bsa_fwd.restype = ctypes.c_int
    lib.bsa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, i32, i32, vp]
    lib.bsa_fwd_noalloc.restype = ctypes.c_int
    lib.bsa_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(i64)]
    lib.bsa_fwd_workspace_size.restype = ctypes.c_int
    lib.bsa_tile_layout.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32,
                                    i64, i64, i64, i64, i32, vp]
    lib.bsa_tile_layout.restype = ctypes.c_int
    lib.bsa_fwd_lse.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i32, i32,
                                vp, i64, vp]
    lib.bsa_fwd_lse.restype = ctypes.c_int
    lib.bsa_bwd_k2q.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp, i32, vp]
    lib.bsa_bwd_k2q.restype = ctypes.c_int
    lib.bsa_bwd.argtypes = [vp] * 12 + [i32] + [vp] * 4 + [i64, i64, i64, i32, i32, i32, vp]
    lib.bsa_bwd.restype = ctypes.c_int
    lib.bsa_tile_unlayout.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32,
                                      i64, i64, i64, i64, i32, vp]
    lib.bsa_tile_unlayout.restype = ctypes.c_int
    lib.bsa_cube_num_tiles.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.bsa_cube_num_tiles.restype = i64
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.bsa_cube_tile_map.argtypes = [i64, i64, i64, i32, i32, i32, i32, ip, ip, ip]
    lib.bsa_cube_tile_map.restype = ctypes.c_int
    lib.bsa_coarse_workspace_size.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(i64)]
    lib.bsa_coarse_workspace_size.restype = ctypes.c_int
    lib.bsa_coarse.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, i64, i64, i64, i32, i32, vp,
                               i64, vp]
    lib.bsa_coarse.restype = ctypes.c_int
    lib.bsa_coarse_combine.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, vp]
    lib.bsa_coarse_combine.restype = ctypes.c_int
    lib.bsa_tile_layout_pool.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, vp, i32,
                                         i64, i64, i64, i64, i32, vp, vp]
    lib.bsa_tile_layout_pool.restype = ctypes.c_int
    lib.bsa_coarse_pooled.argtypes = [vp, vp, i32, i32, vp, vp, vp, i64, i64, i64, i32, i32, vp,
                                      i64, vp]
    lib.bsa_coarse_pooled.restype = ctypes.c_int
    lib.bsa_tile_unlayout_combine.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, vp,
                                              vp]
    lib.bsa_tile_unlayout_combine.restype = ctypes.c_int
    lib.bsa_status_string.argtypes = [ctypes.c_int]
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_abi_version.argtypes = []
    lib.bsa_abi_version.restype = ctypes.c_int
    lib.bsa_test_override_arch.argtypes = [ctypes.c_char_p]
    lib.bsa_test_override_arch.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise BsaError(status, load().bsa_status_string(status).decode())


def status_string(status: int) -> str:
    return load().bsa_status_string(status).decode()


def within_launch_limits(batch: int, heads: int, rows: int, tiles: int) -> bool:
    """The library's launch-limit check (rows = batch*heads*NT*T, tiles = NT)."""
    return bool(load().bsa_within_launch_limits(batch, heads, rows, tiles))


def within_launch_limits_py(batch: int, heads: int, rows: int, tiles: int) -> bool:
    """Pure-Python mirror of the same limits, usable without the library."""
    if min(batch, heads, rows, tiles) < 0:
        return False
    return batch * heads <= MAX_BATCH_HEADS and rows < ROWS_LIMIT and tiles < TILES_LIMIT


def _stream_handle(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else ctypes.c_void_p(0)


def _require(t, name, dtype, device, ndim):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd_out_shape(q_shape):
    """Shape of bsa.fwd's output for a q of this shape (it equals q's)."""
    return tuple(q_shape)


def workspace_size(batch, heads, num_tiles, tile, head_dim, max_sel):
    """Bytes of workspace ``fwd`` and ``fwd_lse`` use for this shape on the current
    device: per-XCD work-queue counters for long launches and the partials of split
    query tiles (0 when the call needs neither)."""
    lib = load()
    n = ctypes.c_int64(0)
    _check(lib.bsa_fwd_workspace_size(batch, heads, num_tiles, tile, head_dim, max_sel,
                                      ctypes.byref(n)))
    return int(n.value)


def _workspace(workspace, device, B, H, NT, tile, D, MS):
    """(pointer, bytes) of the workspace argument: "auto" allocates the size the
    library asks for (through torch's caching allocator), None passes none (whole
    query tiles only), a uint8 cuda tensor is used as given."""
    import torch

    if workspace is None:
        return None, ctypes.c_void_p(0), 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 cuda tensor')
        with torch.cuda.device(device):
            n = workspace_size(B, H, NT, tile, D, MS)
        if n == 0:
            return None, ctypes.c_void_p(0), 0
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    _require(workspace, "workspace", torch.uint8, device, 1)
    return workspace, _ptr(workspace), workspace.numel()


def fwd(q, k, v, q2k_idx, q2k_num, block_sizes, tile, out=None, workspace="auto"):
    """Block-sparse tiled attention forward on the current stream.

    q, k, v: bf16 [B, H, NT*tile, D] cuda tensors; q2k_idx int32 [B, H, NT, MS];
    q2k_num int32 [B, H, NT]; block_sizes int32 [NT].  Returns ``out`` (bf16,
    same shape as q), allocated with ``torch.empty`` when not given.  ``workspace``:
    "auto" (allocate what the library asks for), None (no workspace: whole query
    tiles only) or a uint8 cuda tensor of at least ``workspace_size`` bytes.
    """
    import torch

    lib = load()
    device, B, H, S, D, NT = _fwd_args(q, k, v, q2k_idx, q2k_num, block_sizes, tile)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", torch.bfloat16, device, 4)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    MS = int(q2k_idx.shape[3])
    ws, ws_ptr, ws_bytes = _workspace(workspace, device, B, H, NT, tile, D, MS)
    with torch.cuda.device(device):
        _check(lib.bsa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num),
                           _ptr(block_sizes), tile, _ptr(out), B, H, NT, D, MS, ws_ptr, ws_bytes,
                           _stream_handle(device)))
    return out


def fwd_noalloc(q, k, v, q2k_idx, q2k_num, block_sizes, tile, out):
    """``fwd`` through bsa_fwd_noalloc: no device memory is allocated (the library's
    fixed per-GPU scratch array holds the split workspace; calls that overlap on one GPU
    race on it).  ``out`` must be given."""
    import torch

    lib = load()
    device, B, H, S, D, NT = _fwd_args(q, k, v, q2k_idx, q2k_num, block_sizes, tile)
    _require(out, "out", torch.bfloat16, device, 4)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    with torch.cuda.device(device):
        _check(lib.bsa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num),
                                   _ptr(block_sizes), tile, _ptr(out), B, H, NT, D,
                                   int(q2k_idx.shape[3]), _stream_handle(device)))
    return out


def tile_layout(srcs, tile_src_token, tile, outs=None):
    """Fused token-to-tile layout of 1..4 token-major bf16 tensors [B, S_tok, H, D].

    ``tile_src_token`` is an int32 cuda tensor [NT*tile] naming the source
    token of each tile row (-1 = padding).  Returns tensors [B, H, NT*tile, D].
    """
    import torch

    lib = load()
    srcs = list(srcs)
    if not 1 <= len(srcs) <= 4:
        raise ValueError("tile_layout takes 1 to 4 tensors")
    device = srcs[0].device
    if device.type != "cuda":
        raise ValueError("bsa.tile_layout runs on a GPU")
    for n, x in enumerate(srcs):
        _require(x, f"src[{n}]", torch.bfloat16, device, 4)
        if x.shape != srcs[0].shape:
            raise ValueError("all layout inputs must share one shape")
    _require(tile_src_token, "tile_src_token", torch.int32, device, 1)
    B, S_tok, H, D = srcs[0].shape
    rows = tile_src_token.shape[0]
    if tile not in TILES or rows % tile:
        raise ValueError("the map must cover a whole number of 64-, 128- or 256-row tiles")
    NT = rows // tile
    if outs is None:
        outs = [torch.empty((B, H, rows, D), dtype=torch.bfloat16, device=device) for _ in srcs]
    else:
        outs = list(outs)
        if len(outs) != len(srcs):
            raise ValueError("one output per input")
        for n, o in enumerate(outs):
            _require(o, f"out[{n}]", torch.bfloat16, device, 4)
            if tuple(o.shape) != (B, H, rows, D):
                raise ValueError("outputs must be [B, H, NT*tile, D]")
    src_arr = (ctypes.c_void_p * len(srcs))(*[_ptr(x) for x in srcs])
    dst_arr = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    with torch.cuda.device(device):
        _check(lib.bsa_tile_layout(src_arr, dst_arr, len(srcs), _ptr(tile_src_token), tile,
                                   B, S_tok, H, NT, D, _stream_handle(device)))
    return outs


def tile_layout_pool(srcs, tile_src_token, block_sizes, tile, outs=None, pooled=None):
    """``tile_layout`` of Q, K, V (and optionally the gate: 3 or 4 tensors) that also forms
    the coarse stage's pooled tiles from the rows it moves.  Returns (outs, pooled), pooled
    float32 [3, B, H, NT, D] (the means of each tile's first block_sizes[t] rows of Q, K and
    V), for ``coarse_pooled``."""
    import torch

    lib = load()
    srcs = list(srcs)
    if not 3 <= len(srcs) <= 4:
        raise ValueError("tile_layout_pool takes Q, K, V and optionally the gate")
    device = srcs[0].device
    if device.type != "cuda":
        raise ValueError("bsa.tile_layout_pool runs on a GPU")
    for n, x in enumerate(srcs):
        _require(x, f"src[{n}]", torch.bfloat16, device, 4)
        if x.shape != srcs[0].shape:
            raise ValueError("all layout inputs must share one shape")
    _require(tile_src_token, "tile_src_token", torch.int32, device, 1)
    B, S_tok, H, D = srcs[0].shape
    rows = tile_src_token.shape[0]
    if tile not in TILES or rows % tile:
        raise ValueError("the map must cover a whole number of 64-, 128- or 256-row tiles")
    NT = rows // tile
    _require(block_sizes, "block_sizes", torch.int32, device, 1)
    if tuple(block_sizes.shape) != (NT,):
        raise ValueError("block_sizes must be [NT]")
    if outs is None:
        outs = [torch.empty((B, H, rows, D), dtype=torch.bfloat16, device=device) for _ in srcs]
    else:
        outs = list(outs)
        if len(outs) != len(srcs):
            raise ValueError("one output per input")
        for n, o in enumerate(outs):
            _require(o, f"out[{n}]", torch.bfloat16, device, 4)
            if tuple(o.shape) != (B, H, rows, D):
                raise ValueError("outputs must be [B, H, NT*tile, D]")
    if pooled is None:
        pooled = torch.empty((3, B, H, NT, D), dtype=torch.float32, device=device)
    _require(pooled, "pooled", torch.float32, device, 5)
    if tuple(pooled.shape) != (3, B, H, NT, D):
        raise ValueError("pooled must be [3, B, H, NT, D]")
    src_arr = (ctypes.c_void_p * len(srcs))(*[_ptr(x) for x in srcs])
    dst_arr = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    with torch.cuda.device(device):
        _check(lib.bsa_tile_layout_pool(src_arr, dst_arr, len(srcs), _ptr(tile_src_token),
                                        _ptr(block_sizes), tile, B, S_tok, H, NT, D, _ptr(pooled),
                                        _stream_handle(device)))
    return outs, pooled


def tile_unlayout(tiled, token_row, tile, tokens=None, outs=None):
    """Inverse of ``tile_layout``: 1..4 bf16 tile buffers [B, H, NT*tile, D] gathered
    back to token-major [B, S_tok, H, D].

    ``token_row`` is an int32 cuda tensor [S_tok] naming the tile row of each
    token (entries outside the buffer give +0 rows).
    """
    import torch

    lib = load()
    tiled = list(tiled)
    if not 1 <= len(tiled) <= 4:
        raise ValueError("tile_unlayout takes 1 to 4 tensors")
    device = tiled[0].device
    if device.type != "cuda":
        raise ValueError("bsa.tile_unlayout runs on a GPU")
    for n, x in enumerate(tiled):
        _require(x, f"tiled[{n}]", torch.bfloat16, device, 4)
        if x.shape != tiled[0].shape:
            raise ValueError("all tile buffers must share one shape")
    _require(token_row, "token_row", torch.int32, device, 1)
    B, H, rows, D = tiled[0].shape
    if tile not in TILES or rows % tile:
        raise ValueError("the tile buffers must hold a whole number of 64-, 128- or 256-row tiles")
    S_tok = token_row.shape[0] if tokens is None else tokens
    if token_row.shape[0] != S_tok:
        raise ValueError("token_row must have one entry per token")
    if outs is None:
        outs = [torch.empty((B, S_tok, H, D), dtype=torch.bfloat16, device=device) for _ in tiled]
    else:
        outs = list(outs)
        if len(outs) != len(tiled):
            raise ValueError("one output per input")
        for n, o in enumerate(outs):
            _require(o, f"out[{n}]", torch.bfloat16, device, 4)
            if tuple(o.shape) != (B, S_tok, H, D):
                raise ValueError("outputs must be [B, S_tok, H, D]")
    src_arr = (ctypes.c_void_p * len(tiled))(*[_ptr(x) for x in tiled])
    dst_arr = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    with torch.cuda.device(device):
        _check(lib.bsa_tile_unlayout(src_arr, dst_arr, len(tiled), _ptr(token_row), tile,
                                     B, S_tok, H, rows // tile, D, _stream_handle(device)))
    return outs


def cube_tile_map(latent, cube):
    """Maps of a video latent (t, h, w) tiled into cubes (ct, ch, cw), computed by the library
    on the host.

    Returns numpy int32 arrays ``(block_sizes [NT], tile_src_token [NT*tile],
    token_row [t*h*w])`` with tile = ct*ch*cw.
    """
    import numpy as np

    lib = load()
    t, h, w = (int(x) for x in latent)
    ct, ch, cw = (int(x) for x in cube)
    tile = ct * ch * cw
    nt = lib.bsa_cube_num_tiles(t, h, w, ct, ch, cw)
    if nt < 0:
        raise BsaError(1, f"invalid latent {latent} or cube {cube}")
    vbs = np.empty(nt, np.int32)
    src = np.empty(nt * tile, np.int32)
    row = np.empty(t * h * w, np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    _check(lib.bsa_cube_tile_map(t, h, w, ct, ch, cw, tile, vbs.ctypes.data_as(ip),
                                 src.ctypes.data_as(ip), row.ctypes.data_as(ip)))
    return vbs, src, row


def _fwd_args(q, k, v, q2k_idx, q2k_num, block_sizes, tile):
    import torch

    device = q.device
    if device.type != "cuda":
        raise ValueError("block-sparse attention runs on a GPU: q must be a cuda tensor")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, name, torch.bfloat16, device, 4)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    B, H, S, D = q.shape
    if tile not in TILES:
        raise ValueError(f"tile must be 64, 128 or 256, got {tile}")
    if S % tile:
        raise ValueError(f"sequence length {S} is not a multiple of the tile {tile}")
    NT = S // tile
    _require(q2k_idx, "q2k_idx", torch.int32, device, 4)
    _require(q2k_num, "q2k_num", torch.int32, device, 3)
    _require(block_sizes, "block_sizes", torch.int32, device, 1)
    if tuple(q2k_idx.shape[:3]) != (B, H, NT) or tuple(q2k_num.shape) != (B, H, NT):
        raise ValueError("q2k_idx must be [B, H, NT, MS] and q2k_num [B, H, NT]")
    if tuple(block_sizes.shape) != (NT,):
        raise ValueError("block_sizes must be [NT]")
    return device, B, H, S, D, NT


def fwd_lse(q, k, v, q2k_idx, q2k_num, block_sizes, tile, out=None, lse=None, out_lo=None,
            workspace="auto"):
    """``fwd`` that also returns the statistics the backward needs: (out, lse, out_lo)
    with lse float32 [B, H, NT*tile] (each row's log-sum-exp) and out_lo bf16 like out
    (the rounding residual of out: out + out_lo is the fp32 result)."""
    import torch

    lib = load()
    device, B, H, S, D, NT = _fwd_args(q, k, v, q2k_idx, q2k_num, block_sizes, tile)
    out = torch.empty_like(q) if out is None else out
    out_lo = torch.empty_like(q) if out_lo is None else out_lo
    lse = torch.empty((B, H, S), dtype=torch.float32, device=device) if lse is None else lse
    _require(out, "out", torch.bfloat16, device, 4)
    _require(out_lo, "out_lo", torch.bfloat16, device, 4)
    _require(lse, "lse", torch.float32, device, 3)
    if out.shape != q.shape or out_lo.shape != q.shape or tuple(lse.shape) != (B, H, S):
        raise ValueError("out and out_lo must have q's shape and lse [B, H, S]")
    MS = int(q2k_idx.shape[3])
    ws, ws_ptr, ws_bytes = _workspace(workspace, device, B, H, NT, tile, D, MS)
    with torch.cuda.device(device):
        _check(lib.bsa_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num),
                               _ptr(block_sizes), tile, _ptr(out), _ptr(out_lo), _ptr(lse), B, H,
                               NT, D, MS, ws_ptr, ws_bytes, _stream_handle(device)))
    return out, lse, out_lo


def bwd_k2q(q2k_idx, q2k_num, max_k=None):
    """Transposed tile lists for the backward: (k2q_idx int32 [B, H, NT, max_k],
    k2q_num int32 [B, H, NT] with the true lengths).  max_k defaults to NT, enough
    whenever the forward lists hold distinct tiles."""
    import torch

    lib = load()
    device = q2k_num.device
    _require(q2k_idx, "q2k_idx", torch.int32, device, 4)
    _require(q2k_num, "q2k_num", torch.int32, device, 3)
    B, H, NT, MS = q2k_idx.shape
    max_k = NT if max_k is None else int(max_k)
    k2q_idx = torch.empty((B, H, NT, max_k), dtype=torch.int32, device=device)
    k2q_num = torch.empty((B, H, NT), dtype=torch.int32, device=device)
    with torch.cuda.device(device):
        _check(lib.bsa_bwd_k2q(_ptr(q2k_idx), _ptr(q2k_num), B, H, NT, MS, _ptr(k2q_idx),
                               _ptr(k2q_num), max_k, _stream_handle(device)))
    return k2q_idx, k2q_num


def bwd(q, k, v, out, out_lo, dout, lse, q2k_idx, q2k_num, k2q_idx, k2q_num, block_sizes, tile,
        dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv), bf16 like q, of the block-sparse forward for the upstream
    gradient ``dout``; ``out``, ``out_lo`` and ``lse`` come from ``fwd_lse``, the
    transposed lists from ``bwd_k2q``."""
    import torch

    lib = load()
    device, B, H, S, D, NT = _fwd_args(q, k, v, q2k_idx, q2k_num, block_sizes, tile)
    for t, name in ((out, "out"), (out_lo, "out_lo"), (dout, "dout")):
        _require(t, name, torch.bfloat16, device, 4)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
    _require(lse, "lse", torch.float32, device, 3)
    _require(k2q_idx, "k2q_idx", torch.int32, device, 4)
    _require(k2q_num, "k2q_num", torch.int32, device, 3)
    if tuple(lse.shape) != (B, H, S) or tuple(k2q_idx.shape[:3]) != (B, H, NT) or \
            tuple(k2q_num.shape) != (B, H, NT):
        raise ValueError("lse must be [B, H, S], k2q_idx [B, H, NT, MK] and k2q_num [B, H, NT]")
    grads = []
    for g, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        g = torch.empty_like(q) if g is None else g
        _require(g, name, torch.bfloat16, device, 4)
        if g.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
        grads.append(g)
    delta = torch.empty((B, H, S), dtype=torch.float32, device=device)
    with torch.cuda.device(device):
        _check(lib.bsa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(dout),
                           _ptr(lse),
                           _ptr(q2k_idx), _ptr(q2k_num), _ptr(k2q_idx), _ptr(k2q_num),
                           _ptr(block_sizes), tile, _ptr(grads[0]), _ptr(grads[1]),
                           _ptr(grads[2]), _ptr(delta), B, H, NT, D, int(q2k_idx.shape[3]),
                           int(k2q_idx.shape[3]), _stream_handle(device)))
    return tuple(grads)


COARSE_MAX_TILES = 4096  # mirrored from include/bsa.h


def coarse_workspace_size(batch, heads, num_tiles, tile, head_dim):
    """Bytes of workspace ``coarse`` needs."""
    lib = load()
    n = ctypes.c_int64(0)
    _check(lib.bsa_coarse_workspace_size(batch, heads, num_tiles, tile, head_dim, ctypes.byref(n)))
    return int(n.value)


def _coarse_outputs(device, B, H, NT, D, topk, max_sel, coarse_out, q2k_idx, q2k_num):
    import torch

    MS = int(topk if max_sel is None else max_sel)
    if q2k_idx is None:
        q2k_idx = torch.empty((B, H, NT, MS), dtype=torch.int32, device=device)
    if q2k_num is None:
        q2k_num = torch.empty((B, H, NT), dtype=torch.int32, device=device)
    _require(q2k_idx, "q2k_idx", torch.int32, device, 4)
    _require(q2k_num, "q2k_num", torch.int32, device, 3)
    if tuple(q2k_idx.shape) != (B, H, NT, MS) or tuple(q2k_num.shape) != (B, H, NT):
        raise ValueError("q2k_idx must be [B, H, NT, max_sel] and q2k_num [B, H, NT]")
    oc = None
    if coarse_out is True:
        oc = torch.empty((B, H, NT, D), dtype=torch.float32, device=device)
    elif coarse_out is not None and coarse_out is not False:
        oc = coarse_out
        _require(oc, "coarse_out", torch.float32, device, 4)
        if tuple(oc.shape) != (B, H, NT, D):
            raise ValueError("coarse_out must be [B, H, NT, D]")
    return MS, q2k_idx, q2k_num, oc


def coarse(q, k, v, block_sizes, tile, topk, max_sel=None, coarse_out=True, q2k_idx=None,
           q2k_num=None, workspace=None):
    """Coarse stage on tiled q, k, v [B, H, NT*tile, D] (bf16, cuda): each query tile's key
    tiles and the coarse output.  Returns (q2k_idx int32 [B, H, NT, max_sel], q2k_num int32
    [B, H, NT], coarse_out float32 [B, H, NT, D] or None).  ``max_sel`` defaults to topk."""
    import torch

    lib = load()
    device = q.device
    if device.type != "cuda":
        raise ValueError("the coarse stage runs on a GPU: q must be a cuda tensor")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, name, torch.bfloat16, device, 4)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    B, H, S, D = q.shape
    if tile not in TILES or S % tile:
        raise ValueError(f"tile must be 64, 128 or 256 and divide the sequence ({S})")
    NT = S // tile
    _require(block_sizes, "block_sizes", torch.int32, device, 1)
    if tuple(block_sizes.shape) != (NT,):
        raise ValueError("block_sizes must be [NT]")
    MS, q2k_idx, q2k_num, oc = _coarse_outputs(device, B, H, NT, D, topk, max_sel, coarse_out,
                                               q2k_idx, q2k_num)
    with torch.cuda.device(device):
        need = coarse_workspace_size(B, H, NT, tile, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _require(workspace, "workspace", torch.uint8, device, 1)
    with torch.cuda.device(device):
        _check(lib.bsa_coarse(_ptr(q), _ptr(k), _ptr(v), _ptr(block_sizes), tile, int(topk),
                              _ptr(q2k_idx), _ptr(q2k_num), _ptr(oc), B, H, NT, D, MS,
                              _ptr(workspace), workspace.numel(), _stream_handle(device)))
    return q2k_idx, q2k_num, oc


def coarse_pooled(pooled, block_sizes, tile, topk, max_sel=None, coarse_out=True, q2k_idx=None,
                  q2k_num=None, workspace=None):
    """``coarse`` from pooled tiles already formed by ``tile_layout_pool`` (float32
    [3, B, H, NT, D]): the same lists, counts and coarse output, without reading q, k, v."""
    import torch

    lib = load()
    device = pooled.device
    if device.type != "cuda":
        raise ValueError("the coarse stage runs on a GPU: pooled must be a cuda tensor")
    _require(pooled, "pooled", torch.float32, device, 5)
    _, B, H, NT, D = pooled.shape
    if pooled.shape[0] != 3:
        raise ValueError("pooled must be [3, B, H, NT, D]")
    if tile not in TILES:
        raise ValueError("tile must be 64, 128 or 256")
    _require(block_sizes, "block_sizes", torch.int32, device, 1)
    if tuple(block_sizes.shape) != (NT,):
        raise ValueError("block_sizes must be [NT]")
    MS, q2k_idx, q2k_num, oc = _coarse_outputs(device, B, H, NT, D, topk, max_sel, coarse_out,
                                               q2k_idx, q2k_num)
    need = 4 * B * H * NT * NT
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _require(workspace, "workspace", torch.uint8, device, 1)
    with torch.cuda.device(device):
        _check(lib.bsa_coarse_pooled(_ptr(pooled), _ptr(block_sizes), tile, int(topk),
                                     _ptr(q2k_idx), _ptr(q2k_num), _ptr(oc), B, H, NT, D, MS,
                                     _ptr(workspace), workspace.numel(), _stream_handle(device)))
    return q2k_idx, q2k_num, oc


def coarse_combine(out, gate, coarse_out, block_sizes, tile):
    """In place: out = out + gate * coarse output of each valid row's tile (bf16, one
    rounding); padding rows keep their value.  Returns ``out``."""
    import torch

    lib = load()
    device = out.device
    _require(out, "out", torch.bfloat16, device, 4)
    _require(gate, "gate", torch.bfloat16, device, 4)
    _require(coarse_out, "coarse_out", torch.float32, device, 4)
    _require(block_sizes, "block_sizes", torch.int32, device, 1)
    B, H, S, D = out.shape
    if gate.shape != out.shape or tile not in TILES or S % tile:
        raise ValueError("gate must have out's shape and tile divide the sequence")
    NT = S // tile
    if tuple(coarse_out.shape) != (B, H, NT, D) or tuple(block_sizes.shape) != (NT,):
        raise ValueError("coarse_out must be [B, H, NT, D] and block_sizes [NT]")
    with torch.cuda.device(device):
        _check(lib.bsa_coarse_combine(_ptr(out), _ptr(gate), _ptr(coarse_out), _ptr(block_sizes),
                                      tile, B, H, NT, D, _stream_handle(device)))
    return out


def tile_unlayout_combine(out, gate, coarse_out, block_sizes, token_row, tile, tokens=None,
                          dst=None):
    """``coarse_combine`` then ``tile_unlayout`` in one pass, leaving ``out`` unchanged:
    the layer output gathered to token-major bf16 [B, S_tok, H, D]."""
    import torch

    lib = load()
    device = out.device
    _require(out, "out", torch.bfloat16, device, 4)
    _require(gate, "gate", torch.bfloat16, device, 4)
    _require(coarse_out, "coarse_out", torch.float32, device, 4)
    _require(block_sizes, "block_sizes", torch.int32, device, 1)
    _require(token_row, "token_row", torch.int32, device, 1)
    B, H, S, D = out.shape
    if gate.shape != out.shape or tile not in TILES or S % tile:
        raise ValueError("gate must have out's shape and tile divide the sequence")
    NT = S // tile
    if tuple(coarse_out.shape) != (B, H, NT, D) or tuple(block_sizes.shape) != (NT,):
        raise ValueError("coarse_out must be [B, H, NT, D] and block_sizes [NT]")
    S_tok = int(token_row.shape[0]) if tokens is None else int(tokens)
    if token_row.shape[0] != S_tok:
        raise ValueError("token_row must have one entry per token")
    if dst is None:
        dst = torch.empty((B, S_tok, H, D), dtype=torch.bfloat16, device=device)
    _require(dst, "dst", torch.bfloat16, device, 4)
    if tuple(dst.shape) != (B, S_tok, H, D):
        raise ValueError("dst must be [B, S_tok, H, D]")
    with torch.cuda.device(device):
        _check(lib.bsa_tile_unlayout_combine(_ptr(out), _ptr(gate), _ptr(coarse_out),
                                             _ptr(block_sizes), _ptr(token_row), tile, B, S_tok, H,
                                             NT, D, _ptr(dst), _stream_handle(device)))
    return dst
