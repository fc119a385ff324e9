"""Plain CPU oracle for block-sparse tiled attention and its token-to-tile layout.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
shares no code with it and never falls back to it.

The functions here follow the FastVideo fastvideo-kernel commit list (page 3):

* ``fwd`` / ``fwd_rows`` -- block-sparse softmax attention, the plain
  definition written out in ``bsa_oracle.c`` (binary32, the precision the pages'
  kernel tests compare against; see the 128-token sm_121a forward commit for the
  binding's arguments and the hardening commit for the zero-row, NaN-sum and
  padding-key rules).
* ``tile_layout`` -- the fused layout commit's scatter of token-major Q, K, V
  and the gate to their tile rows in B*H*S*D order, written as the gather it
  is equivalent to: output row t of head h reads token ``tile_src_token[t]`` of
  that head, and a row whose source is -1 is padding and holds +0.
* ``tile_unlayout`` -- the way back from the tile buffer to token-major order
  after attention: token n of head h reads tile row ``token_row[n]``.
* ``fwd64`` / ``bwd`` (module ``bsa_bwd``) -- the same forward in fp64 with
  its log-sum-exp, and its gradients dq, dk, dv (the pages' LSE-requiring
  autograd path; formulas in that module's docstring).
* ``coarse_pool`` / ``coarse_select`` / ``coarse`` -- the coarse stage that
  chooses each query tile's key tiles (``q2k_idx``, ``q2k_num``) and gives the
  coarse output.  The pages name the block-sparse kernel the fine attention
  but do not define this stage; the definition adopted is Video Sparse
  Attention's coarse stage, written out in ``bsa_oracle.c``: tiles pooled to
  the mean of their valid rows, binary32 logits of pooled queries against
  pooled keys, the top-k key tiles per query tile (ties to the lower index),
  and softmax attention over the pooled tokens.  Its pins
  (``tests/test_oracle_coarse_pins.py``) are fp64 library routines, brute
  force and hand-worked cases, not the pages (parity unpinned by the pages).
* ``cube_tile_map`` -- the tiling of a video latent into 3D cubes that the
  layout step applies (the pages name the scatter into tiles but not the cube
  shape; the cube is an argument, and the plainest order is taken: cubes
  row-major over the cube grid, tokens row-major inside a cube, padding rows
  last).

Parity pins for both live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

ERRORS = {
    -1: "invalid argument",
    -2: "key-tile index outside [0, NT)",
    -3: "q2k_num outside [0, MS]",
    -4: "tile length outside [0, T]",
    -5: "out of memory",
}


def build() -> str:
    """Compile the C oracle with the host compiler (IEEE semantics kept)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_bsa_fwd.argtypes = [p] * 6 + [i64] * 6 + [p, i32]
    lib.oracle_bsa_fwd.restype = i32
    lib.oracle_bsa_fwd_rows.argtypes = [p] * 6 + [i64] * 6 + [p, i64, p, i32]
    lib.oracle_bsa_fwd_rows.restype = i32
    lib.oracle_softmax_scale.argtypes = [i64]
    lib.oracle_softmax_scale.restype = ctypes.c_float
    lib.oracle_coarse_pool.argtypes = [p, p, i64, i64, i64, i64, p]
    lib.oracle_coarse_pool.restype = i32
    lib.oracle_coarse_select.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, p, p, p]
    lib.oracle_coarse_select.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _prep(q, k, v, q2k_idx, q2k_num, vbs, tile):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    q2k_num = np.ascontiguousarray(q2k_num, dtype=np.int32)
    vbs = np.ascontiguousarray(vbs, dtype=np.int32)
    B, H, S, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share the shape [B, H, NT*T, D]")
    if S % tile:
        raise ValueError("sequence is not a whole number of tiles")
    NT = S // tile
    if q2k_num.shape != (B, H, NT) or vbs.shape != (NT,):
        raise ValueError("q2k_num must be [B, H, NT] and block sizes [NT]")
    if q2k_idx is None:
        q2k_idx = np.zeros((B, H, NT, 0), np.int32)
    q2k_idx = np.ascontiguousarray(q2k_idx, dtype=np.int32)
    if q2k_idx.shape[:3] != (B, H, NT) or q2k_idx.ndim != 4:
        raise ValueError("q2k_idx must be [B, H, NT, MS]")
    MS = q2k_idx.shape[3]
    return q, k, v, q2k_idx, q2k_num, vbs, (B, H, NT, tile, D, MS)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, q2k_idx, q2k_num, vbs, tile, nthreads=None):
    """float32 [B, H, NT*T, D]: every row of the block-sparse attention output."""
    lib = _load()
    q, k, v, q2k_idx, q2k_num, vbs, dims = _prep(q, k, v, q2k_idx, q2k_num, vbs, tile)
    out = np.empty(q.shape, np.float32)
    rc = lib.oracle_bsa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num),
                            _ptr(vbs), *dims, _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem: {ERRORS.get(rc, rc)}")
    return out


def fwd_rows(q, k, v, q2k_idx, q2k_num, vbs, tile, rows, nthreads=None):
    """float32 [len(rows), D] for flat rows (b*H + h)*(NT*T) + t."""
    lib = _load()
    q, k, v, q2k_idx, q2k_num, vbs, dims = _prep(q, k, v, q2k_idx, q2k_num, vbs, tile)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, q.shape[3]), np.float32)
    rc = lib.oracle_bsa_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(q2k_idx), _ptr(q2k_num),
                                 _ptr(vbs), *dims, _ptr(rows), rows.size, _ptr(out),
                                 nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem: {ERRORS.get(rc, rc)}")
    return out


def softmax_scale(head_dim: int) -> float:
    """The binary32 scale 1/sqrt(D) the oracle multiplies q.k by."""
    return float(_load().oracle_softmax_scale(head_dim))


def tile_layout(srcs, tile_src_token, tile):
    """Gather token-major [B, S_tok, H, D] tensors into [B, H, NT*T, D] tiles.

    ``tile_src_token`` ([NT*T] int) names the source token of every tiled row;
    -1 marks a padding row, which is +0.  Values are moved bit for bit.
    """
    tile_src_token = np.asarray(tile_src_token, dtype=np.int64)
    if tile_src_token.ndim != 1 or tile_src_token.size % tile:
        raise ValueError("the map must hold NT*T entries")
    outs = []
    for x in srcs:
        x = np.asarray(x)
        B, S_tok, H, D = x.shape
        if np.any(tile_src_token >= S_tok) or np.any(tile_src_token < -1):
            raise ValueError("map entry outside [-1, S_tok)")
        out = np.zeros((B, H, tile_src_token.size, D), dtype=x.dtype)
        valid = tile_src_token >= 0
        # out[b, h, t, :] = x[b, src[t], h, :] for every valid row t
        out[:, :, valid, :] = np.transpose(x[:, tile_src_token[valid], :, :], (0, 2, 1, 3))
        outs.append(out)
    return outs


def tile_unlayout(tiled, token_row):
    """Gather [B, H, NT*T, D] tile buffers back to token-major [B, S_tok, H, D].

    Token n of head h reads tile row ``token_row[n]``; an entry outside the
    buffer gives a +0 row.  Values are moved bit for bit.
    """
    token_row = np.asarray(token_row, dtype=np.int64)
    outs = []
    for x in tiled:
        x = np.asarray(x)
        B, H, rows, D = x.shape
        out = np.zeros((B, token_row.size, H, D), dtype=x.dtype)
        ok = (token_row >= 0) & (token_row < rows)
        # out[b, n, h, :] = x[b, h, token_row[n], :] for every token n with a row
        out[:, ok, :, :] = np.transpose(x[:, :, token_row[ok], :], (0, 2, 1, 3))
        outs.append(out)
    return outs


def cube_tile_map(latent, cube):
    """Tiling of a t x h x w video latent (token (z*h + y)*w + x) into ct x ch x cw cubes.

    Returns ``(block_sizes [NT], tile_src_token [NT*T], token_row [t*h*w])``
    with T = ct*ch*cw and NT = ceil(t/ct)*ceil(h/ch)*ceil(w/cw).  Written per
    token: a token's cube is its coordinates divided by the cube, the cube
    index runs row-major over the cube grid, and its row inside the tile is its
    row-major rank within the cube's (edge-clipped) extent.
    """
    t, h, w = (int(x) for x in latent)
    ct, ch, cw = (int(x) for x in cube)
    tile = ct * ch * cw
    gz, gy, gx = -(-t // ct), -(-h // ch), -(-w // cw)
    n_tiles = gz * gy * gx
    block_sizes = np.zeros(n_tiles, np.int32)
    tile_src_token = np.full(n_tiles * tile, -1, np.int32)
    token_row = np.zeros(t * h * w, np.int32)
    for z in range(t):
        for y in range(h):
            for x in range(w):
                cz, cy, cx = z // ct, y // ch, x // cw
                c = (cz * gy + cy) * gx + cx
                ez = min(ct, t - cz * ct)  # extent of this cube after the edge cut
                ey = min(ch, h - cy * ch)
                ex = min(cw, w - cx * cw)
                rank = ((z - cz * ct) * ey + (y - cy * ch)) * ex + (x - cx * cw)
                token = (z * h + y) * w + x
                token_row[token] = c * tile + rank
                tile_src_token[c * tile + rank] = token
                block_sizes[c] = ez * ey * ex
    return block_sizes, tile_src_token, token_row


from .bsa_bwd import bwd, fwd64  # noqa: E402,F401


def coarse_pool(x, vbs, tile):
    """float32 [B, H, NT, D]: the mean of each tile's valid rows (rows summed in order in
    binary32, then divided by the count); 0 for a tile with no valid row."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    vbs = np.ascontiguousarray(vbs, dtype=np.int32)
    B, H, S, D = x.shape
    if S % tile or vbs.shape != (S // tile,):
        raise ValueError("x must be [B, H, NT*T, D] and block sizes [NT]")
    NT = S // tile
    xm = np.empty((B, H, NT, D), np.float32)
    rc = lib.oracle_coarse_pool(_ptr(x), _ptr(vbs), B * H, NT, tile, D, _ptr(xm))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem: {ERRORS.get(rc, rc)}")
    return xm


def coarse_select(qm, km, vm, vbs, topk, max_sel=None):
    """From pooled tensors [B, H, NT, D] (float32): (q2k_idx int32 [B, H, NT, max_sel],
    q2k_num int32 [B, H, NT], oc float32 [B, H, NT, D]).  Unused list entries are -1."""
    lib = _load()
    qm, km, vm = (np.ascontiguousarray(a, dtype=np.float32) for a in (qm, km, vm))
    vbs = np.ascontiguousarray(vbs, dtype=np.int32)
    B, H, NT, D = qm.shape
    MS = topk if max_sel is None else max_sel
    idx = np.empty((B, H, NT, MS), np.int32)
    num = np.empty((B, H, NT), np.int32)
    oc = np.empty((B, H, NT, D), np.float32)
    rc = lib.oracle_coarse_select(_ptr(qm), _ptr(km), _ptr(vm), _ptr(vbs), B * H, NT, D, topk, MS,
                                  _ptr(idx), _ptr(num), _ptr(oc))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem: {ERRORS.get(rc, rc)}")
    return idx, num, oc


def coarse(q, k, v, vbs, tile, topk, max_sel=None):
    """The whole coarse stage on tiled bf16 q, k, v [B, H, NT*T, D]: (q2k_idx, q2k_num, oc)."""
    return coarse_select(coarse_pool(q, vbs, tile), coarse_pool(k, vbs, tile),
                         coarse_pool(v, vbs, tile), vbs, topk, max_sel)
