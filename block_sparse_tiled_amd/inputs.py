"""Seeded synthetic workloads for block-sparse tiled attention.

This module only draws inputs: tensors, tile lengths and tile lists.  It holds
none of the attention arithmetic, so both the GPU path and the CPU oracle can
consume exactly the same bytes.  All floating-point draws are binary32 normals
rounded to bfloat16 (round to nearest even); tensors are returned as uint16
bit patterns.

Workload shapes follow the five configurations the method is measured on (the
64- and 128-token tiles, ragged tile lengths, empty selections, the video
latent of 21x30x52 tokens and the dense 31200-token shape of the FastVideo
fastvideo-kernel commit list, page 3); the pages measure real FastWan
activations, which are not available, so seeded Gaussians stand in.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
BF16_POS_INF = np.uint16(0x7F80)
BF16_NEG_INF = np.uint16(0xFF80)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # only NaN patterns can wrap around here, and those are replaced below
    lsb = np.right_shift(u, 16)
    np.bitwise_and(lsb, 1, out=lsb)
    lsb += np.uint32(0x7FFF)
    lsb += u
    np.right_shift(lsb, 16, out=lsb)
    rounded = lsb.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to binary32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One problem instance.

    ``q, k, v`` are [B, H, NT*T, D] bf16 bits (the tile buffer); ``tok`` holds
    the same tensors token-major [B, S_tok, H, D] (plus ``gate``) with
    ``tile_src_token`` mapping every tiled row to its source token (-1 for a
    padding row).  ``q2k_idx`` is [B, H, NT, MS], ``q2k_num`` [B, H, NT] and
    ``vbs`` (variable block sizes) [NT], all int32.
    """

    name: str
    B: int
    H: int
    D: int
    T: int
    NT: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q2k_idx: np.ndarray
    q2k_num: np.ndarray
    vbs: np.ndarray
    tok: dict = field(default_factory=dict)
    tile_src_token: np.ndarray | None = None
    notes: dict = field(default_factory=dict)

    @property
    def MS(self) -> int:
        return int(self.q2k_idx.shape[3])

    @property
    def S(self) -> int:
        return self.NT * self.T

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k, self.v, self.q2k_idx, self.q2k_num, self.vbs):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def contiguous_map(vbs: np.ndarray, T: int) -> np.ndarray:
    """Tiled row -> source token for tiles filled in token order.

    Tile t holds tokens [start_t, start_t + vbs[t]) with start_t the sum of the
    earlier lengths; its remaining rows are padding (-1).
    """
    vbs = np.asarray(vbs, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(vbs)[:-1]])
    s = np.arange(T)[None, :]
    src = np.where(s < vbs[:, None], starts[:, None] + s, -1)
    return src.reshape(-1).astype(np.int32)


def place_tokens(tok: np.ndarray, src_map: np.ndarray) -> np.ndarray:
    """Put token-major rows [B, S_tok, H, D] into tile rows [B, H, NT*T, D] (+0 padding)."""
    B, _, H, D = tok.shape
    out = np.zeros((B, H, src_map.size, D), dtype=tok.dtype)
    rows = np.nonzero(src_map >= 0)[0]
    out[:, :, rows, :] = tok[:, src_map[rows], :, :].transpose(0, 2, 1, 3)
    return out


def fill_padding(x: np.ndarray, vbs: np.ndarray, T: int, pattern: str) -> None:
    """Overwrite the padding rows (r >= vbs[t]) of a tile buffer in place.

    ``pattern`` is ``"zero"``, ``"nan"``, ``"inf"``, ``"random"`` or
    ``"naninf"`` (NaN, +Inf, -Inf cycling over (r + d) mod 3).
    """
    B, H, S, D = x.shape
    NT = S // T
    r = np.arange(T)
    for t in range(NT):
        pad = r[r >= vbs[t]]
        if pad.size == 0:
            continue
        rows = t * T + pad
        if pattern == "zero":
            x[:, :, rows, :] = 0
        elif pattern == "nan":
            x[:, :, rows, :] = BF16_NAN
        elif pattern == "inf":
            x[:, :, rows, :] = BF16_POS_INF
        elif pattern == "random":
            rng = np.random.default_rng(1000 + t)
            x[:, :, rows, :] = to_bf16_bits(rng.standard_normal((B, H, rows.size, D), np.float32) * 64)
        elif pattern == "naninf":
            cyc = np.array([BF16_NAN, BF16_POS_INF, BF16_NEG_INF], np.uint16)
            sel = (pad[:, None] + np.arange(D)[None, :]) % 3
            x[:, :, rows, :] = cyc[sel][None, None]
        else:
            raise ValueError(pattern)


def _normals(rng, shape, sigma=1.0):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def _distinct(rng, n_total, n_pick, exclude=None):
    pool = np.arange(n_total)
    if exclude is not None:
        pool = np.setdiff1d(pool, exclude)
    return rng.choice(pool, size=n_pick, replace=False)


def build(name, B, H, D, T, vbs, counts_fn, pick_fn, rng, sigma=1.0, MS=None,
          gate=False, tok_hook=None):
    """Draw token-major tensors, tile them and draw the per-tile key lists.

    ``counts_fn(rng) -> int array [B, H, NT]`` gives q2k_num and
    ``pick_fn(rng, b, h, i, n) -> ids`` the distinct key tiles of one list.
    Unused list slots are filled with in-range poison ids, so a reader that
    goes past q2k_num picks up real tiles.
    """
    vbs = np.asarray(vbs, dtype=np.int32)
    NT = vbs.size
    S_tok = int(vbs.sum())
    tok = {}
    for key in ("q", "k", "v"):
        tok[key] = _normals(rng, (B, S_tok, H, D), sigma)
    if tok_hook is not None:
        tok_hook(tok)
    counts = np.asarray(counts_fn(rng), dtype=np.int32)
    MS = int(counts.max(initial=0)) if MS is None else MS
    MS = max(MS, 1)
    idx = rng.integers(0, NT, size=(B, H, NT, MS), dtype=np.int32)  # poison first
    for b in range(B):
        for h in range(H):
            for i in range(NT):
                n = int(counts[b, h, i])
                if n:
                    idx[b, h, i, :n] = np.sort(pick_fn(rng, b, h, i, n))
    if gate:
        tok["gate"] = _normals(rng, (B, S_tok, H, D), sigma)
    src = contiguous_map(vbs, T)
    tiled = {key: place_tokens(val, src) for key, val in tok.items() if key in ("q", "k", "v")}
    return Workload(name=name, B=B, H=H, D=D, T=T, NT=NT, q=tiled["q"], k=tiled["k"],
                    v=tiled["v"], q2k_idx=idx, q2k_num=counts, vbs=vbs, tok=tok,
                    tile_src_token=src)


# --- the five measured configurations -------------------------------------------------


def tiny(seed=0, gate=False):
    """B=1, H=2, D=64, 8 full tiles of 64; 3 distinct tiles per list, one list empty."""
    rng = np.random.default_rng(seed)
    B, H, NT, T = 1, 2, 8, 64
    vbs = np.full(NT, T, np.int32)

    def counts(rng):
        c = np.full((B, H, NT), 3, np.int32)
        c.reshape(-1)[rng.integers(0, B * H * NT)] = 0
        return c

    return build("tiny", B, H, 64, T, vbs, counts,
                 lambda rng, b, h, i, n: _distinct(rng, NT, n), rng, gate=gate)


def ragged(seed=1, gate=False):
    """B=1, H=12, D=128, 64 tiles of 128, lengths U{96..128} and a last tile of 57;
    38 of the 768 lists empty, the rest pick 16 of 64 tiles (25 %)."""
    rng = np.random.default_rng(seed)
    B, H, NT, T = 1, 12, 64, 128
    vbs = np.concatenate([rng.integers(96, 129, size=NT - 1), [57]]).astype(np.int32)

    def counts(rng):
        c = np.full((B, H, NT), 16, np.int32)
        c.reshape(-1)[rng.choice(B * H * NT, size=38, replace=False)] = 0
        return c

    return build("ragged", B, H, 128, T, vbs, counts,
                 lambda rng, b, h, i, n: _distinct(rng, NT, n), rng, MS=16, gate=gate)


def video_nearest_tiles(n_tokens=32760, dims=(21, 30, 52), T=64, n_near=8):
    """The n_near tiles whose token-coordinate centroids are closest to each tile's.

    Token n sits at (t, y, x) of the latent, x fastest; tile i holds tokens
    [T*i, T*i + T).  Ties go to the lower tile index; the set includes i.
    """
    n = np.arange(n_tokens)
    coords = np.stack([n // (dims[1] * dims[2]), (n // dims[2]) % dims[1], n % dims[2]], 1)
    NT = -(-n_tokens // T)
    tile = n // T
    cent = np.zeros((NT, 3))
    np.add.at(cent, tile, coords.astype(np.float64))
    cent /= np.bincount(tile, minlength=NT)[:, None]
    d2 = ((cent[:, None, :] - cent[None, :, :]) ** 2).sum(-1)
    order = np.lexsort((np.broadcast_to(np.arange(NT), d2.shape), d2), axis=1)
    return order[:, :n_near].astype(np.int32)


def video(seed=2, gate=False):
    """B=1, H=12, D=128, 32760 tokens (21x30x52) in 512 tiles of 64 (last 56);
    N(0, 0.5); 8 spatially nearest tiles plus 24 random ones per list."""
    rng = np.random.default_rng(seed)
    B, H, T, n_tok = 1, 12, 64, 32760
    NT = -(-n_tok // T)
    vbs = np.full(NT, T, np.int32)
    vbs[-1] = n_tok - T * (NT - 1)
    near = video_nearest_tiles(n_tok, (21, 30, 52), T, 8)

    def pick(rng, b, h, i, n):
        far = _distinct(rng, NT, n - near.shape[1], exclude=near[i])
        return np.concatenate([near[i], far])

    w = build("video", B, H, 128, T, vbs, lambda rng: np.full((B, H, NT), 32, np.int32),
              pick, rng, sigma=0.5, MS=32, gate=gate)
    w.notes["nearest"] = near
    return w


def video_cube_tiles(dims=(21, 30, 52), cube=(4, 4, 4), n_near=8):
    """A t x h x w latent cut into ct x ch x cw cubes, numbered row-major over the cube
    grid: each cube's token count (edge cubes clipped) and the n_near cubes whose token
    centroids are closest to its own (ties to the lower index; the set includes the cube).
    Token n sits at (t, y, x), x fastest."""
    n = np.arange(int(np.prod(dims)))
    coords = np.stack([n // (dims[1] * dims[2]), (n // dims[2]) % dims[1], n % dims[2]], 1)
    grid = [-(-d // c) for d, c in zip(dims, cube)]
    cid = ((coords[:, 0] // cube[0]) * grid[1] + coords[:, 1] // cube[1]) * grid[2] + coords[:, 2] // cube[2]
    NT = int(np.prod(grid))
    counts = np.bincount(cid, minlength=NT)
    cent = np.zeros((NT, 3))
    np.add.at(cent, cid, coords.astype(np.float64))
    cent /= counts[:, None]
    d2 = ((cent[:, None, :] - cent[None, :, :]) ** 2).sum(-1)
    order = np.lexsort((np.broadcast_to(np.arange(NT), d2.shape), d2), axis=1)
    return counts.astype(np.int32), order[:, :n_near].astype(np.int32)


def video_cube(seed=7, gate=False):
    """The video shape in the cube tiling: B=1, H=12, D=128, the 21x30x52 latent in
    4x4x4 cubes, one tile of 64 per cube: 455 whole cubes and 169 edge cubes of 32, 16
    or 8 tokens; N(0, 0.5); the 8 nearest cubes plus 24 random ones per list.  Tokens are
    drawn independently, so each cube's tokens are placed tile by tile (the cube map's
    gather belongs to the layout step)."""
    rng = np.random.default_rng(seed)
    B, H, T = 1, 12, 64
    vbs, near = video_cube_tiles((21, 30, 52), (4, 4, 4), 8)
    NT = vbs.size

    def pick(rng, b, h, i, n):
        far = _distinct(rng, NT, n - near.shape[1], exclude=near[i])
        return np.concatenate([near[i], far])

    w = build("video_cube", B, H, 128, T, vbs, lambda rng: np.full((B, H, NT), 32, np.int32),
              pick, rng, sigma=0.5, MS=32, gate=gate)
    w.notes["nearest"] = near
    return w


def dense(seed=3, gate=False, density_tiles=None, name="dense"):
    """B=1, H=6, D=128, 31200 tokens in 244 tiles of 128 (last 96); every list holds
    every tile in order (or ``density_tiles`` random ones)."""
    rng = np.random.default_rng(seed)
    B, H, NT, T = 1, 6, 244, 128
    vbs = np.full(NT, T, np.int32)
    vbs[-1] = 31200 - T * (NT - 1)
    n = NT if density_tiles is None else density_tiles
    if density_tiles is None:
        pick = lambda rng, b, h, i, n: np.arange(NT)  # noqa: E731
    else:
        pick = lambda rng, b, h, i, n: _distinct(rng, NT, n)  # noqa: E731
    return build(name, B, H, 128, T, vbs, lambda rng: np.full((B, H, NT), n, np.int32),
                 pick, rng, MS=n, gate=gate)


def dense256(seed=6, gate=False):
    """The dense shape in 256-token tiles: B=1, H=6, D=128, 31200 tokens in 122 tiles of 256
    (last 224); every list holds every tile in order."""
    rng = np.random.default_rng(seed)
    B, H, NT, T = 1, 6, 122, 256
    vbs = np.full(NT, T, np.int32)
    vbs[-1] = 31200 - T * (NT - 1)
    return build("dense256", B, H, 128, T, vbs, lambda rng: np.full((B, H, NT), NT, np.int32),
                 lambda rng, b, h, i, n: np.arange(NT), rng, MS=NT, gate=gate)


def dense25(seed=5, gate=False):
    """The dense shape at 25 % tile density: 61 random tiles of 244 per list."""
    return dense(seed, gate, density_tiles=61, name="dense25")


def stress(seed=4, gate=False):
    """B=8, H=12, D=128, 128 tiles of 128 with lengths U{1..128}; q2k_num U{0..128};
    K/V padding rows hold NaN/+Inf/-Inf; one query row has only -inf logits."""
    rng = np.random.default_rng(seed)
    B, H, NT, T = 8, 12, 128, 128
    vbs = rng.integers(1, 129, size=NT).astype(np.int32)
    S_tok = int(vbs.sum())
    w = build("stress", B, H, 128, T, vbs,
              lambda rng: rng.integers(0, NT + 1, size=(B, H, NT)),
              lambda rng, b, h, i, n: _distinct(rng, NT, n), rng, MS=NT, gate=gate)
    # the all-(-inf) query row: q = (-inf, 0, ..., 0) against keys whose column 0 > 0
    cand = np.argwhere(w.q2k_num >= 1)
    b, h, i = cand[rng.integers(0, len(cand))]
    r = int(rng.integers(0, vbs[i]))
    token = int(np.concatenate([[0], np.cumsum(vbs)])[i]) + r
    qrow = np.zeros(w.D, np.uint16)
    qrow[0] = BF16_NEG_INF
    w.tok["q"][b, token, h, :] = qrow
    kcol = bf16_bits_to_f32(w.tok["k"][b, :, h, 0])
    w.tok["k"][b, :, h, 0] = to_bf16_bits(np.abs(kcol) + 1.0)
    src = w.tile_src_token
    w.q = place_tokens(w.tok["q"], src)
    w.k = place_tokens(w.tok["k"], src)
    fill_padding(w.k, vbs, T, "naninf")
    fill_padding(w.v, vbs, T, "naninf")
    w.notes["neg_inf_row"] = (int(b), int(h), int(i) * T + r)
    assert S_tok == w.tok["q"].shape[1]
    return w


CONFIGS = {
    "tiny": tiny,
    "ragged": ragged,
    "video": video,
    "dense": dense,
    "stress": stress,
    "dense25": dense25,
    "dense256": dense256,
    "video_cube": video_cube,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)


def random_problem(seed, B, H, D, T, vbs, counts=None, density=0.5, sigma=1.0, MS=None,
                   pad="zero", duplicates=False):
    """A small seeded problem for parity sweeps: arbitrary tile lengths, list sizes and
    padding contents.  ``counts`` (if given) fixes q2k_num for every list."""
    rng = np.random.default_rng(seed)
    vbs = np.asarray(vbs, np.int32)
    NT = vbs.size

    def count_fn(rng):
        if counts is not None:
            return np.broadcast_to(np.asarray(counts, np.int32), (B, H, NT)).copy()
        return rng.binomial(NT, density, size=(B, H, NT))

    def pick(rng, b, h, i, n):
        if duplicates:
            return rng.integers(0, NT, size=n)
        return _distinct(rng, NT, n)

    w = build("random", B, H, D, T, vbs, count_fn, pick, rng, sigma=sigma,
              MS=MS if MS is not None else NT)
    for x in (w.q, w.k, w.v):
        fill_padding(x, vbs, T, pad)
    return w
