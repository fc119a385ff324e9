"""Video-latent cube tiling and the inverse layout map (host side, no GPU).

The pages name the scatter that moves Q, K, V and gate tokens to tile rows
(FastVideo fastvideo-kernel commit list, page 3, fused-layout commit) but not
the cube shape or the order inside a cube; both readings are stated in the
oracle's docstring.  The oracle's map is pinned here to a hand-worked example
and to properties any correct tiling has; the library's map (C, host) must
equal it bit for bit.
"""
import ctypes

import numpy as np
import pytest

import block_sparse_tiled_amd as bsa
import oracle

OK, INVALID, SHAPE, LIMITS, NO_DEVICE = range(5)
FAKE = ctypes.c_void_p(0x1000)
NUL = ctypes.c_void_p(0)

LATENTS = [((21, 30, 52), (4, 4, 4)), ((5, 7, 9), (4, 4, 8)), ((3, 17, 33), (2, 8, 8)),
           ((4, 4, 4), (4, 4, 4)), ((1, 1, 1), (4, 4, 4)), ((9, 1, 70), (1, 1, 64)),
           ((21, 30, 52), (4, 8, 8))]


def test_hand_worked_example():
    """A 2 x 3 x 3 latent in 2 x 2 x 2 cubes, worked out on paper.

    Token index (z*3 + y)*3 + x.  Cube grid 1 x 2 x 2.  Cube 0 (y, x < 2) holds
    (0,0,0) (0,0,1) (0,1,0) (0,1,1) (1,0,0) (1,0,1) (1,1,0) (1,1,1) = 0 1 3 4 9
    10 12 13; cube 1 (y < 2, x = 2): 2 5 11 14; cube 2 (y = 2, x < 2): 6 7 15
    16; cube 3 (y = x = 2): 8 17.
    """
    vbs, src, row = oracle.cube_tile_map((2, 3, 3), (2, 2, 2))
    assert vbs.tolist() == [8, 4, 4, 2]
    pad = [-1] * 4
    assert src.tolist() == ([0, 1, 3, 4, 9, 10, 12, 13] + [2, 5, 11, 14] + pad
                            + [6, 7, 15, 16] + pad + [8, 17] + pad + [-1, -1])
    for token, r in enumerate(row):
        assert src[r] == token


@pytest.mark.parametrize("latent,cube", LATENTS)
def test_oracle_map_is_a_cube_tiling(latent, cube):
    t, h, w = latent
    ct, ch, cw = cube
    tile = ct * ch * cw
    vbs, src, row = oracle.cube_tile_map(latent, cube)
    gz, gy, gx = -(-t // ct), -(-h // ch), -(-w // cw)
    assert vbs.size == gz * gy * gx and src.size == vbs.size * tile and row.size == t * h * w
    assert int(vbs.sum()) == t * h * w
    # a permutation between tokens and the valid rows, with padding rows last in each tile
    assert np.array_equal(np.sort(row), np.sort(np.flatnonzero(src >= 0)))
    np.testing.assert_array_equal(src[row], np.arange(t * h * w))
    for c in range(vbs.size):
        rows = src[c * tile:(c + 1) * tile]
        assert np.all(rows[:vbs[c]] >= 0) and np.all(rows[vbs[c]:] == -1)
        z, rem = np.divmod(rows[:vbs[c]], h * w)
        y, x = np.divmod(rem, w)
        cz, cy, cx = np.unravel_index(c, (gz, gy, gx))
        # inside the cube, in row-major order (which is ascending token order)
        assert np.all(z // ct == cz) and np.all(y // ch == cy) and np.all(x // cw == cx)
        assert np.all(np.diff(rows[:vbs[c]]) > 0)
        assert vbs[c] == min(ct, t - cz * ct) * min(ch, h - cy * ch) * min(cw, w - cx * cw)


@pytest.mark.parametrize("latent,cube", LATENTS)
def test_library_map_equals_the_oracle(latent, cube):
    got = bsa.cube_tile_map(latent, cube)
    want = oracle.cube_tile_map(latent, cube)
    for g, e in zip(got, want):
        np.testing.assert_array_equal(g, e)


def test_unlayout_inverts_layout_in_the_oracle():
    """The oracle's two gathers compose to the identity on tokens (both directions)."""
    rng = np.random.default_rng(3)
    vbs, src, row = oracle.cube_tile_map((5, 6, 7), (4, 4, 4))
    x = rng.integers(0, 65536, size=(2, 5 * 6 * 7, 3, 64), dtype=np.uint16)
    (tiled,) = oracle.tile_layout([x], src, 64)
    (back,) = oracle.tile_unlayout([tiled], row)
    np.testing.assert_array_equal(back, x)
    # padding rows of the tile buffer are +0, so unlayout then layout restores it
    (again,) = oracle.tile_layout([back], src, 64)
    np.testing.assert_array_equal(again, tiled)
    # a token whose row is out of range comes back +0
    bad = row.copy()
    bad[[0, 5]] = [-1, tiled.shape[2]]
    (partial,) = oracle.tile_unlayout([tiled], bad)
    assert not partial[:, [0, 5]].any()
    np.testing.assert_array_equal(partial[:, 1:5], x[:, 1:5])


def test_cube_map_rejects_bad_arguments():
    lib = bsa.load()
    assert lib.bsa_cube_num_tiles(21, 30, 52, 4, 4, 4) == 624
    assert lib.bsa_cube_num_tiles(0, 30, 52, 4, 4, 4) == -1
    assert lib.bsa_cube_num_tiles(21, 30, 52, 4, 0, 4) == -1
    assert lib.bsa_cube_num_tiles(1 << 23, 1, 1, 1, 1, 1) == -1
    buf = (ctypes.c_int32 * 4096)()
    p = ctypes.cast(buf, ctypes.POINTER(ctypes.c_int32))
    assert lib.bsa_cube_tile_map(4, 4, 4, 4, 4, 4, 64, p, p, None) == INVALID
    assert lib.bsa_cube_tile_map(4, 4, 4, 4, 4, 2, 64, p, p, p) == INVALID  # 32 != 64
    assert lib.bsa_cube_tile_map(4, 4, 2, 4, 4, 2, 32, p, p, p) == SHAPE
    assert lib.bsa_cube_tile_map(4, 8, 16, 4, 8, 16, 512, p, p, p) == SHAPE
    assert lib.bsa_cube_tile_map(4, -4, 4, 4, 4, 4, 64, p, p, p) == INVALID
    with pytest.raises(bsa.BsaError):
        bsa.cube_tile_map((4, 4, 4), (4, 4, 3))


def test_unlayout_rejects_bad_arguments():
    lib = bsa.load()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    call = lambda n=1, tile=64, D=64, B=1, H=1, NT=1, tok=64, m=FAKE: lib.bsa_tile_unlayout(  # noqa
        arr, arr, n, m, tile, B, tok, H, NT, D, NUL)
    assert call(n=0) == INVALID
    assert call(n=5) == INVALID
    assert call(tile=96) == SHAPE
    assert call(tile=512) == SHAPE
    assert call(D=32) == SHAPE
    assert call(m=NUL) == INVALID
    assert call(tok=-1) == INVALID
    assert call(H=70000) == LIMITS
    assert call(B=0, m=NUL) == OK
    assert call(tok=0, m=NUL) == OK
