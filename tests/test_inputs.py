"""The seeded workload generators: determinism and the shapes the pages print."""
import json
import os

import numpy as np
import pytest

from block_sparse_tiled_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as f:
        return json.load(f)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, np.inf, -np.inf], np.float32)
    bits = gen.to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert list(bits) == [0x3F80, 0x3F80, 0x3F81, 0x3F81, 0xC020, 0x7F80, 0xFF80]
    assert np.isnan(gen.bf16_bits_to_f32(gen.to_bf16_bits(np.float32([np.nan])))).all()


def test_tiny_is_deterministic_and_matches_its_recipe():
    a, b = gen.tiny(), gen.tiny()
    assert a.digest() == b.digest()
    assert a.q.shape == (1, 2, 512, 64) and a.MS == 3
    assert (a.q2k_num == 0).sum() == 1 and (a.q2k_num == 3).sum() == 15
    for lst, n in zip(a.q2k_idx.reshape(-1, 3), a.q2k_num.reshape(-1)):
        if n:
            assert len(set(lst.tolist())) == 3 and list(lst) == sorted(lst)
    assert gen.tiny(seed=7).digest() != a.digest()


def test_ragged_recipe():
    w = gen.ragged()
    assert w.q.shape == (1, 12, 64 * 128, 128)
    assert w.vbs[-1] == 57 and w.vbs[:-1].min() >= 96 and w.vbs[:-1].max() <= 128
    assert (w.q2k_num == 0).sum() == 38 and set(np.unique(w.q2k_num)) == {0, 16}
    assert w.MS == 16
    # unused slots of an empty list still hold in-range tile ids (poison)
    empty = w.q2k_idx[w.q2k_num == 0]
    assert empty.min() >= 0 and empty.max() < 64


def test_video_recipe(page):
    w = gen.video()
    assert 21 * 30 * 52 == 32760 and int(w.vbs.sum()) == 32760
    assert w.NT == 512 and w.vbs[-1] == 56 and w.T in page["tile_sizes"]["values"]
    near = w.notes["nearest"]
    assert (near[:, 0] == np.arange(512)).all(), "a tile is its own nearest tile"
    for i in (0, 100, 511):
        for h in range(12):
            lst = w.q2k_idx[0, h, i]
            assert set(near[i]) <= set(lst.tolist()) and len(set(lst.tolist())) == 32


def test_video_cube_recipe():
    w = gen.video_cube()
    # 21 x 30 x 52 in 4 x 4 x 4 cubes: 6 x 8 x 13 cubes, clipped to 1 frame and 2 rows at the edges
    assert w.NT == 6 * 8 * 13 and int(w.vbs.sum()) == 21 * 30 * 52 and w.T == 64
    sizes, n = np.unique(w.vbs, return_counts=True)
    assert dict(zip(sizes.tolist(), n.tolist())) == {8: 13, 16: 91, 32: 65, 64: 455}
    assert w.vbs[0] == 64 and w.vbs[7 * 13] == 32 and w.vbs[5 * 8 * 13] == 16 and w.vbs[-1] == 8
    near = w.notes["nearest"]
    assert (near[:, 0] == np.arange(w.NT)).all(), "a cube is its own nearest cube"
    for i in (0, 300, w.NT - 1):
        lst = w.q2k_idx[0, 3, i]
        assert set(near[i]) <= set(lst.tolist()) and len(set(lst.tolist())) == 32


def test_dense_recipe(page):
    w = gen.dense()
    assert w.H == page["dense_shape"]["heads"]
    assert int(w.vbs.sum()) == page["dense_shape"]["tokens"] and w.NT == 244 and w.vbs[-1] == 96
    assert (w.q2k_idx == np.arange(244)).all() and (w.q2k_num == 244).all()


@pytest.mark.slow
def test_stress_recipe():
    w = gen.stress()
    assert w.q.shape == (8, 12, 16384, 128)
    assert w.vbs.min() >= 1 and w.vbs.max() <= 128
    assert w.q2k_num.min() >= 0 and w.q2k_num.max() <= 128
    b, h, row = w.notes["neg_inf_row"]
    qrow = gen.bf16_bits_to_f32(w.q[b, h, row])
    assert qrow[0] == -np.inf and (qrow[1:] == 0).all()
    valid = gen.contiguous_map(w.vbs, 128) >= 0
    assert (gen.bf16_bits_to_f32(w.k[b, h, valid, 0]) > 0).all()
    pad_v = gen.bf16_bits_to_f32(w.v[0, 0, ~valid])
    assert np.isnan(pad_v).any() and np.isposinf(pad_v).any() and np.isneginf(pad_v).any()


def test_contiguous_map_is_token_order():
    m = gen.contiguous_map(np.array([3, 0, 2]), 4)
    assert m.tolist() == [0, 1, 2, -1, -1, -1, -1, -1, 3, 4, -1, -1]
