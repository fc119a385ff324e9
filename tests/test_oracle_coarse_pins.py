"""Pins of the coarse-stage oracle (oracle.coarse_pool / coarse_select / coarse).

The pages leave the choice of q2k_idx to a stage they do not define (parity
unpinned by the pages); the oracle follows Video Sparse Attention's coarse
stage.  These CPU tests tie it to things other than itself: fp64 NumPy means,
brute-force fp64 ranking, PyTorch's scaled_dot_product_attention in fp64 on the
pooled tokens, and a hand-worked ranking with ties, NaN and empty tiles.
"""
import numpy as np
import pytest

import oracle
from block_sparse_tiled_amd import inputs as gen


def bf16(x):
    return gen.to_bf16_bits(np.asarray(x, np.float32))


def test_pool_is_the_mean_of_the_valid_rows():
    rng = np.random.default_rng(0)
    T, D, vbs = 64, 64, np.array([64, 1, 0, 17, 63], np.int32)
    x = bf16(rng.standard_normal((2, 3, T * vbs.size, D)))
    xf = gen.bf16_bits_to_f32(x).astype(np.float64)
    got = oracle.coarse_pool(x, vbs, T)
    for t, n in enumerate(vbs):
        want = xf[:, :, t * T:t * T + n].mean(axis=2) if n else np.zeros((2, 3, D))
        np.testing.assert_allclose(got[:, :, t], want, rtol=0, atol=1e-6)
    # padding rows are never read
    x2 = x.copy()
    for t, n in enumerate(vbs):
        x2[:, :, t * T + n:(t + 1) * T] = 0x7FC0  # NaN
    np.testing.assert_array_equal(oracle.coarse_pool(x2, vbs, T), got)


def _pooled(g_row, D=64):
    """Pooled q (one tile, e0) and pooled k with the given logits along e0."""
    qm = np.zeros((1, 1, len(g_row), D), np.float32)
    km = np.zeros_like(qm)
    qm[0, 0, :, 0] = 1.0
    km[0, 0, :, 0] = g_row
    return qm, km


def test_hand_worked_ranking():
    """Logits (per key tile, the same for every query tile) 0.5, 2, -1, 2, 3: the order
    is 4, 1, 3 (1 before 3 on the tie), 0, 2."""
    g = np.array([0.5, 2.0, -1.0, 2.0, 3.0], np.float32)
    qm, km = _pooled(g)
    vbs = np.full(5, 64, np.int32)
    for topk, want in ((1, [4]), (2, [1, 4]), (3, [1, 3, 4]), (4, [0, 1, 3, 4]), (5, [0, 1, 2, 3, 4]),
                       (7, [0, 1, 2, 3, 4])):
        idx, num, _ = oracle.coarse_select(qm, km, km, vbs, topk, max_sel=7)
        assert np.all(num == len(want))
        for i in range(5):
            assert idx[0, 0, i, :len(want)].tolist() == want, (topk, i)
            assert np.all(idx[0, 0, i, len(want):] == -1)


def test_ties_nan_signed_zero_and_empty_tiles():
    # equal logits everywhere: the lowest indices win
    qm, km = _pooled(np.ones(6, np.float32))
    idx, num, _ = oracle.coarse_select(qm, km, km, np.full(6, 8, np.int32), 3)
    assert np.all(idx[0, 0, :, :3] == [0, 1, 2]) and np.all(num == 3)
    # a NaN logit ranks as -inf; -0 and +0 tie (lower index first)
    g = np.array([np.nan, -np.inf, -0.0, 0.0, -5.0], np.float32)
    qm, km = _pooled(g)
    idx, _, _ = oracle.coarse_select(qm, km, km, np.full(5, 8, np.int32), 2)
    assert idx[0, 0, 0, :2].tolist() == [2, 3]
    idx, _, _ = oracle.coarse_select(qm, km, km, np.full(5, 8, np.int32), 4)
    # -5 is fourth of the finite ones; then NaN (tile 0) and -inf (tile 1) tie at -inf
    assert idx[0, 0, 0, :4].tolist() == [0, 2, 3, 4]
    idx, _, _ = oracle.coarse_select(qm, km, km, np.full(5, 8, np.int32), 3)
    assert idx[0, 0, 0, :3].tolist() == [2, 3, 4]
    # empty key tiles are never candidates; an empty query tile keeps nothing
    g = np.array([5.0, 4.0, 3.0, 2.0], np.float32)
    qm, km = _pooled(g)
    vbs = np.array([8, 0, 8, 8], np.int32)
    idx, num, oc = oracle.coarse_select(qm, km, km, vbs, 2, max_sel=3)
    assert idx[0, 0, 0].tolist() == [0, 2, -1] and num[0, 0, 0] == 2
    assert idx[0, 0, 1].tolist() == [-1, -1, -1] and num[0, 0, 1] == 0
    assert np.all(oc[0, 0, 1] == 0)
    # more requested than there are candidates: all of them
    idx, num, _ = oracle.coarse_select(qm, km, km, vbs, 4, max_sel=4)
    assert idx[0, 0, 0].tolist() == [0, 2, 3, -1] and num[0, 0, 0] == 3


@pytest.mark.parametrize("seed", range(6))
def test_selection_against_brute_force_fp64(seed):
    """The kept set equals the top-k of the fp64 logits (ties to the lower index),
    except where the k-th and (k+1)-th fp64 logits lie within the binary32 error bound
    of a dot product; there either choice is accepted, and the kept logits must all be
    at least the k-th largest minus that bound."""
    rng = np.random.default_rng(100 + seed)
    B, H, NT, D = 1, 2, int(rng.integers(3, 40)), int(rng.choice([64, 128]))
    topk = int(rng.integers(1, NT + 2))
    vbs = rng.integers(0, 3, NT).astype(np.int32) * 32
    qm = rng.standard_normal((B, H, NT, D)).astype(np.float32)
    km = rng.standard_normal((B, H, NT, D)).astype(np.float32)
    idx, num, _ = oracle.coarse_select(qm, km, km, vbs, topk, max_sel=NT + 2)
    cand = [j for j in range(NT) if vbs[j] > 0]
    for b in range(B):
        for h in range(H):
            g64 = qm[b, h].astype(np.float64) @ km[b, h].astype(np.float64).T
            bound = D * 2.0 ** -23 * (np.abs(qm[b, h]).astype(np.float64) @ np.abs(km[b, h]).T)
            for i in range(NT):
                n = int(num[b, h, i])
                kept = idx[b, h, i, :n].tolist()
                if vbs[i] == 0:
                    assert n == 0
                    continue
                k = min(topk, len(cand))
                assert n == k and kept == sorted(kept) and set(kept) <= set(cand)
                order = sorted(cand, key=lambda j: (-g64[i, j], j))
                if k < len(cand) and g64[i, order[k - 1]] - g64[i, order[k]] <= 2 * bound[i].max():
                    kth = g64[i, order[k - 1]]
                    assert all(g64[i, j] >= kth - 2 * bound[i].max() for j in kept)
                else:
                    assert set(kept) == set(order[:k])


def test_coarse_output_is_attention_over_pooled_tokens():
    """oc = softmax(scale * qm km^T) vm over the non-empty key tiles: PyTorch's SDPA in
    fp64 with a key mask, as a library routine."""
    import torch

    rng = np.random.default_rng(7)
    B, H, NT, D = 2, 3, 11, 128
    vbs = np.array([8, 0, 8, 8, 1, 8, 8, 0, 8, 8, 8], np.int32)
    qm, km, vm = (rng.standard_normal((B, H, NT, D)).astype(np.float32) for _ in range(3))
    _, _, oc = oracle.coarse_select(qm, km, vm, vbs, 3)
    mask = torch.from_numpy(vbs > 0)[None, None, None, :].expand(B, H, NT, NT)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qm).double(), torch.from_numpy(km).double(), torch.from_numpy(vm).double(),
        attn_mask=mask).numpy()
    want[:, :, vbs == 0] = 0.0  # empty query tiles give 0
    np.testing.assert_allclose(oc, want, rtol=0, atol=2e-5)


def test_whole_stage_on_tiled_inputs():
    """coarse() on tiled bf16 tensors equals pooling then selection; with topk at least
    the number of non-empty tiles every non-empty query tile lists every non-empty key
    tile; NaN padding rows change nothing."""
    rng = np.random.default_rng(9)
    T, D, vbs = 64, 64, np.array([64, 40, 0, 64, 3], np.int32)
    q, k, v = (bf16(rng.standard_normal((1, 2, T * vbs.size, D))) for _ in range(3))
    idx, num, oc = oracle.coarse(q, k, v, vbs, T, 2)
    pm = [oracle.coarse_pool(x, vbs, T) for x in (q, k, v)]
    idx2, num2, oc2 = oracle.coarse_select(*pm, vbs, 2)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(num, num2)
    np.testing.assert_array_equal(oc, oc2)
    full, fnum, _ = oracle.coarse(q, k, v, vbs, T, 9, max_sel=9)
    for i in range(vbs.size):
        want = [0, 1, 3, 4] if vbs[i] else []
        assert full[0, 0, i, :fnum[0, 0, i]].tolist() == want
    pad = [x.copy() for x in (q, k, v)]
    for x in pad:
        for t, n in enumerate(vbs):
            x[:, :, t * T + n:(t + 1) * T] = 0x7F80  # +Inf
    idx3, num3, oc3 = oracle.coarse(*pad, vbs, T, 2)
    np.testing.assert_array_equal(idx3, idx)
    np.testing.assert_array_equal(oc3, oc)
