"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test names what it pins the oracle to: textbook softmax attention in fp64
(NumPy and PyTorch's scaled_dot_product_attention), an independent pure-Python
fp64 loop, closed forms, invariants and the special-value rules of the
FastVideo fastvideo-kernel commit list (page 3, hardening commit: NaN softmax
sum gives a NaN row, rows without keys stay zero, padding keys never reach the
output).
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_tiled_amd import inputs as gen

F32 = gen.bf16_bits_to_f32


def scale_of(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def key_mask(w):
    """bool [B, H, S, S]: query row attends key row (True = attend)."""
    B, H, S, T, NT = w.B, w.H, w.S, w.T, w.NT
    mask = np.zeros((B, H, S, S), bool)
    r = np.arange(T)
    for b in range(B):
        for h in range(H):
            for i in range(NT):
                qrows = i * T + r[r < w.vbs[i]]
                for n in range(int(w.q2k_num[b, h, i])):
                    j = int(w.q2k_idx[b, h, i, n])
                    krows = j * T + r[r < w.vbs[j]]
                    mask[b, h, qrows[:, None], krows[None, :]] = True
    return mask


def sdpa_fp64(w, mask):
    # SDPA multiplies masked keys by a zero weight, so NaN padding would leak into
    # its result; the padding rows (which the mask never selects) are cleared first.
    valid = gen.contiguous_map(w.vbs, w.T) >= 0
    q, k, v = (np.where(valid[None, None, :, None], F32(x).astype(np.float64), 0.0)
               for x in (w.q, w.k, w.v))
    q, k, v = torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    m = torch.from_numpy(mask)
    # rows without any key are excluded by the caller; give them one key so SDPA stays finite
    safe = m.clone()
    safe[..., 0] |= ~m.any(-1)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=safe,
                                                           scale=scale_of(w.D))
    return out.numpy()


def python_bruteforce(w):
    """Independent fp64 loops: the definition, written without NumPy reductions."""
    qf, kf, vf = (F32(x).astype(np.float64) for x in (w.q, w.k, w.v))
    out = np.zeros(w.q.shape, np.float64)
    sc = scale_of(w.D)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(w.NT):
                keys = []
                for n in range(int(w.q2k_num[b, h, i])):
                    j = int(w.q2k_idx[b, h, i, n])
                    keys += [j * w.T + c for c in range(int(w.vbs[j]))]
                for r in range(int(w.vbs[i])):
                    row = i * w.T + r
                    if not keys:
                        continue
                    s = []
                    for key in keys:
                        acc = 0.0
                        for d in range(w.D):
                            acc += qf[b, h, row, d] * kf[b, h, key, d]
                        s.append(sc * acc)
                    m = max(s)
                    p = [math.exp(x - m) for x in s]
                    l = sum(p)
                    for d in range(w.D):
                        out[b, h, row, d] = sum(p[t] * vf[b, h, key, d]
                                                for t, key in enumerate(keys)) / l
    return out


def run_oracle(oracle_mod, w, **kw):
    return oracle_mod.fwd(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, **kw)


def rows_with_keys(w):
    has = np.zeros((w.B, w.H, w.S), bool)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(w.NT):
                n = int(w.q2k_num[b, h, i])
                tot = sum(int(w.vbs[w.q2k_idx[b, h, i, x]]) for x in range(n))
                if tot:
                    has[b, h, i * w.T: i * w.T + w.vbs[i]] = True
    return has


def test_softmax_scale_is_binary32_inverse_sqrt(oracle_mod):
    assert oracle_mod.softmax_scale(64) == 0.125
    assert oracle_mod.softmax_scale(128) == float(np.float32(1 / math.sqrt(128)))


def test_dense_full_tiles_match_fp64_textbook_attention(oracle_mod):
    """Every tile listed, every tile full: plain softmax(q k^T / sqrt(D)) v."""
    w = gen.random_problem(11, B=1, H=2, D=64, T=64, vbs=[64] * 3, counts=3)
    out = run_oracle(oracle_mod, w)
    qf, kf, vf = (F32(x).astype(np.float64) for x in (w.q, w.k, w.v))
    s = np.einsum("bhqd,bhkd->bhqk", qf, kf) * scale_of(64)
    p = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("bhqk,bhkd->bhqd", p / p.sum(-1, keepdims=True), vf)
    np.testing.assert_allclose(out, ref, atol=2e-6, rtol=1e-5)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qf), torch.from_numpy(kf), torch.from_numpy(vf),
        scale=scale_of(64)).numpy()
    np.testing.assert_allclose(out, sdpa, atol=2e-6, rtol=1e-5)


@pytest.mark.parametrize("D,T", [(64, 64), (128, 128)])
def test_ragged_all_selected_matches_sdpa_on_compacted_tokens(oracle_mod, D, T):
    """Ragged tiles with every tile listed equal dense attention over the valid tokens."""
    vbs = [T, 17, T // 2 + 3, 1] if T == 64 else [T, 100, 57]
    w = gen.random_problem(12, B=2, H=2, D=D, T=T, vbs=vbs, counts=len(vbs), pad="random")
    out = run_oracle(oracle_mod, w)
    valid = gen.contiguous_map(w.vbs, T) >= 0
    qf, kf, vf = (torch.from_numpy(F32(x)[:, :, valid].astype(np.float64)) for x in (w.q, w.k, w.v))
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, scale=scale_of(D)).numpy()
    np.testing.assert_allclose(out[:, :, valid], ref, atol=2e-6, rtol=1e-5)
    pad = out[:, :, ~valid]
    assert np.all(pad.view(np.uint32) == 0), "padding query rows must be +0"


@pytest.mark.parametrize("seed,D,T,vbs", [
    (13, 64, 64, [64, 64, 40, 64, 9, 0, 64]),
    (14, 128, 128, [128, 77, 128, 3, 128]),
])
def test_block_mask_matches_masked_sdpa(oracle_mod, seed, D, T, vbs):
    """General block mask == fp64 SDPA with the token-level boolean mask (True = attend)."""
    w = gen.random_problem(seed, B=1, H=3, D=D, T=T, vbs=vbs, density=0.45, pad="nan")
    out = run_oracle(oracle_mod, w)
    mask = key_mask(w)
    has = mask.any(-1)
    assert has.sum() > 0 and (~has).sum() > 0
    ref = sdpa_fp64(w, mask)
    np.testing.assert_allclose(out[has], ref[has], atol=2e-6, rtol=1e-5)
    assert np.all(out[~has].view(np.uint32) == 0)


def test_matches_independent_python_loops_with_duplicates(oracle_mod):
    """Tiny shapes against pure-Python fp64 loops, including repeated list entries."""
    w = gen.random_problem(15, B=1, H=2, D=16, T=8, vbs=[8, 3, 0, 5, 1], density=0.6,
                           duplicates=True, pad="random")
    w.q2k_num[0, 0, 0] = 3
    w.q2k_idx[0, 0, 0, :3] = [1, 1, 3]  # tile 1 twice: its keys count twice
    out = run_oracle(oracle_mod, w)
    ref = python_bruteforce(w)
    np.testing.assert_allclose(out, ref, atol=2e-6, rtol=1e-5)


def test_duplicate_entry_doubles_that_tiles_weight(oracle_mod):
    """[A, A, B] weighs A's keys twice: equals a list where A's values are repeated."""
    w = gen.random_problem(16, B=1, H=1, D=16, T=8, vbs=[8, 6, 8], counts=0, MS=3)
    w.q2k_num[0, 0, 0] = 3
    w.q2k_idx[0, 0, 0] = [1, 1, 2]
    out = run_oracle(oracle_mod, w)[0, 0, :8]
    qf, kf, vf = (F32(x)[0, 0].astype(np.float64) for x in (w.q, w.k, w.v))
    keys = list(range(8, 14)) * 2 + list(range(16, 24))
    s = qf[:8] @ kf[keys].T * scale_of(16)
    p = np.exp(s - s.max(-1, keepdims=True))
    ref = (p / p.sum(-1, keepdims=True)) @ vf[keys]
    np.testing.assert_allclose(out, ref, atol=2e-6, rtol=1e-5)


def test_rows_without_keys_are_positive_zero(oracle_mod):
    """Empty lists, and lists whose tiles are all empty, give +0 rows."""
    w = gen.random_problem(17, B=1, H=2, D=16, T=8, vbs=[8, 0, 5, 0], counts=2, MS=2)
    w.q2k_idx[0, 0, 0, :2] = [1, 3]  # both listed tiles are empty
    w.q2k_num[0, 1, 2] = 0  # empty list
    out = run_oracle(oracle_mod, w)
    assert np.all(out[0, 0, 0:8].view(np.uint32) == 0)
    assert np.all(out[0, 1, 16:24].view(np.uint32) == 0)
    assert np.isfinite(out[0, 1, 0:5]).all() and np.abs(out[0, 1, 0:5]).sum() > 0


def test_all_minus_inf_logits_give_a_nan_row(oracle_mod):
    """q = (-inf, 0, ...) against keys with k[0] > 0: every logit is -inf, the softmax
    sum is NaN and the whole row is NaN; other rows stay finite."""
    w = gen.random_problem(18, B=1, H=1, D=16, T=8, vbs=[8, 5, 8], counts=2, MS=2, pad="naninf")
    q = w.q.copy()
    q[0, 0, 3] = 0
    q[0, 0, 3, 0] = gen.BF16_NEG_INF
    k = w.k.copy()
    valid = gen.contiguous_map(w.vbs, 8) >= 0
    kcol = F32(k[0, 0, valid, 0])
    k[0, 0, valid, 0] = gen.to_bf16_bits(np.abs(kcol) + 1)
    out = oracle_mod.fwd(q, k, w.v, w.q2k_idx, w.q2k_num, w.vbs, 8)
    assert np.isnan(out[0, 0, 3]).all()
    others = np.ones(24, bool)
    others[3] = False
    others[13:16] = False  # padding rows of tile 1 (+0, checked below)
    assert np.isfinite(out[0, 0, others]).all()
    assert np.all(out[0, 0, 13:16].view(np.uint32) == 0)


def test_plus_inf_logit_gives_a_nan_row(oracle_mod):
    """A +inf logit makes exp(s - m) = exp(inf - inf) NaN: NaN row."""
    w = gen.random_problem(19, B=1, H=1, D=16, T=8, vbs=[8, 8], counts=2, MS=2)
    q = w.q.copy()
    k = w.k.copy()
    q[0, 0, 2, 0] = gen.to_bf16_bits(np.float32([1.0]))[0]
    k[0, 0, 9, 0] = gen.BF16_POS_INF
    out = oracle_mod.fwd(q, k, w.v, w.q2k_idx, w.q2k_num, w.vbs, 8)
    assert np.isnan(out[0, 0, 2]).all()


def test_tile_of_minus_inf_logits_with_a_finite_max_is_finite(oracle_mod):
    """Keys with -inf logits get weight 0 when the row max is finite: listing such a
    tile first changes nothing, bit for bit."""
    w = gen.random_problem(20, B=1, H=1, D=16, T=8, vbs=[8, 8, 8], counts=0, MS=2)
    q = w.q.copy()
    k = w.k.copy()
    q[0, 0, 0:8, 0] = gen.to_bf16_bits(np.full(8, -1.0, np.float32))
    k[0, 0, 8:16, 0] = gen.BF16_POS_INF  # tile 1: every logit is -inf
    w.q2k_num[0, 0, 0] = 2
    w.q2k_idx[0, 0, 0] = [1, 2]
    both = oracle_mod.fwd(q, k, w.v, w.q2k_idx, w.q2k_num, w.vbs, 8)[0, 0, :8]
    w.q2k_num[0, 0, 0] = 1
    w.q2k_idx[0, 0, 0] = [2, 0]
    alone = oracle_mod.fwd(q, k, w.v, w.q2k_idx, w.q2k_num, w.vbs, 8)[0, 0, :8]
    assert np.isfinite(both).all()
    np.testing.assert_array_equal(both.view(np.uint32), alone.view(np.uint32))


@pytest.mark.parametrize("pattern", ["random", "nan", "inf", "naninf"])
def test_padding_contents_never_reach_the_output(oracle_mod, pattern):
    w = gen.random_problem(21, B=1, H=2, D=16, T=8, vbs=[8, 3, 0, 7, 1], density=0.7)
    base = run_oracle(oracle_mod, w)
    for x in (w.q, w.k, w.v):
        gen.fill_padding(x, w.vbs, 8, pattern)
    poisoned = run_oracle(oracle_mod, w)
    np.testing.assert_array_equal(base.view(np.uint32), poisoned.view(np.uint32))


def test_single_valid_key_returns_its_value_exactly(oracle_mod):
    w = gen.random_problem(22, B=1, H=2, D=16, T=8, vbs=[8, 1, 8], counts=1, MS=1)
    w.q2k_idx[...] = 1
    out = run_oracle(oracle_mod, w)
    vrow = F32(w.v[:, :, 8])  # the single valid key row of tile 1
    for i in range(3):
        for r in range(int(w.vbs[i])):
            np.testing.assert_array_equal(out[:, :, i * 8 + r], vrow)


def test_zero_query_averages_the_selected_values(oracle_mod):
    w = gen.random_problem(23, B=1, H=2, D=16, T=8, vbs=[8, 6, 3, 8], density=0.6)
    w.q[...] = 0
    out = run_oracle(oracle_mod, w)
    vf = F32(w.v).astype(np.float64)
    mask = key_mask(w)
    for b, h, row in zip(*np.nonzero(mask.any(-1))):
        ref = vf[b, h, mask[b, h, row]].mean(0)
        np.testing.assert_allclose(out[b, h, row], ref, atol=1e-6, rtol=1e-5)


def test_constant_values_give_that_constant(oracle_mod):
    w = gen.random_problem(24, B=1, H=1, D=16, T=8, vbs=[8, 5, 8], density=0.7)
    c = gen.to_bf16_bits(np.linspace(-3, 3, 16, dtype=np.float32))
    w.v[...] = c
    out = run_oracle(oracle_mod, w)
    has = key_mask(w).any(-1)
    np.testing.assert_allclose(out[has], np.broadcast_to(F32(c), out[has].shape), rtol=2e-6)


def test_two_keys_logistic_closed_form(oracle_mod):
    """q = (x, 0...), keys (1, 0...) and 0: weights are a logistic in scale*x."""
    D, T = 16, 8
    w = gen.random_problem(25, B=1, H=1, D=D, T=T, vbs=[1, 2], counts=0, MS=1)
    x = 3.0
    w.q[...] = 0
    w.q[0, 0, 0, 0] = gen.to_bf16_bits(np.float32([x]))[0]
    w.k[...] = 0
    w.k[0, 0, 8, 0] = gen.to_bf16_bits(np.float32([1.0]))[0]
    w.q2k_num[0, 0, 0] = 1
    w.q2k_idx[0, 0, 0, 0] = 1
    out = run_oracle(oracle_mod, w)[0, 0, 0]
    s = scale_of(D) * x
    w1 = 1.0 / (1.0 + math.exp(-s))
    v = F32(w.v[0, 0, 8:10]).astype(np.float64)
    np.testing.assert_allclose(out, w1 * v[0] + (1 - w1) * v[1], atol=1e-6, rtol=1e-6)


def test_list_order_does_not_change_the_result(oracle_mod):
    w = gen.random_problem(26, B=1, H=2, D=64, T=64, vbs=[64, 30, 64, 64, 12], density=0.8)
    base = run_oracle(oracle_mod, w)
    rng = np.random.default_rng(0)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(w.NT):
                n = int(w.q2k_num[b, h, i])
                w.q2k_idx[b, h, i, :n] = rng.permutation(w.q2k_idx[b, h, i, :n])
    np.testing.assert_allclose(run_oracle(oracle_mod, w), base, atol=1e-6, rtol=1e-5)


def test_two_selections_combine_through_their_log_sum_exp(oracle_mod):
    """out({A,B}) = sigma*out({A}) + (1-sigma)*out({B}), sigma from the fp64
    log-sum-exps of the two key sets."""
    D, T = 32, 8
    w = gen.random_problem(27, B=1, H=1, D=D, T=T, vbs=[8, 7, 8], counts=0, MS=2)

    def run(lst):
        w.q2k_num[0, 0, 0] = len(lst)
        w.q2k_idx[0, 0, 0, :len(lst)] = lst
        return run_oracle(oracle_mod, w)[0, 0, :8].astype(np.float64)

    ab, a, b = run([1, 2]), run([1]), run([2])
    qf, kf = F32(w.q[0, 0, :8]).astype(np.float64), F32(w.k[0, 0]).astype(np.float64)

    def lse(rows):
        s = qf @ kf[rows].T * scale_of(D)
        mx = s.max(-1, keepdims=True)
        return (mx + np.log(np.exp(s - mx).sum(-1, keepdims=True)))

    la, lb = lse(list(range(8, 15))), lse(list(range(16, 24)))
    sig = 1.0 / (1.0 + np.exp(lb - la))
    np.testing.assert_allclose(ab, sig * a + (1 - sig) * b, atol=2e-6, rtol=1e-5)


def test_large_logits_do_not_overflow(oracle_mod):
    """Logits in the thousands: the max subtraction keeps the result finite and exact."""
    w = gen.random_problem(28, B=1, H=1, D=64, T=64, vbs=[64, 50, 64], counts=3, sigma=12.0)
    out = run_oracle(oracle_mod, w)
    assert np.isfinite(out).all()
    mask = key_mask(w)
    ref = sdpa_fp64(w, mask)
    has = mask.any(-1)
    qf, kf, vf = (F32(x)[0, 0].astype(np.float64) for x in (w.q, w.k, w.v))
    s = qf @ kf.T * scale_of(64)
    assert np.abs(s[mask[0, 0]]).max() > 88.8, "some exp(s) must overflow binary32 unshifted"
    # binary32 rounding of a D-term dot product: |err(s)| <= D * 2^-24 * scale * sum|q_d k_d|;
    # the softmax weights then move by at most ~2*|err(s)| relative, the output by that times max|v|
    err_s = 64 * 2.0 ** -24 * scale_of(64) * (np.abs(qf) @ np.abs(kf).T)
    bound = 2 * np.where(mask[0, 0], err_s, 0).max(-1) * np.abs(vf).max() + 1e-5
    diff = np.abs(out[0, 0] - ref[0, 0]).max(-1)
    assert np.all(diff[has[0, 0]] <= bound[has[0, 0]])


def test_rows_entry_point_agrees_with_full_run(oracle_mod):
    w = gen.random_problem(29, B=2, H=2, D=64, T=64, vbs=[64, 20, 64], density=0.6)
    full = run_oracle(oracle_mod, w)
    rows = np.array([0, 5, 70, 64 + 19, 64 + 20, w.B * w.H * w.S - 1], np.int64)
    got = oracle_mod.fwd_rows(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, rows)
    np.testing.assert_array_equal(got.view(np.uint32), full.reshape(-1, w.D)[rows].view(np.uint32))


def test_thread_count_does_not_change_bits(oracle_mod):
    w = gen.random_problem(30, B=1, H=3, D=64, T=64, vbs=[64, 33, 64, 64], density=0.7)
    a = run_oracle(oracle_mod, w, nthreads=1)
    b = run_oracle(oracle_mod, w, nthreads=7)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("what", ["index", "count", "length"])
def test_invalid_contents_are_rejected(oracle_mod, what):
    w = gen.random_problem(31, B=1, H=1, D=16, T=8, vbs=[8, 8], counts=1, MS=1)
    if what == "index":
        w.q2k_idx[0, 0, 1, 0] = 2
    elif what == "count":
        w.q2k_num[0, 0, 0] = 2
    else:
        w.vbs[1] = 9
    with pytest.raises(ValueError):
        run_oracle(oracle_mod, w)


def test_layout_gather_matches_python_loops(oracle_mod):
    """The layout oracle against an explicit loop, for a shuffled map with padding."""
    rng = np.random.default_rng(3)
    B, S_tok, H, D, T, NT = 2, 37, 3, 8, 8, 6
    x = rng.integers(0, 65536, size=(B, S_tok, H, D), dtype=np.uint16)
    src = np.full(NT * T, -1, np.int32)
    rows = rng.choice(NT * T, size=S_tok, replace=False)
    src[rows] = rng.permutation(S_tok)
    (out,) = oracle_mod.tile_layout([x], src, T)
    ref = np.zeros((B, H, NT * T, D), np.uint16)
    for b in range(B):
        for h in range(H):
            for t in range(NT * T):
                if src[t] >= 0:
                    ref[b, h, t] = x[b, src[t], h]
    np.testing.assert_array_equal(out, ref)
    # a permutation: gathering back by the inverse map recovers every token
    inv = np.empty(S_tok, np.int64)
    inv[src[src >= 0]] = np.nonzero(src >= 0)[0]
    np.testing.assert_array_equal(out[:, :, inv, :].transpose(0, 2, 1, 3), x)


def test_layout_contiguous_map_agrees_with_generator_placement(oracle_mod):
    w = gen.random_problem(32, B=1, H=2, D=16, T=8, vbs=[8, 3, 0, 6], density=0.5)
    outs = oracle_mod.tile_layout([w.tok["q"], w.tok["k"], w.tok["v"]], w.tile_src_token, 8)
    for got, want in zip(outs, (w.q, w.k, w.v)):
        np.testing.assert_array_equal(got, want)
