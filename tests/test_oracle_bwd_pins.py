"""Pins of the fp64 forward-with-LSE and backward oracle (oracle.bsa_bwd).

Each test checks the oracle against something other than itself: the binary32
C oracle, PyTorch's scaled_dot_product_attention and its autograd in fp64 (a
library routine), central finite differences, and closed forms.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from block_sparse_tiled_amd import inputs as gen


def f64(x):
    return oracle.bsa_bwd._widen(x)


def rand_dout(rng, shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("seed,T,D,vbs,dup", [(1, 64, 64, [64, 40, 64, 17], False),
                                              (2, 128, 128, [128, 100, 0, 128], False),
                                              (3, 64, 128, [64, 64, 33], True)])
def test_forward_matches_the_binary32_oracle(seed, T, D, vbs, dup):
    w = gen.random_problem(seed, B=1, H=2, D=D, T=T, vbs=vbs, density=0.6, duplicates=dup)
    o32 = oracle.fwd(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T)
    o64, lse = oracle.fwd64(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T)
    assert np.abs(o32 - o64).max() < 2e-5
    # lse is -inf exactly on the rows the forward leaves at +0
    zero = np.all(o32 == 0, axis=-1)
    assert np.array_equal(np.isneginf(lse), zero)


def _sdpa_grads(q, k, v, dout, mask=None):
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=None if mask is None else
                                         torch.tensor(mask))
    out.backward(torch.tensor(dout, dtype=torch.float64))
    return out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def test_dense_equals_sdpa_autograd():
    """Every tile listed, all full: textbook attention; PyTorch autograd gives the gradients."""
    rng = np.random.default_rng(7)
    B, H, T, NT, D = 1, 2, 64, 3, 64
    w = gen.random_problem(7, B=B, H=H, D=D, T=T, vbs=[T] * NT, counts=NT, MS=NT)
    w.q2k_idx[...] = np.arange(NT)
    dout = rand_dout(rng, w.q.shape)
    out, lse = oracle.fwd64(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, T)
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q2k_idx, w.q2k_num, w.vbs, T)
    ro, rdq, rdk, rdv = _sdpa_grads(f64(w.q), f64(w.k), f64(w.v), dout)
    for a, b in ((out, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - b).max() < 1e-10
    s = f64(w.q) @ np.swapaxes(f64(w.k), -1, -2) / np.sqrt(D)
    m = s.max(-1)
    np.testing.assert_allclose(lse, m + np.log(np.exp(s - m[..., None]).sum(-1)), rtol=0, atol=1e-12)


def test_ragged_all_listed_equals_sdpa_on_valid_tokens():
    """Every tile listed with ragged lengths: SDPA on the compacted valid tokens;
    padding rows get no gradient."""
    rng = np.random.default_rng(8)
    T, vbs, D = 64, [64, 23, 50], 64
    NT = len(vbs)
    w = gen.random_problem(8, B=1, H=1, D=D, T=T, vbs=vbs, counts=NT, MS=NT, pad="nan")
    w.q2k_idx[...] = np.arange(NT)
    dout = rand_dout(rng, w.q.shape)
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q2k_idx, w.q2k_num, w.vbs, T)
    valid = np.concatenate([i * T + np.arange(n) for i, n in enumerate(vbs)])
    pad = np.setdiff1d(np.arange(NT * T), valid)
    _, rdq, rdk, rdv = _sdpa_grads(f64(w.q)[:, :, valid], f64(w.k)[:, :, valid],
                                   f64(w.v)[:, :, valid], dout[:, :, valid])
    for a, b in ((dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a[:, :, valid] - b).max() < 1e-10
        assert not a[:, :, pad].any()


def test_block_mask_equals_masked_sdpa_autograd():
    """A general block mask: SDPA with a token-level boolean mask (True = attend) on the
    query rows that have keys; rows without keys get no gradient."""
    rng = np.random.default_rng(9)
    T, vbs, D = 64, [64, 64, 31, 64, 50], 64
    NT = len(vbs)
    w = gen.random_problem(9, B=1, H=2, D=D, T=T, vbs=vbs, density=0.45)
    dout = rand_dout(rng, w.q.shape)
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q2k_idx, w.q2k_num, w.vbs, T)
    valid_tok = np.zeros(NT * T, bool)
    for i, n in enumerate(vbs):
        valid_tok[i * T:i * T + n] = True
    for h in range(2):
        mask = np.zeros((NT * T, NT * T), bool)
        for i in range(NT):
            for j in w.q2k_idx[0, h, i, :w.q2k_num[0, h, i]]:
                mask[i * T:(i + 1) * T, j * T:j * T + vbs[j]] = True
        rows = np.flatnonzero(valid_tok & mask.any(axis=1))
        _, rdq, rdk, rdv = _sdpa_grads(f64(w.q)[0, h, rows], f64(w.k)[0, h], f64(w.v)[0, h],
                                       dout[0, h, rows], mask=mask[rows])
        assert np.abs(dq[0, h, rows] - rdq).max() < 1e-10
        assert np.abs(dk[0, h] - rdk).max() < 1e-10
        assert np.abs(dv[0, h] - rdv).max() < 1e-10
        others = np.setdiff1d(np.arange(NT * T), rows)
        assert not dq[0, h, others].any()


def test_finite_differences_with_duplicates_and_ragged_tiles():
    """d/dx of sum(dO * out) by central differences on the fp64 forward, at sampled
    elements of q, k and v; lists hold a duplicated tile."""
    rng = np.random.default_rng(10)
    T, vbs, D = 64, [64, 37, 64], 64
    w = gen.random_problem(10, B=1, H=1, D=D, T=T, vbs=vbs, counts=3, MS=3)
    w.q2k_idx[0, 0, 0] = [1, 2, 1]  # tile 1 listed twice
    x = {n: f64(getattr(w, n)) for n in ("q", "k", "v")}
    dout = rand_dout(rng, x["q"].shape)
    grads = dict(zip(("q", "k", "v"), oracle.bwd(x["q"], x["k"], x["v"], dout, w.q2k_idx,
                                                  w.q2k_num, w.vbs, T)))
    eps = 1e-6

    def loss(xs):
        out, _ = oracle.fwd64(xs["q"], xs["k"], xs["v"], w.q2k_idx, w.q2k_num, w.vbs, T)
        return float((out * dout).sum())

    for name in ("q", "k", "v"):
        for _ in range(12):
            r = int(rng.integers(0, 3 * T))
            d = int(rng.integers(0, D))
            if r % T >= vbs[r // T]:
                continue
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][0, 0, r, d] += eps
            xm[name][0, 0, r, d] -= eps
            fd = (loss(xp) - loss(xm)) / (2 * eps)
            assert abs(fd - grads[name][0, 0, r, d]) < 1e-6 * max(1.0, abs(fd))


def test_closed_forms():
    """A single valid key: P = 1, so dq = dk = 0 and dv = dO.  Rows without keys,
    padding query rows and padding key rows get exactly zero gradient."""
    rng = np.random.default_rng(11)
    T, D = 64, 64
    w = gen.random_problem(11, B=1, H=1, D=D, T=T, vbs=[64, 1, 20], counts=1, MS=1, pad="nan")
    w.q2k_idx[0, 0, :, 0] = 1  # every query tile lists tile 1, whose only key is row T
    w.q2k_num[0, 0, 2] = 0     # tile 2 lists nothing
    dout = rand_dout(rng, w.q.shape)
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q2k_idx, w.q2k_num, w.vbs, T)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    rows = np.r_[0:64, T:T + 1]
    np.testing.assert_allclose(dv[0, 0, T], dout[0, 0, rows].sum(0), rtol=1e-13, atol=1e-13)
    mask = np.ones(3 * T, bool)
    mask[T] = False
    assert not dv[0, 0, mask].any()
    _, lse = oracle.fwd64(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, T)
    assert np.all(np.isneginf(lse[0, 0, 2 * T:]))  # no keys
    assert np.all(np.isneginf(lse[0, 0, T + 1:2 * T]))  # padding query rows


def test_all_minus_inf_row_has_nan_gradients():
    """The constructed all-(-inf) row is NaN (hardening commit's l != 0 rule); its
    gradient is NaN too, and the other rows stay finite."""
    rng = np.random.default_rng(12)
    T, D = 64, 64
    w = gen.random_problem(12, B=1, H=1, D=D, T=T, vbs=[64, 64], counts=2, MS=2)
    q, k = f64(w.q), f64(w.k)
    q[0, 0, 5] = 0.0
    q[0, 0, 5, 0] = -np.inf
    k[0, 0, :, 0] = np.abs(k[0, 0, :, 0]) + 1
    dout = rand_dout(rng, q.shape)
    out, lse = oracle.fwd64(q, k, w.v, w.q2k_idx, w.q2k_num, w.vbs, T)
    dq, dk, dv = oracle.bwd(q, k, w.v, dout, w.q2k_idx, w.q2k_num, w.vbs, T)
    assert np.all(np.isnan(out[0, 0, 5])) and np.all(np.isnan(dq[0, 0, 5]))
    assert np.isneginf(lse[0, 0, 5])  # log of a sum of zeros
    others = np.setdiff1d(np.arange(2 * T), [5])
    assert np.isfinite(out[0, 0, others]).all() and np.isfinite(dq[0, 0, others]).all()


def test_structural_zero_rows_of_the_gradients():
    """The rows the GPU tests require to be +0 bit for bit (padding rows, rows with
    no key, key tiles nobody lists) are exactly 0 in the oracle; a query row whose
    only key is a one-row tile has dq = 0 by cancellation (P = 1, dS = dP - D = 0)
    although it is not such a row."""
    import sys, os

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from parity import grad_zero_rows

    rng = np.random.default_rng(13)
    for seed, T, vbs in ((21, 64, [64, 1, 0, 37, 64]), (22, 128, [128, 5, 128, 1]), (23, 64, [0, 64, 1])):
        w = gen.random_problem(seed, B=2, H=2, D=64, T=T, vbs=vbs, density=0.4)
        dout = rand_dout(rng, w.q.shape)
        dq, dk, dv = oracle.bwd(w.q, w.k, w.v, dout, w.q2k_idx, w.q2k_num, w.vbs, T)
        zq, zkv = grad_zero_rows(w.q2k_idx, w.q2k_num, w.vbs, T)
        assert zq.any() and (~zq).any() and zkv.any() and (~zkv).any()
        assert not dq[zq].any() and not dk[zkv].any() and not dv[zkv].any()
        assert np.all(np.abs(dv[~zkv]).sum(-1) > 0)  # every other key row gets dO weight
    # the cancellation case: query tile 0 lists only the one-row tile 1
    w = gen.random_problem(24, B=1, H=1, D=64, T=64, vbs=[64, 1], counts=1, MS=1)
    w.q2k_idx[0, 0, 0, 0] = 1
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, rand_dout(rng, w.q.shape), w.q2k_idx, w.q2k_num, w.vbs, 64)
    zq, _ = grad_zero_rows(w.q2k_idx, w.q2k_num, w.vbs, 64)
    assert not zq[0, 0, :64].any()
    assert np.abs(dq[0, 0, :64]).max() < 1e-12
