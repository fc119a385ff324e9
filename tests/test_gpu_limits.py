"""GPU parity at the largest sizes the launch limits admit, through the C ABI.

* The largest batch x heads (65535, also the largest grid height of the layout
  kernel): layout of four tensors, forward with log-sum-exp, transposed lists,
  backward and the inverse gather, checked on sampled heads against the oracle.
* Tensors past 4 GiB: 65 heads of 2048 tiles of 128 x 128, so the last head
  starts exactly 2^32 bytes (2^31 elements) into every tensor; layout,
  forward and backward checked on the first and the last head.

Inputs are seeded: torch's generator on the device for the bulk, NumPy for the
lists.  The oracle sees the sampled heads' own inputs, copied back.
"""
import numpy as np
import pytest

import block_sparse_tiled_amd as bsa
from parity import bits_from_dev, compare, compare_grad, grad_zero_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bsa.load()


def randn_bf16(shape, seed, scale=1.0):
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    return x.mul_(scale).to(torch.bfloat16)


def host_bits(t):
    return bits_from_dev(t.contiguous())


def contiguous_map(vbs, T):
    """tile row -> source token for tiles holding consecutive tokens (-1 = padding)."""
    src = np.full(vbs.size * T, -1, np.int32)
    start = 0
    for i, n in enumerate(vbs):
        src[i * T:i * T + n] = np.arange(start, start + n)
        start += n
    return src


def check_head(oracle_mod, dev, b, h, T, idx, num, vbs, label, grads=True):
    """Forward, log-sum-exp and (optionally) gradients of head (b, h) against the oracle."""
    import oracle

    q, k, v, dout = (host_bits(dev[x][b:b + 1, h:h + 1]) for x in ("q", "k", "v", "dout"))
    i1, n1 = idx[b:b + 1, h:h + 1], num[b:b + 1, h:h + 1]
    ref = oracle_mod.fwd(q, k, v, i1, n1, vbs, T)
    compare(host_bits(dev["out"][b:b + 1, h:h + 1]), ref, label=f"{label} out")
    out64, lse64 = oracle.fwd64(q, k, v, i1, n1, vbs, T)
    lse = dev["lse"][b:b + 1, h:h + 1].cpu().numpy()
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse64)), f"{label}: lse -inf mask"
    fin = np.isfinite(lse64)
    np.testing.assert_allclose(lse[fin], lse64[fin], rtol=1e-5, atol=1e-4)
    if grads:
        dq, dk, dv = oracle.bwd(q, k, v, dout, i1, n1, vbs, T)
        dq_zero, dkv_zero = grad_zero_rows(i1, n1, vbs, T)
        compare_grad(host_bits(dev["dq"][b:b + 1, h:h + 1]), dq, f"{label} dq", dq_zero)
        compare_grad(host_bits(dev["dk"][b:b + 1, h:h + 1]), dk, f"{label} dk", dkv_zero)
        compare_grad(host_bits(dev["dv"][b:b + 1, h:h + 1]), dv, f"{label} dv", dkv_zero)


def run_path(tok, src_map, T, idx, num, vbs, dout_seed):
    """Layout of the token-major tensors, forward with lse, lists, backward."""
    import torch

    q, k, v, *rest = bsa.tile_layout(tok, to_dev(src_map), T)
    d_idx, d_num, d_vbs = to_dev(idx), to_dev(num), to_dev(vbs)
    out, lse, out_lo = bsa.fwd_lse(q, k, v, d_idx, d_num, d_vbs, T)
    k2q_idx, k2q_num = bsa.bwd_k2q(d_idx, d_num)
    dout = randn_bf16(tuple(q.shape), dout_seed)
    dq, dk, dv = bsa.bwd(q, k, v, out, out_lo, dout, lse, d_idx, d_num, k2q_idx, k2q_num, d_vbs, T)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, out=out, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, rest=rest)


def test_largest_batch_heads(oracle_mod):
    import torch

    B, H, T, D = 3, 21845, 64, 64  # B * H = 65535
    vbs = np.array([T, T - 7], np.int32)
    NT, S_tok = vbs.size, int(vbs.sum())
    assert bsa.within_launch_limits(B, H, B * H * NT * T, NT)
    assert not bsa.within_launch_limits(B, H + 1, B * (H + 1) * NT * T, NT)
    print(f"largest batch*heads: B={B} H={H} NT={NT} T={T} D={D}", flush=True)
    tok = [randn_bf16((B, S_tok, H, D), 100 + x) for x in range(4)]
    src = contiguous_map(vbs, T)
    rng = np.random.default_rng(31)
    idx = np.stack([rng.permutation(NT) for _ in range(B * H * NT)]).reshape(B, H, NT, NT)
    idx = idx.astype(np.int32)
    num = rng.integers(0, NT + 1, size=(B, H, NT)).astype(np.int32)
    dev = run_path(tok, src, T, idx, num, vbs, 200)
    (back,) = bsa.tile_unlayout([dev["out"]], to_dev(_token_rows(src, S_tok)), T)
    torch.cuda.synchronize()
    for bh in (0, 1, H - 1, H, 2 * H + 5, B * H - 1):
        b, h = divmod(bh, H)
        label = f"b{b} h{h}"
        # layout of all four tensors, bit for bit
        host_tok = [host_bits(t[b:b + 1, :, h:h + 1]) for t in tok]
        want = oracle_mod.tile_layout(host_tok, src, T)
        got = [dev["q"], dev["k"], dev["v"], dev["rest"][0]]
        for x, (g, e) in enumerate(zip(got, want)):
            np.testing.assert_array_equal(host_bits(g[b:b + 1, h:h + 1]), e, err_msg=f"{label} t{x}")
        check_head(oracle_mod, dev, b, h, T, idx, num, vbs, label)
        # the inverse gather returns the output rows to their tokens
        (want_back,) = oracle_mod.tile_unlayout([host_bits(dev["out"][b:b + 1, h:h + 1])],
                                                _token_rows(src, S_tok))
        np.testing.assert_array_equal(host_bits(back[b:b + 1, :, h:h + 1]), want_back)
    # the transposed lists of one head, exactly
    k2q_idx, k2q_num = bsa.bwd_k2q(to_dev(idx), to_dev(num))
    kn = k2q_num.cpu().numpy()
    ki = k2q_idx.cpu().numpy()
    b, h = 2, H - 1
    for j in range(NT):
        lst = [i for i in range(NT) for t in idx[b, h, i, :num[b, h, i]] if t == j]
        assert kn[b, h, j] == len(lst) and ki[b, h, j, :len(lst)].tolist() == lst


def _token_rows(src, S_tok):
    """token -> tile row, the inverse of a gather map."""
    row = np.full(S_tok, -1, np.int32)
    ok = src >= 0
    row[src[ok]] = np.nonzero(ok)[0]
    return row


def test_offsets_past_4_gib(oracle_mod):
    """65 heads of 2048 tiles of 128 x 128: head 64 starts 2^32 bytes into every
    tensor; its lists always hold the last tile."""
    B, H, T, D, NT, MS = 1, 65, 128, 128, 2048, 4
    vbs = np.full(NT, T, np.int32)
    vbs[5], vbs[-1] = 33, 77
    S_tok = int(vbs.sum())
    assert bsa.within_launch_limits(B, H, B * H * NT * T, NT)
    assert H * NT * T * D * 2 > 1 << 32
    print(f"past 4 GiB: H={H} NT={NT} T={T} D={D}", flush=True)
    tok = [randn_bf16((B, S_tok, H, D), 300 + x) for x in range(3)]
    src = contiguous_map(vbs, T)
    rng = np.random.default_rng(47)
    idx = np.empty((B, H, NT, MS), np.int32)
    for h in range(H):
        for i in range(NT):
            other = rng.choice(NT - 1, MS - 1, replace=False)
            idx[0, h, i] = np.concatenate([[NT - 1], other])
    num = rng.integers(1, MS + 1, size=(B, H, NT)).astype(np.int32)
    dev = run_path(tok, src, T, idx, num, vbs, 400)
    for h in (0, H - 1):
        label = f"h{h}"
        host_tok = [host_bits(t[:, :, h:h + 1]) for t in tok]
        want = oracle_mod.tile_layout(host_tok, src, T)
        for x, (g, e) in enumerate(zip((dev["q"], dev["k"], dev["v"]), want)):
            np.testing.assert_array_equal(host_bits(g[:, h:h + 1]), e, err_msg=f"{label} t{x}")
        check_head(oracle_mod, dev, 0, h, T, idx, num, vbs, label, grads=h == H - 1)
