"""bsa_fwd_noalloc (the forward for callers that cannot allocate) against bsa_fwd.

Through the C ABI: two calls in a row, the second on a smaller problem, both of which
cut their lists (so both use the fixed scratch array, the second over the first's
leftovers).  Each output meets the forward's bar against bsa_fwd's output and is in fact
the same bits (the same plan and kernels), and the calls allocate no device memory.
"""
import numpy as np
import pytest

import block_sparse_tiled_amd as bsa
from block_sparse_tiled_amd import inputs as gen
from parity import bits_from_dev, compare, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bsa.load()


def test_noalloc_matches_fwd_on_two_calls_in_a_row():
    import torch

    big = gen.ragged()
    # the small one also has two short tiles, so that its lists pair tiles into steps
    small = gen.random_problem(67, B=1, H=2, D=128, T=128, vbs=[128] * 18 + [90, 40, 20], density=0.8,
                               pad="naninf")
    cases = []
    for w in (big, small):
        assert bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS) > 0, "meant to split its lists"
        args = [to_dev(x) for x in (w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs)]
        out = torch.empty_like(args[0])
        cases.append((w, args, out))
    assert (bsa.workspace_size(small.B, small.H, small.NT, small.T, small.D, small.MS)
            < bsa.workspace_size(big.B, big.H, big.NT, big.T, big.D, big.MS))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for w, args, out in cases:  # back to back, no sync between
        print(f"noalloc B={w.B} H={w.H} NT={w.NT}", flush=True)
        bsa.fwd_noalloc(*args, w.T, out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "bsa_fwd_noalloc allocated device memory"
    for w, args, out in cases:
        got = bits_from_dev(out)
        ref = bits_from_dev(bsa.fwd(*args, w.T))
        compare(got, gen.bf16_bits_to_f32(ref), label=f"noalloc vs fwd NT={w.NT}")
        np.testing.assert_array_equal(got, ref)
