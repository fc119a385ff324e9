"""The rule by which the kernels let two key (or query) tiles share a step.

With a list chunk's parts sorted by length, the kernels take the largest k for which the
2k shortest, paired first with 2k-th, second with (2k-1)-th and so on, all fit in T rows,
and use those k pairs.  That is the most disjoint pairs of total length <= T that any
pairing of the chunk has: checked here against an exhaustive maximum matching on small
random multisets, with the same ordering and binary search the kernels use.  CPU only.
"""
import functools

import numpy as np
import pytest


def nested_fits(s, k, T):
    return all(s[i] + s[2 * k - 1 - i] <= T for i in range(k))


def kernel_pair_count(lengths, T):
    """The count the kernels reach: a binary search over k in [1, n/2] of the nested
    test, started only when the two shortest parts fit together."""
    s = sorted(lengths)
    if len(s) < 2 or s[0] + s[1] > T:
        return 0
    lo, hi = 1, len(s) // 2
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if nested_fits(s, mid, T):
            lo = mid
        else:
            hi = mid - 1
    return lo


def max_matching(lengths, T):
    """The most disjoint pairs with length sum <= T, by exhaustive search over subsets."""
    n = len(lengths)

    @functools.lru_cache(maxsize=None)
    def best(mask):
        i = next((b for b in range(n) if not mask >> b & 1), None)
        if i is None:
            return 0
        res = best(mask | 1 << i)  # part i alone
        for j in range(i + 1, n):
            if not mask >> j & 1 and lengths[i] + lengths[j] <= T:
                res = max(res, 1 + best(mask | 1 << i | 1 << j))
        return res

    return best(0)


@pytest.mark.parametrize("T", [64, 128])
def test_nested_pairing_is_a_maximum_matching(T):
    rng = np.random.default_rng(11 + T)
    for _ in range(400):
        n = int(rng.integers(0, 13))
        kind = rng.integers(0, 3)
        if kind == 0:
            lengths = rng.integers(1, T + 1, size=n)
        elif kind == 1:  # mostly short parts
            lengths = rng.integers(1, T // 2 + 8, size=n)
        else:  # lengths near T/2, where ties and exact fits are common
            lengths = rng.integers(T // 2 - 3, T // 2 + 4, size=n)
        lengths = tuple(int(x) for x in lengths)
        assert kernel_pair_count(lengths, T) == max_matching(lengths, T), lengths


def test_the_nested_test_is_monotone_in_k():
    """The binary search needs: if the 2k shortest nest, so do the 2(k-1) shortest."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        s = sorted(int(x) for x in rng.integers(1, 129, size=int(rng.integers(2, 40))))
        ok = [nested_fits(s, k, 128) for k in range(1, len(s) // 2 + 1)]
        assert ok == sorted(ok, reverse=True), s


def test_steps_cover_every_part_once():
    """Pairs (rank i, rank 2k-1-i) for i < k, then ranks 2k.. one per step: every part
    lands in exactly one step, and every pair fits."""
    rng = np.random.default_rng(9)
    for _ in range(200):
        T = 128
        lengths = [int(x) for x in rng.integers(1, T + 1, size=int(rng.integers(1, 60)))]
        order = sorted(range(len(lengths)), key=lambda p: (lengths[p], p))  # ties in list order
        k = kernel_pair_count(lengths, T)
        steps = [(order[i], order[2 * k - 1 - i]) for i in range(k)] + [(order[r],) for r in range(2 * k, len(order))]
        assert sorted(p for st in steps for p in st) == list(range(len(lengths)))
        assert all(sum(lengths[p] for p in st) <= T for st in steps)
        assert len(steps) == len(lengths) - k
