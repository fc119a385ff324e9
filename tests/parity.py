"""Shared helpers for the GPU parity tests: device transfer and the compare rule.

Compare rule (GPU bf16 output widened to fp32 vs the fp32 oracle):
  * NaN positions identical;
  * rows the oracle leaves at +0 (padding rows, rows without keys) are +0 bit
    for bit on the GPU;
  * over all other finite elements: max |diff| <= 2e-2 and mean |diff| <= 2e-3;
  * no Inf on the GPU where the oracle has none.
"""
import numpy as np

from block_sparse_tiled_amd import inputs as gen

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# gradients: the same bar on the gradients' own scale, max(1, RMS of the oracle's values)
MAX_REL = 2e-2
MEAN_REL = 2e-3


def to_dev(a, device="cuda"):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def bits_from_dev(t):
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def run_fwd(w, out=None, idx=None, num=None, vbs=None, q=None, k=None, v=None):
    import block_sparse_tiled_amd as bsa

    args = [to_dev(x) for x in (w.q if q is None else q, w.k if k is None else k,
                                w.v if v is None else v,
                                w.q2k_idx if idx is None else idx,
                                w.q2k_num if num is None else num,
                                w.vbs if vbs is None else vbs)]
    res = bsa.fwd(*args, w.T, out=out)
    return bits_from_dev(res)


def compare(gpu_bits, ref, zero_rows=None, label=""):
    """Apply the compare rule; ``gpu_bits`` uint16 [..., D], ``ref`` float32 [..., D].

    ``zero_rows`` (bool [...]) marks rows that must be +0 bit for bit; by default
    those are the rows the oracle returns as all-+0.
    """
    got = gen.bf16_bits_to_f32(gpu_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if zero_rows is None:
        zero_rows = np.all(ref.view(np.uint32) == 0, axis=-1)
    zero_bits = gpu_bits[zero_rows]
    assert np.all(zero_bits == 0), f"{label}: {int((zero_bits != 0).sum())} non-(+0) values in zero rows"
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got), (
        f"{label}: NaN mask differs ({int(nan_ref.sum())} in oracle, {int(nan_got.sum())} on GPU)")
    inf_got = np.isinf(got) & ~np.isinf(ref)
    assert not inf_got.any(), f"{label}: {int(inf_got.sum())} Inf values the oracle does not have"
    fin = np.isfinite(ref) & np.isfinite(got)
    fin &= ~zero_rows[..., None]
    if fin.any():
        diff = np.abs(got[fin].astype(np.float64) - ref[fin])
        mx, mean = float(diff.max()), float(diff.mean())
        assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{label}: max {mx:.3e} mean {mean:.3e}"
        return mx, mean
    return 0.0, 0.0


def sample_rows(w, n, rng, extra=()):
    """Flat row ids (b*H + h)*S + t: random valid rows plus edges and ``extra``."""
    S = w.S
    total = w.B * w.H * S
    rows = set(int(x) for x in rng.integers(0, total, size=n))
    last = (w.NT - 1) * w.T
    for bh in (0, w.B * w.H - 1):
        rows.update([bh * S, bh * S + 1, bh * S + last, bh * S + last + int(w.vbs[-1]) - 1,
                     bh * S + S - 1])
    rows.update(int(x) for x in extra)
    return np.array(sorted(r for r in rows if 0 <= r < total), np.int64)


def grad_zero_rows(q2k_idx, q2k_num, vbs, T):
    """Rows every gradient must leave at +0 by construction: (dq [B, H, NT*T], dk/dv [B, H, NT*T]).

    dq: padding query rows and rows whose list holds no valid key.  dk, dv:
    padding key rows and key tiles that no query tile with a valid row lists.
    (A row can also be 0 in the oracle by cancellation, e.g. dq of a row with a
    single key, where dS = dP - D vanishes; the GPU's rounding leaves such a
    row near 0, and the tolerance judges it.)
    """
    B, H, NT = q2k_num.shape
    MS = q2k_idx.shape[3]
    vbs = np.asarray(vbs)
    pad = (np.arange(NT * T) % T) >= np.repeat(vbs, T)
    no_keys = np.zeros((B, H, NT), bool)
    listed = np.zeros((B, H, NT), bool)
    for b in range(B):
        for h in range(H):
            for i in range(NT):
                n = min(max(int(q2k_num[b, h, i]), 0), MS)
                tiles = [int(j) for j in q2k_idx[b, h, i, :n] if 0 <= j < NT]
                no_keys[b, h, i] = sum(int(vbs[j]) for j in tiles) == 0
                if vbs[i] > 0:
                    for j in tiles:
                        listed[b, h, j] |= vbs[j] > 0
    dq_zero = pad[None, None, :] | np.repeat(no_keys, T, axis=2)
    dkv_zero = pad[None, None, :] | np.repeat(~listed, T, axis=2)
    return dq_zero, dkv_zero


def compare_grad(got_bits, ref, label, zero_rows=None):
    """Gradients (bf16 on the GPU) against the fp64 oracle.

    NaN and Inf positions identical; the rows in ``zero_rows`` (structural
    zeros, see grad_zero_rows; by default the rows the oracle leaves at exactly
    0) are +0 bit for bit; with s = max(1, RMS of the oracle's finite values), every
    element within 2e-2 s + 2^-7 max(|ref|, RMS of its row), and the mean
    difference within 2e-3 s.  The second term is a bf16 ulp of the larger of
    the value and its row's scale: the result is bf16, and P and dS enter the
    products as bf16, so each row carries rounding noise of relative size
    2^-9 sqrt(n) over its n terms, as large as the row itself is (a row's
    values are sums of n terms of either sign).  It matters only where a key
    tile is listed by very many query tiles and its gradients stand far above s.
    """
    got = gen.bf16_bits_to_f32(got_bits).astype(np.float64)
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got), (
        f"{label}: NaN mask differs ({int(nan_ref.sum())} oracle, {int(nan_got.sum())} GPU)")
    if zero_rows is None:
        zero_rows = np.all(ref == 0, axis=-1)
    assert np.all(got_bits[zero_rows] == 0), f"{label}: rows that must be +0 are not"
    assert np.all(ref[zero_rows] == 0), f"{label}: the oracle is not 0 on a structural zero row"
    fin = np.isfinite(ref) & ~nan_ref
    assert np.array_equal(np.isinf(got), np.isinf(ref)), f"{label}: Inf mask differs"
    diff = np.abs(got[fin] - ref[fin])
    s = max(1.0, float(np.sqrt(np.mean(ref[fin] ** 2)))) if fin.any() else 1.0
    fin_ref = np.where(fin, ref, 0.0)
    row_rms = np.sqrt(np.mean(fin_ref ** 2, axis=-1, keepdims=True))
    bar = MAX_REL * s + 2.0 ** -7 * np.maximum(np.abs(fin_ref), row_rms)[fin]
    over = diff > bar
    mx = float(diff.max()) if diff.size else 0.0
    mean = float(diff.mean()) if diff.size else 0.0
    print(f"{label}: max {mx:.3e} mean {mean:.3e} (scale {s:.3f})", flush=True)
    if over.any():  # where the worst elements are, for the failure message
        idx = np.argwhere(fin)[over][:5]
        worst = [(tuple(int(x) for x in w), float(ref[tuple(w)]), float(got[tuple(w)])) for w in idx]
        print(f"{label}: {int(over.sum())} elements over the bar; first (index, oracle, GPU): {worst}",
              flush=True)
    assert not over.any() and mean <= MEAN_REL * s, f"{label}: max {mx:.3e} mean {mean:.3e} scale {s:.3f}"
    return mx / s, mean / s
