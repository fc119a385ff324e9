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
