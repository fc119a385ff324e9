"""Plain fp64 definition of block-sparse attention with its log-sum-exp and gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the GPU
library imports, links or calls this module.

The forward is the plain definition the C oracle writes out in binary32
(FastVideo fastvideo-kernel commit list, page 3: the 128-token sm_121a forward
commit's binding, the hardening commit's zero-row, NaN-sum and padding rules),
here in fp64 so that it can be differentiated and checked by finite
differences.  The pages name an LSE-requiring autograd path but print no
backward formula; the gradients below are those of that same plain
definition, per query row r with a non-empty key list K_r (the listed tiles'
valid key rows in list order, a tile listed twice counted twice):

    s = scale * q_r . k          P = softmax(s)        out_r = P V
    dV[key] += P[key] dO_r       dP = dO_r V^T         D_r = dO_r . out_r
    dS = P * (dP - D_r)          dq_r = scale * dS K   dK[key] += scale * dS[key] q_r

Rows without keys and padding query rows (r >= block_sizes[i]) have a
constant output (+0), so they produce no gradient; padding key rows are never
read, so their dk and dv are 0.  lse_r = log sum exp(s) in natural-log units,
-inf for rows without keys, for padding rows and for rows whose logits are all
-inf (log 0; their output is the NaN row of the hardening commit).
"""
from __future__ import annotations

import numpy as np


def _widen(x):
    """bf16 bit patterns (uint16) -> float64 exactly; float arrays pass through as float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _check(q2k_idx, q2k_num, vbs, B, H, NT, T):
    q2k_num = np.asarray(q2k_num)
    vbs = np.asarray(vbs)
    if q2k_num.shape != (B, H, NT) or vbs.shape != (NT,):
        raise ValueError("q2k_num must be [B, H, NT] and block sizes [NT]")
    MS = 0 if q2k_idx is None else np.asarray(q2k_idx).shape[3]
    if np.any(q2k_num < 0) or np.any(q2k_num > MS):
        raise ValueError("q2k_num outside [0, MS]")
    if np.any(vbs < 0) or np.any(vbs > T):
        raise ValueError("tile length outside [0, T]")
    for b in range(B):
        for h in range(H):
            for i in range(NT):
                lst = np.asarray(q2k_idx)[b, h, i, :q2k_num[b, h, i]]
                if np.any(lst < 0) or np.any(lst >= NT):
                    raise ValueError("key-tile index outside [0, NT)")


def _keys(q2k_idx, q2k_num, vbs, T, b, h, i):
    """Key rows of query tile i's list: listed tiles' valid rows, in list order."""
    n = int(q2k_num[b, h, i])
    if n == 0:
        return np.zeros(0, np.int64)
    return np.concatenate([j * T + np.arange(vbs[j], dtype=np.int64)
                           for j in np.asarray(q2k_idx)[b, h, i, :n]])


def scale_of(D):
    return 1.0 / np.sqrt(float(D))


def fwd64(q, k, v, q2k_idx, q2k_num, vbs, tile):
    """(out [B, H, S, D], lse [B, H, S]) in fp64."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    B, H, S, D = q.shape
    T = tile
    NT = S // T
    vbs = np.asarray(vbs, np.int64)
    _check(q2k_idx, q2k_num, vbs, B, H, NT, T)
    sc = scale_of(D)
    out = np.zeros_like(q)
    lse = np.full((B, H, S), -np.inf)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for b in range(B):
            for h in range(H):
                for i in range(NT):
                    vq = int(vbs[i])
                    keys = _keys(q2k_idx, q2k_num, vbs, T, b, h, i)
                    if vq == 0 or keys.size == 0:
                        continue
                    rows = slice(i * T, i * T + vq)
                    s = sc * (q[b, h, rows] @ k[b, h, keys].T)
                    m = s.max(axis=1, keepdims=True)
                    p = np.exp(s - m)
                    l = p.sum(axis=1, keepdims=True)
                    out[b, h, rows] = (p / l) @ v[b, h, keys]
                    # log sum exp(s): log 0 = -inf when every logit is -inf (the max
                    # shift would give -inf - -inf there)
                    lse[b, h, rows] = np.where(np.isneginf(m), -np.inf, m + np.log(l))[:, 0]
    return out, lse


def bwd(q, k, v, dout, q2k_idx, q2k_num, vbs, tile):
    """(dq, dk, dv) in fp64, each [B, H, S, D], for the upstream gradient dout."""
    q, k, v, dout = _widen(q), _widen(k), _widen(v), _widen(dout)
    B, H, S, D = q.shape
    T = tile
    NT = S // T
    vbs = np.asarray(vbs, np.int64)
    _check(q2k_idx, q2k_num, vbs, B, H, NT, T)
    sc = scale_of(D)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for b in range(B):
            for h in range(H):
                for i in range(NT):
                    vq = int(vbs[i])
                    keys = _keys(q2k_idx, q2k_num, vbs, T, b, h, i)
                    if vq == 0 or keys.size == 0:
                        continue
                    rows = slice(i * T, i * T + vq)
                    qi, do = q[b, h, rows], dout[b, h, rows]
                    kk, vv = k[b, h, keys], v[b, h, keys]
                    s = sc * (qi @ kk.T)
                    p = np.exp(s - s.max(axis=1, keepdims=True))
                    p /= p.sum(axis=1, keepdims=True)
                    o = p @ vv
                    dp = do @ vv.T
                    d_row = (do * o).sum(axis=1, keepdims=True)
                    ds = p * (dp - d_row)
                    dq[b, h, rows] = sc * (ds @ kk)
                    np.add.at(dk[b, h], keys, sc * (ds.T @ qi))
                    np.add.at(dv[b, h], keys, p.T @ do)
    return dq, dk, dv
