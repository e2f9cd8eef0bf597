"""Block-sparse causal attention, float64 reference (oracle; test infrastructure only).

For query block i of head h with selected key blocks J (a CSR row), every query
token t of block i attends to the keys k <= t whose block is in J, with the
scaled-dot-product softmax of the explainer's section 1.1 taken over exactly
those keys (explainer 1.2, figure 3: each query block interacts only with the
KV blocks its sparse index names).  Block i itself is always in J, so the set
is never empty.

W8A8 (explainer 3.3 and 4.2: INT8 x INT8 with INT32 accumulation; re-telling
3.3): scores are sigma * s_q[t] * s_k[k] * (q8 . k8) with the integer dot
exact, and P V uses the dequantised values s_v[k] * v8[k].
"""
from __future__ import annotations

import numpy as np


def as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _row_keys(cols, b: int) -> np.ndarray:
    return np.concatenate([np.arange(j * b, (j + 1) * b) for j in cols])


def _softmax_rows_masked(s: np.ndarray, visible: np.ndarray) -> np.ndarray:
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    e[~visible] = 0.0
    return e / e.sum(axis=1, keepdims=True)


def attn_row(q_blk, k, v, cols, i: int, b: int, sigma: float) -> np.ndarray:
    """Output [b, d] of query block i (q_blk = its b query rows) over key blocks `cols`."""
    keys = _row_keys(cols, b)
    s = sigma * (as64(q_blk) @ as64(k[keys]).T)
    qpos = i * b + np.arange(b)
    p = _softmax_rows_masked(s, keys[None, :] <= qpos[:, None])
    return p @ as64(v[keys])


def attn_row_i8(q8_blk, sq_blk, k8, sk, v8, sv, cols, i: int, b: int, sigma: float) -> np.ndarray:
    keys = _row_keys(cols, b)
    dots = np.asarray(q8_blk, dtype=np.float64) @ np.asarray(k8[keys], dtype=np.float64).T
    s = sigma * as64(sq_blk)[:, None] * as64(sk[keys])[None, :] * dots
    qpos = i * b + np.arange(b)
    p = _softmax_rows_masked(s, keys[None, :] <= qpos[:, None])
    return p @ (as64(sv[keys])[:, None] * as64(v8[keys]))


def attn(Q, K, V, row_ptr, col_idx, b: int, rows=None):
    """Sparse attention for bf16-valued Q [Hq,S,d], K/V [Hkv,S,d] under CSR (row = h*N + i).

    rows=None returns the full output [Hq, S, d]; otherwise a dict {(h, i): [b, d]}
    for the listed (h, i) pairs only.
    """
    Hq, S, d = Q.shape
    G, N, sigma = Hq // K.shape[0], S // b, 1.0 / np.sqrt(d)
    todo = [(h, i) for h in range(Hq) for i in range(N)] if rows is None else list(rows)
    res = {}
    for h, i in todo:
        r = h * N + i
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        res[(h, i)] = attn_row(Q[h, i * b:(i + 1) * b], K[h // G], V[h // G], cols, i, b, sigma)
    if rows is not None:
        return res
    out = np.zeros((Hq, S, d))
    for (h, i), o in res.items():
        out[h, i * b:(i + 1) * b] = o
    return out


def attn_i8(Q8, sQ, K8, sK, V8, sV, row_ptr, col_idx, b: int, rows=None):
    """W8A8 sparse attention; same conventions as attn()."""
    Hq, S, d = Q8.shape
    G, N, sigma = Hq // K8.shape[0], S // b, 1.0 / np.sqrt(d)
    todo = [(h, i) for h in range(Hq) for i in range(N)] if rows is None else list(rows)
    res = {}
    for h, i in todo:
        r = h * N + i
        g = h // G
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        sl = slice(i * b, (i + 1) * b)
        res[(h, i)] = attn_row_i8(Q8[h, sl], sQ[h, sl], K8[g], sK[g], V8[g], sV[g], cols, i, b, sigma)
    if rows is not None:
        return res
    out = np.zeros((Hq, S, d))
    for (h, i), o in res.items():
        out[h, i * b:(i + 1) * b] = o
    return out
