"""Brute-force and alternative forms used only to pin oracle.index / oracle.attn.

Each function here reaches the same quantity as the oracle by a different
route, so that a dropped term, wrong sign, wrong index or transposed operand in
either one shows up as a disagreement in the tests:

* dense_masked_attention: the full S x S score matrix with an explicit token
  mask, instead of gathering selected key blocks;
* token_mask_from_csr: expands a block-level CSR to that token mask;
* streamed_stats: one pass over key blocks in increasing order with per-row
  running max / sum and per-(row, block) partials split at the token diagonal
  (the stream-and-accumulate form of the explainer's section 3.1), instead of
  materialising the b x S matrix;
* exhaustive_select: the fewest-items-reaching-a-mass optimum by enumerating
  every subset (tiny n only);
* qa_rows_dense: query-aware rows from the whole N x N matrix of pooled
  logits (pooling as a matrix product, causal block mask, row softmax through
  scipy's log-sum-exp, exhaustive subset search per row), instead of one row
  at a time with greedy selection.
"""
from __future__ import annotations

import itertools

import numpy as np
import scipy.special


def as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def dense_masked_attention(q, k, v, mask) -> np.ndarray:
    """One head: softmax over the keys allowed by mask [S, S] (query row, key column), then @ v."""
    q, k, v = as64(q), as64(k), as64(v)
    s = (q @ k.T) / np.sqrt(q.shape[1])
    s[~mask] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v


def causal_mask(S: int) -> np.ndarray:
    return np.tril(np.ones((S, S), dtype=bool))


def token_mask_from_csr(row_ptr, col_idx, h: int, S: int, b: int) -> np.ndarray:
    N = S // b
    blk = np.zeros((N, N), dtype=bool)
    for i in range(N):
        r = h * N + i
        blk[i, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return np.kron(blk, np.ones((b, b), dtype=bool)) & causal_mask(S)


def streamed_stats(q_last, k, b: int):
    """Vertical / slash mass of the last query block computed in one pass over key blocks.

    Per row r (query t_r = S - b + r) and key block j, the partial sums of
    exp(score - m) over keys with in-block offset c <= r ("lo") and c > r ("hi")
    are kept together with the running max m they were taken against; the row
    softmax denominator is only known after the last block, so the partials are
    renormalised at the end.  Slash offset block o collects lo of key block
    N-1-o and hi of key block N-2-o.
    """
    q_last, k = as64(q_last), as64(k)
    bq, d = q_last.shape
    S = k.shape[0]
    N = S // b
    sigma = 1.0 / np.sqrt(d)
    m = np.full(bq, -np.inf)
    ref = np.zeros((N, bq))
    lo = np.zeros((N, bq))
    hi = np.zeros((N, bq))
    r = np.arange(bq)
    c = np.arange(b)
    for j in range(N):
        s = sigma * (q_last @ k[j * b:(j + 1) * b].T)          # [bq, b]
        if j == N - 1:
            s = np.where(c[None, :] <= r[:, None], s, -np.inf)  # causal mask on the diagonal block
        m = np.maximum(m, s.max(axis=1))
        e = np.exp(s - m[:, None])
        low = c[None, :] <= r[:, None]
        lo[j] = np.where(low, e, 0.0).sum(axis=1)
        hi[j] = np.where(low, 0.0, e).sum(axis=1)
        ref[j] = m
    scale = np.exp(ref - m[None, :])                             # bring every partial to the final max
    L = ((lo + hi) * scale).sum(axis=0)
    w = scale / (bq * L[None, :])
    LO = (lo * w).sum(axis=1)
    HI = (hi * w).sum(axis=1)
    v = LO + HI
    sl = np.zeros(N)
    for o in range(N):
        sl[o] = LO[N - 1 - o] + (HI[N - 2 - o] if N - 2 - o >= 0 else 0.0)
    return v, sl, LO, HI


def exhaustive_select(x, gamma: float):
    """(k_min, best_mass, optimal_sets) for: fewest indices whose sum reaches gamma * sum(x)."""
    x = as64(x)
    n = x.shape[0]
    T = x.sum()
    if gamma >= 1.0:
        return n, T, [tuple(range(n))]
    for kk in range(1, n + 1):
        masses = {}
        for comb in itertools.combinations(range(n), kk):
            mass = x[list(comb)].sum()
            if mass >= gamma * T:
                masses[comb] = mass
        if masses:
            best = max(masses.values())
            opt = [c for c, ms in masses.items() if ms == best]
            return kk, best, opt
    return n, T, [tuple(range(n))]


def pooling_matrix(S: int, b: int) -> np.ndarray:
    """[N, S] matrix whose row i averages tokens i*b .. i*b + b - 1."""
    return np.kron(np.eye(S // b), np.full((1, b), 1.0 / b))


def qa_rows_dense(q, k, b: int, gamma: float):
    """Query-aware rows of one head by brute force.

    q: [S, d] queries of the head, k: [S, d] keys of its KV head.  The pooled
    logits of every (query block i, key block j) pair form one N x N matrix
    scaled by 1/sqrt(d); key blocks after the query block are masked out,
    each row is normalised with log-sum-exp, and each row's selection is the
    exhaustive optimum (fewest blocks reaching gamma of the row's mass, most
    mass among those).  Returns one (p_i, optimal sets, k_min) per row, where
    every optimal set already contains block 0 and the diagonal block i.
    """
    q, k = as64(q), as64(k)
    S, d = q.shape
    P = pooling_matrix(S, b)
    logits = (P @ q) @ (P @ k).T / np.sqrt(d)
    N = logits.shape[0]
    causal = np.tril(np.ones((N, N), dtype=bool))
    masked = np.where(causal, logits, -np.inf)
    logp = masked - scipy.special.logsumexp(masked, axis=1, keepdims=True)
    out = []
    for i in range(N):
        p_i = np.exp(logp[i, : i + 1])
        kmin, _, opt = exhaustive_select(p_i, gamma)
        sets = sorted({tuple(sorted(set(o) | {0, i})) for o in opt})
        out.append((p_i, sets, kmin))
    return out
