"""Sparse-index generation, float64 reference (oracle; test infrastructure only).

Notation: S tokens, block size b, N = S/b blocks, Hq query heads over Hkv KV
heads (head h reads KV head h // (Hq/Hkv)), head dimension d, sigma = 1/sqrt(d),
gamma the cumulative-mass threshold, tau the divergence threshold.

Steps, in the order the explainer's section 3.1 (streaming sparse-index
generation) and section 1.2 (Flex-Prefill's two patterns) describe them:

  1. score the last query block against every key (scaled dot product with a
     causal row softmax, the attention of section 1.1);
  2. vertical mass: attention summed along key columns, pooled into key blocks;
     slash mass: attention summed along token diagonals, pooled into offset blocks;
  3. pooled estimate: mean-pooled last query block against mean-pooled key blocks;
  4. Jensen-Shannon divergence between the estimate and the vertical mass decides
     query-aware (small divergence) or vertical-slash (explainer 1.2; tau = 0.1
     in the re-telling's section 1.1);
  5. blocks are taken in descending score until the cumulative mass reaches
     gamma (explainer 3.1, "streaming top-k"), always adding block 0 and the
     diagonal block;
  6. query-aware heads score every query block's pooled query against the
     pooled keys (re-telling 1.1, "block-level index generation for every query
     block");
  7. optionally, heads share sparse patterns (re-telling section 5, item 1:
     similar heads share one pattern): share_rows().

This module computes each step in its materialised form (the b x S score
matrix is built explicitly); the streamed form the hardware uses is pinned
against it in the tests.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

VS, QA = 0, 1


def as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- step 1
def last_block_scores(q_last, k, sigma: float) -> np.ndarray:
    """sigma * Q_last K^T for one head: [b, S] float64 (explainer 2.1: the b x S intermediate)."""
    return sigma * (as64(q_last) @ as64(k).T)


def last_block_scores_i8(q8_last, sq_last, k8, sk, sigma: float) -> np.ndarray:
    """W8A8 scores sigma * s_q[t] * s_k[k] * (q8 . k8).

    The integer dot is exact: |q8 . k8| <= 128 * 127^2 < 2^53, so every product
    and partial sum is an integer float64 represents exactly, whatever the
    summation order.
    """
    dots = np.asarray(q8_last, dtype=np.float64) @ np.asarray(k8, dtype=np.float64).T
    return sigma * as64(sq_last)[:, None] * as64(sk)[None, :] * dots


def causal_row_softmax(scores: np.ndarray) -> np.ndarray:
    """Row softmax of the last block's scores; row r is query t_r = S - b + r, keys k <= t_r."""
    bq, S = scores.shape
    t = S - bq + np.arange(bq)
    visible = np.arange(S)[None, :] <= t[:, None]
    s = np.where(visible, scores, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    e[~visible] = 0.0
    return e / e.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------- step 2
def vertical_mass(a: np.ndarray, b: int) -> np.ndarray:
    """v[j] = (1/b) * sum over the b last-block rows of the attention on key block j."""
    bq, S = a.shape
    return a.reshape(bq, S // b, b).sum(axis=(0, 2)) / bq


def slash_mass(a: np.ndarray, b: int) -> np.ndarray:
    """sl[o] = (1/b) * attention summed over token diagonals delta = t - k, pooled as o = delta // b.

    Reading: "slash" is the token-diagonal offset (query position minus key
    position) pooled into width-b offset blocks; offset block o maps to key
    block i - o for query block i.
    """
    bq, S = a.shape
    t = S - bq + np.arange(bq)
    delta = t[:, None] - np.arange(S)[None, :]
    vis = delta >= 0
    return np.bincount(delta[vis] // b, weights=a[vis], minlength=S // b)[: S // b] / bq


# ---------------------------------------------------------------- step 3
def block_means(x, b: int) -> np.ndarray:
    """Mean-pool rows of x [S, d] into [S/b, d] (arithmetic mean of each block)."""
    x = as64(x)
    return x.reshape(x.shape[0] // b, b, x.shape[1]).mean(axis=1)


def softmax(e: np.ndarray) -> np.ndarray:
    e = as64(e)
    z = np.exp(e - e.max())
    return z / z.sum()


def pooled_estimate(qbar_last, kbar, sigma: float) -> np.ndarray:
    """p[j] = softmax_j(sigma * qbar_last . kbar_j) over all N key blocks."""
    return softmax(sigma * (as64(kbar) @ as64(qbar_last)))


# ---------------------------------------------------------------- step 4
def jsd(p, q) -> float:
    """Jensen-Shannon divergence with the natural log, 0 * ln 0 = 0 (no square root)."""
    p, q = as64(p), as64(q)
    m = 0.5 * (p + q)
    out = 0.0
    for x in (p, q):
        nz = x > 0
        out += 0.5 * float(np.sum(x[nz] * np.log(x[nz] / m[nz])))
    return out


def pattern_of(D: float, tau: float) -> int:
    """Query-aware when the pooled estimate agrees with the true block mass (D < tau)."""
    return QA if D < tau else VS


# ---------------------------------------------------------------- step 5
@dataclass
class Selection:
    idx: np.ndarray          # selected indices, ascending
    order: np.ndarray        # all indices in descending value order (ties: lower index first)
    k: int                   # number selected
    total: float             # T = sum(x)


def select(x, gamma: float) -> Selection:
    """Fewest blocks, taken in descending value, whose cumulative mass reaches gamma * sum(x).

    Ties are broken by lower index first; the comparison is >= gamma * T; gamma >= 1
    selects every block.
    """
    x = as64(x)
    n = x.shape[0]
    order = np.lexsort((np.arange(n), -x))
    T = float(x.sum())
    if gamma >= 1.0 or n == 0:
        k = n
    else:
        csum = np.cumsum(x[order])
        hit = np.nonzero(csum >= gamma * T)[0]
        k = int(hit[0]) + 1 if hit.size else n
    return Selection(idx=np.sort(order[:k]), order=order, k=k, total=T)


def vs_row(vsel: np.ndarray, ssel: np.ndarray, i: int) -> np.ndarray:
    """Vertical-slash row for query block i: selected columns j <= i, diagonals i - o, and {0, i}."""
    cols = set(int(j) for j in vsel if j <= i)
    cols.update(int(i - o) for o in ssel if o <= i)
    cols.update((0, i))
    return np.array(sorted(cols), dtype=np.int64)


def qa_row(qbar_i, kbar, i: int, sigma: float, gamma: float):
    """Query-aware row for query block i: pooled scores over key blocks j <= i, softmax, select."""
    p = softmax(sigma * (as64(kbar[: i + 1]) @ as64(qbar_i)))
    sel = select(p, gamma)
    cols = set(int(j) for j in sel.idx)
    cols.update((0, i))
    return np.array(sorted(cols), dtype=np.int64), p, sel


# ---------------------------------------------------------------- whole step
@dataclass
class HeadIndex:
    v: np.ndarray
    sl: np.ndarray
    p: np.ndarray
    D: float
    pattern: int
    vsel: Optional[Selection] = None
    ssel: Optional[Selection] = None
    rows: List[np.ndarray] = field(default_factory=list)
    qa_p: List[np.ndarray] = field(default_factory=list)       # per-row softmax (QA heads)
    qa_sel: List[Selection] = field(default_factory=list)


@dataclass
class IndexResult:
    S: int
    b: int
    Hq: int
    Hkv: int
    heads: List[HeadIndex]

    @property
    def N(self) -> int:
        return self.S // self.b

    @property
    def pattern(self) -> np.ndarray:
        return np.array([hd.pattern for hd in self.heads], dtype=np.uint8)

    @property
    def jsd(self) -> np.ndarray:
        return np.array([hd.D for hd in self.heads])

    def csr(self):
        """row (h, i) -> index h*N + i; columns ascending.  Returns (row_ptr int32, col_idx int32)."""
        counts = [len(r) for hd in self.heads for r in hd.rows]
        row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
        row_ptr[1:] = np.cumsum(counts)
        col = np.concatenate([r for hd in self.heads for r in hd.rows]) if counts else np.zeros(0)
        return row_ptr.astype(np.int32), col.astype(np.int32)

    def density(self) -> float:
        N = self.N
        nnz = sum(len(r) for hd in self.heads for r in hd.rows)
        return nnz / (self.Hq * N * (N + 1) / 2)


def head_stats(scores_last, qbar_last, kbar, b: int, tau: float, sigma: float) -> HeadIndex:
    """Steps 1-4 for one query head: vertical and slash mass, pooled estimate, divergence, pattern.

    scores_last: [b, S] sigma-scaled scores of the last query block;
    qbar_last:   [d] pooled last query block of this head;
    kbar:        [N, d] pooled keys of this head's KV head.
    """
    a = causal_row_softmax(as64(scores_last))
    v = vertical_mass(a, b)
    sl = slash_mass(a, b)
    p = pooled_estimate(qbar_last, kbar, sigma)
    D = jsd(p, v)
    return HeadIndex(v=v, sl=sl, p=p, D=D, pattern=pattern_of(D, tau))


def head_rows(hd: HeadIndex, qbar_all, kbar, gamma: float, sigma: float) -> HeadIndex:
    """Step 5/6 for one head: per-query-block index sets under the head's pattern."""
    N = hd.v.shape[0]
    hd.vsel = hd.ssel = None
    hd.rows, hd.qa_p, hd.qa_sel = [], [], []
    if hd.pattern == VS:
        hd.vsel = select(hd.v, gamma)
        hd.ssel = select(hd.sl, gamma)
        hd.rows = [vs_row(hd.vsel.idx, hd.ssel.idx, i) for i in range(N)]
    else:
        for i in range(N):
            row, pi, sel = qa_row(qbar_all[i], kbar, i, sigma, gamma)
            hd.rows.append(row)
            hd.qa_p.append(pi)
            hd.qa_sel.append(sel)
    return hd


def _run(score_fn, qbar_fn, kbar_fn, Hq, Hkv, S, d, b, gamma, tau, heads, force_pattern):
    G, sigma = Hq // Hkv, 1.0 / np.sqrt(d)
    out, kbars = [], {}
    for h in (range(Hq) if heads is None else heads):
        g = h // G
        if g not in kbars:
            kbars[g] = kbar_fn(g)
        qbar_all = qbar_fn(h)
        hd = head_stats(score_fn(h, g, sigma), qbar_all[-1], kbars[g], b, tau, sigma)
        if force_pattern is not None and h in force_pattern:
            hd.pattern = int(force_pattern[h])
        out.append(head_rows(hd, qbar_all, kbars[g], gamma, sigma))
    return IndexResult(S=S, b=b, Hq=Hq, Hkv=Hkv, heads=out)


def index(Q, K, b: int, gamma: float, tau: float, heads=None, force_pattern=None) -> IndexResult:
    """Sparse index for bf16-valued inputs Q [Hq, S, d], K [Hkv, S, d] (any float dtype, upcast exactly).

    force_pattern: optional {head: VS|QA} overriding the divergence test (used
    when a test compares rows under the pattern the device chose at a tie).
    """
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    return _run(lambda h, g, sg: last_block_scores(Q[h, S - b:], K[g], sg),
                lambda h: block_means(Q[h], b),
                lambda g: block_means(K[g], b),
                Hq, Hkv, S, d, b, gamma, tau, heads, force_pattern)


def index_i8(Q8, sQ, K8, sK, b: int, gamma: float, tau: float, heads=None, force_pattern=None) -> IndexResult:
    """Sparse index for W8A8 inputs: int8 [H, S, d] with float32 per-(head, token) scales [H, S].

    Scores use the exact integer dot; pooled vectors use the dequantised values s * x8.
    """
    Hq, S, d = Q8.shape
    Hkv = K8.shape[0]
    return _run(lambda h, g, sg: last_block_scores_i8(Q8[h, S - b:], sQ[h, S - b:], K8[g], sK[g], sg),
                lambda h: block_means(as64(sQ[h])[:, None] * as64(Q8[h]), b),
                lambda g: block_means(as64(sK[g])[:, None] * as64(K8[g]), b),
                Hq, Hkv, S, d, b, gamma, tau, heads, force_pattern)


# ---------------------------------------------------------------- step 7 (optional)
def share_rows(res: IndexResult) -> IndexResult:
    """Head-pattern sharing: every head h of KV group g takes, per query block i, the union of the
    index sets of the heads of g whose pattern equals h's (re-telling section 5, item 1: similar
    heads share one sparse pattern; "similar" is read as same KV group and same pattern).

    Returns a new IndexResult whose heads keep their statistics, pattern and selections and carry
    the shared rows; the input is not modified."""
    G = res.Hq // res.Hkv
    N = res.N
    heads = []
    for h, hd in enumerate(res.heads):
        g = h // G
        peers = [res.heads[p] for p in range(g * G, (g + 1) * G) if res.heads[p].pattern == hd.pattern]
        rows = [np.array(sorted(set().union(*(set(int(j) for j in pr.rows[i]) for pr in peers))), dtype=np.int64)
                for i in range(N)]
        heads.append(HeadIndex(v=hd.v, sl=hd.sl, p=hd.p, D=hd.D, pattern=hd.pattern, vsel=hd.vsel, ssel=hd.ssel,
                               rows=rows, qa_p=hd.qa_p, qa_sel=hd.qa_sel))
    return IndexResult(S=res.S, b=res.b, Hq=res.Hq, Hkv=res.Hkv, heads=heads)


def block_uses(res: IndexResult):
    """Use counters of the key blocks (explainer section 3.2: each KV block's number of consumers,
    counted while the job list is built): uses[g, j] = number of query blocks i whose grouped job
    (the union of J(h, i) over the heads h of KV group g) holds j; head_uses[g, j] = number of
    (head, query block) pairs of group g whose index set holds j."""
    G, N = res.Hq // res.Hkv, res.N
    uses = np.zeros((res.Hkv, N), dtype=np.int64)
    head_uses = np.zeros((res.Hkv, N), dtype=np.int64)
    for g in range(res.Hkv):
        for i in range(N):
            union = set()
            for h in range(g * G, (g + 1) * G):
                row = res.heads[h].rows[i]
                union.update(int(j) for j in row)
                head_uses[g, row] += 1
            uses[g, sorted(union)] += 1
    return uses, head_uses
