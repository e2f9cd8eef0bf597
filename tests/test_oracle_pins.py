"""Pins for the float64 oracle against facts fixed outside the oracle itself.

Each test compares the oracle with a closed form, a hand-worked example, a
library routine, brute force on tiny inputs, or an invariant of the
mathematics, chosen so that a plausible slip (dropped term, wrong sign or
index, transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.spatial.distance
import torch
from hypothesis import given, settings, strategies as st

import gen
import oracle
from oracle import brute
from oracle import index as oi

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(rng, S, b, Hq, Hkv, d, scale=1.0):
    Q = rng.standard_normal((Hq, S, d)) * scale
    K = rng.standard_normal((Hkv, S, d)) * scale
    V = rng.standard_normal((Hkv, S, d))
    return Q, K, V


# ------------------------------------------------------------ statistics
def test_hand_example():
    ex = json.load(open(os.path.join(GOLD, "hand_example_S4.json")))
    q = np.array(ex["q"])
    k = np.log(np.array(ex["k_exp"]))[:, None]
    sc = oi.last_block_scores(q[2:], k, 1.0)
    a = oi.causal_row_softmax(sc)
    np.testing.assert_allclose(oi.vertical_mass(a, 2), ex["v"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oi.slash_mass(a, 2), ex["sl"], rtol=0, atol=1e-15)
    qbar = oi.block_means(q, 2)
    kbar = oi.block_means(k, 2)
    np.testing.assert_allclose(oi.pooled_estimate(qbar[-1], kbar, 1.0), ex["p_est"], atol=1e-15)
    assert list(oi.select(ex["v"], 0.5).idx) == ex["select_v_gamma_0.5"]
    assert list(oi.select(ex["sl"], 0.5).idx) == ex["select_sl_gamma_0.5"]


def test_page_facts():
    f = json.load(open(os.path.join(GOLD, "page_facts.json")))
    cfg = gen.CONFIGS["3b-128k"]
    assert cfg.tau == f["tau"]["value"]
    stated = set(f["block_sizes"]["value"]) | set(f["tuned_block_sizes"]["value"])
    assert all(c.b in stated for c in gen.CONFIGS.values())
    assert (cfg.b, cfg.S) == (f["naive_intermediate_per_head"]["rows"], f["naive_intermediate_per_head"]["cols"])
    # one fp32 block score per key block of one head
    assert cfg.N * 4 == f["score_buffer_bytes_128k"]["approx"]


@pytest.mark.parametrize("S,b,d", [(512, 128, 32), (1024, 128, 128), (1024, 256, 64), (256, 128, 16)])
def test_streamed_equals_materialised(S, b, d):
    rng = np.random.default_rng(S + b + d)
    q = rng.standard_normal((b, d)) * 2
    k = rng.standard_normal((S, d)) * 2
    k[5] += 3 * q.mean(0)
    a = oi.causal_row_softmax(oi.last_block_scores(q, k, 1 / math.sqrt(d)))
    v, sl = oi.vertical_mass(a, b), oi.slash_mass(a, b)
    v2, sl2, LO, HI = brute.streamed_stats(q, k, b)
    np.testing.assert_allclose(v, v2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sl, sl2, rtol=1e-12, atol=1e-15)
    assert abs(v.sum() - 1) < 1e-12 and abs(sl.sum() - 1) < 1e-12
    np.testing.assert_allclose(v, LO + HI, rtol=1e-12, atol=1e-15)
    N = S // b
    assert HI[N - 1] == 0.0
    for o in range(N):
        ref = LO[N - 1 - o] + (HI[N - 2 - o] if o <= N - 2 else 0.0)
        assert abs(sl[o] - ref) < 1e-12


def test_streamed_equals_materialised_on_planted_layer():
    L = gen.make("tiny")
    Q, K = L.f32("q"), L.f32("k")
    for h in range(4):
        a = oi.causal_row_softmax(oi.last_block_scores(Q[h, -128:], K[h // 2], 1 / math.sqrt(128)))
        v2, sl2, _, _ = brute.streamed_stats(Q[h, -128:], K[h // 2], 128)
        np.testing.assert_allclose(oi.vertical_mass(a, 128), v2, rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(oi.slash_mass(a, 128), sl2, rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("S,b", [(512, 128), (1024, 256), (128, 128)])
def test_zero_keys_closed_form(S, b):
    """K = 0: every visible key is equally likely, a_r[k] = 1/(t_r + 1)."""
    d = 8
    rng = np.random.default_rng(0)
    q = rng.standard_normal((b, d))
    k = np.zeros((S, d))
    N = S // b
    t = S - b + np.arange(b)
    r = np.arange(b)
    full = np.sum(b / (t + 1.0)) / b
    last = np.sum((r + 1.0) / (t + 1.0)) / b
    v_exp = np.full(N, full)
    v_exp[N - 1] = last
    sl_exp = np.full(N, full)
    sl_exp[N - 1] = last
    a = oi.causal_row_softmax(oi.last_block_scores(q, k, 1 / math.sqrt(d)))
    np.testing.assert_allclose(oi.vertical_mass(a, b), v_exp, rtol=1e-12)
    np.testing.assert_allclose(oi.slash_mass(a, b), sl_exp, rtol=1e-12)
    p = oi.pooled_estimate(q.mean(0), oi.block_means(k, b), 1 / math.sqrt(d))
    np.testing.assert_allclose(p, np.full(N, 1.0 / N), rtol=1e-14)


def test_huge_logit_one_hot():
    """One key at the start of block j* with a huge logit takes all the mass of every last-block row."""
    S, b, d = 1024, 128, 16
    N = S // b
    rng = np.random.default_rng(1)
    q = rng.standard_normal((b, d)) * 0.1 + 1.0
    k = rng.standard_normal((S, d)) * 0.1
    jstar = 3
    k[jstar * b] = 200.0
    a = oi.causal_row_softmax(oi.last_block_scores(q, k, 1 / math.sqrt(d)))
    v, sl = oi.vertical_mass(a, b), oi.slash_mass(a, b)
    e_v = np.zeros(N)
    e_v[jstar] = 1
    e_s = np.zeros(N)
    e_s[N - 1 - jstar] = 1
    np.testing.assert_allclose(v, e_v, atol=1e-12)
    np.testing.assert_allclose(sl, e_s, atol=1e-12)


# ------------------------------------------------------------ divergence
def test_jsd_special_cases():
    p = np.array([0.2, 0.3, 0.5])
    assert oi.jsd(p, p) == 0.0
    assert abs(oi.jsd([1, 0, 0, 0], [0, 0.5, 0.5, 0]) - math.log(2)) < 1e-15
    q = np.array([0.6, 0.1, 0.3])
    assert abs(oi.jsd(p, q) - oi.jsd(q, p)) < 1e-16


@pytest.mark.parametrize("seed", range(5))
def test_jsd_matches_scipy(seed):
    rng = np.random.default_rng(seed)
    p = rng.random(37) ** 3
    q = rng.random(37)
    q[3] = 0.0
    p /= p.sum()
    q /= q.sum()
    ref = scipy.spatial.distance.jensenshannon(p, q) ** 2  # natural log by default
    assert abs(oi.jsd(p, q) - ref) < 1e-13


# ------------------------------------------------------------ selection
@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("gamma", [0.3, 0.5, 0.9, 0.95, 0.999])
def test_select_exhaustive(seed, gamma):
    rng = np.random.default_rng(seed)
    n = 4 + seed % 7
    x = rng.random(n) ** (1 + seed % 3)
    if seed % 4 == 0:
        x = np.round(x * 4)          # ties
        x[0] = max(x[0], 1.0)
    sel = oi.select(x, gamma)
    kmin, best, opt = brute.exhaustive_select(x, gamma)
    assert sel.k == kmin
    assert abs(x[sel.idx].sum() - best) < 1e-12
    assert tuple(sel.idx) in [tuple(sorted(o)) for o in opt] or any(
        abs(x[list(o)].sum() - x[sel.idx].sum()) < 1e-12 for o in opt)


def test_select_ties_lower_index_first_and_gamma_one():
    x = np.array([1.0, 2.0, 1.0, 2.0, 1.0])
    assert list(oi.select(x, 0.5).idx) == [1, 3]        # 4 of 7 >= 3.5 with the two 2's
    assert list(oi.select(x, 0.6).idx) == [0, 1, 3]     # a third element: the lowest-index 1
    assert list(oi.select(x, 1.0).idx) == [0, 1, 2, 3, 4]
    assert list(oi.select(np.zeros(3) + 1e-300, 1.0).idx) == [0, 1, 2]


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(min_value=0.0, max_value=1.0, allow_nan=False), min_size=1, max_size=40),
       st.floats(min_value=0.01, max_value=0.999))
def test_select_properties(xs, gamma):
    x = np.array(xs)
    if x.sum() <= 0:
        x[0] = 1.0
    sel = oi.select(x, gamma)
    T = x.sum()
    mass = x[sel.idx].sum()
    assert mass >= gamma * T * (1 - 1e-12)
    # every unselected value is <= every selected value
    uns = np.setdiff1d(np.arange(len(x)), sel.idx)
    if uns.size:
        assert x[uns].max() <= x[sel.idx].min()
    # dropping the smallest selected element falls short (minimal count)
    if sel.k > 1:
        assert mass - x[sel.idx].min() < gamma * T * (1 + 1e-12)


# ------------------------------------------------------------ rows and csr
def test_rows_structure_and_planted_labels():
    L = gen.make("tiny")
    Q, K = L.f32("q"), L.f32("k")
    res = oi.index(Q, K, 128, 0.9, 0.1)
    assert list(res.pattern) == list(L.planted)          # VS heads planted VS, QA heads planted QA
    N = res.N
    for hd in res.heads:
        assert len(hd.rows) == N
        for i, row in enumerate(hd.rows):
            assert row[0] == 0 and i in row and row.max() <= i
            assert np.all(np.diff(row) > 0)
        if hd.pattern == oi.VS:
            assert hd.v[hd.vsel.idx].sum() >= 0.9 * hd.v.sum()
            assert hd.sl[hd.ssel.idx].sum() >= 0.9 * hd.sl.sum()
        else:
            for pi, sel in zip(hd.qa_p, hd.qa_sel):
                assert pi[sel.idx].sum() >= 0.9 * pi.sum() * (1 - 1e-15)
    rp, ci = res.csr()
    assert rp[0] == 0 and rp[-1] == ci.size and np.all(np.diff(rp) >= 1)


def _qa_hand_layer():
    ex = json.load(open(os.path.join(GOLD, "qa_rows_hand.json")))
    S, b, d = ex["S"], ex["b"], ex["d"]
    N = S // b
    a, c = np.array(ex["a"], float), np.array(ex["c"], float)
    kbar = np.zeros((N, d))
    kbar[:, 0], kbar[:, 1] = 2 * np.log(a), 2 * np.log(c)
    dk, dq = np.array(ex["k_delta"]), np.array(ex["q_eps"])
    qbar = np.array(ex["qbar"], float)
    K = np.zeros((1, S, d))
    Q = np.zeros((1, S, d))
    for j in range(N):
        K[0, 2 * j], K[0, 2 * j + 1] = kbar[j] + dk, kbar[j] - dk
        Q[0, 2 * j], Q[0, 2 * j + 1] = qbar[j] + dq, qbar[j] - dq
    return ex, Q, K


def test_qa_rows_hand_example():
    """Query-aware rows and the pooled estimate against exact fractions (d = 4, so sigma = 1/2)."""
    ex, Q, K = _qa_hand_layer()
    res = oi.index(Q, K, ex["b"], ex["gamma"], 0.1, force_pattern={0: oi.QA})
    hd = res.heads[0]
    for want, row, p in zip(ex["rows"], hd.rows, hd.qa_p):
        w = np.array(want["weights"], float)
        np.testing.assert_allclose(p, w / want["den"], rtol=1e-13, atol=0)
        assert list(row) == want["row"], want["i"]
    pe = np.array(ex["p_est"]["weights"], float) / ex["p_est"]["den"]
    np.testing.assert_allclose(hd.p, pe, rtol=1e-13, atol=0)
    # the vertical mass through index() uses the same sigma as the independent streamed form
    v2, sl2, _, _ = brute.streamed_stats(Q[0, -ex["b"]:], K[0], ex["b"])
    np.testing.assert_allclose(hd.v, v2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(hd.sl, sl2, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("gamma", [0.5, 0.8, 0.9, 0.97])
def test_qa_rows_match_brute_force(seed, gamma):
    """qa_row (greedy, one row at a time) against the dense pooled-logit matrix with exhaustive selection."""
    rng = np.random.default_rng(100 + seed)
    b, d = (2, 4, 8)[seed % 3], (4, 8, 16)[seed % 3]
    N = 3 + seed % 8
    S = N * b
    scale = 1.0 + seed % 4
    Q = rng.standard_normal((1, S, d)) * scale
    K = rng.standard_normal((1, S, d)) * scale
    res = oi.index(Q, K, b, gamma, 0.1, force_pattern={0: oi.QA})
    ref = brute.qa_rows_dense(Q[0], K[0], b, gamma)
    for i, (row, p, sel) in enumerate(zip(res.heads[0].rows, res.heads[0].qa_p, res.heads[0].qa_sel)):
        p_ref, sets, kmin = ref[i]
        np.testing.assert_allclose(p, p_ref, rtol=1e-11, atol=1e-15)
        assert sel.k == kmin, (i, sel.k, kmin)
        assert tuple(row) in sets, (i, list(row), sets)


def test_share_rows_by_hand():
    """Head-pattern sharing on hand-written rows: one group of three heads (two query-aware, one
    vertical-slash) and one group of a single head."""
    def hd(pattern, rows):
        return oi.HeadIndex(v=np.zeros(3), sl=np.zeros(3), p=np.zeros(3), D=0.0, pattern=pattern,
                            rows=[np.array(r) for r in rows])
    res = oi.IndexResult(S=6, b=2, Hq=4, Hkv=2, heads=[
        hd(oi.QA, [[0], [0, 1], [0, 2]]),
        hd(oi.VS, [[0], [0, 1], [0, 1, 2]]),
        hd(oi.QA, [[0], [0, 1], [0, 1, 2]]),
        hd(oi.VS, [[0], [0, 1], [0, 2]]),
    ])
    # G = 2: group 0 = heads 0, 1 (QA, VS: nothing shared), group 1 = heads 2, 3 (QA, VS)
    sh = oi.share_rows(res)
    assert [list(r) for r in sh.heads[0].rows] == [[0], [0, 1], [0, 2]]
    assert [list(r) for r in sh.heads[1].rows] == [[0], [0, 1], [0, 1, 2]]
    res.Hkv = 1   # G = 4: heads 0 and 2 share (QA), heads 1 and 3 share (VS)
    sh = oi.share_rows(res)
    assert [list(r) for r in sh.heads[0].rows] == [[0], [0, 1], [0, 1, 2]]
    assert [list(r) for r in sh.heads[2].rows] == [[0], [0, 1], [0, 1, 2]]
    assert [list(r) for r in sh.heads[1].rows] == [[0], [0, 1], [0, 1, 2]]
    assert [list(r) for r in sh.heads[3].rows] == [[0], [0, 1], [0, 1, 2]]
    assert [list(r) for r in res.heads[3].rows] == [[0], [0, 1], [0, 2]]     # input untouched


def test_share_rows_invariants_on_planted_layer():
    L = gen.make(gen.CONFIGS["tiny"].with_(S=1024, Hq=6, Hkv=2))
    res = oi.index(L.f32("q"), L.f32("k"), 128, 0.9, 0.1)
    sh = oi.share_rows(res)
    G = 3
    for h, (a, b_) in enumerate(zip(res.heads, sh.heads)):
        peers = [p for p in range(h // G * G, h // G * G + G) if res.heads[p].pattern == a.pattern]
        for i in range(res.N):
            assert set(a.rows[i]) <= set(b_.rows[i])                   # a superset of the head's own row
            assert set(b_.rows[i]) == set().union(*(set(res.heads[p].rows[i]) for p in peers))
            assert np.all(np.diff(b_.rows[i]) > 0) and b_.rows[i][0] == 0 and b_.rows[i][-1] == i
    assert sh.density() >= res.density()
    # one head per group: sharing changes nothing
    r1 = oi.index(L.f32("q")[:2], L.f32("k"), 128, 0.9, 0.1)
    assert all(np.array_equal(x, y) for a, b_ in zip(r1.heads, oi.share_rows(r1).heads) for x, y in zip(a.rows, b_.rows))


def test_block_uses_by_hand():
    """Use counters on hand-written rows: G = 2, N = 3."""
    def hd(rows):
        return oi.HeadIndex(v=np.zeros(3), sl=np.zeros(3), p=np.zeros(3), D=0.0, pattern=oi.QA,
                            rows=[np.array(r) for r in rows])
    res = oi.IndexResult(S=6, b=2, Hq=2, Hkv=1, heads=[hd([[0], [0, 1], [0, 2]]), hd([[0], [0, 1], [0, 1, 2]])])
    uses, head_uses = oi.block_uses(res)
    # jobs: i=0 {0}, i=1 {0,1}, i=2 {0,1,2}
    assert uses.tolist() == [[3, 2, 1]]
    assert head_uses.tolist() == [[6, 3, 2]]


def test_block_uses_totals_on_planted_layer():
    L = gen.make(gen.CONFIGS["tiny"].with_(S=1024, Hq=6, Hkv=2))
    res = oi.index(L.f32("q"), L.f32("k"), 128, 0.9, 0.1)
    uses, head_uses = oi.block_uses(res)
    rp, ci = res.csr()
    assert head_uses.sum() == ci.size                          # every (h, i, j) counted once
    G, N = 3, res.N
    unions = sum(len(set().union(*(set(res.heads[h].rows[i]) for h in range(g * G, g * G + G))))
                 for g in range(2) for i in range(N))
    assert uses.sum() == unions                                # every job entry counted once
    assert np.all(uses[:, 0] == N)                             # block 0 is in every row
    assert np.all(uses <= head_uses) and np.all(head_uses <= G * uses)


def test_single_block_sequence():
    rng = np.random.default_rng(2)
    Q, K, V = rand_layer(rng, 128, 128, 2, 1, 16)
    res = oi.index(Q, K, 128, 0.9, 0.1)
    for hd in res.heads:
        assert [list(r) for r in hd.rows] == [[0]]


def test_vs_row_expansion_by_hand():
    # V = {2, 5}, slash offsets {0, 3}; row 4: columns {2} (5 > 4), diagonals {4, 1}, plus {0, 4}
    assert list(oi.vs_row(np.array([2, 5]), np.array([0, 3]), 4)) == [0, 1, 2, 4]
    assert list(oi.vs_row(np.array([2, 5]), np.array([0, 3]), 0)) == [0]
    assert list(oi.vs_row(np.array([2, 5]), np.array([0, 3]), 7)) == [0, 2, 4, 5, 7]


def test_gamma_one_selects_everything():
    L = gen.make("tiny")
    res = oi.index(L.f32("q"), L.f32("k"), 128, 1.0, 0.1)
    for hd in res.heads:
        for i, row in enumerate(hd.rows):
            assert list(row) == list(range(i + 1))
    assert res.density() == 1.0


# ------------------------------------------------------------ attention
def _sdpa_causal(Q, K, V):
    G = Q.shape[0] // K.shape[0]
    Kr = torch.from_numpy(np.repeat(K, G, axis=0))
    Vr = torch.from_numpy(np.repeat(V, G, axis=0))
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), Kr, Vr, is_causal=True).numpy()


def test_gamma_one_equals_dense_causal():
    rng = np.random.default_rng(3)
    S, b = 512, 128
    Q, K, V = rand_layer(rng, S, b, 4, 2, 32, scale=1.5)
    res = oi.index(Q, K, b, 1.0, 0.1)
    rp, ci = res.csr()
    O = oracle.attn.attn(Q, K, V, rp, ci, b)
    ref = _sdpa_causal(Q, K, V)
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)
    for h in range(4):
        dense = brute.dense_masked_attention(Q[h], K[h // 2], V[h // 2], brute.causal_mask(S))
        np.testing.assert_allclose(O[h], dense, rtol=1e-10, atol=1e-12)


def test_sparse_attention_equals_token_masked_dense():
    L = gen.make(gen.CONFIGS["tiny"].with_(S=1024))
    Q, K, V = L.f32("q").astype(np.float64), L.f32("k").astype(np.float64), L.f32("v").astype(np.float64)
    res = oi.index(Q, K, 128, 0.9, 0.1)
    rp, ci = res.csr()
    assert res.density() < 1.0
    O = oracle.attn.attn(Q, K, V, rp, ci, 128)
    for h in range(4):
        mask = brute.token_mask_from_csr(rp, ci, h, 1024, 128)
        ref = brute.dense_masked_attention(Q[h], K[h // 2], V[h // 2], mask)
        np.testing.assert_allclose(O[h], ref, rtol=1e-10, atol=1e-12)


def test_attention_row_subset_matches_full():
    rng = np.random.default_rng(4)
    Q, K, V = rand_layer(rng, 512, 128, 4, 2, 16)
    res = oi.index(Q, K, 128, 0.8, 0.1)
    rp, ci = res.csr()
    full = oracle.attn.attn(Q, K, V, rp, ci, 128)
    part = oracle.attn.attn(Q, K, V, rp, ci, 128, rows=[(3, 2), (0, 0)])
    np.testing.assert_array_equal(part[(3, 2)], full[3, 256:384])
    np.testing.assert_array_equal(part[(0, 0)], full[0, 0:128])


# ------------------------------------------------------------ W8A8
def test_quantiser_round_trip():
    L = gen.make(gen.CONFIGS["tiny"].with_(S=512))
    i8 = L.int8()
    for name in ("q", "k", "v"):
        x = L.f32(name).astype(np.float64)
        q8, s = i8[name + "8"].astype(np.float64), i8["s" + name].astype(np.float64)
        assert np.all(np.abs(x - s[..., None] * q8) <= s[..., None] * (0.5 + 1e-5))
        assert np.all(np.abs(q8).max(axis=-1) == 127)


def test_quantiser_zero_row_and_rounding():
    x = np.zeros((2, 4), dtype=np.float32)
    x[1] = [127.0, -63.5, 0.5, 1.5]
    q, s = gen.quantize_rows(x)
    assert s[0] == 1.0 and np.all(q[0] == 0)
    assert s[1] == 1.0 and list(q[1]) == [127, -64, 0, 2]   # half to even


def test_i8_exact_dot_and_dequant_equivalence():
    rng = np.random.default_rng(5)
    q8 = rng.integers(-127, 128, size=(128, 128), dtype=np.int64)
    k8 = rng.integers(-127, 128, size=(512, 128), dtype=np.int64)
    exact = q8 @ k8.T
    viaf = oi.last_block_scores_i8(q8, np.ones(128), k8, np.ones(512), 1.0)
    np.testing.assert_array_equal(viaf, exact.astype(np.float64))
    # extreme values stay exact
    big = np.full((1, 128), -127)
    assert oi.last_block_scores_i8(big, [1.0], big, [1.0], 1.0)[0, 0] == 128 * 127 * 127


def test_i8_paths_match_dequantised_paths():
    L = gen.make(gen.CONFIGS["tiny"].with_(S=1024))
    i8 = L.int8()
    deq = {n: i8["s" + n].astype(np.float64)[..., None] * i8[n + "8"] for n in ("q", "k", "v")}
    r8 = oi.index_i8(i8["q8"], i8["sq"], i8["k8"], i8["sk"], 128, 0.9, 0.1)
    rd = oi.index(deq["q"], deq["k"], 128, 0.9, 0.1)
    for a, c in zip(r8.heads, rd.heads):
        np.testing.assert_allclose(a.v, c.v, rtol=1e-10, atol=1e-15)
        np.testing.assert_allclose(a.sl, c.sl, rtol=1e-10, atol=1e-15)
        np.testing.assert_allclose(a.p, c.p, rtol=1e-10)
    rp, ci = rd.csr()
    O8 = oracle.attn.attn_i8(i8["q8"], i8["sq"], i8["k8"], i8["sk"], i8["v8"], i8["sv"], rp, ci, 128)
    Od = oracle.attn.attn(deq["q"], deq["k"], deq["v"], rp, ci, 128)
    np.testing.assert_allclose(O8, Od, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------ generator
def test_generator_deterministic_and_shaped():
    a = gen.make("tiny", seed=0)
    b_ = gen.make("tiny", seed=0)
    c = gen.make("tiny", seed=1)
    assert a.q.shape == (4, 2048, 128) and a.k.shape == (2, 2048, 128) and a.q.dtype == np.uint16
    assert np.array_equal(a.q, b_.q) and np.array_equal(a.k, b_.k) and np.array_equal(a.v, b_.v)
    assert not np.array_equal(a.q, c.q)
    assert list(a.planted) == [0, 0, 1, 1]
    assert list(a.spikes[0][:4]) == [0, 1, 2, 3] and len(a.spikes[0]) == 12


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-5, 5, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.bf16_bits_from_f32(x), ref)
    back = gen.f32_from_bf16_bits(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())
