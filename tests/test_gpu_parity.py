"""Parity of the HIP path (through the C ABI) against the float64 oracle.

Index sets must equal the oracle's up to the selection-boundary rule (see
tests/parity.py); attention is compared with both sides on the same CSR:
bf16 max-abs <= 2e-2 and RMS <= 4e-3; W8A8 int32 scores bit-exact and
outputs max-abs <= 2e-2.  Inputs are the seeded planted-v1 layers.
"""
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_flexprefill_amd as fpa
import gen
import oracle
from oracle import index as oi
from tests import parity as P

pytestmark = pytest.mark.gpu

MAXABS, RMS = 2e-2, 4e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fpa.lib()   # a GPU without the built library is a failure, not a skip


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cfg(name="tiny", **kw):
    return gen.CONFIGS[name].with_(**kw) if kw else gen.CONFIGS[name]


# ------------------------------------------------------------------ int8 tile
# (b, Hq, Hkv): the G = 3 shapes run the production workgroup sizes of the headline-like layers
PROBE_SHAPES = [(64, 4, 2), (64, 6, 2), (128, 4, 2), (128, 6, 2), (256, 4, 2), (256, 6, 2)]


@pytest.mark.parametrize("path", [fpa.PROBE_ATTN, fpa.PROBE_STATS], ids=["attn", "stats"])
@pytest.mark.parametrize("b,Hq,Hkv", PROBE_SHAPES, ids=[f"b{b}-G{hq // hk}" for b, hq, hk in PROBE_SHAPES])
def test_probe_qk_i8_exact(b, Hq, Hkv, path):
    """The int32 Q8.K8^T tile through each W8A8 kernel's own staging and tile code equals the
    exact integer product."""
    say(f"probe_qk_i8 path={path} b={b} Hq={Hq} Hkv={Hkv}")
    rng = np.random.default_rng(11)
    S, G = 4 * b, Hq // Hkv
    q8 = rng.integers(-127, 128, size=(Hq, S, 128), dtype=np.int8)
    k8 = rng.integers(-127, 128, size=(Hkv, S, 128), dtype=np.int8)
    q8[1, b:b + 3] = -127
    k8[0, 2 * b:2 * b + 5] = -127
    Q8, K8 = P.dev(q8), P.dev(k8)
    for h, i, j in [(0, 0, 0), (1, 1, 2), (Hq - 1, 3, 1), (Hq - 1, 3, 3)]:
        out = fpa.probe_qk_i8(Q8, K8, b, h, i, j, path=path).cpu().numpy().astype(np.int64)
        ref = k8[h // G, j * b:(j + 1) * b].astype(np.int64) @ q8[h, i * b:(i + 1) * b].astype(np.int64).T
        np.testing.assert_array_equal(out, ref)


# ------------------------------------------------------------------ attention on the oracle's CSR
def _attn_case(c, gamma, i8=False):
    L = gen.make(c)
    Q, K, V = L.f32("q"), L.f32("k"), L.f32("v")
    if i8:
        d = L.int8()
        ref = oi.index_i8(d["q8"], d["sq"], d["k8"], d["sk"], c.b, gamma, c.tau)
    else:
        ref = oi.index(Q, K, c.b, gamma, c.tau)
    rp, ci = ref.csr()
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    idx = fpa.build_jobs(sh, P.dev(rp), P.dev(ci))
    torch.cuda.synchronize()
    assert int(idx.status.item()) == 0
    P.check_jobs(idx, c.G)
    if i8:
        t = P.layer_i8_on_device(L)
        O = fpa.attn_i8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], idx)
        Oref = oracle.attn.attn_i8(d["q8"], d["sq"], d["k8"], d["sk"], d["v8"], d["sv"], rp, ci, c.b)
    else:
        Qd, Kd, Vd = P.layer_on_device(L)
        O = fpa.attn(Qd, Kd, Vd, idx)
        Oref = oracle.attn.attn(Q, K, V, rp, ci, c.b)
    torch.cuda.synchronize()
    mx, rms = P.attn_errors(O, Oref)
    say(f"  maxabs={mx:.3e} rms={rms:.3e} density={ref.density():.3f}")
    assert mx <= MAXABS and rms <= RMS, (mx, rms)


ATTN_CASES = [
    ("tiny", {}, 0.9),
    ("tiny", {}, 1.0),
    ("tiny-N1", dict(S=128, Hq=2, Hkv=1), 0.9),
    ("tiny-G1", dict(Hq=2, Hkv=2), 0.9),
    ("tiny-N37", dict(S=128 * 37), 0.9),
    ("tiny-b256-G4", dict(S=2048, b=256, Hq=8, Hkv=2), 0.95),
    ("tiny-G8", dict(S=1024, Hq=8, Hkv=1), 0.9),
    ("tiny-G5", dict(S=1024, Hq=10, Hkv=2), 0.9),        # 10 waves per job: two spare waves
    ("tiny-G7-b256", dict(S=2048, b=256, Hq=7, Hkv=1), 0.9),
    ("tiny-b64", dict(S=1024, b=64, Hq=4, Hkv=2), 0.9),     # two 64-key blocks per staged chunk
    ("tiny-b64-G3", dict(S=2048, b=64, Hq=6, Hkv=2), 0.9),
    ("tiny-G3", dict(Hq=6, Hkv=2), 0.9),                    # one wave per query tile for all three heads
    ("tiny-G3-b256", dict(S=2048, b=256, Hq=3, Hkv=1), 0.9),
]


@pytest.mark.parametrize("name,kw,gamma", ATTN_CASES, ids=[c[0] + f"-g{c[2]}" for c in ATTN_CASES])
def test_attn_bf16_on_oracle_csr(name, kw, gamma):
    say(f"attn bf16 {name} gamma={gamma}")
    _attn_case(cfg(**kw), gamma)


ATTN_I8_CASES = ATTN_CASES[:4] + ATTN_CASES[5:6] + ATTN_CASES[7:8] + ATTN_CASES[9:11]


@pytest.mark.parametrize("name,kw,gamma", ATTN_I8_CASES, ids=[c[0] + f"-g{c[2]}" for c in ATTN_I8_CASES])
def test_attn_i8_on_oracle_csr(name, kw, gamma):
    say(f"attn i8 {name} gamma={gamma}")
    _attn_case(cfg(**kw), gamma, i8=True)


def test_attn_gamma_one_is_dense_causal():
    say("attn gamma=1 vs dense")
    c = cfg(S=1024)
    L = gen.make(c)
    Q, K, V = L.f32("q"), L.f32("k"), L.f32("v")
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    N = c.N
    rp = np.zeros(c.Hq * N + 1, dtype=np.int32)
    cols = []
    for h in range(c.Hq):
        for i in range(N):
            cols.extend(range(i + 1))
            rp[h * N + i + 1] = len(cols)
    idx = fpa.build_jobs(sh, P.dev(rp), P.dev(np.array(cols, dtype=np.int32)))
    Qd, Kd, Vd = P.layer_on_device(L)
    O = fpa.attn(Qd, Kd, Vd, idx)
    from oracle import brute
    ref = np.stack([brute.dense_masked_attention(Q[h], K[h // c.G], V[h // c.G], brute.causal_mask(c.S))
                    for h in range(c.Hq)])
    mx, rms = P.attn_errors(O, ref)
    assert mx <= MAXABS and rms <= RMS, (mx, rms)


def _irregular_csr(c, seed):
    """Random causal rows: about 15% empty, 25% without their diagonal block, the rest random
    subsets that keep it; entry counts odd and even."""
    rng = np.random.default_rng(seed)
    N = c.N
    rp = np.zeros(c.Hq * N + 1, dtype=np.int32)
    cols, empty = [], []
    for h in range(c.Hq):
        for i in range(N):
            u = rng.random()
            if u < 0.15:
                sel = []
            elif u < 0.40 and i > 0:
                sel = sorted(rng.choice(i, size=int(rng.integers(1, i + 1)), replace=False).tolist())
            else:
                sel = sorted(set(rng.choice(i + 1, size=int(rng.integers(1, i + 2)), replace=False).tolist()) | {i})
            if not sel:
                empty.append((h, i))
            cols.extend(sel)
            rp[h * N + i + 1] = len(cols)
    return rp, np.array(cols, dtype=np.int32), empty


@pytest.mark.parametrize("i8", [False, True], ids=["bf16", "i8"])
@pytest.mark.parametrize("b,Hq,Hkv", [(128, 6, 2), (64, 6, 2), (256, 4, 2)], ids=["b128-G3", "b64-G3", "b256-G2"])
def test_attn_on_irregular_csr(b, Hq, Hkv, i8):
    """A caller's CSR through fp_build_jobs with empty rows (also beside heads of the same group
    that have entries), rows without their diagonal block and odd entry counts (single-block
    chunks at b = 64): rows with entries match the oracle, and an empty row's output is zero,
    as fp_attn defines it."""
    say(f"attn on an irregular CSR b={b} Hq={Hq} Hkv={Hkv} {'i8' if i8 else 'bf16'}")
    c = cfg(S=2048, b=b, Hq=Hq, Hkv=Hkv)
    L = gen.make(c, seed=5)
    rp, ci, empty = _irregular_csr(c, 7)
    assert empty
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    idx = fpa.build_jobs(sh, P.dev(rp), P.dev(ci))
    torch.cuda.synchronize()
    assert int(idx.status.item()) == 0
    P.check_jobs(idx, c.G)
    rows = [(h, i) for h in range(c.Hq) for i in range(c.N) if (h, i) not in set(empty)]
    if i8:
        t = P.layer_i8_on_device(L)
        O = fpa.attn_i8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], idx)
        d = L.int8()
        res = oracle.attn.attn_i8(d["q8"], d["sq"], d["k8"], d["sk"], d["v8"], d["sv"], rp, ci, c.b, rows=rows)
    else:
        Qd, Kd, Vd = P.layer_on_device(L)
        O = fpa.attn(Qd, Kd, Vd, idx)
        Q, K, V = L.f32("q"), L.f32("k"), L.f32("v")
        res = oracle.attn.attn(Q, K, V, rp, ci, c.b, rows=rows)
    torch.cuda.synchronize()
    Oref = np.zeros((c.Hq, c.S, c.d))
    for (h, i), o in res.items():
        Oref[h, i * c.b:(i + 1) * c.b] = o
    Of = O.float().cpu()
    for h, i in empty:
        assert torch.count_nonzero(Of[h, i * c.b:(i + 1) * c.b]) == 0, (h, i)
    mx, rms = P.attn_errors(O, Oref)
    say(f"  maxabs={mx:.3e} rms={rms:.3e}, {len(empty)} empty rows")
    assert mx <= MAXABS and rms <= RMS, (mx, rms)


@pytest.mark.parametrize("b,Hq,Hkv", [(128, 2, 2), (128, 4, 2), (128, 6, 2), (64, 4, 2), (64, 6, 2)],
                         ids=["G1", "G2", "G3", "b64-G2", "b64-G3"])
def test_attn_score_spike(b, Hq, Hkv):
    """Keys of block 0 scaled by 3: rows that meet them after other keys see scores 80 to 140
    (log2 units) above everything before, far beyond the headroom the kernel allows before it
    rescales O to a raised reference maximum; dense causal index, oracle attention.  With b = 64
    and two or three heads per group the chunks hold one 64-key block."""
    say(f"attn score spike b={b} Hq={Hq} Hkv={Hkv}")
    c = cfg(S=1024, b=b, Hq=Hq, Hkv=Hkv)
    L = gen.make(c)
    kf = L.f32("k")
    kf[:, :c.b] *= 3.0
    kbits = gen.bf16_bits_from_f32(kf)
    K = gen.f32_from_bf16_bits(kbits)
    Q, V = L.f32("q"), L.f32("v")
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    N = c.N
    rp = np.zeros(c.Hq * N + 1, dtype=np.int32)
    cols = []
    for h in range(c.Hq):
        for i in range(N):
            cols.extend(range(i + 1))
            rp[h * N + i + 1] = len(cols)
    idx = fpa.build_jobs(sh, P.dev(rp), P.dev(np.array(cols, dtype=np.int32)))
    O = fpa.attn(P.dev_bf16(L.q), P.dev_bf16(kbits), P.dev_bf16(L.v), idx)
    from oracle import brute
    ref = np.stack([brute.dense_masked_attention(Q[h], K[h // c.G], V[h // c.G], brute.causal_mask(c.S))
                    for h in range(c.Hq)])
    torch.cuda.synchronize()
    mx, rms = P.attn_errors(O, ref)
    say(f"  maxabs={mx:.3e} rms={rms:.3e}")
    assert np.isfinite(mx) and mx <= MAXABS and rms <= RMS, (mx, rms)


# ------------------------------------------------------------------ index generation
INDEX_CASES = [
    ("tiny", {}, 0.9),
    ("tiny-g1", {}, 1.0),
    ("tiny-g0.5", {}, 0.5),
    ("tiny-N1", dict(S=128, Hq=2, Hkv=1), 0.9),
    ("tiny-G1", dict(Hq=2, Hkv=2), 0.9),
    ("tiny-N37", dict(S=128 * 37), 0.9),
    ("tiny-b256-G4", dict(S=4096, b=256, Hq=8, Hkv=2, vs_frac=0.5), 0.95),
    ("tiny-b256-G8", dict(S=4096, b=256, Hq=8, Hkv=1), 0.9),       # 64 query tiles: four per wave
    ("tiny-G8", dict(S=2048, Hq=8, Hkv=1), 0.9),
    ("tiny-G16", dict(S=1024, Hq=16, Hkv=1), 0.9),
    ("tiny-N70", dict(S=128 * 70, Hq=4, Hkv=2), 0.9),
    ("tiny-G5", dict(S=2048, Hq=10, Hkv=2), 0.9),
    ("tiny-b64", dict(S=2048, b=64, Hq=4, Hkv=2), 0.9),
    ("tiny-b64-G3", dict(S=4096, b=64, Hq=6, Hkv=2), 0.9),
    # N = 2560 > 2048: query blocks pooled through the workspace (two launches), rows longer
    # than 1024 blocks selected from LDS; one vertical-slash and one query-aware group
    ("N2560-b64", dict(S=64 * 2560, b=64, Hq=2, Hkv=2), 0.9),
]
# the largest block counts: N = 4608 (> 4096: two query-aware rows per workgroup) and the
# supported maximum N = 8192 (one vertical-slash head)
LARGE_N_CASES = [
    ("N4608-b64", dict(S=64 * 4608, b=64, Hq=2, Hkv=2), 0.9),
    ("N8192-b64-vs", dict(S=64 * 8192, b=64, Hq=1, Hkv=1, vs_frac=1.0), 0.9),
]


def _index_case(c, gamma, i8=False):
    L = gen.make(c)
    if i8:
        d = L.int8()
        ref = oi.index_i8(d["q8"], d["sq"], d["k8"], d["sk"], c.b, gamma, c.tau)
        t = P.layer_i8_on_device(L)
        idx = fpa.index_i8(t["q8"], t["sq"], t["k8"], t["sk"], c.b, gamma, c.tau, stats=True)
    else:
        ref = oi.index(L.f32("q"), L.f32("k"), c.b, gamma, c.tau)
        Qd, Kd, _ = P.layer_on_device(L)
        idx = fpa.index(Qd, Kd, c.b, gamma, c.tau, stats=True)
    torch.cuda.synchronize()
    s = P.compare_index(idx, ref, gamma, c.tau)
    pat = idx.pattern.cpu().numpy()
    mism = {h: int(pat[h]) for h in range(c.Hq) if pat[h] != ref.heads[h].pattern}
    if mism:   # tie at tau: compare against the oracle forced to the device's pattern
        if i8:
            ref2 = oi.index_i8(d["q8"], d["sq"], d["k8"], d["sk"], c.b, gamma, c.tau, force_pattern=mism)
        else:
            ref2 = oi.index(L.f32("q"), L.f32("k"), c.b, gamma, c.tau, force_pattern=mism)
        P.compare_index(idx, ref2, gamma, c.tau)
    P.check_jobs(idx, c.G)
    say(f"  {s} density gpu={idx.density():.4f} oracle={ref.density():.4f} jsd={np.round(idx.jsd.cpu().numpy(), 4)}")
    return idx, ref


@pytest.mark.parametrize("name,kw,gamma", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_index_bf16(name, kw, gamma):
    say(f"index bf16 {name} gamma={gamma}")
    _index_case(cfg(**kw), gamma)


INDEX_I8_CASES = INDEX_CASES[:2] + INDEX_CASES[4:7] + INDEX_CASES[11:14]


@pytest.mark.parametrize("name,kw,gamma", INDEX_I8_CASES, ids=[c[0] for c in INDEX_I8_CASES])
def test_index_i8(name, kw, gamma):
    say(f"index i8 {name} gamma={gamma}")
    _index_case(cfg(**kw), gamma, i8=True)


@pytest.mark.parametrize("name,kw,gamma", LARGE_N_CASES, ids=[c[0] for c in LARGE_N_CASES])
def test_index_and_attn_large_n(name, kw, gamma):
    """Index parity at the largest block counts, then attention on sampled query blocks
    (the first, the last and six others) against the oracle on the device's CSR."""
    say(f"index + attn bf16 {name} gamma={gamma}")
    c = cfg(**kw)
    idx, _ = _index_case(c, gamma)
    L = gen.make(c)
    Qd, Kd, Vd = P.layer_on_device(L)
    O = fpa.attn(Qd, Kd, Vd, idx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = [(h, i) for h in range(c.Hq) for i in sorted({0, c.N - 1, *rng.integers(1, c.N - 1, 6).tolist()})]
    rp, ci = P.gpu_rows(idx)
    ref = oracle.attn.attn(L.f32("q"), L.f32("k"), L.f32("v"), rp, ci, c.b, rows=rows)
    Oh = O.float().cpu().numpy()
    worst, sq, cnt = 0.0, 0.0, 0
    for (h, i), ref_o in ref.items():
        dlt = Oh[h, i * c.b:(i + 1) * c.b].astype(np.float64) - ref_o
        worst = max(worst, float(np.abs(dlt).max()))
        sq += float((dlt * dlt).sum())
        cnt += dlt.size
    rms = (sq / cnt) ** 0.5
    say(f"  attention on {len(rows)} sampled query blocks: maxabs {worst:.3e} rms {rms:.3e}")
    assert worst <= MAXABS and rms <= RMS


def test_ragged_batch():
    """fp_index_batch / fp_attn_batch on three sequences of different lengths packed one
    after another: every sequence's index and attention against the oracle."""
    say("ragged batch: S = 1024, 384, 2048 (b = 128, Hq = 4, Hkv = 2)")
    lens = [1024, 384, 2048]
    cs = [cfg(S=S) for S in lens]
    Ls = [gen.make(c) for c in cs]
    dev = "cuda"
    pack = lambda name: torch.cat([P.dev_bf16(getattr(L, name), dev).reshape(-1) for L in Ls])
    Q, K, V = pack("q"), pack("k"), pack("v")
    c0 = cs[0]
    idxs = fpa.index_batch(Q, K, lens, c0.b, c0.Hq, c0.Hkv, c0.gamma, c0.tau)
    O = fpa.attn_batch(Q, K, V, lens, idxs)
    torch.cuda.synchronize()
    Os = fpa.unpack(O, lens, c0.Hq)
    for c, L, idx, Oc in zip(cs, Ls, idxs, Os):
        assert int(idx.status.item()) == 0
        ref = oi.index(L.f32("q"), L.f32("k"), c.b, c.gamma, c.tau)
        P.compare_index(idx, ref, c.gamma, c.tau)
        P.check_jobs(idx, c.G)
        rp, ci = P.gpu_rows(idx)
        mx, rms = P.attn_errors(Oc, oracle.attn.attn(L.f32("q"), L.f32("k"), L.f32("v"), rp, ci, c.b))
        say(f"  S={c.S}: density {idx.density():.3f}, attention maxabs {mx:.2e} rms {rms:.2e}")
        assert mx <= MAXABS and rms <= RMS


def test_ragged_batch_i8():
    """fp_index_i8_batch / fp_attn_i8_batch on three W8A8 sequences of different lengths packed
    one after another (int8 tensors and fp32 scales alike): index and attention per sequence
    against the oracle."""
    say("ragged batch i8: S = 768, 2048, 256 (b = 128, Hq = 6, Hkv = 2)")
    lens = [768, 2048, 256]
    cs = [cfg(S=S, Hq=6, Hkv=2) for S in lens]
    Ls = [gen.make(c) for c in cs]
    ts = [P.layer_i8_on_device(L) for L in Ls]
    pack = lambda name: torch.cat([t[name].reshape(-1) for t in ts])
    Q8, sQ, K8, sK, V8, sV = (pack(n) for n in ("q8", "sq", "k8", "sk", "v8", "sv"))
    c0 = cs[0]
    idxs = fpa.index_i8_batch(Q8, sQ, K8, sK, lens, c0.b, c0.Hq, c0.Hkv, c0.gamma, c0.tau)
    O = fpa.attn_i8_batch(Q8, sQ, K8, sK, V8, sV, lens, idxs)
    torch.cuda.synchronize()
    Os = fpa.unpack(O, lens, c0.Hq)
    for c, L, idx, Oc in zip(cs, Ls, idxs, Os):
        assert int(idx.status.item()) == 0
        d = L.int8()
        ref = oi.index_i8(d["q8"], d["sq"], d["k8"], d["sk"], c.b, c.gamma, c.tau)
        P.compare_index(idx, ref, c.gamma, c.tau)
        P.check_jobs(idx, c.G)
        rp, ci = P.gpu_rows(idx)
        Oref = oracle.attn.attn_i8(d["q8"], d["sq"], d["k8"], d["sk"], d["v8"], d["sv"], rp, ci, c.b)
        mx, rms = P.attn_errors(Oc, Oref)
        say(f"  S={c.S}: density {idx.density():.3f}, attention maxabs {mx:.2e} rms {rms:.2e}")
        assert mx <= MAXABS and rms <= RMS


INDEX_FIELDS = ("row_ptr", "col_idx", "job_ptr", "job_blk", "job_mask", "job_order", "pattern", "jsd", "stats",
                "status")


def _index_equal(a, b, upto=None):
    """Every field of two Index results equal (col_idx / job arrays up to their written length)."""
    nnz = min(a.nnz, a.col_idx.numel()) if upto is None else upto
    njob = min(int(a.job_ptr[-1].item()), a.job_blk.numel())
    assert nnz == min(b.nnz, b.col_idx.numel()) and njob == min(int(b.job_ptr[-1].item()), b.job_blk.numel())
    lens = {"col_idx": nnz, "job_blk": njob, "job_mask": njob}
    for f in INDEX_FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        if x is None and y is None:
            continue
        n = lens.get(f, x.numel())
        assert torch.equal(x.flatten()[:n], y.flatten()[:n]), f


@pytest.mark.parametrize("i8", [False, True], ids=["bf16", "i8"])
def test_batch_runs_of_equal_lengths_match_single_calls(i8):
    """Runs of equal-length sequences run as one call with their heads side by side; every
    sequence's index (statistics included) and attention output equal those of a call of its own,
    bit for bit, and so does attention over indices from single calls."""
    lens = [1024, 1024, 1024, 384, 2048, 2048, 256]
    say(f"batch with runs of equal lengths vs single calls ({'i8' if i8 else 'bf16'}): S = {lens}")
    cs = [cfg(S=S, Hq=6, Hkv=2) for S in lens]
    Ls = [gen.make(c, seed=11 + k) for k, c in enumerate(cs)]
    c0 = cs[0]
    singles, Os = [], []
    if i8:
        ts = [P.layer_i8_on_device(L) for L in Ls]
        for c, t in zip(cs, ts):
            ix = fpa.index_i8(t["q8"], t["sq"], t["k8"], t["sk"], c.b, c.gamma, c.tau, stats=True)
            singles.append(ix)
            Os.append(fpa.attn_i8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], ix))
        pack = lambda name: torch.cat([t[name].reshape(-1) for t in ts])
        Q8, sQ, K8, sK, V8, sV = (pack(n) for n in ("q8", "sq", "k8", "sk", "v8", "sv"))
        idxs = fpa.index_i8_batch(Q8, sQ, K8, sK, lens, c0.b, c0.Hq, c0.Hkv, c0.gamma, c0.tau, stats=True)
        O = fpa.attn_i8_batch(Q8, sQ, K8, sK, V8, sV, lens, idxs)
        O2 = fpa.attn_i8_batch(Q8, sQ, K8, sK, V8, sV, lens, singles)
    else:
        for c, L in zip(cs, Ls):
            Qd, Kd, Vd = P.layer_on_device(L)
            ix = fpa.index(Qd, Kd, c.b, c.gamma, c.tau, stats=True)
            singles.append(ix)
            Os.append(fpa.attn(Qd, Kd, Vd, ix))
        pack = lambda name: torch.cat([P.dev_bf16(getattr(L, name), "cuda").reshape(-1) for L in Ls])
        Q, K, V = pack("q"), pack("k"), pack("v")
        idxs = fpa.index_batch(Q, K, lens, c0.b, c0.Hq, c0.Hkv, c0.gamma, c0.tau, stats=True)
        O = fpa.attn_batch(Q, K, V, lens, idxs)
        O2 = fpa.attn_batch(Q, K, V, lens, singles)
    torch.cuda.synchronize()
    for s, (a, b_) in enumerate(zip(idxs, singles)):
        _index_equal(a, b_)
    for Ob in (O, O2):
        for s, (x, y) in enumerate(zip(fpa.unpack(Ob, lens, c0.Hq), Os)):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), s


def test_batch_long_run_matches_single_calls():
    """A run of 30 equal-length sequences (its outputs split, and its job lists merged, by
    launches of 24 and 6 sequences) and a run of 3: every index and output equals a call of its
    own, bit for bit."""
    lens = [256] * 30 + [512] * 3
    say(f"batch with a run of 30 sequences, S = 256, then 3 of S = 512")
    cs = [cfg(S=S, Hq=4, Hkv=2) for S in lens]
    Ls = [gen.make(c, seed=40 + k) for k, c in enumerate(cs)]
    c0 = cs[0]
    singles, Os = [], []
    for c, L in zip(cs, Ls):
        Qd, Kd, Vd = P.layer_on_device(L)
        ix = fpa.index(Qd, Kd, c.b, c.gamma, c.tau)
        singles.append(ix)
        Os.append(fpa.attn(Qd, Kd, Vd, ix))
    pack = lambda name: torch.cat([P.dev_bf16(getattr(L, name), "cuda").reshape(-1) for L in Ls])
    Q, K, V = pack("q"), pack("k"), pack("v")
    idxs = fpa.index_batch(Q, K, lens, c0.b, c0.Hq, c0.Hkv, c0.gamma, c0.tau)
    O = fpa.attn_batch(Q, K, V, lens, idxs)
    O2 = fpa.attn_batch(Q, K, V, lens, singles)
    torch.cuda.synchronize()
    for a, b_ in zip(idxs, singles):
        _index_equal(a, b_)
    for Ob in (O, O2):
        for s_, (x, y) in enumerate(zip(fpa.unpack(Ob, lens, c0.Hq), Os)):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), s_


@pytest.mark.parametrize("b,Hq,Hkv,lens", [
    (64, 4, 2, [16384, 16384, 2048]),           # a run at the folding limit of 256 key blocks
    (64, 6, 2, [16448, 16448, 1024, 1024]),     # 257 blocks go one at a time, then a run of two
    (256, 8, 8, [4096, 4096, 4096]),            # G = 1
    (128, 16, 1, [2048, 2048]),                 # G = 16, G * b = 2048
], ids=["b64-limit", "b64-over-limit", "b256-G1", "b128-G16"])
def test_batch_runs_at_other_shapes_match_single_calls(b, Hq, Hkv, lens):
    """Folded runs at 64- and 256-token blocks, at the 256-block folding limit and one block past
    it, and with one and sixteen query heads per KV head: every index and attention output equals
    a call of its own, bit for bit."""
    say(f"batch vs single calls: b = {b}, Hq = {Hq}, Hkv = {Hkv}, S = {lens}")
    cs = [cfg(S=S, b=b, Hq=Hq, Hkv=Hkv) for S in lens]
    Ls = [gen.make(c, seed=70 + k) for k, c in enumerate(cs)]
    c0 = cs[0]
    singles, Os = [], []
    for c, L in zip(cs, Ls):
        Qd, Kd, Vd = P.layer_on_device(L)
        ix = fpa.index(Qd, Kd, c.b, c.gamma, c.tau, stats=True)
        singles.append(ix)
        Os.append(fpa.attn(Qd, Kd, Vd, ix))
    pack = lambda name: torch.cat([P.dev_bf16(getattr(L, name), "cuda").reshape(-1) for L in Ls])
    Q, K, V = pack("q"), pack("k"), pack("v")
    idxs = fpa.index_batch(Q, K, lens, b, Hq, Hkv, c0.gamma, c0.tau, stats=True)
    O = fpa.attn_batch(Q, K, V, lens, idxs)
    O2 = fpa.attn_batch(Q, K, V, lens, singles)
    torch.cuda.synchronize()
    for a, b_ in zip(idxs, singles):
        assert int(a.status.item()) == 0
        _index_equal(a, b_)
    for Ob in (O, O2):
        for s_, (x, y) in enumerate(zip(fpa.unpack(Ob, lens, Hq), Os)):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), s_


def test_batch_run_keeps_each_sequences_capacity():
    """One sequence of a run of equal lengths with a column capacity too small for its rows: its
    status word reports the overflow and its outputs equal those of a call of its own with that
    capacity; the others are complete."""
    lens = [1024] * 3
    say("batch run with one small capacity")
    cs = [cfg(S=S, Hq=4, Hkv=2) for S in lens]
    Ls = [gen.make(c, seed=23 + k) for k, c in enumerate(cs)]
    c0 = cs[0]
    sh = fpa.shape_of(1024, c0.b, c0.Hq, c0.Hkv)
    small = c0.Hq * c0.N + 5
    outs = [fpa.Index.empty(sh, "cuda", col_cap=(small if k == 1 else None)) for k in range(3)]
    pack = lambda name: torch.cat([P.dev_bf16(getattr(L, name), "cuda").reshape(-1) for L in Ls])
    idxs = fpa.index_batch(pack("q"), pack("k"), lens, c0.b, c0.Hq, c0.Hkv, c0.gamma, c0.tau, outs=outs)
    ref = []
    for k, L in enumerate(Ls):
        Qd, Kd, _ = P.layer_on_device(L)
        out = fpa.Index.empty(sh, "cuda", col_cap=(small if k == 1 else None))
        ref.append(fpa.index(Qd, Kd, c0.b, c0.gamma, c0.tau, out=out))
    torch.cuda.synchronize()
    assert [int(ix.status.item()) for ix in idxs] == [0, fpa.FP_STATUS_CSR_OVERFLOW, 0]
    for a, b_ in zip(idxs, ref):
        _index_equal(a, b_)


def test_index_deterministic_and_end_to_end():
    say("index + attn determinism, tiny")
    c = cfg()
    L = gen.make(c)
    Qd, Kd, Vd = P.layer_on_device(L)
    a = fpa.index(Qd, Kd, c.b, c.gamma, c.tau, stats=True)
    b_ = fpa.index(Qd, Kd, c.b, c.gamma, c.tau, stats=True)
    Oa = fpa.attn(Qd, Kd, Vd, a)
    Ob = fpa.attn(Qd, Kd, Vd, b_)
    torch.cuda.synchronize()
    nnz, njob = a.nnz, int(a.job_ptr[-1].item())
    lens = {"col_idx": nnz, "job_blk": njob, "job_mask": njob}   # capacity tails are never written
    for f in ("row_ptr", "col_idx", "job_ptr", "job_blk", "job_mask", "job_order", "pattern", "jsd", "stats"):
        x, y = getattr(a, f), getattr(b_, f)
        n = lens.get(f, x.numel())
        assert torch.equal(x.flatten()[:n], y.flatten()[:n]), f
    assert torch.equal(Oa.view(torch.int16), Ob.view(torch.int16))
    # the device CSR drives attention to the oracle's output on that CSR
    rp, ci = P.gpu_rows(a)
    Oref = oracle.attn.attn(L.f32("q"), L.f32("k"), L.f32("v"), rp, ci, c.b)
    mx, rms = P.attn_errors(Oa, Oref)
    assert mx <= MAXABS and rms <= RMS


@pytest.mark.parametrize("i8", [False, True], ids=["bf16", "i8"])
def test_attn_repeated_calls_share_one_workspace(i8):
    """The persistent attention kernel keeps its unit table and claim counter in the workspace.
    Calls that reuse one workspace, with a call of another shape (b = 64) in between, must give
    bit-identical outputs, each equal to the oracle's within the attention tolerance."""
    say(f"attn repeated calls on one workspace, {'i8' if i8 else 'bf16'}")
    ca, cb = cfg(S=4096, Hq=6, Hkv=2), cfg(S=2048, b=64, Hq=6, Hkv=2)
    sa, sb = fpa.shape_of(ca.S, ca.b, ca.Hq, ca.Hkv), fpa.shape_of(cb.S, cb.b, cb.Hq, cb.Hkv)
    ws = fpa.Workspace(sa if fpa.workspace_bytes(sa) >= fpa.workspace_bytes(sb) else sb, "cuda")
    La, Lb = gen.make(ca), gen.make(cb)

    def run(c, L):
        if i8:
            t = P.layer_i8_on_device(L)
            idx = fpa.index_i8(t["q8"], t["sq"], t["k8"], t["sk"], c.b, c.gamma, c.tau, ws=ws)
            return fpa.attn_i8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], idx, ws=ws), idx
        Qd, Kd, Vd = P.layer_on_device(L)
        idx = fpa.index(Qd, Kd, c.b, c.gamma, c.tau, ws=ws)
        return fpa.attn(Qd, Kd, Vd, idx, ws=ws), idx

    O1, idx = run(ca, La)
    Ob, _ = run(cb, Lb)
    O2, _ = run(ca, La)
    O3, _ = run(ca, La)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(O1.view(torch.int16), O3.view(torch.int16))
    rp, ci = P.gpu_rows(idx)
    if i8:
        d = La.int8()
        Oref = oracle.attn.attn_i8(d["q8"], d["sq"], d["k8"], d["sk"], d["v8"], d["sv"], rp, ci, ca.b)
    else:
        Oref = oracle.attn.attn(La.f32("q"), La.f32("k"), La.f32("v"), rp, ci, ca.b)
    mx, rms = P.attn_errors(O1, Oref)
    assert mx <= MAXABS and rms <= RMS, (mx, rms)


def test_capacity_overflow_sets_status():
    say("capacity overflow status")
    c = cfg()
    L = gen.make(c)
    Qd, Kd, _ = P.layer_on_device(L)
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    out = fpa.Index.empty(sh, Qd.device, col_cap=c.Hq * c.N + 5, job_cap=c.Hkv * c.N + 3)
    fpa.index(Qd, Kd, c.b, 1.0, c.tau, out=out)
    torch.cuda.synchronize()
    st = int(out.status.item())
    assert st & fpa.FP_STATUS_CSR_OVERFLOW
    rp = out.row_ptr.cpu().numpy()
    assert rp[-1] == c.Hq * c.N + 5 and np.all(np.diff(rp) >= 0)


# ------------------------------------------------------------------ head-pattern sharing
SHARED_CASES = [("tiny-G3", dict(S=2048, Hq=6, Hkv=2)), ("tiny-G4-b256", dict(S=4096, b=256, Hq=8, Hkv=2)),
                ("tiny-b64-G3", dict(S=2048, b=64, Hq=6, Hkv=2))]


@pytest.mark.parametrize("name,kw", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
@pytest.mark.parametrize("i8", [False, True], ids=["bf16", "i8"])
def test_index_shared(name, kw, i8):
    """fp_index_shared: each head's rows are exactly the union of the plain rows of its group's heads
    with the same pattern (the plain rows being oracle-checked); the oracle's shared rows agree
    under the boundary rule; attention on the shared index matches the oracle on that CSR."""
    say(f"index shared {'i8' if i8 else 'bf16'} {name}")
    c = cfg(**kw)
    idx, ref = _index_case(c, c.gamma, i8=i8)
    L = gen.make(c)
    if i8:
        t = P.layer_i8_on_device(L)
        sh = fpa.index_shared(t["q8"], t["k8"], c.b, c.gamma, c.tau, sQ=t["sq"], sK=t["sk"])
    else:
        Qd, Kd, Vd = P.layer_on_device(L)
        sh = fpa.index_shared(Qd, Kd, c.b, c.gamma, c.tau)
    torch.cuda.synchronize()
    assert int(sh.status.item()) == 0
    pat = idx.pattern.cpu().numpy()
    assert np.array_equal(pat, sh.pattern.cpu().numpy())
    rp, ci = P.gpu_rows(idx)
    rs, cs = P.gpu_rows(sh)
    N, G = c.N, c.G
    for h in range(c.Hq):
        peers = [p for p in range(h // G * G, h // G * G + G) if pat[p] == pat[h]]
        for i in range(N):
            want = sorted(set().union(*(set(ci[rp[p * N + i]:rp[p * N + i + 1]].tolist()) for p in peers)))
            assert cs[rs[h * N + i]:rs[h * N + i + 1]].tolist() == want, (h, i)
    P.check_jobs(sh, G)
    # the oracle's shared rows, where no member's selection sits at an ambiguous boundary
    shared_ref = oi.share_rows(ref)
    same = sum(np.array_equal(cs[rs[h * N + i]:rs[h * N + i + 1]], shared_ref.heads[h].rows[i])
               for h in range(c.Hq) for i in range(N))
    say(f"  shared rows equal to the oracle's: {same} / {c.Hq * N}; density {sh.density():.3f} vs {idx.density():.3f}")
    summ = P.compare_index(idx, ref, c.gamma, c.tau)
    if summ["boundary_rows"] == 0 and summ["pattern_mismatch"] == 0:
        assert same == c.Hq * N
    assert sh.density() >= idx.density()
    if i8:
        d = L.int8()
        O = fpa.attn_i8(t["q8"], t["sq"], t["k8"], t["sk"], t["v8"], t["sv"], sh)
        Oref = oracle.attn.attn_i8(d["q8"], d["sq"], d["k8"], d["sk"], d["v8"], d["sv"], rs, cs, c.b)
    else:
        O = fpa.attn(Qd, Kd, Vd, sh)
        Oref = oracle.attn.attn(L.f32("q"), L.f32("k"), L.f32("v"), rs, cs, c.b)
    mx, rms = P.attn_errors(O, Oref)
    say(f"  attention on the shared index: maxabs {mx:.2e} rms {rms:.2e}")
    assert mx <= MAXABS and rms <= RMS


def test_block_uses_match_oracle():
    """fp_block_uses (consumer counts per key block) against the oracle's counts on the device CSR."""
    say("block uses, tiny G3 and b256")
    for kw in (dict(S=2048, Hq=6, Hkv=2), dict(S=4096, b=256, Hq=8, Hkv=2)):
        c = cfg(**kw)
        L = gen.make(c)
        Qd, Kd, _ = P.layer_on_device(L)
        idx = fpa.index(Qd, Kd, c.b, c.gamma, c.tau)
        uses, head_uses = fpa.block_uses(idx)
        torch.cuda.synchronize()
        rp, ci = P.gpu_rows(idx)
        N = c.N
        heads = [oi.HeadIndex(v=None, sl=None, p=None, D=0.0, pattern=0,
                              rows=[ci[rp[h * N + i]:rp[h * N + i + 1]] for i in range(N)]) for h in range(c.Hq)]
        want_u, want_h = oi.block_uses(oi.IndexResult(S=c.S, b=c.b, Hq=c.Hq, Hkv=c.Hkv, heads=heads))
        np.testing.assert_array_equal(uses.cpu().numpy(), want_u)
        np.testing.assert_array_equal(head_uses.cpu().numpy(), want_h)


# ------------------------------------------------------------------ split-KV schedule
SPLIT_CASES = [("tiny-all-2", {}, 1 << 20, 2), ("tiny-4-3", {}, 4, 3), ("tiny-b256-G4-5", dict(S=2048, b=256, Hq=8, Hkv=2), 3, 5),
               ("tiny-G8-all-4", dict(S=1024, Hq=8, Hkv=1), 1 << 20, 4), ("tiny-N37-16-2", dict(S=128 * 37), 16, 2),
               ("tiny-g1-all-3", dict(gamma=1.0), 1 << 20, 3)]


@pytest.mark.parametrize("name,kw,nsplit,nseg", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_attn_split_on_oracle_csr(name, kw, nsplit, nseg):
    """fp_attn_split (split-KV segments merged by the keyed combine) against the oracle on the oracle's
    CSR, and against fp_attn on the same index."""
    say(f"attn split {name}: nsplit={nsplit} nseg={nseg}")
    c = cfg(**kw)
    L = gen.make(c)
    Q, K, V = L.f32("q"), L.f32("k"), L.f32("v")
    ref = oi.index(Q, K, c.b, c.gamma, c.tau)
    rp, ci = ref.csr()
    idx = fpa.build_jobs(fpa.shape_of(c.S, c.b, c.Hq, c.Hkv), P.dev(rp), P.dev(ci))
    Qd, Kd, Vd = P.layer_on_device(L)
    Os = fpa.attn_split(Qd, Kd, Vd, idx, nsplit, nseg)
    Op = fpa.attn(Qd, Kd, Vd, idx)
    torch.cuda.synchronize()
    Oref = oracle.attn.attn(Q, K, V, rp, ci, c.b)
    mx, rms = P.attn_errors(Os, Oref)
    dmx = float((Os.float() - Op.float()).abs().max().item())
    say(f"  maxabs={mx:.3e} rms={rms:.3e}; vs fp_attn maxabs {dmx:.3e}")
    assert mx <= MAXABS and rms <= RMS, (mx, rms)
    assert dmx <= MAXABS
