"""Host-side checks of bench.py (no GPU): the one-GPU guard, the arithmetic that turns
rocprofv3 counter passes into HBM bytes per attention launch, the rule that a traffic
record goes stale once the attention source changes, and the index-stage byte count."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counters(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f'"{name}",X,{value}\n')


def test_traffic_from_counter_passes(tmp_path, monkeypatch):
    kib = bench.COPY_BYTES / 1024.0
    # the copy reads half its bytes in FETCH_SIZE and writes all of them in WRITE_SIZE
    _counters(tmp_path / "copy_FETCH_SIZE_counter_collection.csv", [("__amd_rocclr_copyBuffer", kib / 2)] * 3)
    _counters(tmp_path / "copy_WRITE_SIZE_counter_collection.csv", [("__amd_rocclr_copyBuffer", kib)] * 3)
    attn = "void fp::(anonymous namespace)::k_attn_dl<768, false>(fp::AttnArgs, int)"
    st = "void fp::(anonymous namespace)::k_ig_stream<128, 768, 1, false>(fp::(anonymous namespace)::StreamArgs)"
    qa = "void fp::(anonymous namespace)::k_qa_rows16<128, false, false, false>(fp::(anonymous namespace)::QaArgs)"
    sort = "fp::(anonymous namespace)::k_scan_sort(fp::(anonymous namespace)::ScanJob, int)"
    other = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<int> >(int)"
    _counters(tmp_path / "bench_FETCH_SIZE_counter_collection.csv",
              [(attn, 1000.0), (attn, 1200.0), (st, 5.0), (st, 7.0), (qa, 10.0), (sort, 1.0), (other, 99.0)])
    _counters(tmp_path / "bench_WRITE_SIZE_counter_collection.csv",
              [(attn, 300.0), (attn, 300.0), (st, 2.0), (qa, 4.0), (sort, 0.5), (other, 99.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda name: str(out))
    bench.traffic_from(str(tmp_path), "3b-128k")
    rec = json.load(open(out))
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    # per launch: the mean over the kernel's dispatches, each counter scaled by its factor
    assert rec["bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2.0 + 300.0 * 1024 * 1.0)
    assert bench.measured_traffic("3b-128k") == pytest.approx(rec["bytes_per_launch"])
    # per index call: each index kernel's mean per dispatch, summed over the kernels (not the fill)
    assert sorted(rec["index"]["kernels"]) == sorted([st, qa, sort])
    assert rec["index"]["bytes_per_call"] == pytest.approx((6.0 + 10.0 + 1.0) * 1024 * 2.0 + (2.0 + 4.0 + 0.5) * 1024)
    assert bench.measured_index_traffic("3b-128k") == pytest.approx(rec["index"]["bytes_per_call"])
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("3b-128k") is None
    monkeypatch.setattr(bench, "index_source_hash", lambda: "0" * 64)
    assert bench.measured_index_traffic("3b-128k") is None


def test_traffic_needs_a_dispatch_of_the_kernel(tmp_path):
    _counters(tmp_path / "x_counter_collection.csv", [("void fp::k_pool_q<128>(args)", 7.0)])
    with pytest.raises(RuntimeError):
        bench._counter(str(tmp_path / "x_counter_collection.csv"), "k_attn_dl<")


def test_index_bytes_small_layer():
    c = SimpleNamespace(S=256, b=128, Hq=2, Hkv=1, d=128, N=2)
    pattern = np.array([1, 0])             # one query-aware head, one vertical-slash head
    got = bench.index_bytes(c, pattern, nnz=3, njob=2, i8=False)
    k = 1 * 256 * 128 * 2                  # K once
    qlast = 2 * 128 * 128 * 2              # the last query block of both heads
    qa = 1 * 256 * 128 * 2                 # Q of the query-aware head only
    kbar = 2 * 1 * 2 * 128 * 4             # pooled keys written, then read
    csr = 4 * 5 + 4 * 3 + 4 * 3 + 8 * 2 + 4 * 2
    assert got == k + qlast + qa + kbar + csr
    # int8: one byte per element plus the fp32 row scales
    got8 = bench.index_bytes(c, pattern, nnz=3, njob=2, i8=True)
    assert got8 == (k // 2 + 256 * 4) + (qlast // 2 + 2 * 128 * 4) + (qa // 2 + 256 * 4) + kbar + csr


def test_attention_flop_counts():
    """Full count 4 b^2 d per selected block; the causally exact count keeps only the (query, key)
    pairs with key <= query inside each diagonal block (counted here by enumeration)."""
    for b, d, Hq, N, nnz in [(4, 2, 1, 1, 1), (8, 4, 2, 3, 9), (128, 128, 24, 1024, 175947)]:
        c = SimpleNamespace(b=b, d=d, Hq=Hq, N=N)
        full, exact = bench.attn_flops(c, nnz)
        assert full == 4 * b * b * d * nnz
        causal_pairs = sum(1 for q in range(b) for k in range(b) if k <= q)
        # every pair costs a d-term dot product (2d) and a d-wide weighted sum (2d)
        diag = Hq * N
        assert exact == (nnz - diag) * 4 * b * b * d + diag * causal_pairs * 4 * d
        assert exact < full
    # the 128K headline: 1.4760e12 in full, 1.3737e12 causally exact
    full, exact = bench.attn_flops(SimpleNamespace(b=128, d=128, Hq=24, N=1024), 175947)
    assert round(full / 1e12, 4) == 1.4760 and round(exact / 1e12, 4) == 1.3737


def test_w8a8_peak_is_the_time_sum_roofline():
    """Half the operations on the int8 peak, half on the bf16 peak: time per 4b^2d operations is
    2b^2d / P_i8 + 2b^2d / P_bf16."""
    ops = 4.0
    t = (ops / 2) / bench.PEAK_I8_TOPS + (ops / 2) / bench.PEAK_BF16_TFLOPS
    assert bench.PEAK_W8A8_TOPS == pytest.approx(ops / t)
    assert bench.PEAK_W8A8_TOPS == pytest.approx(3333.333, rel=1e-6)


def test_full_size_parity_record_on_host_tensors():
    """bench.compare_full on an index that is the oracle's own (as host tensors): every row equal,
    and a row changed away from the boundary is counted outside the rule."""
    import torch
    import gen
    import oracle
    from oracle import index as oi
    from tests import parity as P
    c = gen.CONFIGS["tiny"].with_(S=1024)
    L = gen.make(c)
    Q, K, V = L.f32("q"), L.f32("k"), L.f32("v")
    ref = oi.index(Q, K, c.b, c.gamma, c.tau)
    rp, ci = ref.csr()
    Oref = oracle.attn.attn(Q, K, V, rp, ci, c.b)

    def fake(rp, ci):
        return SimpleNamespace(row_ptr=torch.from_numpy(rp), col_idx=torch.from_numpy(ci),
                               pattern=torch.from_numpy(ref.pattern), jsd=torch.from_numpy(ref.jsd.astype(np.float32)))
    O = torch.from_numpy(Oref.astype(np.float32)).to(torch.bfloat16)
    out = bench.compare_full(c, fake(rp, ci), ref, O, Oref, P, oi)
    assert out["rows_equal"] == c.Hq * c.N and out["rows_outside_rule"] == 0 and out["gate"] == "pass"
    assert out["attn_maxabs"] <= 2e-2 and out["attn_elements"] == Oref.size
    # drop a middle block from the last row of head 0 (rows always keep 0 and i)
    r = c.N - 1
    row = ci[rp[r]:rp[r + 1]]
    mid = [j for j in row if 0 < j < r]
    assert mid
    keep = np.concatenate([ci[:rp[r]], row[row != mid[0]], ci[rp[r + 1]:]]).astype(np.int32)
    rp2 = rp.copy()
    rp2[r + 1:] -= 1
    out2 = bench.compare_full(c, fake(rp2, keep), ref, O, Oref, P, oi)
    assert out2["rows_outside_rule"] == 1 and out2["gate"] == "fail"
