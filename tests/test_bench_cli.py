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
    _counters(tmp_path / "bench_FETCH_SIZE_counter_collection.csv",
              [(attn, 1000.0), (attn, 1200.0), ("void fp::k_ig_stats1<128>(args)", 5.0)])
    _counters(tmp_path / "bench_WRITE_SIZE_counter_collection.csv", [(attn, 300.0), (attn, 300.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda name: str(out))
    bench.traffic_from(str(tmp_path), "3b-128k")
    rec = json.load(open(out))
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    # per launch: the mean over the kernel's dispatches, each counter scaled by its factor
    assert rec["bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2.0 + 300.0 * 1024 * 1.0)
    assert bench.measured_traffic("3b-128k") == pytest.approx(rec["bytes_per_launch"])
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("3b-128k") is None


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
