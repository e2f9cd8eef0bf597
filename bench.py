"""Benchmark: one dynamic block-sparse prefill attention layer on one MI355X.

A step is the whole hot path on one layer: fp_index (last-block statistics,
pattern test, selection, CSR and job list) followed by fp_attn (block-sparse
attention), inputs resident in HBM.  Default workload: a Llama-3.2-3B-shaped
layer at S = 131072 (b = 128, Hq = 24, Hkv = 8, d = 128, bf16), seeded
planted-v1 synthetic Q/K/V, gamma = 0.9, tau = 0.1.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu]

Prints progress on stderr and ONE JSON line on stdout.  Only one GPU is used;
--gpus above 1 exits with a message.

Measured HBM traffic of the attention kernel (the `traffic` field) comes from
two rocprofv3 counter passes over this script, scaled by the same counters on
a copy of known size:
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D -o copy_FETCH_SIZE -- python3 bench.py --copy-calibration
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D -o copy_WRITE_SIZE -- python3 bench.py --copy-calibration
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D -o bench_FETCH_SIZE -- python3 bench.py --steps 1 --warmup 0 --no-cpu
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D -o bench_WRITE_SIZE -- python3 bench.py --steps 1 --warmup 0 --no-cpu
    python bench.py --traffic-from D        # writes profiles/traffic_<config>.json
The file records a hash of the attention source; once the kernel changes the
field reads null until the passes are taken again.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 matrix cores
PEAK_I8_TOPS = 5000.0          # dense int8 matrix cores

CONFIG_TEXT = {
    "tiny": "one attention layer, S=2048, b=128, Hq=4, Hkv=2, d=128",
    "3b-32k": "Llama-3.2-3B-shaped attention layer, S=32768, b=128, Hq=24, Hkv=8, d=128",
    "3b-128k": "Llama-3.2-3B-shaped attention layer, S=131072, b=128, Hq=24, Hkv=8, d=128",
    "8b-64k": "Llama-3-8B-shaped attention layer, S=65536, b=256, Hq=32, Hkv=8, d=128, 3/4 heads vertical-slash",
    "w8a8-128k": "W8A8 Llama-3.2-3B-shaped attention layer, S=131072, b=128, Hq=24, Hkv=8, d=128",
    "3b-128k-b64": "Llama-3.2-3B-shaped attention layer with 64-token blocks, S=131072, b=64, Hq=24, Hkv=8, d=128",
}


ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SRC = os.path.join(ROOT, "dynamic_block_sparse_flexprefill_amd", "csrc", "attn.hip")
# the attention kernel whose launches the roofline and traffic figures describe
ATTN_KERNEL = {False: "k_attn_dl<", True: "k_attn_dl<"}
COPY_BYTES = 1 << 30


def attn_source_hash() -> str:
    return hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{name}.json")


def copy_calibration():
    """A device copy of COPY_BYTES bytes (three times), for scaling the traffic counters."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3", flush=True)


def _counter(csv_path: str, name_part: str) -> float:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path)) if name_part in r["Kernel_Name"]]
    if not vals:
        raise RuntimeError(f"no dispatch of {name_part} in {csv_path}")
    return sum(vals) / len(vals)


def traffic_from(d: str, config: str):
    """Combine the four counter passes in directory d into profiles/traffic_<config>.json."""
    f = lambda stem: os.path.join(d, f"{stem}_counter_collection.csv")
    copy_kib = COPY_BYTES / 1024.0
    fetch_factor = copy_kib / _counter(f("copy_FETCH_SIZE"), "copyBuffer")
    write_factor = copy_kib / _counter(f("copy_WRITE_SIZE"), "copyBuffer")
    import gen
    kname = ATTN_KERNEL[gen.CONFIGS[config].int8]
    fetch = _counter(f("bench_FETCH_SIZE"), kname)
    write = _counter(f("bench_WRITE_SIZE"), kname)
    rec = {"config": config, "kernel": kname, "attn_source_sha256": attn_source_hash(),
           "fetch_size_kib": fetch, "write_size_kib": write,
           "fetch_factor": fetch_factor, "write_factor": write_factor,
           "bytes_per_launch": fetch * 1024 * fetch_factor + write * 1024 * write_factor,
           "commands": [
               f"rocprofv3 --pmc {c} --output-format csv -d D -o copy_{c} -- python3 bench.py --copy-calibration"
               for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
               f"rocprofv3 --pmc {c} --output-format csv -d D -o bench_{c} -- python3 bench.py --steps 1 --warmup 0 --no-cpu --config {config}"
               for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    os.makedirs(os.path.dirname(traffic_file(config)), exist_ok=True)
    json.dump(rec, open(traffic_file(config), "w"), indent=1)
    print(json.dumps(rec))


def measured_traffic(config: str):
    """HBM bytes per attention launch from the counter passes, or None if stale or absent."""
    try:
        rec = json.load(open(traffic_file(config)))
    except (OSError, ValueError):
        return None
    if rec.get("attn_source_sha256") != attn_source_hash():
        return None
    return rec.get("bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def index_bytes(c, pattern: np.ndarray, nnz: int, njob: int, i8: bool) -> int:
    """Algorithmic HBM bytes of fp_index: K once, the last query block, Q of the
    query-aware heads only, the pooled keys written and read back, the CSR and jobs."""
    e = 1 if i8 else 2
    S, b, Hq, Hkv, d, N = c.S, c.b, c.Hq, c.Hkv, c.d, c.N
    k = Hkv * S * d * e + (Hkv * S * 4 if i8 else 0)
    qlast = Hq * b * d * e + (Hq * b * 4 if i8 else 0)
    n_qa = int((pattern == 1).sum())
    qa = n_qa * S * d * e + (n_qa * S * 4 if i8 else 0)
    kbar = 2 * Hkv * N * d * 4
    csr = 4 * (Hq * N + 1) + 4 * nnz + 4 * (Hkv * N + 1) + 8 * njob + 4 * Hkv * N
    return k + qlast + qa + kbar + csr


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="3b-128k", choices=sorted(CONFIG_TEXT))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work to sample")
    ap.add_argument("--copy-calibration", action="store_true", help="run the copy used to scale traffic counters")
    ap.add_argument("--traffic-from", metavar="DIR", help="write profiles/traffic_<config>.json from counter CSVs")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.traffic_from:
        traffic_from(args.traffic_from, args.config)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path shards by KV group "
              "with no exchange, so there is no multi-GPU run to time here.", file=sys.stderr)
        return 2

    import torch
    import gen
    import dynamic_block_sparse_flexprefill_amd as fpa

    torch.cuda.init()
    dev = torch.device("cuda:0")
    c = gen.CONFIGS[args.config]
    i8 = c.int8
    log(f"[bench] config {c.name}: S={c.S} b={c.b} Hq={c.Hq} Hkv={c.Hkv} gamma={c.gamma} tau={c.tau} "
        f"{'W8A8' if i8 else 'bf16'}; generating planted-v1 seed 0 ...")
    t0 = time.time()
    L = gen.make(c, seed=0)
    log(f"[bench] generated in {time.time() - t0:.1f}s; uploading")

    def up16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    if i8:
        q8 = L.int8()
        T = {k: torch.from_numpy(v).to(dev) for k, v in q8.items()}
    else:
        Q, K, V = up16(L.q), up16(L.k), up16(L.v)
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    ws = fpa.Workspace(sh, dev)
    idx = fpa.Index.empty(sh, dev)
    O = torch.empty(c.Hq, c.S, c.d, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        if i8:
            fpa.index_i8(T["q8"], T["sq"], T["k8"], T["sk"], c.b, c.gamma, c.tau, out=idx, ws=ws)
            fpa.attn_i8(T["q8"], T["sq"], T["k8"], T["sk"], T["v8"], T["sv"], idx, out=O, ws=ws)
        else:
            fpa.index(Q, K, c.b, c.gamma, c.tau, out=idx, ws=ws)
            fpa.attn(Q, K, V, idx, out=O, ws=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = int(idx.status.item())
    if status != 0:
        raise RuntimeError(f"device status {status} after fp_index")

    # timed region: K whole steps, with per-stage events on the launch stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        a, b_, e = ev[k]
        a.record(stream)
        if i8:
            fpa.index_i8(T["q8"], T["sq"], T["k8"], T["sk"], c.b, c.gamma, c.tau, out=idx, ws=ws)
        else:
            fpa.index(Q, K, c.b, c.gamma, c.tau, out=idx, ws=ws)
        b_.record(stream)
        if i8:
            fpa.attn_i8(T["q8"], T["sq"], T["k8"], T["sk"], T["v8"], T["sv"], idx, out=O, ws=ws)
        else:
            fpa.attn(Q, K, V, idx, out=O, ws=ws)
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_idx = np.array([a.elapsed_time(b_) for a, b_, _ in ev])
    t_att = np.array([b_.elapsed_time(e) for _, b_, e in ev])
    ms_step = wall * 1e3 / args.steps

    nnz = idx.nnz
    njob = int(idx.job_ptr[-1].item())
    pattern = idx.pattern.cpu().numpy()
    N = c.N
    density = nnz / (c.Hq * N * (N + 1) / 2)
    flops = 4.0 * c.b * c.b * c.d * nnz              # executed blocks, diagonal counted in full
    flops_exact = flops - 4.0 * c.b * c.b * c.d * c.Hq * N / 2 + 2.0 * c.b * (c.b + 1) * c.d * c.Hq * N
    att_ms = float(np.median(t_att))
    idx_ms = float(np.median(t_idx))
    achieved_tf = flops / (att_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if not i8 else 0.5 * (PEAK_I8_TOPS + PEAK_BF16_TFLOPS)
    ibytes = index_bytes(c, pattern, nnz, njob, i8)
    idx_gbs = ibytes / (idx_ms * 1e-3) / 1e9
    log(f"[bench] index {idx_ms:.3f} ms ({idx_gbs:.0f} GB/s algorithmic), attn {att_ms:.3f} ms "
        f"({achieved_tf:.1f} TFLOP/s), density {density:.4f}, patterns {np.bincount(pattern, minlength=2)}")

    rec = {
        "metric": "sparse prefill attn ms/layer @128K (3B shape); % HBM peak idx-gen, % MFMA attn",
        "value": round(ms_step, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16" if i8 else "bf16",
        "data": "synthetic (planted-v1 generator, seed 0)",
        "config": {"workload": CONFIG_TEXT[c.name], "name": c.name, "S": c.S, "b": c.b, "Hq": c.Hq,
                   "Hkv": c.Hkv, "d": c.d, "gamma": c.gamma, "tau": c.tau, "seed": 0},
        "roofline": {"bound": "mfma", "kernel": ATTN_KERNEL[i8].rstrip("<") + " (fp_attn)", "achieved": round(achieved_tf, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved_tf / peak, 4),
                     "traffic": measured_traffic(c.name)},
        "roofline_index": {"bound": "hbm", "kernel": "fp_index (all kernels)", "achieved": round(idx_gbs, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(idx_gbs / PEAK_HBM_GBS, 4),
                           "algorithmic_bytes": ibytes},
        "stages_ms": {"index_median": round(idx_ms, 4), "index_min": round(float(t_idx.min()), 4),
                      "attn_median": round(att_ms, 4), "attn_min": round(float(t_att.min()), 4)},
        "density": round(density, 6),
        "nnz_blocks": nnz,
        "job_entries": njob,
        "attn_flop": flops,
        "attn_flop_causal_exact": flops_exact,
        "patterns": {"vertical_slash": int((pattern == 0).sum()), "query_aware": int((pattern == 1).sum())},
        "cpu_baseline": None,
    }

    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(c, L, idx, args.cpu_budget, ms_step)
    print(json.dumps(rec), flush=True)
    return 0


def cpu_baseline(c, L, idx, budget_s: float, gpu_ms: float):
    """The float64 oracle on a bounded sample of the same layer, scaled to ms/layer."""
    import threadpoolctl
    from oracle import index as oi
    from oracle import attn as oa

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    log(f"[bench] oracle CPU baseline (~{budget_s:.0f}s, {threads} BLAS threads)")
    rp = idx.row_ptr.cpu().numpy()
    ci = idx.col_idx[: int(rp[-1])].cpu().numpy()
    pattern = idx.pattern.cpu().numpy()
    N, G = c.N, c.Hq // c.Hkv
    rng = np.random.default_rng(1)
    i8 = c.int8
    if i8:
        d8 = L.int8()
    else:
        Q, K, V = L.f32("q"), L.f32("k"), L.f32("v")
    # index: whole heads (statistics + rows), one VS and one QA head when both exist
    heads = []
    for pat in (0, 1):
        hs = np.nonzero(pattern == pat)[0]
        if hs.size:
            heads.append(int(hs[0]))
    t_heads = []
    for h in heads:
        t = time.perf_counter()
        if i8:
            oi.index_i8(d8["q8"], d8["sq"], d8["k8"], d8["sk"], c.b, c.gamma, c.tau, heads=[h])
        else:
            oi.index(Q, K, c.b, c.gamma, c.tau, heads=[h])
        t_heads.append(time.perf_counter() - t)
    per_head = {int(pattern[h]): t for h, t in zip(heads, t_heads)}
    n_vs = int((pattern == 0).sum())
    t_index = n_vs * per_head.get(0, per_head.get(1, 0.0)) + (c.Hq - n_vs) * per_head.get(1, per_head.get(0, 0.0))
    # attention: random rows until the budget is spent, then per-block cost x total blocks
    spent, blocks, rows = 0.0, 0, 0
    t_end = time.perf_counter() + max(1.0, budget_s - sum(t_heads))
    while time.perf_counter() < t_end:
        h, i = int(rng.integers(c.Hq)), int(rng.integers(N))
        t = time.perf_counter()
        if i8:
            oa.attn_i8(d8["q8"], d8["sq"], d8["k8"], d8["sk"], d8["v8"], d8["sv"], rp, ci, c.b, rows=[(h, i)])
        else:
            oa.attn(Q, K, V, rp, ci, c.b, rows=[(h, i)])
        spent += time.perf_counter() - t
        blocks += int(rp[h * N + i + 1] - rp[h * N + i])
        rows += 1
    nnz = int(rp[-1])
    t_attn = spent / max(blocks, 1) * nnz
    total_ms = (t_index + t_attn) * 1e3
    return {"value": round(total_ms, 1), "unit": "ms/layer", "cores": threads, "kind": "oracle",
            "sample": f"oracle.index on heads {heads} (one per pattern) scaled by pattern counts to {c.Hq} heads; "
                      f"oracle.attn on {rows} random CSR rows ({blocks} blocks) scaled per block to {nnz} blocks",
            "index_s": round(t_index, 2), "attn_s": round(t_attn, 2),
            "cpu": platform.processor() or platform.machine(), "gpu_speedup": round(total_ms / gpu_ms, 1)}


if __name__ == "__main__":
    sys.exit(main())
