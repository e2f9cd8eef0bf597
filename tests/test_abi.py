"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest
import torch

import dynamic_block_sparse_flexprefill_amd as fpa

# The argument checks below pass placeholder device pointers (0x1000) that validation rejects
# before anything is enqueued; on a machine with a GPU a regression in that validation would
# launch on them, so those checks run on GPU-less hosts only.
no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="placeholder device pointers: CPU-only argument checks")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fpattn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("fp_index", "fp_index_i8", "fp_attn", "fp_attn_i8", "fp_build_jobs",
              "fp_workspace_bytes", "fp_csr_capacity", "fp_job_capacity", "fp_strerror",
              "fp_version", "fp_probe_qk_i8", "fp_index_batch", "fp_attn_batch",
              "fp_index_i8_batch", "fp_attn_i8_batch", "fp_index_static", "fp_index_shared",
              "fp_index_pooled", "fp_qkv_project", "fp_attn_split", "fp_block_uses",
              "fp_batch_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = fpa.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_strerror():
    assert fpa.lib().fp_version() >= 100
    for code in range(0, -8, -1):
        assert isinstance(fpa.strerror(code), str) and fpa.strerror(code)
    assert "unknown" in fpa.strerror(-99)


@pytest.mark.parametrize("S,b,Hq,Hkv,d,code", [
    (2048, 128, 4, 2, 128, fpa.FP_OK),
    (2000, 128, 4, 2, 128, fpa.FP_EINVAL),        # S % b
    (2048, 128, 5, 2, 128, fpa.FP_EINVAL),        # Hq % Hkv
    (0, 128, 4, 2, 128, fpa.FP_EINVAL),
    (2048, 128, 4, 2, 64, fpa.FP_EUNSUPPORTED),   # d
    (2048, 32, 4, 2, 128, fpa.FP_EUNSUPPORTED),   # b
    (2048, 64, 4, 2, 128, fpa.FP_OK),             # b = 64
    (4096, 64, 32, 1, 128, fpa.FP_EUNSUPPORTED),  # G = 32: more heads per group than attention waves
    (128 * 8193, 128, 4, 2, 128, fpa.FP_EUNSUPPORTED),  # N > 8192
    (4096, 256, 16, 1, 128, fpa.FP_EUNSUPPORTED),  # G * b > 2048
    (4096, 128, 16, 1, 128, fpa.FP_OK),            # G * b = 2048
])
def test_shape_validation(S, b, Hq, Hkv, d, code):
    sh = fpa.shape_of(S, b, Hq, Hkv, d)
    n = ctypes.c_size_t(0)
    rc = fpa.lib().fp_workspace_bytes(ctypes.byref(sh), 0, ctypes.byref(n))
    assert rc == code
    if code == fpa.FP_OK:
        assert n.value > 0
        N = S // b
        assert fpa.csr_capacity(sh) == Hq * N * (N + 1) // 2
        assert fpa.job_capacity(sh) == Hkv * N * (N + 1) // 2
    else:
        assert fpa.csr_capacity(sh) == code


def _dummy_out(sh, col_cap=None):
    N = sh.S // sh.b
    o = fpa.FpIndexOut()
    for f in ("row_ptr", "col_idx", "job_ptr", "job_blk", "job_mask", "job_order", "pattern", "jsd", "status"):
        setattr(o, f, 0x1000)   # never dereferenced: every case below fails validation first
    o.col_cap = sh.Hq * N * (N + 1) // 2 if col_cap is None else col_cap
    o.job_cap = sh.Hkv * N * (N + 1) // 2
    o.stats = None
    return o


@no_gpu_only
@pytest.mark.parametrize("gamma,tau,ok", [(0.0, 0.1, False), (1.5, 0.1, False), (float("nan"), 0.1, False),
                                          (0.9, -0.1, False), (0.9, float("nan"), False)])
def test_index_rejects_bad_parameters(gamma, tau, ok):
    sh = fpa.shape_of(2048, 128, 4, 2)
    o = _dummy_out(sh)
    rc = fpa.lib().fp_index(ctypes.byref(sh), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000),
                            gamma, tau, ctypes.byref(o), ctypes.c_void_p(0x1000), 1 << 30, None)
    assert rc == fpa.FP_EINVAL


@no_gpu_only
def test_index_rejects_null_and_small_workspace():
    sh = fpa.shape_of(2048, 128, 4, 2)
    L = fpa.lib()
    o = _dummy_out(sh)
    P = ctypes.c_void_p(0x1000)
    assert L.fp_index(ctypes.byref(sh), None, P, 0.9, 0.1, ctypes.byref(o), P, 1 << 30, None) == fpa.FP_EINVAL
    assert L.fp_index(ctypes.byref(sh), P, P, 0.9, 0.1, None, P, 1 << 30, None) == fpa.FP_EINVAL
    assert L.fp_index(ctypes.byref(sh), P, P, 0.9, 0.1, ctypes.byref(o), None, 1 << 30, None) == fpa.FP_EINVAL
    assert L.fp_index(ctypes.byref(sh), P, P, 0.9, 0.1, ctypes.byref(o), P, 16, None) == fpa.FP_EWORKSPACE
    small = _dummy_out(sh, col_cap=10)   # fewer entries than rows
    assert L.fp_index(ctypes.byref(sh), P, P, 0.9, 0.1, ctypes.byref(small), P, 1 << 30, None) == fpa.FP_EINVAL
    o.status = None
    assert L.fp_index(ctypes.byref(sh), P, P, 0.9, 0.1, ctypes.byref(o), P, 1 << 30, None) == fpa.FP_EINVAL
    bad = fpa.shape_of(2048, 128, 4, 2, 64)
    assert L.fp_index(ctypes.byref(bad), P, P, 0.9, 0.1, ctypes.byref(o), P, 1 << 30, None) == fpa.FP_EUNSUPPORTED


@no_gpu_only
def test_attn_and_probe_reject_bad_arguments():
    sh = fpa.shape_of(2048, 128, 4, 2)
    L = fpa.lib()
    o = _dummy_out(sh)
    P = ctypes.c_void_p(0x1000)
    assert L.fp_attn(ctypes.byref(sh), P, P, None, ctypes.byref(o), P, P, 1 << 30, None) == fpa.FP_EINVAL
    assert L.fp_attn(ctypes.byref(sh), P, P, P, ctypes.byref(o), P, P, 8, None) == fpa.FP_EWORKSPACE
    assert L.fp_attn_i8(ctypes.byref(sh), P, None, P, P, P, P, ctypes.byref(o), P, P, 1 << 30, None) == fpa.FP_EINVAL
    assert L.fp_probe_qk_i8(ctypes.byref(sh), P, P, 4, 0, 0, 0, P, None) == fpa.FP_EINVAL   # h out of range
    assert L.fp_probe_qk_i8(ctypes.byref(sh), P, P, 0, 16, 0, 0, P, None) == fpa.FP_EINVAL  # i out of range
    assert L.fp_probe_qk_i8(ctypes.byref(sh), P, P, 0, 0, 0, 2, P, None) == fpa.FP_EINVAL   # unknown path
    assert L.fp_probe_qk_i8(ctypes.byref(sh), P, None, 0, 0, 0, 1, P, None) == fpa.FP_EINVAL
    # head-pattern sharing: unknown variant, missing int8 scales, and fp_index's own checks
    big = 1 << 30
    assert L.fp_index_shared(ctypes.byref(sh), 2, P, None, P, None, 0.9, 0.1, ctypes.byref(o), P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_shared(ctypes.byref(sh), 1, P, None, P, P, 0.9, 0.1, ctypes.byref(o), P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_shared(ctypes.byref(sh), 0, P, None, P, None, 1.5, 0.1, ctypes.byref(o), P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_shared(ctypes.byref(sh), 0, P, None, P, None, 0.9, 0.1, ctypes.byref(o), P, 8, None) == fpa.FP_EWORKSPACE
    # the projection and the pooled-query index
    assert L.fp_index_pooled(ctypes.byref(sh), P, P, None, 0.9, 0.1, ctypes.byref(o), P, big, None) == fpa.FP_EINVAL
    nul = [None] * 6
    assert L.fp_qkv_project(ctypes.byref(sh), 256, None, P, None, None, P, P, P, None, None, *nul, None) == fpa.FP_EINVAL
    assert L.fp_qkv_project(ctypes.byref(sh), 256, P, P, P, None, P, P, P, None, None, *nul, None) == fpa.FP_EINVAL   # cos without sin
    assert L.fp_qkv_project(ctypes.byref(sh), 100, P, P, None, None, P, P, P, None, None, *nul, None) == fpa.FP_EUNSUPPORTED
    assert L.fp_qkv_project(ctypes.byref(sh), 256, P, P, None, None, P, P, P, None, None, P, None, None, None, None, None, None) == fpa.FP_EINVAL
    sh256 = fpa.shape_of(2048, 256, 4, 2)
    assert L.fp_qkv_project(ctypes.byref(sh256), 256, P, P, None, None, P, P, P, P, None, *nul, None) == fpa.FP_EUNSUPPORTED
    o2 = _dummy_out(sh)
    o2.job_ptr = None
    assert L.fp_build_jobs(ctypes.byref(sh), ctypes.byref(o2), P, 1 << 30, None) == fpa.FP_EINVAL


def test_workspace_grows_with_shape():
    a = fpa.workspace_bytes(fpa.shape_of(2048, 128, 4, 2), 0)
    b = fpa.workspace_bytes(fpa.shape_of(131072, 128, 24, 8), 0)
    assert b > a > 0
    # nothing of size Hq x S x b: the 128K workspace stays far below the b x S score matrix of one head
    assert b < 128 * 131072 * 4
    # variant 1 adds fp_attn_i8's bf16 widening of V8 (Hkv x S x d), 256-byte aligned
    b1 = fpa.workspace_bytes(fpa.shape_of(131072, 128, 24, 8), 1)
    assert b1 == b + 2 * 8 * 131072 * 128


def test_batch_workspace_bytes():
    """Distinct lengths need the longest sequence's workspace; a run of equal short lengths runs as
    one call and needs more; equal long sequences (more than 256 key blocks) are not folded."""
    sh = fpa.shape_of(4096, 128, 6, 2)
    one = lambda S, v: fpa.workspace_bytes(fpa.shape_of(S, 128, 6, 2), v)
    for v in (0, 1):
        assert fpa.batch_workspace_bytes(sh, [2048, 1024, 512], v) == max(one(S, v) for S in (2048, 1024, 512))
        assert fpa.batch_workspace_bytes(sh, [1024] * 4, v) > one(1024, v)
        assert fpa.batch_workspace_bytes(sh, [1024] * 4, v) > fpa.batch_workspace_bytes(sh, [1024] * 2, v)
        long_ = 128 * 300
        assert fpa.batch_workspace_bytes(sh, [long_] * 3, v) == one(long_, v)
    assert fpa.batch_workspace_bytes(sh, [1024] * 4, 1) >= fpa.batch_workspace_bytes(sh, [1024] * 4, 0)
    # a run whose folded worst case would not fit 32-bit offsets is not folded
    big = fpa.shape_of(32768, 128, 1024, 1024)
    assert fpa.batch_workspace_bytes(big, [32768] * 64, 0) == fpa.workspace_bytes(big, 0)
    L = fpa.lib()
    n = ctypes.c_size_t(0)
    lens = (ctypes.c_int32 * 2)(1024, 1024)
    assert L.fp_batch_workspace_bytes(ctypes.byref(sh), 0, lens, 0, ctypes.byref(n)) == fpa.FP_EINVAL
    assert L.fp_batch_workspace_bytes(ctypes.byref(sh), 2, None, 0, ctypes.byref(n)) == fpa.FP_EINVAL
    assert L.fp_batch_workspace_bytes(ctypes.byref(sh), 2, lens, 2, ctypes.byref(n)) == fpa.FP_EINVAL
    assert L.fp_batch_workspace_bytes(ctypes.byref(sh), 2, lens, 0, None) == fpa.FP_EINVAL
    bad = (ctypes.c_int32 * 2)(1000, 1000)          # not a multiple of b
    assert L.fp_batch_workspace_bytes(ctypes.byref(sh), 2, bad, 0, ctypes.byref(n)) == fpa.FP_EINVAL


@no_gpu_only
def test_batch_rejects_bad_arguments():
    """Ragged batches: every sequence is checked before anything is enqueued."""
    L = fpa.lib()
    P = ctypes.c_void_p(0x1000)
    sh = fpa.shape_of(2048, 128, 4, 2)
    lens = [1024, 384, 2048]
    outs = (fpa.FpIndexOut * 3)(*[_dummy_out(fpa.shape_of(S, 128, 4, 2)) for S in lens])
    arr = (ctypes.c_int32 * 3)(*lens)
    big = 1 << 30
    assert L.fp_index_batch(ctypes.byref(sh), 0, arr, P, P, 0.9, 0.1, outs, P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_batch(ctypes.byref(sh), 3, None, P, P, 0.9, 0.1, outs, P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_batch(ctypes.byref(sh), 3, arr, P, P, 1.5, 0.1, outs, P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_batch(ctypes.byref(sh), 3, arr, P, P, 0.9, 0.1, outs, P, 64, None) == fpa.FP_EWORKSPACE
    ragged = (ctypes.c_int32 * 3)(1024, 300, 2048)       # 300 is not a multiple of b
    assert L.fp_index_batch(ctypes.byref(sh), 3, ragged, P, P, 0.9, 0.1, outs, P, big, None) == fpa.FP_EINVAL
    small = (fpa.FpIndexOut * 3)(outs[0], _dummy_out(fpa.shape_of(384, 128, 4, 2), col_cap=4), outs[2])
    assert L.fp_index_batch(ctypes.byref(sh), 3, arr, P, P, 0.9, 0.1, small, P, big, None) == fpa.FP_EINVAL
    # the workspace must cover the longest sequence (its int8 attention form for fp_attn_i8_batch)
    need = fpa.workspace_bytes(fpa.shape_of(2048, 128, 4, 2), 0)
    need_i8 = fpa.workspace_bytes(fpa.shape_of(2048, 128, 4, 2), 1)
    assert need_i8 > need
    assert L.fp_attn_batch(ctypes.byref(sh), 3, arr, P, P, P, outs, P, P, need - 1, None) == fpa.FP_EWORKSPACE
    assert L.fp_attn_batch(ctypes.byref(sh), 3, arr, P, P, None, outs, P, P, big, None) == fpa.FP_EINVAL
    bad = fpa.shape_of(2048, 128, 4, 2, 64)
    assert L.fp_attn_batch(ctypes.byref(bad), 3, arr, P, P, P, outs, P, P, big, None) == fpa.FP_EUNSUPPORTED
    # W8A8 forms: the same checks, and the per-token scales are required
    assert L.fp_index_i8_batch(ctypes.byref(sh), 3, arr, P, None, P, P, 0.9, 0.1, outs, P, big, None) == fpa.FP_EINVAL
    assert L.fp_index_i8_batch(ctypes.byref(sh), 3, arr, P, P, P, P, 0.9, 0.1, outs, P, 64, None) == fpa.FP_EWORKSPACE
    assert L.fp_index_i8_batch(ctypes.byref(sh), 3, ragged, P, P, P, P, 0.9, 0.1, outs, P, big, None) == fpa.FP_EINVAL
    assert L.fp_attn_i8_batch(ctypes.byref(sh), 3, arr, P, P, P, P, P, None, outs, P, P, big, None) == fpa.FP_EINVAL
    assert L.fp_attn_i8_batch(ctypes.byref(sh), 3, arr, P, P, P, P, P, P, outs, P, P, need_i8 - 1, None) == fpa.FP_EWORKSPACE
    assert L.fp_attn_i8(ctypes.byref(sh), P, P, P, P, P, P, ctypes.byref(outs[2]), P, P, need_i8 - 1, None) == fpa.FP_EWORKSPACE


@no_gpu_only
def test_static_scratch_entry_point_rejects_before_enqueuing():
    """fp_index_static checks its arguments like fp_index, and a shape whose scratch exceeds the
    library's static buffer gets FP_ESCRATCH before any device call."""
    L = fpa.lib()
    P = ctypes.c_void_p(0x1000)
    sh = fpa.shape_of(2048, 128, 4, 2)
    o = _dummy_out(sh)
    assert L.fp_index_static(ctypes.byref(sh), None, P, 0.9, 0.1, ctypes.byref(o), None) == fpa.FP_EINVAL
    assert L.fp_index_static(ctypes.byref(sh), P, P, 1.5, 0.1, ctypes.byref(o), None) == fpa.FP_EINVAL
    assert L.fp_index_static(ctypes.byref(sh), P, P, 0.9, 0.1, None, None) == fpa.FP_EINVAL
    big = fpa.shape_of(64 * 8192, 64, 24, 8)
    assert fpa.workspace_bytes(big, 0) > fpa.binding.FP_STATIC_SCRATCH_BYTES
    ob = _dummy_out(big)
    assert L.fp_index_static(ctypes.byref(big), P, P, 0.9, 0.1, ctypes.byref(ob), None) == fpa.FP_ESCRATCH
    assert "scratch" in fpa.strerror(fpa.FP_ESCRATCH)


def test_static_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define FP_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == fpa.binding.FP_STATIC_SCRATCH_BYTES
    # the 3B-shaped 128K layer fits with 64- and 128-token blocks
    for b in (64, 128):
        assert fpa.workspace_bytes(fpa.shape_of(131072, b, 24, 8), 0) <= fpa.binding.FP_STATIC_SCRATCH_BYTES


@no_gpu_only
def test_attn_split_rejects_bad_arguments():
    L = fpa.lib()
    P = ctypes.c_void_p(0x1000)
    sh = fpa.shape_of(2048, 128, 4, 2)
    o = _dummy_out(sh)
    n = ctypes.c_size_t(0)
    assert L.fp_attn_split_workspace_bytes(ctypes.byref(sh), 4, 2, ctypes.byref(n)) == fpa.FP_OK
    need = n.value
    assert need > fpa.workspace_bytes(sh)
    assert L.fp_attn_split_workspace_bytes(ctypes.byref(sh), 4, 1, ctypes.byref(n)) == fpa.FP_EINVAL      # nseg < 2
    assert L.fp_attn_split_workspace_bytes(ctypes.byref(sh), -1, 2, ctypes.byref(n)) == fpa.FP_EINVAL
    b64 = fpa.shape_of(2048, 64, 4, 2)
    assert L.fp_attn_split_workspace_bytes(ctypes.byref(b64), 4, 2, ctypes.byref(n)) == fpa.FP_EUNSUPPORTED
    assert L.fp_attn_split(ctypes.byref(sh), P, P, P, ctypes.byref(o), 4, 2, P, P, need - 1, None) == fpa.FP_EWORKSPACE
    assert L.fp_attn_split(ctypes.byref(sh), P, P, None, ctypes.byref(o), 4, 2, P, P, need, None) == fpa.FP_EINVAL
    assert L.fp_attn_split(ctypes.byref(sh), P, P, P, ctypes.byref(o), 4, 65, P, P, 1 << 30, None) == fpa.FP_EINVAL
    # the partial slots grow with the split jobs and segments, clamped to the job count
    a = ctypes.c_size_t(0)
    b = ctypes.c_size_t(0)
    L.fp_attn_split_workspace_bytes(ctypes.byref(sh), 1 << 20, 2, ctypes.byref(a))
    L.fp_attn_split_workspace_bytes(ctypes.byref(sh), 32, 2, ctypes.byref(b))     # 32 = Hkv * N jobs
    assert a.value == b.value > need
