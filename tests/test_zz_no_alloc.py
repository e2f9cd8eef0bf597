"""fp_index_static, the entry point for callers that cannot allocate device memory: its outputs
against fp_index's (same kernels, caller workspace) through the C ABI, on two calls in a row, the
second with a smaller layer, and bit-identical (the index is deterministic for identical inputs)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_flexprefill_amd as fpa
import gen
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fpa.lib()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _same(a, b):
    nnz, njob = a.nnz, int(a.job_ptr[-1].item())
    assert b.nnz == nnz and int(b.job_ptr[-1].item()) == njob
    lens = {"col_idx": nnz, "job_blk": njob, "job_mask": njob}
    for f in ("row_ptr", "col_idx", "job_ptr", "job_blk", "job_mask", "job_order", "pattern", "jsd", "stats",
              "status"):
        x, y = getattr(a, f), getattr(b, f)
        n = lens.get(f, x.numel())
        assert torch.equal(x.flatten()[:n], y.flatten()[:n]), f


def _static_call(Q, K, c, out):
    """fp_index_static through the C ABI (ctypes), on torch's current stream."""
    L = fpa.lib()
    sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
    o = out.c_struct()
    rc = L.fp_index_static(ctypes.byref(sh), ctypes.c_void_p(Q.data_ptr()), ctypes.c_void_p(K.data_ptr()),
                           c.gamma, c.tau, ctypes.byref(o), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == fpa.FP_OK, fpa.strerror(rc)


@pytest.mark.parametrize("first,second", [
    (dict(S=4096, Hq=8, Hkv=2), dict(S=1024, Hq=4, Hkv=2)),
    (dict(S=32768, Hq=6, Hkv=2), dict(S=2048, b=64, Hq=4, Hkv=2)),
])
def test_static_scratch_matches_workspace_call(first, second):
    for kw in (first, second):
        c = gen.CONFIGS["tiny"].with_(**kw)
        say(f"fp_index_static vs fp_index: S={c.S} b={c.b} Hq={c.Hq} Hkv={c.Hkv}")
        L = gen.make(c)
        Qd, Kd, _ = P.layer_on_device(L)
        sh = fpa.shape_of(c.S, c.b, c.Hq, c.Hkv)
        assert fpa.workspace_bytes(sh, 0) <= fpa.binding.FP_STATIC_SCRATCH_BYTES
        want = fpa.index(Qd, Kd, c.b, c.gamma, c.tau, stats=True)
        got = fpa.Index.empty(sh, Qd.device, stats=True)
        got.status.fill_(-1)
        _static_call(Qd, Kd, c, got)
        torch.cuda.synchronize()
        assert int(got.status.item()) == 0
        _same(want, got)
        P.check_jobs(got, c.G)
