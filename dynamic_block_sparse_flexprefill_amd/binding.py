"""ctypes binding of libfpattn.so (the C ABI in include/fpattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Torch supplies device memory and the current stream.
If the library is missing the import of this module still works, but every
call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfpattn.so")

FP_OK = 0
FP_EINVAL = -1
FP_EUNSUPPORTED = -2
FP_EWORKSPACE = -3
FP_ECAPACITY = -4
FP_EHIP = -5
FP_EJOBCAPACITY = -6
FP_ETIMEOUT = -7
FP_ESCRATCH = -8
FP_STATIC_SCRATCH_BYTES = 64 << 20    # include/fpattn.h
FP_STATUS_CSR_OVERFLOW = 1
FP_STATUS_JOB_OVERFLOW = 2
FP_STATUS_WAIT_TIMEOUT = 4
VERTICAL_SLASH = 0
QUERY_AWARE = 1
PROBE_ATTN = 0
PROBE_STATS = 1


class FpShape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("b", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32)]


class FpIndexOut(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("col_cap", ctypes.c_int64),
                ("job_ptr", ctypes.c_void_p), ("job_blk", ctypes.c_void_p), ("job_mask", ctypes.c_void_p),
                ("job_cap", ctypes.c_int64), ("job_order", ctypes.c_void_p), ("pattern", ctypes.c_void_p),
                ("jsd", ctypes.c_void_p), ("stats", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class FpError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} (code {code})")


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded library; raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m dynamic_block_sparse_flexprefill_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sp, op = ctypes.POINTER(FpShape), ctypes.POINTER(FpIndexOut)
        f = ctypes.c_float
        L.fp_version.restype = ctypes.c_int
        L.fp_strerror.restype = ctypes.c_char_p
        L.fp_strerror.argtypes = [ctypes.c_int]
        L.fp_workspace_bytes.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.fp_batch_workspace_bytes.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.fp_csr_capacity.restype = ctypes.c_int64
        L.fp_csr_capacity.argtypes = [sp]
        L.fp_job_capacity.restype = ctypes.c_int64
        L.fp_job_capacity.argtypes = [sp]
        L.fp_index.argtypes = [sp, _P, _P, f, f, op, _P, ctypes.c_size_t, _P]
        L.fp_index_i8.argtypes = [sp, _P, _P, _P, _P, f, f, op, _P, ctypes.c_size_t, _P]
        L.fp_build_jobs.argtypes = [sp, op, _P, ctypes.c_size_t, _P]
        L.fp_attn.argtypes = [sp, _P, _P, _P, op, _P, _P, ctypes.c_size_t, _P]
        L.fp_attn_i8.argtypes = [sp, _P, _P, _P, _P, _P, _P, op, _P, _P, ctypes.c_size_t, _P]
        L.fp_probe_qk_i8.argtypes = [sp, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P]
        L.fp_index_static.argtypes = [sp, _P, _P, f, f, op, _P]
        L.fp_index_shared.argtypes = [sp, ctypes.c_int, _P, _P, _P, _P, f, f, op, _P, ctypes.c_size_t, _P]
        L.fp_block_uses.argtypes = [sp, op, _P, _P, _P]
        L.fp_attn_split_workspace_bytes.argtypes = [sp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.fp_attn_split.argtypes = [sp, _P, _P, _P, op, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_size_t, _P]
        L.fp_qkv_project.argtypes = [sp, ctypes.c_int] + [_P] * 16
        L.fp_index_pooled.argtypes = [sp, _P, _P, _P, f, f, op, _P, ctypes.c_size_t, _P]
        lp = ctypes.POINTER(ctypes.c_int32)
        L.fp_index_batch.argtypes = [sp, ctypes.c_int, lp, _P, _P, f, f, op, _P, ctypes.c_size_t, _P]
        L.fp_attn_batch.argtypes = [sp, ctypes.c_int, lp, _P, _P, _P, op, _P, _P, ctypes.c_size_t, _P]
        L.fp_index_i8_batch.argtypes = [sp, ctypes.c_int, lp, _P, _P, _P, _P, f, f, op, _P, ctypes.c_size_t, _P]
        L.fp_attn_i8_batch.argtypes = [sp, ctypes.c_int, lp, _P, _P, _P, _P, _P, _P, op, _P, _P,
                                       ctypes.c_size_t, _P]
        for name in ("fp_workspace_bytes", "fp_batch_workspace_bytes", "fp_index", "fp_index_i8", "fp_build_jobs", "fp_attn",
                     "fp_attn_i8", "fp_probe_qk_i8", "fp_index_static", "fp_index_shared", "fp_block_uses", "fp_attn_split_workspace_bytes", "fp_attn_split", "fp_qkv_project", "fp_index_pooled", "fp_index_batch", "fp_attn_batch",
                     "fp_index_i8_batch", "fp_attn_i8_batch"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().fp_strerror(code).decode()


def shape_of(S: int, b: int, Hq: int, Hkv: int, d: int = 128) -> FpShape:
    return FpShape(S, b, Hq, Hkv, d)


def workspace_bytes(shape: FpShape, variant: int = 1) -> int:
    n = ctypes.c_size_t(0)
    rc = lib().fp_workspace_bytes(ctypes.byref(shape), variant, ctypes.byref(n))
    if rc:
        raise FpError(rc, "fp_workspace_bytes")
    return n.value


def batch_workspace_bytes(shape: FpShape, seqlens, variant: int = 1) -> int:
    """fp_batch_workspace_bytes: the workspace with which every run of equal-length sequences of a
    batch runs as one call (shape.S is ignored)."""
    lens = [int(S) for S in seqlens]
    n = ctypes.c_size_t(0)
    rc = lib().fp_batch_workspace_bytes(ctypes.byref(shape), len(lens), (ctypes.c_int32 * len(lens))(*lens), variant,
                                        ctypes.byref(n))
    if rc:
        raise FpError(rc, "fp_batch_workspace_bytes")
    return n.value


def csr_capacity(shape: FpShape) -> int:
    return int(lib().fp_csr_capacity(ctypes.byref(shape)))


def job_capacity(shape: FpShape) -> int:
    return int(lib().fp_job_capacity(ctypes.byref(shape)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise TypeError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                        f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


@dataclass
class Index:
    """Device tensors of one fp_index result (see fp_index_out in fpattn.h)."""
    shape: FpShape
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    job_ptr: torch.Tensor
    job_blk: torch.Tensor
    job_mask: torch.Tensor
    job_order: torch.Tensor
    pattern: torch.Tensor
    jsd: torch.Tensor
    status: torch.Tensor
    stats: Optional[torch.Tensor] = None

    @classmethod
    def empty(cls, shape: FpShape, device, stats: bool = False, col_cap: Optional[int] = None,
              job_cap: Optional[int] = None) -> "Index":
        N = shape.S // shape.b
        col_cap = csr_capacity(shape) if col_cap is None else col_cap
        job_cap = job_capacity(shape) if job_cap is None else job_cap
        i32 = dict(dtype=torch.int32, device=device)
        return cls(shape=shape,
                   row_ptr=torch.empty(shape.Hq * N + 1, **i32),
                   col_idx=torch.empty(max(col_cap, 1), **i32),
                   job_ptr=torch.empty(shape.Hkv * N + 1, **i32),
                   job_blk=torch.empty(max(job_cap, 1), **i32),
                   job_mask=torch.empty(max(job_cap, 1), **i32),
                   job_order=torch.empty(shape.Hkv * N, **i32),
                   pattern=torch.empty(shape.Hq, dtype=torch.uint8, device=device),
                   jsd=torch.empty(shape.Hq, dtype=torch.float32, device=device),
                   status=torch.zeros(1, **i32),
                   stats=torch.empty(3, shape.Hq, N, dtype=torch.float32, device=device) if stats else None)

    def c_struct(self) -> FpIndexOut:
        return FpIndexOut(self.row_ptr.data_ptr(), self.col_idx.data_ptr(), self.col_idx.numel(),
                          self.job_ptr.data_ptr(), self.job_blk.data_ptr(), self.job_mask.data_ptr(),
                          self.job_blk.numel(), self.job_order.data_ptr(), self.pattern.data_ptr(),
                          self.jsd.data_ptr(), 0 if self.stats is None else self.stats.data_ptr(),
                          self.status.data_ptr())

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())

    def density(self) -> float:
        N = self.shape.S // self.shape.b
        return self.nnz / (self.shape.Hq * N * (N + 1) / 2)


class Workspace:
    """A device byte buffer sized by fp_workspace_bytes for a shape, or with seqlens given, by
    fp_batch_workspace_bytes for a batch of sequences of those lengths."""

    def __init__(self, shape: FpShape, device, seqlens=None):
        self.nbytes = workspace_bytes(shape, 1) if seqlens is None else batch_workspace_bytes(shape, seqlens, 1)
        self.buf = torch.empty(max(self.nbytes, 1), dtype=torch.uint8, device=device)


def _ws(shape, ws, device, seqlens=None):
    return Workspace(shape, device, seqlens) if ws is None else ws


def index(Q: torch.Tensor, K: torch.Tensor, b: int, gamma: float, tau: float, *, stats: bool = False,
          out: Optional[Index] = None, ws: Optional[Workspace] = None, stream=None) -> Index:
    """fp_index: sparse key-block CSR, job list, pattern and divergence per head (bf16 Q, K)."""
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    shape = shape_of(S, b, Hq, Hkv, d)
    _check(Q, "Q", torch.bfloat16, (Hq, S, d))
    _check(K, "K", torch.bfloat16, (Hkv, S, d))
    out = Index.empty(shape, Q.device, stats=stats) if out is None else out
    ws = _ws(shape, ws, Q.device)
    o = out.c_struct()
    rc = lib().fp_index(ctypes.byref(shape), _ptr(Q), _ptr(K), gamma, tau, ctypes.byref(o),
                        _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_index")
    return out


def index_i8(Q8, sQ, K8, sK, b: int, gamma: float, tau: float, *, stats: bool = False,
             out: Optional[Index] = None, ws: Optional[Workspace] = None, stream=None) -> Index:
    """fp_index_i8: W8A8 sparse-index generation (int8 Q/K with fp32 per-token scales)."""
    Hq, S, d = Q8.shape
    Hkv = K8.shape[0]
    shape = shape_of(S, b, Hq, Hkv, d)
    _check(Q8, "Q8", torch.int8, (Hq, S, d))
    _check(K8, "K8", torch.int8, (Hkv, S, d))
    _check(sQ, "sQ", torch.float32, (Hq, S))
    _check(sK, "sK", torch.float32, (Hkv, S))
    out = Index.empty(shape, Q8.device, stats=stats) if out is None else out
    ws = _ws(shape, ws, Q8.device)
    o = out.c_struct()
    rc = lib().fp_index_i8(ctypes.byref(shape), _ptr(Q8), _ptr(sQ), _ptr(K8), _ptr(sK), gamma, tau,
                           ctypes.byref(o), _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_index_i8")
    return out


def index_static(Q: torch.Tensor, K: torch.Tensor, b: int, gamma: float, tau: float, *, stats: bool = False,
                 out: Optional[Index] = None, stream=None) -> Index:
    """fp_index_static: fp_index with the library's per-GPU scratch buffer instead of a workspace
    (for callers that cannot allocate device memory; out must then be supplied preallocated)."""
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    shape = shape_of(S, b, Hq, Hkv, d)
    _check(Q, "Q", torch.bfloat16, (Hq, S, d))
    _check(K, "K", torch.bfloat16, (Hkv, S, d))
    out = Index.empty(shape, Q.device, stats=stats) if out is None else out
    o = out.c_struct()
    rc = lib().fp_index_static(ctypes.byref(shape), _ptr(Q), _ptr(K), gamma, tau, ctypes.byref(o), _stream(stream))
    if rc:
        raise FpError(rc, "fp_index_static")
    return out


def _index_variant(fn: str, Q, K, b, gamma, tau, sQ, sK, stats, out, ws, stream) -> Index:
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    shape = shape_of(S, b, Hq, Hkv, d)
    i8 = Q.dtype == torch.int8
    dt = torch.int8 if i8 else torch.bfloat16
    _check(Q, "Q", dt, (Hq, S, d))
    _check(K, "K", dt, (Hkv, S, d))
    if i8:
        _check(sQ, "sQ", torch.float32, (Hq, S))
        _check(sK, "sK", torch.float32, (Hkv, S))
    out = Index.empty(shape, Q.device, stats=stats) if out is None else out
    ws = _ws(shape, ws, Q.device)
    o = out.c_struct()
    rc = getattr(lib(), fn)(ctypes.byref(shape), 1 if i8 else 0, _ptr(Q), _ptr(sQ) if i8 else None, _ptr(K),
                            _ptr(sK) if i8 else None, gamma, tau, ctypes.byref(o), _ptr(ws.buf), ws.nbytes,
                            _stream(stream))
    if rc:
        raise FpError(rc, fn)
    return out


def qkv_project(X: torch.Tensor, W: torch.Tensor, Hq: int, Hkv: int, b: int, *, rope_cos=None, rope_sin=None,
                pooled: bool = True, int8: bool = False, out=None, stream=None) -> dict:
    """fp_qkv_project: Q, K, V (bf16, head-major) = rotary(X W^T) split by heads, with the block means
    qbar / kbar (pooled=True) and the per-(head, token) int8 codes and scales (int8=True) from the
    same epilogue.  X: bf16 [S, D]; W: bf16 [(Hq + 2 Hkv) * 128, D]; rope tables fp32 [S, 64]."""
    S, D = X.shape
    d = 128
    _check(X, "X", torch.bfloat16, (S, D))
    _check(W, "W", torch.bfloat16, ((Hq + 2 * Hkv) * d, D))
    if rope_cos is not None:
        _check(rope_cos, "rope_cos", torch.float32, (S, d // 2))
        _check(rope_sin, "rope_sin", torch.float32, (S, d // 2))
    dev = X.device
    o = {} if out is None else out
    mk = lambda key, shp, dt: o.setdefault(key, torch.empty(*shp, dtype=dt, device=dev))
    Q, K, V = mk("q", (Hq, S, d), torch.bfloat16), mk("k", (Hkv, S, d), torch.bfloat16), mk("v", (Hkv, S, d), torch.bfloat16)
    qb = mk("qbar", (Hq, S // b, d), torch.float32) if pooled else None
    kb = mk("kbar", (Hkv, S // b, d), torch.float32) if pooled else None
    i8 = [mk("q8", (Hq, S, d), torch.int8), mk("sq", (Hq, S), torch.float32), mk("k8", (Hkv, S, d), torch.int8),
          mk("sk", (Hkv, S), torch.float32), mk("v8", (Hkv, S, d), torch.int8),
          mk("sv", (Hkv, S), torch.float32)] if int8 else [None] * 6
    shape = shape_of(S, b, Hq, Hkv, d)
    rc = lib().fp_qkv_project(ctypes.byref(shape), D, _ptr(X), _ptr(W), _ptr(rope_cos), _ptr(rope_sin), _ptr(Q),
                              _ptr(K), _ptr(V), _ptr(qb), _ptr(kb), *[_ptr(t) for t in i8], _stream(stream))
    if rc:
        raise FpError(rc, "fp_qkv_project")
    return o


def index_pooled(Q: torch.Tensor, K: torch.Tensor, qbar: torch.Tensor, b: int, gamma: float, tau: float, *,
                 stats: bool = False, out: Optional[Index] = None, ws: Optional[Workspace] = None,
                 stream=None) -> Index:
    """fp_index_pooled: fp_index with the pooled query blocks qbar (fp32 [Hq, N, 128]) from upstream."""
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    shape = shape_of(S, b, Hq, Hkv, d)
    _check(Q, "Q", torch.bfloat16, (Hq, S, d))
    _check(K, "K", torch.bfloat16, (Hkv, S, d))
    _check(qbar, "qbar", torch.float32, (Hq, S // b, d))
    out = Index.empty(shape, Q.device, stats=stats) if out is None else out
    ws = _ws(shape, ws, Q.device)
    o = out.c_struct()
    rc = lib().fp_index_pooled(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(qbar), gamma, tau, ctypes.byref(o),
                               _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_index_pooled")
    return out


def index_shared(Q, K, b: int, gamma: float, tau: float, *, sQ=None, sK=None, stats: bool = False,
                 out: Optional[Index] = None, ws: Optional[Workspace] = None, stream=None) -> Index:
    """fp_index_shared: fp_index (bf16 Q, K) or fp_index_i8 (int8 Q, K with scales sQ, sK) with
    head-pattern sharing: heads of a KV group with the same pattern take the union of their rows."""
    return _index_variant("fp_index_shared", Q, K, b, gamma, tau, sQ, sK, stats, out, ws, stream)


def block_uses(idx: Index, *, heads: bool = True, stream=None):
    """fp_block_uses: (uses, head_uses) int32 [Hkv, N] -- job entries and (head, query block) pairs
    per key block of each KV group (head_uses is None when heads is False)."""
    sh = idx.shape
    N = sh.S // sh.b
    uses = torch.empty(sh.Hkv, N, dtype=torch.int32, device=idx.job_ptr.device)
    hu = torch.empty_like(uses) if heads else None
    o = idx.c_struct()
    rc = lib().fp_block_uses(ctypes.byref(sh), ctypes.byref(o), _ptr(uses), _ptr(hu), _stream(stream))
    if rc:
        raise FpError(rc, "fp_block_uses")
    return uses, hu



def build_jobs(shape: FpShape, row_ptr: torch.Tensor, col_idx: torch.Tensor, *,
               ws: Optional[Workspace] = None, stream=None) -> Index:
    """fp_build_jobs: job list from an existing CSR (e.g. one computed elsewhere)."""
    N = shape.S // shape.b
    dev = row_ptr.device
    _check(row_ptr, "row_ptr", torch.int32, (shape.Hq * N + 1,))
    if col_idx.dtype != torch.int32 or not col_idx.is_cuda or not col_idx.is_contiguous():
        raise TypeError("col_idx must be a contiguous int32 device tensor")
    out = Index.empty(shape, dev, col_cap=0)
    out.row_ptr = row_ptr
    out.col_idx = col_idx if col_idx.numel() > 0 else torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _ws(shape, ws, dev)
    o = out.c_struct()
    o.pattern = None
    o.jsd = None
    rc = lib().fp_build_jobs(ctypes.byref(shape), ctypes.byref(o), _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_build_jobs")
    return out


def attn(Q, K, V, idx: Index, *, out: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None,
         stream=None) -> torch.Tensor:
    """fp_attn: block-sparse causal attention (bf16) over idx's CSR."""
    shape = idx.shape
    _check(Q, "Q", torch.bfloat16, (shape.Hq, shape.S, shape.d))
    _check(K, "K", torch.bfloat16, (shape.Hkv, shape.S, shape.d))
    _check(V, "V", torch.bfloat16, (shape.Hkv, shape.S, shape.d))
    O = torch.empty_like(Q) if out is None else out
    _check(O, "O", torch.bfloat16, (shape.Hq, shape.S, shape.d))
    ws = _ws(shape, ws, Q.device)
    o = idx.c_struct()
    rc = lib().fp_attn(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(o), _ptr(O),
                       _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_attn")
    return O


class SplitWorkspace:
    """A device byte buffer sized by fp_attn_split_workspace_bytes."""

    def __init__(self, shape: FpShape, nsplit: int, nseg: int, device):
        n = ctypes.c_size_t(0)
        rc = lib().fp_attn_split_workspace_bytes(ctypes.byref(shape), nsplit, nseg, ctypes.byref(n))
        if rc:
            raise FpError(rc, "fp_attn_split_workspace_bytes")
        self.nbytes = n.value
        self.buf = torch.empty(max(self.nbytes, 1), dtype=torch.uint8, device=device)


def attn_split(Q, K, V, idx: Index, nsplit: int, nseg: int, *, out: Optional[torch.Tensor] = None,
               ws: Optional[SplitWorkspace] = None, stream=None) -> torch.Tensor:
    """fp_attn_split: the attention with the nsplit longest jobs cut into nseg split-KV segments whose
    partial results are merged by a keyed combine step (bf16, b >= 128)."""
    shape = idx.shape
    _check(Q, "Q", torch.bfloat16, (shape.Hq, shape.S, shape.d))
    _check(K, "K", torch.bfloat16, (shape.Hkv, shape.S, shape.d))
    _check(V, "V", torch.bfloat16, (shape.Hkv, shape.S, shape.d))
    O = torch.empty_like(Q) if out is None else out
    _check(O, "O", torch.bfloat16, (shape.Hq, shape.S, shape.d))
    ws = SplitWorkspace(shape, nsplit, nseg, Q.device) if ws is None else ws
    o = idx.c_struct()
    rc = lib().fp_attn_split(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(o), nsplit, nseg, _ptr(O),
                             _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_attn_split")
    return O


def attn_i8(Q8, sQ, K8, sK, V8, sV, idx: Index, *, out: Optional[torch.Tensor] = None,
            ws: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """fp_attn_i8: W8A8 block-sparse causal attention, bf16 output."""
    shape = idx.shape
    Hq, S, d, Hkv = shape.Hq, shape.S, shape.d, shape.Hkv
    _check(Q8, "Q8", torch.int8, (Hq, S, d))
    _check(K8, "K8", torch.int8, (Hkv, S, d))
    _check(V8, "V8", torch.int8, (Hkv, S, d))
    _check(sQ, "sQ", torch.float32, (Hq, S))
    _check(sK, "sK", torch.float32, (Hkv, S))
    _check(sV, "sV", torch.float32, (Hkv, S))
    O = torch.empty(Hq, S, d, dtype=torch.bfloat16, device=Q8.device) if out is None else out
    _check(O, "O", torch.bfloat16, (Hq, S, d))
    ws = _ws(shape, ws, Q8.device)
    o = idx.c_struct()
    rc = lib().fp_attn_i8(ctypes.byref(shape), _ptr(Q8), _ptr(sQ), _ptr(K8), _ptr(sK), _ptr(V8), _ptr(sV),
                          ctypes.byref(o), _ptr(O), _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_attn_i8")
    return O


def unpack(t: torch.Tensor, seqlens, H: int, d: int = 128) -> list:
    """Views [H, S_s, d] of the sequences packed one after another in t (no copy)."""
    views, off = [], 0
    for S in seqlens:
        n = H * int(S) * d
        views.append(t[off:off + n].view(H, int(S), d))
        off += n
    return views


def index_batch(Q: torch.Tensor, K: torch.Tensor, seqlens, b: int, Hq: int, Hkv: int, gamma: float,
                tau: float, *, d: int = 128, stats: bool = False, outs: Optional[list] = None,
                ws: Optional[Workspace] = None, stream=None) -> list:
    """fp_index_batch: one Index per sequence of a ragged batch; Q (K) holds the sequences'
    [Hq, S_s, d] ([Hkv, S_s, d]) bf16 blocks one after another, as 1-D tensors.  outs: the
    sequences' Index objects to write (e.g. with capacities of the caller's choice)."""
    lens = [int(S) for S in seqlens]
    tot = sum(lens)
    _check(Q, "Q", torch.bfloat16, (Hq * tot * d,))
    _check(K, "K", torch.bfloat16, (Hkv * tot * d,))
    if outs is None:
        outs = [Index.empty(shape_of(S, b, Hq, Hkv, d), Q.device, stats=stats) for S in lens]
    elif len(outs) != len(lens):
        raise TypeError("one Index per sequence is needed")
    shape = shape_of(max(lens), b, Hq, Hkv, d)     # S is ignored
    ws = _ws(shape, ws, Q.device, lens)
    arr = (FpIndexOut * len(lens))(*[o.c_struct() for o in outs])
    rc = lib().fp_index_batch(ctypes.byref(shape), len(lens), (ctypes.c_int32 * len(lens))(*lens), _ptr(Q),
                              _ptr(K), gamma, tau, arr, _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_index_batch")
    return outs


def attn_batch(Q, K, V, seqlens, idxs: list, *, out: Optional[torch.Tensor] = None,
               ws: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """fp_attn_batch: block-sparse attention of a ragged batch packed as for index_batch;
    returns O packed like Q."""
    lens = [int(S) for S in seqlens]
    if len(idxs) != len(lens):
        raise TypeError("one Index per sequence is needed")
    sh = idxs[0].shape
    Hq, Hkv, d, b, tot = sh.Hq, sh.Hkv, sh.d, sh.b, sum(lens)
    _check(Q, "Q", torch.bfloat16, (Hq * tot * d,))
    _check(K, "K", torch.bfloat16, (Hkv * tot * d,))
    _check(V, "V", torch.bfloat16, (Hkv * tot * d,))
    O = torch.empty_like(Q) if out is None else out
    _check(O, "O", torch.bfloat16, (Hq * tot * d,))
    shape = shape_of(max(lens), b, Hq, Hkv, d)
    ws = _ws(shape, ws, Q.device, lens)
    arr = (FpIndexOut * len(lens))(*[ix.c_struct() for ix in idxs])
    rc = lib().fp_attn_batch(ctypes.byref(shape), len(lens), (ctypes.c_int32 * len(lens))(*lens), _ptr(Q),
                             _ptr(K), _ptr(V), arr, _ptr(O), _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_attn_batch")
    return O


def index_i8_batch(Q8, sQ, K8, sK, seqlens, b: int, Hq: int, Hkv: int, gamma: float, tau: float, *,
                   d: int = 128, stats: bool = False, outs: Optional[list] = None, ws: Optional[Workspace] = None,
                   stream=None) -> list:
    """fp_index_i8_batch: index_batch for W8A8 inputs; Q8 / K8 int8 and their per-token scales
    sQ / sK fp32, each packed sequence after sequence as 1-D tensors."""
    lens = [int(S) for S in seqlens]
    tot = sum(lens)
    _check(Q8, "Q8", torch.int8, (Hq * tot * d,))
    _check(K8, "K8", torch.int8, (Hkv * tot * d,))
    _check(sQ, "sQ", torch.float32, (Hq * tot,))
    _check(sK, "sK", torch.float32, (Hkv * tot,))
    if outs is None:
        outs = [Index.empty(shape_of(S, b, Hq, Hkv, d), Q8.device, stats=stats) for S in lens]
    elif len(outs) != len(lens):
        raise TypeError("one Index per sequence is needed")
    shape = shape_of(max(lens), b, Hq, Hkv, d)
    ws = _ws(shape, ws, Q8.device, lens)
    arr = (FpIndexOut * len(lens))(*[o.c_struct() for o in outs])
    rc = lib().fp_index_i8_batch(ctypes.byref(shape), len(lens), (ctypes.c_int32 * len(lens))(*lens),
                                 _ptr(Q8), _ptr(sQ), _ptr(K8), _ptr(sK), gamma, tau, arr, _ptr(ws.buf),
                                 ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_index_i8_batch")
    return outs


def attn_i8_batch(Q8, sQ, K8, sK, V8, sV, seqlens, idxs: list, *, out: Optional[torch.Tensor] = None,
                  ws: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """fp_attn_i8_batch: W8A8 attention of a ragged batch packed as for index_i8_batch;
    returns bf16 O packed like Q8."""
    lens = [int(S) for S in seqlens]
    if len(idxs) != len(lens):
        raise TypeError("one Index per sequence is needed")
    sh = idxs[0].shape
    Hq, Hkv, d, b, tot = sh.Hq, sh.Hkv, sh.d, sh.b, sum(lens)
    _check(Q8, "Q8", torch.int8, (Hq * tot * d,))
    _check(K8, "K8", torch.int8, (Hkv * tot * d,))
    _check(V8, "V8", torch.int8, (Hkv * tot * d,))
    _check(sQ, "sQ", torch.float32, (Hq * tot,))
    _check(sK, "sK", torch.float32, (Hkv * tot,))
    _check(sV, "sV", torch.float32, (Hkv * tot,))
    O = torch.empty(Hq * tot * d, dtype=torch.bfloat16, device=Q8.device) if out is None else out
    _check(O, "O", torch.bfloat16, (Hq * tot * d,))
    shape = shape_of(max(lens), b, Hq, Hkv, d)
    ws = _ws(shape, ws, Q8.device, lens)
    arr = (FpIndexOut * len(lens))(*[ix.c_struct() for ix in idxs])
    rc = lib().fp_attn_i8_batch(ctypes.byref(shape), len(lens), (ctypes.c_int32 * len(lens))(*lens),
                                _ptr(Q8), _ptr(sQ), _ptr(K8), _ptr(sK), _ptr(V8), _ptr(sV), arr, _ptr(O),
                                _ptr(ws.buf), ws.nbytes, _stream(stream))
    if rc:
        raise FpError(rc, "fp_attn_i8_batch")
    return O


def probe_qk_i8(Q8, K8, b: int, h: int, i: int, j: int, path: int = PROBE_ATTN, stream=None) -> torch.Tensor:
    """fp_probe_qk_i8: exact int32 tile out[c, r] = Q8[h, i*b+r] . K8[h/G, j*b+c] through the staging
    and tile code of the attention kernel (PROBE_ATTN) or the statistics kernel (PROBE_STATS)."""
    Hq, S, d = Q8.shape
    shape = shape_of(S, b, Hq, K8.shape[0], d)
    _check(Q8, "Q8", torch.int8, (Hq, S, d))
    _check(K8, "K8", torch.int8, (K8.shape[0], S, d))
    out = torch.empty(b, b, dtype=torch.int32, device=Q8.device)
    rc = lib().fp_probe_qk_i8(ctypes.byref(shape), _ptr(Q8), _ptr(K8), h, i, j, path, _ptr(out), _stream(stream))
    if rc:
        raise FpError(rc, "fp_probe_qk_i8")
    return out
