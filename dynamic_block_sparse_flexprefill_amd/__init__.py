"""Dynamic block-sparse prefill attention (Flex-Prefill's method, as the
FAST-Prefill write-ups describe it) for AMD MI355X / gfx950.

Two calls, both HIP kernels in libfpattn.so behind the C ABI of
include/fpattn.h:

  index(Q, K, b, gamma, tau)   -> Index  (per-head pattern, divergence, CSR of
                                          key blocks, grouped-query job list)
  attn(Q, K, V, index)         -> O      (block-sparse causal attention, bf16)

plus their W8A8 forms index_i8 / attn_i8, and index_batch / attn_batch (and
index_i8_batch / attn_i8_batch) for ragged batches of sequences packed one
after another.  This package only marshals
arguments; there is no CPU path.
"""
from .binding import (  # noqa: F401
    FP_OK, FP_EINVAL, FP_EUNSUPPORTED, FP_EWORKSPACE, FP_ECAPACITY, FP_EHIP, FP_EJOBCAPACITY,
    FP_ETIMEOUT, FP_ESCRATCH, FP_STATUS_CSR_OVERFLOW, FP_STATUS_JOB_OVERFLOW, FP_STATUS_WAIT_TIMEOUT,
    VERTICAL_SLASH, QUERY_AWARE, PROBE_ATTN, PROBE_STATS, FpError, FpShape, FpIndexOut, Index, Workspace,
    lib, strerror, shape_of, workspace_bytes, batch_workspace_bytes, csr_capacity, job_capacity,
    index, index_i8, index_pooled, qkv_project, index_static, index_shared, block_uses, build_jobs, attn, attn_split, SplitWorkspace, attn_i8, probe_qk_i8, LIB_PATH,
    index_batch, attn_batch, index_i8_batch, attn_i8_batch, unpack,
)
