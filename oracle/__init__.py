"""Oracle for the dynamic block-sparse prefill path: plain, slow, float64, CPU only.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path (the HIP
library and its Python binding) never does, and shares no code with it.

Sources: the FAST-Prefill explainer ("FPGA24成果：FAST-Prefill稀疏注意力加速器",
yunpan.plus) sections 1.1-1.2 and 3.1-3.3, and the re-telling
("FPGA加速动态稀疏注意力技术解析与优化", maplevalley.com.cn) sections 1.1 and
3.2-3.3.  The pages leave Flex-Prefill's exact statistics, divergence and
selection rule unwritten; the readings taken here are listed per function.

Modules:
  index  -- last-block statistics, divergence test, cumulative selection, CSR rows
  attn   -- block-sparse causal attention over a CSR (bf16-valued and W8A8 inputs)
  brute  -- independent brute-force forms used only to pin the two modules above
  project -- the QKV projection with the rotary embedding, block means and int8 codes its
             epilogue emits
"""
from . import index, attn, brute, project  # noqa: F401
