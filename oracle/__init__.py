"""Plain fp64 CPU oracle for the Compressed Sparse Attention (CSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or constant generators) and imports
nothing from it.  The only module both sides use is ``workloads`` (seeded
synthetic inputs, which holds none of the method's arithmetic).

Sources (web pages describing DeepSeek-V4; cited by title and section):

* "DeepSeek V4: Compressed Sparse Attention and the Million-Token Context"
  (octagono.org), section "Hybrid Attention: CSA and HCA".
* "DeepSeek AI Releases DeepSeek-V4: Compressed Sparse Attention and Highly
  Compressed Attention Enable Million Token Content" (dataforcee.us),
  sections "Hybrid Attention: CSA and HCA" and "Muon Optimizer and FP4 QAT".
* "DeepSeek V4 technical review" (takeshell.com), section 2.1 "CSA
  (Compressed Sparse Attention)", 2.2 "HCA", 5 "FP4 Quantization-Aware
  Training".
* "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence"
  (agihunt.info paper summary), the hybrid-attention paragraph.

Where the pages leave a step open the oracle takes one stated reading; every
such reading is listed in the repository's design notes.

Pinning status: every public function here is pinned by the ``-m "not gpu"``
tests (closed forms, special cases that reduce to library routines, brute
force on tiny inputs, hand-worked fixtures under ``tests/golden/``).
"""

from .codecs import (
    bf16_decode,
    e4m3_decode,
    e4m3_encode,
    quantize_fp8_rows,
    e2m1_decode,
    e2m1_encode,
    e8m0_decode,
    quantize_mxfp4_rows,
    mxfp4_decode_rows,
)
from .csa import (
    visible_count,
    compress,
    indexer_scores,
    topk_select,
    attend,
    hca_indices,
    hca_attend,
    csa_forward,
)
from .backward import attend_backward, hca_attend_backward, compress_backward

__all__ = [
    "bf16_decode",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_fp8_rows",
    "e2m1_decode",
    "e2m1_encode",
    "e8m0_decode",
    "quantize_mxfp4_rows",
    "mxfp4_decode_rows",
    "visible_count",
    "compress",
    "indexer_scores",
    "topk_select",
    "attend",
    "hca_indices",
    "hca_attend",
    "csa_forward",
    "attend_backward",
    "hca_attend_backward",
    "compress_backward",
]
