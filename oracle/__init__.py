"""CPU oracle for the sparse FP4-KV decode path (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, obviously-correct statement of what the GPU
library computes.  It exists to check the GPU kernels; it is not part of the
product.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The GPU library never calls it and shares no
code with it: every format routine here (E2M1 / E4M3 encode and decode, the
pack, the scores, the selection, the attention) is written independently of the
HIP sources.

All floating-point reference arithmetic is float64 (numpy) unless the method
itself fixes a precision (the E4M3 scale is computed from an fp32 quotient, and
the E2M1 decision compares fp32 inputs against exact thresholds).

Sources (web pages on DeepSeek-V4.1-Flash; cited by page and section):
  [P1] discuss.pytorch.kr, "DeepSeek-V4.1-Flash, KV 캐시를 토큰당 890바이트로 줄이고 ..."
       sections: "Causal Encoder-Decoder" (CED formula), "CSA2" (mode table and
       layer layout), "Hierarchical Sparse Indexer", "FP4 KV cache" (format and
       range argument), "why the KV cache became the bottleneck" (bytes/token
       history).
  [P3] llmfeed.kr news summary, section "규모와 구조" (scale and structure).
  [P4] ingu627.github.io asymmetric-serving blog, sections 2 (CED split,
       config numbers) and 3 (KV cache compression).

Modules:
  fp4        E2M1 / E4M3FN definitions, the per-16-channel pack and its inverse.
  ced        the CED projection C_l = H W_l^KV, Z_l = H W_l^Z (+ fused pack).
  indexer    indexer scores, top-K, the hierarchical block pool, Reindex, Reuse.
  attention  sparse decode attention over dequantized FP4 entries.
  paged      paged-cache addressing and the bytes-per-token arithmetic.
  latent     RMSNorm + RoPE of a KV latent before the pack, and the indexer key
             projected from the cached entry.
  swa        the sliding-window branch: FP8 window entries and the merge with the
             global branch.

Parity status of every function is stated in its docstring; the pins live in
``tests/test_oracle_*.py`` and ``tests/golden/``.
"""

from . import fp4, ced, indexer, attention, paged, latent, swa  # noqa: F401
