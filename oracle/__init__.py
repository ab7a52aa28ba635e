"""CPU oracle for the CacheBlend blended prefill -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The GPU library never calls it and never falls back
to it.  It shares no code with the HIP path; its only shared dependency is the
seeded input module ``cbinputs``, which produces numbers, not results.

Sources ("the pages"):
  [CB]  "CacheBlend 完全拆解：RAG 多段 KV 缓存拼接，为什么还要重算一小部分 token"
        (pinghaoyang.com.cn) -- the method.
  [KV]  LMCache KV-cache essay (blog.thunguo.space), "KV 容量" formula S_token.
  [BI]  LMCache coordinator "Blend Index" article (nxmr.cn), section 6.2 -- the
        (chunk_hash, old_st, cur_st) match tuple: old_st is the re-RoPE source,
        cur_st the target; sections 3-7 -- fragment matching (``oracle/match.py``).

Precision: every computation runs in float32 (NumPy arrays, OpenBLAS sgemm);
the RoPE angles and their cos/sin are evaluated in float64 and rounded once to
float32.  Values the method *stores* (the KV cache, in the model's storage
dtype) are rounded to that dtype (bf16 = round to nearest even) at the point of
storage, exactly where the method writes them.  ``precision("f64")`` runs the
same code in float64; the tests use it only as an extra pin.
``operands("bf16")`` rounds the operands of every matrix product to bf16 (fp32
sums): the arithmetic of a bf16 model computed with bf16 operands.

Parity status of each function is listed in ``oracle/blend.py``; every function
there is pinned by at least one test under ``tests/`` that does not re-use the
oracle's own formulas (library special cases, closed forms, brute force).
"""
from .blend import (  # noqa: F401
    OracleModel, precision, operands, ct, store_round, rms_norm, rope_cos_sin, rope, rerope, causal_attention,
    swiglu_mlp, kv_deviation, select_hkvd, full_prefill, chunk_prefill,
    assemble_blended, full_reuse_prefill, blend_prefill, blend_prefill_masked,
    blend_layer, flop_count, decode_step,
)
from .match import POLY_BASE, UNKNOWN_TOKEN_OFFSET  # noqa: F401  (the matcher itself: oracle.match)
