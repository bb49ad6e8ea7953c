"""CPU oracle for the routed-MoE + Engram hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 NumPy restatement of what the hot path
computes.  It exists to check the HIP library, nothing else: only the test
suite, the smoke check and the bench's CPU-baseline leg may import it.  The
product path (``bit_moe_amd``) never imports it, and it never imports the
product path; the two share no code.  The seeded input generators live in
``synthdata`` and hold none of the method's arithmetic.

Sources (web pages on the subject; citations name page and section):

* "Feature Request: support DeepSeek V4.1 Flash with bounded SSD expert
  caching" (strix-llama.cpp issue 48) -- §Feature Description (Q2_K / Q8_0
  formats, 264-byte Engram rows of 256 E4M3 values + 8 E8M0 scales),
  §Possible Implementation (rows decoded straight to BF16),
  §Engram graph integration, §Runtime stack progress (single expert
  reduction order).
* "Strata-DSV4.1" README -- §DeepSeek-V4.1-Flash (384 experts, top-6),
  §Results / §How it works (shared expert + routed sum, verify-batch union).
* "run the DeepSeek-V4-Flash-Vision tower on CUDA" (vllm.cpp PR) -- commit
  notes on SwiGLU operand order (gate first) and the 34-byte Q8_0 block.

Readings taken where the pages are silent are stated in each function's
docstring.

Modules
-------
formats  -- Q2 super-block / Q8_0 dequantisation, E4M3, E8M0, BF16 rounding
moe      -- router, top-k, plan, expert FFN, combine, brute-force dense MoE
engram   -- Engram row decode (gather)
engram_inject -- Engram KV projection and gated injection into the residual branches
int8_mode -- int8 activation numerics of the expert FFN (block quantiser, integer row dots)
compare  -- parity comparators (tie-aware ids, tolerance, NaN = failure)

Parity status per function is stated in its docstring.  The pins are the
``-m "not gpu"`` tests in tests/test_oracle_*.py: closed forms, hand-worked
cases with literal expected values, brute force and independent library
routes.  The MoE outputs themselves have no value printed on the pages
("parity unpinned" by the pages); they are pinned by construction (the
brute-force dense layer and special cases that reduce to textbook routines).
"""
