"""fp64 CPU oracle for batched attention over a paged / block-sparse KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library (no headers, helpers, tables or
constants) and never takes an input or an expected value from it.

Sources (the pages are cited by title and section):

* [FI-paper]  "FLASHINFER: EFFICIENT AND CUSTOMIZABLE ATTENTION ENGINE FOR LLM
  INFERENCE SERVING" (blog summary of the FlashInfer paper) -- sections
  "Results" (end-to-end and kernel level) and "Research methodology"
  items 1 (unified block-sparse KV format, composable formats), 2
  (attention templates) and 3 (dynamic load-balanced scheduling).
* [FI-0.6]    "FlashInfer 0.6: JIT compilation, MLA, MoE EP, Blackwell" (wiki
  page) -- sections "Background: the decode bottleneck", "Architecture"
  item 1 (block-sparse KV format, page indices prefetched into shared
  memory), "Kernel types" (Decode, Prefill incl. chunked prefill, the
  Blackwell CuTe-DSL GQA decode with sliding-window and attention-sink
  masking, split-KV).
* [FI-PR5329] "FlashInfer BatchAttention: K/V stride optimisation" (analysis
  of PR #5329) -- sections "Code analysis" 1 (persistent BatchAttention
  kernel, two tile classes, plan_info grid) and 2 (plan/run API with float
  and int workspaces, q, kv cache, out, lse).

The pages name the operations but print no formulas.  Where they leave a
step open the oracle takes the plainest reading (standard scaled
dot-product softmax attention, natural-log LSE, rotate-half RoPE, ...);
each reading is stated at the function that takes it.

Every function here is pinned by ``tests/test_oracle.py`` against
something other than itself (library routines, closed forms, invariants,
brute force); see each docstring.
"""
from .attention import (attention, attention_partial, gather_kv, merge, rope_rotate,
                        visible, key_positions, composable, flat_from_composable, round_to_bf16,
                        attention_rope_stored)
from .plan import plan_ref, PlanParams, PlanError
from .append import append_paged_kv

__all__ = ["attention", "attention_partial", "gather_kv", "merge", "rope_rotate", "visible",
           "key_positions", "composable", "flat_from_composable", "round_to_bf16",
           "attention_rope_stored", "plan_ref", "PlanParams", "PlanError",
           "append_paged_kv"]
