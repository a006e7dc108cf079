"""fp64 CPU oracle — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the GPU path
computes, used to judge it.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package; the product path
(``logits_parity_amd``) never does, and it shares no code with it.  The only
thing both sides share is the seeded input module ``synth`` (bytes, no
arithmetic).

Modules
  prefill  Phi-3-style decoder prefill, ids -> per-position logits (fp64).
  decode   K16/V8 paged decode attention and KV-pool sizing (fp64).
  parity   per-position cosine and argmax agreement with top-2 gaps.

Sources: the pages "Phi-3-mini: fused-tensor direct loading in a sovereign
inference engine" (P1), "The direct HF-logits parity harness" (P2) and
"Phi-4: quality transfer and interrupted throughput studies" (P3).  Each
function names the passage it follows.

Parity status: every function here is pinned by tests under ``tests/``
(test_oracle_*.py) against the HuggingFace transformers Phi-3 forward, torch's
fp64 scaled-dot-product attention, torch's float8_e4m3fn decoding, closed
forms, invariants, and the KV-pool numbers printed on P3.
"""
