"""CPU oracle for the target model's verification step of speculative decoding.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the GPU library.

It is a plain, slow, obviously-correct NumPy implementation of what one
verification pass computes, written from the pages' description of the
method:

* the block forward pass -- one target pass over [pending, d_1..d_k] gives
  k+1 rows of logits, row j being what the target would write after block
  token j (essay "LLM Inference: Speculative Decoding", section "The loop",
  step 2; nesting argument in "The four sentences are already inside one
  sentence");
* greedy acceptance -- longest agreeing prefix, then the target's own token
  (same essay, "The loop", steps 3-4; "The output does not change");
* stochastic acceptance -- the Leviathan et al. rule the essay names in
  "What is not here" (accept with prob. min(1, p/q), else resample from the
  normalized positive part of p - q);
* KV commit / rollback -- only accepted entries survive (essay, "The loop",
  step 5; S2-MoE section 4.3 "Context-aligned Self-speculative");
* the MoE union of experts for a verification block (S2-MoE section 3,
  Challenge 2, and section 2.1).

Floating point is float64 unless a caller asks for float32 (used only to
prefill long prompt caches quickly; the prefilled values are inputs).

Modules: numerics (elementwise definitions), model (block forward, prefill,
autoregressive decode), accept (acceptance rules and near-tie flags),
accounting (the essay's per-run counters and the expected-tokens formula).
"""
