"""CPU oracle for exact Lookahead decoding -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the packed
lookahead + verification step computes.  It follows the pages in their order
and notation:

* "M7.3 - Lookahead Decoding: Jacobi Iterations, N-Gram Pools, and Parallel
  Verification" (the primary specification: window, pool, packed rows and
  branch visibility, greedy and one-hot sampling verification, publication);
* "Break the Sequential Dependency of LLM Inference Using Lookahead Decoding"
  (paper summary: lossless claim, G = W practice, expected-accepted model);
* "Speculative Decoding" lesson, Chapters 1-2 (general p/q rejection
  sampling, the three-token vocabulary, the acceptance-rate arithmetic) and
  Chapter 7 (speculation under batch occupancy).

Floating point is fp64 except where the method fixes a storage precision
(the model's storage dtype at every stored activation, float32 logits).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP path and imports
nothing from it; the only common dependency is the seeded input generator
module `synthetic`, which holds none of the method's arithmetic.

Parity status per module:
  numerics, rows, window, pool, commit, verify, philox, jacobi, acceptance,
  attention -- pinned by page values, closed forms or brute force in
  tests/test_oracle_*.py.
  model -- the pages print no activations; pinned by a second, independent
  fp64 forward written in torch (tests/test_oracle_forward_torch.py: bit-equal
  K/V and logits within one fp32 rounding on tiny, small bf16 GQA and
  7B-width rounds), by textbook identities (softmax attention against an
  explicit loop, RoPE rotation invariants, RMSNorm scale invariance) and by
  the separate-forwards == dense-mask == autoregressive equalities.
  batch -- the occupancy throttle ("Speculative Decoding" lesson, Chapter 7);
  plan_rows pinned by closed forms for uniform requests, the chapter's worked
  numbers and its defining properties (tests/test_oracle_batch.py); its
  rounds are decode.LookaheadRequest's.
"""
