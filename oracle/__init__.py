"""FP64 CPU oracle for exact streaming attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything in this package; only the
tests, the smoke check and the benchmark's CPU-baseline leg do.

Two independent references live here and share no code with each other or
with the HIP path:

* ``oracle.dense``  -- numpy float64, the plain dense definition
  O = softmax(scale * Q K^T [+ causal mask]) V with a natural-log logsumexp,
  plus the plain definitions of the split-KV partial states and their merge.
* ``oracle.backward`` -- numpy float64 gradients (dQ, dK, dV) of the loss
  sum(dO * O), from the softmax row derivative; grouped KV heads sum their
  query heads' gradients.
* ``oracle.online`` -- standard library only (``math``), the mergeable
  (running max m, rescaled exp-sum l, rescaled numerator acc) state with an
  explicit empty identity.

Sources (pages, by title and section):
  * "Intermediate and advanced extension", workshop table (online normalization
    row: mergeable (maximum, exponential sum) state with partition and
    merge-order invariance; streaming attention row: the score and value
    products tile by tile under a running rescale, causal or not) and "Logic review before implementation"
    (a state with no keys yet, whose maximum is -inf, is a special case of its
    own; the output sum is scaled together with the exponential sum; a causal
    row sees the key at its own position).
  * "Intermediate and advanced workshop validation", "Correctness and review"
    (dense FP64 references, future-value perturbation, large-logit cases,
    explicit empty+empty identity).
  * "Attention algorithms and data movement", lessons 01 (tile outputs are
    combined through their rescaled sums, never averaged; a defined result for a row with no key),
    03 (saved normalization state), 04 (packed causal eligibility from logical
    positions), 05 (GQA query-head to KV-head mapping).

Every function is pinned by CPU tests (tests/test_oracle_*.py) to closed
forms, invariants, hand-derived golden cases and independent library routines
(torch CPU float64 scaled_dot_product_attention, torch.logsumexp).
"""
