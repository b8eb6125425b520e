"""CPU oracle for Twilight-style top-p sparse decode attention.  TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct numpy implementation of every step of the
select-then-prune decode path.  Only the tests, the smoke check and the bench's ``cpu_baseline`` leg
may import it; the product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product path.  The two share no code: only the seeded input
generators in ``gen/`` serve both.

Sources (the pages this follows; cited by title and section):

* "Twilight: Adaptive Attention Sparsity with Hierarchical Top-p Pruning", Paper-Notes summary
  (NeurIPS 2025) -- sections "整体框架" (framework), "关键设计" (key design: oracle top-p
  formulation, error bound, binary-search top-p, 4-bit K cache, load balancing), "局限与展望".
* The paperlayer.ai summary of arXiv 2502.02770v5 -- §3.1, §3.2, §4.1 (Fig. 5), §4.2 (Fig. 6),
  §4.3, §B.1 (Fig. 12), §B.2 (Fig. 13).
* "Double-P: Hierarchical Top-P Sparse Attention for Long-Context LLMs" (shd-paper.top summary) --
  "方法详解" (cluster-level top-p on size-weighted centroids, then token-level top-p).

Precision: float64 wherever the pages leave the precision open.  Two steps are encodings or
heuristics whose exact floating-point arithmetic is itself the specification, because an integer or a
set is decided from them on both sides (quantisation codes, page scores, estimated logits, cluster
logits): those are written as explicit float32 operation sequences that numpy evaluates one IEEE
operation at a time.  Each such function says so and is pinned against its float64 definition.

Modules:
  numerics   bit-level conversions (bf16, fp16) and an fp32 order-preserving key
  quantize   O1 INT4 K quantisation, O2 page key bounds
  select     O3 Quest-style page scores and top-K page selection, O4 candidate lists
  estimate   O5 INT4 logit estimate, O6 softmax weights
  topp       O7 minimal top-p set (sort-based), ambiguity sets, bisection model
  attention  O8 GQA union, O9 sparse attention, O10 dense attention and the (1-p)||V||_F bound
  doublep    O11 cluster-level then token-level top-p
  pipeline   the whole decode step composed from the above
"""

from . import numerics, quantize, select, estimate, topp, attention, doublep, pipeline  # noqa: F401
