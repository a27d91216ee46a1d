"""CPU oracle for block-sparse attention with pooled block routing.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
anything in this package: only the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark call it.  It shares no code with the HIP
path (no kernels, helpers, tables or pre/post-processing); the two meet only in
the seeded input draws of the ``synth`` package.

Everything is plain numpy in float64.  Each function cites the passage of the
source pages it follows:

* "PISA explainer" -- the Korean blog post on PISA (Piecewise Sparse
  Attention) at kodorricoding.tistory.com/108;
* "FlashAttention tutorial" -- "플래시 어텐션 — IO를 아는 어텐션"
  (blog.mna-game.duckdns.org, post 22);
* "FlashPrefill summary" -- "FlashPrefill: Instantaneous Pattern Discovery and
  Thresholding for Ultra-Fast Long-Context Prefilling" (gist.science/ko/paper/
  2603.06199), technical summary section 2.

Pin status (what ties each function to something other than itself):

* pooling, block scores: pinned (2D-reduction identity against a full token
  score matrix; brute-force loops);
* selection (alpha threshold, top-k at a density): pinned by invariants
  (argmax always kept, exact count, ordering property of top-k, positive-scale
  invariance, alpha=1 keeps the argmax set) and brute force.  The pages print no
  worked selection example, so the *readings* of the threshold rule (raw pooled
  logits, non-positive row maxima, >= at the threshold, count rounding, tie
  order) are pinned to those readings only;
* attention with the 0th-order tail: pinned (density 1 equals dense softmax
  attention from a library routine; identical keys inside every block make the
  tail exact; online recurrence equals the closed form; hand-derived closed-form
  cases; brute force);
* gradients of the attention step (``backward``): pinned by central finite
  differences of the forward on small inputs (exact keys and the tail, causal,
  grouped queries, ragged blocks) and, for density 1, by torch's autograd of
  dense softmax attention.
"""

from .reference import (  # noqa: F401
    attend_block,
    attend_block_grad,
    backward,
    band_mask,
    block_bounds,
    block_scores,
    block_sizes,
    eligible_mask,
    forward,
    kv_group,
    mask_to_lists,
    pool_mean,
    pool_sum,
    select,
    select_alpha,
    select_density,
    thresholds,
    topk_count,
)
