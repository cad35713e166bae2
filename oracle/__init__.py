"""CPU oracle for the RECE / SCE reduced cross-entropy loss (forward and backward).

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 NumPy written from the pages'
definitions.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the GPU library and its
Python binding never do, and this package imports nothing from them.

Sources (the page is "RECE: Reduced Cross-Entropy Loss for Large-Catalogue
Sequential Recommenders", arXiv 2408.02354, ar5iv rendering):
  * Eq. (3) full cross-entropy and Eq. (4) its gradient (Section 3);
  * Algorithm 1 (Section 3) and the method paragraph before it: random vectors,
    argmax bucketing, argsort, n_c equal chunks, current-plus-adjacent chunk
    window, in-chunk logits, positive logit, per-position loss, mean;
  * the same paragraph's rounds r with the "minus ln(count)" duplicate rule.
SCE ("Scalable Cross-Entropy Loss for Sequential Recommendations with Large
Item Catalogs", abstract only) is the bucket variant in ``oracle.sce``.

Parity unpinned: the SCE bucket variant's exact procedure (the SCE page gives
only its idea), see ``oracle.sce``.
"""
from .rece import (  # noqa: F401
    seq_dot, bucket_scores, bucket_ids, stable_argsort, chunk_of, chunk_bounds, chunk_members,
    window_chunks, round_negatives, rece_forward, loss_from_negatives, rece_backward, full_ce,
    full_ce_grad, logsumexp,
)
from .sce import (  # noqa: F401
    projection_scores, column_top, bucket_lists, bucket_negatives, merge_negatives,
    sce_forward, sce_backward,
)
