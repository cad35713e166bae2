"""SCE bucket-variant oracle, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The SCE page (abstract) approximates the softmax over the catalogue by a subset
of the model outputs found through maximum inner product search, without
printing the procedure.  What is computed here is the bucket variant of that
idea as the workload fixes it: n_b random projection vectors (buckets); each
bucket takes the b_x positions and the b_y items with the largest projection
scores, computes the logits between them, and each position keeps its k largest
negatives over all the buckets that took it, duplicates merged.

Readings (each listed with its reason in the design notes of the repository):
  * scores and logits are float64 sums of the d coordinate products in index
    order, as in the RECE oracle;
  * projection scores are signed; a bucket takes the b_x (b_y) largest by
    (score descending, index ascending);
  * within a bucket the position's own positive item is excluded;
  * the position's negatives are the k largest by (logit descending, item id
    ascending) over the union, without duplicates, of the items of the buckets
    that took it (one round);
  * a position taken by no bucket has no negatives: its loss is 0;
  * the loss is the mean over positions; gradients hold the selection fixed.

Parity unpinned: the SCE page's own algorithm (its exact steps are not on the
pages).  Pinned are the reductions to full cross-entropy, a brute-force
recomputation on tiny inputs and the invariants (see the oracle tests).
"""
from __future__ import annotations

import numpy as np

from .rece import logsumexp, rece_backward, seq_dot

__all__ = ["projection_scores", "column_top", "bucket_lists", "bucket_negatives",
           "merge_negatives", "sce_forward", "sce_backward"]


def projection_scores(V, B) -> np.ndarray:
    """scores[n, b] = v_n . B[:, b] for B of shape [d, n_b] (float64, coordinate order)."""
    return seq_dot(V, np.asarray(B, dtype=np.float64).T)


def column_top(col, b: int) -> np.ndarray:
    """Indices of the b largest entries of one score column, order (score desc,
    index asc), returned as a set in ascending index order.  All when b >= len."""
    col = np.asarray(col, dtype=np.float64)
    n = col.shape[0]
    if b >= n:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -col))   # primary: score desc; then index asc
    return np.sort(order[:b]).astype(np.int64)


def bucket_lists(X, Y, B, b_x: int, b_y: int):
    """R[b] (positions) and Q[b] (items) taken by every bucket b."""
    PX = projection_scores(X, B)
    PY = projection_scores(Y, B)
    n_b = PX.shape[1]
    R = [column_top(PX[:, b], b_x) for b in range(n_b)]
    Q = [column_top(PY[:, b], b_y) for b in range(n_b)]
    return R, Q


def _top_k(ids, logits, k):
    """The k largest (logit desc, id asc), or all of them; sorted in that order."""
    order = np.lexsort((ids, -logits))
    keep = order[:k] if k < len(order) else order
    return ids[keep], logits[keep]


def bucket_negatives(X, Y, pos, R, Q, k: int) -> dict:
    """Per bucket and taken position: the top-k of the bucket's items (positive excluded).

    Returns {(b, i): (ids, logits, n)} with n the number of candidates the bucket
    offered.  Keeping only a bucket's top-k loses nothing: a member of the top-k
    over a union is in the top-k of every part containing it.
    """
    out = {}
    for b in range(len(R)):
        items = Q[b]
        if len(R[b]) == 0:
            continue
        L = seq_dot(X[R[b]], Y[items])
        for n, i in enumerate(R[b]):
            m = items != pos[i]
            out[(b, int(i))] = _top_k(items[m], L[n][m], k) + (int(m.sum()),)
    return out


def merge_negatives(per_bucket: dict, s: int, k: int):
    """N_i: the top-k over the duplicate-free union of a position's bucket lists.

    Returns {i: (ids, logits, thr)} with thr = (id, logit) of the k-th kept pair,
    None when the union of the candidates has at most k members (every one kept).
    The union exceeds k when the pruned union does or some bucket offered more
    than k candidates."""
    acc, cut = {}, set()
    for (b, i), (ids, lg, n) in per_bucket.items():
        d = acc.setdefault(i, {})
        for j, l in zip(ids.tolist(), lg.tolist()):
            d[j] = l        # the same pair has the same float64 logit in every bucket
        if n > k:
            cut.add(i)
    out = {}
    for i in range(s):
        d = acc.get(i, {})
        ids = np.array(sorted(d), dtype=np.int64)
        lg = np.array([d[j] for j in ids.tolist()], dtype=np.float64)
        kid, kl = _top_k(ids, lg, k)
        thr = (int(kid[-1]), float(kl[-1])) if ((len(ids) > k or i in cut) and k > 0) else None
        out[i] = (kid, kl, thr)
    return out


def sce_forward(X, Y, pos, B, b_x: int, b_y: int, k: int, ignore_negative: bool = False) -> dict:
    """SCE bucket-variant loss; B has shape [d, n_b].  The result uses the same
    keys as the RECE oracle (one round), so its backward applies unchanged.
    ``ignore_negative``: positions with a negative positive id are padding, taken
    by buckets like any other row (nothing excluded from their candidates), with
    loss 0 and outside the mean."""
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    s = X.shape[0]
    R, Q = bucket_lists(X, Y, B, b_x, b_y)
    negs = merge_negatives(bucket_negatives(X, Y, pos, R, Q, k), s, k)
    rows = np.arange(s)
    pad = np.array([bool(ignore_negative) and pos[i] < 0 for i in rows], dtype=bool)
    l_pos = np.array([0.0 if pad[i] else seq_dot(X[i], Y[pos[i]][None, :])[0, 0] for i in rows])
    lse = np.array([logsumexp(np.concatenate([[l_pos[i]], negs[i][1]])) for i in rows])
    loss = np.where(pad, 0.0, lse - l_pos)
    union = [negs[i][0] for i in rows]
    mult = [np.ones(len(u), dtype=np.int64) for u in union]
    counted = int(np.sum(~pad))
    return {"R": R, "Q": Q, "negs": [negs], "rows": rows, "l_pos": l_pos, "lse": lse,
            "loss_pp": loss, "union": union, "mult": mult, "pad": pad,
            "loss": float(np.sum(loss) / counted) if counted else 0.0}


def sce_backward(X, Y, pos, fwd: dict, dloss: float = 1.0, dloss_pp=None):
    """Gradients with the selection fixed: Eq. 4 of the RECE page over {positive} + N_i."""
    return rece_backward(X, Y, pos, fwd, dloss=dloss, dloss_pp=dloss_pp)
