"""RECE oracle: the RECE page's method (Section 3, Algorithm 1), step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows the RECE page (Section 3, Algorithm 1): positions (batch and
sequence collapsed) are the rows of X (s of them), items the rows of Y (C of
them), a logit is the scalar product of a position row and an item row, pos
holds each position's positive (next-item) id, B holds n_b random vectors, n_c
is the number of chunks, n_ec the neighbouring chunks on each side of a window,
r the number of rounds.

Readings of points the page leaves open (each is listed with its reason in the
design notes of the repository):
  * every scalar product is the float64 sum of the d coordinate products taken in
    index order (Algorithm 1 writes the positive logit as exactly this sum);
    products of float32 / bfloat16 inputs are exact in float64;
  * bucket = argmax of the signed score b.x over b, lowest index on ties;
  * argsort is stable and ascending;
  * chunk c of N sorted elements holds the slots p with c*N/n_c <= p < (c+1)*N/n_c,
    read over the rationals (sizes differ by at most one);
  * the window of chunk c is the set of chunks c-n_ec .. c+n_ec (n_ec = 1: the
    current and the two adjacent chunks); cyclic reading: indices taken modulo
    n_c, so 2*n_ec + 1 >= n_c gives the whole catalogue; clipped reading
    (wrap=False): only the chunks inside [0, n_c);
  * only wrong classes are negatives: the position's own positive item is excluded;
  * per position, per round, the k largest window logits are kept, order
    (logit descending, item id ascending); all are kept when there are <= k;
  * rounds use independent random vectors; a pair kept in n rounds enters the
    loss n times with its logit reduced by ln(n) (the page's duplicate rule);
  * the positive logit uses the original item id of the positive;
  * the loss is the mean over all positions (Algorithm 1, last line);
  * gradients are those of the loss with the selection held fixed (the argmax,
    argsort and top-k steps are piecewise constant); B is not learned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "seq_dot", "bucket_scores", "bucket_ids", "stable_argsort", "chunk_of",
    "chunk_bounds", "chunk_members", "window_chunks", "round_negatives",
    "rece_forward", "loss_from_negatives", "rece_backward", "full_ce", "full_ce_grad",
    "logsumexp",
]


def seq_dot(A, Bm, block_elems: int = 1 << 22) -> np.ndarray:
    """out[i, j] = sum over t = 0..d-1 of A[i, t] * Bm[j, t], float64, in index order t.

    RECE page, Section 3: a logit is the scalar product of a position's hidden
    state and an item embedding; Algorithm 1 writes the positive logit as the sum
    of the d coordinate products, which is the order taken here.
    """
    A = np.asarray(A, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    if A.ndim == 1:
        A = A[None, :]
    n, d = A.shape
    m = Bm.shape[0]
    assert Bm.shape[1] == d
    out = np.empty((n, m), dtype=np.float64)
    rows = max(1, block_elems // max(m, 1))
    for r0 in range(0, n, rows):
        a = A[r0:r0 + rows]
        acc = np.zeros((a.shape[0], m), dtype=np.float64)
        for t in range(d):
            acc += a[:, t:t + 1] * Bm[None, :, t]
        out[r0:r0 + rows] = acc
    return out


def bucket_scores(V, B_round) -> np.ndarray:
    """Scores b . v for every row v of V and every random vector b.

    B_round has shape [d, n_b]; its column b is one random vector (RECE page,
    Algorithm 1: n_b Gaussian vectors of dimension d are drawn, and every position
    and item is scored against each of them).
    """
    return seq_dot(V, np.asarray(B_round).T)


def bucket_ids(V, B_round) -> np.ndarray:
    """Index of the random vector with the largest scalar product (ties: lowest index).

    RECE page, Section 3 (method paragraph) and Algorithm 1, the two indexing
    steps: each position and each item is labelled with the random vector nearest
    to it by scalar product.
    """
    return np.argmax(bucket_scores(V, B_round), axis=1).astype(np.int64)


def stable_argsort(keys) -> np.ndarray:
    """Order of the elements by bucket label (RECE page, Algorithm 1, the two sorting
    steps); read as a stable ascending argsort."""
    return np.argsort(np.asarray(keys), kind="stable").astype(np.int64)


def chunk_bounds(N: int, n_c: int) -> np.ndarray:
    """Start slots of the n_c chunks (plus N at the end).

    RECE page, Algorithm 1, the chunk step: the sorted order is cut into n_c equal
    chunks, chunk c holding the slots p with c*N/n_c <= p < (c+1)*N/n_c; the
    smallest such p is ceil(c*N/n_c).
    """
    c = np.arange(n_c + 1, dtype=np.int64)
    return (c * N + n_c - 1) // n_c


def chunk_members(c: int, N: int, n_c: int) -> np.ndarray:
    """Sorted slots of chunk c, straight from the inequality c*N/n_c <= p < (c+1)*N/n_c."""
    p = np.arange(N, dtype=np.int64)
    return np.nonzero((c * N <= p * n_c) & (p * n_c < (c + 1) * N))[0]


def chunk_of(p, N: int, n_c: int):
    """Chunk of sorted slot p: the c with c*N/n_c <= p < (c+1)*N/n_c, i.e. floor(p*n_c/N)."""
    return (np.asarray(p, dtype=np.int64) * n_c) // N


def window_chunks(c: int, n_c: int, n_ec: int = 1, wrap: bool = True) -> list:
    """Chunks whose items the positions of chunk c are scored against.

    RECE page, Algorithm 1 (the current chunk and its neighbours on both sides) and
    the method paragraph of Section 3 (n_ec, the number of neighbouring chunks
    looked into).  Chunks c - n_ec .. c + n_ec as a set: modulo n_c when ``wrap``
    (cyclic reading), else only those inside [0, n_c) (clipped reading).
    """
    if wrap:
        return sorted({(c + t) % n_c for t in range(-n_ec, n_ec + 1)})
    return [cc for cc in range(c - n_ec, c + n_ec + 1) if 0 <= cc < n_c]


def _top_k(ids: np.ndarray, logits: np.ndarray, k: int):
    """The k candidates with the largest logits; order (logit descending, id ascending)."""
    order = np.lexsort((ids, -logits))
    return order[:k]


def round_negatives(X, Y, pos, perm_x, perm_y, n_c: int, k: int, rows=None, n_ec: int = 1,
                    wrap: bool = True):
    """Negatives of one round for every position (or for the positions in ``rows``).

    For position chunk c (RECE page, Algorithm 1, the chunk, window and negative-logit
    steps): the logits of its positions against the items of the window chunks, the
    position's own positive excluded (only wrong classes are negatives), then the k
    largest per position.

    Returns a dict  i -> (ids, logits, threshold)  where ids/logits are in rank order
    and threshold is (logit, id) of the k-th kept candidate when more than k
    candidates existed, else None (all candidates kept).
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    s, C = len(perm_x), len(perm_y)
    want = None if rows is None else set(int(i) for i in rows)
    out = {}
    for c in range(n_c):
        I = np.asarray(perm_x)[chunk_members(c, s, n_c)]
        if want is not None:
            I = np.array([i for i in I if int(i) in want], dtype=np.int64)
        if len(I) == 0:
            continue
        J = np.concatenate([np.asarray(perm_y)[chunk_members(cc, C, n_c)]
                            for cc in window_chunks(c, n_c, n_ec, wrap)])
        L = seq_dot(X[I], Y[J])
        for r, i in enumerate(I):
            keep = J != pos[i]
            ids, lg = J[keep], L[r, keep]
            sel = _top_k(ids, lg, k)
            thr = (float(lg[sel[-1]]), int(ids[sel[-1]])) if (len(ids) > k and k > 0) else None
            out[int(i)] = (ids[sel].astype(np.int64), lg[sel], thr)
    return out


def logsumexp(v) -> float:
    """log(sum(exp(v))) with the maximum shifted out (empty sum: -inf)."""
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0:
        return -np.inf
    m = np.max(v)
    return float(m + np.log(np.sum(np.exp(v - m))))


def rece_forward(X, Y, pos, B, n_c: int, k: int, rows=None, n_ec: int = 1, wrap: bool = True,
                 buckets=None, ignore_negative: bool = False) -> dict:
    """RECE loss (RECE page, Section 3: Algorithm 1 and the rounds paragraph).

    B has shape [r, d, n_b] (one independent draw of the random vectors per round).
    Per round: bucket labels of positions and items, their stable orders, chunks,
    each chunk's window, the k largest negatives of every position; then the loss
    of every position over its positive and the union of its rounds' negatives.
    With ``rows`` the per-position work (negatives, loss) is done for those
    positions only and the mean is taken over them; bucketing and sorting always
    cover every position and item, since they decide the chunks.  ``buckets``
    (optional, one (bx, by) pair per round) replaces the bucket labels: the steps
    after the labelling are then recomputed from the given labels.
    ``ignore_negative``: a position with a negative positive id is padding; it is
    bucketed, sorted and chunked like any other row of X (and no item is excluded
    from its candidates), but its loss is 0 and the mean is over the other positions.
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    B = np.asarray(B, dtype=np.float64)
    rounds = B.shape[0]
    st = {"bx": [], "by": [], "perm_x": [], "perm_y": [], "negs": []}
    for rho in range(rounds):
        if buckets is None:
            bx, by = bucket_ids(X, B[rho]), bucket_ids(Y, B[rho])
        else:
            bx, by = (np.asarray(v, dtype=np.int64) for v in buckets[rho])
        px, py = stable_argsort(bx), stable_argsort(by)
        st["bx"].append(bx)
        st["by"].append(by)
        st["perm_x"].append(px)
        st["perm_y"].append(py)
        st["negs"].append(round_negatives(X, Y, pos, px, py, n_c, k, rows, n_ec, wrap))
    st.update(_loss(X, Y, pos, st["negs"], rows, ignore_negative))
    return st


def loss_from_negatives(X, Y, pos, negs, rows=None, ignore_negative: bool = False) -> dict:
    """The loss given each round's negative sets, the steps after the selection.

    ``negs[rho]`` maps a position id to the item ids it kept in round rho (any
    order).  Logits are recomputed here in float64; the result has the fields of
    ``rece_forward`` that ``rece_backward`` reads.  This is the injection point
    for sets produced elsewhere (for example read back from another
    implementation after checking them on samples).
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    full = []
    for per in negs:
        d = {}
        for i, ids in per.items():
            ids = np.asarray(ids, dtype=np.int64)
            lg = seq_dot(X[int(i)], Y[ids])[0] if len(ids) else np.zeros(0)
            d[int(i)] = (ids, lg, None)
        full.append(d)
    st = {"negs": full}
    st.update(_loss(X, Y, pos, full, rows, ignore_negative))
    return st


def _loss(X, Y, pos, negs, rows, ignore_negative=False) -> dict:
    """Per-position loss over the positive and the rounds' negatives (RECE page,
    Algorithm 1, the positive-logit, loss and mean steps; Section 3, the duplicate
    rule for pairs kept in several rounds).  Padding positions (``ignore_negative``
    and a negative positive id) have loss 0 and stay out of the mean."""
    s = X.shape[0]
    rounds = len(negs)
    rows = np.arange(s) if rows is None else np.asarray(rows, dtype=np.int64)
    pad = np.array([bool(ignore_negative) and pos[i] < 0 for i in rows], dtype=bool)
    # positive logit: the scalar product with the positive's own (original) item row
    l_pos = np.array([0.0 if pad[n] else seq_dot(X[i], Y[pos[i]][None, :])[0, 0] for n, i in enumerate(rows)])
    lse = np.empty(len(rows))
    loss = np.empty(len(rows))
    union, mult = [], []
    for n, i in enumerate(rows):
        i = int(i)
        copy_ids = np.concatenate([np.asarray(negs[rho][i][0], dtype=np.int64) for rho in range(rounds)])
        copy_lg = np.concatenate([np.asarray(negs[rho][i][1], dtype=np.float64) for rho in range(rounds)])
        uniq, cnt = np.unique(copy_ids, return_counts=True)
        count = dict(zip(uniq.tolist(), cnt.tolist()))
        # duplicate rule: every copy of a pair enters with its logit lowered by the log
        # of the number of rounds that kept the pair
        adj = np.array([lg - np.log(count[int(j)]) for j, lg in zip(copy_ids, copy_lg)])
        lse[n] = logsumexp(np.concatenate([[l_pos[n]], adj]))
        # negative log of the positive's softmax share over the scored set
        loss[n] = 0.0 if pad[n] else lse[n] - l_pos[n]
        union.append(uniq.astype(np.int64))
        mult.append(cnt.astype(np.int64))
    counted = int(np.sum(~pad))
    return dict(rows=rows, l_pos=l_pos, lse=lse, loss_pp=loss, union=union, mult=mult, pad=pad,
                loss=float(np.sum(loss) / counted) if counted else 0.0)


def rece_backward(X, Y, pos, fwd: dict, dloss: float = 1.0, dloss_pp=None):
    """Gradients of the RECE loss with respect to X and Y, selection held fixed.

    RECE page Eq. (4) restricted to the scored set: d loss_i / d logit_{i,j} is the
    softmax over {positive} + copies minus 1 for the positive.  A pair kept in n
    rounds contributes n copies of exp(l - ln n)/Z, i.e. exp(l)/Z in total.
    Upstream gradient: dloss (of the mean) or dloss_pp[i] per position.  One
    position at a time; inside a round's list every item appears once, so the
    item rows it touches are updated together.
    """
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    rounds = len(fwd["negs"])
    dX = np.zeros_like(X)
    dY = np.zeros_like(Y)
    pad = fwd.get("pad", np.zeros(len(fwd["rows"]), dtype=bool))
    counted = int(np.sum(~pad))
    for n, i in enumerate(fwd["rows"]):
        i = int(i)
        if pad[n]:   # padding: no gradient
            continue
        gbar = (dloss / counted) if dloss_pp is None else float(dloss_pp[i])
        lse = fwd["lse"][n]
        count = dict(zip(fwd["union"][n].tolist(), fwd["mult"][n].tolist()))
        g_pos = np.exp(fwd["l_pos"][n] - lse) - 1.0
        dX[i] += gbar * g_pos * Y[pos[i]]
        dY[pos[i]] += gbar * g_pos * X[i]
        for rho in range(rounds):
            ids, lg, _ = fwd["negs"][rho][i]
            ids = np.asarray(ids, dtype=np.int64)
            if len(ids) == 0:
                continue
            mult = np.array([count[int(j)] for j in ids], dtype=np.float64)
            g = gbar * np.exp(np.asarray(lg, dtype=np.float64) - np.log(mult) - lse)
            dX[i] += g @ Y[ids]
            dY[ids] += g[:, None] * X[i][None, :]
    return dX, dY


def full_ce(X, Y, pos) -> np.ndarray:
    """Per-position full cross-entropy over the whole catalogue (RECE page, Eq. 3)."""
    from scipy.special import logsumexp as _lse
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    logits = X @ Y.T
    rows = np.arange(X.shape[0])
    return _lse(logits, axis=1) - logits[rows, np.asarray(pos)]


def full_ce_grad(X, Y, pos, dloss: float = 1.0):
    """Gradients of mean full CE: softmax minus one-hot (RECE page, Eq. 4), chained to X, Y."""
    from scipy.special import softmax
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    P = softmax(X @ Y.T, axis=1)
    P[np.arange(X.shape[0]), np.asarray(pos)] -= 1.0
    G = P * (dloss / X.shape[0])
    return G @ Y, G.T @ X
