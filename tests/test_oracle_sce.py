"""Pins of the SCE bucket-variant oracle.

The SCE page gives the idea (a softmax over a subset found by maximum inner
product search), the workload description the bucket procedure.  Pinned here:
a hand-worked example (closed-form losses), the reductions to full
cross-entropy (every bucket takes every position and item, k = C - 1), a
brute-force recomputation on tiny inputs written with Python sorting and no
per-bucket pruning, invariants (lower bound, monotone in k, uncovered positions
have zero loss) and finite differences.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, s=24, C=60, d=8, n_b=5):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((s, d))
    Y = rng.standard_normal((C, d))
    pos = rng.integers(0, C, s)
    B = rng.standard_normal((d, n_b))
    return X, Y, pos, B


def _dot(a, b):
    acc = 0.0
    for t in range(len(a)):
        acc += float(a[t]) * float(b[t])
    return acc


def test_column_top_brute_force_with_ties():
    rng = np.random.default_rng(3)
    col = rng.integers(-3, 4, 40).astype(np.float64)     # many equal scores
    for b in (0, 1, 5, 13, 39, 40, 55):
        want = sorted(range(40), key=lambda i: (-col[i], i))[:b]
        assert oracle.column_top(col, b).tolist() == sorted(want)


def test_hand_example():
    with open(os.path.join(GOLDEN, "sce_hand_example.json")) as f:
        g = json.load(f)
    X = np.array(g["X"], dtype=np.float64)
    Y = np.array(g["Y"], dtype=np.float64)
    B = np.array(g["B_columns"], dtype=np.float64).T     # columns are the projection vectors
    pos = np.array(g["pos"])
    R, Q = oracle.bucket_lists(X, Y, B, g["b_x"], g["b_y"])
    assert [r.tolist() for r in R] == g["R"]
    assert [q.tolist() for q in Q] == g["Q"]
    closed = {"log(1 + e)": math.log(1 + math.e), "log(1 + e^-1)": math.log(1 + math.exp(-1)),
              "log(2)": math.log(2), "log(2 + e^-2)": math.log(2 + math.exp(-2))}
    for case in g["cases"]:
        f = oracle.sce_forward(X, Y, pos, B, g["b_x"], g["b_y"], case["k"])
        assert [f["negs"][0][i][0].tolist() for i in range(3)] == case["negatives"]
        want = [closed[e] for e in case["loss_pp"]]
        assert np.allclose(f["loss_pp"], want, rtol=1e-14, atol=0)


def _brute(X, Y, pos, B, b_x, b_y, k):
    """Literal definition, no pruning: per position, the union over the buckets that
    took it, top-k of the union, loss from Eq. 3 restricted to the scored set."""
    s, C, n_b = X.shape[0], Y.shape[0], B.shape[1]
    R, Q = [], []
    for b in range(n_b):
        px = [_dot(X[i], B[:, b]) for i in range(s)]
        py = [_dot(Y[j], B[:, b]) for j in range(C)]
        R.append(set(sorted(range(s), key=lambda i: (-px[i], i))[:b_x]))
        Q.append(set(sorted(range(C), key=lambda j: (-py[j], j))[:b_y]))
    negs, loss, thr = [], [], []
    for i in range(s):
        U = set()
        for b in range(n_b):
            if i in R[b]:
                U |= Q[b] - {int(pos[i])}
        lg = {j: _dot(X[i], Y[j]) for j in U}
        keep = sorted(U, key=lambda j: (-lg[j], j))[:k]
        lp = _dot(X[i], Y[pos[i]])
        z = math.exp(lp) + sum(math.exp(lg[j]) for j in keep)
        negs.append(keep)
        loss.append(math.log(z) - lp)
        thr.append((keep[-1], lg[keep[-1]]) if (len(U) > k and k > 0) else None)
    return R, Q, negs, loss, thr


@pytest.mark.parametrize("seed,b_x,b_y,k", [(1, 6, 15, 4), (2, 3, 30, 10), (3, 10, 5, 8), (4, 24, 60, 59)])
def test_brute_force(seed, b_x, b_y, k):
    X, Y, pos, B = _case(seed)
    R, Q, negs, loss, thr = _brute(X, Y, pos, B, b_x, b_y, k)
    f = oracle.sce_forward(X, Y, pos, B, b_x, b_y, k)
    assert [f["negs"][0][i][2] for i in range(len(pos))] == thr
    assert [set(r.tolist()) for r in f["R"]] == R
    assert [set(q.tolist()) for q in f["Q"]] == Q
    assert [f["negs"][0][i][0].tolist() for i in range(len(pos))] == negs
    assert np.allclose(f["loss_pp"], loss, rtol=1e-12, atol=1e-14)


def test_positions_in_no_bucket_have_zero_loss():
    X, Y, pos, B = _case(5, s=40, n_b=3)
    f = oracle.sce_forward(X, Y, pos, B, b_x=4, b_y=20, k=5)
    taken = set().union(*[set(r.tolist()) for r in f["R"]])
    assert len(taken) < 40
    for i in range(40):
        if i not in taken:
            assert len(f["negs"][0][i][0]) == 0 and f["loss_pp"][i] == 0.0
        else:
            assert f["loss_pp"][i] > 0.0


@pytest.mark.parametrize("n_b", [1, 3])
def test_everything_taken_is_full_ce(n_b):
    X, Y, pos, B = _case(6, s=20, C=30, n_b=n_b)
    f = oracle.sce_forward(X, Y, pos, B, b_x=20, b_y=30, k=29)
    assert np.allclose(f["loss_pp"], oracle.full_ce(X, Y, pos), rtol=1e-12, atol=0)
    dX, dY = oracle.sce_backward(X, Y, pos, f)
    gX, gY = oracle.full_ce_grad(X, Y, pos)
    assert np.allclose(dX, gX, rtol=1e-10, atol=1e-14)
    assert np.allclose(dY, gY, rtol=1e-10, atol=1e-14)


def test_lower_bound_and_monotone_in_k():
    X, Y, pos, B = _case(7)
    ce = oracle.full_ce(X, Y, pos)
    prev = None
    for k in (0, 1, 3, 8, 20):
        f = oracle.sce_forward(X, Y, pos, B, b_x=8, b_y=20, k=k)
        assert np.all(f["loss_pp"] >= 0) and np.all(f["loss_pp"] <= ce + 1e-12)
        if k == 0:
            assert np.all(f["loss_pp"] == 0)
        if prev is not None:
            assert np.all(f["loss_pp"] >= prev - 1e-12)
        prev = f["loss_pp"]


def test_finite_differences():
    X, Y, pos, B = _case(8, s=12, C=30, d=6, n_b=4)
    b_x, b_y, k, h = 5, 10, 4, 1e-6
    fwd = oracle.sce_forward(X, Y, pos, B, b_x, b_y, k)
    dX, dY = oracle.sce_backward(X, Y, pos, fwd)

    def sel(f):
        return ([r.tolist() for r in f["R"]], [q.tolist() for q in f["Q"]],
                [f["negs"][0][i][0].tolist() for i in range(12)])

    ref = sel(fwd)
    checked = 0
    for which, M, G in (("X", X, dX), ("Y", Y, dY)):
        for idx in itertools.product(range(M.shape[0]), range(M.shape[1])):
            vals = []
            for sgn in (1, -1):
                M2 = M.copy()
                M2[idx] += sgn * h
                f = oracle.sce_forward(*((M2, Y) if which == "X" else (X, M2)), pos, B, b_x, b_y, k)
                if sel(f) != ref:
                    break
                vals.append(f["loss"])
            else:
                fd = (vals[0] - vals[1]) / (2 * h)
                assert abs(fd - G[idx]) <= 1e-7 + 1e-5 * abs(G[idx]), (which, idx, fd, G[idx])
                checked += 1
    assert checked > 0.9 * (X.size + Y.size)
