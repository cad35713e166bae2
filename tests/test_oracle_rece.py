"""Pins of the RECE oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle is pinned by: a hand-worked
example of Algorithm 1 (closed-form losses), the special cases that reduce to
full cross-entropy (Eq. 3, Eq. 4) computed with a dense matrix product and
scipy, brute force on tiny inputs, invariants (subset log-sum-exp is a lower
bound, monotonicity, the duplicate rule), and finite differences.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from rece_inputs import make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, s=24, C=60, d=8, n_b=4, rounds=2):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((s, d))
    Y = rng.standard_normal((C, d))
    pos = rng.integers(0, C, s)
    B = rng.standard_normal((rounds, d, n_b))
    return X, Y, pos, B


# ---------------------------------------------------------------- scalar products

def test_seq_dot_exact_on_integers():
    rng = np.random.default_rng(0)
    A = rng.integers(-50, 50, (7, 13)).astype(np.float64)
    Bm = rng.integers(-50, 50, (9, 13)).astype(np.float64)
    ref = (A.astype(np.int64) @ Bm.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(oracle.seq_dot(A, Bm), ref)


def test_seq_dot_index_order():
    # 1 + 2^53 - 2^53 depends on the order: index order gives (1 + 2^53) - 2^53 = 0 in float64.
    A = np.array([[1.0, 2.0 ** 53, -(2.0 ** 53)]])
    Bm = np.ones((1, 3))
    assert oracle.seq_dot(A, Bm)[0, 0] == 0.0
    A2 = np.array([[2.0 ** 53, -(2.0 ** 53), 1.0]])
    assert oracle.seq_dot(A2, Bm)[0, 0] == 1.0


def test_seq_dot_close_to_blas():
    X, Y, _, _ = _rand_case(1, s=30, C=50, d=17)
    assert np.allclose(oracle.seq_dot(X, Y), X @ Y.T, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- bucketing

def test_bucket_ids_brute_force():
    X, _, _, B = _rand_case(2, s=40, d=5, n_b=7, rounds=1)
    got = oracle.bucket_ids(X, B[0])
    for i in range(X.shape[0]):
        scores = [sum(X[i, t] * B[0][t, b] for t in range(5)) for b in range(7)]
        assert got[i] == max(range(7), key=lambda b: (scores[b], -b))


def test_bucket_ids_signed_and_lowest_tie():
    B = np.array([[1.0, -1.0, 1.0], [0.0, 0.0, 0.0]])   # b_0 = (1,0), b_1 = (-1,0), b_2 = (1,0)
    V = np.array([[-3.0, 1.0], [2.0, 5.0]])
    # signed: -3 -> bucket 1 (score +3); +2 -> buckets 0 and 2 tie, lowest wins
    assert oracle.bucket_ids(V, B).tolist() == [1, 0]


def test_bucket_ids_single_vector_and_scale_invariance():
    X, _, _, B = _rand_case(3, s=50, d=6, n_b=1, rounds=1)
    assert np.all(oracle.bucket_ids(X, B[0]) == 0)
    X, _, _, B = _rand_case(4, s=50, d=6, n_b=9, rounds=1)
    ref = oracle.bucket_ids(X, B[0])
    for f in (0.25, 8.0):          # powers of two scale every score exactly
        assert np.array_equal(oracle.bucket_ids(X * f, B[0]), ref)


# ---------------------------------------------------------------- sort and chunks

def test_stable_argsort_properties():
    rng = np.random.default_rng(5)
    keys = rng.integers(0, 6, 200)
    p = oracle.stable_argsort(keys)
    assert sorted(p.tolist()) == list(range(200))
    ks = keys[p]
    assert np.all(np.diff(ks) >= 0)
    for v in range(6):
        idx = p[ks == v]
        assert np.all(np.diff(idx) > 0)      # equal keys keep their original order


@pytest.mark.parametrize("N,n_c", [(10, 3), (8, 4), (30000, 64), (1000000, 256), (7, 7), (5, 1)])
def test_chunk_sizes_and_consistency(N, n_c):
    b = oracle.chunk_bounds(N, n_c)
    sizes = np.diff(b)
    assert b[0] == 0 and b[-1] == N and sizes.sum() == N
    assert set(sizes.tolist()) <= {N // n_c, -(-N // n_c)}
    if N <= 10:
        for c in range(n_c):
            m = oracle.chunk_members(c, N, n_c)
            assert m.tolist() == list(range(b[c], b[c + 1]))
            assert np.all(oracle.chunk_of(m, N, n_c) == c)
    else:
        p = np.arange(N)
        c = oracle.chunk_of(p, N, n_c)
        assert np.all((b[c] <= p) & (p < b[c + 1]))


def test_window_cyclic():
    assert oracle.window_chunks(0, 5) == [0, 1, 4]
    assert oracle.window_chunks(4, 5) == [0, 3, 4]
    assert oracle.window_chunks(2, 5) == [1, 2, 3]
    for n_c in (1, 2, 3):
        for c in range(n_c):
            assert oracle.window_chunks(c, n_c) == list(range(n_c))


def test_window_neighbour_count_and_clipping():
    # n_ec neighbouring chunks on each side (RECE page, Section 3, method paragraph)
    assert oracle.window_chunks(2, 7, n_ec=0) == [2]
    assert oracle.window_chunks(3, 9, n_ec=2) == [1, 2, 3, 4, 5]
    assert oracle.window_chunks(0, 9, n_ec=2) == [0, 1, 2, 7, 8]
    assert oracle.window_chunks(8, 9, n_ec=3) == [0, 1, 2, 5, 6, 7, 8]
    for n_c in range(1, 8):   # 2 n_ec + 1 >= n_c: every chunk
        for c in range(n_c):
            assert oracle.window_chunks(c, n_c, n_ec=(n_c - 1 + 1) // 2) == list(range(n_c))
    # clipped: the chunks inside [0, n_c) only
    assert oracle.window_chunks(0, 5, wrap=False) == [0, 1]
    assert oracle.window_chunks(4, 5, wrap=False) == [3, 4]
    assert oracle.window_chunks(2, 5, wrap=False) == [1, 2, 3]
    assert oracle.window_chunks(1, 6, n_ec=3, wrap=False) == [0, 1, 2, 3, 4]
    # the two readings agree away from the ends and for a single chunk
    for n_ec in range(4):
        assert oracle.window_chunks(0, 1, n_ec, True) == oracle.window_chunks(0, 1, n_ec, False) == [0]
        for c in range(n_ec, 12 - n_ec):
            assert oracle.window_chunks(c, 12, n_ec, True) == oracle.window_chunks(c, 12, n_ec, False)


@pytest.mark.parametrize("n_ec,wrap", [(0, True), (2, True), (1, False), (2, False), (0, False)])
def test_windows_brute_force(n_ec, wrap):
    """Each position's candidates, straight from the definitions: every sorted item
    slot whose chunk is within n_ec of the position's chunk (cyclic distance, or
    plain distance when clipped), the positive left out; then the k largest."""
    s, C, n_c, k = 21, 47, 7, 4
    X, Y, pos, B = _rand_case(60 + n_ec + 10 * wrap, s=s, C=C, d=4, n_b=3, rounds=1)
    px = oracle.stable_argsort(oracle.bucket_ids(X, B[0]))
    py = oracle.stable_argsort(oracle.bucket_ids(Y, B[0]))
    negs = oracle.round_negatives(X, Y, pos, px, py, n_c, k, n_ec=n_ec, wrap=wrap)
    for slot, i in enumerate(px):
        c = slot * n_c // s
        cand = []
        for q in range(C):
            cq = q * n_c // C
            dist = abs(cq - c)
            if wrap:
                dist = min(dist, n_c - dist)
            if dist <= n_ec and py[q] != pos[i]:
                cand.append(int(py[q]))
        lg = {j: sum(X[i, t] * Y[j, t] for t in range(4)) for j in cand}
        want = sorted(cand, key=lambda j: (-lg[j], j))[:k]
        assert negs[int(i)][0].tolist() == want


@pytest.mark.parametrize("n_c,n_ec,n_b", [(5, 2, 3), (7, 3, 4), (4, 5, 2)])
def test_wide_cyclic_window_is_full_ce(n_c, n_ec, n_b):
    # 2 n_ec + 1 >= n_c: every window is the whole catalogue, so k = C - 1 is full CE (Eq. 3)
    X, Y, pos, B = _rand_case(70 + n_c, s=20, C=37, d=5, n_b=n_b, rounds=1)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=n_c, k=36, n_ec=n_ec)
    assert np.allclose(fwd["loss_pp"], oracle.full_ce(X, Y, pos), rtol=1e-12, atol=1e-12)


def test_loss_grows_with_the_window():
    # one round: the i-th largest of a larger window is no smaller, so each position's
    # top-k sum grows (over several rounds the union may overlap more and need not)
    X, Y, pos, B = _rand_case(75, s=30, C=90, d=6, n_b=5, rounds=1)
    prev = None
    for n_ec in range(0, 5):
        cur = oracle.rece_forward(X, Y, pos, B, n_c=9, k=5, n_ec=n_ec)["loss_pp"]
        if prev is not None:
            assert np.all(cur >= prev - 1e-12)
        prev = cur
    clipped = oracle.rece_forward(X, Y, pos, B, n_c=9, k=5, n_ec=2, wrap=False)["loss_pp"]
    cyclic = oracle.rece_forward(X, Y, pos, B, n_c=9, k=5, n_ec=2, wrap=True)["loss_pp"]
    assert np.all(cyclic >= clipped - 1e-12)


def test_injected_sets_and_buckets():
    X, Y, pos, B = _rand_case(76, s=24, C=50, d=5, n_b=4, rounds=2)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=4, k=6)
    # the loss from the forward pass's own sets is the forward pass's loss
    sets = [{i: fwd["negs"][r][i][0] for i in range(24)} for r in range(2)]
    inj = oracle.loss_from_negatives(X, Y, pos, sets)
    assert np.array_equal(inj["loss_pp"], fwd["loss_pp"]) and np.array_equal(inj["lse"], fwd["lse"])
    g1, g2 = oracle.rece_backward(X, Y, pos, fwd), oracle.rece_backward(X, Y, pos, inj)
    assert np.allclose(g1[0], g2[0], atol=1e-15) and np.allclose(g1[1], g2[1], atol=1e-15)
    # a hand-chosen set: the loss is the closed-form log-sum-exp over it
    hand = [{0: [3, 7]}, {0: [7, 11]}]
    one = oracle.loss_from_negatives(X, Y, pos, hand, rows=[0])
    L = X[0] @ Y.T
    want = np.log(np.exp(L[pos[0]]) + np.exp(L[[3, 7, 11]]).sum()) - L[pos[0]]
    assert math.isclose(one["loss_pp"][0], want, rel_tol=1e-13)
    # bucket labels given: the same result as computing them, and labels of one's own choice
    # give the chunks they define
    same = oracle.rece_forward(X, Y, pos, B, n_c=4, k=6, buckets=list(zip(fwd["bx"], fwd["by"])))
    assert np.array_equal(same["loss_pp"], fwd["loss_pp"])
    bx, by = np.arange(24) % 3, (np.arange(50) * 7) % 5
    other = oracle.rece_forward(X, Y, pos, B[:1], n_c=4, k=6, buckets=[(bx, by)])
    assert other["perm_x"][0].tolist() == sorted(range(24), key=lambda i: (bx[i], i))
    assert other["perm_y"][0].tolist() == sorted(range(50), key=lambda j: (by[j], j))


# ---------------------------------------------------------------- top-k

def test_topk_brute_force():
    X, Y, pos, B = _rand_case(6, s=16, C=30, d=4, n_b=2, rounds=1)
    # make exact ties: duplicate some item rows
    Y[5] = Y[9]
    Y[11] = Y[9]
    bx = oracle.bucket_ids(X, B[0])
    by = oracle.bucket_ids(Y, B[0])
    px, py = oracle.stable_argsort(bx), oracle.stable_argsort(by)
    n_c, k = 4, 5
    negs = oracle.round_negatives(X, Y, pos, px, py, n_c, k)
    cy = oracle.chunk_of(np.arange(30), 30, n_c)
    for slot, i in enumerate(px):
        c = oracle.chunk_of(slot, 16, n_c)
        win = [int(py[q]) for q in range(30) if cy[q] in oracle.window_chunks(int(c), n_c)]
        cand = [j for j in win if j != pos[i]]
        lg = {j: sum(X[i, t] * Y[j, t] for t in range(4)) for j in cand}
        want = sorted(cand, key=lambda j: (-lg[j], j))[:k]
        ids, vals, thr = negs[int(i)]
        assert ids.tolist() == want
        assert thr == (lg[want[-1]], want[-1])


# ---------------------------------------------------------------- hand-worked example

def test_hand_example():
    with open(os.path.join(GOLDEN, "rece_hand_example.json")) as f:
        g = json.load(f)
    X, Y, pos = np.array(g["X"]), np.array(g["Y"]), np.array(g["pos"])
    B = np.array(g["B"])[None]
    fwd = oracle.rece_forward(X, Y, pos, B, g["n_c"], g["k"])
    assert fwd["bx"][0].tolist() == g["bx"]
    assert fwd["by"][0].tolist() == g["by"]
    assert fwd["perm_x"][0].tolist() == g["perm_x"]
    assert fwd["perm_y"][0].tolist() == g["perm_y"]
    for c, items in enumerate(g["item_chunks"]):
        assert fwd["perm_y"][0][oracle.chunk_members(c, 8, 4)].tolist() == items
    for i in range(4):
        ids, _, thr = fwd["negs"][0][i]
        assert ids.tolist() == g["negatives"][str(i)]
        assert list(thr) == g["thresholds"][str(i)]
        assert fwd["l_pos"][i] == g["l_pos"][str(i)]
    e = math.e
    closed = [math.log(1 + 2 * e ** 2), math.log(2 + e ** 2),
              math.log(1 + e ** 2 + e ** -2), math.log(2 + e ** -1)]
    assert np.allclose(fwd["loss_pp"], closed, rtol=1e-14)
    assert math.isclose(fwd["loss"], sum(closed) / 4, rel_tol=1e-14)
    # gradient of position 3 (scored set: positive 6 at logit 1, item 3 at 1, item 1 at 0)
    dX, dY = oracle.rece_backward(X, Y, pos, fwd)
    Z = 2 * e + 1
    want = 0.25 * ((e / Z - 1) * Y[6] + (e / Z) * Y[3] + (1 / Z) * Y[1])
    assert np.allclose(dX[3], want, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- reductions to full CE

def test_single_bucket_single_chunk_is_full_ce():
    X, Y, pos, B = _rand_case(7, s=20, C=45, d=6, n_b=1, rounds=1)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=1, k=44)
    ce = oracle.full_ce(X, Y, pos)
    assert np.allclose(fwd["loss_pp"], ce, rtol=1e-12, atol=1e-12)
    dX, dY = oracle.rece_backward(X, Y, pos, fwd)
    gX, gY = oracle.full_ce_grad(X, Y, pos)
    assert np.allclose(dX, gX, rtol=1e-10, atol=1e-13)
    assert np.allclose(dY, gY, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("n_c,n_b", [(2, 3), (3, 5), (3, 1)])
def test_two_or_three_chunks_window_is_catalogue(n_c, n_b):
    X, Y, pos, B = _rand_case(8 + n_c, s=18, C=33, d=5, n_b=n_b, rounds=1)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=n_c, k=32)
    assert np.allclose(fwd["loss_pp"], oracle.full_ce(X, Y, pos), rtol=1e-12, atol=1e-12)


def test_tiny_fullce_workload_is_full_ce():
    inp = make_inputs(scaled("tiny_fullce"))
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, n_c=1, k=1999)
    ce = oracle.full_ce(inp.X, inp.Y, inp.pos)
    assert np.allclose(fwd["loss_pp"], ce, rtol=1e-12)
    assert math.isclose(fwd["loss"], float(np.mean(ce)), rel_tol=1e-12)


# ---------------------------------------------------------------- invariants

def test_lower_bound_and_nonnegative():
    X, Y, pos, B = _rand_case(11, s=40, C=80, d=6, n_b=5, rounds=2)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=5, k=7)
    ce = oracle.full_ce(X, Y, pos)
    assert np.all(fwd["loss_pp"] >= 0)
    assert np.all(fwd["loss_pp"] <= ce + 1e-12)


def test_monotone_in_k_and_rounds():
    X, Y, pos, B = _rand_case(12, s=30, C=70, d=6, n_b=5, rounds=3)
    prev = None
    for k in (0, 1, 3, 8, 30):
        cur = oracle.rece_forward(X, Y, pos, B[:1], n_c=5, k=k)["loss_pp"]
        if prev is not None:
            assert np.all(cur >= prev - 1e-12)
        prev = cur
    prev = None
    for r in (1, 2, 3):
        cur = oracle.rece_forward(X, Y, pos, B[:r], n_c=5, k=4)["loss_pp"]
        if prev is not None:
            assert np.all(cur >= prev - 1e-12)
        prev = cur


def test_repeated_rounds_equal_one_round():
    # the ln(count) correction makes r copies of the same round count once
    X, Y, pos, B = _rand_case(13, s=30, C=70, d=6, n_b=5, rounds=1)
    one = oracle.rece_forward(X, Y, pos, B, n_c=5, k=6)
    three = oracle.rece_forward(X, Y, pos, np.concatenate([B, B, B]), n_c=5, k=6)
    assert np.allclose(one["loss_pp"], three["loss_pp"], rtol=1e-13, atol=1e-14)
    g1 = oracle.rece_backward(X, Y, pos, one)
    g3 = oracle.rece_backward(X, Y, pos, three)
    assert np.allclose(g1[0], g3[0], atol=1e-14) and np.allclose(g1[1], g3[1], atol=1e-14)


def test_union_counts_each_pair_once():
    X, Y, pos, B = _rand_case(14, s=25, C=50, d=6, n_b=4, rounds=3)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=4, k=5)
    L = oracle.seq_dot(X, Y)
    for n, i in enumerate(fwd["rows"]):
        U = fwd["union"][n]
        want = oracle.logsumexp(np.concatenate([[L[i, pos[i]]], L[i, U]])) - L[i, pos[i]]
        assert math.isclose(fwd["loss_pp"][n], want, rel_tol=1e-13, abs_tol=1e-14)
        assert pos[i] not in U


def test_zero_negatives_zero_loss():
    X, Y, pos, B = _rand_case(15, s=10, C=20, d=4, n_b=3, rounds=2)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=3, k=0)
    assert np.all(fwd["loss_pp"] == 0.0)
    dX, dY = oracle.rece_backward(X, Y, pos, fwd)
    assert np.all(dX == 0) and np.all(dY == 0)


def test_gradient_rows_sum_to_zero():
    X, Y, pos, B = _rand_case(16, s=30, C=60, d=5, n_b=4, rounds=2)
    fwd = oracle.rece_forward(X, Y, pos, B, n_c=4, k=6)
    dX, dY = oracle.rece_backward(X, Y, pos, fwd)
    # sum_j g_ij = 0 for every position => sum over items of dY = 0
    assert np.allclose(dY.sum(axis=0), 0.0, atol=1e-14)
    # dloss_pp = ones/s equals the mean's gradient
    dX2, dY2 = oracle.rece_backward(X, Y, pos, fwd, dloss_pp=np.full(30, 1 / 30))
    assert np.allclose(dX, dX2, atol=1e-15) and np.allclose(dY, dY2, atol=1e-15)


def test_finite_differences():
    X, Y, pos, B = _rand_case(17, s=12, C=40, d=8, n_b=4, rounds=2)
    n_c, k, h = 4, 6, 1e-6
    fwd = oracle.rece_forward(X, Y, pos, B, n_c, k)
    dX, dY = oracle.rece_backward(X, Y, pos, fwd)

    def sel(f):
        return [[f["negs"][r][i][0].tolist() for i in range(12)] for r in range(2)]

    ref_sel = sel(fwd)
    checked = 0
    for which, M, G in (("X", X, dX), ("Y", Y, dY)):
        for idx in itertools.product(range(M.shape[0]), range(M.shape[1])):
            vals = []
            for sgn in (1, -1):
                M2 = M.copy()
                M2[idx] += sgn * h
                f = oracle.rece_forward(*((M2, Y) if which == "X" else (X, M2)), pos, B, n_c, k)
                if sel(f) != ref_sel or any(
                        not np.array_equal(a, b) for a, b in zip(f["perm_x"] + f["perm_y"],
                                                                 fwd["perm_x"] + fwd["perm_y"])):
                    break
                vals.append(f["loss"])
            else:
                fd = (vals[0] - vals[1]) / (2 * h)
                assert abs(fd - G[idx]) <= 1e-7 + 1e-5 * abs(G[idx]), (which, idx, fd, G[idx])
                checked += 1
    assert checked > 0.9 * (X.size + Y.size)


def test_rows_subset_matches_full():
    X, Y, pos, B = _rand_case(18, s=40, C=70, d=5, n_b=4, rounds=2)
    full = oracle.rece_forward(X, Y, pos, B, n_c=4, k=5)
    rows = np.array([3, 17, 31])
    sub = oracle.rece_forward(X, Y, pos, B, n_c=4, k=5, rows=rows)
    assert np.allclose(sub["loss_pp"], full["loss_pp"][rows], rtol=0, atol=0)


def test_full_ce_matches_plain_definition():
    X, Y, pos, _ = _rand_case(19, s=6, C=9, d=3)
    ce = oracle.full_ce(X, Y, pos)
    for i in range(6):
        lg = [sum(X[i, t] * Y[j, t] for t in range(3)) for j in range(9)]
        want = -math.log(math.exp(lg[pos[i]]) / sum(math.exp(v) for v in lg))
        assert math.isclose(ce[i], want, rel_tol=1e-12)
    gX, gY = oracle.full_ce_grad(X, Y, pos)
    # Eq. 4 range: every logit gradient in (-1, 1) / s, chained: check gY sums to zero over items
    assert np.allclose(gY.sum(axis=0), 0.0, atol=1e-14)


def test_padding_mask_equals_weighted_unmasked_loss():
    """Padding (a negative positive id, the mask reading): the masked loss is the mean,
    over the other positions, of the per-position losses of a run in which the
    padding rows carry any positive (a row's selection depends only on its own
    positive), and the masked gradients are that run's gradients with upstream
    weights 1/n_valid on the other positions and 0 on padding."""
    import numpy as np
    import oracle
    from rece_inputs import make_inputs, scaled
    w = scaled("tiny", seqs=2, seqlen=40, C=300, n_b=4, n_c=4, k=12, rounds=2, seed=31)
    inp = make_inputs(w)
    rng = np.random.default_rng(4)
    pad = rng.random(w.s) < 0.25
    pos_m = inp.pos.copy()
    pos_m[pad] = -1
    pos_u = inp.pos.copy()                                  # padding rows given their original positive
    f_m = oracle.rece_forward(inp.X, inp.Y, pos_m, inp.B, w.n_c, w.k, ignore_negative=True)
    f_u = oracle.rece_forward(inp.X, inp.Y, pos_u, inp.B, w.n_c, w.k)
    nv = int((~pad).sum())
    assert np.all(f_m["loss_pp"][pad] == 0.0)
    assert np.allclose(f_m["loss_pp"][~pad], f_u["loss_pp"][~pad], rtol=1e-12, atol=0)
    assert abs(f_m["loss"] - f_u["loss_pp"][~pad].mean()) <= 1e-12 * max(1.0, abs(f_m["loss"]))
    gX_m, gY_m = oracle.rece_backward(inp.X, inp.Y, pos_m, f_m)
    wts = np.where(pad, 0.0, 1.0 / nv)
    gX_u, gY_u = oracle.rece_backward(inp.X, inp.Y, pos_u, f_u, dloss_pp=wts)
    assert np.all(gX_m[pad] == 0.0)
    assert np.allclose(gX_m, gX_u, rtol=1e-12, atol=1e-15) and np.allclose(gY_m, gY_u, rtol=1e-12, atol=1e-15)
    # without padding ids the mask changes nothing
    f_0 = oracle.rece_forward(inp.X, inp.Y, pos_u, inp.B, w.n_c, w.k, ignore_negative=True)
    assert f_0["loss"] == f_u["loss"]
