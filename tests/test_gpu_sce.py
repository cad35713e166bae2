"""GPU parity of the bucket (SCE) variant against the CPU oracle.

The positions and items each bucket takes, every position's final threshold
(float64 logit and id of its k-th kept negative) and kept set are compared
exactly; loss within 1e-5 relative (float32 inputs) or 1e-3 (bf16 inputs);
gradients within 2e-3 of max|grad|."""
import numpy as np
import pytest

import oracle
from gpu_helpers import grad_err, run_sce
from rece_inputs import make_inputs, scaled

pytestmark = pytest.mark.gpu

CASES = {
    # the SCE workload's shape (d = 256, bf16, Zipf positives) at a size the oracle finishes quickly
    "sce_small": scaled("sce", seqs=4, seqlen=128, C=8000, n_b=16, b_x=64, b_y=512, k=64),
    "sce_many_buckets": scaled("sce", seqs=2, seqlen=300, C=5000, d=64, n_b=48, b_x=40, b_y=300, k=32),
    "sce_f32_d32": scaled("sce", seqs=3, seqlen=100, C=2500, d=32, dtype="f32", n_b=12, b_x=50, b_y=300, k=20),
    # every bucket list shorter than k: each slot keeps all its candidates, the union is cut to k
    "sce_lists_below_k": scaled("sce", seqs=2, seqlen=100, C=3000, d=64, n_b=10, b_x=60, b_y=30, k=40),
    "sce_k_one": scaled("sce", seqs=2, seqlen=64, C=2000, d=64, n_b=8, b_x=32, b_y=200, k=1),
    "sce_k_zero": scaled("sce", seqs=2, seqlen=64, C=2000, d=64, n_b=8, b_x=32, b_y=200, k=0),
    # buckets taking most of their rows: the boundary lies low in every column's score range
    "sce_most_rows": scaled("sce", seqs=2, seqlen=100, C=2000, d=64, n_b=5, b_x=150, b_y=1200, k=48),
    # more than 4096 items per bucket: the stored-score selection instead of the listed one
    "sce_wide_buckets": scaled("sce", seqs=2, seqlen=64, C=12000, d=64, n_b=3, b_x=32, b_y=5000, k=32),
    # one bucket taking everything with k = C - 1 is full cross-entropy
    "sce_full_ce": scaled("sce", seqs=2, seqlen=128, C=700, d=64, dtype="f32", n_b=1, b_x=256, b_y=700, k=699),
}


def _check(name, inp, g, fwd):
    w = inp.w
    tol = 1e-5 if w.dtype == "f32" else 1e-3
    R, Q = g["sce_rows"], g["sce_items"]
    for b in range(w.n_b):
        assert np.array_equal(np.sort(R[b]), fwd["R"][b]), (name, "R", b)
        assert np.array_equal(np.sort(Q[b]), fwd["Q"][b]), (name, "Q", b)
    taken = np.zeros(w.s, dtype=bool)
    taken[np.concatenate(fwd["R"])] = True
    tid, te, negs = g["thresh_id"], g["thresh_logit"], g["neg_ids"]
    for i in range(w.s):
        ids, _, thr = fwd["negs"][0][i]
        if w.k == 0 or not taken[i]:
            assert tid[i] == -2, (name, i, tid[i])
        elif thr is None:
            assert tid[i] == -1, (name, i, tid[i])
        else:
            assert tid[i] == thr[0] and te[i] == thr[1], (name, i, tid[i], te[i], thr)
        gs = np.sort(negs[i][negs[i] >= 0]) if w.k > 0 else np.array([], dtype=np.int64)
        assert np.array_equal(gs, np.sort(ids)), (name, i)
        u = g["union_ids"][i] if w.k > 0 else np.array([], dtype=np.int64)
        assert np.array_equal(np.sort(u[u >= 0]), np.sort(ids)), (name, i)
    rel = abs(g["loss"] - fwd["loss"]) / max(abs(fwd["loss"]), 1e-30)
    assert rel <= tol, (name, g["loss"], fwd["loss"])
    lpp_err = np.max(np.abs(g["loss_pp"] - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0))
    assert lpp_err <= tol, (name, lpp_err)
    c = g["counters"]
    assert c[0] == 0 and c[4] == 0, (name, c)


@pytest.mark.parametrize("name", list(CASES))
def test_sce_parity(name):
    w = CASES[name]
    inp = make_inputs(w)
    g = run_sce(inp)
    fwd = oracle.sce_forward(inp.X, inp.Y, inp.pos, inp.B[0], w.b_x, w.b_y, w.k)
    _check(name, inp, g, fwd)
    gX, gY = oracle.sce_backward(inp.X, inp.Y, inp.pos, fwd)
    if w.k == 0:
        assert np.all(g["dX"] == 0) and np.all(g["dY"] == 0)
        return
    ex, ey = grad_err(g["dX"], gX), grad_err(g["dY"], gY)
    print(f"{name}: loss {g['loss']:.7f} vs {fwd['loss']:.7f}; dX err {ex:.2e}; dY err {ey:.2e}; "
          f"counters {g['counters'].tolist()}")
    assert ex <= 2e-3 and ey <= 2e-3, (name, ex, ey)


def test_sce_hundreds_of_ties():
    """10 distinct item rows repeated 600 times: every bucket's item boundary falls
    inside 600 equal projection scores, every slot's top-k inside 600 equal logits
    (the chunk kernel's exact pass), and the merge of a position's buckets ranks
    more near-ties than its float64 buffer holds (the recomputing path).  Every
    selection must equal the oracle's: ties to the lowest index."""
    import dataclasses
    w = scaled("sce", seqs=2, seqlen=64, C=6000, d=64, n_b=6, b_x=48, b_y=1000, k=128)
    inp = make_inputs(w)
    inp = dataclasses.replace(inp, Y=np.ascontiguousarray(inp.Y[np.arange(w.C) % 10]))
    print("[gpu] sce: 10 distinct rows x 600 copies, k=128", flush=True)
    g = run_sce(inp)
    fwd = oracle.sce_forward(inp.X, inp.Y, inp.pos, inp.B[0], w.b_x, w.b_y, w.k)
    _check("sce_ties", inp, g, fwd)
    gX, gY = oracle.sce_backward(inp.X, inp.Y, inp.pos, fwd)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3


def test_sce_full_ce_equals_dense_cross_entropy():
    w = CASES["sce_full_ce"]
    inp = make_inputs(w)
    g = run_sce(inp, keep_stages=False)
    ce = oracle.full_ce(inp.X, inp.Y, inp.pos)
    assert abs(g["loss"] - ce.mean()) / ce.mean() <= 1e-5
    gX, gY = oracle.full_ce_grad(inp.X, inp.Y, inp.pos)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3


def test_sce_per_position_upstream_and_repeatable():
    w = CASES["sce_many_buckets"]
    inp = make_inputs(w)
    dpp = np.random.default_rng(11).standard_normal(w.s) * 0.01
    a = run_sce(inp, keep_stages=False, dloss_pp=dpp)
    b = run_sce(inp, keep_stages=False, dloss_pp=dpp)
    assert np.array_equal(a["dX"], b["dX"]) and np.array_equal(a["dY"], b["dY"])
    assert a["loss"] == b["loss"]
    fwd = oracle.sce_forward(inp.X, inp.Y, inp.pos, inp.B[0], w.b_x, w.b_y, w.k)
    gX, gY = oracle.sce_backward(inp.X, inp.Y, inp.pos, fwd, dloss_pp=dpp.astype(np.float32))
    assert grad_err(a["dX"], gX) <= 2e-3 and grad_err(a["dY"], gY) <= 2e-3


def test_sce_one_far_item_takes_a_finer_level():
    """One item row 64 times longer than the others stretches every bucket column's
    score range, so the first 32-bin histogram leaves nearly all 20,000 items in the
    listing bins, more than a column's list holds: those columns take the next
    histogram level (counter 7) and the selection must still equal the oracle's."""
    import dataclasses
    w = scaled("sce", seqs=2, seqlen=64, C=20000, d=64, n_b=4, b_x=32, b_y=256, k=32)
    inp = make_inputs(w)
    Y = inp.Y.copy()
    Y[1234] *= 64.0   # a power of two: the row stays exactly representable in bfloat16
    inp = dataclasses.replace(inp, Y=Y)
    print("[gpu] sce: one item row x64, C=20000, b_y=256", flush=True)
    g = run_sce(inp)
    fwd = oracle.sce_forward(inp.X, inp.Y, inp.pos, inp.B[0], w.b_x, w.b_y, w.k)
    _check("sce_far_item", inp, g, fwd)
    assert g["counters"][7] >= 1, g["counters"]   # columns nearly orthogonal to the row need not
    gX, gY = oracle.sce_backward(inp.X, inp.Y, inp.pos, fwd)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3
