"""GPU parity of the RECE path against the CPU oracle, stage by stage.

Bucket ids, permutations, per-round thresholds (float64 logit and id of the
k-th kept negative) and kept-negative sets are compared exactly: both sides
take every selection decision on the float64 coordinate-order scalar product.
Loss within 1e-5 relative (float32 inputs) or 1e-3 (bf16 inputs); gradients
within 2e-3 of max|grad| (max-abs error normalised)."""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_helpers import grad_err, run_rece
from rece_inputs import make_inputs, scaled

pytestmark = pytest.mark.gpu

CASES = {
    # full-size tiny workload (float32) and its full-CE twin
    "tiny": scaled("tiny"),
    "tiny_fullce": scaled("tiny_fullce"),
    # reduced workloads of the same recipes: several tiles, ragged chunks and tails
    "sasrec_small": scaled("sasrec", seqs=3, seqlen=700, C=5003, n_b=16, n_c=16, k=64, rounds=2),
    "million_small": scaled("million", seqs=8, seqlen=200, C=40000, n_b=32, n_c=32, k=128, rounds=2),
    "tenmillion_small": scaled("tenmillion", seqs=4, seqlen=256, C=60000, n_b=64, n_c=64, k=256,
                               rounds=3),
    "d256": scaled("sasrec", seqs=2, seqlen=256, C=8000, d=256, n_b=8, n_c=8, k=64, rounds=1),
    "d32_f32": scaled("tiny", seqs=5, seqlen=77, C=3001, d=32, n_b=7, n_c=11, k=9, rounds=3),
    "one_chunk_topk": scaled("tiny", seqs=2, seqlen=100, C=900, n_b=4, n_c=1, k=50, rounds=2),
    "two_chunks": scaled("sasrec", seqs=2, seqlen=150, C=1200, n_b=4, n_c=2, k=40, rounds=2),
    "chunk_per_position": scaled("tiny", seqs=1, seqlen=40, C=400, n_b=5, n_c=40, k=3, rounds=2),
    "k_zero": scaled("sasrec", seqs=2, seqlen=64, C=700, n_b=4, n_c=4, k=0, rounds=1),
    "k_one_8_rounds": scaled("sasrec", seqs=2, seqlen=96, C=1000, n_b=6, n_c=6, k=1, rounds=8),
    # earlier rounds' kept ids too many for the dedup's LDS tables ((rounds - 1) * k > 2048):
    # the dedup scans the earlier lists; windows of three of four chunks overlap partly
    "dedup_scan": scaled("tiny", seqs=1, seqlen=64, C=4000, n_b=4, n_c=4, k=2100, rounds=2),
    # windows of n_ec neighbouring chunks on each side, cyclic and clipped
    "own_chunk_only": scaled("sasrec", seqs=2, seqlen=150, C=3001, n_b=12, n_c=12, k=20, rounds=2, n_ec=0),
    "two_neighbours": scaled("sasrec", seqs=3, seqlen=128, C=6007, n_b=16, n_c=16, k=48, rounds=2, n_ec=2),
    "clipped": scaled("sasrec", seqs=3, seqlen=100, C=4001, n_b=10, n_c=10, k=40, rounds=2,
                      window_wrap=False),
    "clipped_wide": scaled("tiny", seqs=2, seqlen=90, C=2500, d=32, n_b=9, n_c=9, k=30, rounds=1, n_ec=3,
                           window_wrap=False),
    "neighbours_cover_all": scaled("sasrec", seqs=1, seqlen=128, C=1500, n_b=5, n_c=5, k=60, rounds=2, n_ec=2),
    # one chunk: every window is the whole catalogue of 70001 items, more than a 16-bit
    # histogram bin can count (the chunk kernel counts in 32 bits); many compactions
    "window_over_16_bits": scaled("tiny", seqs=1, seqlen=96, C=70001, d=32, n_b=3, n_c=1, k=40, rounds=1),
}


def _compare(name, inp, g, fwd):
    w = inp.w
    tol = 1e-5 if w.dtype == "f32" else 1e-3
    for r in range(w.rounds):
        assert np.array_equal(g[("bucket_x", r)], fwd["bx"][r]), (name, r, "bucket_x")
        assert np.array_equal(g[("bucket_y", r)], fwd["by"][r]), (name, r, "bucket_y")
        assert np.array_equal(g[("perm_x", r)], fwd["perm_x"][r]), (name, r, "perm_x")
        assert np.array_equal(g[("perm_y", r)], fwd["perm_y"][r]), (name, r, "perm_y")
        tid, te = g[("thresh_id", r)], g[("thresh_logit", r)]
        negs = g[("neg_ids", r)]
        for i in range(w.s):
            ids, _, thr = fwd["negs"][r][i]
            if w.k == 0:
                assert tid[i] == -2
            elif thr is None:
                assert tid[i] == -1, (name, r, i)
            else:
                assert tid[i] == thr[1] and te[i] == thr[0], (name, r, i, tid[i], te[i], thr)
            gs = np.sort(negs[i][negs[i] >= 0]) if w.k > 0 else np.array([], dtype=np.int64)
            assert np.array_equal(gs, np.sort(ids)), (name, r, i)
    rel = abs(g["loss"] - fwd["loss"]) / max(abs(fwd["loss"]), 1e-30)
    assert rel <= tol, (name, g["loss"], fwd["loss"])
    lpp_err = np.max(np.abs(g["loss_pp"] - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0))
    assert lpp_err <= tol, (name, lpp_err)
    c = g["counters"]
    assert c[0] == 0 and c[4] == 0, (name, c)
    # the union over rounds, each id once
    for n, i in enumerate(fwd["rows"]):
        u = g["union_ids"][int(i)]
        assert np.array_equal(np.sort(u[u >= 0]), fwd["union"][n]), (name, i)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_backward_parity(name):
    w = CASES[name]
    inp = make_inputs(w)
    g = run_rece(inp)
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k, n_ec=w.n_ec, wrap=w.window_wrap)
    _compare(name, inp, g, fwd)
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    if w.k == 0:
        # only the positive is scored: loss 0, gradient exp(0) - 1 = 0
        assert np.all(g["dX"] == 0) and np.all(g["dY"] == 0)
        return
    ex, ey = grad_err(g["dX"], gX), grad_err(g["dY"], gY)
    print(f"{name}: loss {g['loss']:.7f} vs {fwd['loss']:.7f}; dX err {ex:.2e}; dY err {ey:.2e}; "
          f"counters {g['counters'].tolist()}")
    assert ex <= 2e-3 and ey <= 2e-3, (name, ex, ey)


def test_fullce_twin_equals_dense_cross_entropy():
    w = CASES["tiny_fullce"]
    inp = make_inputs(w)
    g = run_rece(inp, keep_stages=False)
    ce = oracle.full_ce(inp.X, inp.Y, inp.pos)
    assert abs(g["loss"] - ce.mean()) / ce.mean() <= 1e-5
    gX, gY = oracle.full_ce_grad(inp.X, inp.Y, inp.pos)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3


def test_loss_below_full_ce_and_per_position_upstream():
    w = CASES["sasrec_small"]
    inp = make_inputs(w)
    rng = np.random.default_rng(7)
    dpp = rng.standard_normal(w.s) * 0.01
    g = run_rece(inp, keep_stages=False, dloss_pp=dpp)
    ce = oracle.full_ce(inp.X, inp.Y, inp.pos)
    assert np.all(g["loss_pp"] <= ce + 1e-3 * np.maximum(ce, 1))
    assert np.all(g["loss_pp"] >= -1e-6)
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k)
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd, dloss_pp=dpp.astype(np.float32))
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3


def test_run_twice_bit_identical():
    w = CASES["million_small"]
    inp = make_inputs(w)
    a = run_rece(inp, keep_stages=False)
    b = run_rece(inp, keep_stages=False)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["loss_pp"], b["loss_pp"])
    assert np.array_equal(a["dX"], b["dX"]) and np.array_equal(a["dY"], b["dY"])


def test_exact_topk_ties_from_duplicate_items():
    """Every item row appears four times (ids j, j + U, j + 2U, j + 3U): equal logits
    at most k-th boundaries, so each row sends several entries through the float64
    ranking, and the ties must go to the lowest ids as in the oracle."""
    w = scaled("sasrec", seqs=2, seqlen=200, C=4000, n_b=8, n_c=8, k=64, rounds=2)
    inp = make_inputs(w)
    U = w.C // 4
    Y = np.ascontiguousarray(inp.Y[np.arange(w.C) % U])
    inp = dataclasses.replace(inp, Y=Y)
    print("[gpu] duplicate items, C=4000 (1000 distinct rows)", flush=True)
    g = run_rece(inp)
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k)
    _compare("duplicate_items", inp, g, fwd)
    # the ties are real: most rows' k-th kept item has an equal copy left out
    tied = 0
    for i in range(w.s):
        ids, _, thr = fwd["negs"][0][i]
        if thr is not None:
            kept = set(int(j) for j in ids)
            tied += any(int(c) not in kept and int(c) != int(inp.pos[i])
                        for c in (thr[1] % U + U * np.arange(4)))
    assert tied > w.s // 4, tied
    assert g["counters"][2] > 0   # rows whose k-th element needed the float64 ranking
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3


def test_window_of_mostly_zero_rows():
    """A window of 70,000 items of which 66,000 are zero rows (66,000 equal logits
    of 0 in every row): the selection matches the oracle exactly."""
    w = scaled("tiny", seqs=1, seqlen=64, C=70000, d=32, n_b=1, n_c=1, k=40, rounds=1)
    inp = make_inputs(w)
    Y = inp.Y.copy()
    Y[:66000] = 0.0
    inp = dataclasses.replace(inp, Y=Y)
    print("[gpu] window of 70000 items, 66000 zero rows", flush=True)
    g = run_rece(inp)
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k)
    _compare("bin_above_16_bits", inp, g, fwd)
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3


@pytest.mark.parametrize("k", [32, 128])
def test_hundreds_of_ties_take_the_exact_pass(k):
    """The catalogue is 10 distinct rows repeated 600 times each, so every position
    scores 600 equal copies of its best row: far more ties at the k-th logit than a
    candidate list holds (3k + 2 tiles), which no histogram compaction can shrink.
    Those rows are redone by the chunk kernel's exact pass, which ranks the ties in
    float64 and by id; at k = 128 the finishing kernel then ranks more near-ties
    than its float64 buffer holds (the recomputing path).  The kept sets (the k
    lowest ids among the copies) must equal the oracle's."""
    w = scaled("sasrec", seqs=2, seqlen=64, C=6000, n_b=2, n_c=1, k=k, rounds=1)
    inp = make_inputs(w)
    Y = np.ascontiguousarray(inp.Y[np.arange(w.C) % 10])
    inp = dataclasses.replace(inp, Y=Y)
    print(f"[gpu] 10 distinct rows x 600 copies, k={k}", flush=True)
    g = run_rece(inp)
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k)
    _compare("exact_pass", inp, g, fwd)
    assert g["counters"][5] > w.s // 2, g["counters"]   # rows redone by the exact pass
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    assert grad_err(g["dX"], gX) <= 2e-3 and grad_err(g["dY"], gY) <= 2e-3
