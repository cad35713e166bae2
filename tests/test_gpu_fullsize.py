"""GPU results at the full workload sizes, in the launch configuration bench.py
times, checked against the oracle on sampled outputs and by properties that
hold at any size.

* sasrec (s = 51,200, C = 30,000): the oracle's own bucketing and sorting of
  every vector; thresholds, kept sets, losses and dX rows of a seeded sample of
  positions compared exactly (selections) or within the tolerances.
* million, ten million items and the bucket variant: the oracle cannot bucket
  every item in a test's time, so: bucket ids of sampled rows (the oracle's
  own values); the sort is a stable permutation of the GPU's bucket ids; the
  kept set of a sampled position is the oracle's top-k of the window that
  sort defines; its loss is the float64 loss of that set and it lies between 0
  and the full cross-entropy of the row (the oracle's); and the gradients obey
  sum_i dX_i . x_i = sum_j dY_j . y_j (both equal sum over scored pairs of
  g_ij * logit_ij).
"""
import numpy as np
import pytest
import torch

import catalogue_cross_entropy_amd as rece
import oracle
from gpu_helpers import grad_err, to_device
from rece_inputs import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

N_ROWS = 48        # sampled positions
N_BUCKET = 2048    # sampled rows for bucket ids


def _run(w, inp):
    X, Y, pos, B = to_device(inp)
    if w.variant == "sce":
        B = B[0].contiguous()
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, variant=w.variant,
                     b_x=w.b_x, b_y=w.b_y, keep_stages=True, validate_ids=True)
    print(f"[gpu] full size {w.name}", flush=True)
    loss, lpp, scratch, saved = plan.forward(X, Y, pos, B)
    dX, dY = plan.backward(X, Y, pos, scratch, saved)
    plan.check(saved)
    torch.cuda.synchronize()
    del scratch
    return plan, saved, lpp.cpu().numpy(), dX, dY, X, Y


def _full_ce_rows(Xr, Y, pos_r, block=1 << 20):
    """Full cross-entropy (RECE page, Eq. 3) of a few rows against every item, float64,
    the catalogue taken in blocks so no [C, d] float64 copy is ever made."""
    Xr = np.asarray(Xr, dtype=np.float64)
    m = np.full(len(Xr), -np.inf)
    z = np.zeros(len(Xr))
    for j0 in range(0, Y.shape[0], block):
        L = Y[j0:j0 + block].astype(np.float64) @ Xr.T          # [block, rows]
        mb = L.max(axis=0)
        mn = np.maximum(m, mb)
        z = z * np.exp(m - mn) + np.exp(L - mn).sum(axis=0)
        m = mn
    lp = np.einsum("rd,rd->r", Xr, np.asarray(Y[pos_r], dtype=np.float64))
    return m + np.log(z) - lp


def _bilinear(dX, dY, X, Y):
    """sum_i dX_i . x_i and sum_j dY_j . y_j in float64 (on the device)."""
    a = (dX.double() * X.double()).sum().item()
    b = (dY.double() * Y.double()).sum().item()
    return a, b


def _row_loss(x, Y, pos_i, ids):
    lp = oracle.seq_dot(x, Y[pos_i][None, :])[0, 0]
    lg = oracle.seq_dot(x, Y[np.asarray(ids, dtype=np.int64)])[0] if len(ids) else np.zeros(0)
    return oracle.logsumexp(np.concatenate([[lp], lg])) - lp


def test_sasrec_full_size_against_oracle():
    w = WORKLOADS["sasrec"]
    inp = make_inputs(w)
    plan, saved, lpp, dX, dY, Xd, Yd = _run(w, inp)
    rows = np.sort(np.random.default_rng(123).choice(w.s, N_ROWS, replace=False))
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k, rows=rows)
    for r in range(w.rounds):
        assert np.array_equal(plan.export(saved, "bucket_x", r).cpu().numpy(), fwd["bx"][r])
        assert np.array_equal(plan.export(saved, "bucket_y", r).cpu().numpy(), fwd["by"][r])
        assert np.array_equal(plan.export(saved, "perm_x", r).cpu().numpy(), fwd["perm_x"][r])
        assert np.array_equal(plan.export(saved, "perm_y", r).cpu().numpy(), fwd["perm_y"][r])
        tid = plan.export(saved, "thresh_id", r).cpu().numpy()
        te = plan.export(saved, "thresh_logit", r).cpu().numpy()
        negs = plan.export(saved, "neg_ids", r).cpu().numpy()
        for i in rows:
            ids, _, thr = fwd["negs"][r][int(i)]
            assert thr is not None and tid[i] == thr[1] and te[i] == thr[0], (r, i)
            assert np.array_equal(np.sort(negs[i]), np.sort(ids)), (r, i)
    assert np.max(np.abs(lpp[rows] - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0)) <= 1e-3
    gX, _ = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    # the oracle's dX rows of the sampled positions are exact (a row depends on its own set only);
    # its gradient scale is 1/len(rows), the GPU's 1/s
    got = dX.cpu().numpy()[rows] * w.s / len(rows)
    assert grad_err(got, gX[rows]) <= 2e-3
    a, b = _bilinear(dX, dY, Xd, Yd)
    assert abs(a - b) <= 2e-3 * max(abs(a), abs(b), 1e-12)


def _check_sort(keys, perm):
    n = len(keys)
    assert np.array_equal(np.sort(perm), np.arange(n))
    k = keys[perm]
    assert np.all(k[1:] >= k[:-1])
    same = k[1:] == k[:-1]
    assert np.all(perm[1:][same] > perm[:-1][same])     # stable


@pytest.mark.parametrize("name", ["million", "tenmillion"])
def test_rece_full_size_properties(name):
    w = WORKLOADS[name]
    inp = make_inputs(w)
    plan, saved, lpp, dX, dY, Xd, Yd = _run(w, inp)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.s, N_ROWS, replace=False))
    kept = {int(i): set() for i in rows}
    for r in range(w.rounds):
        bx = plan.export(saved, "bucket_x", r).cpu().numpy()
        by = plan.export(saved, "bucket_y", r).cpu().numpy()
        sx = rng.choice(w.s, N_BUCKET, replace=False)
        sy = rng.choice(w.C, N_BUCKET, replace=False)
        assert np.array_equal(bx[sx], oracle.bucket_ids(inp.X[sx], inp.B[r]))
        assert np.array_equal(by[sy], oracle.bucket_ids(inp.Y[sy], inp.B[r]))
        px = plan.export(saved, "perm_x", r).cpu().numpy()
        py = plan.export(saved, "perm_y", r).cpu().numpy()
        _check_sort(bx, px)
        _check_sort(by, py)
        negs = plan.export(saved, "neg_ids", r).cpu().numpy()
        tid = plan.export(saved, "thresh_id", r).cpu().numpy()
        want = oracle.round_negatives(inp.X, inp.Y, inp.pos, px, py, w.n_c, w.k, rows=rows)
        for i in rows:
            ids, _, thr = want[int(i)]
            assert np.array_equal(np.sort(negs[i]), np.sort(ids)), (name, r, i)
            assert thr is not None and tid[i] == thr[1], (name, r, i)
            kept[int(i)] |= set(ids.tolist())
    ce = _full_ce_rows(inp.X[rows], inp.Y, inp.pos[rows])
    for n, i in enumerate(rows):
        li = _row_loss(inp.X[i], inp.Y, int(inp.pos[i]), sorted(kept[int(i)]))
        assert abs(lpp[i] - li) <= 1e-3 * max(abs(li), 1.0), (name, i, lpp[i], li)
        assert -1e-6 <= lpp[i] <= ce[n] * (1 + 1e-3) + 1e-6
    a, b = _bilinear(dX, dY, Xd, Yd)
    assert abs(a - b) <= 2e-3 * max(abs(a), abs(b), 1e-12)


def test_sce_full_size_properties():
    w = WORKLOADS["sce"]
    inp = make_inputs(w)
    plan, saved, lpp, dX, dY, Xd, Yd = _run(w, inp)
    R = plan.export(saved, "sce_rows").cpu().numpy()
    Q = plan.export(saved, "sce_items").cpu().numpy()
    rng = np.random.default_rng(9)
    B = inp.B[0].astype(np.float64)
    for b in rng.choice(w.n_b, 3, replace=False):   # whole columns, the oracle's own scores
        assert np.array_equal(np.sort(R[b]), oracle.column_top(oracle.seq_dot(inp.X, B[:, b][None, :])[:, 0], w.b_x))
        assert np.array_equal(np.sort(Q[b]), oracle.column_top(oracle.seq_dot(inp.Y, B[:, b][None, :])[:, 0], w.b_y))
    negs = plan.export(saved, "neg_ids").cpu().numpy()
    member = {}
    for b in range(w.n_b):
        for i in R[b]:
            member.setdefault(int(i), []).append(b)
    rows = np.sort(rng.choice(list(member), N_ROWS, replace=False))
    for i in rows:
        # the kept set is the oracle's top-k of the union of the GPU's bucket lists of i
        per = {}
        for b in member[int(i)]:
            items = Q[b][Q[b] != inp.pos[i]].astype(np.int64)
            lg = oracle.seq_dot(inp.X[i], inp.Y[items])[0]
            per[(b, int(i))] = oracle.sce._top_k(items, lg, w.k) + (len(items),)
        ids, _, _ = oracle.merge_negatives(per, w.s, w.k)[int(i)]
        got = negs[i][negs[i] >= 0]
        assert np.array_equal(np.sort(got), np.sort(ids)), i
        li = _row_loss(inp.X[i], inp.Y, int(inp.pos[i]), ids)
        assert abs(lpp[i] - li) <= 1e-3 * max(abs(li), 1.0), (i, lpp[i], li)
    uncovered = np.setdiff1d(np.arange(w.s), np.array(list(member)))
    assert np.all(lpp[uncovered] == 0.0)
    a, b = _bilinear(dX, dY, Xd, Yd)
    assert abs(a - b) <= 2e-3 * max(abs(a), abs(b), 1e-12)


def test_bucketing_ties_on_large_input_decided_in_float64():
    """Inputs large enough for the multi-fragment bucketing kernel, whose undecided
    rows go to the float64 list kernel: random vector 1 equals vector 0, so every
    row whose best vector is one of the two has a zero float32 gap and must get
    index 0 (lowest index among equal float64 scores, the oracle's rule)."""
    w = scaled("million", seqs=16, seqlen=256, C=600_000, n_b=64, n_c=64, k=32, rounds=1)
    inp = make_inputs(w)
    inp.B[0][:, 1] = inp.B[0][:, 0]
    X, Y, pos, B = to_device(inp)
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, keep_stages=True,
                     validate_ids=True)
    print("[gpu] bucketing ties, C=600000", flush=True)
    loss, lpp, scratch, saved = plan.forward(X, Y, pos, B)
    plan.check(saved)
    by = plan.export(saved, "bucket_y", 0).cpu().numpy()
    cnt = plan.export(saved, "counters").cpu().numpy()
    torch.cuda.synchronize()
    assert not np.any(by == 1)                 # the duplicate never wins
    rng = np.random.default_rng(11)
    tied = np.flatnonzero(by == 0)
    assert len(tied) > 1000                    # about 1 in 32 items
    sy = np.concatenate([rng.choice(tied, 256, replace=False), rng.choice(w.C, 2048, replace=False)])
    assert np.array_equal(by[sy], oracle.bucket_ids(inp.Y[sy], inp.B[0]))
    assert cnt[1] >= len(tied)                 # each of them went through the float64 decision
