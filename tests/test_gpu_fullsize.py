"""GPU results at the full workload sizes, in the launch configuration bench.py
times, compared element by element with the oracle.

* sasrec (s = 51,200, C = 30,000): the whole oracle over every position: bucket
  ids, orders, every threshold and kept set, every per-position loss, the mean
  loss, and every element of dX and dY.
* million and ten million items, and the bucket variant: the oracle cannot
  select over every window in a test's time, so the selection is checked on
  samples and everything after it on every position:
  - bucket ids: all of them at a million items (both rounds); at ten million,
    every position and whole contiguous blocks of items (the first and last
    4,096, and random blocks);
  - the sort is the stable permutation of the GPU's bucket ids (one result);
  - the kept set (and threshold) of sampled positions is the oracle's top-k of
    the window that sort defines;
  - given the GPU's kept sets (the oracle's injection point,
    oracle.loss_from_negatives), the oracle's loss of every position, the mean
    loss and every element of dX and dY; rows of items that no position scores
    are exactly zero.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import catalogue_cross_entropy_amd as rece
import oracle
from gpu_helpers import to_device
from rece_inputs import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

N_ROWS = 64        # sampled positions for the selection
LOSS_TOL = {"f32": 1e-5, "bf16": 1e-3}
GRAD_TOL = 2e-3


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 4


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
    out = {"loss": loss.item(), "lpp": lpp.cpu().numpy(), "dX": dX.cpu().numpy(), "dY": dY.cpu().numpy()}
    del dX, dY, X, Y, B, pos
    torch.cuda.empty_cache()
    return plan, saved, out


def _bucket_ids(V, B_round, rows=None, block=8192):
    """oracle.bucket_ids over many rows, blocks of rows on a thread pool (NumPy
    releases the interpreter lock inside its array loops)."""
    idx = np.arange(V.shape[0]) if rows is None else np.asarray(rows)
    blocks = [idx[i:i + block] for i in range(0, len(idx), block)]
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda b: oracle.bucket_ids(V[b], B_round), blocks))
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def _check_sort(keys, perm):
    n = len(keys)
    assert np.array_equal(np.sort(perm), np.arange(n))
    k = keys[perm]
    assert np.all(k[1:] >= k[:-1])
    same = k[1:] == k[:-1]
    assert np.all(perm[1:][same] > perm[:-1][same])     # stable


def _kept(negs_r, s):
    """{position: kept ids} of one round from the exported [s, k] array (-1: empty)."""
    return {i: negs_r[i][negs_r[i] >= 0].astype(np.int64) for i in range(s)}


def _injected(inp, X64, Y64, kept_rounds, rows=None):
    """The oracle's loss and gradients given the kept sets (upstream 1/s per position,
    the gradient of the mean over all s positions)."""
    s = X64.shape[0]
    fwd = oracle.loss_from_negatives(X64, Y64, inp.pos, kept_rounds, rows=rows)
    gX, gY = oracle.rece_backward(X64, Y64, inp.pos, fwd, dloss_pp=np.full(s, 1.0 / s))
    return fwd, gX, gY


def _check_grads(got, want, what, block=1 << 20):
    """max |got - want| <= GRAD_TOL * max |want|, in row blocks (no full-size temporaries)."""
    num = den = 0.0
    for r0 in range(0, want.shape[0], block):
        g, h = got[r0:r0 + block], want[r0:r0 + block]
        num = max(num, float(np.abs(g - h).max()))
        den = max(den, float(np.abs(h).max()))
    err = num / max(den, 1e-30)
    assert err <= GRAD_TOL, (what, err)


@pytest.mark.timeout(600)
def test_sasrec_full_size_against_oracle():
    w = WORKLOADS["sasrec"]
    inp = make_inputs(w)
    plan, saved, out = _run(w, inp)
    print("[oracle] sasrec, every position", flush=True)
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k)
    for r in range(w.rounds):
        assert np.array_equal(plan.export(saved, "bucket_x", r).cpu().numpy(), fwd["bx"][r])
        assert np.array_equal(plan.export(saved, "bucket_y", r).cpu().numpy(), fwd["by"][r])
        assert np.array_equal(plan.export(saved, "perm_x", r).cpu().numpy(), fwd["perm_x"][r])
        assert np.array_equal(plan.export(saved, "perm_y", r).cpu().numpy(), fwd["perm_y"][r])
        tid = plan.export(saved, "thresh_id", r).cpu().numpy()
        te = plan.export(saved, "thresh_logit", r).cpu().numpy()
        negs = plan.export(saved, "neg_ids", r).cpu().numpy()
        for i in range(w.s):
            ids, _, thr = fwd["negs"][r][i]
            assert thr is not None and tid[i] == thr[1] and te[i] == thr[0], (r, i)
            assert np.array_equal(np.sort(negs[i]), np.sort(ids)), (r, i)
    tol = LOSS_TOL[w.dtype]
    lpp = out["lpp"]
    assert np.max(np.abs(lpp - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0)) <= tol
    assert abs(out["loss"] - fwd["loss"]) <= tol * max(abs(fwd["loss"]), 1.0)
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    _check_grads(out["dX"], gX, "dX")
    _check_grads(out["dY"], gY, "dY")


def _selection_sample(w, inp, plan, saved, rows):
    """Kept sets and thresholds of sampled positions against the oracle's top-k of
    the windows the GPU's (checked) sort defines; returns every round's kept sets."""
    kept_rounds = []
    for r in range(w.rounds):
        bx = plan.export(saved, "bucket_x", r).cpu().numpy()
        by = plan.export(saved, "bucket_y", r).cpu().numpy()
        px = plan.export(saved, "perm_x", r).cpu().numpy()
        py = plan.export(saved, "perm_y", r).cpu().numpy()
        _check_sort(bx, px)
        _check_sort(by, py)
        negs = plan.export(saved, "neg_ids", r).cpu().numpy()
        tid = plan.export(saved, "thresh_id", r).cpu().numpy()
        te = plan.export(saved, "thresh_logit", r).cpu().numpy()
        want = oracle.round_negatives(inp.X, inp.Y, inp.pos, px, py, w.n_c, w.k, rows=rows)
        for i in rows:
            ids, _, thr = want[int(i)]
            assert np.array_equal(np.sort(negs[i]), np.sort(ids)), (w.name, r, i)
            assert thr is not None and tid[i] == thr[1] and te[i] == thr[0], (w.name, r, i)
        kept_rounds.append(_kept(negs, w.s))
    return kept_rounds


def _boundary_rows(n, block, rng, extra_blocks=2):
    """The first and last `block` indices and a few random contiguous blocks."""
    starts = [0, n - block] + [int(x) for x in rng.integers(0, n - block, size=extra_blocks)]
    return np.unique(np.concatenate([np.arange(a, a + block) for a in starts]))


@pytest.mark.timeout(600)
def test_million_full_size():
    w = WORKLOADS["million"]
    inp = make_inputs(w)
    plan, saved, out = _run(w, inp)
    print("[oracle] million: every bucket id", flush=True)
    for r in range(w.rounds):
        assert np.array_equal(plan.export(saved, "bucket_x", r).cpu().numpy(), _bucket_ids(inp.X, inp.B[r]))
        assert np.array_equal(plan.export(saved, "bucket_y", r).cpu().numpy(), _bucket_ids(inp.Y, inp.B[r]))
    rows = np.sort(np.random.default_rng(7).choice(w.s, N_ROWS, replace=False))
    print("[oracle] million: sampled selections", flush=True)
    kept_rounds = _selection_sample(w, inp, plan, saved, rows)
    print("[oracle] million: loss and gradients of every position, given the kept sets", flush=True)
    X64, Y64 = inp.X.astype(np.float64), inp.Y.astype(np.float64)
    fwd, gX, gY = _injected(inp, X64, Y64, kept_rounds)
    tol = LOSS_TOL[w.dtype]
    assert np.max(np.abs(out["lpp"] - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0)) <= tol
    assert abs(out["loss"] - fwd["loss"]) <= tol * max(abs(fwd["loss"]), 1.0)
    _check_grads(out["dX"], gX, "dX")
    _check_grads(out["dY"], gY, "dY")


@pytest.mark.timeout(900)
def test_tenmillion_full_size():
    w = WORKLOADS["tenmillion"]
    inp = make_inputs(w)
    plan, saved, out = _run(w, inp)
    rng = np.random.default_rng(13)
    yrows = _boundary_rows(w.C, 4096, rng)
    print(f"[oracle] ten million: every position's bucket id, {len(yrows)} item rows", flush=True)
    for r in range(w.rounds):
        assert np.array_equal(plan.export(saved, "bucket_x", r).cpu().numpy(), _bucket_ids(inp.X, inp.B[r]))
        by = plan.export(saved, "bucket_y", r).cpu().numpy()
        assert np.array_equal(by[yrows], _bucket_ids(inp.Y, inp.B[r], yrows))
    rows = np.sort(rng.choice(w.s, N_ROWS, replace=False))
    print("[oracle] ten million: sampled selections", flush=True)
    kept_rounds = _selection_sample(w, inp, plan, saved, rows)
    listed = np.zeros(w.C, dtype=bool)
    for kr in kept_rounds:
        for ids in kr.values():
            listed[ids] = True
    listed[inp.pos] = True
    print("[oracle] ten million: loss and gradients of every position, given the kept sets", flush=True)
    X64, Y64 = inp.X.astype(np.float64), inp.Y.astype(np.float64)
    fwd, gX, gY = _injected(inp, X64, Y64, kept_rounds)
    tol = LOSS_TOL[w.dtype]
    assert np.max(np.abs(out["lpp"] - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0)) <= tol
    assert abs(out["loss"] - fwd["loss"]) <= tol * max(abs(fwd["loss"]), 1.0)
    _check_grads(out["dX"], gX, "dX")
    _check_grads(out["dY"], gY, "dY")
    # items no position scores: exactly zero rows (the dense dY is written everywhere)
    assert not np.any(out["dY"][~listed])


@pytest.mark.timeout(600)
def test_sce_full_size():
    w = WORKLOADS["sce"]
    inp = make_inputs(w)
    plan, saved, out = _run(w, inp)
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
    print("[oracle] bucket variant: sampled selections", flush=True)
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
    uncovered = np.setdiff1d(np.arange(w.s), np.array(list(member)))
    assert np.all(out["lpp"][uncovered] == 0.0)
    print("[oracle] bucket variant: loss and gradients of every position, given the kept sets", flush=True)
    X64, Y64 = inp.X.astype(np.float64), inp.Y.astype(np.float64)
    fwd, gX, gY = _injected(inp, X64, Y64, [_kept(negs, w.s)])
    tol = LOSS_TOL[w.dtype]
    assert np.max(np.abs(out["lpp"] - fwd["loss_pp"]) / np.maximum(np.abs(fwd["loss_pp"]), 1.0)) <= tol
    assert abs(out["loss"] - fwd["loss"]) <= tol * max(abs(fwd["loss"]), 1.0)
    _check_grads(out["dX"], gX, "dX")
    _check_grads(out["dY"], gY, "dY")


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


def test_bucketing_many_equal_vectors_on_large_input():
    """Random vector 0 is copied to vectors 1, 2, 3, 16, 17, 18 and 19, which one
    lane of the float64 list kernel scores together: rows whose best vector is a
    copy have eight equal float32 scores in that lane's share, more than its four
    kept keys, so they take the kernel's fallback over every vector in float64.
    Each must get index 0 (lowest index among equal float64 scores)."""
    w = scaled("million", seqs=16, seqlen=256, C=600_000, n_b=64, n_c=64, k=32, rounds=1)
    inp = make_inputs(w)
    for j in (1, 2, 3, 16, 17, 18, 19):
        inp.B[0][:, j] = inp.B[0][:, 0]
    X, Y, pos, B = to_device(inp)
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, keep_stages=True,
                     validate_ids=True)
    print("[gpu] bucketing, eight equal vectors, C=600000", flush=True)
    loss, lpp, scratch, saved = plan.forward(X, Y, pos, B)
    plan.check(saved)
    by = plan.export(saved, "bucket_y", 0).cpu().numpy()
    torch.cuda.synchronize()
    assert not np.any(np.isin(by, [1, 2, 3, 16, 17, 18, 19]))   # a copy never wins
    rng = np.random.default_rng(12)
    tied = np.flatnonzero(by == 0)
    assert len(tied) > 1000
    sy = np.concatenate([rng.choice(tied, 256, replace=False), rng.choice(w.C, 2048, replace=False)])
    assert np.array_equal(by[sy], oracle.bucket_ids(inp.Y[sy], inp.B[0]))
