"""The exact full cross-entropy entry points (no [s, C] tensor on the GPU)
against the oracle's full cross-entropy and its gradient (RECE page, Eq. 3 and
Eq. 4), and against the reduced loss in its degenerate full-CE configuration
(one bucket, one chunk, k = C - 1: every item is scored)."""
import numpy as np
import pytest
import torch

import catalogue_cross_entropy_amd as rece
import oracle
from gpu_helpers import grad_err, run_rece, to_device
from rece_inputs import WORKLOADS, make_inputs, scaled

pytestmark = pytest.mark.gpu

LOSS_TOL = {"f32": 1e-5, "bf16": 1e-3}


def _full_ce(inp, dloss_pp=None):
    w = inp.w
    X, Y, pos, _ = to_device(inp)
    f = rece.FullCE(w.s, w.C, w.d, dtype=w.dtype)
    print(f"[gpu] full CE s={w.s} C={w.C} d={w.d} dtype={w.dtype}", flush=True)
    loss, lpp, ws = f.forward(X, Y, pos)
    dpp = None if dloss_pp is None else torch.from_numpy(dloss_pp.astype(np.float32)).cuda()
    dX, dY = f.backward(X, Y, pos, ws, dloss_pp=dpp)
    torch.cuda.synchronize()
    return loss.item(), lpp.cpu().numpy(), dX.cpu().numpy(), dY.cpu().numpy()


CASES = {
    "tiny_f32": scaled("tiny", C=2000),
    "ragged_f32_d32": scaled("tiny", seqs=3, seqlen=67, C=1237, d=32, seed=21),
    "bf16_d128_ragged": scaled("sasrec", seqs=3, seqlen=101, C=3001, d=128, n_b=4, n_c=4, k=8, rounds=1, seed=22),
    "bf16_d64": scaled("sasrec", seqs=8, seqlen=64, C=5000, d=64, n_b=4, n_c=4, k=8, rounds=1, seed=23),
    "f32_d256": scaled("tiny", seqs=2, seqlen=48, C=700, d=256, seed=24),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_ce_against_oracle(name):
    w = CASES[name]
    inp = make_inputs(w)
    loss, lpp, dX, dY = _full_ce(inp)
    want = oracle.full_ce(inp.X, inp.Y, inp.pos)
    tol = LOSS_TOL[w.dtype]
    assert np.max(np.abs(lpp - want) / np.maximum(np.abs(want), 1.0)) <= tol
    assert abs(loss - want.mean()) <= tol * max(abs(want.mean()), 1.0)
    gX, gY = oracle.full_ce_grad(inp.X, inp.Y, inp.pos)
    assert grad_err(dX, gX) <= 2e-3
    assert grad_err(dY, gY) <= 2e-3


def test_full_ce_per_position_upstream_and_repeatable():
    w = CASES["bf16_d64"]
    inp = make_inputs(w)
    g = np.random.default_rng(5).standard_normal(w.s).astype(np.float32)
    _, _, dX, dY = _full_ce(inp, dloss_pp=g)
    _, _, dX2, dY2 = _full_ce(inp, dloss_pp=g)
    assert np.array_equal(dX, dX2) and np.array_equal(dY, dY2)      # no atomics: identical bits
    # the gradient of sum_i g_i loss_i is the mean-loss gradient with per-row weights g_i * s
    from scipy.special import softmax
    L = inp.X.astype(np.float64) @ inp.Y.astype(np.float64).T
    P = softmax(L, axis=1)
    P[np.arange(w.s), inp.pos] -= 1.0
    G = P * g[:, None].astype(np.float64)
    assert grad_err(dX, G @ inp.Y.astype(np.float64)) <= 2e-3
    assert grad_err(dY, G.T @ inp.X.astype(np.float64)) <= 2e-3


def test_reduced_loss_with_every_item_scored_equals_full_ce():
    """One bucket, one chunk, k = C - 1 (RECE page, Section 3: the window is the
    whole catalogue, every negative kept): the reduced loss and its gradients are
    the full cross-entropy's, computed by the two independent GPU paths."""
    w = WORKLOADS["tiny_fullce"]
    inp = make_inputs(w)
    red = run_rece(inp, keep_stages=False)
    loss, lpp, dX, dY = _full_ce(inp)
    assert np.max(np.abs(red["loss_pp"] - lpp) / np.maximum(np.abs(lpp), 1.0)) <= 1e-5
    assert grad_err(red["dX"], dX) <= 2e-3 and grad_err(red["dY"], dY) <= 2e-3


def test_full_ce_at_scale_sampled_rows():
    """s = 8,192, C = 200,000, d = 128, bf16: sampled rows against the oracle
    (loss and dX rows depend on their own row only), and sum_i dX_i . x_i =
    sum_j dY_j . y_j for the whole gradient."""
    w = scaled("million", seqs=32, seqlen=256, C=200_000, d=128, n_b=4, n_c=4, k=8, rounds=1, seed=25)
    inp = make_inputs(w)
    loss, lpp, dX, dY = _full_ce(inp)
    rows = np.sort(np.random.default_rng(3).choice(w.s, 24, replace=False))
    want = oracle.full_ce(inp.X[rows], inp.Y, inp.pos[rows])
    assert np.max(np.abs(lpp[rows] - want) / np.maximum(np.abs(want), 1.0)) <= 1e-3
    gX, _ = oracle.full_ce_grad(inp.X[rows], inp.Y, inp.pos[rows])
    assert grad_err(dX[rows] * w.s / len(rows), gX) <= 2e-3
    a = float((dX.astype(np.float64) * inp.X).sum())
    b = float((dY.astype(np.float64) * inp.Y).sum())
    assert abs(a - b) <= 2e-3 * max(abs(a), abs(b), 1e-12)
