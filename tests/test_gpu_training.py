"""What a training loop needs around the loss: a padding mask (negative positive
ids), bf16 gradient outputs and the torch.autograd wrapper, all against the
oracle or against the float32 path of the same kernels."""
import numpy as np
import pytest
import torch

import catalogue_cross_entropy_amd as rece
import oracle
from gpu_helpers import grad_err, to_device
from rece_inputs import make_inputs, scaled

pytestmark = pytest.mark.gpu


def _padded(w, frac=0.25, seed=6):
    inp = make_inputs(w)
    pad = np.random.default_rng(seed).random(w.s) < frac
    inp.pos[pad] = -1
    return inp, pad


def _plan(w, **kw):
    if w.variant == "sce":
        return rece.Plan(w.s, w.C, w.d, w.n_b, 0, w.k, 1, dtype=w.dtype, variant="sce", b_x=w.b_x, b_y=w.b_y,
                         validate_ids=True, **kw)
    return rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, validate_ids=True,
                     n_ec=w.n_ec, window_wrap=w.window_wrap, **kw)


def _run(w, inp, **kw):
    X, Y, pos, B = to_device(inp)
    if w.variant == "sce":
        B = B[0].contiguous()
    plan = _plan(w, **kw)
    print(f"[gpu] {w.name} s={w.s} C={w.C} d={w.d} {kw}", flush=True)
    loss, lpp, scratch, saved = plan.forward(X, Y, pos, B)
    dX, dY = plan.backward(X, Y, pos, scratch, saved)
    plan.check(saved)
    torch.cuda.synchronize()
    return loss.item(), lpp.cpu(), dX.cpu(), dY.cpu()


RECE_W = scaled("sasrec", seqs=4, seqlen=60, C=1800, n_b=8, n_c=8, k=24, rounds=2, seed=41)
SCE_W = scaled("sce", seqs=4, seqlen=64, C=2500, d=64, n_b=8, b_x=64, b_y=300, k=24, seed=42)


def test_padding_mask_rece():
    w = RECE_W
    inp, pad = _padded(w)
    loss, lpp, dX, dY = _run(w, inp, ignore_negative_pos=True)
    f = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k, ignore_negative=True)
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, f)
    lpp = lpp.numpy()
    assert np.all(lpp[pad] == 0.0) and np.all(dX.numpy()[pad] == 0.0)
    assert np.max(np.abs(lpp - f["loss_pp"]) / np.maximum(np.abs(f["loss_pp"]), 1.0)) <= 1e-3
    assert abs(loss - f["loss"]) <= 1e-3 * max(abs(f["loss"]), 1.0)
    assert grad_err(dX.numpy(), gX) <= 2e-3 and grad_err(dY.numpy(), gY) <= 2e-3


def test_padding_mask_sce():
    w = SCE_W
    inp, pad = _padded(w)
    loss, lpp, dX, dY = _run(w, inp, ignore_negative_pos=True)
    f = oracle.sce_forward(inp.X, inp.Y, inp.pos, inp.B[0], w.b_x, w.b_y, w.k, ignore_negative=True)
    gX, gY = oracle.sce_backward(inp.X, inp.Y, inp.pos, f)
    lpp = lpp.numpy()
    assert np.all(lpp[pad] == 0.0)
    assert np.max(np.abs(lpp - f["loss_pp"]) / np.maximum(np.abs(f["loss_pp"]), 1.0)) <= 1e-3
    assert abs(loss - f["loss"]) <= 1e-3 * max(abs(f["loss"]), 1.0)
    assert grad_err(dX.numpy(), gX) <= 2e-3 and grad_err(dY.numpy(), gY) <= 2e-3


def test_every_position_padding_gives_zero():
    w = RECE_W
    inp = make_inputs(w)
    inp.pos[:] = -1
    loss, lpp, dX, dY = _run(w, inp, ignore_negative_pos=True)
    assert loss == 0.0 and not lpp.any() and not dX.any() and not dY.any()


@pytest.mark.parametrize("w", [RECE_W, SCE_W], ids=["rece", "sce"])
def test_bf16_gradients_are_the_float32_ones_rounded(w):
    inp = make_inputs(w)
    _, _, dX, dY = _run(w, inp)
    _, _, dXb, dYb = _run(w, inp, bf16_grads=True)
    assert dXb.dtype == torch.bfloat16 and dYb.dtype == torch.bfloat16
    # the same float32 values (the kernels are deterministic), rounded to nearest even
    assert torch.equal(dXb, dX.to(torch.bfloat16)) and torch.equal(dYb, dY.to(torch.bfloat16))


def test_autograd_wrapper():
    w = scaled("tiny", seqs=2, seqlen=64, C=900, n_b=8, n_c=8, k=16, rounds=1, seed=43)
    inp = make_inputs(w)
    X, Y, pos, B = to_device(inp)
    plan = _plan(w)
    loss0, _, scratch, saved = plan.forward(X, Y, pos, B)
    # the library's backward with the upstream gradient autograd will pass (3)
    dX0, dY0 = plan.backward(X, Y, pos, scratch, saved, dloss=torch.full((1,), 3.0, device=X.device))
    Xg, Yg = X.clone().requires_grad_(True), Y.clone().requires_grad_(True)
    loss = rece.rece_loss(Xg, Yg, pos, B, plan)
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    assert loss.item() == loss0.item()
    assert torch.equal(Xg.grad, dX0) and torch.equal(Yg.grad, dY0)
    # bf16 inputs: bf16 gradients come back in the inputs' dtype
    wb = scaled("sasrec", seqs=2, seqlen=64, C=900, n_b=8, n_c=8, k=16, rounds=1, seed=44)
    inb = make_inputs(wb)
    Xb, Yb, posb, Bb = to_device(inb)
    pb = _plan(wb, bf16_grads=True)
    Xb.requires_grad_(True)
    Yb.requires_grad_(True)
    rece.rece_loss(Xb, Yb, posb, Bb, pb).backward()
    assert Xb.grad.dtype == torch.bfloat16 and Yb.grad.dtype == torch.bfloat16
    f = oracle.rece_forward(inb.X, inb.Y, inb.pos, inb.B, wb.n_c, wb.k)
    gX, gY = oracle.rece_backward(inb.X, inb.Y, inb.pos, f)
    assert grad_err(Xb.grad.float().cpu().numpy(), gX) <= 5e-3


def test_auto_sized_plan_matches_oracle():
    """A plan sized by the page's rule (n_b* and n_c from rece_auto_size) on a small
    workload: the GPU result equals the oracle's at those sizes."""
    base = scaled("sasrec", seqs=4, seqlen=64, C=3000, n_b=8, n_c=8, k=16, rounds=2, seed=45)
    a = rece.auto_size(base.s, base.C, base.n_ec, 1.0, base.rounds)
    w = base.with_(n_b=a["n_b"], n_c=a["n_c"])
    inp = make_inputs(w)
    loss, lpp, dX, dY = _run(w, inp)
    f = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k)
    gX, gY = oracle.rece_backward(inp.X, inp.Y, inp.pos, f)
    assert np.max(np.abs(lpp.numpy() - f["loss_pp"]) / np.maximum(np.abs(f["loss_pp"]), 1.0)) <= 1e-3
    assert grad_err(dX.numpy(), gX) <= 2e-3 and grad_err(dY.numpy(), gY) <= 2e-3
