"""rece_forward_static, the forward entry point that allocates nothing (its
scratch is the library's static device array), called through the C ABI and
compared with rece_forward on the same inputs: the loss, the per-position
losses, every round's thresholds and kept sets, and the gradients of a backward
pass from the saved buffer each of them wrote, all bit for bit.  Two calls in a
row, the second on a smaller input (the array keeps the first call's contents),
for both variants."""
import numpy as np
import pytest
import torch

import catalogue_cross_entropy_amd as rece
from gpu_helpers import to_device
from rece_inputs import make_inputs, scaled

pytestmark = pytest.mark.gpu

CALLS = [
    scaled("sasrec", seqs=3, seqlen=300, C=5003, n_b=16, n_c=16, k=64, rounds=2),
    scaled("sasrec", seqs=2, seqlen=64, C=1200, n_b=6, n_c=6, k=24, rounds=3),
]
SCE_CALLS = [
    scaled("sce", seqs=2, seqlen=128, C=4000, d=64, n_b=12, b_x=64, b_y=300, k=32),
    scaled("sce", seqs=1, seqlen=100, C=1500, d=64, n_b=5, b_x=30, b_y=120, k=16),
]


def _stages(plan, saved, w):
    out = {"lse": plan.export(saved, "lse").cpu().numpy()}
    rounds = w.rounds if w.variant == "rece" else 1
    for r in range(rounds):
        for st in ("thresh_id", "thresh_logit"):
            out[(st, r)] = plan.export(saved, st, r).cpu().numpy()
        out[("neg_ids", r)] = np.sort(plan.export(saved, "neg_ids", r).cpu().numpy(), axis=1)
    return out


def _compare_one(w):
    inp = make_inputs(w)
    X, Y, pos, B = to_device(inp)
    if w.variant == "sce":
        B = B[0].contiguous()
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, variant=w.variant,
                     b_x=w.b_x, b_y=w.b_y)
    print(f"[gpu] static forward vs rece_forward: {w.variant} s={w.s} C={w.C} d={w.d} k={w.k}", flush=True)
    loss_r, lpp_r, scratch, saved_r = plan.forward(X, Y, pos, B)
    dX_r, dY_r = plan.backward(X, Y, pos, scratch, saved_r)
    torch.cuda.synchronize()
    ref = _stages(plan, saved_r, w)

    dev = X.device
    saved = torch.empty(plan.saved_bytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lpp = torch.empty(w.s, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    status = rece.lib().rece_forward_static(plan._h, st, X.data_ptr(), Y.data_ptr(), pos.data_ptr(), B.data_ptr(),
                                            saved.data_ptr(), loss.data_ptr(), lpp.data_ptr())
    assert status == 0, rece.lib().rece_last_error().decode()
    dX, dY = plan.backward(X, Y, pos, scratch, saved)
    plan.check(saved)
    torch.cuda.synchronize()
    got = _stages(plan, saved, w)
    assert torch.equal(loss, loss_r) and torch.equal(lpp, lpp_r)
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key
    assert torch.equal(dX, dX_r) and torch.equal(dY, dY_r)


@pytest.mark.parametrize("calls", [CALLS, SCE_CALLS], ids=["rece", "sce"])
def test_static_forward_matches_rece_forward(calls):
    for w in calls:   # the second call is smaller than the first
        _compare_one(w)
