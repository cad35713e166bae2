"""Shared helpers of the GPU tests: run librece on a seeded workload and gather
its outputs and kept stages as NumPy arrays."""
import numpy as np
import torch

import catalogue_cross_entropy_amd as rece


def to_device(inp):
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if inp.w.dtype == "bf16" else torch.float32
    X = torch.from_numpy(inp.X).to(dev).to(dt).contiguous()
    Y = torch.from_numpy(inp.Y).to(dev).to(dt).contiguous()
    B = torch.from_numpy(inp.B).to(dev).to(dt).contiguous()
    pos = torch.from_numpy(inp.pos).to(dev)
    return X, Y, pos, B


def run_rece(inp, keep_stages=True, backward=True, dloss_pp=None, tensors=None):
    w = inp.w
    X, Y, pos, B = tensors if tensors is not None else to_device(inp)
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype,
                     keep_stages=keep_stages, validate_ids=True, n_ec=w.n_ec, window_wrap=w.window_wrap)
    print(f"[gpu] rece s={w.s} C={w.C} d={w.d} n_b={w.n_b} n_c={w.n_c} n_ec={w.n_ec} "
          f"wrap={int(w.window_wrap)} k={w.k} r={w.rounds} dtype={w.dtype} seed={w.seed}", flush=True)
    loss, lpp, scratch, saved = plan.forward(X, Y, pos, B)
    out = {"loss": None}
    if backward:
        dpp = None if dloss_pp is None else torch.from_numpy(dloss_pp.astype(np.float32)).cuda()
        dX, dY = plan.backward(X, Y, pos, scratch, saved, dloss_pp=dpp)
    plan.check(saved)
    torch.cuda.synchronize()
    out["loss"] = loss.item()
    out["loss_pp"] = lpp.cpu().numpy()
    if backward:
        out["dX"] = dX.cpu().numpy()
        out["dY"] = dY.cpu().numpy()
    out["counters"] = plan.export(saved, "counters").cpu().numpy()
    out["lse"] = plan.export(saved, "lse").cpu().numpy()
    out["union_ids"] = plan.export(saved, "union_ids").cpu().numpy()
    for r in range(w.rounds):
        for st in ("bucket_x", "bucket_y", "perm_x", "perm_y", "thresh_id", "thresh_logit"):
            out[(st, r)] = plan.export(saved, st, r).cpu().numpy()
        if keep_stages:
            out[("neg_ids", r)] = plan.export(saved, "neg_ids", r).cpu().numpy()
    torch.cuda.synchronize()
    out["plan"] = plan
    return out


def run_sce(inp, keep_stages=True, backward=True, dloss_pp=None):
    """The bucket (SCE) variant on a seeded workload; B is the [d, n_b] slice."""
    w = inp.w
    X, Y, pos, B = to_device(inp)
    B = B[0].contiguous()
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, 0, w.k, 1, dtype=w.dtype, variant="sce", b_x=w.b_x, b_y=w.b_y,
                     keep_stages=keep_stages, validate_ids=True)
    print(f"[gpu] sce s={w.s} C={w.C} d={w.d} n_b={w.n_b} b_x={w.b_x} b_y={w.b_y} k={w.k} "
          f"dtype={w.dtype} seed={w.seed}", flush=True)
    loss, lpp, scratch, saved = plan.forward(X, Y, pos, B)
    out = {}
    if backward:
        dpp = None if dloss_pp is None else torch.from_numpy(dloss_pp.astype(np.float32)).cuda()
        dX, dY = plan.backward(X, Y, pos, scratch, saved, dloss_pp=dpp)
    plan.check(saved)
    torch.cuda.synchronize()
    out["loss"] = loss.item()
    out["loss_pp"] = lpp.cpu().numpy()
    if backward:
        out["dX"] = dX.cpu().numpy()
        out["dY"] = dY.cpu().numpy()
    for st in ("counters", "lse", "thresh_id", "thresh_logit", "sce_rows", "sce_items", "union_ids"):
        out[st] = plan.export(saved, st).cpu().numpy()
    if keep_stages:
        out["neg_ids"] = plan.export(saved, "neg_ids").cpu().numpy()
    torch.cuda.synchronize()
    return out


def grad_err(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))
