"""A forward + backward step captured into a HIP graph (torch.cuda.CUDAGraph on
a side stream) and replayed: every replay, with eager steps and host
synchronisations in between, gives the eager result bit for bit (the step is
deterministic: no float atomics, the plan's extra stream is forked and joined
with events, and no memset nodes are recorded)."""
import numpy as np
import pytest
import torch

import catalogue_cross_entropy_amd as rece
from gpu_helpers import to_device
from rece_inputs import make_inputs, scaled

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    w = scaled("sasrec", seqs=4, seqlen=300, C=6000, n_b=16, n_c=16, k=64, rounds=2)
    inp = make_inputs(w)
    X, Y, pos, B = to_device(inp)
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype)
    dev = X.device
    scratch, saved = plan.workspace(dev)
    dX = torch.empty((w.s, w.d), dtype=torch.float32, device=dev)
    dY = torch.empty((w.C, w.d), dtype=torch.float32, device=dev)
    dloss = torch.ones(1, dtype=torch.float32, device=dev)
    out = {}

    def step(stream=None):
        loss, lpp, _, _ = plan.forward(X, Y, pos, B, scratch, saved, stream=stream)
        plan.backward(X, Y, pos, scratch, saved, dloss=dloss, dX=dX, dY=dY, stream=stream)
        out["loss"], out["lpp"] = loss, lpp

    print("[gpu] graph capture, eager reference", flush=True)
    step()
    torch.cuda.synchronize()
    ref = (out["loss"].clone(), out["lpp"].clone(), dX.clone(), dY.clone())

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(stream=s)
    torch.cuda.synchronize()
    gl, glpp = out["loss"], out["lpp"]   # the graph's own output buffers
    for r in range(3):
        print(f"[gpu] graph replay {r}", flush=True)
        for t in (dX, dY, gl, glpp):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = (gl, glpp, dX, dY)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), r
        step()   # eager work between replays
        torch.cuda.synchronize()
