"""Host-side parts of bench.py: the work model its roofline divides by, and the
one-GPU contract (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rece_inputs import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("name,expected", [
    ("tiny", 96_000),               # 256 positions x a window of 3 x 125 items
    ("tiny_fullce", 512_000),       # one chunk: the whole catalogue of 2,000
    ("sasrec", 72_000_000),
    ("million", 300_000_000),
    ("tenmillion", 960_000_000),
])
def test_window_logits_closed_form(name, expected):
    # cyclic window {c-1, c, c+1}: with n_c >= 3 every item chunk lies in exactly three
    # windows, so the sum over positions is (s / n_c) * 3C when n_c divides s; with
    # n_c <= 2 the window is the whole catalogue, s * C
    w = WORKLOADS[name]
    closed = w.s * w.C if w.n_c <= 2 else (w.s // w.n_c) * 3 * w.C
    assert w.s % w.n_c == 0
    assert bench.window_logits(w) == closed == expected


@pytest.mark.parametrize("n_ec,wrap", [(1, True), (2, True), (1, False), (3, False)])
def test_window_logits_ragged_chunks(n_ec, wrap):
    # chunk sizes differing by one (C not divisible by n_c): brute force over positions
    w = WORKLOADS["sasrec"]
    import dataclasses
    w = dataclasses.replace(w, seqs=1, seqlen=101, C=1003, n_c=7, n_b=7, n_ec=n_ec, window_wrap=wrap)
    xs, ys = bench.chunk_starts(w.s, w.n_c), bench.chunk_starts(w.C, w.n_c)
    chunk_of_item = [max(c for c in range(w.n_c) if ys[c] <= j) for j in range(w.C)]
    brute = 0
    for i in range(w.s):
        c = max(q for q in range(w.n_c) if xs[q] <= i)
        win = {(c + t) % w.n_c if wrap else c + t for t in range(-n_ec, n_ec + 1)}
        brute += sum(1 for j in range(w.C) if chunk_of_item[j] in win)
    assert bench.window_logits(w) == brute


def test_select_work_and_both_fractions():
    w = WORKLOADS["tenmillion"]
    flops, nbytes = bench.algorithmic_work(w)["select"]
    # every window logit is a d-long scalar product (2 flops per coordinate), every round
    assert flops == 2.0 * w.d * 960_000_000 * w.rounds
    # every position and item vector once per round, and the kept ids
    assert nbytes == w.rounds * ((w.s + w.C) * w.d * 2 + w.s * w.k * 4)
    fr = bench.fractions(2.0, flops / w.rounds, nbytes / w.rounds, "bf16",
                         {"bf16_tflops": 2000.0, "copy_gbs": 5000.0})
    t = 2.0e-3
    assert fr["bound"] == "hbm"            # 92 flop per byte, far below the bf16 ridge
    assert fr["mfma_frac"] == pytest.approx(flops / w.rounds / t / 2.5e15, rel=1e-3)
    assert fr["hbm_frac"] == pytest.approx(nbytes / w.rounds / t / 8e12, rel=1e-3)
    assert fr["mfma_frac_measured_peak"] == pytest.approx(flops / w.rounds / t / 2.0e15, rel=1e-3)
    assert fr["hbm_frac_measured_peak"] == pytest.approx(nbytes / w.rounds / t / 5.0e12, rel=1e-3)
    # the projection at 1,024 buckets sits above the ridge: matrix-core bound
    pf, pb = bench.algorithmic_work(w)["project"]
    assert bench.fractions(1.0, pf, pb, "bf16", None)["bound"] == "mfma"


def test_cpu_baseline_extrapolation_on_a_small_workload():
    # the baseline runs the oracle on samples and extrapolates; on a workload small
    # enough that the samples cover everything the terms must still be positive and
    # the formula's inputs recorded
    from rece_inputs import make_inputs, scaled
    w = scaled("sasrec", seqs=2, seqlen=64, C=600, n_b=4, n_c=4, k=8, rounds=2)
    res = bench.cpu_baseline(make_inputs(w), per_worker_items=64, chunks_per_worker=1)
    assert res["kind"] == "oracle" and res["value"] > 0
    assert res["threads"] == res["cores"] >= 1 and res["nproc"] >= 1 and res["cpu_model"]
    assert all(v >= 0 for v in res["terms_s"].values())


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
