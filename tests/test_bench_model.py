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


def test_window_logits_ragged_chunks():
    # chunk sizes differing by one (C not divisible by n_c): brute force over positions
    w = WORKLOADS["sasrec"]
    import dataclasses
    w = dataclasses.replace(w, seqs=1, seqlen=101, C=1003, n_c=7, n_b=7)
    xs, ys = bench.chunk_starts(w.s, w.n_c), bench.chunk_starts(w.C, w.n_c)
    chunk_of_item = [max(c for c in range(w.n_c) if ys[c] <= j) for j in range(w.C)]
    brute = 0
    for i in range(w.s):
        c = max(q for q in range(w.n_c) if xs[q] <= i)
        win = {(c - 1) % w.n_c, c, (c + 1) % w.n_c}
        brute += sum(1 for j in range(w.C) if chunk_of_item[j] in win)
    assert bench.window_logits(w) == brute


def test_select_roofline_is_alu_bound():
    w = WORKLOADS["sasrec"]
    flops, _ = bench.algorithmic_work(w)["select"]
    per_launch = flops / w.rounds
    assert per_launch == bench.ALU_OPS_PER_LOGIT * 72_000_000
    r = bench.roofline("select", 0.5, per_launch, 1.0, "bf16")
    assert r["bound"] == "alu" and r["unit"] == "Tops/s"
    assert r["frac"] == pytest.approx(per_launch / 0.5e-3 / 1e12 / bench.PEAK_ALU_TOPS)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
