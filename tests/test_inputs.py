"""The seeded input generator: bf16 rounding, Zipf positives, determinism."""
import numpy as np
import torch

from rece_inputs import (WORKLOADS, from_bf16_bits, make_inputs, round_to_bf16, scaled,
                         to_bf16_bits, zipf_ranks)


def test_bf16_round_is_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1e-40]])
    y = round_to_bf16(x)
    bits = to_bf16_bits(y)
    assert np.array_equal(from_bf16_bits(bits).astype(np.float64), y)   # representable
    up = from_bf16_bits((bits.astype(np.int64) + 1).astype(np.uint16)).astype(np.float64)
    dn = from_bf16_bits((bits.astype(np.int64) - 1).astype(np.uint16)).astype(np.float64)
    err = np.abs(x - y)
    nz = y != 0
    assert np.all(err[nz] <= np.abs(x - up)[nz]) and np.all(err[nz] <= np.abs(x - dn)[nz])
    # halfway cases go to the even significand
    assert round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32)
    ours = round_to_bf16(x.astype(np.float64)).astype(np.float32)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, theirs)


def test_zipf_rank_frequencies():
    rng = np.random.default_rng(2)
    C, a = 1000, 1.1
    r = zipf_ranks(rng, 200000, C, a)
    assert r.min() >= 1 and r.max() <= C
    p1 = 1.0 / np.sum(np.arange(1, C + 1) ** -a)
    assert abs(np.mean(r == 1) - p1) < 5 * np.sqrt(p1 / 200000)
    assert abs(np.mean(r == 2) - p1 * 2 ** -a) < 5 * np.sqrt(p1 / 200000)


def test_workloads_deterministic_and_shaped():
    w = scaled("sasrec", seqs=4, seqlen=50, C=3000)
    a, b = make_inputs(w), make_inputs(w)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.Y, b.Y) and np.array_equal(a.pos, b.pos)
    assert a.X.shape == (200, 64) and a.Y.shape == (3000, 64) and a.B.shape == (2, 64, 64)
    assert np.array_equal(round_to_bf16(a.X.astype(np.float64)), a.X.astype(np.float64))
    assert a.pos.min() >= 0 and a.pos.max() < 3000
    # variance 1/sqrt(d): logits x.y have unit variance
    assert abs(np.var(a.X) - 64 ** -0.5) < 0.01
    t = make_inputs(WORKLOADS["tiny"])
    f = make_inputs(WORKLOADS["tiny_fullce"])
    assert np.array_equal(t.X, f.X) and np.array_equal(t.Y, f.Y) and np.array_equal(t.pos, f.pos)
    assert f.B.shape == (1, 64, 1)


def test_popular_rows_scaled():
    w = scaled("million", seqs=2, seqlen=10, C=5000)
    inp = make_inputs(w)
    pop = inp.perm[: 50]
    rest = inp.perm[50:]
    ratio = np.sqrt(np.mean(inp.Y[pop] ** 2) / np.mean(inp.Y[rest] ** 2))
    assert 2.7 < ratio < 3.3
