"""Benchmark: RECE forward + backward throughput on one MI355X.

One step = rece_forward + rece_backward over one batch of the workload (all
rounds: bucketing, sorting, chunk logits + top-k, loss, dX, dY).  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sasrec]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 matrix cores
PEAK_FP32_TFLOPS = 157.3       # fp32 matrix cores
RIDGE_BF16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
# vector ALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-operations per second
# (the fp32 vector peak of 157.3 TFLOP/s counts an FMA as 2 flops on 2 packed lanes)
PEAK_ALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
ALU_OPS_PER_LOGIT = 4          # mask the positive, bin + count (histogram pass), compare (filter pass)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "select_sasrec_hbm_traffic.md")
SELECT_SOURCES = ["k_select.hip", "rece_stream.h", "rece_device.h", "rece_internal.h"]


def chunk_starts(N, n_c):
    return [(c * N + n_c - 1) // n_c for c in range(n_c + 1)]


def window_logits(w):
    """sum over positions of the window size of the position's chunk (logits per round)."""
    xs, ys = chunk_starts(w.s, w.n_c), chunk_starts(w.C, w.n_c)
    tot = 0
    for c in range(w.n_c):
        wins = {c, (c - 1) % w.n_c, (c + 1) % w.n_c}
        W = sum(ys[q + 1] - ys[q] for q in wins)
        tot += (xs[c + 1] - xs[c]) * W
    return tot


def algorithmic_work_sce(w):
    """Per-step algorithmic (flops, bytes) of the bucket variant's phases."""
    es = 2 if w.dtype == "bf16" else 4
    s, C, d, nb = w.s, w.C, w.d, w.n_b
    sx, sy = nb * w.b_x, nb * w.b_y
    logits = sx * w.b_y
    return {
        "project": (2.0 * d * nb * (s + C), (s + C) * d * es),
        "sort": (0.0, nb * (s + C) * 4 + (sx + sy) * (d * es + 8)),      # score columns, bucket rows
        "select": (float(ALU_OPS_PER_LOGIT * logits), (sx + sy) * d * es + sx * w.k * 8),
        "loss": (2.0 * d * s, s * (2 * d * es + 24)),
        **backward_work(w, 1),
    }


def algorithmic_work(w):
    """Per-step algorithmic (flops, bytes) of each phase: what the method must compute and
    move; logits never go to HBM, every vector is read once per pass.  The chunk kernel's
    flops entry is its vector-ALU work (ALU_OPS_PER_LOGIT per window logit), which bounds it
    before the matrix cores do."""
    es = 2 if w.dtype == "bf16" else 4
    s, C, d, r, nb = w.s, w.C, w.d, w.rounds, w.n_b
    wl = window_logits(w)
    state = 32            # per position and round: threshold (12 B), bounds, shift, sum, count
    return {
        "project": (2.0 * d * nb * (s + C) * r, r * ((s + C) * (d * es + 4) + nb * d * es)),
        "sort": (0.0, r * (s + C) * 12 + s * 12),
        "select": (float(ALU_OPS_PER_LOGIT * wl * r),
                   r * ((s + C) * d * es + 8 * (s + C) + state * s + s * w.k * 4)),   # + kept lists
        "loss": (2.0 * d * s, s * (2 * d * es + 12 + 12 * r)),
        **backward_work(w, r),
    }


def backward_work(w, r):
    """Backward phases (both variants): dX from the kept lists; the (item, position)
    records of the lists and positives sorted by item; dY from the sorted records."""
    es = 2 if w.dtype == "bf16" else 4
    s, C, d = w.s, w.C, w.d
    pairs = r * s * w.k + s
    kb = max(1, (C - 1).bit_length())
    npass = (kb + 11) // 12
    return {
        # kept lists, every vector once, per-position state, dX
        "bwd_dx": (2.0 * 2 * d * (w.k * r + 1) * s, r * s * w.k * 4 + (s + C) * d * es + 12 * s + s * d * 4),
        # read the lists once, then each pass reads and writes 8-byte records
        "bwd_sort": (0.0, r * s * w.k * 4 + s * 4 + npass * 16 * pairs),
        # sorted records, every vector once, per-position state, dY written once
        "bwd_dy": (2.0 * 2 * d * pairs, 8 * pairs + (s + C) * d * es + 12 * s + C * d * 4),
    }


def roofline(name, ms_per_launch, flops, nbytes, dtype):
    ai = flops / max(nbytes, 1)
    t = ms_per_launch * 1e-3
    if name == "select":
        ach = flops / t / 1e12
        return {"bound": "alu", "achieved": ach, "peak": PEAK_ALU_TOPS, "unit": "Tops/s",
                "frac": ach / PEAK_ALU_TOPS}
    if name == "project" and ai > RIDGE_BF16:
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
        ach = flops / t / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak}
    ach = nbytes / t / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}


def source_digest(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "catalogue_cross_entropy_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of the chunk kernel from the committed counter summary, or None
    when that summary is missing or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("TRAFFIC "):
            rec = json.loads(line[len("TRAFFIC "):])
            if rec.get("kernel") == kernel and rec.get("sources") == source_digest(SELECT_SOURCES):
                return rec["bytes_per_launch"]
    return None


def copy_probe(mb):
    """One plain device copy of known size: the calibration dispatch for HBM byte counters."""
    import torch
    n = mb * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy probe: {n} bytes read, {n} bytes written", file=sys.stderr)


def cpu_baseline(inp, n_rows, seed=0):
    """The float64 oracle, as it is, on a seeded sample of positions (all rounds, fwd + bwd)."""
    import numpy as np
    import oracle
    w = inp.w
    rows = np.sort(np.random.default_rng(seed).choice(w.s, size=n_rows, replace=False))
    t0 = time.perf_counter()
    fwd = oracle.rece_forward(inp.X, inp.Y, inp.pos, inp.B, w.n_c, w.k, rows=rows)
    oracle.rece_backward(inp.X, inp.Y, inp.pos, fwd)
    dt = time.perf_counter() - t0
    return {"value": n_rows / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_rows} of {w.s} positions (seeded), all {w.rounds} rounds, forward + backward; "
                      f"bucketing and sorting of all {w.s}+{w.C} vectors included; {dt:.1f} s; "
                      f"NumPy elementwise float64 (one thread)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sasrec")
    ap.add_argument("--cpu-rows", type=int, default=12800,
                    help="positions the oracle baseline computes (about 10-30 s of host work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after the run, one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the loss runs on a single MI355X, see the sharding notes in the design document)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import catalogue_cross_entropy_amd as rece
    from rece_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    X = torch.from_numpy(inp.X).to(dev).to(dt)
    Y = torch.from_numpy(inp.Y).to(dev).to(dt)
    B = torch.from_numpy(inp.B).to(dev).to(dt)
    if w.variant == "sce":
        B = B[0].contiguous()
    pos = torch.from_numpy(inp.pos).to(dev)
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, variant=w.variant,
                     b_x=w.b_x, b_y=w.b_y)
    scratch, saved = plan.workspace(dev)
    dX = torch.empty((w.s, w.d), dtype=torch.float32, device=dev)
    dY = torch.empty((w.C, w.d), dtype=torch.float32, device=dev)
    dloss = torch.ones(1, dtype=torch.float32, device=dev)

    def step():
        plan.forward(X, Y, pos, B, scratch, saved, loss_pp=False)
        plan.backward(X, Y, pos, scratch, saved, dloss=dloss, dX=dX, dY=dY)

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan.check(saved)
    # device memory of a whole step: the library allocates nothing itself, so torch's peak
    # covers inputs, outputs and the two workspaces; a dense bf16 [s, C] logit tensor must
    # be larger than every buffer the step holds
    logit_bytes = 2 * w.s * w.C
    largest = max(scratch.numel(), saved.numel(), dX.numel() * 4, dY.numel() * 4,
                  X.numel() * X.element_size(), Y.numel() * Y.element_size())
    memory = {"scratch_bytes": plan.scratch_bytes, "saved_bytes": plan.saved_bytes,
              "peak_allocated_bytes": torch.cuda.max_memory_allocated(dev),
              "largest_buffer_bytes": largest, "dense_logits_bf16_bytes": logit_bytes,
              "no_dense_logits": largest < logit_bytes}
    if not memory["no_dense_logits"]:
        sys.exit(f"a buffer of {largest} bytes is at least the size of a dense [s, C] logit tensor")

    # phase breakdown on a few untimed steps (events around every launch)
    plan.profile()
    nprof = 3
    for _ in range(nprof):
        step()
    torch.cuda.synchronize()
    phases = plan.profile_read()
    plan.profile(enable=False)
    work = algorithmic_work_sce(w) if w.variant == "sce" else algorithmic_work(w)
    dom = max((k for k in work), key=lambda k: phases[k][0])

    # timed region: events only around the dominant kernel's launches
    plan.profile([dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms, dom_launches = plan.profile_read()[dom]
    plan.profile(enable=False)
    plan.check(saved)
    counters = plan.export(saved, "counters").cpu().tolist()

    ms_step = elapsed * 1e3 / args.steps
    flops, nbytes = work[dom]
    per_launch = dom_launches / args.steps
    rl = roofline(dom, dom_ms / dom_launches, flops / per_launch, nbytes / per_launch, w.dtype)
    rl["kernel"] = dom
    rl["traffic"] = measured_traffic(f"select:{w.name}") if dom == "select" else None

    breakdown = {}
    for name, (f, b) in work.items():
        ms, n = phases[name]
        if n == 0:
            continue
        r = roofline(name, ms / n, f * nprof / n, b * nprof / n, w.dtype)
        breakdown[name] = {"ms_per_step": ms / nprof, "launches_per_step": n / nprof,
                           "bound": r["bound"], "frac": round(r["frac"], 4)}

    out = {
        "metric": "RECE fwd+bwd positions/sec at C items, d; % MFMA and % HBM peak",
        "value": w.s / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": (f"{w.name}: s={w.s} ({w.seqs}x{w.seqlen}), C={w.C}, d={w.d}, "
                                + (f"n_b={w.n_b}, n_c={w.n_c}, k={w.k}, rounds={w.rounds}, " if w.variant == "rece"
                                   else f"n_b={w.n_b}, b_x={w.b_x}, b_y={w.b_y}, k={w.k}, ")
                                + f"{w.dtype}, positives {w.positives}"), "parallelism": "single GPU"},
        "roofline": rl,
        "phases": breakdown,
        "memory": memory,
        "counters": {"argmax_rows_float64": counters[1], "topk_rows_near_tie": counters[2],
                     "logits_float64": counters[3], "overflows": counters[4]},
    }
    if not args.no_cpu_baseline and w.variant == "rece":
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows)
    print(json.dumps(out), flush=True)
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb)


if __name__ == "__main__":
    main()
