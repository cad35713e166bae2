"""Benchmark: RECE forward + backward throughput on one MI355X.

One step = rece_forward + rece_backward over one batch of the workload (all
rounds: bucketing, sorting, chunk logits + top-k, loss, dX, dY).  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload tenmillion]

Default workload: ten million items (s = 32768 positions of 128 sequences x 256,
d = 128, bf16, n_b = n_c = 1024, k = 256, 3 rounds), the largest that the loss
is specified on; the other workloads are selected with --workload.

Per phase the line reports both roofline fractions (matrix cores and HBM) of the
phase's algorithmic work, against the datasheet peaks and against the peaks that
a matrix-core loop and a plain copy reach on the device in the same run.
"""
import argparse
import glob
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X datasheet peaks (dense; no sparsity)
SPEC_HBM_GBS = 8000.0
SPEC_BF16_TFLOPS = 2500.0
SPEC_FP32_TFLOPS = 157.3

# phases the library times, and the kernels each one launches
PHASE_KERNELS = {
    "project": "k_project_argmax, k_argmax_near",
    "sort": "k_seg_hist, k_scan_*, k_seg_scatter*",
    "select": "k_sel_stream (histogram pass, exact pass), k_sel_finish",
    "loss": "k_round_dedup, k_ce, k_mean",
    "bwd_dx": "k_dx_lists",
    "bwd_sort": "k_pair_hist, k_pair_scatter",
    "bwd_dy": "k_dy_pieces, k_dy_combine",
}
# sources of each phase's kernels: a counter summary is used only while their digest matches
PHASE_SOURCES = {
    "project": ["k_bucket.hip", "rece_stream.h", "rece_device.h", "rece_internal.h"],
    "select": ["k_select.hip", "rece_stream.h", "rece_device.h", "rece_internal.h", "rece_kth.h"],
}


def chunk_starts(N, n_c):
    return [(c * N + n_c - 1) // n_c for c in range(n_c + 1)]


def window_logits(w):
    """Sum over positions of the size of the position's window (logits per round)."""
    xs, ys = chunk_starts(w.s, w.n_c), chunk_starts(w.C, w.n_c)
    tot = 0
    for c in range(w.n_c):
        if w.window_wrap:
            wins = {(c + t) % w.n_c for t in range(-w.n_ec, w.n_ec + 1)}
        else:
            wins = {q for q in range(c - w.n_ec, c + w.n_ec + 1) if 0 <= q < w.n_c}
        W = sum(ys[q + 1] - ys[q] for q in wins)
        tot += (xs[c + 1] - xs[c]) * W
    return tot


def backward_work(w, r):
    """Backward phases (both variants): dX from the kept lists; the (item, position)
    records of the lists and positives sorted by item; dY from the sorted records."""
    es = 2 if w.dtype == "bf16" else 4
    s, C, d = w.s, w.C, w.d
    pairs = r * s * w.k + s
    kb = max(1, (C - 1).bit_length())
    npass = (kb + 7) // 8
    return {
        # kept lists, every vector once, per-position state; 2 flops per coordinate for
        # the logit and 2 for the accumulation, per kept pair and the positive
        "bwd_dx": (4.0 * d * (w.k * r + 1) * s, r * s * w.k * 4 + (s + C) * d * es + 16 * s + s * d * 4),
        # read the lists once, then each digit pass reads and writes 8-byte records
        "bwd_sort": (0.0, r * s * w.k * 4 + s * 4 + npass * 16 * pairs),
        # sorted records, every vector once, per-position state, dY written once
        "bwd_dy": (4.0 * d * pairs, 8 * pairs + (s + C) * d * es + 16 * s + C * d * 4),
    }


def algorithmic_work(w):
    """Per-step algorithmic (flops, bytes) of each phase: what the method must compute
    and move.  Logits never go to HBM; every vector is read once per pass (window
    overlap through the caches); selections are 4-byte ids; dX, dY are written once
    in float32.  It does not count the dense s x C work the method avoids."""
    es = 2 if w.dtype == "bf16" else 4
    s, C, d, r, nb = w.s, w.C, w.d, w.rounds, w.n_b
    wl = window_logits(w)
    return {
        # X.B and Y.B per round, argmax written as a 4-byte id
        "project": (2.0 * d * nb * (s + C) * r, r * ((s + C) * (d * es + 4) + nb * d * es)),
        # per round: the keys read, the order written (4 + 4 bytes per element)
        "sort": (0.0, r * (s + C) * 8),
        # every position and item vector once per round, the kept ids written
        "select": (2.0 * d * wl * r, r * ((s + C) * d * es + s * w.k * 4)),
        # kept ids of every round, the positive's two vectors, per-round sums, loss out
        "loss": (2.0 * d * s, r * s * w.k * 4 + s * (2 * d * es) + r * s * 12 + s * 8),
        **backward_work(w, r),
    }


def algorithmic_work_sce(w):
    """Per-step algorithmic (flops, bytes) of the bucket variant's phases."""
    es = 2 if w.dtype == "bf16" else 4
    s, C, d, nb = w.s, w.C, w.d, w.n_b
    sx, sy = nb * w.b_x, nb * w.b_y
    return {
        "project": (2.0 * d * nb * (s + C), (s + C) * d * es),
        "sort": (0.0, (sx + sy) * 4),      # the bucket lists (the scores need not be stored)
        "select": (2.0 * d * sx * w.b_y, (sx + sy) * d * es + sx * w.k * 8),
        "loss": (2.0 * d * s, s * (2 * d * es + 24)),
        **backward_work(w, 1),
    }


def fractions(ms, flops, nbytes, dtype, peaks):
    """Both roofline fractions of a phase: matrix cores and HBM, against the datasheet
    and the measured peaks; `bound` is the roof the arithmetic intensity sits under."""
    t = ms * 1e-3
    mf_spec = SPEC_BF16_TFLOPS if dtype == "bf16" else SPEC_FP32_TFLOPS
    tf = flops / t / 1e12 if t > 0 else 0.0
    gbs = nbytes / t / 1e9 if t > 0 else 0.0
    ridge = mf_spec * 1e12 / (SPEC_HBM_GBS * 1e9)
    out = {"bound": "mfma" if flops > ridge * nbytes else "hbm",
           "tflops": round(tf, 3), "gbs": round(gbs, 1),
           "mfma_frac": round(tf / mf_spec, 5), "hbm_frac": round(gbs / SPEC_HBM_GBS, 5)}
    if peaks:
        mf_meas = peaks["bf16_tflops"] if dtype == "bf16" else None
        if mf_meas:
            out["mfma_frac_measured_peak"] = round(tf / mf_meas, 5)
        out["hbm_frac_measured_peak"] = round(gbs / peaks["copy_gbs"], 5)
    return out


def source_digest(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "catalogue_cross_entropy_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(phase, workload):
    """HBM bytes per launch of a phase from the committed counter summaries
    (profiles/*_hbm_traffic.md), or None when none covers it or the one that does
    was taken on other kernel sources."""
    if phase not in PHASE_SOURCES:
        return None
    digest = source_digest(PHASE_SOURCES[phase])
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.md"))):
        for line in open(path).read().splitlines():
            if line.startswith("TRAFFIC "):
                rec = json.loads(line[len("TRAFFIC "):])
                if rec.get("kernel") == f"{phase}:{workload}" and rec.get("sources") == digest:
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


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

_G = {}   # arrays the forked workers share (read-only)


def _w_bucket(idx):
    import oracle
    t0 = time.perf_counter()
    oracle.bucket_ids(_G["Y"][idx], _G["B0"])
    return time.perf_counter() - t0


def _w_window(rows):
    import oracle
    g = _G
    t0 = time.perf_counter()
    negs = oracle.round_negatives(g["X"], g["Y"], g["pos"], g["px"], g["py"], g["n_c"], g["k"], rows=rows,
                                  n_ec=g["n_ec"], wrap=g["wrap"])
    return time.perf_counter() - t0, {i: v[0] for i, v in negs.items()}


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, os.cpu_count() or 1, avail


def cpu_baseline(inp, per_worker_items=8192, chunks_per_worker=2, seed=0):
    """The oracle as it stands (float64 NumPy, elementwise), timed on samples of each
    stage of one step and extrapolated to the whole step.  P forked worker processes
    run the two dominant stages side by side:
      bucketing: oracle.bucket_ids on P * per_worker_items sampled item rows;
      windows:   oracle.round_negatives on the positions of P * chunks_per_worker
                 whole position chunks (seeded labels: equal-size chunks make every
                 chunk's window the same size whatever the labels are);
    then the parent times, on one core, the stable sorts of full-size label arrays and
    the loss and backward (oracle.loss_from_negatives, oracle.rece_backward) of the
    sampled positions, less the one-off zeroing of the dense dY they allocate.
    Step time with P workers:
      T = r (s + C) t_bucket + r n_c t_chunk + r t_sort + s t_lossbwd / P + t_zero
    with t_bucket, t_chunk the wall time per sampled row / chunk of the parallel stages,
    t_sort, t_lossbwd the serial per-sort / per-position times and t_zero the dY zeroing."""
    import multiprocessing as mp

    import numpy as np
    import oracle

    w = inp.w
    model, ncpu, avail = cpu_info()
    P = max(1, min(16, avail))
    rng = np.random.default_rng(seed)
    s, C, r = w.s, w.C, w.rounds
    X64 = inp.X.astype(np.float64)
    Y64 = inp.Y.astype(np.float64)
    # seeded labels for the window stage (not the method's: its cost does not depend on them)
    bx = rng.integers(0, w.n_b, size=s)
    by = rng.integers(0, w.n_b, size=C)
    t0 = time.perf_counter()
    px = oracle.stable_argsort(bx)
    py = oracle.stable_argsort(by)
    t_sorts = time.perf_counter() - t0          # one position sort and one item sort
    n_items = P * per_worker_items
    item_idx = np.sort(rng.choice(C, size=min(n_items, C), replace=False))
    n_chunks = min(w.n_c, P * chunks_per_worker)
    chunks = np.sort(rng.choice(w.n_c, size=n_chunks, replace=False))
    xb = oracle.chunk_bounds(s, w.n_c)
    chunk_rows = [px[xb[c]:xb[c + 1]] for c in chunks]
    _G.update(X=X64, Y=Y64, pos=inp.pos, px=px, py=py, n_c=w.n_c, k=w.k, n_ec=w.n_ec, wrap=w.window_wrap,
              B0=np.asarray(inp.B[0], dtype=np.float64))
    ctx = mp.get_context("fork")
    with ctx.Pool(P) as pool:
        t0 = time.perf_counter()
        pool.map(_w_bucket, np.array_split(item_idx, P))
        t_bucket_wall = time.perf_counter() - t0
        groups = [np.concatenate(g) if len(g) else np.zeros(0, np.int64)
                  for g in (chunk_rows[i::P] for i in range(P))]
        t0 = time.perf_counter()
        res = pool.map(_w_window, groups)
        t_window_wall = time.perf_counter() - t0
    negs = {}
    for _, d in res:
        negs.update(d)
    rows = np.sort(np.fromiter(negs.keys(), dtype=np.int64))
    t0 = time.perf_counter()
    fwd = oracle.loss_from_negatives(X64, Y64, inp.pos, [negs] * r, rows=rows)
    oracle.rece_backward(X64, Y64, inp.pos, fwd)
    t_lossbwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    np.zeros_like(Y64)
    t_zero = time.perf_counter() - t0
    _G.clear()
    per_row = max(t_lossbwd - t_zero, 0.0) / len(rows)
    T = (r * (s + C) * t_bucket_wall / len(item_idx) + r * w.n_c * t_window_wall / n_chunks
         + r * t_sorts + s * per_row / P + t_zero)
    measured = t_bucket_wall + t_window_wall + t_sorts + t_lossbwd + t_zero
    return {"value": s / T, "unit": "positions/s", "cores": P, "kind": "oracle",
            "sample": (f"{len(item_idx)} of {C} item rows bucketed and {n_chunks} of {w.n_c} position chunks "
                       f"({len(rows)} positions) through the window top-k, in {P} worker processes; one position "
                       f"and one item sort of full-size seeded labels; loss and backward of the sampled positions "
                       f"on one core; {measured:.1f} s measured, extrapolated to the whole step "
                       f"({T:.0f} s at {P} cores)"),
           "extrapolation": "T = r(s+C) t_bucket + r n_c t_chunk + r t_sort + s t_lossbwd / P + t_zero",
           "terms_s": {"t_bucket": t_bucket_wall / len(item_idx), "t_chunk": t_window_wall / n_chunks,
                       "t_sort": t_sorts, "t_lossbwd_per_position": per_row, "t_zero": t_zero},
           "cpu_model": model, "nproc": ncpu, "cpus_available": avail, "threads": P,
           "math": "NumPy float64 elementwise (no BLAS call on the timed path)"}


def time_full_ce(w, X, Y, pos, steps):
    """The exact full cross-entropy (every item scored, no [s, C] tensor) on the same
    inputs: one untimed step, then `steps` timed fwd+bwd steps."""
    import torch
    import catalogue_cross_entropy_amd as rece
    f = rece.FullCE(w.s, w.C, w.d, dtype=w.dtype)
    ws = torch.empty(f.workspace_bytes, dtype=torch.uint8, device=X.device)
    dX = torch.empty((w.s, w.d), dtype=torch.float32, device=X.device)
    dY = torch.empty((w.C, w.d), dtype=torch.float32, device=X.device)

    def step():
        f.forward(X, Y, pos, ws, loss_pp=False)
        f.backward(X, Y, pos, ws, dX=dX, dY=dY)

    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flops = 2.0 * w.s * w.C * w.d * 5     # logits (3 sweeps) and the two gradient products
    return {"ms_per_step": round(ms, 3), "value": w.s / (ms * 1e-3), "unit": "positions/s", "steps": steps,
            "workspace_bytes": f.workspace_bytes, "mfma_frac": round(flops / (ms * 1e-3) / 1e12 /
                                                                     (SPEC_BF16_TFLOPS if w.dtype == "bf16"
                                                                      else SPEC_FP32_TFLOPS), 4)}


def measure_peaks(dev):
    from catalogue_cross_entropy_amd import peaks
    return {"bf16_tflops": round(peaks.mfma_bf16_tflops(dev), 1), "copy_gbs": round(peaks.copy_gbs(dev), 1),
            "note": "bf16 matrix-core loop with no memory traffic; 1 GiB device copy, read + write bytes"}


def note(msg):
    """Progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="tenmillion")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the device peak probes")
    ap.add_argument("--full-ce-steps", type=int, default=1,
                    help="exact full cross-entropy fwd+bwd steps timed next to the reduced loss (0: skip)")
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
    note(f"inputs of {w.name} generated")
    # the CPU baseline forks worker processes: it runs before anything touches the GPU
    cpu = None
    if not args.no_cpu_baseline and w.variant == "rece":
        cpu = cpu_baseline(inp)
        print(f"cpu baseline: {cpu['value']:.1f} positions/s ({cpu['sample']})", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    X = torch.from_numpy(inp.X).to(dev).to(dt)
    Y = torch.from_numpy(inp.Y).to(dev).to(dt)
    B = torch.from_numpy(inp.B).to(dev).to(dt)
    if w.variant == "sce":
        B = B[0].contiguous()
    pos = torch.from_numpy(inp.pos).to(dev)
    plan = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, variant=w.variant,
                     b_x=w.b_x, b_y=w.b_y, n_ec=w.n_ec, window_wrap=w.window_wrap)
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
    note(f"{args.warmup} warm-up steps done")
    # device memory of a whole step: the library allocates nothing itself, so torch's peak
    # covers inputs, outputs and the two workspaces; a dense bf16 [s, C] logit tensor must
    # be larger than every buffer the step holds
    logit_bytes = 2 * w.s * w.C
    largest = max(scratch.numel(), saved.numel(), dX.numel() * 4, dY.numel() * 4,
                  X.numel() * X.element_size(), Y.numel() * Y.element_size())
    model = rece.auto_size(w.s, w.C, w.n_ec, w.n_b / max(w.n_c, 1), w.rounds) if w.variant == "rece" else None
    memory = {"scratch_bytes": plan.scratch_bytes, "saved_bytes": plan.saved_bytes,
              "pages_memory_model_bytes_4B": None if model is None else 4 * model["model_elems"],
              "pages_optimal_n_b": None if model is None else model["n_b"],
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

    # timed region: events only around the dominant phase's launches
    plan.profile([dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms, dom_launches = plan.profile_read()[dom]
    note(f"{args.steps} timed steps: {elapsed * 1e3 / args.steps:.3f} ms per step")
    plan.profile(enable=False)
    plan.check(saved)
    counters = plan.export(saved, "counters").cpu().tolist()

    full = time_full_ce(w, X, Y, pos, args.full_ce_steps) if args.full_ce_steps > 0 else None
    peaks = None if args.no_peaks else measure_peaks(dev)

    ms_step = elapsed * 1e3 / args.steps
    flops, nbytes = work[dom]
    per_launch = dom_launches / args.steps
    ms_launch = dom_ms / dom_launches
    fr = fractions(ms_launch, flops / per_launch, nbytes / per_launch, w.dtype, peaks)
    if fr["bound"] == "mfma":
        peak = SPEC_BF16_TFLOPS if w.dtype == "bf16" else SPEC_FP32_TFLOPS
        rl = {"bound": "mfma", "achieved": fr["tflops"], "peak": peak, "unit": "TFLOP/s",
              "frac": fr["mfma_frac"]}
    else:
        rl = {"bound": "hbm", "achieved": fr["gbs"], "peak": SPEC_HBM_GBS, "unit": "GB/s",
              "frac": fr["hbm_frac"]}
    rl.update(kernel=f"{dom} ({PHASE_KERNELS.get(dom, dom)})", ms_per_launch=round(ms_launch, 4),
              launches_per_step=per_launch, other_roof=fr,
              traffic=measured_traffic(dom, w.name))

    breakdown = {}
    for name, (f, b) in work.items():
        ms, n = phases[name]
        if n == 0:
            continue
        breakdown[name] = {"ms_per_step": round(ms / nprof, 4), "launches_per_step": n / nprof,
                           "kernels": PHASE_KERNELS.get(name, name),
                           "gflop": round(f / 1e9, 3), "mbytes": round(b / 1e6, 2),
                           **fractions(ms / nprof, f, b, w.dtype, peaks)}

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
                                + (f"n_b={w.n_b}, n_c={w.n_c}, n_ec={w.n_ec}, k={w.k}, rounds={w.rounds}, "
                                   if w.variant == "rece"
                                   else f"n_b={w.n_b}, b_x={w.b_x}, b_y={w.b_y}, k={w.k}, ")
                                + f"{w.dtype}, positives {w.positives}"), "parallelism": "single GPU"},
        "roofline": rl,
        "peaks": {"datasheet": {"bf16_tflops": SPEC_BF16_TFLOPS, "fp32_tflops": SPEC_FP32_TFLOPS,
                                "hbm_gbs": SPEC_HBM_GBS},
                  "measured": peaks},
        "phases": breakdown,
        "memory": memory,
        "counters": {"argmax_rows_float64": counters[1], "topk_rows_near_tie": counters[2],
                     "logits_float64": counters[3], "overflows": counters[4],
                     "select_rows_exact_pass": counters[5], "select_list_entries": counters[6]},
    }
    if full is not None:
        full["rece_speedup"] = round(full["ms_per_step"] / ms_step, 2)
        out["full_ce"] = full
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb)


if __name__ == "__main__":
    main()
