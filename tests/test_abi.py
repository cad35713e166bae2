"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, validates configurations and sizes its workspaces (host-only calls)."""
import ctypes
import os
import re

import pytest

import catalogue_cross_entropy_amd as rece

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "rece.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:rece_status|const char\*)\s+(rece_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = rece.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(rece.EXPORTED)


def test_peaks_library_exports_every_declared_symbol():
    from catalogue_cross_entropy_amd import peaks
    with open(os.path.join(ROOT, "include", "peaks.h")) as f:
        text = f.read()
    names = set(re.findall(r"^\s*(?:int|double)\s+(rece_\w+)\s*\(", text, re.M))
    assert names == set(peaks.EXPORTED)
    L = peaks.lib()
    for n in names:
        assert hasattr(L, n), n
    # host-side arithmetic only: 8 chains x 4 waves of 16x16x32 multiply-adds per iteration
    assert L.rece_peak_mfma_flops(3, 5) == 2.0 * 16 * 16 * 32 * 8 * 4 * 5 * 3
    # argument checks return before anything is enqueued
    assert L.rece_peak_copy(None, None, None, 16) != 0
    assert L.rece_peak_mfma_bf16(None, 0, 1, None) != 0


def test_version_and_status_strings():
    assert "gfx950" in rece.version()
    L = rece.lib()
    for code in range(7):
        assert L.rece_status_string(code).decode()


def _plan(**kw):
    base = dict(s=256, C=2000, d=64, n_b=16, n_c=16, k=32, rounds=1, dtype="f32")
    base.update(kw)
    return rece.Plan(**base)


@pytest.mark.parametrize("bad,status", [
    (dict(k=2000), 1),          # k > C - 1
    (dict(k=-1), 1),
    (dict(n_c=0), 1),
    (dict(n_c=257), 1),         # n_c > s
    (dict(n_b=0), 1),
    (dict(n_b=5000), 1),
    (dict(rounds=0), 1),
    (dict(rounds=9), 1),
    (dict(d=48), 2),            # unsupported width
    (dict(s=0), 1),
    (dict(C=1, k=0, n_c=1), 1),
    (dict(variant="sce", b_x=0, b_y=8), 1),          # bucket variant: b_x in 1..s
    (dict(variant="sce", b_x=4, b_y=2001), 1),       # b_y in 1..C
    (dict(variant="sce", b_x=4, b_y=8, rounds=2), 1),
    (dict(variant="sce", b_x=4, b_y=1500, k=1025), 2),   # k above the merge capacity
    (dict(n_ec=-1), 1),                                  # neighbouring chunks >= 0
    (dict(n_ec=(1 << 20) + 1), 1),
    (dict(window_wrap=2), 1),                            # 0 (clipped) or 1 (cyclic)
    (dict(s=1 << 20, C=1 << 20, n_c=16, k=2047, rounds=1), 2),   # s * k + s beyond int32 pair records
])
def test_plan_rejects_invalid(bad, status):
    with pytest.raises(rece.ReceError) as ei:
        _plan(**bad)
    assert ei.value.status == status
    assert rece.lib().rece_last_error().decode()


def test_plan_null_arguments():
    L = rece.lib()
    h = ctypes.c_void_p()
    assert L.rece_plan(None, ctypes.byref(h)) == 1
    # s, C, d, n_b, n_c, n_ec, k, rounds, b_x, b_y, dtype, variant, window_wrap, flags
    cfg = rece.ReceConfig(256, 2000, 64, 16, 16, 1, 32, 1, 0, 0, 0, 0, 1, 0)
    assert L.rece_plan(ctypes.byref(cfg), None) == 1
    assert L.rece_plan(ctypes.byref(cfg), ctypes.byref(h)) == 0
    # forward with NULL pointers fails before touching the GPU
    assert L.rece_forward(h, None, None, None, None, None, None, None, None, None) == 1
    assert L.rece_backward(h, None, None, None, None, None, None, None, None, None, None) == 1
    # misaligned pointers are rejected
    assert L.rece_forward(h, None, 8, 16, 16, 16, 16, 16, 16, None) == 1
    L.rece_plan_destroy(h)


@pytest.mark.parametrize("name", ["tiny", "tiny_fullce", "sasrec", "million", "tenmillion", "sce"])
def test_workspace_never_holds_a_logit_tensor(name):
    from rece_inputs import WORKLOADS
    w = WORKLOADS[name]
    p = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype, variant=w.variant,
                  b_x=w.b_x, b_y=w.b_y)
    # no buffer of s*C*2 bytes (a bf16 [s, C] logit tensor) is ever needed; what the
    # forward pass keeps grows with the kept negatives (one int32 id per position,
    # round and kept pair), not with the catalogue
    rounds = w.rounds if w.variant == "rece" else 1
    lists = rounds * w.s * w.k * 4
    es = 2 if w.dtype == "bf16" else 4
    # scratch: the sorted copies of every round (rows), the backward's pair records
    # (four int32 arrays over the kept pairs and positives, plus the dY work area of two
    # float32 rows per 256 pairs) and small per-element arrays
    pairs = rounds * w.s * w.k + w.s
    rows = rounds * (w.s + w.C) * w.d * es
    slots = w.n_b * (w.b_x + w.b_y) * (w.d * es + 64) + w.n_b * (w.s + w.C) * 4
    # the chunk kernels' candidate lists: per row (position, or bucket slot) 3k + 2 tiles of
    # (id, logit) entries, its length and threshold, and per wave of 16 rows as many
    # float64 values for the exact pass; two sets for RECE (its rounds run on two streams)
    list_rows = 2 * w.s if w.variant == "rece" else w.n_b * w.b_x
    cand = list_rows * ((3 * w.k + 128) * 8 * 9 // 8 + 8)
    assert p.scratch_bytes <= rows + slots + cand + pairs * (16 + 2 * w.d * 4 // 256 + 1) \
        + 16 * (w.s + w.C) * rounds + (32 << 20)
    if w.k * 8 < w.C:   # a reduced set (not the full-CE twin): far below a dense logit tensor
        assert p.scratch_bytes < w.s * w.C * 2
    assert p.saved_bytes - lists < w.s * w.C * 2
    assert p.scratch_bytes > 0 and p.saved_bytes > 0
    # saved holds no row of X or Y: the per-round labels, orders and thresholds, the
    # kept lists and per-position values (int32 / float32 / float64 scalars)
    # (per position and round: bucket, order slot, threshold and sums, 40 bytes; per item and
    # round: bucket and order slot, 8 bytes)
    assert p.saved_bytes < lists + rounds * (40 * w.s + 8 * w.C) + 16 * w.s + (1 << 16) \
        + w.n_b * (w.b_x + w.b_y) * 4
    assert p.saved_bytes < (w.s + w.C) * w.d * es + lists


def test_export_sizes():
    p = _plan(keep_stages=True, rounds=2)
    L = rece.lib()
    nb = ctypes.c_size_t()
    for stage, want in (("bucket_x", 256 * 4), ("bucket_y", 2000 * 4), ("perm_y", 2000 * 4),
                        ("thresh_logit", 256 * 8), ("neg_ids", 256 * 32 * 4), ("counters", 32),
                        ("union_ids", 256 * 2 * 32 * 4)):
        assert L.rece_export_bytes(p._h, rece.STAGES[stage], ctypes.byref(nb)) == 0
        assert nb.value == want
    q = _plan()   # the kept lists are always kept: the backward pass reads them
    assert L.rece_export_bytes(q._h, rece.STAGES["neg_ids"], ctypes.byref(nb)) == 0 and nb.value == 256 * 32 * 4
    assert L.rece_export_bytes(q._h, rece.STAGES["union_ids"], ctypes.byref(nb)) == 0 and nb.value == 256 * 32 * 4
    assert L.rece_export_bytes(q._h, 99, ctypes.byref(nb)) == 1


@pytest.mark.parametrize("kw", [
    dict(n_ec=0), dict(n_ec=2), dict(n_ec=7), dict(n_ec=3, window_wrap=False), dict(n_c=1, n_ec=0),
    dict(n_ec=1 << 20),
])
def test_window_options_accepted(kw):
    p = _plan(**kw)
    assert p.cfg.n_ec == kw.get("n_ec", 1)
    assert p.cfg.window_wrap == (0 if kw.get("window_wrap") is False else 1)


def test_windows_beyond_16_bit_histogram_counts_are_planned():
    """A window of more than 65535 items (here the whole catalogue of 70000) would
    wrap a 16-bit histogram bin; the plan accepts it (the chunk kernel then counts
    in 32 bits), with and without a top-k that keeps every candidate."""
    for k in (16, 69999):
        p = rece.Plan(64, 70000, 32, 1, 1, k, 1, dtype="f32")
        assert p.scratch_bytes > 0
    rece.Plan(64, 200000, 32, 8, 2, 16, 1, dtype="bf16", n_ec=0)   # two chunks of 100000 items


def test_product_path_has_no_fallback():
    import catalogue_cross_entropy_amd as pkg
    src = open(pkg.__file__).read()
    assert "import oracle" not in src and "from oracle" not in src
    for f in os.listdir(os.path.join(ROOT, "catalogue_cross_entropy_amd")):
        if f.endswith(".py"):
            text = open(os.path.join(ROOT, "catalogue_cross_entropy_amd", f)).read()
            assert "oracle" not in text, f


def test_sce_plan_and_exports():
    p = _plan(variant="sce", n_c=0, b_x=40, b_y=300, k=16, keep_stages=True)
    L = rece.lib()
    nb = ctypes.c_size_t()
    sizes = {}
    for name, st in rece.STAGES.items():
        assert L.rece_export_bytes(p._h, st, ctypes.byref(nb)) == 0
        sizes[name] = nb.value
    assert sizes["sce_rows"] == 16 * 40 * 4 and sizes["sce_items"] == 16 * 300 * 4
    assert sizes["bucket_x"] == sizes["perm_y"] == 0       # not kept by the bucket variant
    assert sizes["neg_ids"] == 256 * 16 * 4 and sizes["lse"] == 256 * 4
    assert sizes["union_ids"] == 256 * 16 * 4
    r = _plan(keep_stages=True)
    assert L.rece_export_bytes(r._h, rece.STAGES["sce_rows"], ctypes.byref(nb)) == 0 and nb.value == 0


def test_static_forward_rejects_plans_beyond_its_array():
    """rece_forward_static checks the plan's forward scratch against the static
    array before any GPU call: the ten-million-item plan needs gigabytes."""
    from rece_inputs import WORKLOADS
    w = WORKLOADS["tenmillion"]
    p = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype)
    L = rece.lib()
    assert L.rece_forward_static(p._h, None, 16, 16, 16, 16, 16, 16, None) == 3
    assert "static scratch" in L.rece_last_error().decode()
    assert L.rece_forward_static(None, None, 16, 16, 16, 16, 16, 16, None) == 1


def test_full_ce_entry_points_reject_bad_arguments():
    import ctypes as C
    L = rece.lib()
    n = C.c_size_t()
    assert L.rece_full_ce_workspace_bytes(0, C.byref(n)) == 1
    assert L.rece_full_ce_workspace_bytes(1000, C.byref(n)) == 0
    # log-sum-exp and upstream gradient per position, plus the per-wave loss sums
    assert n.value >= 1000 * 8
    fake = C.c_void_p(1 << 20)   # never dereferenced: the checks come before any launch
    args = dict(s=1000, C=5000, d=64, dtype=rece.RECE_BF16)

    def fwd(**kw):
        a = dict(args, **kw)
        return L.rece_full_ce_forward(None, a["s"], a["C"], a["d"], a["dtype"], fake, fake, fake,
                                      kw.get("ws", fake), kw.get("wsb", n.value), kw.get("loss", fake), None)

    assert fwd(d=48) == 2                      # unsupported d
    assert fwd(dtype=7) == 2                   # unsupported dtype
    assert fwd(s=0) == 1 and fwd(C=0) == 1     # empty
    assert fwd(s=1 << 31) == 2                 # beyond int32 ids
    assert fwd(ws=None) == 1                   # NULL workspace
    assert fwd(wsb=n.value - 1) == 3           # workspace too small
    assert fwd(loss=None) == 1                 # NULL loss
    assert L.rece_full_ce_backward(None, 1000, 5000, 64, rece.RECE_BF16, fake, fake, fake, fake, n.value,
                                   None, None, fake, fake) == 1   # no upstream gradient
    assert L.rece_full_ce_backward(None, 1000, 5000, 64, rece.RECE_BF16, fake, fake, fake, fake, n.value,
                                   fake, None, None, fake) == 1   # NULL dX


def test_auto_size_follows_the_pages_rule():
    import math
    # n_b* = sqrt(4 alpha (1 + 2 n_ec) min(C, s)); the model 2 r sqrt(alpha (1 + 2 n_ec) min) max
    a = rece.auto_size(32768, 10_000_000, n_ec=1, alpha_bc=1.0, rounds=3)
    assert a["n_b"] == round(math.sqrt(4 * 3 * 32768)) == 627 and a["n_c"] == 627
    assert a["model_elems"] == pytest.approx(2 * 3 * math.sqrt(3 * 32768) * 10_000_000)
    assert a["full_ratio"] == pytest.approx(math.sqrt(32768) / (2 * 3 * math.sqrt(3)))
    # the model times the ratio is full cross-entropy's s x C
    assert a["model_elems"] * a["full_ratio"] == pytest.approx(32768 * 10_000_000)
    b = rece.auto_size(51200, 30000, n_ec=2, alpha_bc=0.5, rounds=2)
    assert b["n_b"] == round(math.sqrt(4 * 0.5 * 5 * 30000)) and b["n_c"] == round(b["n_b"] / 0.5)
    for bad in (dict(s=0), dict(C=0), dict(n_ec=-1), dict(alpha_bc=0.0), dict(rounds=0)):
        args = dict(s=10, C=10, n_ec=1, alpha_bc=1.0, rounds=1)
        args.update(bad)
        with pytest.raises(rece.ReceError):
            rece.auto_size(**args)


@pytest.mark.parametrize("name,below", [("sasrec", False), ("million", True), ("tenmillion", True)])
def test_workspace_against_the_pages_memory_model(name, below):
    """The page's model counts the method's intermediate arrays (chunk logit blocks
    among them) at its optimal n_b, in elements (taken as 4 bytes).  This
    implementation never stores a logit: at a million items and more its two
    workspaces together stay several times below the model, at the auto-sized plan
    and at the workload's own n_b.  At 30,000 items the model is small and the
    candidate lists (3k + 2 tiles of 8-byte entries per position, two sets for the
    rounds running side by side) take more; there the workspace stays within 3x."""
    from rece_inputs import WORKLOADS
    w = WORKLOADS[name]
    a = rece.auto_size(w.s, w.C, w.n_ec, 1.0, w.rounds)
    p = rece.auto_plan(w.s, w.C, w.d, w.k, w.rounds, n_ec=w.n_ec, dtype=w.dtype)
    assert (p.cfg.n_b, p.cfg.n_c) == (a["n_b"], a["n_c"])
    q = rece.Plan(w.s, w.C, w.d, w.n_b, w.n_c, w.k, w.rounds, dtype=w.dtype)
    model = 4 * a["model_elems"]
    for plan in (p, q):
        ws = plan.scratch_bytes + plan.saved_bytes
        if below:
            assert ws < model / 4
        else:
            assert ws < 3 * model
        assert ws < 4 * w.s * w.C            # always far below full cross-entropy's s x C logits
