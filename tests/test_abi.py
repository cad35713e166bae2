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
    cfg = rece.ReceConfig(256, 2000, 64, 16, 16, 32, 1, 0, 0, 0, 0, 0)
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
    lists = w.rounds * w.s * w.k * 4 if w.variant == "rece" else 0
    assert p.scratch_bytes < w.s * w.C * 2
    assert p.saved_bytes - lists < w.s * w.C * 2
    assert p.scratch_bytes > 0 and p.saved_bytes > 0


def test_export_sizes():
    p = _plan(keep_stages=True, rounds=2)
    L = rece.lib()
    nb = ctypes.c_size_t()
    for stage, want in (("bucket_x", 256 * 4), ("bucket_y", 2000 * 4), ("perm_y", 2000 * 4),
                        ("thresh_logit", 256 * 8), ("neg_ids", 256 * 32 * 4), ("counters", 32)):
        assert L.rece_export_bytes(p._h, rece.STAGES[stage], ctypes.byref(nb)) == 0
        assert nb.value == want
    q = _plan()
    assert L.rece_export_bytes(q._h, rece.STAGES["neg_ids"], ctypes.byref(nb)) == 0 and nb.value == 0
    assert L.rece_export_bytes(q._h, 99, ctypes.byref(nb)) == 1


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
    r = _plan(keep_stages=True)
    assert L.rece_export_bytes(r._h, rece.STAGES["sce_rows"], ctypes.byref(nb)) == 0 and nb.value == 0
