"""Python binding of librece (RECE / SCE reduced cross-entropy on MI355X).

Argument marshalling only: every step of the loss runs in librece's HIP
kernels.  PyTorch supplies device memory (tensors) and the current stream.
There is no fallback: if librece.so is missing or cannot be loaded, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librece.so")

RECE_F32, RECE_BF16 = 0, 1
RECE_VARIANT_RECE, RECE_VARIANT_SCE = 0, 1
FLAG_VALIDATE_IDS, FLAG_KEEP_STAGES, FLAG_IGNORE_NEGATIVE_POS, FLAG_BF16_GRADS = 1, 2, 4, 8

STAGES = {
    "bucket_x": 0, "bucket_y": 1, "perm_x": 2, "perm_y": 3, "thresh_id": 4,
    "thresh_logit": 5, "neg_ids": 6, "lse": 7, "counters": 8, "sce_rows": 9, "sce_items": 10,
    "union_ids": 11,
}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
          4: "HIP runtime error", 5: "device check failed", 6: "internal error"}

EXPORTED = ["rece_plan", "rece_plan_destroy", "rece_workspace_bytes", "rece_forward",
            "rece_forward_static", "rece_backward", "rece_export", "rece_export_bytes", "rece_check",
            "rece_profile_enable", "rece_profile_read",
            "rece_full_ce_workspace_bytes", "rece_full_ce_forward", "rece_full_ce_backward", "rece_auto_size",
            "rece_status_string", "rece_last_error", "rece_version"]
PHASES = ["project", "sort", "select", "loss", "bwd_dx", "bwd_dy", "bwd_sort", "other"]


class ReceConfig(ctypes.Structure):
    """Mirror of rece_config in include/rece.h (field order and types)."""
    _fields_ = [("s", ctypes.c_int64), ("C", ctypes.c_int64), ("d", ctypes.c_int32),
                ("n_b", ctypes.c_int32), ("n_c", ctypes.c_int32), ("n_ec", ctypes.c_int32),
                ("k", ctypes.c_int32), ("rounds", ctypes.c_int32), ("b_x", ctypes.c_int32),
                ("b_y", ctypes.c_int32), ("dtype", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("window_wrap", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class ReceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"librece: {STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load librece.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"librece.so not found at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
        L.rece_plan.argtypes = [ctypes.POINTER(ReceConfig), ctypes.POINTER(vp)]
        L.rece_plan_destroy.argtypes = [vp]
        L.rece_workspace_bytes.argtypes = [vp, sz, sz]
        L.rece_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rece_forward_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rece_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rece_export.argtypes = [vp, vp, vp, i32, i32, vp]
        L.rece_export_bytes.argtypes = [vp, i32, sz]
        L.rece_check.argtypes = [vp, vp, vp]
        L.rece_profile_enable.argtypes = [vp, i32]
        L.rece_profile_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
        i64 = ctypes.c_int64
        L.rece_full_ce_workspace_bytes.argtypes = [i64, sz]
        L.rece_full_ce_forward.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
        L.rece_full_ce_backward.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp,
                                            vp]
        L.rece_auto_size.argtypes = [i64, i64, i32, ctypes.c_double, i32, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double)]
        L.rece_status_string.argtypes = [i32]
        L.rece_status_string.restype = ctypes.c_char_p
        L.rece_last_error.restype = ctypes.c_char_p
        L.rece_version.restype = ctypes.c_char_p
        for name in ("rece_plan", "rece_plan_destroy", "rece_workspace_bytes", "rece_forward",
                     "rece_forward_static", "rece_backward", "rece_export", "rece_export_bytes", "rece_check",
                     "rece_profile_enable", "rece_profile_read", "rece_full_ce_workspace_bytes",
                     "rece_full_ce_forward", "rece_full_ce_backward", "rece_auto_size"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise ReceError(status, lib().rece_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Plan:
    """An immutable librece plan (host only) plus its workspace sizes."""

    def __init__(self, s: int, C: int, d: int, n_b: int, n_c: int, k: int, rounds: int = 1,
                 dtype: str = "bf16", variant: str = "rece", b_x: int = 0, b_y: int = 0,
                 keep_stages: bool = False, validate_ids: bool = False, n_ec: int = 1,
                 window_wrap: bool = True, ignore_negative_pos: bool = False, bf16_grads: bool = False):
        self.cfg = ReceConfig(s, C, d, n_b, n_c, n_ec, k, rounds, b_x, b_y,
                              RECE_BF16 if dtype == "bf16" else RECE_F32,
                              RECE_VARIANT_SCE if variant == "sce" else RECE_VARIANT_RECE,
                              int(window_wrap),
                              (FLAG_KEEP_STAGES if keep_stages else 0)
                              | (FLAG_VALIDATE_IDS if validate_ids else 0)
                              | (FLAG_IGNORE_NEGATIVE_POS if ignore_negative_pos else 0)
                              | (FLAG_BF16_GRADS if bf16_grads else 0))
        self.bf16_grads = bool(bf16_grads)
        self.dtype = dtype
        self._h = ctypes.c_void_p()
        _check(lib().rece_plan(ctypes.byref(self.cfg), ctypes.byref(self._h)))
        sc, sv = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().rece_workspace_bytes(self._h, ctypes.byref(sc), ctypes.byref(sv)))
        self.scratch_bytes, self.saved_bytes = sc.value, sv.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.rece_plan_destroy(h)
            self._h = None

    # -- argument checks (shapes, dtypes, devices); the library checks pointers again
    def _check_inputs(self, X, Y, pos, B=None):
        import torch
        c = self.cfg
        want = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        for name, t, shape in (("X", X, (c.s, c.d)), ("Y", Y, (c.C, c.d))):
            if t.dtype != want or tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous CUDA {want} tensor of shape {shape}")
        if (pos.dtype != torch.int32 or tuple(pos.shape) != (c.s,) or not pos.is_cuda
                or not pos.is_contiguous()):
            raise ValueError(f"pos must be a contiguous CUDA int32 tensor of shape ({c.s},)")
        for name, t in (("Y", Y), ("pos", pos)) + ((("B", B),) if B is not None else ()):
            if t.device != X.device:
                raise ValueError(f"{name} must be on the same device as X ({X.device})")
        if B is not None:
            shape = (c.rounds, c.d, c.n_b) if c.variant == RECE_VARIANT_RECE else (c.d, c.n_b)
            if B.dtype != want or tuple(B.shape) != shape or not B.is_cuda or not B.is_contiguous():
                raise ValueError(f"B must be a contiguous CUDA {want} tensor of shape {shape}")

    def _check_workspace(self, scratch, saved, device):
        for name, t, size in (("scratch", scratch, self.scratch_bytes), ("saved", saved, self.saved_bytes)):
            if t.device != device or t.numel() * t.element_size() < size or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous buffer of at least {size} bytes on {device}")

    def workspace(self, device="cuda"):
        import torch
        scratch = torch.empty(max(self.scratch_bytes, 16), dtype=torch.uint8, device=device)
        saved = torch.empty(max(self.saved_bytes, 16), dtype=torch.uint8, device=device)
        return scratch, saved

    def forward(self, X, Y, pos, B, scratch=None, saved=None, loss_pp=True, stream=None):
        """Returns (loss [1], loss_pp [s] or None, scratch, saved)."""
        import torch
        self._check_inputs(X, Y, pos, B)
        if scratch is None or saved is None:
            scratch, saved = self.workspace(X.device)
        self._check_workspace(scratch, saved, X.device)
        loss = torch.empty(1, dtype=torch.float32, device=X.device)
        lpp = torch.empty(self.cfg.s, dtype=torch.float32, device=X.device) if loss_pp else None
        _check(lib().rece_forward(self._h, _stream(stream), _ptr(X), _ptr(Y), _ptr(pos), _ptr(B),
                                  _ptr(scratch), _ptr(saved), _ptr(loss), _ptr(lpp)))
        return loss, lpp, scratch, saved

    def forward_static(self, X, Y, pos, B, saved=None, loss=None, loss_pp=None, stream=None):
        """rece_forward_static: the forward pass on the library's static scratch array.
        saved, loss [1] and loss_pp [s] (optional) are the caller's; returns (loss, loss_pp, saved)."""
        import torch
        self._check_inputs(X, Y, pos, B)
        if saved is None:
            saved = torch.empty(max(self.saved_bytes, 16), dtype=torch.uint8, device=X.device)
        if loss is None:
            loss = torch.empty(1, dtype=torch.float32, device=X.device)
        for name, t, shape in (("loss", loss, (1,)), ("loss_pp", loss_pp, (self.cfg.s,))):
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()
                                  or t.device != X.device):
                raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shape} on {X.device}")
        if saved.device != X.device or saved.numel() * saved.element_size() < self.saved_bytes:
            raise ValueError(f"saved must hold at least {self.saved_bytes} bytes on {X.device}")
        _check(lib().rece_forward_static(self._h, _stream(stream), _ptr(X), _ptr(Y), _ptr(pos), _ptr(B),
                                         _ptr(saved), _ptr(loss), _ptr(loss_pp)))
        return loss, loss_pp, saved

    def backward(self, X, Y, pos, scratch, saved, dloss=None, dloss_pp=None, dX=None, dY=None,
                 stream=None):
        """Returns (dX [s, d], dY [C, d]): float32, or bf16 for a plan made with bf16_grads."""
        import torch
        self._check_inputs(X, Y, pos)
        c = self.cfg
        gdt = torch.bfloat16 if self.bf16_grads else torch.float32
        if dloss is None and dloss_pp is None:
            dloss = torch.ones(1, dtype=torch.float32, device=X.device)
        if dX is None:
            dX = torch.empty((c.s, c.d), dtype=gdt, device=X.device)
        if dY is None:
            dY = torch.empty((c.C, c.d), dtype=gdt, device=X.device)
        for name, t, shape, dt in (("dX", dX, (c.s, c.d), gdt), ("dY", dY, (c.C, c.d), gdt),
                                   ("dloss", dloss, (1,), torch.float32),
                                   ("dloss_pp", dloss_pp, (c.s,), torch.float32)):
            if t is None:
                continue
            if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != X.device:
                raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape} on {X.device}")
        self._check_workspace(scratch, saved, X.device)
        _check(lib().rece_backward(self._h, _stream(stream), _ptr(X), _ptr(Y), _ptr(pos),
                                   _ptr(dloss), _ptr(dloss_pp), _ptr(scratch), _ptr(saved),
                                   _ptr(dX), _ptr(dY)))
        return dX, dY

    def export(self, saved, stage: str, round: int = 0, stream=None):
        import torch
        st = STAGES[stage]
        nb = ctypes.c_size_t()
        _check(lib().rece_export_bytes(self._h, st, ctypes.byref(nb)))
        dt = {"thresh_logit": torch.float64, "lse": torch.float32, "counters": torch.int32}.get(stage, torch.int32)
        n = nb.value // torch.empty(0, dtype=dt).element_size()
        out = torch.empty(n, dtype=dt, device=saved.device)
        _check(lib().rece_export(self._h, _stream(stream), _ptr(saved), st, round, _ptr(out)))
        if stage == "neg_ids":
            out = out.view(self.cfg.s, max(self.cfg.k, 1))
        elif stage == "union_ids":
            r = self.cfg.rounds if self.cfg.variant == RECE_VARIANT_RECE else 1
            out = out.view(self.cfg.s, r * max(self.cfg.k, 1))
        elif stage == "sce_rows":
            out = out.view(self.cfg.n_b, self.cfg.b_x)
        elif stage == "sce_items":
            out = out.view(self.cfg.n_b, self.cfg.b_y)
        return out

    def profile(self, phases=None, enable: bool = True):
        """Start (clearing earlier records) or stop event timing of this plan's kernels.
        phases: None for all, else an iterable of phase names."""
        if not enable:
            mask = 0
        elif phases is None:
            mask = -1
        else:
            mask = 0
            for ph in phases:
                mask |= 1 << PHASES.index(ph)
        _check(lib().rece_profile_enable(self._h, mask))

    def profile_read(self):
        """{phase: (total ms, launches)} since profiling was last enabled (waits for the GPU)."""
        out = {}
        for i, name in enumerate(PHASES):
            ms, n = ctypes.c_double(), ctypes.c_int64()
            _check(lib().rece_profile_read(self._h, i, ctypes.byref(ms), ctypes.byref(n)))
            out[name] = (ms.value, n.value)
        return out

    def check(self, saved, stream=None):
        _check(lib().rece_check(self._h, _stream(stream), _ptr(saved)))


def auto_size(s: int, C: int, n_ec: int = 1, alpha_bc: float = 1.0, rounds: int = 1) -> dict:
    """The RECE page's sizing rule (n_b*, n_c) and memory model; see rece_auto_size."""
    nb, nc = ctypes.c_int32(), ctypes.c_int32()
    me, fr = ctypes.c_double(), ctypes.c_double()
    _check(lib().rece_auto_size(s, C, n_ec, float(alpha_bc), rounds, ctypes.byref(nb), ctypes.byref(nc),
                                ctypes.byref(me), ctypes.byref(fr)))
    return {"n_b": nb.value, "n_c": nc.value, "model_elems": me.value, "full_ratio": fr.value}


def auto_plan(s: int, C: int, d: int, k: int, rounds: int = 1, n_ec: int = 1, alpha_bc: float = 1.0,
              **kw) -> "Plan":
    """A Plan with n_b and n_c from the page's rule for the lowest peak memory."""
    a = auto_size(s, C, n_ec, alpha_bc, rounds)
    return Plan(s, C, d, a["n_b"], a["n_c"], k, rounds, n_ec=n_ec, **kw)


class ReceLossFunction:
    """torch.autograd.Function over a Plan: forward = rece_forward (mean loss),
    backward = rece_backward with the incoming gradient of the loss.  The random
    vectors B (RECE: [rounds, d, n_b]; SCE: [d, n_b]) are an input: the caller
    draws them (fresh per step, as the method does) and they get no gradient.
    Gradients come back in the plan's gradient dtype (bf16_grads: bf16), which must
    match X and Y's dtype for autograd."""

    _fn = None

    @classmethod
    def get(cls):
        if cls._fn is None:
            import torch

            class _F(torch.autograd.Function):
                @staticmethod
                def forward(ctx, X, Y, pos, B, plan):
                    loss, _, scratch, saved = plan.forward(X, Y, pos, B, loss_pp=False)
                    ctx.save_for_backward(X, Y, pos)
                    ctx.plan, ctx.scratch, ctx.saved = plan, scratch, saved
                    return loss.reshape(())

                @staticmethod
                def backward(ctx, g):
                    X, Y, pos = ctx.saved_tensors
                    dloss = g.reshape(1).to(torch.float32).contiguous()
                    dX, dY = ctx.plan.backward(X, Y, pos, ctx.scratch, ctx.saved, dloss=dloss)
                    ctx.scratch = ctx.saved = None
                    return (dX if ctx.needs_input_grad[0] else None, dY if ctx.needs_input_grad[1] else None,
                            None, None, None)

            cls._fn = _F
        return cls._fn


def rece_loss(X, Y, pos, B, plan: "Plan"):
    """Mean RECE (or SCE) loss with autograd: X [s, d], Y [C, d], pos [s] int32 (with
    a plan made with ignore_negative_pos, negative ids mark padding)."""
    return ReceLossFunction.get().apply(X, Y, pos, B, plan)


class FullCE:
    """Exact full cross-entropy over the whole catalogue (no [s, C] tensor): the
    forward pass leaves each position's log-sum-exp in `workspace` for the backward
    pass.  Marshalling only; the sweeps run in librece's kernels."""

    def __init__(self, s: int, C: int, d: int, dtype: str = "bf16"):
        self.s, self.C, self.d, self.dtype = s, C, d, dtype
        n = ctypes.c_size_t()
        _check(lib().rece_full_ce_workspace_bytes(s, ctypes.byref(n)))
        self.workspace_bytes = n.value

    def _check_inputs(self, X, Y, pos, workspace):
        import torch
        want = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if X.shape != (self.s, self.d) or Y.shape != (self.C, self.d) or pos.shape != (self.s,):
            raise ValueError("X, Y, pos shapes do not match the full cross-entropy sizes")
        if X.dtype != want or Y.dtype != want or pos.dtype != torch.int32:
            raise ValueError("X, Y must have the plan dtype and pos int32")
        if not (X.is_contiguous() and Y.is_contiguous() and pos.is_contiguous()):
            raise ValueError("X, Y, pos must be contiguous")
        if workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        devs = {t.device for t in (X, Y, pos, workspace)}
        if len(devs) != 1 or next(iter(devs)).type != "cuda":
            raise ValueError("all tensors must be on one GPU")

    def forward(self, X, Y, pos, workspace=None, loss_pp=True, stream=None):
        import torch
        dev = X.device
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=dev)
        self._check_inputs(X, Y, pos, workspace)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lpp = torch.empty(self.s, dtype=torch.float32, device=dev) if loss_pp else None
        _check(lib().rece_full_ce_forward(_stream(stream), self.s, self.C, self.d,
                                          RECE_BF16 if self.dtype == "bf16" else RECE_F32, _ptr(X), _ptr(Y),
                                          _ptr(pos), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _ptr(loss), _ptr(lpp)))
        return loss, lpp, workspace

    def backward(self, X, Y, pos, workspace, dloss=None, dloss_pp=None, dX=None, dY=None, stream=None):
        import torch
        dev = X.device
        self._check_inputs(X, Y, pos, workspace)
        if dloss is None and dloss_pp is None:
            dloss = torch.ones(1, dtype=torch.float32, device=dev)
        for t, n in ((dloss, 1), (dloss_pp, self.s)):
            if t is not None and (t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous()):
                raise ValueError("dloss / dloss_pp must be contiguous float32 of 1 / s elements")
        if dX is None:
            dX = torch.empty((self.s, self.d), dtype=torch.float32, device=dev)
        if dY is None:
            dY = torch.empty((self.C, self.d), dtype=torch.float32, device=dev)
        if dX.shape != (self.s, self.d) or dY.shape != (self.C, self.d) or dX.dtype != torch.float32 \
                or dY.dtype != torch.float32 or not (dX.is_contiguous() and dY.is_contiguous()):
            raise ValueError("dX, dY must be contiguous float32 [s, d] and [C, d]")
        _check(lib().rece_full_ce_backward(_stream(stream), self.s, self.C, self.d,
                                           RECE_BF16 if self.dtype == "bf16" else RECE_F32, _ptr(X), _ptr(Y),
                                           _ptr(pos), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _ptr(dloss), _ptr(dloss_pp), _ptr(dX), _ptr(dY)))
        return dX, dY


def version() -> str:
    return lib().rece_version().decode()
