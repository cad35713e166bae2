"""Binding of libpeaks: what the device in hand sustains, for roofline fractions.

Two probes (include/peaks.h): a bf16 matrix-core loop with no memory traffic,
and a plain 16-byte-vector device copy.  Each is launched on torch's current
stream and timed there with events; the best of a few launches is reported.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpeaks.so")
EXPORTED = ["rece_peak_mfma_flops", "rece_peak_mfma_bf16", "rece_peak_copy"]

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpeaks.so not found at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.rece_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        L.rece_peak_mfma_flops.restype = ctypes.c_double
        L.rece_peak_mfma_bf16.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
        L.rece_peak_mfma_bf16.restype = ctypes.c_int
        L.rece_peak_copy.argtypes = [vp, vp, vp, ctypes.c_size_t]
        L.rece_peak_copy.restype = ctypes.c_int
        _lib = L
    return _lib


def _timed(launch, reps: int) -> float:
    """Best time in ms of `reps` launches on the current stream."""
    import torch
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rc = launch()
        b.record()
        if rc != 0:
            raise RuntimeError(f"libpeaks launch failed with HIP error {rc}")
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    return best


def mfma_bf16_tflops(device, blocks: int = 2048, iters: int = 2000, reps: int = 5) -> float:
    """Sustained dense bf16 matrix-core rate (TFLOP/s) of a loop that touches no memory."""
    import torch
    L = lib()
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    ptr = ctypes.c_void_p(sink.data_ptr())
    L.rece_peak_mfma_bf16(stream, blocks, 16, ptr)     # warm-up (code load)
    ms = _timed(lambda: L.rece_peak_mfma_bf16(stream, blocks, iters, ptr), reps)
    return L.rece_peak_mfma_flops(blocks, iters) / (ms * 1e-3) / 1e12


def copy_gbs(device, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Sustained HBM rate (GB/s) of a plain copy: 2 * nbytes moved per launch."""
    import torch
    L = lib()
    src = torch.ones(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    s, d = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())
    L.rece_peak_copy(stream, s, d, nbytes)
    ms = _timed(lambda: L.rece_peak_copy(stream, s, d, nbytes), reps)
    if not torch.equal(src[:: 1 << 20], dst[:: 1 << 20]):
        raise RuntimeError("copy probe: destination differs from source")
    return 2.0 * nbytes / (ms * 1e-3) / 1e9
