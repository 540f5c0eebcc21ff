"""ctypes binding of ``libattn_probe.so``: the HBM read probe declared in
include/attn_probe.h (argument marshalling only; the benchmark's read ceiling)."""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(HERE, "libattn_probe.so")
EXPORTS = ("attn_probe_read", "attn_probe_mfma", "attn_probe_clock", "attn_probe_rates", "attn_probe_grid")

_lib = None
_lock = threading.Lock()


def lib():
    """Load ``libattn_probe.so`` once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(PROBE_PATH):
                raise RuntimeError(f"{PROBE_PATH} is missing: build the HIP libraries first "
                                   "(python -m exact_attention_64_amd.build)")
            L = ctypes.CDLL(PROBE_PATH)
            L.attn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
            L.attn_probe_read.restype = ctypes.c_int32
            L.attn_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p]
            L.attn_probe_mfma.restype = ctypes.c_int32
            L.attn_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
            L.attn_probe_clock.restype = ctypes.c_int32
            L.attn_probe_rates.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
            L.attn_probe_rates.restype = ctypes.c_int32
            L.attn_probe_grid.argtypes = [ctypes.c_int32]
            L.attn_probe_grid.restype = ctypes.c_int32
            _lib = L
    return _lib


def probe_read(buf: torch.Tensor, nbytes: int = 0, chunk: int = 0, stride: int = 0, grid: int = 0,
               sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Read ``nbytes`` (default: all of ``buf``) in ``chunk``-byte pieces ``stride``
    bytes apart (default: contiguous) and return the per-work-group word sums
    (uint32 values in an int32 tensor)."""
    L = lib()
    nbytes = nbytes or buf.numel() * buf.element_size()
    chunk = chunk or nbytes
    stride = stride or chunk
    need = (nbytes // chunk - 1) * stride + chunk
    if need > buf.numel() * buf.element_size():
        raise ValueError(f"the pattern reaches byte {need}, past the buffer")
    g = L.attn_probe_grid(grid)
    if g < 0:
        raise RuntimeError(f"attn_probe_grid: status {g}")
    if sink is None:
        sink = torch.empty(g, dtype=torch.int32, device=buf.device)
    if sink.numel() < g or sink.dtype != torch.int32 or not sink.is_contiguous():
        raise ValueError(f"sink must be a contiguous int32 tensor of at least {g} entries")
    st = stream.cuda_stream if stream is not None else torch.cuda.current_stream(buf.device).cuda_stream
    rc = L.attn_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, chunk, stride,
                           ctypes.c_void_p(sink.data_ptr()), grid, ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"attn_probe_read: status {rc}")
    return sink


def _stream(dev, stream):
    return stream.cuda_stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream


def probe_mfma(iters: int, random_operands: bool, device="cuda:0", stream=None):
    """Enqueue the register-only MFMA loop; returns (out, ticks, flops): ``ticks``
    (int64 (2,)) receives the cycle- and steady-counter deltas of wave 0."""
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device=device)
    ticks = torch.zeros(2, dtype=torch.int64, device=device)
    rc = lib().attn_probe_mfma(ctypes.c_void_p(out.data_ptr()), iters, int(bool(random_operands)),
                               ctypes.c_void_p(ticks.data_ptr()), ctypes.c_void_p(_stream(device, stream)))
    if rc != 0:
        raise RuntimeError(f"attn_probe_mfma: status {rc}")
    return out, ticks, iters * 16 * 32768 * 8 * cus


def probe_clock(wall_ticks: int, device="cuda:0", stream=None, out=None):
    """Enqueue the one-wave clock probe; ``out`` (int64 (4,)) receives the cycle
    counter and the steady counter at its start and its end."""
    if out is None:
        out = torch.zeros(4, dtype=torch.int64, device=device)
    rc = lib().attn_probe_clock(ctypes.c_void_p(out.data_ptr()), int(wall_ticks),
                                ctypes.c_void_p(_stream(device, stream)))
    if rc != 0:
        raise RuntimeError(f"attn_probe_clock: status {rc}")
    return out


def rates():
    """(steady-counter rate, peak shader clock) of the current device, in Hz."""
    w, c = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().attn_probe_rates(ctypes.byref(w), ctypes.byref(c))
    if rc != 0:
        raise RuntimeError(f"attn_probe_rates: status {rc}")
    return w.value * 1000, c.value * 1000
