"""Binding of libbgg_probe.so: streaming kernels of known byte counts that
the benchmark uses for the achievable HBM read rate and for calibrating the
profiler's byte counters (measurement only; not part of the library)."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbgg_probe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python bit_gemv_gemm_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_lib.bgg_probe_sink_words.restype = ctypes.c_size_t
_lib.bgg_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
_lib.bgg_probe_write.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
_lib.bgg_probe_empty.argtypes = [ctypes.c_uint, ctypes.c_uint, ctypes.c_void_p, ctypes.c_void_p]


def sink(device="cuda"):
    return torch.zeros(int(_lib.bgg_probe_sink_words()), dtype=torch.int32, device=device)


def read(buf: torch.Tensor, sink_t: torch.Tensor, stream=None) -> None:
    """Read all of buf (a multiple of 16 bytes) once."""
    assert buf.is_cuda and sink_t.numel() >= _lib.bgg_probe_sink_words()
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = _lib.bgg_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink_t.data_ptr(), s)
    if rc:
        raise RuntimeError(f"bgg_probe_read: HIP error {rc}")


def write(buf: torch.Tensor, stream=None) -> None:
    """Write zeros over all of buf (a multiple of 16 bytes)."""
    assert buf.is_cuda
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = _lib.bgg_probe_write(buf.data_ptr(), buf.numel() * buf.element_size(), s)
    if rc:
        raise RuntimeError(f"bgg_probe_write: HIP error {rc}")


def empty(grid: int, block: int, sink_t: torch.Tensor, stream=None) -> None:
    """Launch a kernel of grid x block threads that does no work."""
    assert sink_t.is_cuda
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = _lib.bgg_probe_empty(grid, block, sink_t.data_ptr(), s)
    if rc:
        raise RuntimeError(f"bgg_probe_empty: HIP error {rc}")
