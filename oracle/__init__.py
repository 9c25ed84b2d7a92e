"""CPU oracle for the ternary Hadamard-rotated linear layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only code that may import this package.  The GPU
library never does, and this package imports nothing from it.

A thin ctypes wrapper over oracle.c (plain C loops in fp64, OpenMP over output
rows).  What each function follows on the source pages is stated in oracle.c:

* ``sylvester(n)``       explicit Sylvester Hadamard matrix, entries +-1;
* ``rotate(x)``          x' = blockdiag(H_128/sqrt(128)) x, dense mat-vecs, fp64;
* ``pack / unpack``      canonical PQ2_0 (2-bit slot, code t+1) and PTQ1_0
                         (5 trits per byte, little-endian base 3 of t+1), and
                         the sister formats Q1_0 (one sign bit per weight) and
                         Q2_0_g64 (the PQ2_0 stream);
* ``scale_group(fmt)``   weights per fp16 scale: 128, or 64 for Q2_0_g64;
* ``format_bytes``       bytes of a packed matrix incl. its fp16 scales;
* ``matvec(T, S, xr)``   y = sum_k S[n][k/group] T[n][k] xr[m][k] in fp64
                         (group = K / scales per row);
* ``linear(...)``        unpack + rotate + matvec from the stored form;
* ``f64_to_f16(v)``      one round-to-nearest-even conversion to fp16 bits;
* ``ternarize(W)``       the offline front end: rotate float weight rows per
                         128-block, scale = fp16(mean |w'|) per group (a
                         reading), trits = nearest of {-s, 0, s}.

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, library routines, brute force and the numbers the pages print.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

PQ2_0 = 1
PTQ1_0 = 2
Q1_0 = 3
Q2_0_G64 = 4
BLOCK = 128
FORMATS = {"PQ2_0": PQ2_0, "PTQ1_0": PTQ1_0, "Q1_0": Q1_0, "Q2_0_G64": Q2_0_G64}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into _oracle.so (gcc -O2 -fopenmp, no intrinsics, no BLAS)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_sylvester.argtypes = [ci, vp]
    lib.oracle_rotate.argtypes = [vp, i64, i64, vp]
    lib.oracle_row_bytes.argtypes = [ci, i64]
    lib.oracle_row_bytes.restype = i64
    lib.oracle_format_bytes.argtypes = [ci, i64, i64]
    lib.oracle_format_bytes.restype = i64
    lib.oracle_scale_group.argtypes = [ci]
    lib.oracle_scale_group.restype = i64
    lib.oracle_matvec_group.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
    lib.oracle_matvec_group.restype = ci
    lib.oracle_pack.argtypes = [ci, vp, i64, i64, vp]
    lib.oracle_unpack.argtypes = [ci, vp, i64, i64, vp]
    lib.oracle_matvec.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.oracle_linear.argtypes = [ci, vp, vp, vp, i64, i64, i64, ci, vp]
    lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_ternarize.argtypes = [vp, i64, i64, vp, vp]
    lib.oracle_ternarize.restype = ci
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ci
    lib.oracle_set_num_threads.argtypes = [ci]
    lib.oracle_set_num_threads.restype = None
    for f in (lib.oracle_sylvester, lib.oracle_rotate, lib.oracle_pack, lib.oracle_unpack,
              lib.oracle_matvec, lib.oracle_linear):
        f.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def swap_library(lib):
    """Route this module's functions to another build of oracle.c (used by the
    tests that plant mistakes in a copy of the oracle); returns the previous."""
    global _lib
    prev = _load()
    _lib = lib
    return prev


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _f16bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype == np.uint16:
        return a
    raise TypeError("expected float16 (or its uint16 bits)")


def num_threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Run the oracle's loops on n threads from now on (for timing)."""
    _load().oracle_set_num_threads(int(n))


def f16_to_f64(bits: int) -> float:
    return float(_load().oracle_f16_to_f64(int(bits) & 0xFFFF))


def sylvester(n: int) -> np.ndarray:
    H = np.empty((n, n), dtype=np.float64)
    _check(_load().oracle_sylvester(n, H.ctypes.data), "sylvester")
    return H


def rotate(x) -> np.ndarray:
    """fp64 [M, K] rotated activations from fp16 [M, K]."""
    xb = _f16bits(x)
    if xb.ndim == 1:
        xb = xb[None, :]
    M, K = xb.shape
    out = np.empty((M, K), dtype=np.float64)
    _check(_load().oracle_rotate(xb.ctypes.data, M, K, out.ctypes.data), "rotate")
    return out


def row_bytes(fmt, K: int) -> int:
    return int(_load().oracle_row_bytes(_fmt(fmt), K))


def scale_group(fmt) -> int:
    return int(_load().oracle_scale_group(_fmt(fmt)))


def format_bytes(fmt, N: int, K: int) -> int:
    return int(_load().oracle_format_bytes(_fmt(fmt), N, K))


def bits_per_weight(fmt, N: int, K: int) -> float:
    return 8.0 * format_bytes(fmt, N, K) / (N * K)


def pack(fmt, T) -> np.ndarray:
    T = np.ascontiguousarray(T, dtype=np.int8)
    N, K = T.shape
    out = np.empty((N, row_bytes(fmt, K)), dtype=np.uint8)
    _check(_load().oracle_pack(_fmt(fmt), T.ctypes.data, N, K, out.ctypes.data), "pack")
    return out


def unpack(fmt, packed, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] == row_bytes(fmt, K)
    T = np.empty((N, K), dtype=np.int8)
    _check(_load().oracle_unpack(_fmt(fmt), packed.ctypes.data, N, K, T.ctypes.data), "unpack")
    return T


def matvec(T, S, xr) -> np.ndarray:
    """fp64 [M, N] = products of weight rows T [N, K] with scales S (fp16
    [N, K/group]: K/128 scales per row, or K/64) and rotated activations xr
    (fp64 [M, K])."""
    T = np.ascontiguousarray(T, dtype=np.int8)
    Sb = _f16bits(S)
    xr = np.ascontiguousarray(xr, dtype=np.float64)
    if xr.ndim == 1:
        xr = xr[None, :]
    N, K = T.shape
    M = xr.shape[0]
    assert Sb.shape[0] == N and Sb.shape[1] >= 1 and K % Sb.shape[1] == 0 and xr.shape[1] == K
    group = K // Sb.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    if group == BLOCK:
        rc = _load().oracle_matvec(T.ctypes.data, Sb.ctypes.data, xr.ctypes.data, M, N, K,
                                   y.ctypes.data)
    else:
        rc = _load().oracle_matvec_group(T.ctypes.data, Sb.ctypes.data, xr.ctypes.data, M, N, K,
                                         group, y.ctypes.data)
    _check(rc, "matvec")
    return y


def linear(fmt, packed, S, x, rotate: bool = True) -> np.ndarray:
    """fp64 [M, N] output of the layer from canonical packed bytes, fp16
    scales and fp16 activations."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    Sb = _f16bits(S)
    xb = _f16bits(x)
    if xb.ndim == 1:
        xb = xb[None, :]
    N = packed.shape[0]
    M, K = xb.shape
    assert packed.shape[1] == row_bytes(fmt, K) and Sb.shape == (N, K // scale_group(fmt))
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_linear(_fmt(fmt), packed.ctypes.data, Sb.ctypes.data, xb.ctypes.data,
                                 M, N, K, 1 if rotate else 0, y.ctypes.data), "linear")
    return y


def f64_to_f16(v: float) -> int:
    """fp16 bits of v, rounded to nearest even (inf past the fp16 range)."""
    return int(_load().oracle_f64_to_f16(float(v)))


def ternarize(W):
    """Trits int8 [N, K] and fp16 scales [N, K/128] of float32 weights
    W [N, K] in the layer's stored coordinates (rotate, mean-magnitude
    scale per 128-group, nearest of {-s, 0, s})."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    T = np.empty((N, K), dtype=np.int8)
    S = np.empty((N, K // BLOCK), dtype=np.uint16)
    _check(_load().oracle_ternarize(W.ctypes.data, N, K, T.ctypes.data, S.ctypes.data),
           "ternarize")
    return T, S.view(np.float16)
