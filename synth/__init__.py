"""Seeded synthetic inputs for the ternary linear layer y = W.x.

This module is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It draws random numbers and names workloads; it
holds none of the layer's arithmetic (no packing, no Hadamard transform, no
products).

Distributions (stand-ins for the weights and activations of the 27B-class
ternary model on the source pages; no trained weights exist here):

* trits   i.i.d., P(-1) = P(+1) = 0.31, P(0) = 0.38 (a 62 % non-zero rate, the
  order of the rate reported in lpnh.cn/news/2428882, section 2.1);
* signs   (the 1-bit weights of Q1_0) i.i.d., P(-1) = P(+1) = 1/2;
* float weights (input of the offline front end) i.i.d. N(0, 0.02^2), each
  an outlier 40 times larger with probability 0.004;
* scales  one per 128 weights along K (per 64 for Q2_0_g64), uniform in
  [0.005, 0.05], rounded to fp16 (round to nearest even);
* x       i.i.d. N(0, 1), rounded to fp16.

Every element is a counter-based SplitMix64 draw (see synth.c), so a row of a
matrix can be regenerated without generating the rest.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "_synth.so")
_lib = None

GROUP = 128  # weights per fp16 scale (and Hadamard block) along K
# Stream ids are 16 bits wide (synth.c keys a stream by id << 40 below an
# 8-bit tag); matrix ids stay below 0x4000, and the streams derived from a
# matrix id (its signs, its outlier mask) set one of the two top bits, so
# they never reuse the draws of another stream.
SIGN_STREAM = 0x4000
OUTLIER_STREAM = 0x8000


def build(force: bool = False) -> str:
    """Compile synth.c into _synth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, u64 = ctypes.c_int64, ctypes.c_uint64
        lib.synth_trits.argtypes = [u64, u64, i64, i64, ctypes.c_void_p]
        lib.synth_uniform.argtypes = [u64, u64, i64, i64, ctypes.c_void_p]
        lib.synth_normal.argtypes = [u64, u64, i64, i64, ctypes.c_void_p]
        lib.synth_hash.argtypes = [u64, u64, u64, u64]
        lib.synth_hash.restype = u64
        for f in (lib.synth_trits, lib.synth_uniform, lib.synth_normal):
            f.restype = None
        _lib = lib
    return _lib


def splitmix_hash(seed: int, tag: int, ident: int, index: int) -> int:
    return int(_load().synth_hash(seed, tag, ident, index))


def trits(seed: int, matrix_id: int, n: int, k: int, row0: int = 0) -> np.ndarray:
    """int8 [n, k] trits of rows row0..row0+n-1 of a matrix with k columns."""
    out = np.empty((n, k), dtype=np.int8)
    if out.size:
        _load().synth_trits(seed, matrix_id, row0 * k, out.size, out.ctypes.data)
    return out


def float_weights(seed: int, matrix_id: int, n: int, k: int, row0: int = 0) -> np.ndarray:
    """float32 [n, k] weights before ternarization: N(0, 0.02^2), and each
    element independently (probability 0.004) an outlier 40 times larger --
    a stand-in for the few large weights the pages say carry most of a
    layer's information (no trained weights exist here)."""
    z = np.empty((n, k), dtype=np.float64)
    u = np.empty((n, k), dtype=np.float64)
    if z.size:
        _load().synth_normal(seed, matrix_id, row0 * k, z.size, z.ctypes.data)
        _load().synth_uniform(seed, matrix_id ^ OUTLIER_STREAM, row0 * k, u.size, u.ctypes.data)
    return (0.02 * z * np.where(u < 0.004, 40.0, 1.0)).astype(np.float32)


def signs(seed: int, matrix_id: int, n: int, k: int, row0: int = 0) -> np.ndarray:
    """int8 [n, k] weights in {-1, +1}, each +1 with probability 1/2."""
    u = np.empty((n, k), dtype=np.float64)
    if u.size:
        _load().synth_uniform(seed, matrix_id ^ SIGN_STREAM, row0 * k, u.size, u.ctypes.data)
    return np.where(u < 0.5, 1, -1).astype(np.int8)


def weights(fmt: str, seed: int, matrix_id: int, n: int, k: int, row0: int = 0) -> np.ndarray:
    """The weights of a matrix stored in format fmt: signs for Q1_0, else trits."""
    return (signs if fmt == "Q1_0" else trits)(seed, matrix_id, n, k, row0)


def scale_group(fmt: str) -> int:
    """Weights per fp16 scale along K in format fmt (a property of the file
    format, used to size the scale arrays drawn here)."""
    return 64 if fmt == "Q2_0_G64" else GROUP


def scales_f16(seed: int, matrix_id: int, n: int, k: int, row0: int = 0,
               group: int = GROUP) -> np.ndarray:
    """fp16 [n, k/group] scales, uniform in [0.005, 0.05] then rounded to fp16."""
    g = k // group
    u = np.empty((n, g), dtype=np.float64)
    if u.size:
        _load().synth_uniform(seed, matrix_id, row0 * g, u.size, u.ctypes.data)
    return (0.005 + 0.045 * u).astype(np.float16)


def activations_f16(seed: int, stream_id: int, m: int, k: int, row0: int = 0) -> np.ndarray:
    """fp16 [m, k] activations, N(0,1) rounded to fp16."""
    z = np.empty((m, k), dtype=np.float64)
    if z.size:
        _load().synth_normal(seed, stream_id, row0 * k, z.size, z.ctypes.data)
    return z.astype(np.float16)


# ---------------------------------------------------------------------------
# Workloads: the five shapes of the 27B-class ternary stack.
# ---------------------------------------------------------------------------
HIDDEN, QDIM, KVDIM, FFN, LAYERS = 5120, 6144, 1024, 17408, 64

# projection name -> (K in, N out, id offset within a layer)
PROJECTIONS = {
    "q": (HIDDEN, QDIM, 0),
    "k": (HIDDEN, KVDIM, 1),
    "v": (HIDDEN, KVDIM, 2),
    "o": (QDIM, HIDDEN, 3),
    "gate": (HIDDEN, FFN, 4),
    "up": (HIDDEN, FFN, 5),
    "down": (FFN, HIDDEN, 6),
}


@dataclass(frozen=True)
class Matrix:
    name: str
    matrix_id: int
    n: int  # output rows
    k: int  # input columns


def matrix_id(layer: int, proj: str) -> int:
    return 7 * layer + PROJECTIONS[proj][2]


def decode_stack(layers: int = LAYERS):
    """All projections of a `layers`-deep stack, in execution order."""
    out = []
    for layer in range(layers):
        for proj in ("q", "k", "v", "o", "gate", "up", "down"):
            k, n, _ = PROJECTIONS[proj]
            out.append(Matrix(f"L{layer}.{proj}", matrix_id(layer, proj), n, k))
    return out


WORKLOADS = {
    "tiny": dict(seed=2027, matrices=[Matrix("tiny", 0, 256, 512)], m=[1]),
    "projection": dict(
        seed=2028,
        matrices=[Matrix("gate_up", matrix_id(0, "gate"), FFN, HIDDEN),
                  Matrix("down", matrix_id(0, "down"), HIDDEN, FFN)],
        m=[1]),
    "decode_step": dict(seed=2029, matrices=decode_stack(), m=[1]),
    "small_batch": dict(seed=2030, matrices=decode_stack(), m=[2, 4, 8, 16]),
    "prefill": dict(
        seed=2031,
        matrices=[Matrix("gate_up", matrix_id(0, "gate"), FFN, HIDDEN),
                  Matrix("down", matrix_id(0, "down"), HIDDEN, FFN)],
        m=[4096]),
}

ACT_STREAM = 1000  # activation stream ids start here (one per input width)


def workload_matrix(m: Matrix, seed: int, fmt: str = "PQ2_0"):
    """(weights int8 [n,k], scales fp16 [n,k/group]) of one workload matrix
    stored in format fmt (trits and a scale per 128 for PQ2_0 and PTQ1_0)."""
    return (weights(fmt, seed, m.matrix_id, m.n, m.k),
            scales_f16(seed, m.matrix_id, m.n, m.k, group=scale_group(fmt)))


def workload_x(seed: int, m: int, k: int) -> np.ndarray:
    return activations_f16(seed, ACT_STREAM + k, m, k)
