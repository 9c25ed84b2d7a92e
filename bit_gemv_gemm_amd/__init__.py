"""Python binding of libbgg.so (include/bgg.h), argument marshalling only.

Every function has the name of the C entry point it calls.  Host buffers are
numpy arrays; device buffers are torch tensors on the ROCm device (PyTorch is
used for device memory and streams, nothing else).  A non-OK status raises
BggError carrying the library's message.  There is no fallback: if
libbgg.so is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# PyTorch ships its own HIP runtime (libamdhip64.so.7, same soname as the
# system one).  libbgg.so must bind to the runtime PyTorch uses, so PyTorch
# is loaded first; loading libbgg.so first would pull the system runtime into
# the process and leave PyTorch running on a runtime it was not built for.
import torch  # noqa: F401  (load order matters, see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbgg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python bit_gemv_gemm_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

BGG_FMT_PQ2_0 = 1
BGG_FMT_PTQ1_0 = 2
BGG_FMT_Q1_0 = 3
BGG_FMT_Q2_0_G64 = 4
FORMATS = {"PQ2_0": BGG_FMT_PQ2_0, "PTQ1_0": BGG_FMT_PTQ1_0, "Q1_0": BGG_FMT_Q1_0,
           "Q2_0_G64": BGG_FMT_Q2_0_G64}
BGG_ROTATE_INPUT = 1
BGG_GROUP = 128
BGG_ROW_TILE = 64
BGG_CHUNK = 16
BGG_MAX_GEMV_M = 16
BGG_READ_SLACK = 8192
STATUS = {0: "BGG_OK", 1: "BGG_ERR_NULL", 2: "BGG_ERR_FORMAT", 3: "BGG_ERR_SHAPE",
          4: "BGG_ERR_TRIT", 5: "BGG_ERR_PACKED_BYTE", 6: "BGG_ERR_BUFFER", 7: "BGG_ERR_DESC",
          8: "BGG_ERR_HIP", 9: "BGG_ERR_SCALE"}


class bgg_weights_desc(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("format", ctypes.c_int32), ("row_tile", ctypes.c_int32),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("groups", ctypes.c_int64),
                ("row_tiles", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                ("chunks", ctypes.c_int64), ("trit_bytes", ctypes.c_uint64),
                ("scale_offset", ctypes.c_uint64), ("scale_bytes", ctypes.c_uint64),
                ("total_bytes", ctypes.c_uint64), ("format_bytes", ctypes.c_uint64),
                ("scale_group", ctypes.c_int64), ("scales", ctypes.c_int64)]

    def __repr__(self):
        return "bgg_weights_desc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class BggError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.bgg_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


_P = ctypes.POINTER(bgg_weights_desc)
_vp, _i64, _u32, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "bgg_describe": ([_i32, _i64, _i64, _P], _i32),
    "bgg_pack_weights": ([_P, _vp, _vp, _vp], _i32),
    "bgg_repack_canonical": ([_P, _vp, _vp, _vp], _i32),
    "bgg_validate_packed": ([_P, _vp], _i32),
    "bgg_unpack_weights": ([_P, _vp, _vp, _vp, _vp], _i32),
    "bgg_hadamard_rotate": ([_vp, _vp, _i64, _i64, _vp], _i32),
    "bgg_rotate_ternarize": ([_vp, _i64, _i64, _vp, _vp, _vp], _i32),
    "bgg_gemv_workspace_size": ([_P, _i64], _sz),
    "bgg_gemv_workspace_reset": ([_vp, _sz, _vp], _i32),
    "bgg_ternary_gemv": ([_P, _vp, _vp, _vp, _i64, _u32, _vp, _sz, _vp], _i32),
    "bgg_ternary_gemv_noalloc": ([_P, _vp, _vp, _vp, _i64, _u32, _vp], _i32),
    "bgg_gemv_prepare": ([_P, _vp, _i64, _u32, _vp, _sz, _vp], _i32),
    "bgg_gemv_run": ([_P, _vp, _vp, _i64, _vp, _sz, _vp], _i32),
    "bgg_gemv_kernel_name": ([_P, _i64, ctypes.c_char_p, _sz], _i32),
    "bgg_gemm_workspace_size": ([_P, _i64], _sz),
    "bgg_ternary_gemm": ([_P, _vp, _vp, _vp, _i64, _u32, _vp, _sz, _vp], _i32),
    "bgg_status_string": ([_i32], ctypes.c_char_p),
    "bgg_last_error": ([], ctypes.c_char_p),
    "bgg_abi_version": ([], _u32),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


def _ok(status: int, where: str):
    if status != 0:
        raise BggError(status, where)


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _host_ptr(a, dtype, shape=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16 and dtype == np.uint16:
        a = a.view(np.uint16)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    return a, a.ctypes.data


def _dev_ptr(t, min_bytes=0, what="buffer"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    nbytes = t.numel() * t.element_size()
    if nbytes < min_bytes:
        raise ValueError(f"{what} has {nbytes} bytes, needs {min_bytes}")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# host calls
# ---------------------------------------------------------------------------
def bgg_describe(fmt, N: int, K: int) -> bgg_weights_desc:
    d = bgg_weights_desc()
    _ok(_lib.bgg_describe(_fmt(fmt), N, K, ctypes.byref(d)), "bgg_describe")
    return d


def bgg_pack_weights(desc: bgg_weights_desc, trits, scales) -> np.ndarray:
    """Host int8 trits [N][K] and fp16 scales [N][K/128] -> packed bytes (host)."""
    t, tp = _host_ptr(trits, np.int8, (desc.N, desc.K))
    s, sp = _host_ptr(scales, np.uint16, (desc.N, desc.scales))
    out = np.empty(desc.total_bytes, dtype=np.uint8)
    _ok(_lib.bgg_pack_weights(ctypes.byref(desc), tp, sp, out.ctypes.data), "bgg_pack_weights")
    return out


def bgg_repack_canonical(desc: bgg_weights_desc, canonical, scales) -> np.ndarray:
    c, cp = _host_ptr(canonical, np.uint8, (desc.N, desc.row_bytes))
    s, sp = _host_ptr(scales, np.uint16, (desc.N, desc.scales))
    out = np.empty(desc.total_bytes, dtype=np.uint8)
    _ok(_lib.bgg_repack_canonical(ctypes.byref(desc), cp, sp, out.ctypes.data), "bgg_repack_canonical")
    return out


def bgg_validate_packed(desc: bgg_weights_desc, packed) -> None:
    p, pp = _host_ptr(packed, np.uint8)
    if p.size < desc.total_bytes:
        raise ValueError("packed buffer too small")
    _ok(_lib.bgg_validate_packed(ctypes.byref(desc), pp), "bgg_validate_packed")


def bgg_status_string(status: int) -> str:
    return _lib.bgg_status_string(status).decode()


def bgg_last_error() -> str:
    return _lib.bgg_last_error().decode()


def bgg_abi_version() -> int:
    return int(_lib.bgg_abi_version())


def bgg_gemv_workspace_size(desc: bgg_weights_desc, M: int) -> int:
    return int(_lib.bgg_gemv_workspace_size(ctypes.byref(desc), M))


def bgg_gemv_kernel_name(desc: bgg_weights_desc, M: int) -> str:
    buf = ctypes.create_string_buffer(96)
    _ok(_lib.bgg_gemv_kernel_name(ctypes.byref(desc), M, buf, len(buf)), "bgg_gemv_kernel_name")
    return buf.value.decode()


def bgg_gemm_workspace_size(desc: bgg_weights_desc, M: int) -> int:
    return int(_lib.bgg_gemm_workspace_size(ctypes.byref(desc), M))


# ---------------------------------------------------------------------------
# device calls (torch tensors on the ROCm device)
# ---------------------------------------------------------------------------
def bgg_unpack_weights(desc, packed_dev, trits_dev, scales_dev, stream=None) -> None:
    _ok(_lib.bgg_unpack_weights(
        ctypes.byref(desc), _dev_ptr(packed_dev, desc.total_bytes, "packed"),
        _dev_ptr(trits_dev, desc.N * desc.K, "trits"),
        _dev_ptr(scales_dev, desc.N * desc.scales * 2, "scales"), _stream(stream)),
        "bgg_unpack_weights")


def bgg_hadamard_rotate(x_dev, xr_dev, M: int, K: int, stream=None) -> None:
    _ok(_lib.bgg_hadamard_rotate(_dev_ptr(x_dev, M * K * 2, "x"), _dev_ptr(xr_dev, M * K * 2, "xr"),
                                 M, K, _stream(stream)), "bgg_hadamard_rotate")


def bgg_rotate_ternarize(w_dev, N: int, K: int, trits_dev, scales_dev, stream=None) -> None:
    """Device float32 weights [N, K] -> device int8 trits [N, K] and fp16
    scales [N, K/128] in the layer's stored coordinates."""
    _ok(_lib.bgg_rotate_ternarize(_dev_ptr(w_dev, N * K * 4, "w"), N, K,
                                  _dev_ptr(trits_dev, N * K, "trits"),
                                  _dev_ptr(scales_dev, N * (K // 128) * 2, "scales"),
                                  _stream(stream)), "bgg_rotate_ternarize")


def bgg_ternary_gemv(desc, packed_dev, x_dev, y_dev, M: int, flags: int, workspace, stream=None) -> None:
    ws = _dev_ptr(workspace, 0, "workspace")
    wsb = workspace.numel() * workspace.element_size()
    _ok(_lib.bgg_ternary_gemv(ctypes.byref(desc), _dev_ptr(packed_dev, desc.total_bytes, "packed"),
                              _dev_ptr(x_dev, M * desc.K * 2, "x"), _dev_ptr(y_dev, M * desc.N * 2, "y"),
                              M, flags, ws, wsb, _stream(stream)), "bgg_ternary_gemv")


def bgg_gemv_workspace_reset(workspace, stream=None) -> None:
    wsb = workspace.numel() * workspace.element_size()
    _ok(_lib.bgg_gemv_workspace_reset(_dev_ptr(workspace, 0, "workspace"), wsb, _stream(stream)),
        "bgg_gemv_workspace_reset")


def bgg_ternary_gemv_noalloc(desc, packed_dev, x_dev, y_dev, M: int, flags: int, stream=None) -> None:
    _ok(_lib.bgg_ternary_gemv_noalloc(ctypes.byref(desc), _dev_ptr(packed_dev, desc.total_bytes, "packed"),
                                      _dev_ptr(x_dev, M * desc.K * 2, "x"), _dev_ptr(y_dev, M * desc.N * 2, "y"),
                                      M, flags, _stream(stream)), "bgg_ternary_gemv_noalloc")


def bgg_gemv_prepare(desc, x_dev, M: int, flags: int, workspace, stream=None) -> None:
    ws = _dev_ptr(workspace, 0, "workspace")
    wsb = workspace.numel() * workspace.element_size()
    _ok(_lib.bgg_gemv_prepare(ctypes.byref(desc), _dev_ptr(x_dev, M * desc.K * 2, "x"), M, flags, ws,
                              wsb, _stream(stream)), "bgg_gemv_prepare")


def bgg_gemv_run(desc, packed_dev, y_dev, M: int, workspace, stream=None) -> None:
    ws = _dev_ptr(workspace, 0, "workspace")
    wsb = workspace.numel() * workspace.element_size()
    _ok(_lib.bgg_gemv_run(ctypes.byref(desc), _dev_ptr(packed_dev, desc.total_bytes, "packed"),
                          _dev_ptr(y_dev, M * desc.N * 2, "y"), M, ws, wsb, _stream(stream)),
        "bgg_gemv_run")


def bgg_ternary_gemm(desc, packed_dev, x_dev, y_dev, M: int, flags: int, workspace, stream=None) -> None:
    ws = _dev_ptr(workspace, 0, "workspace") if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _ok(_lib.bgg_ternary_gemm(ctypes.byref(desc), _dev_ptr(packed_dev, desc.total_bytes, "packed"),
                              _dev_ptr(x_dev, M * desc.K * 2, "x"), _dev_ptr(y_dev, M * desc.N * 2, "y"),
                              M, flags, ws, wsb, _stream(stream)), "bgg_ternary_gemm")


# ---------------------------------------------------------------------------
# small conveniences over the calls above (allocation through torch)
# ---------------------------------------------------------------------------
def upload(host_bytes: np.ndarray, device="cuda"):
    """Copy a packed host buffer to a new device uint8 tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(host_bytes)).to(device)


def workspace(nbytes: int, device="cuda"):
    """A zero-filled device workspace (the GEMV's split-K row sums must start
    at zero; every GEMV call leaves them so)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
