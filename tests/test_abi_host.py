"""Host-side tests of libbgg.so: exported symbols, descriptors, packing into
the device layout, validation and error codes.  No GPU calls."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_gemv_gemm_amd as bgg
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bgg.h")
FMTS = ("PQ2_0", "PTQ1_0", "Q1_0", "Q2_0_G64")
# the byte of zero trits (Q1_0: all -1, under a zero scale in padding rows)
ZERO_BYTE = {"PQ2_0": 0x55, "PTQ1_0": 121, "Q1_0": 0x00, "Q2_0_G64": 0x55}
RNG = np.random.default_rng(99)


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bgg_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(bgg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in bgg.h but not exported"
    assert set(names) == set(bgg.EXPORTED), "binding and header disagree"


def test_abi_version_and_status_strings():
    assert bgg.bgg_abi_version() == 3
    for s in range(10):
        assert bgg.bgg_status_string(s)
    assert bgg.bgg_status_string(0) == "ok"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 128), (64, 512), (100, 640), (256, 5120), (5120, 17408), (17408, 5120)])
def test_describe_sizes(fmt, N, K):
    d = bgg.bgg_describe(fmt, N, K)
    assert d.groups == K // 128
    assert d.scale_group == oracle.scale_group(fmt)
    assert d.scales == K // d.scale_group
    assert d.row_bytes == oracle.row_bytes(fmt, K)
    assert d.format_bytes == oracle.format_bytes(fmt, N, K)
    assert d.row_tiles == -(-N // 64)
    assert d.chunks == -(-d.row_bytes // 16)
    assert d.trit_bytes == d.row_tiles * d.chunks * 1024
    assert d.scale_offset % 256 == 0 and d.scale_offset >= d.trit_bytes
    assert d.scale_bytes == d.row_tiles * d.scales * 128
    assert d.total_bytes == d.scale_offset + d.scale_bytes + bgg.BGG_READ_SLACK


def test_describe_rejects_bad_shapes_and_formats():
    for (f, N, K, st) in [(5, 64, 128, 2), (0, 64, 128, 2), (3, 64, 64, 3), (4, 64, 192, 3), (1, 0, 128, 3), (1, 64, 100, 3),
                          (2, 64, 0, 3), (2, 64, 64, 3), (1, -5, 128, 3)]:
        with pytest.raises(bgg.BggError) as e:
            bgg.bgg_describe(f, N, K)
        assert e.value.status == st


def _canonical_from_layout(d, packed):
    """Read row r's canonical byte stream back out of the tiled device layout
    (the layout documented in bgg.h)."""
    C, G = d.chunks, d.scales
    tiles = packed[:d.trit_bytes].reshape(d.row_tiles, C, 64, 16)
    rows = tiles.transpose(0, 2, 1, 3).reshape(d.row_tiles * 64, C * 16)
    sc = packed[d.scale_offset:d.scale_offset + d.scale_bytes].view(np.uint16)
    sc = sc.reshape(d.row_tiles, G, 64).transpose(0, 2, 1).reshape(d.row_tiles * 64, G)
    return rows, sc


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 128), (100, 640), (130, 1152), (64, 6144)])
def test_pack_layout_matches_oracle_canonical_bytes(fmt, N, K):
    T = synth.weights(fmt, 5, 1, N, K)
    S = synth.scales_f16(5, 1, N, K, group=synth.scale_group(fmt))
    d = bgg.bgg_describe(fmt, N, K)
    packed = bgg.bgg_pack_weights(d, T, S)
    rows, sc = _canonical_from_layout(d, packed)
    canon = oracle.pack(fmt, T)
    assert np.array_equal(rows[:N, :d.row_bytes], canon)
    zero = ZERO_BYTE[fmt]
    assert np.all(rows[:N, d.row_bytes:] == zero)       # zero trits past the row stream
    assert np.all(rows[N:] == zero)                      # zero trits in padding rows
    assert np.array_equal(sc[:N], S.view(np.uint16))
    assert np.all(sc[N:] == 0)
    bgg.bgg_validate_packed(d, packed)
    # repacking the oracle's canonical bytes gives the same buffer
    assert np.array_equal(bgg.bgg_repack_canonical(d, canon, S), packed)


def test_pack_rejects_bad_trits_and_scales():
    d = bgg.bgg_describe("PQ2_0", 4, 128)
    T = np.zeros((4, 128), np.int8)
    S = np.full((4, 1), 0.01, np.float16)
    T[2, 7] = 2
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_pack_weights(d, T, S)
    assert e.value.status == 4 and "row 2 col 7" in str(e.value)
    T[2, 7] = -2
    with pytest.raises(bgg.BggError):
        bgg.bgg_pack_weights(d, T, S)
    # Q1_0 holds signs only: a zero weight is an error
    d1 = bgg.bgg_describe("Q1_0", 4, 128)
    T1 = np.ones((4, 128), np.int8)
    T1[3, 100] = 0
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_pack_weights(d1, T1, S)
    assert e.value.status == 4 and "row 3 col 100" in str(e.value)
    # Q2_0_G64 wants a scale per 64 weights
    d64 = bgg.bgg_describe("Q2_0_G64", 4, 128)
    with pytest.raises(ValueError):
        bgg.bgg_pack_weights(d64, T, S)
    T[2, 7] = 0
    for bad in (np.inf, -np.inf, np.nan):
        S2 = S.copy()
        S2[1, 0] = bad
        with pytest.raises(bgg.BggError) as e:
            bgg.bgg_pack_weights(d, T, S2)
        assert e.value.status == 9


@pytest.mark.parametrize("fmt", FMTS)
def test_validate_catches_bad_bytes(fmt):
    N, K = 70, 256
    d = bgg.bgg_describe(fmt, N, K)
    T = synth.weights(fmt, 9, 2, N, K)
    S = synth.scales_f16(9, 2, N, K, group=synth.scale_group(fmt))
    p = bgg.bgg_pack_weights(d, T, S)
    bgg.bgg_validate_packed(d, p)
    if fmt != "Q1_0":                  # (every Q1_0 byte is eight valid signs)
        bad = p.copy()
        bad[17] = 0xFF                 # a 2-bit code 3 / base-3 byte 255
        with pytest.raises(bgg.BggError) as e:
            bgg.bgg_validate_packed(d, bad)
        assert e.value.status == 5
        canon = oracle.pack(fmt, T)
        canon[3, 2] = 250 if fmt == "PTQ1_0" else 0xC0
        with pytest.raises(bgg.BggError) as e:
            bgg.bgg_repack_canonical(d, canon, S)
        assert e.value.status == 5
    # a padding row that holds anything but the zero byte is rejected
    rows_layout = p.copy()
    t_last, l_last = (N // 64), (N % 64)   # first padding row
    rows_layout[((t_last * d.chunks) * 64 + l_last) * 16] = 0x01 if fmt == "Q1_0" else 0
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_validate_packed(d, rows_layout)
    assert e.value.status == 5
    # and so is a non-zero scale of a padding row
    sc = p.copy()
    s16 = sc[d.scale_offset:d.scale_offset + d.scale_bytes].view(np.uint16)
    s16[(t_last * d.scales) * 64 + l_last] = 0x3C00
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_validate_packed(d, sc)
    assert e.value.status == 9


def test_descriptor_tampering_is_rejected():
    d = bgg.bgg_describe("PQ2_0", 64, 256)
    T = np.zeros((64, 256), np.int8)
    S = np.zeros((64, 2), np.float16)
    bgg.bgg_pack_weights(d, T, S)
    for field, val in (("magic", 1), ("version", 99), ("format", 2), ("N", 65), ("total_bytes", 5)):
        d2 = bgg.bgg_weights_desc.from_buffer_copy(d)
        setattr(d2, field, val)
        with pytest.raises(bgg.BggError) as e:
            bgg.bgg_pack_weights(d2, np.zeros((d2.N, d2.K), np.int8), np.zeros((d2.N, d2.groups), np.float16))
        assert e.value.status == 7
    # a PQ2_0 descriptor relabelled PTQ1_0 is caught before any work
    d3 = bgg.bgg_weights_desc.from_buffer_copy(d)
    d3.format = 2
    assert bgg.bgg_gemv_workspace_size(d3, 1) == 0


def test_workspace_sizes():
    d = bgg.bgg_describe("PQ2_0", 5120, 17408)
    assert bgg.bgg_gemv_workspace_size(d, 1) > 0
    assert bgg.bgg_gemv_workspace_size(d, 0) == 0
    assert bgg.bgg_gemv_workspace_size(d, 17) == 0
    assert bgg.bgg_gemv_workspace_size(d, 16) >= bgg.bgg_gemv_workspace_size(d, 4)
    assert bgg.bgg_gemm_workspace_size(d, 4096) >= 4096 * 17408 * 2


def test_null_pointers_are_errors_not_crashes():
    lib = ctypes.CDLL(bgg.LIB_PATH)
    lib.bgg_describe.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    assert lib.bgg_describe(1, 64, 128, None) == 1
    d = bgg.bgg_describe("PQ2_0", 64, 128)
    lib.bgg_pack_weights.argtypes = [ctypes.c_void_p] * 4
    assert lib.bgg_pack_weights(ctypes.addressof(d), None, None, None) == 1
    assert lib.bgg_pack_weights(None, None, None, None) == 1
    lib.bgg_ternary_gemv.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_uint32,
                                                             ctypes.c_void_p, ctypes.c_size_t,
                                                             ctypes.c_void_p]
    assert lib.bgg_ternary_gemv(ctypes.addressof(d), None, None, None, 1, 1, None, 0, None) == 1
    lib.bgg_hadamard_rotate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_void_p]
    assert lib.bgg_hadamard_rotate(None, None, 1, 128, None) == 1
    # shape errors are reported before any device work
    assert lib.bgg_hadamard_rotate(16, 16, 1, 100, None) == 3
    wsz = bgg.bgg_gemv_workspace_size(d, 16)
    assert lib.bgg_ternary_gemv(ctypes.addressof(d), 16, 16, 16, 0, 1, 16, wsz, None) == 3
    assert lib.bgg_ternary_gemv(ctypes.addressof(d), 16, 16, 16, 17, 1, 16, wsz, None) == 3
    assert lib.bgg_ternary_gemv(ctypes.addressof(d), 16, 16, 16, 1, 4, 16, wsz, None) == 3
    assert lib.bgg_ternary_gemv(ctypes.addressof(d), 16, 16, 16, 1, 1, 16, 8, None) == 6
    # the no-allocation variant: shape checks, its 32 MiB limit and NULL
    # buffers, all before any device work
    lib.bgg_ternary_gemv_noalloc.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_uint32,
                                                                     ctypes.c_void_p]
    assert lib.bgg_ternary_gemv_noalloc(None, 16, 16, 16, 1, 1, None) == 1
    assert lib.bgg_ternary_gemv_noalloc(ctypes.addressof(d), 16, 16, 16, 0, 1, None) == 3
    assert lib.bgg_ternary_gemv_noalloc(ctypes.addressof(d), 16, 16, 16, 17, 1, None) == 3
    assert lib.bgg_ternary_gemv_noalloc(ctypes.addressof(d), None, 16, 16, 1, 1, None) == 1
    big = bgg.bgg_describe("PQ2_0", 128, 516096)
    assert bgg.bgg_gemv_workspace_size(big, 16) > 32 << 20
    assert lib.bgg_ternary_gemv_noalloc(ctypes.addressof(big), 16, 16, 16, 16, 1, None) == 3
    lib.bgg_last_error.restype = ctypes.c_char_p
    assert b"static workspace" in lib.bgg_last_error()
    assert lib.bgg_ternary_gemv(ctypes.addressof(d), 17, 16, 16, 1, 1, 16, 1 << 20, None) == 6
    # the offline front end: NULL, shape and alignment errors before any work
    lib.bgg_rotate_ternarize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.bgg_rotate_ternarize(None, 4, 128, 16, 16, None) == 1
    assert lib.bgg_rotate_ternarize(16, 4, 100, 16, 16, None) == 3
    assert lib.bgg_rotate_ternarize(16, -1, 128, 16, 16, None) == 3
    assert lib.bgg_rotate_ternarize(24, 4, 128, 16, 16, None) == 6
    assert lib.bgg_rotate_ternarize(16, 4, 128, 12, 16, None) == 6
    assert lib.bgg_rotate_ternarize(16, 4, 128, 16, 17, None) == 6
    assert lib.bgg_rotate_ternarize(16, 0, 128, 16, 16, None) == 0   # N == 0: nothing to do
    dp = bgg.bgg_describe("Q1_0", 64, 128)   # no prompt-time kernel: rejected before any work
    lib.bgg_ternary_gemm.argtypes = lib.bgg_ternary_gemv.argtypes
    assert lib.bgg_ternary_gemm(ctypes.addressof(dp), 16, 16, 16, 4, 0, None, 0, None) == 2


def test_one_hip_runtime_in_the_process():
    """libbgg.so binds to the HIP runtime PyTorch loaded (two runtimes with
    one soname in one process break PyTorch's device calls)."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip


def _declarations_with_comments():
    """(function name, the comment block right above its declaration) for
    every function include/bgg.h declares."""
    text = open(HEADER).read()
    out = []
    for m in re.finditer(r"\n((?:bgg_status|size_t|const char\*|uint32_t)\s+(bgg_\w+)\()", text):
        before = text[:m.start() + 1]
        c1 = before.rfind("*/") + 2
        # only declarations (which may share one comment) between the last
        # comment and this declaration
        between = before[c1:].strip()
        assert all(ln.strip().endswith((",", ");", "(")) or ln.strip().startswith(("bgg_", "size_t", "void*",
                   "int", "const", "uint"))
                   for ln in between.splitlines() if ln.strip()), f"{m.group(2)}: no comment above it"
        out.append((m.group(2), before[before.rfind("/*", 0, c1):c1]))
    return out


def test_every_declaration_cites_a_passage_or_says_it_has_none():
    """Each exported call's comment cites the page passage it implements
    ([A ...], [B ...], [C ...]: the sources listed at the top of the
    header), or says that it is bookkeeping of the interface with no
    passage."""
    decls = _declarations_with_comments()
    assert set(bgg.EXPORTED) <= {name for name, _ in decls}
    for name, comment in decls:
        flat = " ".join(ln.strip().lstrip("/*").strip() for ln in comment.splitlines())
        cites = re.search(r"\[(A|B|C)[ \];]", flat) is not None
        none = "no page passage" in flat
        # (the no-allocation variant names the callers it is for instead)
        for_callers = name == "bgg_ternary_gemv_noalloc" and "cannot allocate" in flat
        assert cites or none or for_callers, name


def test_workspace_reset_argument_errors():
    lib = ctypes.CDLL(bgg.LIB_PATH)
    lib.bgg_gemv_workspace_reset.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert lib.bgg_gemv_workspace_reset(None, 256, None) == 1
    assert lib.bgg_gemv_workspace_reset(8, 256, None) == 6
    assert lib.bgg_gemv_workspace_reset(16, 100, None) == 6
    assert lib.bgg_gemv_workspace_reset(16, 0, None) == 0  # nothing to clear
