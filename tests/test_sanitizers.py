"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
library's host half (bgg_host.cpp: descriptors, the threaded packers, the
validators) and the CPU oracle (oracle.c), each rebuilt with
-fsanitize=address,undefined into a temporary directory, driven by a child
Python process with the sanitizer runtimes preloaded.  Any report fails the
test (UBSan is made fatal).  The device half is not instrumented here (GPU
sanitizers are not available for it).
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined"]

CHILD = textwrap.dedent(r'''
    import ctypes, sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle, synth

    # ---- the oracle, sanitized build
    oracle.swap_library(oracle.configure(ctypes.CDLL(ORACLE_SO)))
    rng = np.random.default_rng(1)
    for n in (1, 2, 4, 8, 16, 32, 64, 128):
        oracle.sylvester(n)
    for fmt in ("PQ2_0", "PTQ1_0", "Q1_0", "Q2_0_G64"):
        for N, K in ((1, 128), (3, 640), (7, 1152), (64, 5248)):
            T = synth.weights(fmt, 5, 1, N, K)
            S = synth.scales_f16(5, 1, N, K, group=synth.scale_group(fmt))
            P = oracle.pack(fmt, T)
            assert np.array_equal(oracle.unpack(fmt, P, K), T)
            x = synth.activations_f16(5, 2, 2, K)
            oracle.linear(fmt, P, S, x)
            oracle.linear(fmt, P, S, x, rotate=False)
    oracle.rotate(synth.activations_f16(5, 3, 3, 256))
    for v in (0.0, -0.0, 1e-8, 6e-8, 65504.0, 65520.0, 1e9, float("inf"), float("-inf"), float("nan")):
        oracle.f64_to_f16(v)
    oracle.ternarize(synth.float_weights(5, 4, 8, 256))

    # ---- the host half of the library, sanitized build
    lib = ctypes.CDLL(HOST_SO)
    class Desc(ctypes.Structure):
        _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                    ("format", ctypes.c_int32), ("row_tile", ctypes.c_int32),
                    ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("groups", ctypes.c_int64),
                    ("row_tiles", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                    ("chunks", ctypes.c_int64), ("trit_bytes", ctypes.c_uint64),
                    ("scale_offset", ctypes.c_uint64), ("scale_bytes", ctypes.c_uint64),
                    ("total_bytes", ctypes.c_uint64), ("format_bytes", ctypes.c_uint64),
                    ("scale_group", ctypes.c_int64), ("scales", ctypes.c_int64)]
    vp = ctypes.c_void_p
    lib.bgg_describe.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, vp]
    lib.bgg_pack_weights.argtypes = [vp] * 4
    lib.bgg_repack_canonical.argtypes = [vp] * 4
    lib.bgg_validate_packed.argtypes = [vp, vp]
    lib.bgg_status_string.restype = ctypes.c_char_p
    lib.bgg_last_error.restype = ctypes.c_char_p
    d = Desc()
    for fmt in range(0, 6):
        for N, K in ((0, 128), (1, 100), (-1, 128), (5, 0), (64, 128)):
            lib.bgg_describe(fmt, N, K, ctypes.byref(d))
            lib.bgg_last_error()
    for s in range(-1, 12):
        lib.bgg_status_string(s)
    names = {1: "PQ2_0", 2: "PTQ1_0", 3: "Q1_0", 4: "Q2_0_G64"}
    for fmt, name in names.items():
        # the second shape is large enough for the threaded packer
        for N, K in ((70, 640), (8192, 4096)):
            assert lib.bgg_describe(fmt, N, K, ctypes.byref(d)) == 0
            T = np.ascontiguousarray(synth.weights(name, 6, 1, N, K))
            S = np.ascontiguousarray(synth.scales_f16(6, 1, N, K, group=synth.scale_group(name)).view(np.uint16))
            buf = np.zeros(d.total_bytes, np.uint8)
            assert lib.bgg_pack_weights(ctypes.byref(d), T.ctypes.data, S.ctypes.data, buf.ctypes.data) == 0
            assert lib.bgg_validate_packed(ctypes.byref(d), buf.ctypes.data) == 0
            canon = np.ascontiguousarray(oracle.pack(name, T))
            buf2 = np.zeros(d.total_bytes, np.uint8)
            assert lib.bgg_repack_canonical(ctypes.byref(d), canon.ctypes.data, S.ctypes.data,
                                            buf2.ctypes.data) == 0
            assert np.array_equal(buf, buf2)
            bad = buf.copy()
            bad[0] = 0xFF
            lib.bgg_validate_packed(ctypes.byref(d), bad.ctypes.data)
            T2 = T.copy()
            T2[N // 2, K // 2] = 2
            assert lib.bgg_pack_weights(ctypes.byref(d), T2.ctypes.data, S.ctypes.data, buf.ctypes.data) != 0
    print("sanitized run done")
''')


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_host_code_and_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    host_so = str(tmp_path / "libbgg_host_san.so")
    oracle_so = str(tmp_path / "_oracle_san.so")
    csrc = os.path.join(ROOT, "bit_gemv_gemm_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-shared", "-fPIC", "-o", host_so,
                           os.path.join(csrc, "bgg_host.cpp"), "-lpthread"])
    subprocess.check_call(["gcc", *SAN, "-fopenmp", "-shared", "-fPIC", "-o", oracle_so,
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    script = tmp_path / "child.py"
    script.write_text(f"ROOT = {ROOT!r}\nHOST_SO = {host_so!r}\nORACLE_SO = {oracle_so!r}\n" + CHILD)
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    res = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True, timeout=600)
    report = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert "sanitized run done" in res.stdout


def test_the_harness_catches_a_planted_overflow(tmp_path):
    """Negative control: a one-byte heap overflow in a throwaway library,
    run the same way, must be reported (so a clean run above means something)."""
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    src = tmp_path / "bad.c"
    src.write_text("#include <stdlib.h>\nint bad(void) { char* p = malloc(8); p[8] = 1; int r = p[0]; free(p); return r; }\n")
    so = str(tmp_path / "libbad.so")
    subprocess.check_call(["gcc", *SAN, "-shared", "-fPIC", "-o", so, str(src)])
    code = f"import ctypes; ctypes.CDLL({so!r}).bad(); print('not caught')"
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode != 0 and "not caught" not in res.stdout
    assert "heap-buffer-overflow" in res.stderr or "runtime error" in res.stderr
