"""Pins of the CPU oracle to things other than itself.

Each pin_* function checks the oracle against something the pages or the
mathematics fix: closed forms, a library routine (scipy, numpy), brute force on
tiny inputs, or a number printed on the pages (tests/golden/page_numbers.json).
test_planted_mistakes_are_caught builds copies of oracle.c with one plausible
mistake each and checks that at least one pin fails for every copy.
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest
import scipy.linalg

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))
RNG = np.random.default_rng(12345)
FMTS = ("PQ2_0", "PTQ1_0")


def _hhat_blockdiag(K):
    """blockdiag(H_128/sqrt(128)) from scipy's Hadamard routine."""
    h = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128.0)
    return scipy.linalg.block_diag(*([h] * (K // 128)))


def _rand_f16(shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float16)


def _rand_trits(n, k):
    return RNG.integers(-1, 2, size=(n, k), dtype=np.int8)


def _rand_scales(n, k):
    return RNG.uniform(0.005, 0.05, size=(n, k // 128)).astype(np.float16)


# --------------------------------------------------------------------------
# fp16 decoding
# --------------------------------------------------------------------------
def pin_f16_decode():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(b) for b in bits[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xFBFF, 0x7C00, 0xFC00):
        assert oracle.f16_to_f64(b) == float(np.uint16(b).view(np.float16))


# --------------------------------------------------------------------------
# Hadamard matrix and rotation
# --------------------------------------------------------------------------
def pin_sylvester_orthogonal():
    for n in (1, 2, 4, 8, 16, 32, 64, 128):
        H = oracle.sylvester(n)
        assert set(np.unique(H)) <= {-1.0, 1.0}
        assert np.array_equal(H @ H.T, n * np.eye(n))


def pin_sylvester_walsh_closed_form():
    # natural (Sylvester) order: H[i][j] = (-1)^popcount(i & j)
    for n in (2, 16, 128):
        H = oracle.sylvester(n)
        i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
        pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
        assert np.array_equal(H, np.where(pc % 2 == 0, 1.0, -1.0))


def pin_sylvester_library():
    for n in (1, 4, 32, 128):
        assert np.array_equal(oracle.sylvester(n), scipy.linalg.hadamard(n).astype(np.float64))


def pin_rotate_basis_vectors():
    K = 384
    for b in range(K // 128):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, 128 * b] = 1.0
        xr = oracle.rotate(x)[0]
        want = np.zeros(K)
        want[128 * b:128 * b + 128] = 1.0 / math.sqrt(128.0)
        assert np.allclose(xr, want, rtol=0, atol=1e-15)
        x = np.zeros((1, K), dtype=np.float16)
        x[0, 128 * b:128 * b + 128] = 1.0
        xr = oracle.rotate(x)[0]
        want = np.zeros(K)
        want[128 * b] = math.sqrt(128.0)
        assert np.allclose(xr, want, rtol=0, atol=1e-13)


def pin_rotate_library_and_parseval():
    M, K = 3, 640
    x = _rand_f16((M, K))
    xr = oracle.rotate(x)
    want = x.astype(np.float64) @ _hhat_blockdiag(K).T
    assert np.allclose(xr, want, rtol=1e-13, atol=1e-13)
    # orthogonal blocks preserve each block's norm, and applying the
    # transform again gives back x
    for b in range(K // 128):
        s = slice(128 * b, 128 * b + 128)
        assert np.allclose(np.linalg.norm(xr[:, s], axis=1),
                           np.linalg.norm(x[:, s].astype(np.float64), axis=1), rtol=1e-13)
    assert np.allclose(xr @ _hhat_blockdiag(K).T, x.astype(np.float64), rtol=1e-12, atol=1e-12)


def pin_rotation_identity_real_w():
    # W x = (W Hhat^T)(Hhat x): a real matrix stored in rotated coordinates
    N, K = 8, 256
    W = RNG.standard_normal((N, K))
    x = _rand_f16((2, K))
    y_direct = x.astype(np.float64) @ W.T
    W_stored = W @ _hhat_blockdiag(K).T
    y_rot = oracle.rotate(x) @ W_stored.T
    assert np.allclose(y_rot, y_direct, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# packings
# --------------------------------------------------------------------------
def _all_tuples(width):
    vals = np.array(np.meshgrid(*([[-1, 0, 1]] * width), indexing="ij")).reshape(width, -1).T
    return vals.astype(np.int8)


def pin_ptq1_exhaustive():
    T = _all_tuples(5)                     # 243 rows of 5 trits
    P = oracle.pack("PTQ1_0", T)           # one byte per row
    assert P.shape == (243, 1)
    assert sorted(P[:, 0].tolist()) == list(range(243))   # a bijection onto 0..242
    assert np.array_equal(oracle.unpack("PTQ1_0", P, 5), T)
    # special rows: all zero trits -> every digit 1, all +1 -> 242, all -1 -> 0
    assert oracle.pack("PTQ1_0", np.zeros((1, 5), np.int8))[0, 0] == 1 + 3 + 9 + 27 + 81
    assert oracle.pack("PTQ1_0", np.ones((1, 5), np.int8))[0, 0] == 242
    assert oracle.pack("PTQ1_0", -np.ones((1, 5), np.int8))[0, 0] == 0
    # one non-zero trit at position i gives digit 2 (t=+1) or 0 (t=-1) at 3^i
    for i in range(5):
        t = np.zeros((1, 5), np.int8)
        t[0, i] = 1
        assert oracle.pack("PTQ1_0", t)[0, 0] == 121 + 3 ** i
        t[0, i] = -1
        assert oracle.pack("PTQ1_0", t)[0, 0] == 121 - 3 ** i
    for bad in range(243, 256):
        with pytest.raises(oracle.OracleError):
            oracle.unpack("PTQ1_0", np.array([[bad]], np.uint8), 5)


def pin_pq2_exhaustive():
    T = _all_tuples(4)
    P = oracle.pack("PQ2_0", T)
    assert P.shape == (81, 1)
    assert len(set(P[:, 0].tolist())) == 81
    assert all(((b >> (2 * i)) & 3) != 3 for b in P[:, 0].tolist() for i in range(4))
    assert np.array_equal(oracle.unpack("PQ2_0", P, 4), T)
    assert oracle.pack("PQ2_0", np.zeros((1, 4), np.int8))[0, 0] == 0x55
    assert oracle.pack("PQ2_0", np.ones((1, 4), np.int8))[0, 0] == 0xAA
    assert oracle.pack("PQ2_0", -np.ones((1, 4), np.int8))[0, 0] == 0x00
    for i in range(4):
        t = np.zeros((1, 4), np.int8)
        t[0, i] = 1
        assert oracle.pack("PQ2_0", t)[0, 0] == 0x55 + (1 << (2 * i))
    for bad in (0x03, 0x0C, 0x30, 0xC0, 0xFF):
        with pytest.raises(oracle.OracleError):
            oracle.unpack("PQ2_0", np.array([[bad]], np.uint8), 4)


def pin_pack_roundtrip_ragged():
    for K in (1, 2, 3, 4, 5, 6, 7, 9, 129, 640, 643):
        T = _rand_trits(5, K)
        for fmt in FMTS:
            P = oracle.pack(fmt, T)
            assert P.shape[1] == (math.ceil(K / 4) if fmt == "PQ2_0" else math.ceil(K / 5))
            assert np.array_equal(oracle.unpack(fmt, P, K), T)
    # padding trits past K are t = 0 (digit / code 1)
    P = oracle.pack("PTQ1_0", np.ones((1, 6), np.int8))
    assert P[0, 1] == 2 + 1 * (3 + 9 + 27 + 81)
    P = oracle.pack("PQ2_0", np.ones((1, 5), np.int8))
    assert P[0, 1] == 2 + (0x55 & ~3)


def pin_bits_per_weight():
    g = GOLDEN
    # PQ2_0: 2 bits per trit + 16 bits per 128 weights, exactly
    for K in (128, 512, 5120, 6144, 17408):
        assert oracle.bits_per_weight("PQ2_0", 64, K) == 2.0 + 16.0 / 128.0
    v = oracle.bits_per_weight("PQ2_0", 64, 5120)
    assert abs(v - g["pq2_0_bits_per_weight"]["value"]) <= 0.5 * 10 ** -g["pq2_0_bits_per_weight"]["printed_decimals"]
    # PTQ1_0 row stream: 8/5 bits per trit + 16/128 = 1.725 when 5 divides K
    v = oracle.bits_per_weight("PTQ1_0", 64, 5120)
    assert v == g["bits_per_trit_five_per_byte"]["value"] + 16.0 / 128.0 == 1.725
    p = g["ternary_bits_per_weight_method_paragraph"]
    assert abs(v - p["value"]) <= 0.5 * 10 ** -p["printed_decimals"] + 1e-12
    for K in (512, 6144, 17408):
        assert oracle.bits_per_weight("PTQ1_0", 64, K) == 8.0 * (math.ceil(K / 5) + K / 64) / K
    # scale overhead = 16 bits per 128 weights, the same overhead that makes
    # the 1-bit sister format 1 + 16/128 = 1.125 bits per weight
    N, K = 64, 5120
    scale_bits = 8.0 * (oracle.format_bytes("PQ2_0", N, K) - N * oracle.row_bytes("PQ2_0", K)) / (N * K)
    assert 1.0 + scale_bits == GOLDEN["one_bit_bits_per_weight"]["value"]
    # the printed PTQ1_0 figure 1.75 is what padding every 128-trit group to
    # whole bytes would give (26 bytes + 2): a reading not taken; the row
    # stream stays strictly below it
    assert 8.0 * (math.ceil(128 / 5) + 2) / 128 == g["ptq1_0_bits_per_weight_packing_paragraph"]["value"]
    assert oracle.bits_per_weight("PTQ1_0", 64, 5120) < 1.75


# --------------------------------------------------------------------------
# products
# --------------------------------------------------------------------------
def pin_matvec_bruteforce():
    M, N, K = 2, 3, 256
    T = _rand_trits(N, K)
    S = _rand_scales(N, K)
    xr = RNG.standard_normal((M, K))
    y = oracle.matvec(T, S, xr)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(S[n, k // 128]) * int(T[n, k]) * xr[m, k]
            assert abs(y[m, n] - acc) <= 1e-12 * (1 + abs(acc))


def pin_matvec_special_cases():
    N, K = 4, 384
    S = _rand_scales(N, K)
    assert np.array_equal(oracle.matvec(np.zeros((N, K), np.int8), S, RNG.standard_normal((2, K))),
                          np.zeros((2, N)))
    T = _rand_trits(N, K)
    for k in (0, 127, 128, 383):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        y = oracle.matvec(T, S, e)[0]
        assert np.array_equal(y, S[:, k // 128].astype(np.float64) * T[:, k])


def pin_linear_model_coordinates():
    # the stored trits are S*T in rotated coordinates; in model coordinates the
    # weight matrix is (S*T) blockdiag(Hhat), and the layer must equal it
    for fmt in FMTS:
        for (M, N, K) in ((1, 5, 128), (3, 7, 640)):
            T = _rand_trits(N, K)
            S = _rand_scales(N, K)
            x = _rand_f16((M, K))
            Wst = S.astype(np.float64).repeat(128, axis=1) * T
            want = x.astype(np.float64) @ (Wst @ _hhat_blockdiag(K)).T
            got = oracle.linear(fmt, oracle.pack(fmt, T), S, x)
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
            # without the rotation the stored weights act on x directly
            got = oracle.linear(fmt, oracle.pack(fmt, T), S, x, rotate=False)
            assert np.allclose(got, x.astype(np.float64) @ Wst.T, rtol=1e-12, atol=1e-12)


def pin_sylvester_row_closed_form():
    # a trit row equal to Sylvester row r in block b picks out sqrt(128) x[128b + r]
    K = 512
    H = scipy.linalg.hadamard(128).astype(np.int8)
    x = _rand_f16((2, K))
    cases = [(0, 0), (1, 5), (2, 127), (3, 64)]
    T = np.zeros((len(cases), K), np.int8)
    S = np.zeros((len(cases), K // 128), np.float16)
    for n, (b, r) in enumerate(cases):
        T[n, 128 * b:128 * b + 128] = H[r]
        S[n, b] = np.float16(0.03125 * (n + 1))
    for fmt in FMTS:
        y = oracle.linear(fmt, oracle.pack(fmt, T), S, x)
        for n, (b, r) in enumerate(cases):
            want = float(S[n, b]) * math.sqrt(128.0) * float(x[0, 128 * b + r])
            assert abs(y[0, n] - want) <= 1e-12 * (1 + abs(want))


# --------------------------------------------------------------------------
# sister formats: Q1_0 (one sign bit per weight, a scale per 128) and
# Q2_0_g64 (the PQ2_0 stream, a scale per 64)
# --------------------------------------------------------------------------
def _rand_signs(n, k):
    return RNG.choice(np.array([-1, 1], np.int8), size=(n, k))


def pin_q1_exhaustive():
    vals = np.array(np.meshgrid(*([[-1, 1]] * 8), indexing="ij")).reshape(8, -1).T.astype(np.int8)
    P = oracle.pack("Q1_0", vals)              # one byte per row of 8 signs
    assert P.shape == (256, 1)
    assert sorted(P[:, 0].tolist()) == list(range(256))   # a bijection onto 0..255
    assert np.array_equal(oracle.unpack("Q1_0", P, 8), vals)
    assert oracle.pack("Q1_0", np.ones((1, 8), np.int8))[0, 0] == 0xFF
    assert oracle.pack("Q1_0", -np.ones((1, 8), np.int8))[0, 0] == 0x00
    for i in range(8):                         # weight i is bit i, 1 for +1
        t = -np.ones((1, 8), np.int8)
        t[0, i] = 1
        assert oracle.pack("Q1_0", t)[0, 0] == 1 << i
    with pytest.raises(oracle.OracleError):    # no zero weight in a 1-bit format
        oracle.pack("Q1_0", np.zeros((1, 8), np.int8))


def pin_sister_formats_sizes_and_streams():
    for K in (128, 5120, 17408):
        # 1 + 16/128: the effective bits per weight printed for 1-bit Bonsai
        assert oracle.bits_per_weight("Q1_0", 64, K) == GOLDEN["one_bit_bits_per_weight"]["value"]
        assert oracle.bits_per_weight("Q2_0_G64", 64, K) == 2.0 + 16.0 / 64.0
    assert oracle.scale_group("Q1_0") == 128 and oracle.scale_group("Q2_0_G64") == 64
    assert oracle.scale_group("PQ2_0") == GOLDEN["group"]["value"]
    T = _rand_trits(4, 640)
    assert np.array_equal(oracle.pack("Q2_0_G64", T), oracle.pack("PQ2_0", T))
    assert np.array_equal(oracle.unpack("Q2_0_G64", oracle.pack("PQ2_0", T), 640), T)
    for K in (1, 7, 8, 9, 129, 640):
        T = _rand_signs(3, K)
        P = oracle.pack("Q1_0", T)
        assert P.shape[1] == math.ceil(K / 8)
        assert np.array_equal(oracle.unpack("Q1_0", P, K), T)


def pin_matvec_group64():
    M, N, K = 2, 3, 256
    T = _rand_trits(N, K)
    S = RNG.uniform(0.005, 0.05, size=(N, K // 64)).astype(np.float16)
    xr = RNG.standard_normal((M, K))
    y = oracle.matvec(T, S, xr)
    for m in range(M):
        for n in range(N):
            acc = sum(float(S[n, k // 64]) * int(T[n, k]) * xr[m, k] for k in range(K))
            assert abs(y[m, n] - acc) <= 1e-12 * (1 + abs(acc))
    for k in (0, 63, 64, 127, 128, 255):       # a basis vector picks its 64-group's scale
        e = np.zeros((1, K))
        e[0, k] = 1.0
        assert np.array_equal(oracle.matvec(T, S, e)[0], S[:, k // 64].astype(np.float64) * T[:, k])


def pin_linear_sister_formats():
    for fmt, group in (("Q1_0", 128), ("Q2_0_G64", 64)):
        for (M, N, K) in ((1, 5, 128), (3, 7, 640)):
            T = _rand_signs(N, K) if fmt == "Q1_0" else _rand_trits(N, K)
            S = RNG.uniform(0.005, 0.05, size=(N, K // group)).astype(np.float16)
            x = _rand_f16((M, K))
            Wst = S.astype(np.float64).repeat(group, axis=1) * T
            want = x.astype(np.float64) @ (Wst @ _hhat_blockdiag(K)).T
            got = oracle.linear(fmt, oracle.pack(fmt, T), S, x)
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# offline front end: fp16 rounding and rotate-then-ternarize
# --------------------------------------------------------------------------
def pin_f64_to_f16_matches_numpy():
    """One round-to-nearest-even conversion, as numpy's double -> half."""
    vals = [0.0, -0.0, 1.0, -2.5, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -14,
            2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -25 * 1.0000001, 6.1e-5, 1e-9,
            0.1, 1.0 / 3.0, np.inf, -np.inf]
    # exact ties between neighbouring halves, both parities, normal and subnormal
    for h in (0x3C00, 0x3C01, 0x0001, 0x0002, 0x03FF, 0x0400, 0x7BFE, 0x1234, 0x5555):
        a = float(np.array([h], np.uint16).view(np.float16)[0])
        b = float(np.array([h + 1], np.uint16).view(np.float16)[0])
        vals += [(a + b) / 2, -(a + b) / 2, np.nextafter((a + b) / 2, 0), np.nextafter((a + b) / 2, 1e9)]
    vals += list(RNG.standard_normal(2000) * 10.0 ** RNG.uniform(-9, 5, 2000))
    for v in vals:
        want = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        assert oracle.f64_to_f16(v) == want, (v, hex(want))


def _rotate_rows_f64(W):
    """W blockdiag(H_128/sqrt(128)) by scipy's Hadamard routine."""
    return np.asarray(W, np.float64) @ _hhat_blockdiag(W.shape[1])


def pin_ternarize_brute_force():
    """Small random inputs: the scale is numpy's fp16 of the mean rotated
    magnitude, and each trit is the candidate of {-1, 0, 1} whose multiple
    of the scale lies nearest to the rotated weight (found by trying all)."""
    for (N, K) in ((3, 128), (5, 384)):
        W = (RNG.standard_normal((N, K)) * 0.02).astype(np.float32)
        T, S = oracle.ternarize(W)
        Wr = _rotate_rows_f64(W)
        for n in range(N):
            for g in range(K // 128):
                blk = Wr[n, 128 * g:128 * g + 128]
                s = np.float16(np.mean(np.abs(blk)))
                assert S[n, g].view(np.uint16) == s.view(np.uint16)
                cand = np.array([-1, 0, 1])
                err = np.abs(blk[:, None] - cand[None, :] * float(s))
                assert np.array_equal(T[n, 128 * g:128 * g + 128], cand[np.argmin(err, axis=1)])


def pin_ternarize_sylvester_rows_and_zeros():
    """A block equal to c times Sylvester row r rotates to c sqrt(128) e_r:
    one trit sign(c) at r, scale fp16(|c| / sqrt(128)); a zero block gives
    zero trits and a zero scale; a constant block is Sylvester row 0."""
    import scipy.linalg
    H = scipy.linalg.hadamard(128)
    K = 512
    cases = [(0, 0, 0.25), (1, 77, -1.5), (2, 127, 3.0), (3, 5, 0.0078125)]
    W = np.zeros((len(cases) + 1, K), np.float32)
    for n, (b, r, c) in enumerate(cases):
        W[n, 128 * b:128 * b + 128] = (c * math.sqrt(128.0)) * H[r]
    W[len(cases), 128:256] = 0.75                       # constant block
    T, S = oracle.ternarize(W)
    for n, (b, r, c) in enumerate(cases):
        want = np.zeros(K, np.int8)
        want[128 * b + r] = 1 if c > 0 else -1
        assert np.array_equal(T[n], want)
        assert S[n, b] == np.float16(abs(c)) and np.all(S[n, np.arange(4) != b] == 0)
    want = np.zeros(K, np.int8)
    want[128] = 1
    assert np.array_equal(T[len(cases)], want)
    assert S[len(cases), 1] == np.float16(0.75 * 128 / math.sqrt(128.0) / 128)
    Tz, Sz = oracle.ternarize(np.zeros((2, 256), np.float32))
    assert not Tz.any() and not Sz.view(np.uint16).any()


def pin_ternarize_rotation_spreads_outliers():
    """The pages' reason for rotating first: with a few large outliers per
    row, ternary rounding after the rotation loses less than rounding the
    weights as they are (same scale rule).  Feeding W Hn to the front end
    makes it round W itself, since Hn Hn = I."""
    N, K = 64, 1024
    W = RNG.standard_normal((N, K)) * 0.02
    idx = RNG.random((N, K)) < 0.004
    W[idx] *= 40.0
    W = W.astype(np.float32)
    T1, S1 = oracle.ternarize(W)
    rec_rot = (T1 * S1.astype(np.float64).repeat(128, axis=1)) @ _hhat_blockdiag(K)
    V = _rotate_rows_f64(W).astype(np.float32)
    T2, S2 = oracle.ternarize(V)
    rec_direct = T2 * S2.astype(np.float64).repeat(128, axis=1)
    err_rot = np.linalg.norm(W - rec_rot) / np.linalg.norm(W)
    err_direct = np.linalg.norm(W - rec_direct) / np.linalg.norm(W)
    assert err_rot < 0.8 * err_direct, (err_rot, err_direct)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes: every mutant of oracle.c must fail at least one pin
# --------------------------------------------------------------------------
MUTANTS = {
    "sylvester_sign": ("H[(i + m) * n + (j + m)] = -h;", "H[(i + m) * n + (j + m)] = h;"),
    "rotate_no_norm": ("xr[m * K + b * BLOCK + r] = acc * norm;", "xr[m * K + b * BLOCK + r] = acc;"),
    "rotate_block_offset": ("blk[i] = oracle_f16_to_f64(x[m * K + b * BLOCK + i]);",
                            "blk[i] = oracle_f16_to_f64(x[m * K + b + i]);"),
    "scale_index": ("S[n * G + k / group]", "S[n * G + k % G]"),
    "dropped_scale": ("acc += oracle_f16_to_f64(S[n * G + k / group]) * (double)T[n * K + k] * xr[m * K + k];",
                      "acc += (double)T[n * K + k] * xr[m * K + k];"),
    "q1_bit_order": ("if (t == 1) byte |= 1u << i;", "if (t == 1) byte |= 0x80u >> i;"),
    "q1_sign": ("T[n * K + k] = (int8_t)(((byte >> i) & 1u) ? 1 : -1);",
                "T[n * K + k] = (int8_t)(((byte >> i) & 1u) ? -1 : 1);"),
    "group64_scale": ("if (fmt == ORACLE_Q2_0_G64) return 64;", "if (fmt == ORACLE_Q2_0_G64) return 128;"),
    "pq2_code_sign": ("T[n * K + k] = (int8_t)((int)code - 1);", "T[n * K + k] = (int8_t)(1 - (int)code);"),
    "pq2_slot_shift": ("byte |= (unsigned)(t + 1) << (2 * i);", "byte |= (unsigned)(t + 1) << i;"),
    "ptq1_digit_order": ("int64_t k = 5 * j + i;\n          if (k < K) T[n * K + k] = (int8_t)((int)digit - 1);",
                         "int64_t k = 5 * j + (4 - i);\n          if (k < K) T[n * K + k] = (int8_t)((int)digit - 1);"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "transposed_x": ("* xr[m * K + k];", "* xr[k * M + m];"),
    "f16_ties_to_odd": ("fmod(m, 2.0) == 1.0", "fmod(m, 2.0) == 0.0"),
    "f16_subnormal_step": ("if (q < -24) q = -24;", "if (q < -25) q = -25;"),
    "f16_exponent_field": ("int ef = q + 25;", "int ef = q + 24;"),
    "ternarize_threshold": ("if (fabs(wr[r]) > 0.5 * s)", "if (fabs(wr[r]) > s)"),
    "ternarize_scale_mean": ("oracle_f64_to_f16(mag / BLOCK)", "oracle_f64_to_f16(mag / K)"),
    "ternarize_rotation_norm": ("wr[r] = acc * norm;", "wr[r] = acc;"),
    "ternarize_no_rotation": ("acc += H[r * BLOCK + i] * blk[i];\n        wr[r]",
                              "acc += (r == i) * blk[i];\n        wr[r]"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"oracle_{name}.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(path), "-lm"])
    return oracle.configure(ctypes.CDLL(str(so)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    prev = oracle.swap_library(lib)
    failed = []
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, oracle.OracleError, ValueError):
                failed.append(pin.__name__)
    finally:
        oracle.swap_library(prev)
    assert failed, f"no pin caught the planted mistake {name}"
