"""GPU parity: the HIP path through the C ABI against the CPU oracle, on
seeded synthetic inputs.  Marked gpu; run on an MI355X.

Bars: unpacking bit-exact; the transform within one fp16 ulp of the rounded
fp64 result; y within 2e-3 of the oracle, measured per token row as
max_n |y - y_oracle| / max_n |y_oracle|.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_helpers import TOL, Dev, gen_matrix, oracle_y, relerr  # noqa: E402

FMTS = ("PQ2_0", "PTQ1_0")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import bit_gemv_gemm_amd as bgg
    return bgg, torch


# ---------------------------------------------------------------------------
# unpack: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 128), (100, 640), (130, 1152), (256, 512), (64, 6144), (5120, 17408)])
def test_unpack_bit_exact(env, fmt, N, K):
    bgg, torch = env
    say(f"unpack {fmt} N={N} K={K}")
    T, S = gen_matrix(11, 3, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    td = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sd = torch.empty((N, K // 128), dtype=torch.float16, device="cuda")
    bgg.bgg_unpack_weights(d.desc, d.packed, td, sd)
    torch.cuda.synchronize()
    want = oracle.unpack(fmt, oracle.pack(fmt, T), K)
    assert np.array_equal(td.cpu().numpy(), want)
    assert np.array_equal(sd.cpu().numpy().view(np.uint16), S.view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS)
def test_unpack_exhaustive_codes(env, fmt):
    """Every valid byte value appears: all 243 base-3 bytes / all 81 code
    bytes, laid out by the oracle's canonical packer."""
    bgg, torch = env
    say(f"unpack exhaustive {fmt}")
    width = 5 if fmt == "PTQ1_0" else 4
    vals = np.array(np.meshgrid(*([[-1, 0, 1]] * width), indexing="ij")).reshape(width, -1).T
    reps = -(-640 // (vals.shape[0] * width)) + 1
    row = np.tile(vals.reshape(-1), reps)[:640].astype(np.int8)
    T = np.stack([np.roll(row, 7 * i) for i in range(70)])
    S = synth.scales_f16(1, 1, 70, 640)
    d = Dev(bgg, torch, fmt, T, S)
    td = torch.empty(T.shape, dtype=torch.int8, device="cuda")
    sd = torch.empty(S.shape, dtype=torch.float16, device="cuda")
    bgg.bgg_unpack_weights(d.desc, d.packed, td, sd)
    torch.cuda.synchronize()
    assert np.array_equal(td.cpu().numpy(), T)


# ---------------------------------------------------------------------------
# Hadamard transform
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K", [(1, 128), (3, 640), (17, 5120), (5, 17408), (300, 1024)])
def test_hadamard_rotate_within_one_ulp(env, M, K):
    bgg, torch = env
    say(f"rotate M={M} K={K}")
    x = synth.activations_f16(5, K, M, K)
    xd = torch.from_numpy(x).cuda()
    yd = torch.empty_like(xd)
    bgg.bgg_hadamard_rotate(xd, yd, M, K)
    torch.cuda.synchronize()
    got = yd.cpu().numpy()
    want = oracle.rotate(x)
    want16 = want.astype(np.float16)
    # one fp16 ulp of the correctly rounded value
    ulp = np.spacing(np.abs(want16)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - want16.astype(np.float64)) <= ulp)
    assert np.mean(got == want16) > 0.95
    # in place
    bgg.bgg_hadamard_rotate(xd, xd, M, K)
    torch.cuda.synchronize()
    assert np.array_equal(xd.cpu().numpy(), got)


def test_hadamard_closed_forms(env):
    bgg, torch = env
    say("rotate closed forms")
    K = 256
    x = np.zeros((2, K), np.float16)
    x[0, 0] = 1.0
    x[1, 128:] = 1.0
    xd = torch.from_numpy(x).cuda()
    bgg.bgg_hadamard_rotate(xd, xd, 2, K)
    torch.cuda.synchronize()
    y = xd.cpu().numpy().astype(np.float64)
    assert np.all(y[0, :128] == np.float16(1 / np.sqrt(128)))
    assert np.all(y[0, 128:] == 0)
    assert y[1, 128] == np.float16(np.sqrt(128)) and np.all(y[1, 129:] == 0) and np.all(y[1, :128] == 0)


# ---------------------------------------------------------------------------
# decode GEMV
# ---------------------------------------------------------------------------
GEMV_CASES = [
    ("tiny", 256, 512, 1),
    ("ragged", 100, 640, 1),
    ("tail-periods", 130, 1152, 2),
    ("one-group", 64, 128, 1),
    ("one-row", 1, 384, 1),
    ("q", 6144, 5120, 1),
    ("o", 5120, 6144, 1),
    ("kv", 1024, 5120, 3),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case,N,K,M", GEMV_CASES)
def test_gemv_parity(env, fmt, case, N, K, M):
    bgg, torch = env
    say(f"gemv {fmt} {case} N={N} K={K} M={M}")
    T, S = gen_matrix(21, 4, N, K)
    x = synth.activations_f16(21, 100 + K, M, K)
    d = Dev(bgg, torch, fmt, T, S)
    y = d.gemv(x)
    assert not np.isnan(y).any()
    ref = oracle_y(fmt, T, S, x)
    e = relerr(y, ref)
    say(f"  rel err {e}")
    assert np.all(e <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13, 16])
def test_gemv_token_counts(env, fmt, M):
    bgg, torch = env
    N, K = 200, 1280
    say(f"gemv {fmt} M={M} N={N} K={K}")
    T, S = gen_matrix(31, 5, N, K)
    x = synth.activations_f16(31, 7, M, K)
    y = Dev(bgg, torch, fmt, T, S).gemv(x)
    ref = oracle_y(fmt, T, S, x)
    e = relerr(y, ref)
    say(f"  rel err {e.max():.3g}")
    assert np.all(e <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_gemv_projection_full_size(env, fmt, name):
    """The single-projection workload at its full shape, every output checked."""
    bgg, torch = env
    w = synth.WORKLOADS["projection"]
    mat = [m for m in w["matrices"] if m.name == name][0]
    say(f"gemv full {fmt} {name} N={mat.n} K={mat.k}")
    T, S = synth.workload_matrix(mat, w["seed"])
    x = synth.workload_x(w["seed"], 1, mat.k)
    y = Dev(bgg, torch, fmt, T, S).gemv(x)
    ref = oracle_y(fmt, T, S, x)
    e = relerr(y, ref)
    say(f"  rel err {e}")
    assert np.all(e <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408), (300, 640), (100, 1152), (64, 128)])
def test_gemv_one_launch_and_two_step(env, fmt, N, K):
    """For one token bgg_ternary_gemv runs a single kernel that also encodes
    x; bgg_gemv_prepare + bgg_gemv_run is the two-step form.  Call after call
    on one workspace with a different x each time (no call may read another
    call's encoded activations or row sums), with and without the transform:
    both forms agree with the oracle (every row where the oracle is cheap,
    else 48 sampled rows), each form gives the same bits when repeated, and
    where both forms run the same kernels (PTQ1_0) their bits agree."""
    bgg, torch = env
    say(f"gemv one-launch and two-step {fmt} {N}x{K}")
    T, S = gen_matrix(71, 9, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 1))
    rows = np.arange(N) if N * K <= 1 << 20 else np.random.default_rng(7).choice(N, 48, replace=False)
    for i in range(4):
        flags = bgg.BGG_ROTATE_INPUT if i != 2 else 0
        x = synth.activations_f16(71, 10 + i, 1, K)
        xd = torch.from_numpy(x).cuda()
        ys = [torch.full((1, N), float("nan"), dtype=torch.float16, device="cuda") for _ in range(4)]
        bgg.bgg_ternary_gemv(d.desc, d.packed, xd, ys[0], 1, flags, ws)
        bgg.bgg_gemv_prepare(d.desc, xd, 1, flags, ws)
        bgg.bgg_gemv_run(d.desc, d.packed, ys[1], 1, ws)
        bgg.bgg_ternary_gemv(d.desc, d.packed, xd, ys[2], 1, flags, ws)
        bgg.bgg_gemv_prepare(d.desc, xd, 1, flags, ws)
        bgg.bgg_gemv_run(d.desc, d.packed, ys[3], 1, ws)
        torch.cuda.synchronize()
        a, b, a2, b2 = (t.cpu().numpy() for t in ys)
        assert not np.isnan(a).any() and not np.isnan(b).any()
        assert np.array_equal(a.view(np.uint16), a2.view(np.uint16)), f"call {i}: one launch repeated"
        assert np.array_equal(b.view(np.uint16), b2.view(np.uint16)), f"call {i}: two steps repeated"
        ref = oracle_y(fmt, T[rows], S[rows], x, rotate=flags != 0)
        den = max(float(np.max(np.abs(ref))), 1e-30)
        for y in (a, b):
            assert float(np.max(np.abs(y[0, rows].astype(np.float64) - ref[0]))) / den <= TOL, f"call {i}"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_basis_vectors_bit_exact(env, fmt):
    """Rotation off and x = e_k: y_n = S[n][k/128] * T[n][k] exactly."""
    bgg, torch = env
    N, K = 130, 768
    say(f"gemv basis {fmt}")
    T, S = gen_matrix(41, 6, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    ks = [0, 1, 127, 128, 129, 383, 640, 767]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    for i0 in range(0, len(ks), 4):
        y = d.gemv(x[i0:i0 + 4], rotate=False)
        for j, k in enumerate(ks[i0:i0 + 4]):
            want = (S[:, k // 128].astype(np.float64) * T[:, k]).astype(np.float16)
            assert np.array_equal(y[j].view(np.uint16), want.view(np.uint16)), f"k={k}"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_sylvester_rows(env, fmt):
    """Trit row n = Sylvester row r of block b with scale s picks out
    s * sqrt(128) * x[128 b + r] (closed form; no oracle involved)."""
    import scipy.linalg
    bgg, torch = env
    say(f"gemv sylvester {fmt}")
    K = 640
    H = scipy.linalg.hadamard(128).astype(np.int8)
    cases = [(b, r) for b in range(5) for r in (0, 1, 77, 127)]
    T = np.zeros((len(cases), K), np.int8)
    S = np.zeros((len(cases), K // 128), np.float16)
    for n, (b, r) in enumerate(cases):
        T[n, 128 * b:128 * b + 128] = H[r]
        S[n, b] = np.float16(0.0078125 * (1 + n % 5))
    x = synth.activations_f16(3, 3, 1, K)
    y = Dev(bgg, torch, fmt, T, S).gemv(x)[0].astype(np.float64)
    want = np.array([float(S[n, b]) * np.sqrt(128.0) * float(x[0, 128 * b + r]) for n, (b, r) in enumerate(cases)])
    assert np.all(np.abs(y - want) <= 2e-3 * np.max(np.abs(want)))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_without_rotation_is_garbage(env, fmt):
    """Skipping the activation transform must fail the tolerance by far (the
    pages warn that the wrong runtime emits garbage silently)."""
    bgg, torch = env
    say(f"gemv no-rotation {fmt}")
    N, K = 512, 2048
    T, S = gen_matrix(51, 7, N, K)
    x = synth.activations_f16(51, 8, 1, K)
    y = Dev(bgg, torch, fmt, T, S).gemv(x, rotate=False)
    ref = oracle_y(fmt, T, S, x)
    assert relerr(y, ref).min() > 100 * TOL
    # while the same call given x' does match
    xr = oracle.rotate(x).astype(np.float16)
    y2 = Dev(bgg, torch, fmt, T, S).gemv(xr, rotate=False)
    assert np.all(relerr(y2, oracle_y(fmt, T, S, xr, rotate=False)) <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_zero_weights_and_repeat_calls(env, fmt):
    bgg, torch = env
    say(f"gemv zeros/repeat {fmt}")
    N, K = 300, 5120
    T = np.zeros((N, K), np.int8)
    S = synth.scales_f16(1, 1, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    x = synth.activations_f16(1, 2, 2, K)
    assert np.all(d.gemv(x) == 0)
    # the same workspace reused across calls and shapes gives the same results
    T2, S2 = gen_matrix(61, 8, N, K)
    d2 = Dev(bgg, torch, fmt, T2, S2)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d2.desc, 16))
    y_a = d2.gemv(x, ws=ws)
    y_b = d2.gemv(x[:1], ws=ws)
    y_c = d2.gemv(x, ws=ws)
    assert np.array_equal(y_a, y_c)
    assert np.array_equal(y_a[:1], y_b)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408), (1000, 1152), (200, 5248),
                                 (8192, 6144)])
def test_gemv_tokens_do_not_mix(env, fmt, N, K):
    """Several tokens share each weight load: a token's y must not depend on
    the other tokens of the call -- the tokens in reverse order give the
    rows in reverse order bit for bit, the same token in every slot gives
    identical rows -- and every token count matches the oracle.  (Token
    counts run on different kernels -- one token, up to four, more -- whose
    summation orders differ, so rows agree across token counts only within
    tolerance.)"""
    bgg, torch = env
    say(f"gemv tokens do not mix {fmt} {N}x{K}")
    T, S = gen_matrix(101, 3, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    x = synth.activations_f16(101, 4, 16, K)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 16))
    rows = np.arange(N) if N * K <= 1 << 21 else np.random.default_rng(5).choice(N, 64, replace=False)
    ref16 = oracle_y(fmt, T[rows], S[rows], x)
    for M in (1, 2, 3, 4, 7, 15, 16):
        xm = x[16 - M:]
        yM = d.gemv(xm, ws=ws)
        assert np.all(relerr(yM[:, rows], ref16[16 - M:]) <= TOL), f"M={M}"
        if M > 1:
            yr = d.gemv(np.ascontiguousarray(xm[::-1]), ws=ws)
            assert np.array_equal(yr[::-1].view(np.uint16), yM.view(np.uint16)), f"M={M} reversed"
            ys = d.gemv(np.repeat(xm[:1], M, axis=0), ws=ws)
            assert np.all(ys.view(np.uint16) == yM[:1].view(np.uint16)), f"M={M} same token"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", [(1, 128, 16), (1, 640, 2), (65, 256, 5), (64, 128, 16),
                                   (4097, 640, 2), (130, 1152, 16), (300, 5248, 9),
                                   (1, 17408, 1), (64, 8192, 1)])
def test_gemv_matrix_core_edges(env, fmt, N, K, M):
    """Matrix-core GEMV edge shapes: one row, one 128-group, ragged tiles
    (65 rows; 4097 rows = 64 tiles and one row), K not a multiple of the
    PTQ1_0 period (5248 = 8 periods and one group), and one row tile with a
    long K, which the one-token kernels cut into the most K ranges (up to
    the 63 the row words count); every output checked.
    With a single output per token the per-row bar would divide by one dot
    product, which can nearly cancel (-9e-5 for one token here); such
    shapes are held to the same bar pooled over all tokens."""
    bgg, torch = env
    say(f"gemv matrix-core edges {fmt} N={N} K={K} M={M}")
    T, S = gen_matrix(111, 5, N, K)
    x = synth.activations_f16(111, 6, M, K)
    d = Dev(bgg, torch, fmt, T, S)
    kn = bgg.bgg_gemv_kernel_name(d.desc, M)
    assert kn.startswith("k_mxv") or "_mx<" in kn, kn
    y = d.gemv(x)
    assert not np.isnan(y).any()
    ref = oracle_y(fmt, T, S, x)
    if N < 64:
        assert np.max(np.abs(y - ref)) <= TOL * np.max(np.abs(ref))
    else:
        assert np.all(relerr(y, ref) <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_matrix_core_every_token_count(env, fmt):
    """Every M from 2 to 16 on one shape, each against the oracle, one
    workspace for all calls (sized for 16 tokens)."""
    bgg, torch = env
    N, K = 257, 1408
    say(f"gemv matrix-core M=2..16 {fmt}")
    T, S = gen_matrix(121, 7, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 16))
    x = synth.activations_f16(121, 8, 16, K)
    ref = oracle_y(fmt, T, S, x)
    for M in range(2, 17):
        y = d.gemv(x[:M], ws=ws)
        assert np.all(relerr(y, ref[:M]) <= TOL), f"M={M}"


@pytest.mark.parametrize("N,K,M", [(8064 - 37, 6144, 1), (12864, 6144, 1), (16064 - 5, 6144, 1),
                                   (24064 + 64, 6144, 1), (4864 - 1, 6144, 2), (9664 + 3, 6144, 2),
                                   (17664, 6144, 2), (300, 1408, 2), (1024, 5120, 1), (6144, 5120, 1),
                                   (5120, 6144, 1), (1000, 5120, 2), (130, 640, 1)])
def test_gemv_ptq1_waves_per_workgroup(env, N, K, M):
    """The PTQ1_0 one- and two-token kernel takes as many row tiles per
    workgroup (one per wave) as keep one workgroup per CU, up to 16 (one
    token) or 12 (two), with at least 5 or 3 waves (the waves past the tiles
    only help with the table and the encoding): these shapes select counts
    across that range, small projections with fewer tiles than waves
    (ragged last row ranges included).  Rows of the first and the last row
    range and a random sample match the oracle."""
    bgg, torch = env
    T, S = gen_matrix(141, 2, N, K, fmt="PTQ1_0")
    d = Dev(bgg, torch, "PTQ1_0", T, S)
    kn = bgg.bgg_gemv_kernel_name(d.desc, M)
    say(f"gemv PTQ1_0 N={N} K={K} M={M}: {kn}")
    nw = int(kn.split("<")[1].split(",")[0])
    assert kn.startswith("k_mxv_ptq1<") and (5 if M == 1 else 3) <= nw <= (16 if M == 1 else 12), kn
    x = synth.activations_f16(141, 3, M, K)
    y = d.gemv(x)
    assert not np.isnan(y).any()
    span = 64 * nw
    rows = np.unique(np.concatenate([np.arange(min(span, N)), np.arange(max(0, N - span - 64), N),
                                     np.random.default_rng(9).choice(N, min(N, 256), replace=False)]))
    ref = oracle_y("PTQ1_0", T[rows], S[rows], x)
    assert np.all(relerr(y[:, rows], ref) <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_workspace_shared_across_shapes(env, fmt):
    """One zero-filled workspace serves calls of different K, N and M in any
    order (the split-K row sums are left at zero by every launch)."""
    bgg, torch = env
    say(f"gemv shared workspace {fmt}")
    shapes = [(5120, 17408), (17408, 5120), (300, 640), (6144, 5120)]
    devs = []
    for i, (N, K) in enumerate(shapes):
        T, S = gen_matrix(131, 10 + i, N, K)
        devs.append((Dev(bgg, torch, fmt, T, S), T, S))
    ws = bgg.workspace(max(bgg.bgg_gemv_workspace_size(d.desc, 16) for d, _, _ in devs))
    for M in (1, 16, 3, 1, 2):
        for d, T, S in devs:
            x = synth.activations_f16(131, 20 + M, M, d.K)
            y = d.gemv(x, ws=ws)
            rows = np.arange(0, d.N, 97)
            ref = oracle.matvec(T[rows], S[rows], oracle.rotate(x))
            assert np.all(relerr(y[:, rows], ref) <= TOL), f"M={M} {d.N}x{d.K}"


# ---------------------------------------------------------------------------
# prompt GEMM
# ---------------------------------------------------------------------------
GEMM_FMTS = ("PQ2_0", "PTQ1_0")


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (96, 256, 512), (200, 300, 640), (129, 1000, 1152),
                                   (257, 129, 2048), (64, 70, 384), (130, 513, 5248)])
def test_gemm_parity(env, fmt, M, N, K):
    """Ragged M and N tiles; for PTQ1_0 also odd chunk counts (K = 384 and
    1152: 5 and 15 chunks of 80 trits) and chunks that straddle 128-groups."""
    bgg, torch = env
    say(f"gemm {fmt} M={M} N={N} K={K}")
    T, S = gen_matrix(71, 9, N, K)
    x = synth.activations_f16(71, 10, M, K)
    d = Dev(bgg, torch, fmt, T, S)
    y = d.gemm(x)
    assert not np.isnan(y).any()
    ref = oracle_y(fmt, T, S, x)
    e = relerr(y, ref)
    say(f"  rel err max {e.max():.3g}")
    assert np.all(e <= TOL)
    # without rotation, given x'
    xr = oracle.rotate(x).astype(np.float16)
    y2 = d.gemm(xr, rotate=False)
    assert np.all(relerr(y2, oracle_y(fmt, T, S, xr, rotate=False)) <= TOL)


def test_gemm_pq2_basis_vectors_bit_exact(env):
    """PQ2_0 GEMM, rotation off, x = e_k for every k of K = 384 (three
    128-wide K steps, so the last one runs alone): y_n = S[n][k/128] T[n][k]
    exactly.  Every activation piece position of the LDS layout and every
    code slot of the weight decode is hit by one token."""
    bgg, torch = env
    N, K = 130, 384
    T, S = gen_matrix(46, 2, N, K)
    d = Dev(bgg, torch, "PQ2_0", T, S)
    x = np.eye(K, dtype=np.float16)
    y = d.gemm(x, rotate=False)
    want = (np.repeat(S.astype(np.float64), 128, axis=1)[:, :K] * T).astype(np.float16).T
    bad = np.argwhere(y.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, f"first mismatches (k, n): {bad[:5].tolist()}"


def test_gemm_ptq1_rewrite_is_the_pq2_layout(env):
    """With room in the workspace, the PTQ1_0 GEMM rewrites its weights to
    PQ2_0 and runs the PQ2_0 kernel.  The rewritten
    trits (at the start of the workspace when nothing is rotated) are the
    PQ2_0 device layout of the same trits, byte for byte: read back to
    canonical rows they equal the oracle's PQ2_0 packing (padding rows: zero
    trits).  K = 1152: 15 PTQ1_0 chunks, 18 PQ2_0 chunks, the last 320-trit
    block partial."""
    bgg, torch = env
    N, K, M = 130, 1152, 256
    T, S = gen_matrix(47, 2, N, K, fmt="PTQ1_0")
    d = Dev(bgg, torch, "PTQ1_0", T, S)
    d2 = bgg.bgg_describe("PQ2_0", N, K)
    ws = bgg.workspace(bgg.bgg_gemm_workspace_size(d.desc, M))
    assert ws.numel() >= d2.trit_bytes
    x = torch.from_numpy(synth.activations_f16(47, 3, M, K)).cuda()
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    bgg.bgg_ternary_gemm(d.desc, d.packed, x, y, M, 0, ws)
    torch.cuda.synchronize()
    C2 = K // 64
    buf = ws[:d2.trit_bytes].cpu().numpy()
    rows = buf.reshape(d2.row_tiles, C2, 64, 16).transpose(0, 2, 1, 3).reshape(d2.row_tiles * 64, C2 * 16)
    assert np.array_equal(rows[:N, :d2.row_bytes], oracle.pack("PQ2_0", T))
    assert np.all(rows[N:] == 0x55)
    ref = oracle_y("PTQ1_0", T, S, x.cpu().numpy(), rotate=False)
    assert np.all(relerr(y.cpu().numpy(), ref) <= TOL)


@pytest.mark.parametrize("M", [15, 1152])
def test_gemm_ptq1_basis_vectors_bit_exact(env, M):
    """PTQ1_0 GEMM, rotation off, x = e_k: y_n = S[n][k/128] T[n][k] exactly
    (one non-zero product per output).  M = 15: the byte-table kernel (no
    workspace), at chunk and group edges; M = 1152: every k, through the
    weights rewritten to PQ2_0 (a workspace is given)."""
    bgg, torch = env
    N, K = 130, 1152
    T, S = gen_matrix(45, 2, N, K)
    d = Dev(bgg, torch, "PTQ1_0", T, S)
    ks = ([0, 1, 79, 80, 127, 128, 159, 160, 639, 640, 1039, 1040, 1119, 1120, 1151] if M == 15
          else list(range(K)))
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    if M == 15:
        y = d.gemm(x, rotate=False)
    else:
        ws = bgg.workspace(bgg.bgg_gemm_workspace_size(d.desc, M))
        xd = torch.from_numpy(x).cuda()
        yd = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        bgg.bgg_ternary_gemm(d.desc, d.packed, xd, yd, M, 0, ws)
        torch.cuda.synchronize()
        y = yd.cpu().numpy()
    want = (np.repeat(S.astype(np.float64), 128, axis=1)[:, :K] * T).astype(np.float16).T[ks]
    bad = np.argwhere(y.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, f"first mismatches (token, n): {bad[:5].tolist()}"


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_gemm_prefill_full_size_sampled(env, fmt, name):
    """The prefill workload (4096 tokens) at full size; 24 token rows checked
    against the oracle over all N outputs."""
    bgg, torch = env
    w = synth.WORKLOADS["prefill"]
    mat = [m for m in w["matrices"] if m.name == name][0]
    say(f"gemm full {fmt} {name} M=4096 N={mat.n} K={mat.k}")
    T, S = synth.workload_matrix(mat, w["seed"])
    x = synth.workload_x(w["seed"], 4096, mat.k)
    y = Dev(bgg, torch, fmt, T, S).gemm(x)
    assert not np.isnan(y).any()
    rows = np.array([0, 1, 2, 31, 32, 127, 128, 255, 256, 1000, 2047, 2048, 3000, 4031, 4064, 4095,
                     511, 512, 767, 1023, 1536, 2560, 3583, 3584])
    ref = oracle.matvec(T, S, oracle.rotate(x[rows]))
    e = relerr(y[rows], ref)
    say(f"  rel err max {e.max():.3g}")
    assert np.all(e <= TOL)


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("K", [1024, 1152])
def test_gemm_two_k_ranges(env, fmt, K):
    """520 output blocks (M = 13312, N = 1280) fill the 512 workgroup slots
    unevenly, so K is cut in two ranges over two workgroups with fp32
    partials in the workspace, for an even (K = 1024) and an odd (K = 1152)
    number of 128-wide K steps.  Sampled token rows match the oracle over
    all N outputs, and a second call gives the same bits."""
    bgg, torch = env
    M, N = 13312, 1280
    say(f"gemm two K ranges {fmt} M={M} N={N} K={K}")
    T, S = gen_matrix(131, 4, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    x = synth.activations_f16(131, 5, M, K)
    y = d.gemm(x)
    assert not np.isnan(y).any()
    assert np.array_equal(d.gemm(x).view(np.uint16), y.view(np.uint16))
    rows = np.array([0, 1, 127, 128, 4095, 4096, 6655, 6656, 9000, 13183, 13184, 13311])
    ref = oracle.matvec(T, S, oracle.rotate(x[rows]))
    assert np.all(relerr(y[rows], ref) <= TOL)


@pytest.mark.parametrize("fmt", GEMM_FMTS)
@pytest.mark.parametrize("rotate", [True, False])
def test_gemm_non_finite_activations(env, fmt, rotate):
    """NaN, +inf and -inf in one position each of three tokens' x: the prefill
    GEMM follows IEEE arithmetic (fp16 MFMA products, fp32 sums), so those
    rows are non-finite exactly where the oracle's fp64 rows are, NaN where
    it has NaN and the same infinity where it has one; the other tokens keep
    the bits of a call without the bad values.  With the transform (and its
    workspace) PTQ1_0 runs on rewritten weights, without it on the byte-table
    kernel."""
    bgg, torch = env
    M, N, K = 6, 300, 1152
    T, S = gen_matrix(233, 1, N, K, fmt=fmt)
    d = Dev(bgg, torch, fmt, T, S)
    x0 = synth.activations_f16(233, 2, M, K)
    y0 = d.gemm(x0, rotate=rotate)
    x = x0.copy()
    bad = {1: np.nan, 3: np.inf, 4: -np.inf}
    for m, v in bad.items():
        x[m, 137 * m] = v
    y = d.gemm(x, rotate=rotate)
    ref = oracle_y(fmt, T, S, x, rotate=rotate).astype(np.float16)
    for m in bad:
        assert not np.isfinite(ref[m]).all(), f"token {m}: the oracle row is finite"
        yr, rr = y[m], ref[m]
        assert np.array_equal(np.isnan(yr), np.isnan(rr)), f"token {m}: NaN pattern"
        inf = np.isinf(rr)
        assert np.array_equal(yr[inf], rr[inf]) and np.isinf(yr).sum() == inf.sum(), f"token {m}: infinities"
        fin = np.isfinite(rr)
        assert np.all(relerr(yr[fin][None], rr[fin][None].astype(np.float64)) <= TOL) if fin.any() else True
    good = [i for i in range(M) if i not in bad]
    assert np.array_equal(y[good].view(np.uint16), y0[good].view(np.uint16))


@pytest.mark.parametrize("fmt", GEMM_FMTS)
def test_gemm_k_split_deterministic(env, fmt):
    """A product with few output blocks (25 here) splits K into ranges (10
    here) when the workspace holds the partials: the same inputs give the
    same bits call after call, and the split and unsplit results agree with
    the oracle and with each other within the bar.  (The parity shapes above
    run 1 to 32 ranges with the rotation workspace, none without.)"""
    bgg, torch = env
    M, N, K = 640, 1280, 5248
    say(f"gemm K split {fmt}")
    T, S = gen_matrix(99, 5, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    x = synth.activations_f16(99, 6, M, K)
    xr = torch.from_numpy(oracle.rotate(x).astype(np.float16)).cuda()
    full = bgg.bgg_gemm_workspace_size(d.desc, M)
    assert full >= M * K * 2 + 2 * M * N * 4      # this shape splits
    ws = bgg.workspace(full)
    outs = []
    for _ in range(3):
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        bgg.bgg_ternary_gemm(d.desc, d.packed, xr, y, M, 0, ws)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    assert all(np.array_equal(o.view(np.uint16), outs[0].view(np.uint16)) for o in outs[1:])
    y1 = d.gemm(xr.cpu().numpy(), rotate=False)    # no workspace: one pass over K
    ref = oracle_y(fmt, T, S, xr.cpu().numpy(), rotate=False)
    assert np.all(relerr(outs[0], ref) <= TOL) and np.all(relerr(y1, ref) <= TOL)
    assert np.all(relerr(outs[0], y1.astype(np.float64)) <= TOL)


@pytest.mark.parametrize("fmt", GEMM_FMTS)
def test_gemm_graph_replay_matches_eager(env, fmt):
    """Transform + GEMM captured in a HIP graph: every replay, with eager work
    on the same workspace between replays, gives the eager bits (no memset
    nodes: the transform writes the whole workspace it reads)."""
    bgg, torch = env
    M, N, K = 300, 1000, 1152
    say(f"gemm graph replay {fmt}")
    T, S = gen_matrix(97, 2, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    x = torch.from_numpy(synth.activations_f16(97, 3, M, K)).cuda()
    x_other = torch.from_numpy(synth.activations_f16(97, 4, M, K)).cuda()
    ws = bgg.workspace(bgg.bgg_gemm_workspace_size(d.desc, M))
    y_eager = torch.empty((M, N), dtype=torch.float16, device="cuda")
    bgg.bgg_ternary_gemm(d.desc, d.packed, x, y_eager, M, bgg.BGG_ROTATE_INPUT, ws)
    torch.cuda.synchronize()
    want = y_eager.cpu().numpy()
    assert np.all(relerr(want, oracle_y(fmt, T, S, x.cpu().numpy())) <= TOL)
    y_graph = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bgg.bgg_ternary_gemm(d.desc, d.packed, x, y_graph, M, bgg.BGG_ROTATE_INPUT, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bgg.bgg_ternary_gemm(d.desc, d.packed, x, y_graph, M, bgg.BGG_ROTATE_INPUT, ws,
                             torch.cuda.current_stream())
    y_other = torch.empty((M, N), dtype=torch.float16, device="cuda")
    for rep in range(4):
        y_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y_graph.cpu().numpy().view(np.uint16), want.view(np.uint16)), \
            f"replay {rep}"
        bgg.bgg_ternary_gemm(d.desc, d.packed, x_other, y_other, M, bgg.BGG_ROTATE_INPUT, ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_shared_preparation(env, fmt):
    """q, k and v read the same input: one prepare, three runs."""
    bgg, torch = env
    say(f"gemv shared prepare {fmt}")
    K, M = 5120, 2
    x = synth.activations_f16(81, 9, M, K)
    mats = [(6144, 1), (1024, 2), (1024, 3)]
    devs = []
    for N, mid in mats:
        T, S = gen_matrix(81, mid, N, K)
        devs.append((Dev(bgg, torch, fmt, T, S), T, S))
    wsb = max(bgg.bgg_gemv_workspace_size(d.desc, M) for d, _, _ in devs)
    ws = bgg.workspace(wsb)
    xd = torch.from_numpy(x).cuda()
    bgg.bgg_gemv_prepare(devs[0][0].desc, xd, M, bgg.BGG_ROTATE_INPUT, ws)
    outs = []
    for d, T, S in devs:
        yd = torch.empty((M, d.N), dtype=torch.float16, device="cuda")
        bgg.bgg_gemv_run(d.desc, d.packed, yd, M, ws)
        outs.append(yd)
    torch.cuda.synchronize()
    for (d, T, S), yd in zip(devs, outs):
        assert np.all(relerr(yd.cpu().numpy(), oracle_y(fmt, T, S, x)) <= TOL)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408), (300, 640)])
def test_gemv_graph_replay_matches_eager(env, fmt, N, K):
    """prepare + run captured in a HIP graph: every replay, with other eager
    work and synchronisations between replays, gives the eager result bit
    for bit (the kernels are deterministic; the prep clears the split-K row
    sums with a kernel, and each run leaves them at zero)."""
    bgg, torch = env
    say(f"gemv graph replay {fmt} {N}x{K}")
    T, S = gen_matrix(91, 3, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    x = torch.from_numpy(synth.activations_f16(91, 4, 1, K)).cuda()
    x_other = torch.from_numpy(synth.activations_f16(91, 5, 1, K)).cuda()
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 1))
    y_eager = torch.empty((1, N), dtype=torch.float16, device="cuda")
    bgg.bgg_ternary_gemv(d.desc, d.packed, x, y_eager, 1, bgg.BGG_ROTATE_INPUT, ws)
    torch.cuda.synchronize()
    want = y_eager.cpu().numpy()
    assert np.all(relerr(want, oracle_y(fmt, T, S, x.cpu().numpy())) <= TOL)

    y_graph = torch.full((1, N), float("nan"), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bgg.bgg_ternary_gemv(d.desc, d.packed, x, y_graph, 1, bgg.BGG_ROTATE_INPUT, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bgg.bgg_ternary_gemv(d.desc, d.packed, x, y_graph, 1, bgg.BGG_ROTATE_INPUT, ws,
                             torch.cuda.current_stream())
    y_other = torch.empty((1, N), dtype=torch.float16, device="cuda")
    for rep in range(4):
        y_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y_graph.cpu().numpy(), want), f"replay {rep}"
        # eager work on the same workspace between replays
        bgg.bgg_ternary_gemv(d.desc, d.packed, x_other, y_other, 1, bgg.BGG_ROTATE_INPUT, ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_rows_beyond_one_launch(env, fmt):
    """N = 65600, K = 8320: K is split over workgroups and the tiles exceed
    what one launch's row words hold (65536 rows), so the call runs as
    several launches that reuse the words.  Rows on both sides of the launch
    boundary and a random sample match the oracle for one and two tokens,
    and the call leaves every row word zero."""
    bgg, torch = env
    N, K = 65600, 8320
    say(f"gemv rows beyond one launch {fmt} N={N} K={K}")
    T, S = gen_matrix(241, 1, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 65535, 65536, 65537, 65599],
                                     rng.choice(N, 56, replace=False)]))
    wsz = bgg.bgg_gemv_workspace_size(d.desc, 2)
    for M in (1, 2):
        ws = bgg.workspace(wsz)
        x = synth.activations_f16(241, 2 + M, M, K)
        y = d.gemv(x, ws=ws)
        assert not np.isnan(y).any()
        ref = oracle_y(fmt, T[rows], S[rows], x)
        assert np.all(relerr(y[:, rows], ref) <= TOL), f"M={M}"
        words = ws[:16 << 20].view(torch.int64)
        assert int(torch.count_nonzero(words)) == 0, f"M={M}: row words left non-zero"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_workspace_reset(env, fmt):
    """A workspace filled with other data: bgg_gemv_workspace_reset zeroes
    its row words (and leaves the rest alone), after which a GEMV whose K is
    split over workgroups (the row words in use) matches the oracle for one
    and three tokens."""
    bgg, torch = env
    N, K = 300, 5120
    say(f"gemv workspace reset {fmt}")
    T, S = gen_matrix(251, 1, N, K)
    d = Dev(bgg, torch, fmt, T, S)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 3))
    ws.fill_(0x5A)
    bgg.bgg_gemv_workspace_reset(ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:16 << 20])) == 0
    assert bool(torch.all(ws[16 << 20:] == 0x5A))
    for M in (1, 3):
        x = synth.activations_f16(251, 2 + M, M, K)
        y = d.gemv(x, ws=ws)
        assert np.all(relerr(y, oracle_y(fmt, T, S, x)) <= TOL), f"M={M}"
