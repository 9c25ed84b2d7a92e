"""GPU parity of the sister formats Q1_0 (one sign bit per weight, an fp16
scale per 128) and Q2_0_G64 (the PQ2_0 row stream, an fp16 scale per 64)
through the C ABI against the CPU oracle, on seeded synthetic inputs.
Marked gpu; run on an MI355X.

Bars as for PQ2_0 and PTQ1_0: unpacking bit-exact; y within 2e-3 of the
oracle per token row; basis vectors bit-exact; a token's y independent of
the other tokens and of M, bit for bit.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_helpers import TOL, Dev, gen_matrix, oracle_y, relerr  # noqa: E402

SISTERS = ("Q1_0", "Q2_0_G64")
KERNEL = {"Q1_0": "k_gemv_q1_mx<", "Q2_0_G64": "k_gemv_q2g64_mx<"}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import bit_gemv_gemm_amd as bgg
    return bgg, torch


def _unpack(bgg, torch, d):
    td = torch.empty((d.N, d.K), dtype=torch.int8, device="cuda")
    sd = torch.empty((d.N, d.desc.scales), dtype=torch.float16, device="cuda")
    bgg.bgg_unpack_weights(d.desc, d.packed, td, sd)
    torch.cuda.synchronize()
    return td.cpu().numpy(), sd.cpu().numpy()


@pytest.mark.parametrize("fmt", SISTERS)
@pytest.mark.parametrize("N,K", [(1, 128), (100, 640), (130, 1152), (64, 6144), (5120, 17408)])
def test_sister_unpack_bit_exact(env, fmt, N, K):
    bgg, torch = env
    say(f"unpack {fmt} N={N} K={K}")
    T, S = gen_matrix(11, 3, N, K, fmt=fmt)
    d = Dev(bgg, torch, fmt, T, S)
    t, s = _unpack(bgg, torch, d)
    assert np.array_equal(t, oracle.unpack(fmt, oracle.pack(fmt, T), K))
    assert np.array_equal(s.view(np.uint16), S.view(np.uint16))


def test_q1_unpack_every_byte(env):
    """All 256 byte values of the Q1_0 row stream, laid out from canonical
    bytes, decode as the oracle decodes them."""
    bgg, torch = env
    say("unpack Q1_0 every byte")
    N, K = 70, 1024
    j, i = np.meshgrid(np.arange(K // 8), np.arange(N))
    canon = ((j + 128 * (i % 2) + 5 * i) % 256).astype(np.uint8)
    S = synth.scales_f16(2, 2, N, K)
    desc = bgg.bgg_describe("Q1_0", N, K)
    packed = bgg.upload(bgg.bgg_repack_canonical(desc, canon, S))
    td = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sd = torch.empty((N, K // 128), dtype=torch.float16, device="cuda")
    bgg.bgg_unpack_weights(desc, packed, td, sd)
    torch.cuda.synchronize()
    assert len(np.unique(canon)) == 256
    assert np.array_equal(td.cpu().numpy(), oracle.unpack("Q1_0", canon, K))


GEMV_CASES = [
    # (N, K, M): one row; one 128 block; ragged tiles; the attention and
    # MLP shapes; 4097 rows = 64 tiles and one row; K = 41 blocks
    (1, 384, 1), (7, 128, 2), (100, 640, 3), (65, 256, 5), (6144, 5120, 1),
    (5120, 6144, 2), (1024, 5120, 16), (4097, 640, 2), (300, 5248, 9), (200, 1280, 8),
]


@pytest.mark.parametrize("fmt", SISTERS)
@pytest.mark.parametrize("N,K,M", GEMV_CASES)
def test_sister_gemv_parity(env, fmt, N, K, M):
    bgg, torch = env
    say(f"gemv {fmt} N={N} K={K} M={M}")
    T, S = gen_matrix(21, 4, N, K, fmt=fmt)
    x = synth.activations_f16(21, 100 + K, M, K)
    d = Dev(bgg, torch, fmt, T, S)
    assert bgg.bgg_gemv_kernel_name(d.desc, M).startswith(KERNEL[fmt])
    y = d.gemv(x)
    assert not np.isnan(y).any()
    ref = oracle_y(fmt, T, S, x)
    if N < 64:  # one dot product per token can nearly cancel: pooled bar
        assert np.max(np.abs(y - ref)) <= TOL * np.max(np.abs(ref))
    else:
        e = relerr(y, ref)
        say(f"  rel err max {e.max():.3g}")
        assert np.all(e <= TOL)


@pytest.mark.parametrize("fmt", SISTERS)
@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_sister_projection_full_size(env, fmt, name):
    """The single-projection workload's shapes in the sister format, one
    token, every output checked."""
    bgg, torch = env
    w = synth.WORKLOADS["projection"]
    mat = [m for m in w["matrices"] if m.name == name][0]
    say(f"gemv full {fmt} {name} N={mat.n} K={mat.k}")
    T, S = synth.workload_matrix(mat, w["seed"], fmt)
    x = synth.workload_x(w["seed"], 1, mat.k)
    y = Dev(bgg, torch, fmt, T, S).gemv(x)
    e = relerr(y, oracle_y(fmt, T, S, x))
    say(f"  rel err {e}")
    assert np.all(e <= TOL)


@pytest.mark.parametrize("fmt", SISTERS)
def test_sister_basis_vectors_bit_exact(env, fmt):
    """Rotation off and x = e_k: y_n = S[n][k / group] * T[n][k] exactly,
    at the edges of the 64- and 128-weight groups."""
    bgg, torch = env
    N, K = 130, 768
    g = synth.scale_group(fmt)
    say(f"gemv basis {fmt}")
    T, S = gen_matrix(41, 6, N, K, fmt=fmt)
    d = Dev(bgg, torch, fmt, T, S)
    ks = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, 191, 192, 383, 640, 704, 767]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = d.gemv(x, rotate=False)
    for j, k in enumerate(ks):
        want = (S[:, k // g].astype(np.float64) * T[:, k]).astype(np.float16)
        assert np.array_equal(y[j].view(np.uint16), want.view(np.uint16)), f"k={k}"


def test_q1_sylvester_rows(env):
    """Q1_0 rows made of Sylvester rows r_b in every block b, scale s_b:
    y = sqrt(128) sum_b s_b x[128 b + r_b] (closed form, no oracle)."""
    import scipy.linalg
    bgg, torch = env
    say("gemv sylvester Q1_0")
    K, N = 640, 24
    H = scipy.linalg.hadamard(128).astype(np.int8)
    rng = np.random.default_rng(5)
    R = rng.integers(0, 128, size=(N, K // 128))
    T = np.concatenate([H[R[:, b]] for b in range(K // 128)], axis=1)
    S = (0.0078125 * rng.integers(1, 6, size=(N, K // 128))).astype(np.float16)
    x = synth.activations_f16(3, 3, 1, K)
    y = Dev(bgg, torch, "Q1_0", T, S).gemv(x)[0].astype(np.float64)
    xb = x[0].astype(np.float64)
    want = np.array([np.sqrt(128.0) * sum(float(S[n, b]) * xb[128 * b + R[n, b]]
                                          for b in range(K // 128)) for n in range(N)])
    assert np.all(np.abs(y - want) <= 2e-3 * np.max(np.abs(want)))


def test_q2g64_sylvester_half_scales(env):
    """Q2_0_G64 row = Sylvester row r of block b with scales s0 (first 64)
    and s1 (second 64).  With r = 64 h + r' (r' < 64), the rotated product
    is (64 / sqrt(128)) (s0 (x_a + x_b) + (-1)^h s1 (x_a - x_b)), where
    x_a = x[128 b + r'] and x_b = x[128 b + r' + 64] (closed form from the
    block structure of the Sylvester matrix; no oracle)."""
    import scipy.linalg
    bgg, torch = env
    say("gemv sylvester Q2_0_G64")
    K = 640
    H = scipy.linalg.hadamard(128).astype(np.int8)
    cases = [(b, r) for b in range(5) for r in (0, 1, 63, 64, 77, 127)]
    T = np.zeros((len(cases), K), np.int8)
    S = np.zeros((len(cases), K // 64), np.float16)
    for n, (b, r) in enumerate(cases):
        T[n, 128 * b:128 * b + 128] = H[r]
        S[n, 2 * b] = np.float16(0.0078125 * (1 + n % 5))
        S[n, 2 * b + 1] = np.float16(0.0078125 * (1 + (3 * n + 2) % 7))
    x = synth.activations_f16(3, 4, 1, K)
    y = Dev(bgg, torch, "Q2_0_G64", T, S).gemv(x)[0].astype(np.float64)
    xb = x[0].astype(np.float64)
    want = []
    for n, (b, r) in enumerate(cases):
        h, rr = divmod(r, 64)
        xa, xq = xb[128 * b + rr], xb[128 * b + rr + 64]
        s0, s1 = float(S[n, 2 * b]), float(S[n, 2 * b + 1])
        want.append(64.0 / np.sqrt(128.0) * (s0 * (xa + xq) + (-1) ** h * s1 * (xa - xq)))
    want = np.array(want)
    assert np.all(np.abs(y - want) <= 2e-3 * np.max(np.abs(want)))


@pytest.mark.parametrize("fmt", SISTERS)
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408), (1000, 1152), (200, 5248)])
def test_sister_tokens_do_not_mix(env, fmt, N, K):
    """Every token count runs the same matrix-core kernel: a token's y does
    not depend on the other tokens or on M, bit for bit, one token included."""
    bgg, torch = env
    say(f"gemv tokens do not mix {fmt} {N}x{K}")
    T, S = gen_matrix(101, 3, N, K, fmt=fmt)
    d = Dev(bgg, torch, fmt, T, S)
    x = synth.activations_f16(101, 4, 16, K)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 16))
    y16 = d.gemv(x, ws=ws)
    rows = np.arange(0, N, 7)
    ref = oracle.matvec(T[rows], S[rows], oracle.rotate(x))
    assert np.all(relerr(y16[:, rows], ref) <= TOL)
    for M in (1, 2, 3, 7, 15):
        yM = d.gemv(x[16 - M:], ws=ws)
        assert np.array_equal(yM.view(np.uint16), y16[16 - M:].view(np.uint16)), f"M={M}"
    ys = d.gemv(np.repeat(x[5:6], 16, axis=0), ws=ws)
    assert np.all(ys.view(np.uint16) == y16[5].view(np.uint16))


def test_sister_formats_share_a_workspace(env):
    """One workspace serves all four formats in turn (the split-K row sums
    are left at zero by every launch; the prepared activations of one call
    are never read by the next)."""
    bgg, torch = env
    say("gemv one workspace, four formats")
    N, K = 5120, 17408
    devs = []
    for i, fmt in enumerate(("PQ2_0", "Q1_0", "PTQ1_0", "Q2_0_G64")):
        T, S = gen_matrix(141, 20 + i, N, K, fmt=fmt)
        devs.append((fmt, Dev(bgg, torch, fmt, T, S), T, S))
    ws = bgg.workspace(max(bgg.bgg_gemv_workspace_size(d.desc, 16) for _, d, _, _ in devs))
    rows = np.arange(0, N, 61)
    for M in (1, 16, 2):
        x = synth.activations_f16(141, 30 + M, M, K)
        xr = oracle.rotate(x)
        for fmt, d, T, S in devs:
            y = d.gemv(x, ws=ws)
            assert np.all(relerr(y[:, rows], oracle.matvec(T[rows], S[rows], xr)) <= TOL), \
                f"{fmt} M={M}"


@pytest.mark.parametrize("fmt", SISTERS)
def test_sister_graph_replay_matches_eager(env, fmt):
    """prepare + run captured in a HIP graph: every replay, with eager work
    on the same workspace between replays, gives the eager bits."""
    bgg, torch = env
    N, K = 6144, 5120
    say(f"gemv graph replay {fmt}")
    T, S = gen_matrix(91, 3, N, K, fmt=fmt)
    d = Dev(bgg, torch, fmt, T, S)
    x = torch.from_numpy(synth.activations_f16(91, 4, 2, K)).cuda()
    x_other = torch.from_numpy(synth.activations_f16(91, 5, 2, K)).cuda()
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, 2))
    y_eager = torch.empty((2, N), dtype=torch.float16, device="cuda")
    bgg.bgg_ternary_gemv(d.desc, d.packed, x, y_eager, 2, bgg.BGG_ROTATE_INPUT, ws)
    torch.cuda.synchronize()
    want = y_eager.cpu().numpy()
    assert np.all(relerr(want, oracle_y(fmt, T, S, x.cpu().numpy())) <= TOL)
    y_graph = torch.full((2, N), float("nan"), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bgg.bgg_ternary_gemv(d.desc, d.packed, x, y_graph, 2, bgg.BGG_ROTATE_INPUT, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bgg.bgg_ternary_gemv(d.desc, d.packed, x, y_graph, 2, bgg.BGG_ROTATE_INPUT, ws,
                             torch.cuda.current_stream())
    y_other = torch.empty((2, N), dtype=torch.float16, device="cuda")
    for rep in range(4):
        y_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y_graph.cpu().numpy(), want), f"replay {rep}"
        bgg.bgg_ternary_gemv(d.desc, d.packed, x_other, y_other, 2, bgg.BGG_ROTATE_INPUT, ws)
        torch.cuda.synchronize()


def test_sister_formats_have_no_prompt_kernel(env):
    bgg, torch = env
    for fmt in SISTERS:
        d = bgg.bgg_describe(fmt, 64, 128)
        with pytest.raises(bgg.BggError) as e:
            bgg.bgg_ternary_gemm(d, torch.zeros(d.total_bytes, dtype=torch.uint8, device="cuda"),
                                 torch.zeros((4, 128), dtype=torch.float16, device="cuda"),
                                 torch.zeros((4, 64), dtype=torch.float16, device="cuda"), 4, 0, None)
        assert e.value.status == 2
