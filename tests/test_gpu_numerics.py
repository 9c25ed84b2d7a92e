"""GPU parity at the edges of the decode GEMV's own arithmetic, against the
CPU oracle, through the C ABI.

The GEMV departs from an fp32 product of x' in three places, each pinned
here on every kernel family that serves a call: one token in one launch
(bgg_ternary_gemv, M = 1), one token in two steps (bgg_gemv_prepare +
bgg_gemv_run), two to four tokens, and five or more; on shapes whose K is cut
over workgroups (split-K row sums) and shapes whose K is not:

* the activations are carried per 128-block as 15-bit integers on a
  power-of-two grid (2^-14 of the block's largest |x'|): blocks with one
  element 2^10 .. 2^14 times the others, x at +-65504 and at fp16
  subnormals;
* split-K partial rows are added as 64-bit fixed-point integers (2^-30
  below 2^17, else in a 1/16 coarse word): partial rows far beyond 2^17
  that cancel, scales near the fp16 maximum and near the smallest normal;
* non-finite activations: a NaN or inf anywhere in a token's x makes the
  token's whole y row NaN.  The fp64 product of the oracle is non-finite in
  every row too: NaN wherever the row has a zero weight in the affected
  block (0 * inf), +-inf or NaN elsewhere; the library does not follow the
  signs of infinities and flags the token instead.  The other tokens of the
  call keep their bits.

y that the fp64 result puts beyond the fp16 range must be the same +-inf;
finite y within the per-row bar of 2e-3 of max |y| (over the finite
entries).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from gpu_helpers import TOL, Dev, gen_matrix, oracle_y  # noqa: E402

FMTS = ("PQ2_0", "PTQ1_0")
# (N, K): K cut over workgroups for every token count (few rows), K cut for
# one token (down projection), K whole for one token (gate/up projection)
SHAPES = [(300, 5120), (5120, 17408), (17408, 5120)]
# token counts: one launch / two steps (M = 1), 2 (one launch in both
# packings), 3 (one launch for PQ2_0, two steps for PTQ1_0), 5+ (6 and 13)
MODES = [("one", 1), ("two", 1), ("one", 2), ("one", 3), ("one", 6), ("one", 13)]
F16_MAX = 65504.0


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import bit_gemv_gemm_amd as bgg
    return bgg, torch


def run(bgg, torch, d, x, mode, rotate=True):
    M = x.shape[0]
    flags = bgg.BGG_ROTATE_INPUT if rotate else 0
    if mode == "one":
        return d.gemv(x, rotate=rotate)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    yd = torch.full((M, d.N), float("nan"), dtype=torch.float16, device="cuda")
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, M))
    bgg.bgg_gemv_prepare(d.desc, xd, M, flags, ws)
    bgg.bgg_gemv_run(d.desc, d.packed, yd, M, ws)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def sample_rows(N, K, seed):
    if N * K <= 1 << 21:
        return np.arange(N)
    return np.sort(np.random.default_rng(seed).choice(N, 96, replace=False))


def check(y, ref, what):
    """y (fp16, GPU) against ref (fp64, oracle), one token row at a time:
    within TOL of the row's largest |y| that fp16 holds; where the exact
    value rounds past the fp16 range by more than that, the same +-inf."""
    y = y.astype(np.float64)
    for m in range(ref.shape[0]):
        r, g = ref[m], y[m]
        assert not np.isnan(r).any(), f"{what} token {m}: the oracle has NaN"
        inrange = np.abs(r) < 65520.0  # rounds to a finite fp16
        den = float(np.max(np.abs(r[inrange]))) if inrange.any() else F16_MAX
        tol = TOL * max(den, 1e-300)
        must_inf = np.abs(r) >= 65520.0 + tol
        must_fin = np.abs(r) <= 65520.0 - tol
        assert np.array_equal(g[must_inf], np.where(r[must_inf] > 0, np.inf, -np.inf)), \
            f"{what} token {m}: overflow"
        assert np.isfinite(g[must_fin]).all(), f"{what} token {m}: non-finite y"
        err = float(np.max(np.abs(g[must_fin] - r[must_fin]), initial=0.0))
        assert err <= tol, f"{what} token {m}: rel err {err / max(den, 1e-300):.3g}"
        mid = ~must_inf & ~must_fin  # either side of the edge is right
        assert (np.where(np.isinf(g[mid]), np.sign(g[mid]) == np.sign(r[mid]),
                         np.abs(g[mid] - r[mid]) <= tol)).all(), f"{what} token {m}: edge"


def cases(env, fmt, T, S, make_x, what, rotate=True):
    """Every kernel family on one packed matrix: x = make_x(M)."""
    bgg, torch = env
    N, K = T.shape
    d = Dev(bgg, torch, fmt, T, S)
    rows = sample_rows(N, K, 3)
    for mode, M in MODES:
        say(f"{what}: {fmt} N={N} K={K} {mode} M={M}")
        x = make_x(M)
        y = run(bgg, torch, d, x, mode, rotate)
        ref = oracle_y(fmt, T[rows], S[rows], x, rotate=rotate)
        check(y[:, rows], ref, f"{what} ({mode}, M={M})")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_outlier_blocks(env, fmt, N, K):
    """Every 128-block has one element 2^10 .. 2^14 times the N(0,1) rest;
    with the transform the outlier spreads over its block, without it (x
    given as x') the small elements sit 10 to 14 bits below the block's
    largest."""
    T, S = gen_matrix(201, 1, N, K)

    def make_x(M):
        x = synth.activations_f16(201, 2, M, K).astype(np.float32)
        rng = np.random.default_rng(11 + M)
        G = K // 128
        pos = rng.integers(0, 128, size=(M, G)) + 128 * np.arange(G)
        mag = 2.0 ** rng.integers(10, 15, size=(M, G)) * rng.choice([-1.0, 1.0], size=(M, G))
        np.put_along_axis(x, pos, mag, axis=1)
        return x.astype(np.float16)

    cases(env, fmt, T, S, make_x, "outliers")
    cases(env, fmt, T, S, make_x, "outliers, no transform", rotate=False)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_fp16_extreme_activations(env, fmt, N, K):
    """x = +-65504 with scales near the smallest normal fp16 (y finite) and
    with scales near 2^-7 (y partly beyond the fp16 range: +-inf), and x among
    the fp16 subnormals with scales near 2^13 (y normal)."""
    T, _ = gen_matrix(211, 1, N, K)
    G = K // 128
    rng = np.random.default_rng(12)

    def big_x(M):
        return (np.random.default_rng(20 + M).choice([-1.0, 1.0], size=(M, K)) * F16_MAX).astype(np.float16)

    def sub_x(M):
        return (np.random.default_rng(30 + M).integers(-1023, 1024, size=(M, K)) * 2.0 ** -24).astype(np.float16)

    S = (2.0 ** -14 * (1 + 3 * rng.random((N, G)))).astype(np.float16)
    cases(env, fmt, T, S, big_x, "x at +-65504")
    S = (2.0 ** -7 * (1 + rng.random((N, G)))).astype(np.float16)
    cases(env, fmt, T, S, big_x, "x at +-65504, y overflowing")
    S = (2.0 ** 13 * (1 + rng.random((N, G)))).astype(np.float16)
    cases(env, fmt, T, S, sub_x, "subnormal x")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_extreme_scales(env, fmt, N, K):
    """Scales in [2^15, 65504] with x ~ N(0,1) 2^-9 (y of order 10^3 .. 10^4),
    and scales in [2^-14, 2^-13]."""
    T, _ = gen_matrix(221, 1, N, K)
    G = K // 128
    rng = np.random.default_rng(13)
    S = np.minimum(2.0 ** 15 * (1 + rng.random((N, G))), F16_MAX).astype(np.float16)
    cases(env, fmt, T, S,
          lambda M: (synth.activations_f16(221, 2, M, K).astype(np.float32) * 2.0 ** -9).astype(np.float16),
          "scales near fp16 max")
    S = (2.0 ** -14 * (1 + rng.random((N, G)))).astype(np.float16)
    cases(env, fmt, T, S, lambda M: synth.activations_f16(221, 3, M, K), "scales near the smallest normal")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_cancelling_partials_exact(env, fmt, N, K):
    """Row n: t = +1 on the first half of K, -1 on the second half but for
    2 (n % 8) zeros, every scale 65504, x' = 2^-6 everywhere (given
    rotated): partial rows of split-K launches reach 2^17 .. 2^23 (the
    coarse words) and cancel to y = 2047 (n % 8).  Every partial is an
    integer below 2^24, so every step is exact and y must be the fp16
    rounding of the exact value, bit for bit, as the oracle's is."""
    bgg, torch = env
    G = K // 128
    T = np.ones((N, K), dtype=np.int8)
    T[:, K // 2:] = -1
    for r in range(8):
        T[r::8, K // 2:K // 2 + 2 * r] = 0
    S = np.full((N, G), F16_MAX, dtype=np.float16)
    d = Dev(bgg, torch, fmt, T, S)
    want = (2047.0 * (np.arange(N) % 8)).astype(np.float16)
    rows = sample_rows(N, K, 4)
    for mode, M in MODES:
        say(f"cancelling partials: {fmt} N={N} K={K} {mode} M={M}")
        x = np.full((M, K), 2.0 ** -6, dtype=np.float16)
        y = run(bgg, torch, d, x, mode, rotate=False)
        assert np.array_equal(y, np.broadcast_to(want, y.shape)), f"{mode} M={M}"
        ref = oracle_y(fmt, T[rows], S[rows], x[:1], rotate=False)
        assert np.array_equal(ref[0].astype(np.float16), want[rows])


@pytest.mark.parametrize("fmt", FMTS + ("Q1_0", "Q2_0_G64"))
@pytest.mark.parametrize("N,K", SHAPES)
def test_non_finite_activations(env, fmt, N, K):
    """A NaN, +inf or -inf in one position of a token's x: that token's y
    row is NaN throughout (the oracle's is non-finite throughout); every
    other token of the call keeps the bits it has without the bad token."""
    bgg, torch = env
    T, S = gen_matrix(231, 1, N, K, fmt=fmt)
    d = Dev(bgg, torch, fmt, T, S)
    rows = sample_rows(N, K, 5)
    rng = np.random.default_rng(14)
    for mode, M in MODES:
        x0 = synth.activations_f16(231, 2, M, K)
        y0 = run(bgg, torch, d, x0, mode)
        for bad in (np.nan, np.inf, -np.inf):
            for rotate in (True, False):
                say(f"non-finite x ({bad}, transform {rotate}): {fmt} N={N} K={K} {mode} M={M}")
                x = x0.copy()
                m = int(rng.integers(0, M))
                x[m, int(rng.integers(0, K))] = bad
                y = run(bgg, torch, d, x, mode, rotate)
                assert np.isnan(y[m]).all(), f"token {m}"
                ref = oracle_y(fmt, T[rows], S[rows], x[m:m + 1], rotate=rotate)
                assert not np.isfinite(ref).any()
                if rotate:
                    others = [i for i in range(M) if i != m]
                    assert np.array_equal(y[others].view(np.uint16), y0[others].view(np.uint16))
