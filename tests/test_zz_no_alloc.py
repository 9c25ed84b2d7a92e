"""bgg_ternary_gemv_noalloc (workspace in a static device array) against
bgg_ternary_gemv with a caller's workspace, through the C ABI: the same
kernels, so the same bits, and both within the bar of the oracle.  Two calls
in a row, the second on a smaller input, then the first again (each call
must find the row words of split-K launches zero)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from gpu_helpers import TOL, Dev, gen_matrix, oracle_y, relerr  # noqa: E402


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import bit_gemv_gemm_amd as bgg
    return bgg, torch


def _both(bgg, torch, d, x, flags):
    M = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    ya = torch.full((M, d.N), float("nan"), dtype=torch.float16, device="cuda")
    yb = torch.full((M, d.N), float("nan"), dtype=torch.float16, device="cuda")
    bgg.bgg_ternary_gemv_noalloc(d.desc, d.packed, xd, ya, M, flags)
    ws = bgg.workspace(bgg.bgg_gemv_workspace_size(d.desc, M))
    bgg.bgg_ternary_gemv(d.desc, d.packed, xd, yb, M, flags, ws)
    torch.cuda.synchronize()
    return ya.cpu().numpy(), yb.cpu().numpy()


@pytest.mark.parametrize("fmt", ("PQ2_0", "PTQ1_0", "Q1_0", "Q2_0_G64"))
@pytest.mark.parametrize("M", (1, 3, 9))
def test_noalloc_matches_workspace_entry(env, fmt, M):
    bgg, torch = env
    flags = bgg.BGG_ROTATE_INPUT
    # a long K (split over workgroups: the row words are used), then a
    # smaller matrix and token count, then the first one again
    shapes = [(5120, 17408, M), (300, 640, max(1, M - 1)), (5120, 17408, M)]
    for i, (N, K, m) in enumerate(shapes):
        say(f"noalloc {fmt} call {i}: N={N} K={K} M={m}")
        T, S = gen_matrix(131, 1 + (i % 2), N, K, fmt=fmt)
        d = Dev(bgg, torch, fmt, T, S)
        x = synth.activations_f16(131, 2 + i, m, K)
        ya, yb = _both(bgg, torch, d, x, flags)
        assert not np.isnan(ya).any()
        assert np.array_equal(ya.view(np.uint16), yb.view(np.uint16)), f"call {i}"
        rows = np.arange(N) if N * K <= 1 << 20 else np.random.default_rng(i).choice(N, 32, replace=False)
        ref = oracle_y(fmt, T[rows], S[rows], x)
        assert np.all(relerr(ya[:, rows], ref) <= TOL), f"call {i}"


def test_noalloc_rejects_beyond_its_workspace(env):
    bgg, torch = env
    d = bgg.bgg_describe("PQ2_0", 128, 516096)
    assert bgg.bgg_gemv_workspace_size(d, 16) > 32 << 20
    x = torch.zeros((16, 516096), dtype=torch.float16, device="cuda")
    y = torch.zeros((16, 128), dtype=torch.float16, device="cuda")
    packed = torch.zeros(d.total_bytes, dtype=torch.uint8, device="cuda")
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_ternary_gemv_noalloc(d, packed, x, y, 16, bgg.BGG_ROTATE_INPUT)
    assert e.value.status == 3 and "static workspace" in str(e.value)
