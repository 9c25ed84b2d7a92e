"""GPU parity of the offline front end bgg_rotate_ternarize (float weight
rows -> trits and fp16 scales in the stored coordinates) against the CPU
oracle, on seeded synthetic weights with outliers.  Marked gpu.

Where floating point decides an integer the two sides can differ only at
the decision boundary: the kernel rotates in fp32 butterflies and the
oracle in fp64.  So
  * a scale must equal the oracle's, except in a group whose exact mean
    magnitude lies within 1e-5 (relative) of a point halfway between two
    fp16 values, where the other neighbour is also correct;
  * a trit must equal the oracle's, except where 2|w'| lies within 1e-5 of
    the group's mean-magnitude sum of the scale; in a group whose scale
    took the other neighbour each trit must be the nearest of -s, 0, +s
    for the kernel's own scale s (same boundary allowance).
Such cases are counted and must stay rare.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_helpers import TOL, Dev, oracle_y, relerr  # noqa: E402


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need the GPU"
    import bit_gemv_gemm_amd as bgg
    return bgg, torch


def run_kernel(bgg, torch, W):
    N, K = W.shape
    wd = torch.from_numpy(np.ascontiguousarray(W)).cuda()
    td = torch.full((N, K), 7, dtype=torch.int8, device="cuda")
    sd = torch.full((N, K // 128), float("nan"), dtype=torch.float16, device="cuda")
    bgg.bgg_rotate_ternarize(wd, N, K, td, sd)
    torch.cuda.synchronize()
    return td.cpu().numpy(), sd.cpu().numpy()


def rotated_f64(W):
    """W blockdiag(H_128/sqrt(128)) in fp64 from scipy's Hadamard matrix (used
    only to find the decision boundaries)."""
    import scipy.linalg
    Hn = scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128.0)
    N, K = W.shape
    return (W.astype(np.float64).reshape(N, K // 128, 128) @ Hn).reshape(N, K)


def f16_midpoint_near(mean, rel=1e-5):
    """True where mean lies within rel of the midpoint between two fp16s."""
    h = mean.astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    hf = h.astype(np.float64)
    mids = np.stack([(hf + up) / 2, (hf + dn) / 2])
    return np.any(np.abs(mids - mean) <= rel * np.abs(mean), axis=0)


def check_against_oracle(W, Tk, Sk, To, So):
    N, K = W.shape
    G = K // 128
    Wr = rotated_f64(W).reshape(N, G, 128)
    mean = np.abs(Wr).mean(axis=2)
    sk = Sk.view(np.uint16)
    so = So.view(np.uint16)
    diff_s = sk != so
    assert np.all(~diff_s | f16_midpoint_near(mean)), "a scale differs away from a rounding midpoint"
    assert np.all(np.abs(sk.astype(np.int32) - so.astype(np.int32))[diff_s] <= 1)
    # trits: the oracle's where the scales agree, else nearest for the kernel's scale
    s_used = np.where(diff_s, Sk.astype(np.float64), So.astype(np.float64))[:, :, None]
    want = np.where(diff_s[:, :, None],
                    np.where(2 * np.abs(Wr) > s_used, np.sign(Wr), 0).astype(np.int8),
                    To.reshape(N, G, 128))
    tk = Tk.reshape(N, G, 128)
    near = np.abs(2 * np.abs(Wr) - s_used) <= 1e-5 * np.abs(Wr).sum(axis=2, keepdims=True) / 64
    bad = (tk != want) & ~near
    assert not bad.any(), f"{bad.sum()} trits differ away from the decision boundary"
    assert np.all(np.isin(Tk, (-1, 0, 1)))
    n_amb = int(diff_s.sum()) + int(((tk != want) & near).sum())
    assert n_amb <= max(2, N * K // 1000), n_amb
    return n_amb


@pytest.mark.parametrize("N,K", [(1, 128), (3, 384), (100, 640), (130, 1152), (64, 6144),
                                 (1000, 5120), (257, 17408)])
def test_ternarize_parity(env, N, K):
    bgg, torch = env
    say(f"ternarize N={N} K={K}")
    W = synth.float_weights(17, 3, N, K)
    Tk, Sk = run_kernel(bgg, torch, W)
    To, So = oracle.ternarize(W)
    n = check_against_oracle(W, Tk, Sk, To, So)
    say(f"  boundary cases {n}; non-zero rate {np.mean(Tk != 0):.3f}")


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_ternarize_full_size_sampled_rows(env, name):
    """The projection shapes whole on the GPU; every 97th row (and the last)
    checked against the oracle, regenerated from its own seed."""
    bgg, torch = env
    w = synth.WORKLOADS["projection"]
    mat = [m for m in w["matrices"] if m.name == name][0]
    say(f"ternarize full {name} {mat.n}x{mat.k}")
    W = synth.float_weights(w["seed"], mat.matrix_id, mat.n, mat.k)
    Tk, Sk = run_kernel(bgg, torch, W)
    rows = np.unique(np.concatenate([np.arange(0, mat.n, 97), [mat.n - 1]]))
    Ws = synth.float_weights(w["seed"], mat.matrix_id, 1, mat.k, row0=0)
    assert np.array_equal(Ws[0], W[0])
    To, So = oracle.ternarize(W[rows])
    check_against_oracle(W[rows], Tk[rows], Sk[rows], To, So)


def test_ternarize_closed_forms(env):
    """c times Sylvester row r in block b -> one trit sign(c) at r and the
    scale fp16(|c|); zero rows -> zero trits and scales (no oracle)."""
    import scipy.linalg
    bgg, torch = env
    H = scipy.linalg.hadamard(128)
    K = 640
    cases = [(b, r, c) for b in range(5) for r, c in ((0, 0.25), (77, -1.5), (127, 0.0078125))]
    W = np.zeros((len(cases) + 2, K), np.float32)
    for n, (b, r, c) in enumerate(cases):
        W[n, 128 * b:128 * b + 128] = (c * math.sqrt(128.0)) * H[r]
    Tk, Sk = run_kernel(bgg, torch, W)
    for n, (b, r, c) in enumerate(cases):
        want = np.zeros(K, np.int8)
        want[128 * b + r] = 1 if c > 0 else -1
        assert np.array_equal(Tk[n], want), n
        assert Sk[n, b] == np.float16(abs(c))
        assert not np.any(Sk[n, np.arange(5) != b].view(np.uint16))
    assert not Tk[len(cases):].any() and not Sk[len(cases):].view(np.uint16).any()


def test_front_end_to_gemv(env):
    """float W -> GPU trits and scales -> host packing (both packings) ->
    GEMV: y matches the oracle's chain (oracle trits, oracle packing, oracle
    layer), and approximates the float layer W x."""
    bgg, torch = env
    N, K, M = 1000, 5120, 2
    say("front end -> pack -> gemv")
    W = synth.float_weights(23, 5, N, K)
    Tk, Sk = run_kernel(bgg, torch, W)
    To, So = oracle.ternarize(W)
    x = synth.activations_f16(23, 6, M, K)
    exact = x.astype(np.float64) @ W.astype(np.float64).T
    for fmt in ("PQ2_0", "PTQ1_0"):
        y = Dev(bgg, torch, fmt, Tk, Sk).gemv(x)
        ref = oracle_y(fmt, To, So, x)
        e = relerr(y, ref)
        say(f"  {fmt} rel err vs oracle chain {e.max():.3g}; vs float layer "
            f"{relerr(y, exact).max():.3g}")
        assert np.all(e <= TOL)
        # ternary weights are an approximation of W: the product keeps most of it
        cos = np.sum(y * exact, axis=1) / (np.linalg.norm(y, axis=1) * np.linalg.norm(exact, axis=1))
        assert np.all(cos > 0.7), cos


def test_ternarize_errors(env):
    bgg, torch = env
    w = torch.zeros((4, 256), dtype=torch.float32, device="cuda")
    t = torch.zeros((4, 256), dtype=torch.int8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.float16, device="cuda")
    bgg.bgg_rotate_ternarize(w, 0, 256, t, s)        # N == 0: no-op
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_rotate_ternarize(w.view(-1)[:4 * 192].view(4, 192), 4, 192, t, s)
    assert e.value.status == 3
    wm = torch.zeros(4 * 256 + 4, dtype=torch.float32, device="cuda")[1:1 + 4 * 256]
    with pytest.raises(bgg.BggError) as e:
        bgg.bgg_rotate_ternarize(wm, 4, 256, t, s)
    assert e.value.status == 6
