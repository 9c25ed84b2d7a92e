"""Helpers for the GPU tests: run the library through its C ABI on seeded
synthetic inputs and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = 2e-3  # max relative error of y, per token row (see relerr)


def relerr(y, ref) -> np.ndarray:
    """Per token row: max_n |y - ref| / max_n |ref|."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return np.max(np.abs(y - ref), axis=-1) / den


def gen_matrix(seed, mid, N, K, row0=0, fmt="PQ2_0"):
    """Seeded weights and scales of a matrix stored in format fmt (signs for
    Q1_0, trits otherwise; a scale per 64 weights for Q2_0_G64)."""
    return (synth.weights(fmt, seed, mid, N, K, row0),
            synth.scales_f16(seed, mid, N, K, row0, group=synth.scale_group(fmt)))


class Dev:
    """Device copies of one packed matrix."""

    def __init__(self, bgg, torch, fmt, T, S, device="cuda"):
        self.bgg, self.torch = bgg, torch
        self.fmt = fmt
        self.N, self.K = T.shape
        self.desc = bgg.bgg_describe(fmt, self.N, self.K)
        self.packed = bgg.upload(bgg.bgg_pack_weights(self.desc, T, S), device)
        self.device = device

    def gemv(self, x_f16: np.ndarray, rotate=True, ws=None):
        bgg, torch = self.bgg, self.torch
        M = x_f16.shape[0]
        xd = torch.from_numpy(np.ascontiguousarray(x_f16)).to(self.device)
        yd = torch.full((M, self.N), float("nan"), dtype=torch.float16, device=self.device)
        if ws is None:
            ws = bgg.workspace(bgg.bgg_gemv_workspace_size(self.desc, M), self.device)
        bgg.bgg_ternary_gemv(self.desc, self.packed, xd, yd, M,
                             bgg.BGG_ROTATE_INPUT if rotate else 0, ws)
        torch.cuda.synchronize()
        return yd.cpu().numpy()

    def gemm(self, x_f16: np.ndarray, rotate=True):
        bgg, torch = self.bgg, self.torch
        M = x_f16.shape[0]
        xd = torch.from_numpy(np.ascontiguousarray(x_f16)).to(self.device)
        yd = torch.full((M, self.N), float("nan"), dtype=torch.float16, device=self.device)
        ws = bgg.workspace(bgg.bgg_gemm_workspace_size(self.desc, M), self.device) if rotate else None
        bgg.bgg_ternary_gemm(self.desc, self.packed, xd, yd, M,
                             bgg.BGG_ROTATE_INPUT if rotate else 0, ws)
        torch.cuda.synchronize()
        return yd.cpu().numpy()


def oracle_y(fmt, T, S, x, rotate=True):
    return oracle.linear(fmt, oracle.pack(fmt, T), S, x, rotate=rotate)
