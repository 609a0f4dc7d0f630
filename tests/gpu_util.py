"""Helpers for GPU parity tests: moving seeded inputs to the device and
comparing results with the oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

from workloads.gen import Drawn, bf16_bits_to_f32

TOL = {"f32": 1e-4, "bf16": 2e-2}   # relative Frobenius error of U
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(d: Drawn) -> torch.Tensor:
    if d.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(d.values)).cuda()
    return torch.from_numpy(np.ascontiguousarray(d.bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / (den if den > 0 else 1.0))


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the dtype's grid at |x| (bf16: 8 significant bits)."""
    bits = 24 if dtype == "f32" else 8
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.exp2(e - (bits - 1))


def check_update_faithful(p_new: np.ndarray, p_old: np.ndarray, u_gpu: np.ndarray, lr: float, scale: float,
                          dtype: str, weight_decay: float = 0.0) -> None:
    """p_new must round p_old (1 - lr wd) - lr*scale*U (with the GPU's own U)
    to within one ulp of the parameter dtype.  With decay, the fp32 decay
    factor and the product p * factor are each rounded once more: 3 * 2^-24 |p|
    covers both."""
    step = float(np.float32(-np.float32(lr) * np.float32(scale)))
    decay = 1.0 - float(np.float32(lr)) * float(np.float32(weight_decay))
    exact = p_old * decay + step * u_gpu
    err = np.abs(p_new - exact)
    bound = ulp(exact, dtype)
    if weight_decay != 0.0:
        bound = bound + 3.0 * 2.0 ** -24 * np.abs(p_old)
    bad = err > bound * 1.0000001
    assert not bad.any(), f"{int(bad.sum())} parameter elements off by more than the bound; max err {err.max():.3e}"


def gpu_lr_scale(scale: float, rows: int, cols: int, moonlight: bool) -> float:
    """The per-matrix multiplier as the library forms it in fp32."""
    s = np.float32(scale)
    if moonlight:
        s = np.float32(s * np.float32(0.2 * math.sqrt(max(rows, cols))))
    return float(s)


def f32_mu(mu: float) -> float:
    return float(np.float32(mu))


def max_ulp_err_f32(gpu: np.ndarray, exact: np.ndarray) -> float:
    return float(np.max(np.abs(gpu - exact) / ulp(exact, "f32"))) if gpu.size else 0.0


def fmt(x: float) -> str:
    return f"{x:.3e}" if not math.isnan(x) else "nan"


def worst_tile_error(got: np.ndarray, want: np.ndarray, tile: int = 256):
    """Largest relative Frobenius error over the tile x tile blocks of a
    matrix (ragged edge blocks included), with that block's (row, col) index.
    A single wrong contraction tile barely moves the whole-matrix error of a
    large matrix; it dominates its own block's."""
    got = np.asarray(got)
    want = np.asarray(want)
    worst, where = 0.0, (0, 0)
    for bi in range(0, want.shape[0], tile):
        for bj in range(0, want.shape[1], tile):
            w = want[bi:bi + tile, bj:bj + tile]
            den = float(np.linalg.norm(w))
            err = float(np.linalg.norm(got[bi:bi + tile, bj:bj + tile] - w)) / (den if den > 0 else 1.0)
            if not err <= worst:   # NaN counts as worst
                worst, where = err, (bi // tile, bj // tile)
    return worst, where
