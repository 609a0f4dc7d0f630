"""Seeded generators for the synthetic matrix sets.

Every tensor is drawn from its own NumPy PCG64 stream, seeded by
``SeedSequence([42, cfg_id, matrix_index, kind])``.  A matrix's values therefore
do not depend on which other matrices are generated or in what order, so a test
can regenerate any single matrix of a large set on the host.

The only arithmetic here is the construction of inputs: Gaussian / Student-t
draws, Haar-distributed orthonormal factors for spectrum-controlled matrices,
and round-to-nearest-even encoding of float32 values as bfloat16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

from .configs import ROOT_SEED, SetConfig

# stream kinds
GRAD = 0
WEIGHT = 1
MOMENTUM = 2
GRAD2 = 3
SPEC_LEFT = 4
SPEC_RIGHT = 5
SPEC_SIGMA = 6


def stream(cfg_id: int, index: int, kind: int) -> np.random.Generator:
    """Independent PCG64 stream for one (set, matrix, tensor kind)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg_id, index, kind])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaNs map to a quiet NaN.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Drawn:
    """One synthetic tensor as the GPU receives it.

    ``values`` holds the exact float32 value of every element (for bfloat16
    tensors, the value of the rounded bit pattern); ``bits`` holds the uint16
    patterns for bfloat16 tensors and is None for float32 ones.
    """
    values: np.ndarray
    bits: Optional[np.ndarray]
    dtype: str

    def as_f64(self) -> np.ndarray:
        return self.values.astype(np.float64)


def encode(values_f32: np.ndarray, dtype: str) -> Drawn:
    values_f32 = np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == "f32":
        return Drawn(values_f32, None, "f32")
    if dtype == "bf16":
        bits = f32_to_bf16_bits(values_f32)
        return Drawn(bf16_bits_to_f32(bits), bits, "bf16")
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape: Tuple[int, int], std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _student_t3(rng: np.random.Generator, shape: Tuple[int, int], scale: float) -> np.ndarray:
    return (rng.standard_t(3.0, size=shape) * scale).astype(np.float32)


def draw_matrix(cfg: SetConfig, index: int, kind: int, dtype: Optional[str] = None) -> Drawn:
    """Draw matrix ``index`` of ``cfg`` for the given tensor kind.

    GRAD / GRAD2 follow the set's gradient distribution; WEIGHT is
    N(0, weight_scale^2); MOMENTUM is N(0, grad_scale^2) (used only by tests that
    start from a non-zero momentum state).  Spectrum sets are drawn with
    :func:`spectrum_matrix`.
    """
    spec = cfg.matrices[index]
    shape = (spec.rows, spec.cols)
    dtype = dtype or cfg.dtype
    rng = stream(cfg.cfg_id, index, kind)
    if kind in (GRAD, GRAD2):
        if cfg.grad_dist == "normal":
            v = _normal(rng, shape, cfg.grad_scale)
        elif cfg.grad_dist == "student_t3":
            v = _student_t3(rng, shape, cfg.grad_scale)
        elif cfg.grad_dist == "spectrum":
            v = spectrum_matrix(cfg.cfg_id, index, spec.rows, spec.cols)[0].astype(np.float32)
        else:
            raise ValueError(cfg.grad_dist)
        return encode(v, dtype)
    if kind == WEIGHT:
        return encode(_normal(rng, shape, cfg.weight_scale if cfg.weight_scale else 1.0), dtype)
    if kind == MOMENTUM:
        return encode(_normal(rng, shape, cfg.grad_scale), "f32")
    raise ValueError(kind)


def haar_orthonormal(rng: np.random.Generator, n: int, r: int) -> np.ndarray:
    """n x r matrix with Haar-distributed orthonormal columns (r <= n).

    QR of a Gaussian matrix, with the signs of R's diagonal folded into Q so the
    distribution is exactly Haar (Mezzadri, "How to generate random matrices
    from the classical compact groups", 2007).
    """
    z = rng.standard_normal((n, r))
    q, rr = np.linalg.qr(z)
    d = np.sign(np.diag(rr))
    d[d == 0] = 1.0
    return q * d[None, :]


def spectrum_matrix(cfg_id: int, index: int, rows: int, cols: int,
                    log10_range: Tuple[float, float] = (-3.0, 0.0),
                    sigma: Optional[np.ndarray] = None):
    """Float64 matrix ``L diag(s) R^T`` with Haar-random orthonormal L, R.

    ``s`` is drawn i.i.d. log-uniform on [10^lo, 10^hi] unless given.  Returns
    ``(G, L, s, R)`` with G of shape (rows, cols), L (rows x r), R (cols x r),
    r = min(rows, cols).
    """
    r = min(rows, cols)
    left = haar_orthonormal(stream(cfg_id, index, SPEC_LEFT), rows, r)
    right = haar_orthonormal(stream(cfg_id, index, SPEC_RIGHT), cols, r)
    if sigma is None:
        lo, hi = log10_range
        sigma = 10.0 ** stream(cfg_id, index, SPEC_SIGMA).uniform(lo, hi, size=r)
    sigma = np.asarray(sigma, dtype=np.float64)
    g = (left * sigma[None, :]) @ right.T
    return g, left, sigma, right


def spectrum_copies(g64: np.ndarray) -> Tuple[Drawn, Drawn]:
    """fp32 copy = RNE(fp64); bf16 copy = RNE(fp32 copy)."""
    f32 = encode(g64.astype(np.float32), "f32")
    return f32, encode(f32.values, "bf16")
