"""Seeded synthetic inputs for the batched Muon step.

This package holds the matrix-set descriptions and the seeded generators that
both the CPU oracle and the GPU path consume.  It contains none of the method's
arithmetic (no momentum, normalisation or Newton-Schulz): only shapes, random
draws and dtype encodings of those draws.
"""
from .configs import CONFIGS, MatrixSpec, SetConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    Drawn,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    draw_matrix,
    haar_orthonormal,
    spectrum_matrix,
    stream,
)
