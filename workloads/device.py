"""Full-size synthetic matrix sets allocated and filled on the GPU.

Values come from torch's seeded device generator (seed 42) with the set's
distributions; they are not bit-identical to the host streams of ``gen.py``.
Matrices listed in ``host_indices`` are instead filled with their host-stream
values, so tests can run a whole set in one call and compare those matrices
with the CPU oracle.  No method arithmetic happens here.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import numpy as np
import torch

from .configs import ROOT_SEED, SetConfig
from . import gen

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _to_device(d: gen.Drawn, device) -> torch.Tensor:
    if d.bits is None:
        return torch.from_numpy(np.ascontiguousarray(d.values)).to(device)
    return torch.from_numpy(np.ascontiguousarray(d.bits).view(np.int16)).to(device).view(torch.bfloat16)


def _grad_on_device(cfg: SetConfig, shape, g: torch.Generator, device) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if cfg.grad_dist == "student_t3":
        # Student-t with 3 degrees of freedom: Z / sqrt(chi^2_3 / 3)
        chi = torch.randn((3,) + tuple(shape), generator=g, device=device).pow_(2).sum(0).div_(3.0).sqrt_()
        x.div_(chi)
        del chi
    if cfg.grad_scale != 1.0:
        x.mul_(cfg.grad_scale)
    return x.to(_TORCH_DT[cfg.dtype])


def make_set(cfg: SetConfig, device="cuda", host_indices: Optional[Iterable[int]] = None,
             seed: int = ROOT_SEED) -> Dict[str, List]:
    """params, grads (set dtype) and zero fp32 momentum for every matrix.

    Returns {"params", "grads", "momentum", "host": {index: (grad Drawn, weight Drawn)}}.
    """
    host_indices = set(host_indices or ())
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    params, grads, moms, host = [], [], [], {}
    for i, spec in enumerate(cfg.matrices):
        shape = (spec.rows, spec.cols)
        if i in host_indices:
            dg = gen.draw_matrix(cfg, i, gen.GRAD)
            dw = gen.draw_matrix(cfg, i, gen.WEIGHT)
            host[i] = (dg, dw)
            grads.append(_to_device(dg, device))
            params.append(_to_device(dw, device))
        else:
            grads.append(_grad_on_device(cfg, shape, g, device))
            w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            if cfg.weight_scale not in (0.0, 1.0):
                w.mul_(cfg.weight_scale)
            params.append(w.to(_TORCH_DT[cfg.dtype]))
        moms.append(torch.zeros(shape, device=device, dtype=torch.float32))
    return {"params": params, "grads": grads, "momentum": moms, "host": host}
