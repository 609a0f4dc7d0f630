"""CPU oracle for the batched Muon step -- TEST INFRASTRUCTURE, not product code.

A plain, slow, float64 NumPy restatement of what the DMuon pages define:

* blog post "DMuon：让矩阵正交化优化器达到接近 AdamW 的分布式训练开销",
  section "Muon 核心：Newton-Schulz 迭代" (normalisation equation, cubic map,
  the ``newton_schulz`` description) and section "代码实现" (``VanillaMuon``:
  momentum buffer, non-matrix branch, weight update);
* DMuon training guide "训练指南", hyper-parameter table ("超参数指南":
  ``nesterov`` -- ns_input = grad + mu * buf; ``lr`` per-parameter scaling) and
  the predicate section ("编写 Predicate": ``numel() < 100_000`` exclusion).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The GPU library never
calls it and shares no code with it; the two meet only in the seeded input
generators of the ``workloads`` package.

Parity pins (tests/test_oracle_pins.py) tie every function here to something
other than itself: closed-form spectra, brute-force loops, the SVD polar factor,
geometric-series momentum, hand-worked fixtures in tests/golden/.
"""
from .muon import (  # noqa: F401
    CLIP_EPS,
    CUBIC,
    EPS,
    adamw_step,
    MIN_NS_NUMEL,
    apply_update,
    clip_grad_norm_buckets,
    coefficient_schedule,
    frobenius_norm,
    momentum_update,
    moonlight_lr_scale,
    muon_direction,
    muon_step,
    newton_schulz,
    ns_input,
    orthogonality_error,
)
