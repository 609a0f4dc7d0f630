"""Float64 reference of one Muon optimizer step (test infrastructure only).

Every function takes and returns float64 NumPy arrays.  Inputs are upcast
exactly from whatever the GPU receives (float32 or bfloat16 values), so the only
rounding in here is float64 rounding.  Nothing is blocked, fused or reordered
beyond what the cited definitions state; matrix products use NumPy's ``@``.

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes of the repository):

* Nesterov uses the *updated* buffer: the blog's VanillaMuon updates ``buf``
  before forming the update, and the training guide defines the Nesterov input
  as ``grad + mu * buf``.
* The normalisation epsilon is added to the Frobenius norm (the blog's code
  divides by ``norm + 1e-7``; its equation shows no epsilon).
* Transposition happens strictly when rows > cols.
* Matrices with fewer than 100,000 elements skip Newton-Schulz and use the
  momentum input directly, as the blog's VanillaMuon does for non-matrix
  parameters and as the training guide's predicate excludes them from NS.
* Custom Newton-Schulz coefficients (the training guide's ``ns_backend`` row:
  a ``NewtonSchulz(...)`` object "to customise the coefficients", none printed)
  are read as the odd matrix polynomial that generalises the blog's cubic map:
  X <- sum_j c_j (X X^T)^j X, with (c0, c1) = (1.5, -0.5) the blog's own map.
  A schedule may give one coefficient set per step.
* Weight decay (the training guide's ``weight_decay`` argument, form unstated)
  is decoupled and uses the unscaled learning rate:
  p <- p * (1 - lr * wd) - lr * s * U.
* Gradient clipping (training guide, "梯度裁剪") follows the global p-norm rule
  of torch.nn.utils.clip_grad_norm_, which the guide names for the other
  parameters, applied per segment.
* The AdamW route for non-matrix parameters ("standard" in the training guide)
  follows PyTorch's AdamW: decoupled decay, bias-corrected moments, eps added
  after the bias-corrected square root, step counted from 1.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

# Blog post, section "代码实现": the normalisation divides by (norm + 1e-7).
EPS = 1e-7
# Training guide, section "编写 Predicate": p.numel() < 100_000 is "too small,
# NS has no benefit".
MIN_NS_NUMEL = 100_000


def _f64_2d(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    if a.ndim != 2:
        # Blog post, section "常见错误" (mistake 2): NS is only defined on 2-D
        # matrices; a bias vector must be rejected.
        raise ValueError(f"expected a 2-D matrix, got shape {a.shape}")
    return a


def frobenius_norm(x: np.ndarray) -> float:
    """sqrt of the sum of squares of all entries (the ||G||_F of the blog's
    normalisation equation)."""
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.sum(x * x)))


# Blog post, "Muon 核心" equation: G_{t+1} = 1.5 G_t - 0.5 G_t G_t^T G_t.
CUBIC = (1.5, -0.5)


def coefficient_schedule(coeffs, steps: int) -> list:
    """Per-step coefficient tuples: None -> the cubic map at every step; one
    sequence of numbers -> that polynomial at every step; a sequence of
    ``steps`` sequences -> one polynomial per step."""
    if coeffs is None:
        return [CUBIC] * steps
    coeffs = list(coeffs)
    if coeffs and all(np.ndim(c) == 0 for c in coeffs):
        one = tuple(float(c) for c in coeffs)
        if len(one) < 2:
            raise ValueError("a Newton-Schulz polynomial needs at least two coefficients")
        return [one] * steps
    if len(coeffs) != steps:
        raise ValueError(f"a per-step schedule needs {steps} coefficient sets, got {len(coeffs)}")
    out = [tuple(float(c) for c in row) for row in coeffs]
    if any(len(row) < 2 for row in out):
        raise ValueError("a Newton-Schulz polynomial needs at least two coefficients")
    return out


def newton_schulz(g, steps: int, coeffs=None) -> np.ndarray:
    """Newton-Schulz orthogonalisation.

    Blog post, section "Muon 核心：Newton-Schulz 迭代": the input is scaled to
    unit Frobenius norm and then mapped ``steps`` times by the odd polynomial
    G <- 1.5 G - 0.5 (G G^T) G, whose cost is two matrix products per step
    (the Gram matrix A = G G^T, then A G).  The same section's implementation
    notes fix three details: a matrix with more rows than columns is iterated
    as its transpose (so A is the smaller square) and transposed back at the
    end, and the norm in the scaling carries +1e-7.

    ``coeffs`` replaces the cubic's (1.5, -0.5) by another odd polynomial
    (training guide, ``ns_backend`` row): each step maps X to
    sum_j c_j A^j X with A = X X^T, the powers formed by repeated products
    A (A^(j-1) X).  The cubic is the case (c0, c1) = (1.5, -0.5).
    """
    g = _f64_2d(g)
    if steps < 0:
        raise ValueError("steps must be >= 0")
    rows, cols = g.shape
    transposed = rows > cols
    x = g.T if transposed else g
    x = x / (frobenius_norm(x) + EPS)
    for c in coefficient_schedule(coeffs, steps):
        a = x @ x.T
        term = x
        y = c[0] * x
        for cj in c[1:]:
            term = a @ term
            y = y + cj * term
        x = y
    return x.T if transposed else x


def momentum_update(buf, grad, mu: float) -> np.ndarray:
    """buf <- mu * buf + grad (blog post, ``VanillaMuon.step``: mul_ then add_)."""
    return mu * np.asarray(buf, dtype=np.float64) + np.asarray(grad, dtype=np.float64)


def ns_input(grad, buf_new, mu: float, nesterov: bool) -> np.ndarray:
    """Matrix fed to Newton-Schulz.

    Training guide, hyper-parameter table, ``nesterov``: ns_input = grad + mu * buf
    (with the buffer already updated this step).  Without Nesterov the buffer
    itself is used, as in the blog's VanillaMuon.
    """
    buf_new = np.asarray(buf_new, dtype=np.float64)
    if nesterov:
        return np.asarray(grad, dtype=np.float64) + mu * buf_new
    return buf_new


def muon_direction(y, steps: int, coeffs=None) -> np.ndarray:
    """Update direction U for one matrix: NS(y), or y itself when the matrix is
    below the NS size threshold (blog VanillaMuon's non-matrix branch applied
    to the training guide's numel < 100,000 exclusion)."""
    y = _f64_2d(y)
    if y.size < MIN_NS_NUMEL:
        return y.copy()
    return newton_schulz(y, steps, coeffs)


def apply_update(p, u, lr: float, lr_scale: float = 1.0, weight_decay: float = 0.0) -> np.ndarray:
    """p <- p - lr * scale * U (blog VanillaMuon: p.add_(update, alpha=-lr)),
    after the decoupled decay p <- p * (1 - lr * weight_decay) when the
    training guide's ``weight_decay`` is non-zero."""
    p = np.asarray(p, dtype=np.float64)
    if weight_decay != 0.0:
        p = p * (1.0 - lr * weight_decay)
    return p - (lr * lr_scale) * np.asarray(u, dtype=np.float64)


def moonlight_lr_scale(rows: int, cols: int) -> float:
    """Per-parameter learning-rate multiplier 0.2 * sqrt(max(m, n)) named in the
    training guide's hyper-parameter table (``lr`` row)."""
    return 0.2 * float(np.sqrt(max(rows, cols)))


def muon_step(params: Sequence[np.ndarray], grads: Sequence[np.ndarray], bufs: Sequence[np.ndarray],
              mu: float, nesterov: bool, steps: int, lr: float,
              lr_scale: Optional[Sequence[float]] = None, weight_decay: float = 0.0,
              moonlight: bool = False, ns_coeffs=None
              ) -> Tuple[list, list, list, list]:
    """One Muon step over a list of matrices, each independent of the others.

    The per-matrix learning-rate multiplier is lr_scale[i] (1 when absent),
    times 0.2 * sqrt(max(rows, cols)) when ``moonlight`` is set.
    Returns (new_params, new_bufs, updates, norms) where ``updates`` are the U
    matrices (in each parameter's own orientation) and ``norms`` are
    ||ns_input||_F per matrix.
    """
    out_p, out_b, out_u, norms = [], [], [], []
    for i, (p, g, b) in enumerate(zip(params, grads, bufs)):
        g = _f64_2d(g)
        b_new = momentum_update(b, g, mu)
        y = ns_input(g, b_new, mu, nesterov)
        u = muon_direction(y, steps, ns_coeffs)
        s = 1.0 if lr_scale is None else float(lr_scale[i])
        if moonlight:
            s *= moonlight_lr_scale(*g.shape)
        out_p.append(apply_update(p, u, lr, s, weight_decay))
        out_b.append(b_new)
        out_u.append(u)
        norms.append(frobenius_norm(y))
    return out_p, out_b, out_u, norms


# Training guide, "梯度裁剪": the Muon-only clip follows the global p-norm rule
# of torch.nn.utils.clip_grad_norm_ (which the guide uses for the other
# parameters), with the +1e-6 and the clamp at 1 of that rule.
CLIP_EPS = 1e-6


def clip_grad_norm_buckets(grads: Sequence[np.ndarray], segments: Sequence[int], max_norms: Sequence[float],
                           norm_type: float = 2.0) -> Tuple[list, list]:
    """Per-segment global p-norm gradient clipping.

    Training guide, "梯度裁剪": clipping happens before momentum and
    Newton-Schulz; the fused bucketed form computes each segment's norm, clip
    coefficient and in-place scaling while "keeping per-segment semantics".
    Segment s holds the tensors i with segments[i] == s:

        total_s = (sum_{i in s} sum |g_i|^p)^(1/p)   (max |g_i| for p = inf)
        coef_s  = min(max_norm_s / (total_s + 1e-6), 1)
        g_i    <- coef_s * g_i

    Returns (clipped grads, per-segment totals).
    """
    p = float(norm_type)
    if not (p > 0.0):
        raise ValueError("norm_type must be positive (or inf)")
    gs = [np.asarray(g, dtype=np.float64) for g in grads]
    nseg = len(max_norms)
    if any(not 0 <= int(sg) < nseg for sg in segments) or len(segments) != len(gs):
        raise ValueError("every gradient needs a segment index in [0, len(max_norms))")
    totals = []
    for s in range(nseg):
        members = [g for g, sg in zip(gs, segments) if int(sg) == s]
        if np.isinf(p):
            totals.append(max([float(np.max(np.abs(g))) for g in members if g.size] or [0.0]))
        else:
            totals.append(float(sum(float(np.sum(np.abs(g) ** p)) for g in members) ** (1.0 / p)))
    out = []
    for g, sg in zip(gs, segments):
        s = int(sg)
        coef = min(float(max_norms[s]) / (totals[s] + CLIP_EPS), 1.0)
        out.append(g * coef)
    return out, totals


def adamw_step(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW step for a non-matrix parameter (training guide: group 1,
    "AdamW — 标准", with ``adamw_lr``, ``adamw_betas``, ``adamw_eps`` and
    ``adamw_weight_decay``; blog post, section "为什么需要矩阵感知优化器",
    whose update subtracts alpha m_hat / (sqrt(v_hat) + eps) with
    bias-corrected moments).  "Standard" is read as PyTorch's AdamW:

        p <- p (1 - lr wd)
        m <- beta1 m + (1 - beta1) g
        v <- beta2 v + (1 - beta2) g^2
        p <- p - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)

    with the step counter t = ``step`` >= 1.  Returns (p, m, v).
    """
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * weight_decay)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    denom = np.sqrt(v) / np.sqrt(bc2) + eps
    return p - (lr / bc1) * m / denom, m, v


def orthogonality_error(x) -> float:
    """||X X^T - I||_F, taken on the wide orientation of X.

    Blog post, section "调试技巧" (``check_orthogonality``): the error of an
    orthogonalised update.  For a tall X, X X^T has rank < rows and the error
    could never approach 0, so the product is formed on the side with fewer
    rows.
    """
    x = _f64_2d(x)
    if x.shape[0] > x.shape[1]:
        x = x.T
    return frobenius_norm(x @ x.T - np.eye(x.shape[0]))
