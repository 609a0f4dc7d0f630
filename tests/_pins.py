"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes the implementation under test as arguments and raises
AssertionError when it disagrees with an independent statement of the result:

* exact rational arithmetic (``fractions.Fraction``) on small integer matrices
  whose Frobenius norm is an integer, so every Newton-Schulz iterate is exact;
* the spectral closed form: an odd matrix polynomial keeps singular vectors, so
  NS_k(L diag(s) R^T) = L diag(f^k(s / (||s|| + eps))) R^T with the scalar map
  f(s) = 1.5 s - 0.5 s^3 (blog post, Newton-Schulz equation);
* the SVD polar factor L R^T as the k -> infinity limit (blog post, "Muon 核心");
* the blog's orthogonality threshold (< 0.01, section "调试技巧") where it
  provably holds: small, well-conditioned matrices;
* geometric-series closed forms of the momentum recurrence;
* hand-worked fixtures in tests/golden/.

``test_oracle_pins.py`` runs them against ``oracle``; ``test_pin_mutants.py``
runs them against deliberately broken copies of the oracle to show that every
planted mistake is caught by at least one pin.
"""
from __future__ import annotations

import math
import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads.gen import haar_orthonormal  # noqa: E402

EPS = 1e-7
EPS_FRAC = Fraction(1, 10**7)


def scalar_map(s: float, k: int) -> float:
    """f applied k times, f(s) = 1.5 s - 0.5 s^3, in plain Python floats."""
    for _ in range(k):
        s = 1.5 * s - 0.5 * s * s * s
    return s


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


# ----------------------------------------------------------------------------- exact
def _isqrt_exact(n: int) -> int:
    r = math.isqrt(n)
    assert r * r == n, "test input must have an integer Frobenius norm"
    return r


def exact_ns(rows, steps):
    """Newton-Schulz over Fractions with explicit loops (no NumPy).

    ``rows`` is a list of lists of ints whose sum of squares is a perfect
    square, so (||G|| + 1e-7) is rational and every iterate is exact.
    """
    g = [[Fraction(v) for v in r] for r in rows]
    m, n = len(g), len(g[0])
    transposed = m > n
    if transposed:
        g = [[g[i][j] for i in range(m)] for j in range(n)]
        m, n = n, m
    ss = sum(int(v) * int(v) for r in rows for v in r)
    scale = Fraction(_isqrt_exact(ss)) + EPS_FRAC
    x = [[v / scale for v in r] for r in g]
    for _ in range(steps):
        a = [[sum(x[i][t] * x[j][t] for t in range(n)) for j in range(m)] for i in range(m)]
        ax = [[sum(a[i][t] * x[t][j] for t in range(m)) for j in range(n)] for i in range(m)]
        x = [[Fraction(3, 2) * x[i][j] - Fraction(1, 2) * ax[i][j] for j in range(n)] for i in range(m)]
    if transposed:
        x = [[x[i][j] for i in range(m)] for j in range(n)]
    return np.array([[float(v) for v in r] for r in x])


EXACT_CASES = [
    [[2, 2, 2], [2, 0, 0]],                # 2x3, ||G|| = 4, rows not orthogonal
    [[2, 2], [2, 0], [2, 0]],              # 3x2 (its transpose pattern, tall route)
    [[0, 3], [4, 0]],                      # 2x2 non-symmetric, ||G|| = 5
    [[1, 2, 2, 0], [0, 1, 0, 2], [4, 0, 1, 1]],  # 3x4, ss = 1+4+4+1+4+16+1+1 = 32 -> not square
]


def pin_exact_rational(ns, steps_list=(0, 1, 2, 3, 4)):
    for case in EXACT_CASES:
        ss = sum(v * v for r in case for v in r)
        if math.isqrt(ss) ** 2 != ss:
            continue
        for k in steps_list:
            want = exact_ns(case, k)
            got = np.asarray(ns(np.array(case, dtype=np.float64), k))
            assert got.shape == want.shape, (case, k, got.shape)
            err = rel_fro(got, want)
            assert err < 1e-14, f"exact NS mismatch case={case} k={k} err={err:.3e}"


# ----------------------------------------------------------------------------- spectral
def _spectral_case(rng, rows, cols, sigma):
    r = min(rows, cols)
    left = haar_orthonormal(rng, rows, r)
    right = haar_orthonormal(rng, cols, r)
    return (left * sigma[None, :]) @ right.T, left, right


def pin_closed_form_spectrum(ns, shapes=((12, 40), (40, 12), (16, 16), (64, 256), (256, 64)),
                             steps_list=(0, 1, 3, 5, 7, 10), seed=7):
    rng = np.random.default_rng(seed)
    for rows, cols in shapes:
        r = min(rows, cols)
        sigma = 10.0 ** rng.uniform(-3.0, 0.0, size=r)
        g, left, right = _spectral_case(rng, rows, cols, sigma)
        s0 = sigma / (float(np.sqrt(np.sum(sigma * sigma))) + EPS)
        for k in steps_list:
            sk = np.array([scalar_map(float(s), k) for s in s0])
            want = (left * sk[None, :]) @ right.T
            got = np.asarray(ns(g, k))
            assert got.shape == want.shape
            err = rel_fro(got, want)
            assert err < 1e-11, f"closed form mismatch {rows}x{cols} k={k}: {err:.3e}"


def pin_flat_recurrence(ns, cases=((4, 12, 5), (8, 24, 5), (16, 40, 6), (256, 1024, 3), (256, 1024, 10))):
    """A flat spectrum of rank r (scaled semi-orthogonal input) starts at
    1/(sqrt(r) + eps) and every singular value follows the scalar map."""
    rng = np.random.default_rng(11)
    for r, n, k in cases:
        q = haar_orthonormal(rng, n, r).T * 3.0   # r x n, all singular values 3
        want = scalar_map(1.0 / (math.sqrt(r) * 3.0 + EPS) * 3.0, k)
        sv = np.linalg.svd(np.asarray(ns(q, k)), compute_uv=False)
        assert np.max(np.abs(sv - want)) < 1e-10, (r, n, k, sv[:3], want)


def pin_monotone(ns, shape=(32, 96), kmax=14, seed=3):
    """||X X^T - I||_F strictly decreases with k while above the rounding floor:
    1 - f(s) = (1 - s)^2 (2 + s) / 2 and f(s) > s on (0, 1)."""
    rng = np.random.default_rng(seed)
    sigma = 10.0 ** rng.uniform(-3.0, 0.0, size=min(shape))
    g, _, _ = _spectral_case(rng, shape[0], shape[1], sigma)
    errs = []
    for k in range(kmax + 1):
        x = np.asarray(ns(g, k))
        errs.append(np.linalg.norm(x @ x.T - np.eye(x.shape[0])))
    for a, b in zip(errs, errs[1:]):
        if a < 1e-12:
            break
        assert b < a, errs


def pin_polar_limit(ns, shapes=((4, 8), (8, 4), (6, 6)), k=60, seed=5):
    """Blog post, "Muon 核心": the target is the polar factor U V^T of G = U S V^T."""
    rng = np.random.default_rng(seed)
    for rows, cols in shapes:
        sigma = np.linspace(1.0, 10.0, min(rows, cols))  # condition number 10
        g, _, _ = _spectral_case(rng, rows, cols, sigma)
        u, _, vt = np.linalg.svd(g, full_matrices=False)
        err = np.max(np.abs(np.asarray(ns(g, k)) - u @ vt))
        assert err < 1e-10, (rows, cols, err)


def pin_page_threshold(ns, trials=20, seed=9):
    """Blog post, "调试技巧": the orthogonality error should be < 0.01 after NS.
    Holds at k=5 for 4x8 matrices with singular values in [2/3, 1]."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        sigma = rng.uniform(2.0 / 3.0, 1.0, size=4)
        g, _, _ = _spectral_case(rng, 4, 8, sigma)
        x = np.asarray(ns(g, 5))
        assert np.linalg.norm(x @ x.T - np.eye(4)) < 0.01


def _loops_ns(g, steps):
    rows = [list(map(float, r)) for r in np.asarray(g)]
    m, n = len(rows), len(rows[0])
    transposed = m > n
    if transposed:
        rows = [[rows[i][j] for i in range(m)] for j in range(n)]
        m, n = n, m
    ss = 0.0
    for r in rows:
        for v in r:
            ss += v * v
    scale = math.sqrt(ss) + EPS
    x = [[v / scale for v in r] for r in rows]
    for _ in range(steps):
        a = [[sum(x[i][t] * x[j][t] for t in range(n)) for j in range(m)] for i in range(m)]
        x = [[1.5 * x[i][j] - 0.5 * sum(a[i][t] * x[t][j] for t in range(m)) for j in range(n)]
             for i in range(m)]
    if transposed:
        x = [[x[i][j] for i in range(m)] for j in range(n)]
    return np.array(x)


def pin_brute_force_loops(ns, shapes=((4, 8), (8, 4)), k=5, seed=13):
    rng = np.random.default_rng(seed)
    for rows, cols in shapes:
        g = rng.standard_normal((rows, cols))
        err = rel_fro(ns(g, k), _loops_ns(g, k))
        assert err < 1e-13, (rows, cols, err)


def pin_scale_invariance(ns, seed=17):
    """NS(c Y) = NS(Y) up to the epsilon's effect, for norms from 1e1 to 1e7
    (the blog's "常见错误" 1: without normalisation large norms blow up)."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((24, 56))  # ||Y|| ~ 37
    ref = np.asarray(ns(y, 5))
    for c in (1.0, 1e2, 1e4, 1e6):
        got = np.asarray(ns(c * y, 5))
        assert np.all(np.isfinite(got))
        assert rel_fro(got, ref) < 1e-7, c


def pin_rank1_and_zero(ns):
    rng = np.random.default_rng(19)
    u = rng.standard_normal(6)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(10)
    v /= np.linalg.norm(v)
    sigma = 7.0
    for k in (1, 5):
        want = scalar_map(sigma / (sigma + EPS), k) * np.outer(u, v)
        assert rel_fro(ns(sigma * np.outer(u, v), k), want) < 1e-12
    z = np.asarray(ns(np.zeros((5, 9)), 5))
    assert np.all(z == 0.0), "zero input must give zero (the epsilon prevents 0/0)"
    zt = np.asarray(ns(np.zeros((9, 5)), 0))
    assert zt.shape == (9, 5) and np.all(zt == 0.0)


def pin_transpose(ns, seed=23):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((20, 52))
    for k in (0, 3, 5):
        assert rel_fro(np.asarray(ns(g.T, k)), np.asarray(ns(g, k)).T) < 1e-15


def pin_steps_zero(ns, seed=29):
    rng = np.random.default_rng(seed)
    for shape in ((6, 15), (15, 6)):
        g = rng.standard_normal(shape)
        nrm = math.sqrt(float(np.sum(g * g)))
        assert rel_fro(ns(g, 0), g / (nrm + EPS)) < 1e-15


NS_PINS = [
    pin_exact_rational, pin_closed_form_spectrum, pin_flat_recurrence, pin_monotone,
    pin_polar_limit, pin_page_threshold, pin_brute_force_loops, pin_scale_invariance,
    pin_rank1_and_zero, pin_transpose, pin_steps_zero,
]


# ----------------------------------------------------------------------------- odd-polynomial NS
# The training guide lets a NewtonSchulz object replace the blog's cubic map; its
# coefficients are not printed.  The pins use the classical quintic
# (15 s - 10 s^3 + 3 s^5) / 8 (rational, so exact arithmetic applies), the
# widely used quintic (3.4445, -4.7750, 2.0315) and mixed per-step schedules.
QUINTIC_EXACT = (Fraction(15, 8), Fraction(-5, 4), Fraction(3, 8))
QUINTIC_FAST = (3.4445, -4.7750, 2.0315)


def poly_scalar(s: float, c) -> float:
    """sum_j c_j s^(2j+1) in plain Python floats."""
    out, p, s2 = 0.0, s, s * s
    for cj in c:
        out += cj * p
        p *= s2
    return out


def exact_poly_ns(rows, schedule):
    """Odd-polynomial Newton-Schulz over Fractions with explicit loops:
    X <- sum_j c_j A^j X with A = X X^T, one coefficient tuple per step."""
    g = [[Fraction(v) for v in r] for r in rows]
    m, n = len(g), len(g[0])
    transposed = m > n
    if transposed:
        g = [[g[i][j] for i in range(m)] for j in range(n)]
        m, n = n, m
    ss = sum(int(v) * int(v) for r in rows for v in r)
    scale = Fraction(_isqrt_exact(ss)) + EPS_FRAC
    x = [[v / scale for v in r] for r in g]
    for c in schedule:
        a = [[sum(x[i][t] * x[j][t] for t in range(n)) for j in range(m)] for i in range(m)]
        term = x
        y = [[c[0] * v for v in r] for r in x]
        for cj in c[1:]:
            term = [[sum(a[i][t] * term[t][j] for t in range(m)) for j in range(n)] for i in range(m)]
            y = [[y[i][j] + cj * term[i][j] for j in range(n)] for i in range(m)]
        x = y
    if transposed:
        x = [[x[i][j] for i in range(m)] for j in range(n)]
    return np.array([[float(v) for v in r] for r in x])


def pin_poly_exact_rational(ns_poly):
    schedules = {
        "quintic x3": [QUINTIC_EXACT] * 3,
        "mixed": [(Fraction(3, 2), Fraction(-1, 2)), QUINTIC_EXACT, (Fraction(2), Fraction(-3, 2), Fraction(1, 2))],
        "cubic as a polynomial": [(Fraction(3, 2), Fraction(-1, 2))] * 2,
    }
    for case in EXACT_CASES:
        ss = sum(v * v for r in case for v in r)
        if math.isqrt(ss) ** 2 != ss:
            continue
        for name, sched in schedules.items():
            want = exact_poly_ns(case, sched)
            coeffs = [tuple(float(c) for c in row) for row in sched]
            got = np.asarray(ns_poly(np.array(case, dtype=np.float64), len(sched), coeffs))
            assert got.shape == want.shape, (case, name)
            err = rel_fro(got, want)
            assert err < 1e-14, f"exact polynomial NS mismatch {case} {name}: {err:.3e}"


def pin_poly_closed_form_spectrum(ns_poly, shapes=((12, 40), (40, 12), (64, 256)), seed=43):
    """An odd matrix polynomial keeps singular vectors: each singular value
    follows the scalar polynomial of its step."""
    rng = np.random.default_rng(seed)
    scheds = [[QUINTIC_FAST] * 5, [QUINTIC_FAST] * 3 + [(1.5, -0.5)] * 2,
              [(1.875, -1.25, 0.375)] * 4, [(2.0, -1.5, 0.5, 0.0)] * 2]
    for rows, cols in shapes:
        r = min(rows, cols)
        sigma = 10.0 ** rng.uniform(-3.0, 0.0, size=r)
        g, left, right = _spectral_case(rng, rows, cols, sigma)
        s0 = sigma / (float(np.sqrt(np.sum(sigma * sigma))) + EPS)
        for sched in scheds:
            sk = s0.copy()
            for c in sched:
                sk = np.array([poly_scalar(float(v), c) for v in sk])
            want = (left * sk[None, :]) @ right.T
            got = np.asarray(ns_poly(g, len(sched), sched))
            err = rel_fro(got, want)
            assert err < 1e-11, f"polynomial closed form {rows}x{cols} {sched[0]}: {err:.3e}"


def _loops_poly_ns(g, schedule):
    rows = [list(map(float, r)) for r in np.asarray(g)]
    m, n = len(rows), len(rows[0])
    transposed = m > n
    if transposed:
        rows = [[rows[i][j] for i in range(m)] for j in range(n)]
        m, n = n, m
    ss = 0.0
    for r in rows:
        for v in r:
            ss += v * v
    scale = math.sqrt(ss) + EPS
    x = [[v / scale for v in r] for r in rows]
    for c in schedule:
        a = [[sum(x[i][t] * x[j][t] for t in range(n)) for j in range(m)] for i in range(m)]
        term = x
        y = [[c[0] * v for v in r] for r in x]
        for cj in c[1:]:
            term = [[sum(a[i][t] * term[t][j] for t in range(m)) for j in range(n)] for i in range(m)]
            y = [[y[i][j] + cj * term[i][j] for j in range(n)] for i in range(m)]
        x = y
    if transposed:
        x = [[x[i][j] for i in range(m)] for j in range(n)]
    return np.array(x)


def pin_poly_brute_force_loops(ns_poly, shapes=((4, 8), (8, 4), (5, 5)), seed=47):
    rng = np.random.default_rng(seed)
    for rows, cols in shapes:
        g = rng.standard_normal((rows, cols))
        for sched in ([QUINTIC_FAST] * 5, [(1.5, -0.5), QUINTIC_FAST, (2.0, -1.5, 0.5)]):
            err = rel_fro(ns_poly(g, len(sched), sched), _loops_poly_ns(g, sched))
            assert err < 1e-13, (rows, cols, err)


def pin_poly_transpose(ns_poly, seed=53):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((20, 52))
    sched = [QUINTIC_FAST] * 4
    assert rel_fro(np.asarray(ns_poly(g.T, 4, sched)), np.asarray(ns_poly(g, 4, sched)).T) < 1e-15


POLY_PINS = [pin_poly_exact_rational, pin_poly_closed_form_spectrum, pin_poly_brute_force_loops, pin_poly_transpose]


# ----------------------------------------------------------------------------- update rule
def pin_weight_decay(apply_update, fixture):
    """tests/golden/weight_decay_worked_example.txt bit for bit; a zero update
    only decays; zero decay is the plain update."""
    lr, wd, sc = fixture["lr"][0], fixture["wd"][0], fixture["scale"][0]
    as2 = lambda k: np.array(fixture[k], dtype=np.float64).reshape(2, 2)  # noqa: E731
    assert np.array_equal(apply_update(as2("p0"), as2("u"), lr, sc, wd), as2("p1"))
    assert np.array_equal(apply_update(as2("p0"), np.zeros((2, 2)), lr, sc, wd), as2("decayed"))
    rng = np.random.default_rng(59)
    p, u = rng.standard_normal((2, 3, 7))
    assert np.array_equal(apply_update(p, u, 0.02, 1.5, 0.0), p - 0.03 * u)


def pin_moonlight_scale(moonlight_lr_scale):
    """Training guide, hyper-parameter table, ``lr`` row: 0.2 * sqrt(max(m, n))."""
    assert moonlight_lr_scale(1024, 4096) == 0.2 * 64.0
    assert moonlight_lr_scale(4096, 1024) == 0.2 * 64.0
    assert moonlight_lr_scale(4096, 4096) == 0.2 * 64.0
    assert moonlight_lr_scale(2048, 32) == 0.2 * math.sqrt(2048.0)
    assert abs(moonlight_lr_scale(14336, 4096) - 0.2 * 119.73303637676612) < 1e-13


# ----------------------------------------------------------------------------- momentum / step
def pin_geometric_series(momentum_update, ns_input, mu=0.95, steps=40, seed=31):
    """Constant gradient g from a zero buffer: B_t = g (1 - mu^t) / (1 - mu);
    Nesterov input g + mu B_t; plain input B_t."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((3, 5))
    b = np.zeros_like(g)
    for t in range(1, steps + 1):
        b = momentum_update(b, g, mu)
        closed = g * (1.0 - mu ** t) / (1.0 - mu)
        assert rel_fro(b, closed) < 1e-13, t
        assert rel_fro(ns_input(g, b, mu, True), g + mu * closed) < 1e-13, t
        assert rel_fro(ns_input(g, b, mu, False), closed) < 1e-13, t


def pin_two_step(momentum_update, ns_input, mu=0.9, seed=37):
    """From B0 = 0 with gradients G1 then G2:
    Nesterov Y2 = G2 + mu (mu G1 + G2); plain Y2 = mu G1 + G2."""
    rng = np.random.default_rng(seed)
    g1, g2 = rng.standard_normal((2, 4, 6))
    b1 = momentum_update(np.zeros_like(g1), g1, mu)
    b2 = momentum_update(b1, g2, mu)
    assert rel_fro(ns_input(g2, b2, mu, True), g2 + mu * (mu * g1 + g2)) < 1e-15
    assert rel_fro(ns_input(g2, b2, mu, False), mu * g1 + g2) < 1e-15


def pin_worked_example(muon_step, fixture):
    """tests/golden/momentum_worked_example.txt, reproduced bit for bit."""
    mu, lr = fixture["mu"][0], fixture["lr"][0]
    as2 = lambda k: np.array(fixture[k], dtype=np.float64).reshape(2, 2)  # noqa: E731
    for nesterov, tag in ((True, "nesterov"), (False, "plain")):
        p, b, u, _ = muon_step([as2("p0")], [as2("grad")], [as2("buf0")], mu, nesterov, 5, lr)
        assert np.array_equal(b[0], as2("buf1"))
        assert np.array_equal(u[0], as2("y_" + tag))
        assert np.array_equal(p[0], as2("p1_" + tag))


def pin_route_threshold(muon_direction, newton_schulz):
    """numel < 100_000 takes the elementwise route (U = Y); 100_000 runs NS."""
    rng = np.random.default_rng(41)
    small = rng.standard_normal((3, 33333))      # 99,999 elements
    assert np.array_equal(muon_direction(small, 5), small)
    tiny = rng.standard_normal((2048, 32))       # hybrid set's a_proj / b_proj
    assert np.array_equal(muon_direction(tiny, 5), tiny)
    edge = rng.standard_normal((4, 25000))       # exactly 100,000 elements
    u = muon_direction(edge, 5)
    assert not np.array_equal(u, edge)
    assert rel_fro(u, newton_schulz(edge, 5)) == 0.0


# ----------------------------------------------------------------------------- gradient clipping
CLIP_EPS = 1e-6


def pin_clip_worked_example(clip, fixture):
    """tests/golden/grad_clip_worked_example.txt (hand-derived, 14 digits)."""
    mn = fixture["max_norm"]
    grads = [np.array(fixture["a"]), np.array(fixture["b"]).reshape(1, 2), np.array(fixture["c"])]
    out, totals = clip(grads, [0, 0, 1], mn)
    assert np.allclose(totals, fixture["total"], rtol=1e-15, atol=0)
    for got, key in zip(out, ("a_clipped", "b_clipped", "c_clipped")):
        assert np.allclose(np.ravel(got), fixture[key], rtol=1e-14, atol=0), key
    assert np.array_equal(out[2], grads[2]), "a segment under its max_norm must be left exactly unchanged"


def pin_clip_closed_forms(clip, seed=61):
    rng = np.random.default_rng(seed)
    gs = [rng.standard_normal((7, 9)), rng.standard_normal(13), rng.standard_normal((3, 4, 5))]
    tot = math.sqrt(sum(float(np.sum(g * g)) for g in gs))
    # above the threshold the clipped 2-norm is max_norm * total / (total + eps)
    out, t = clip(gs, [0, 0, 0], [1.0])
    assert abs(t[0] - tot) < 1e-12 * tot
    new = math.sqrt(sum(float(np.sum(g * g)) for g in out))
    assert abs(new - tot / (tot + CLIP_EPS)) < 1e-12
    # below the threshold nothing changes, bit for bit
    out, _ = clip(gs, [0, 0, 0], [tot * 2])
    assert all(np.array_equal(a, b) for a, b in zip(out, gs))
    # segments are independent; splitting a tensor inside a segment changes nothing
    out2, t2 = clip(gs, [0, 1, 0], [1.0, 100.0])
    assert np.array_equal(out2[1], gs[1])
    flat = np.concatenate([gs[0].ravel(), gs[2].ravel()])
    outf, tf = clip([flat], [0], [1.0])
    assert abs(t2[0] - tf[0]) < 1e-12 * tf[0]
    assert np.allclose(np.concatenate([out2[0].ravel(), out2[2].ravel()]), outf[0], rtol=1e-14, atol=0)
    # p = 1 is the sum of magnitudes, p = inf the largest magnitude
    _, t1 = clip(gs, [0, 0, 0], [1.0], norm_type=1.0)
    assert abs(t1[0] - sum(float(np.sum(np.abs(g))) for g in gs)) < 1e-12 * t1[0]
    _, ti = clip(gs, [0, 0, 0], [1.0], norm_type=float("inf"))
    assert ti[0] == max(float(np.max(np.abs(g))) for g in gs)


def pin_clip_loops(clip, seed=67):
    rng = np.random.default_rng(seed)
    gs = [rng.standard_normal(5) * 3, rng.standard_normal(4), rng.standard_normal(6) * 0.1]
    seg, mn, p = [0, 1, 0], [1.5, 0.2], 3.0
    out, tot = clip(gs, seg, mn, norm_type=p)
    for s in range(2):
        acc = 0.0
        for g, sg in zip(gs, seg):
            if sg == s:
                for v in g:
                    acc += abs(float(v)) ** p
        want = acc ** (1.0 / p)
        assert abs(tot[s] - want) < 1e-13 * want
        coef = min(mn[s] / (want + CLIP_EPS), 1.0)
        for g, o, sg in zip(gs, out, seg):
            if sg == s:
                for v, w in zip(g, o):
                    assert abs(float(w) - float(v) * coef) <= 1e-15 * abs(float(v)) + 1e-300


CLIP_PINS = [pin_clip_closed_forms, pin_clip_loops]


# ----------------------------------------------------------------------------- AdamW
def pin_adamw_worked_example(adamw, fixture):
    """tests/golden/adamw_worked_example.txt, bit for bit."""
    h = {k: v[0] for k, v in fixture.items()}
    args = (h["lr"], h["beta1"], h["beta2"], h["eps"], h["wd"])
    p1, m1, v1 = adamw(np.array([h["p0"]]), np.array([h["g1"]]), np.zeros(1), np.zeros(1), 1, *args)
    assert (p1[0], m1[0], v1[0]) == (h["p1"], h["m1"], h["v1"])
    p2, m2, v2 = adamw(p1, np.array([h["g2"]]), m1, v1, 2, *args)
    assert (p2[0], m2[0], v2[0]) == (h["p2"], h["m2"], h["v2"])


def pin_adamw_closed_forms(adamw, seed=71):
    rng = np.random.default_rng(seed)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    p0, g = rng.standard_normal((2, 50))
    # a constant gradient from a zero state: the bias-corrected moments are g
    # and g^2 at every step, so each step decays p and subtracts lr g / (|g| + eps)
    p, m, v = p0.copy(), np.zeros(50), np.zeros(50)
    want = p0.copy()
    for t in range(1, 8):
        p, m, v = adamw(p, g, m, v, t, lr, b1, b2, eps, wd)
        want = want * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
        assert np.allclose(m, (1 - b1 ** t) * g, rtol=1e-14, atol=0)
        assert np.allclose(v, (1 - b2 ** t) * g * g, rtol=1e-12, atol=0)
        assert np.allclose(p, want, rtol=1e-12, atol=1e-15), t
    # a zero gradient from a zero state only decays
    p, m, v = adamw(p0, np.zeros(50), np.zeros(50), np.zeros(50), 1, lr, b1, b2, eps, wd)
    assert np.array_equal(p, p0 * (1 - lr * wd)) and not m.any() and not v.any()


def pin_adamw_loops(adamw, seed=73):
    rng = np.random.default_rng(seed)
    lr, b1, b2, eps, wd = 3e-3, 0.8, 0.95, 1e-6, 0.1
    p, m, v = rng.standard_normal(5), np.zeros(5), np.zeros(5)
    ref = [float(x) for x in p]
    rm, rv = [0.0] * 5, [0.0] * 5
    for t in range(1, 4):
        g = rng.standard_normal(5)
        p, m, v = adamw(p, g, m, v, t, lr, b1, b2, eps, wd)
        for j in range(5):
            ref[j] *= 1 - lr * wd
            rm[j] = b1 * rm[j] + (1 - b1) * float(g[j])
            rv[j] = b2 * rv[j] + (1 - b2) * float(g[j]) ** 2
            ref[j] -= lr / (1 - b1 ** t) * rm[j] / (math.sqrt(rv[j]) / math.sqrt(1 - b2 ** t) + eps)
        assert np.allclose(p, ref, rtol=1e-13, atol=0)


ADAMW_PINS = [pin_adamw_closed_forms, pin_adamw_loops]


# ----------------------------------------------------------------------------- orthogonality error
def pin_orthogonality_closed_form(orth, seed=79):
    """Blog post, "调试技巧": the check is ||X X^T - I||_F.  For X = L diag(s) R^T
    (L, R with orthonormal columns, r = min(rows, cols)) taken on its wide side,
    X X^T - I = L diag(s^2 - 1) L^T on the range of L and -I on its complement,
    so the error is sqrt(sum_i (s_i^2 - 1)^2 + (m' - r)) with m' the short side.
    A flat spectrum s gives sqrt(r) |1 - s^2|; a spectrum that mixes values
    above and below 1 separates the Frobenius norm from the spectral norm and
    from sums that drop the square."""
    rng = np.random.default_rng(seed)
    for r, n in ((4, 9), (16, 40), (64, 256)):
        q = haar_orthonormal(rng, n, r).T                    # r x n, orthonormal rows
        for s in (0.0, 0.25, 0.9, 1.0, 1.7):
            want = math.sqrt(r) * abs(1.0 - s * s)
            for x in (s * q, s * q.T):                       # wide and tall orientation
                got = float(orth(x))
                assert abs(got - want) <= 1e-12 * max(1.0, want), (r, n, s, got, want)
    for rows, cols in ((6, 20), (20, 6), (12, 12)):
        r = min(rows, cols)
        sigma = np.linspace(0.2, 1.8, r)
        x, _, _ = _spectral_case(rng, rows, cols, sigma)
        want = math.sqrt(float(np.sum((sigma * sigma - 1.0) ** 2)))
        got = float(orth(x))
        assert abs(got - want) <= 1e-12 * want, (rows, cols, got, want)
    # rank-deficient wide input: the missing directions each contribute 1
    left = haar_orthonormal(rng, 8, 5)
    right = haar_orthonormal(rng, 30, 5)
    x = left @ right.T                                       # 8 x 30, rank 5, unit singular values
    got = float(orth(x))
    assert abs(got - math.sqrt(3.0)) <= 1e-12, got


ORTH_PINS = [pin_orthogonality_closed_form]
