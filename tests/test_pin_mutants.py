"""Planted mistakes in copies of the oracle must each fail at least one pin.

The mutants live here, on the CPU; the oracle itself is untouched.
"""
import numpy as np
import pytest

import oracle
import _pins

EPS = 1e-7


def _ns_factory(norm=None, eps_inside=False, no_eps=False, c1=1.5, c2=0.5, gram="xxt",
                steps_off=0, transpose_back=True):
    def ns(g, steps):
        g = np.asarray(g, dtype=np.float64)
        if g.ndim != 2:
            raise ValueError
        m, n = g.shape
        t = m > n
        x = g.T if t else g
        ss = float(np.sum(x * x))
        if norm == "maxabs":
            d = float(np.max(np.abs(x))) + EPS
        elif norm == "spectral":
            d = float(np.linalg.norm(x, 2)) + EPS
        elif no_eps:
            d = np.sqrt(ss)
        elif eps_inside:
            d = np.sqrt(ss + EPS)
        else:
            d = np.sqrt(ss) + EPS
        with np.errstate(invalid="ignore", divide="ignore"):
            x = x / d
        for _ in range(max(steps + steps_off, 0)):
            a = x.T @ x if gram == "xtx" else x @ x.T
            if gram == "xtx":
                x = c1 * x - c2 * (a @ x) if a.shape[0] == x.shape[0] else c1 * x - c2 * (x @ a.T @ a) / 1.0
            else:
                x = c1 * x - c2 * (a @ x)
        return x.T if (t and transpose_back) else x
    return ns


NS_MUTANTS = {
    "no_eps": _ns_factory(no_eps=True),
    "eps_inside_sqrt": _ns_factory(eps_inside=True),
    "maxabs_norm": _ns_factory(norm="maxabs"),
    "spectral_norm": _ns_factory(norm="spectral"),
    "coef_1.4": _ns_factory(c1=1.4),
    "sign_flip": _ns_factory(c2=-0.5),
    "half_coef_0.25": _ns_factory(c2=0.25),
    "gram_transposed": _ns_factory(gram="xtx"),
    "one_step_short": _ns_factory(steps_off=-1),
    "one_step_long": _ns_factory(steps_off=1),
    "no_transpose_back": _ns_factory(transpose_back=False),
}


def _fails_some_pin(ns):
    for pin in _pins.NS_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(NS_MUTANTS))
def test_ns_mutant_is_caught(name):
    assert _fails_some_pin(NS_MUTANTS[name]), f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    assert not _fails_some_pin(_ns_factory())


def _caught(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_momentum_mutants_are_caught(golden):
    fixture = golden("momentum_worked_example.txt")
    damped = lambda b, g, mu: mu * np.asarray(b) + (1 - mu) * np.asarray(g)  # noqa: E731
    old_buf_nesterov = lambda g, b, mu, nest: (np.asarray(g) + mu * (np.asarray(b) - np.asarray(g)) / mu  # noqa: E731
                                                if nest else np.asarray(b))
    assert _caught(lambda: _pins.pin_geometric_series(damped, oracle.ns_input))
    assert _caught(lambda: _pins.pin_two_step(oracle.momentum_update, old_buf_nesterov))

    def step_with_mutant(mutant):
        def muon_step(params, grads, bufs, mu, nesterov, steps, lr, lr_scale=None):
            b = [mutant(bb, g, mu) for bb, g in zip(bufs, grads)]
            y = [oracle.ns_input(g, bb, mu, nesterov) for g, bb in zip(grads, b)]
            return [oracle.apply_update(p, yy, lr) for p, yy in zip(params, y)], b, y, None
        return muon_step
    assert _caught(lambda: _pins.pin_worked_example(step_with_mutant(damped), fixture))

    off_by_one_route = lambda y, k: (np.asarray(y) if np.asarray(y).size <= 100_000  # noqa: E731
                                     else oracle.newton_schulz(y, k))
    assert _caught(lambda: _pins.pin_route_threshold(off_by_one_route, oracle.newton_schulz))


# ----------------------------------------------------------------------------- odd-polynomial NS
def _poly_factory(drop_last=False, wrong_power=False, reverse=False, shift=0, gram="xxt"):
    def ns(g, steps, coeffs):
        g = np.asarray(g, dtype=np.float64)
        m, n = g.shape
        t = m > n
        x = g.T if t else g
        x = x / (np.sqrt(float(np.sum(x * x))) + EPS)
        sched = oracle.coefficient_schedule(coeffs, steps)
        for k in range(steps):
            c = list(sched[min(max(k + shift, 0), steps - 1)])
            if reverse:
                c = c[::-1]
            if drop_last and len(c) > 2:
                c = c[:-1]
            a = x.T @ x if gram == "xtx" and m == n else x @ x.T
            if gram == "xtx" and m != n:
                a = x @ x.T * 1.0000001
            term, y = x, c[0] * x
            for j, cj in enumerate(c[1:], start=1):
                term = (a @ x) if (wrong_power and j > 1) else (a @ term)
                y = y + cj * term
            x = y
        return x.T if t else x
    return ns


POLY_MUTANTS = {
    "drop_last_term": _poly_factory(drop_last=True),
    "wrong_power": _poly_factory(wrong_power=True),
    "reversed_coefficients": _poly_factory(reverse=True),
    "schedule_shifted": _poly_factory(shift=1),
    "gram_perturbed": _poly_factory(gram="xtx"),
}


def _fails_some_poly_pin(ns):
    for pin in _pins.POLY_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(POLY_MUTANTS))
def test_polynomial_mutant_is_caught(name):
    assert _fails_some_poly_pin(POLY_MUTANTS[name]), f"mutant {name} passed every pin"


def test_unmutated_polynomial_copy_passes():
    assert not _fails_some_poly_pin(_poly_factory())


def test_update_rule_mutants_are_caught(golden):
    fixture = golden("weight_decay_worked_example.txt")
    scaled_decay = lambda p, u, lr, s=1.0, wd=0.0: np.asarray(p) * (1 - lr * s * wd) - lr * s * np.asarray(u)  # noqa: E731
    decay_after = lambda p, u, lr, s=1.0, wd=0.0: (np.asarray(p) - lr * s * np.asarray(u)) * (1 - lr * wd)  # noqa: E731
    decay_sign = lambda p, u, lr, s=1.0, wd=0.0: np.asarray(p) * (1 + lr * wd) - lr * s * np.asarray(u)  # noqa: E731
    for mutant in (scaled_decay, decay_after, decay_sign):
        assert _caught(lambda: _pins.pin_weight_decay(mutant, fixture))
    assert _caught(lambda: _pins.pin_moonlight_scale(lambda m, n: 0.2 * np.sqrt(min(m, n))))
    assert _caught(lambda: _pins.pin_moonlight_scale(lambda m, n: np.sqrt(max(m, n))))


# ----------------------------------------------------------------------------- gradient clipping
def _clip_factory(eps_outside=False, no_clamp=False, per_tensor=False, no_root=False, one_segment=False):
    def clip(grads, segments, max_norms, norm_type=2.0):
        gs = [np.asarray(g, dtype=np.float64) for g in grads]
        seg = [0] * len(gs) if one_segment else list(segments)
        p = float(norm_type)
        def norm(members):
            if np.isinf(p):
                return max(float(np.max(np.abs(g))) for g in members)
            acc = sum(float(np.sum(np.abs(g) ** p)) for g in members)
            return acc if no_root else acc ** (1.0 / p)
        totals = [norm([g for g, sg in zip(gs, seg) if sg == s] or [np.zeros(1)]) for s in range(len(max_norms))]
        out = []
        for g, sg in zip(gs, seg):
            t = norm([g]) if per_tensor else totals[sg]
            coef = max_norms[sg] / t + 1e-6 if eps_outside else max_norms[sg] / (t + 1e-6)
            out.append(g * (coef if no_clamp else min(coef, 1.0)))
        return out, totals
    return clip


CLIP_MUTANTS = {
    "eps_outside": _clip_factory(eps_outside=True),
    "no_clamp": _clip_factory(no_clamp=True),
    "per_tensor_norm": _clip_factory(per_tensor=True),
    "no_root": _clip_factory(no_root=True),
    "one_segment": _clip_factory(one_segment=True),
}


@pytest.mark.parametrize("name", sorted(CLIP_MUTANTS))
def test_clip_mutant_is_caught(name, golden):
    fixture = golden("grad_clip_worked_example.txt")
    mutant = CLIP_MUTANTS[name]
    caught = _caught(lambda: _pins.pin_clip_worked_example(mutant, fixture))
    for pin in _pins.CLIP_PINS:
        caught = caught or _caught(lambda: pin(mutant))
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_clip_copy_passes(golden):
    fixture = golden("grad_clip_worked_example.txt")
    _pins.pin_clip_worked_example(_clip_factory(), fixture)
    for pin in _pins.CLIP_PINS:
        pin(_clip_factory())


# ----------------------------------------------------------------------------- AdamW
def _adamw_factory(no_bias=False, coupled=False, eps_inside=False, decay_after=False):
    def adamw(p, g, m, v, step, lr, b1, b2, eps, wd):
        p = np.asarray(p, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        if coupled:
            g = g + wd * p
        elif not decay_after:
            p = p * (1 - lr * wd)
        m = b1 * np.asarray(m) + (1 - b1) * g
        v = b2 * np.asarray(v) + (1 - b2) * g * g
        bc1, bc2 = (1.0, 1.0) if no_bias else (1 - b1 ** step, 1 - b2 ** step)
        denom = np.sqrt(v / bc2 + eps) if eps_inside else np.sqrt(v) / np.sqrt(bc2) + eps
        p = p - lr / bc1 * m / denom
        if decay_after:
            p = p * (1 - lr * wd)
        return p, m, v
    return adamw


ADAMW_MUTANTS = {"no_bias_correction": _adamw_factory(no_bias=True), "coupled_decay": _adamw_factory(coupled=True),
                 "eps_inside_sqrt": _adamw_factory(eps_inside=True), "decay_after": _adamw_factory(decay_after=True)}


@pytest.mark.parametrize("name", sorted(ADAMW_MUTANTS))
def test_adamw_mutant_is_caught(name, golden):
    fixture = golden("adamw_worked_example.txt")
    mutant = ADAMW_MUTANTS[name]
    caught = _caught(lambda: _pins.pin_adamw_worked_example(mutant, fixture))
    for pin in _pins.ADAMW_PINS:
        caught = caught or _caught(lambda: pin(mutant))
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_adamw_copy_passes(golden):
    _pins.pin_adamw_worked_example(_adamw_factory(), golden("adamw_worked_example.txt"))
    for pin in _pins.ADAMW_PINS:
        pin(_adamw_factory())


# ----------------------------------------------------------------------------- orthogonality error
def _orth_factory(kind=None):
    def orth(x):
        x = np.asarray(x, dtype=np.float64)
        if kind != "tall_side" and x.shape[0] > x.shape[1]:
            x = x.T
        if kind == "zero":
            return 0.0
        if kind == "gram_other_side":
            d = x.T @ x - np.eye(x.shape[1])
        else:
            d = x @ x.T - np.eye(x.shape[0])
        if kind == "spectral":
            return float(np.linalg.norm(d, 2))
        if kind == "no_square":
            return float(np.sum(np.abs(d)))
        if kind == "singular_values":
            return float(np.linalg.norm(np.linalg.svd(x, compute_uv=False) - 1.0))
        return float(np.sqrt(np.sum(d * d)))
    return orth


ORTH_MUTANTS = {k: _orth_factory(k) for k in ("zero", "tall_side", "gram_other_side", "spectral", "no_square",
                                              "singular_values")}


@pytest.mark.parametrize("name", sorted(ORTH_MUTANTS))
def test_orthogonality_mutant_is_caught(name):
    caught = False
    for pin in _pins.ORTH_PINS:
        caught = caught or _caught(lambda: pin(ORTH_MUTANTS[name]))
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_orthogonality_copy_passes():
    for pin in _pins.ORTH_PINS:
        pin(_orth_factory())
