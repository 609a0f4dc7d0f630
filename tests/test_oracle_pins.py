"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
import numpy as np
import pytest

import oracle
import _pins


@pytest.mark.parametrize("pin", _pins.NS_PINS, ids=lambda f: f.__name__)
def test_newton_schulz_pin(pin):
    pin(oracle.newton_schulz)


@pytest.mark.parametrize("pin", _pins.POLY_PINS, ids=lambda f: f.__name__)
def test_polynomial_newton_schulz_pin(pin):
    pin(oracle.newton_schulz)


def test_weight_decay(golden):
    _pins.pin_weight_decay(oracle.apply_update, golden("weight_decay_worked_example.txt"))


def test_moonlight_scale():
    _pins.pin_moonlight_scale(oracle.moonlight_lr_scale)


def test_muon_step_update_options():
    """Moonlight mode multiplies an explicit lr_scale; weight decay and custom
    coefficients reach the parameters through apply_update and newton_schulz."""
    rng = np.random.default_rng(2)
    p, g = rng.standard_normal((2, 300, 400))
    b = np.zeros_like(g)
    coeffs = _pins.QUINTIC_FAST
    p1, _, u1, _ = oracle.muon_step([p], [g], [b], 0.95, True, 5, 0.02, lr_scale=[1.5], weight_decay=0.1,
                                    moonlight=True, ns_coeffs=coeffs)
    y = g + 0.95 * g
    assert np.array_equal(u1[0], oracle.newton_schulz(y, 5, coeffs))
    s = 1.5 * oracle.moonlight_lr_scale(300, 400)
    assert np.array_equal(p1[0], oracle.apply_update(p, u1[0], 0.02, s, 0.1))


def test_coefficient_schedule_validation():
    assert oracle.coefficient_schedule(None, 2) == [oracle.CUBIC, oracle.CUBIC]
    with pytest.raises(ValueError):
        oracle.coefficient_schedule([1.0], 3)
    with pytest.raises(ValueError):
        oracle.coefficient_schedule([(1.5, -0.5)] * 2, 3)


def test_grad_clip_worked_example(golden):
    _pins.pin_clip_worked_example(oracle.clip_grad_norm_buckets, golden("grad_clip_worked_example.txt"))


@pytest.mark.parametrize("pin", _pins.CLIP_PINS, ids=lambda f: f.__name__)
def test_grad_clip_pin(pin):
    pin(oracle.clip_grad_norm_buckets)


def test_grad_clip_rejects_bad_segments():
    with pytest.raises(ValueError):
        oracle.clip_grad_norm_buckets([np.ones(3)], [1], [1.0])
    with pytest.raises(ValueError):
        oracle.clip_grad_norm_buckets([np.ones(3)], [0], [1.0], norm_type=0.0)


def test_adamw_worked_example(golden):
    _pins.pin_adamw_worked_example(oracle.adamw_step, golden("adamw_worked_example.txt"))


@pytest.mark.parametrize("pin", _pins.ADAMW_PINS, ids=lambda f: f.__name__)
def test_adamw_pin(pin):
    pin(oracle.adamw_step)


def test_momentum_geometric_series():
    _pins.pin_geometric_series(oracle.momentum_update, oracle.ns_input)


def test_nesterov_two_step():
    _pins.pin_two_step(oracle.momentum_update, oracle.ns_input)


def test_worked_example(golden):
    _pins.pin_worked_example(oracle.muon_step, golden("momentum_worked_example.txt"))


def test_route_threshold():
    _pins.pin_route_threshold(oracle.muon_direction, oracle.newton_schulz)


def test_rejects_non_matrix():
    # blog post, "常见错误" 2: NS on a bias vector must fail
    with pytest.raises(ValueError):
        oracle.newton_schulz(np.ones(8), 5)
    with pytest.raises(ValueError):
        oracle.newton_schulz(np.ones((2, 2)), -1)


def test_lr_scale():
    rng = np.random.default_rng(0)
    p, g = rng.standard_normal((2, 300, 400))
    b = np.zeros_like(g)
    p2, _, u2, _ = oracle.muon_step([p], [g], [b], 0.95, True, 5, 0.02, lr_scale=[2.0])
    p1, _, u1, _ = oracle.muon_step([p], [g], [b], 0.95, True, 5, 0.04)
    assert np.array_equal(u1[0], u2[0])
    assert np.allclose(p1[0], p2[0], rtol=0, atol=1e-15)
    # training guide, hyper-parameter table: 0.2 * sqrt(max(m, n))
    assert oracle.moonlight_lr_scale(4096, 14336) == pytest.approx(0.2 * 14336 ** 0.5)


def test_single_step_nesterov_from_zero_is_scaled_grad():
    # From a zero buffer one Nesterov step feeds (1 + mu) G to NS, which the
    # normalisation removes up to the epsilon.
    rng = np.random.default_rng(1)
    g = rng.standard_normal((320, 400))  # 128,000 elements: NS route
    _, _, u, norms = oracle.muon_step([np.zeros_like(g)], [g], [np.zeros_like(g)], 0.95, True, 5, 0.02)
    assert _pins.rel_fro(u[0], oracle.newton_schulz(g, 5)) < 1e-8  # eps/||G|| ~ 3e-10
    assert norms[0] == pytest.approx(1.95 * np.linalg.norm(g), rel=1e-14)


@pytest.mark.parametrize("pin", _pins.ORTH_PINS, ids=lambda f: f.__name__)
def test_orthogonality_error_pin(pin):
    pin(oracle.orthogonality_error)


def test_orthogonality_error_uses_wide_side():
    rng = np.random.default_rng(2)
    x = oracle.newton_schulz(rng.standard_normal((12, 4)), 40)
    assert oracle.orthogonality_error(x) < 1e-8
    assert oracle.orthogonality_error(x.T) < 1e-8
