"""Pins for the AdamW oracle (Moonlight guide, "The Coordinate-Wise Limitation of AdamW")."""
import numpy as np

import oracle


def test_first_step_from_zero_state_is_a_scaled_sign():
    """m_1 = (1 - b1) g, v_1 = (1 - b2) g^2: the step is lr (1 - b1) / sqrt(1 - b2) sign(g) up
    to eps; with bias correction it is lr sign(g)."""
    g = np.array([3.0, -0.5, 1e-3, -7.0])
    z = np.zeros(4)
    b1, b2, lr = 0.9, 0.999, 1e-2
    th, m, v = oracle.adamw_step(z, g, z, z, lr, b1, b2, 0.0, 0.0)
    assert np.allclose(m, 0.1 * g, rtol=0, atol=1e-15) and np.allclose(v, 0.001 * g * g, rtol=1e-15)
    assert np.allclose(th, -lr * 0.1 / np.sqrt(0.001) * np.sign(g), rtol=1e-14)
    th, _, _ = oracle.adamw_step(z, g, z, z, lr, b1, b2, 0.0, 0.0, step=1, bias_correction=True)
    assert np.allclose(th, -lr * np.sign(g), rtol=1e-14)


def test_constant_gradient_moments_closed_form():
    """After t steps of a constant g from zero state: m_t = (1 - b1^t) g, v_t = (1 - b2^t) g^2,
    and the bias-corrected step is exactly lr g / (|g| + eps) every step."""
    g = np.array([0.25, -2.0, 5.0])
    th, m, v = np.zeros(3), np.zeros(3), np.zeros(3)
    b1, b2, lr, eps = 0.8, 0.95, 1e-3, 1e-8
    for t in range(1, 7):
        prev = th
        th, m, v = oracle.adamw_step(th, g, m, v, lr, b1, b2, eps, 0.0, step=t, bias_correction=True)
        assert np.allclose(m, (1 - b1 ** t) * g, rtol=1e-14)
        assert np.allclose(v, (1 - b2 ** t) * g * g, rtol=1e-14)
        assert np.allclose(prev - th, lr * g / (np.abs(g) + eps), rtol=1e-12)


def test_weight_decay_only_and_zero_lr():
    th = np.array([1.0, -2.0, 0.5])
    z = np.zeros(3)
    out, m, v = oracle.adamw_step(th, z, z, z, 0.1, 0.9, 0.99, 1e-8, 0.01)
    assert np.array_equal(out, th * (1 - 0.1 * 0.01)) and not m.any() and not v.any()
    out, _, _ = oracle.adamw_step(th, np.ones(3), z, z, 0.0, 0.9, 0.99, 1e-8, 0.3)
    assert np.array_equal(out, th)


def test_eps_sits_outside_the_square_root():
    """One coordinate with g = 1e-4, b2 = 0: sqrt(v) = 1e-4, so eps = 1e-4 halves the step
    (inside the root it would shrink it by 1/sqrt(1.00000001 ...) only)."""
    g = np.array([1e-4])
    z = np.zeros(1)
    th, _, _ = oracle.adamw_step(z, g, z, z, 1.0, 0.0, 0.0, 1e-4, 0.0)
    assert np.allclose(th, -0.5, rtol=1e-12)
