"""Pins for the oracle's RoPE, re-RoPE and storage rounding.

Each check compares against something the oracle does not compute itself:
closed forms, complex-number rotation, torch's bfloat16 conversion, or the
algebra of rotations ([CB] "位置恢复": q_m^T k_n depends on n - m only, and
k' = R_{n-p} k_p = R_n k).
"""
import numpy as np
import pytest
import torch

from oracle import rope, rope_cos_sin, rerope, store_round


def test_theta_closed_form():
    # theta_i = base^(-2i/d): d = 4, base = 10000 -> theta = (1, 0.01)
    c, s = rope_cos_sin(np.array([1.0, 3.0]), 4, 10000.0)
    ang = np.array([[1.0, 0.01], [3.0, 0.03]])
    np.testing.assert_allclose(c, np.cos(ang), rtol=0, atol=1e-15)
    np.testing.assert_allclose(s, np.sin(ang), rtol=0, atol=1e-15)


def test_rotation_direction_unit_vector():
    # R_m acting on e_0 in the first pair gives (cos m theta_0, sin m theta_0)
    x = np.zeros((1, 1, 2))
    x[0, 0, 0] = 1.0
    y = rope(x, np.array([1]), 10000.0)
    assert y[0, 0, 0] == pytest.approx(np.cos(1.0), abs=1e-15)
    assert y[0, 0, 1] == pytest.approx(np.sin(1.0), abs=1e-15)


def test_rope_equals_complex_multiplication():
    rng = np.random.default_rng(0)
    n, H, d = 7, 3, 16
    x = rng.standard_normal((n, H, d))
    pos = rng.integers(0, 40000, size=n)
    y = rope(x, pos, 500000.0)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = 500000.0 ** (-np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    np.testing.assert_allclose(y[..., 0::2], zr.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[..., 1::2], zr.imag, rtol=0, atol=1e-12)


def test_rerope_inverse_identity():
    # re-RoPE by delta then -delta is the identity within 1e-6
    rng = np.random.default_rng(1)
    k = rng.standard_normal((3, 50, 2, 64))
    for delta in (1, 255, 4096, 31000):
        back = rerope(rerope(k, delta, 500000.0, "f64"), -delta, 500000.0, "f64")
        assert np.max(np.abs(back - k)) / np.max(np.abs(k)) < 1e-12
        k32 = store_round(k, "f32")
        back32 = rerope(rerope(k32, delta, 500000.0, "f32"), -delta, 500000.0, "f32")
        assert np.max(np.abs(back32 - k32)) / np.max(np.abs(k32)) < 1e-6


def test_rerope_composition():
    # R_{n-p} R_p k = R_n k for p, n up to 32K
    rng = np.random.default_rng(2)
    k = rng.standard_normal((40, 4, 128))
    p = rng.integers(0, 4096, size=40)
    n = rng.integers(0, 32768, size=40)
    kp = rope(k, p, 500000.0)
    lhs = np.stack([rerope(kp[i:i + 1], int(n[i] - p[i]), 500000.0, "f64")[0] for i in range(40)])
    rhs = rope(k, n, 500000.0)
    assert np.max(np.abs(lhs - rhs)) / np.max(np.abs(rhs)) < 1e-10


def test_relative_position_and_norm():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((20, 1, 64))
    k = rng.standard_normal((20, 1, 64))
    m = rng.integers(0, 10000, size=20)
    n = rng.integers(0, 10000, size=20)
    lhs = np.sum(rope(q, m, 10000.0) * rope(k, n, 10000.0), axis=(1, 2))
    rhs = np.sum(q * rope(k, n - m, 10000.0), axis=(1, 2))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(rope(k, n, 10000.0), axis=2), np.linalg.norm(k, axis=2), rtol=1e-12)


def test_v_untouched_and_zero_delta_exact():
    rng = np.random.default_rng(4)
    k = store_round(rng.standard_normal((2, 9, 2, 8)), "bf16")
    assert np.array_equal(rerope(k, 0, 500000.0, "bf16"), k)


def test_store_round_bf16_matches_torch():
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-4, 4, 100000)).astype(np.float32)
    ours = store_round(x32.astype(np.float64), "bf16")
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_store_round_bf16_ties_and_double_rounding():
    # exact halfway between two bf16 values rounds to even
    one = 1.0
    ulp = 2.0 ** -7
    assert store_round(np.array([one + ulp / 2]), "bf16")[0] == one
    assert store_round(np.array([one + 3 * ulp / 2]), "bf16")[0] == one + 2 * ulp
    # just above halfway (below fp32 resolution of the tie) rounds up: direct
    # float64 rounding, no intermediate fp32 step
    assert store_round(np.array([one + ulp / 2 + 2.0 ** -40]), "bf16")[0] == one + ulp
    assert store_round(np.array([-(one + ulp / 2 + 2.0 ** -40)]), "bf16")[0] == -(one + ulp)
