"""Pins for the oracle's RoPE, re-RoPE and storage rounding.

Each check compares against something the oracle does not compute itself:
closed forms, complex-number rotation, torch's bfloat16 conversion, or the
algebra of rotations ([CB] "位置恢复": q_m^T k_n depends on n - m only, and
k' = R_{n-p} k_p = R_n k).  Every check runs in the oracle's float32 (the
default) and again in float64, each at a bound of its own precision.
"""
import numpy as np
import pytest
import torch

from oracle import precision, rope, rope_cos_sin, rerope, store_round

PREC = pytest.mark.parametrize("prec", ["f32", "f64"])


def test_theta_closed_form():
    # theta_i = base^(-2i/d): d = 4, base = 10000 -> theta = (1, 0.01); cos/sin of the
    # float64 angle, rounded once to float32 (float64: unrounded)
    ang = np.array([[1.0, 0.01], [3.0, 0.03]])
    c, s = rope_cos_sin(np.array([1.0, 3.0]), 4, 10000.0)
    assert c.dtype == np.float32 and s.dtype == np.float32
    assert np.array_equal(c, np.cos(ang).astype(np.float32))
    assert np.array_equal(s, np.sin(ang).astype(np.float32))
    with precision("f64"):
        c, s = rope_cos_sin(np.array([1.0, 3.0]), 4, 10000.0)
    np.testing.assert_allclose(c, np.cos(ang), rtol=0, atol=1e-15)
    np.testing.assert_allclose(s, np.sin(ang), rtol=0, atol=1e-15)


@PREC
def test_rotation_direction_unit_vector(prec):
    # R_m acting on e_0 in the first pair gives (cos m theta_0, sin m theta_0): exactly the
    # table entries (1 * c - 0 * s)
    x = np.zeros((1, 1, 2))
    x[0, 0, 0] = 1.0
    with precision(prec):
        y = rope(x, np.array([1]), 10000.0)
    want = np.float32 if prec == "f32" else np.float64
    assert y[0, 0, 0] == want(np.cos(1.0))
    assert y[0, 0, 1] == want(np.sin(1.0))


@PREC
def test_rope_equals_complex_multiplication(prec):
    rng = np.random.default_rng(0)
    n, H, d = 7, 3, 16
    x = rng.standard_normal((n, H, d))
    if prec == "f32":
        x = x.astype(np.float32).astype(np.float64)
    pos = rng.integers(0, 40000, size=n)
    with precision(prec):
        y = rope(x, pos, 500000.0)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = 500000.0 ** (-np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    # float32: cos/sin each within half an fp32 ulp (<= 2^-25), two rounded products and a
    # rounded sum, so |error| <= 2^-22 (|x_2i| + |x_2i+1|) with margin
    pair = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    bound = 2.0 ** -22 * pair if prec == "f32" else 1e-12
    assert np.all(np.abs(y[..., 0::2] - zr.real) <= bound)
    assert np.all(np.abs(y[..., 1::2] - zr.imag) <= bound)


@PREC
def test_rerope_inverse_identity(prec):
    # re-RoPE by delta then -delta is the identity within 1e-6 (float64: 1e-12)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((3, 50, 2, 64)).astype(np.float32)
    tol = 1e-6 if prec == "f32" else 1e-12
    with precision(prec):
        for delta in (1, 255, 4096, 31000):
            back = rerope(rerope(k, delta, 500000.0, "f64"), -delta, 500000.0, "f64")
            assert np.max(np.abs(back - k)) / np.max(np.abs(k)) < tol
            back32 = rerope(rerope(k, delta, 500000.0, "f32"), -delta, 500000.0, "f32")
            assert np.max(np.abs(back32 - k)) / np.max(np.abs(k)) < 1e-6


@PREC
def test_rerope_composition(prec):
    # R_{n-p} R_p k = R_n k for p, n up to 32K: within 1e-6 in float32 (the angles are
    # float64, so only the rounded cos/sin and the rotations' own rounding remain)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((40, 4, 128))
    p = rng.integers(0, 4096, size=40)
    n = rng.integers(0, 32768, size=40)
    with precision(prec):
        kp = rope(k, p, 500000.0)
        lhs = np.stack([rerope(kp[i:i + 1], int(n[i] - p[i]), 500000.0, "f64")[0] for i in range(40)])
        rhs = rope(k, n, 500000.0)
    tol = 1e-6 if prec == "f32" else 1e-10
    assert np.max(np.abs(lhs - rhs)) / np.max(np.abs(rhs)) < tol


@PREC
def test_relative_position_and_norm(prec):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((20, 1, 64))
    k = rng.standard_normal((20, 1, 64))
    m = rng.integers(0, 10000, size=20)
    n = rng.integers(0, 10000, size=20)
    with precision(prec):
        lhs = np.sum(rope(q, m, 10000.0) * rope(k, n, 10000.0), axis=(1, 2), dtype=np.float64)
        rhs = np.sum(q * rope(k, n - m, 10000.0), axis=(1, 2), dtype=np.float64)
        nk = np.linalg.norm(rope(k, n, 10000.0).astype(np.float64), axis=2)
    # a dot product of 64 terms: float32 errors are relative to sum |q_i k_i| <= |q| |k|
    scale = np.linalg.norm(q, axis=2)[:, 0] * np.linalg.norm(k, axis=2)[:, 0]
    tol = 1e-6 if prec == "f32" else 1e-12
    assert np.all(np.abs(lhs - rhs) <= tol * scale)
    np.testing.assert_allclose(nk, np.linalg.norm(k, axis=2), rtol=tol)


@PREC
def test_v_untouched_and_zero_delta_exact(prec):
    rng = np.random.default_rng(4)
    with precision(prec):
        k = store_round(rng.standard_normal((2, 9, 2, 8)), "bf16")
        assert np.array_equal(rerope(k, 0, 500000.0, "bf16"), k)


@PREC
def test_store_round_bf16_matches_torch(prec):
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-4, 4, 100000)).astype(np.float32)
    with precision(prec):
        ours = store_round(x32, "bf16")
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours.astype(np.float64), ref)


def test_store_round_bf16_ties_and_double_rounding():
    # exact halfway between two bf16 values rounds to even, in both precisions
    one = 1.0
    ulp = 2.0 ** -7
    for prec in ("f32", "f64"):
        with precision(prec):
            assert store_round(np.array([one + ulp / 2]), "bf16")[0] == one
            assert store_round(np.array([one + 3 * ulp / 2]), "bf16")[0] == one + 2 * ulp
            assert store_round(np.array([-(one + 3 * ulp / 2)]), "bf16")[0] == -(one + 2 * ulp)
            # one float32 ulp above halfway rounds up
            assert store_round(np.array([one + ulp / 2 + 2.0 ** -23]), "bf16")[0] == one + ulp
    # float64: just above halfway (below fp32 resolution of the tie) rounds up, straight
    # from float64 with no intermediate fp32 step
    with precision("f64"):
        assert store_round(np.array([one + ulp / 2 + 2.0 ** -40]), "bf16")[0] == one + ulp
        assert store_round(np.array([-(one + ulp / 2 + 2.0 ** -40)]), "bf16")[0] == -(one + ulp)
