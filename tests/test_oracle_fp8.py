"""Pins of the oracle's 8-bit KV storage (OCP FP8 E4M3, one scale per cache
tensor): the rounding against the format's own bit definition and against
torch's float8_e4m3fn conversion (a library routine), saturation, scaling,
and the blend's special cases with an 8-bit cache (r = 0 is the re-RoPE'd
concatenation; one chunk reused where it was stored is the full prefill with
the same storage, its deviations bounded by the cache's rounding)."""
import numpy as np
import pytest
import torch

import cbinputs
from oracle.blend import (OracleModel, assemble_blended, blend_prefill, chunk_prefill, fp8_e4m3, full_prefill,
                          full_reuse_prefill, precision, rerope, store_round)

# every pin runs in the oracle's float32 and again in float64; ORDER is the bound for
# two computations that differ only in the order of their sums
PREC = pytest.mark.parametrize("prec", ["f32", "f64"])
ORDER = {"f32": 1e-5, "f64": 1e-12}


def _grid():
    """Every finite E4M3FN value from its bits: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
            vals.append((v, m))
    return sorted(set(vals))


@PREC
def test_every_grid_value_is_kept_and_midpoints_go_to_even(prec):
    with precision(prec):
        _grid_checks()


def _grid_checks():
    g = _grid()
    v = np.array([x for x, _ in g])
    assert v[-1] == 448.0 and v[1] == 2.0 ** -9 and len(v) == 127       # +0 and 126 positive values
    assert np.array_equal(fp8_e4m3(v), v)
    assert np.array_equal(fp8_e4m3(-v), -v)
    for (a, ma), (b, mb) in zip(g[:-1], g[1:]):
        mid = (a + b) / 2
        want = a if ma % 2 == 0 else b
        assert fp8_e4m3(np.array([mid]))[0] == want, (a, b)
        assert fp8_e4m3(np.array([a + (b - a) * 0.49]))[0] == a
        assert fp8_e4m3(np.array([a + (b - a) * 0.51]))[0] == b


@PREC
def test_saturation(prec):
    x = np.array([449.0, 464.0, 480.0, 1e6, -500.0, -1e30])
    with precision(prec):
        assert np.array_equal(fp8_e4m3(x), np.array([448.0, 448.0, 448.0, 448.0, -448.0, -448.0]))


@PREC
def test_matches_torch_float8_in_range(prec):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
                        rng.uniform(-448, 448, 5000)])
    x = x[np.abs(x) <= 448]
    if prec == "f32":
        x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    with precision(prec):
        assert np.array_equal(fp8_e4m3(x), ref)


@PREC
def test_store_round_scale(prec):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000) * 3
    dt = np.float32 if prec == "f32" else np.float64
    x = x.astype(dt)
    with precision(prec):
        for s in (1.0, 0.25, 1 / 64):                                      # powers of two: exact
            y = store_round(x, "fp8", s)
            assert np.array_equal(y / dt(s), fp8_e4m3(x / dt(s)))
            assert np.array_equal(store_round(y, "fp8", s), y)              # idempotent on the grid
        y = store_round(x, "fp8", 0.013)
        # the grid value times the scale, rounded once in the compute precision
        assert np.array_equal(y, fp8_e4m3(x / dt(0.013)) * dt(0.013))
        # 3 mantissa bits: half a step is at most 2^-4 of the value in the normal range
        xn = x[np.abs(x / dt(1 / 16)) >= 2.0 ** -6]
        assert np.max(np.abs(store_round(xn, "fp8", 1 / 16) - xn) / np.abs(xn)) <= 2.0 ** -4 + 1e-12


def _fp8_model(shape, seed, ks, vs):
    w = cbinputs.model_weights(shape, seed)
    for lw in w["layers"]:
        lw["wq"] = lw["wq"] * 15.0
        lw["wk"] = lw["wk"] * 15.0
    m = OracleModel.from_shape(shape, w)
    m.kv_storage, m.k_scale, m.v_scale = "fp8", ks, vs
    return m


def _chunks(m, lens, old, new, nq, seed):
    rng = np.random.default_rng(seed)
    chunks = []
    for ln, p, n in zip(lens, old, new):
        t = rng.integers(0, m.vocab, size=ln)
        chunks.append((t, *chunk_prefill(m, t, p), p, n))
    return chunks, rng.integers(0, m.vocab, size=nq)


GQA = cbinputs.ModelShape("gqa-small", 3, 64, 4, 2, 16, 96, 101, 10000.0, dtype="f32")


@PREC
def test_chunk_cache_is_on_the_fp8_grid(prec):
    with precision(prec):
        _on_grid()


def _on_grid():
    m = _fp8_model(GQA, 2, 1 / 32, 1 / 128)
    chunks, _ = _chunks(m, [20], [3], [0], 0, 2)
    K, V = chunks[0][1], chunks[0][2]
    assert np.array_equal(fp8_e4m3(K / m.k_scale), K / m.k_scale)
    assert np.array_equal(fp8_e4m3(V / m.v_scale), V / m.v_scale)
    assert len(np.unique(np.abs(K / m.k_scale))) <= 127


@PREC
def test_fp8_r0_is_rerope_concatenation_and_full_reuse(prec):
    with precision(prec):
        _fp8_r0(ORDER[prec])


def _fp8_r0(tol):
    m = _fp8_model(GQA, 3, 1 / 32, 1 / 128)
    chunks, q = _chunks(m, [20, 13, 17], [5, 0, 31], [17, 37, 0], 6, 3)
    N = 50
    ks, ch = [N, 0, 0], [0, 1, 1]
    b = blend_prefill(m, chunks, q, ks, ch)
    Kc, Vc = assemble_blended(m, chunks, len(q))
    assert np.array_equal(b["K"][:, :N], Kc[:, :N])
    assert np.array_equal(b["V"][:, :N], Vc[:, :N])
    # the re-RoPE'd keys are on the grid, rotated from the stored ones
    for t, K, V, p, n in chunks:
        assert np.array_equal(Kc[:, n:n + len(t)], rerope(K, n - p, m.rope_theta, "fp8", m.k_scale))
    r = full_reuse_prefill(m, Kc, Vc, q)
    assert np.max(np.abs(b["logits"] - r["logits"])) <= tol * np.max(np.abs(r["logits"]))


@PREC
@pytest.mark.parametrize("ratio", [0.0, 0.5, 1.0])
def test_fp8_single_chunk_prefix_reuse_equals_full_prefill(ratio, prec):
    with precision(prec):
        _fp8_single(ratio, ORDER[prec])


def _fp8_single(ratio, tol):
    # one chunk reused at the offset it was stored at: the re-RoPE rotates by 0, which
    # leaves grid values on the grid, so every stored K/V is what a full prefill stores
    m = _fp8_model(GQA, 5, 1 / 32, 1 / 128)
    chunks, q = _chunks(m, [40], [0], [0], 5, 5)
    N = 40
    k = cbinputs.recompute_count(ratio, N)
    b = blend_prefill(m, chunks, q, [N, k, k], [0, 1, 1])
    f = full_prefill(m, np.concatenate([chunks[0][0], q]), 0)
    assert np.array_equal(b["K"], f["K"]) and np.array_equal(b["V"], f["V"])
    assert np.max(np.abs(b["logits"] - f["logits"])) <= max(tol, 1e-9) * np.max(np.abs(f["logits"]))
    # the fresh values are unrounded, so a deviation is the cache's own rounding error:
    # at most half a step per element (2^-4 of the value, or half the subnormal step)
    for l, (cand, dev) in b["devs"].items():
        n_el = f["K"].shape[2] * f["K"].shape[3]
        bound = 2.0 ** -8 * (np.sum(f["K"][l, cand] ** 2, axis=(1, 2)) + np.sum(f["V"][l, cand] ** 2, axis=(1, 2))) \
            + n_el * ((2.0 ** -10 * m.k_scale) ** 2 + (2.0 ** -10 * m.v_scale) ** 2)
        assert np.all(dev <= bound * (1 + max(tol, 1e-9)))
        assert len(dev) == 0 or np.max(dev) > 0
