"""Pins for the oracle's blended prefill: the method's own special cases.

* r = 100% equals a one-shot full prefill                      ([CB] "背景")
* r = 0% equals the re-RoPE'd concatenation + full KV reuse     ([CB] "背景")
* one chunk at offset 0 reproduces prefix reuse (causality)    ([CB] "问题")
* a chunk prefilled at p, re-RoPE'd by -p, equals one prefilled at 0
                                                                ([CB] "位置恢复")
* sets nest, have the scheduled sizes, never contain the suffix ([CB] "核心思想")
* a masked-dense formulation agrees with the gathered-rows one  ([CB] Fig. 5)
* the compute share at the 8B, 4K, 15% point is about 18%      ([CB] "把账算细")

Each pin runs in the oracle's float32 and again in float64.  Where two
formulations agree only up to rounding order (the blend computes a row inside a
larger or smaller batch than the reference does, so BLAS sums in another order)
the float32 bound is 1e-5 normwise, the float64 bound 1e-12; bitwise claims hold
in both.
"""
import json
import os

import numpy as np
import pytest

import cbinputs
from oracle import (OracleModel, assemble_blended, blend_layer, blend_prefill, blend_prefill_masked,
                    chunk_prefill, flop_count, full_prefill, full_reuse_prefill, kv_deviation, precision,
                    store_round)

PREC = pytest.mark.parametrize("prec", ["f32", "f64"])
# agreement up to rounding order; "r100" is the benchmark spec's bound for r = 100%
TOL = {"f32": {"order": 1e-5, "r100": 1e-5, "dev_floor": 1e-6},
       "f64": {"order": 1e-12, "r100": 1e-5, "dev_floor": 1e-6}}

HERE = os.path.dirname(os.path.abspath(__file__))

# an MHA/GQA decoder small enough for many runs; fp32 storage
GQA = cbinputs.ModelShape("gqa-small", 3, 64, 4, 2, 16, 96, 101, 10000.0, dtype="f32")


def _sharpen(w):
    # larger Q/K weights make attention peaked, so cross-chunk effects are not tiny
    for lw in w["layers"]:
        lw["wq"] = lw["wq"] * 15.0
        lw["wk"] = lw["wk"] * 15.0
    return w


def _setup(shape, lens, old, new, n_query, seed):
    w = _sharpen(cbinputs.model_weights(shape, seed))
    m = OracleModel.from_shape(shape, w)
    rng = np.random.default_rng(seed + 100)
    chunks = []
    for ln, p, n in zip(lens, old, new):
        toks = rng.integers(0, shape.vocab, size=ln)
        K, V = chunk_prefill(m, toks, p)
        chunks.append((toks, K, V, p, n))
    q = rng.integers(0, shape.vocab, size=n_query)
    return m, chunks, q


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(np.asarray(b))), 1e-300)


def _sched(L, N, k):
    return [N] + [k] * (L - 1), [0] + [1] * (L - 1)


def _full_tokens(chunks, q):
    order = sorted(range(len(chunks)), key=lambda c: chunks[c][4])
    return np.concatenate([chunks[c][0] for c in order] + [q])


@PREC
@pytest.mark.parametrize("shape_name", ["gqa", "tiny"])
def test_r100_equals_full_prefill(shape_name, prec):
    with precision(prec):
        _r100(shape_name, TOL[prec]["r100"])


def _r100(shape_name, tol):
    if shape_name == "gqa":
        m, chunks, q = _setup(GQA, [20, 13, 17], [5, 0, 31], [17, 37, 0], 6, 1)
    else:
        wl = cbinputs.make_workload("tiny-2x256-q32", seed=0, chunk_len=64, n_query=8)
        w = cbinputs.model_weights(wl.shape, 0)
        m = OracleModel.from_shape(wl.shape, w)
        chunks = [(t, *chunk_prefill(m, t, p), p, n)
                  for t, p, n in zip(wl.chunk_tokens, wl.old_starts, wl.new_starts)]
        q = wl.query_tokens
    N = sum(len(c[0]) for c in chunks)
    ks, ch = _sched(m.n_layers, N, N)
    b = blend_prefill(m, chunks, q, ks, ch)
    f = full_prefill(m, _full_tokens(chunks, q), 0)
    assert _rel(b["K"], f["K"]) < tol
    assert _rel(b["V"], f["V"]) < tol
    assert _rel(b["logits"], f["logits"]) < tol
    for l in range(1, m.n_layers):
        assert b["sets"][l].tolist() == list(range(N))


@PREC
def test_r0_equals_concatenation_and_full_reuse(prec):
    with precision(prec):
        _r0(TOL[prec]["order"])


def _r0(tol):
    m, chunks, q = _setup(GQA, [20, 13, 17], [5, 0, 31], [17, 37, 0], 6, 2)
    N = 50
    ks, ch = _sched(m.n_layers, N, 0)
    b = blend_prefill(m, chunks, q, ks, ch)
    Kc, Vc = assemble_blended(m, chunks, len(q))
    assert np.array_equal(b["K"][:, :N], Kc[:, :N])     # bitwise
    assert np.array_equal(b["V"][:, :N], Vc[:, :N])
    r = full_reuse_prefill(m, Kc, Vc, q)
    assert _rel(b["logits"], r["logits"]) < tol
    assert _rel(b["K"], r["K"]) < tol
    # and the reuse really differs from the full prefill (cross-chunk attention is missing)
    f = full_prefill(m, _full_tokens(chunks, q), 0)
    assert _rel(r["logits"], f["logits"]) > 1e-3


@PREC
@pytest.mark.parametrize("ratio", [0.0, 0.15, 0.5, 1.0])
def test_single_chunk_prefix_reuse(ratio, prec):
    with precision(prec):
        _single_chunk(ratio, TOL[prec]["r100"], TOL[prec]["dev_floor"])


def _single_chunk(ratio, tol, dev_floor):
    m, chunks, q = _setup(GQA, [40], [0], [0], 5, 3)
    N = 40
    k = cbinputs.recompute_count(ratio, N)
    ks, ch = _sched(m.n_layers, N, k)
    b = blend_prefill(m, chunks, q, ks, ch)
    f = full_prefill(m, _full_tokens(chunks, q), 0)
    assert _rel(b["K"], f["K"]) < tol
    assert _rel(b["V"], f["V"]) < tol
    assert _rel(b["logits"], f["logits"]) < tol
    # every deviation is at the level of rounding (fp32 storage: the cache holds what a
    # recomputation gives, up to the order of the sums)
    for l, (cand, dev) in b["devs"].items():
        if len(cand) == 0:
            continue
        scale = np.mean(np.sum(b["K"][l, cand] ** 2, axis=(1, 2)) + np.sum(b["V"][l, cand] ** 2, axis=(1, 2)))
        assert np.max(dev) <= dev_floor * scale


@PREC
def test_rerope_of_chunk_prefill_is_position_shift(prec):
    # a chunk prefilled at p, re-RoPE'd by -p, equals the same chunk prefilled at 0
    shape = GQA.with_dtype("f64")
    w = _sharpen(cbinputs.model_weights(shape, 4))
    m = OracleModel.from_shape(shape, w)
    toks = np.random.default_rng(4).integers(0, shape.vocab, size=30)
    from oracle import rerope
    with precision(prec):
        K0, V0 = chunk_prefill(m, toks, 0)
        Kp, Vp = chunk_prefill(m, toks, 777)
        back = rerope(Kp, -777, shape.rope_theta, "f64")
    tol = 1e-5 if prec == "f32" else 1e-10
    assert _rel(back, K0) < tol
    assert _rel(Vp, V0) < tol
    assert _rel(Kp, K0) > 1e-2        # the stored keys do carry their position


@PREC
def test_sets_nest_and_masked_twin_agrees(prec):
    with precision(prec):
        _twin(TOL[prec]["order"])


def _twin(tol):
    m, chunks, q = _setup(GQA, [20, 13, 17], [5, 0, 31], [17, 37, 0], 6, 5)
    N = 50
    ks = [N, 30, 22]
    ch = [0, 1, 1]
    b = blend_prefill(m, chunks, q, ks, ch)
    t = blend_prefill_masked(m, chunks, q, ks, ch)
    prev = set(range(N))
    for l in range(1, m.n_layers):
        s = b["sets"][l]
        assert len(s) == ks[l]
        assert np.all(np.diff(s) > 0)
        assert set(s.tolist()) <= prev
        assert np.all(s < N)
        assert s.tolist() == t["sets"][l].tolist()
        prev = set(s.tolist())
    assert _rel(b["K"], t["K"]) < tol
    assert _rel(b["V"], t["V"]) < tol
    assert _rel(b["logits"], t["logits"]) < tol
    for l in b["devs"]:
        np.testing.assert_allclose(b["devs"][l][1], t["devs"][l][1], rtol=100 * tol)


@PREC
def test_selected_rows_get_fresh_kv_others_keep_cache(prec):
    m, chunks, q = _setup(GQA, [20, 13, 17], [5, 0, 31], [17, 37, 0], 6, 6)
    N = 50
    ks, ch = _sched(m.n_layers, N, 8)
    with precision(prec):
        b = blend_prefill(m, chunks, q, ks, ch)
        Kc, Vc = assemble_blended(m, chunks, len(q))
    for l in range(1, m.n_layers):
        s = set(b["sets"][l].tolist())
        others = [j for j in range(N) if j not in s]
        assert np.array_equal(b["K"][l, others], Kc[l, others])
        assert np.array_equal(b["V"][l, others], Vc[l, others])
        changed = [j for j in s if not np.array_equal(b["K"][l, j], Kc[l, j])]
        assert len(changed) == len(s)
    # layer-0 context K/V stay cached (re-RoPE'd) even at r = 100%
    assert np.array_equal(b["K"][0, :N], Kc[0, :N])


@PREC
def test_deviation_is_top_ranked_set(prec):
    m, chunks, q = _setup(GQA, [20, 13, 17], [5, 0, 31], [17, 37, 0], 6, 7)
    N = 50
    ks, ch = _sched(m.n_layers, N, 10)
    with precision(prec):
        b = blend_prefill(m, chunks, q, ks, ch)
    cand, dev = b["devs"][1]
    thr = np.sort(dev)[::-1][9]
    chosen = set(b["sets"][1].tolist())
    for c, d in zip(cand, dev):
        if d > thr:
            assert c in chosen
        elif d < thr:
            assert c not in chosen


def test_compute_share_about_18_percent():
    # [CB] "把账算细": 4096 x 32 x 0.15 ~ 19660 of 131072 token-layers, plus one
    # full layer -> about 18%
    g = json.load(open(os.path.join(HERE, "golden", "token_layer_accounting.json")))
    shape = cbinputs.SHAPES["llama3-8b"]
    N, L, r = g["n_ctx"], g["n_layers"], g["ratio"]
    assert int(N * L * r) == g["recomputed_token_layers"] or round(N * L * r) == g["recomputed_token_layers"]
    assert N * L == g["full_token_layers"]
    k = cbinputs.recompute_count(r, N)
    ks, ch = _sched(L, N, k)
    token_layers = N + sum(ks[1:])
    assert abs(token_layers / (N * L) - g["ratio_with_first_layer"]) < 0.01
    fc = flop_count(shape, N, 64, ks, ch)
    assert abs(fc["ratio"] - g["ratio_with_first_layer"]) < 0.02


def test_kv_bytes_per_token_golden():
    # [KV] S_token = L x 2 x H_kv x D_head x B; [CB] "把账算细"
    g = json.load(open(os.path.join(HERE, "golden", "kv_bytes_per_token.json")))
    for case in g["cases"]:
        b = case["layers"] * 2 * case["kv_heads"] * case["head_dim"] * case["bytes_per_element"]
        assert b == case["bytes_per_token"]
    assert cbinputs.SHAPES["llama3-8b"].kv_bytes_per_token() == 128 * 1024


@PREC
def test_blend_layer_out_rows_are_rows_of_the_full_call(prec):
    with precision(prec):
        _out_rows(TOL[prec]["order"])


def _out_rows(tol):
    # a row's output depends on its own hidden state and the updated cache
    # only, so computing a subset must return those rows (up to the order of sums)
    w = _sharpen(cbinputs.model_weights(GQA, 9))
    m = OracleModel.from_shape(GQA, w)
    rng = np.random.default_rng(9)
    N, Q, k = 40, 5, 9
    T = N + Q
    cand = np.sort(rng.choice(N, 30, replace=False))
    Kl = rng.standard_normal((T, GQA.n_kv_heads, GQA.head_dim))
    Vl = rng.standard_normal((T, GQA.n_kv_heads, GQA.head_dim))
    x = rng.standard_normal((len(cand) + Q, GQA.d_model))
    full = blend_layer(m, 1, Kl.copy(), Vl.copy(), x, cand, Q, True, k)
    rows = np.array([k + Q - 1, 0, 4, k, k - 1])
    K2, V2 = Kl.copy(), Vl.copy()
    part = blend_layer(m, 1, K2, V2, x, cand, Q, True, k, out_rows=rows)
    assert np.array_equal(part[1], full[1])
    assert _rel(part[0], full[0][rows]) < tol
    K3, V3 = Kl.copy(), Vl.copy()
    blend_layer(m, 1, K3, V3, x, cand, Q, True, k)
    assert np.array_equal(K2, K3) and np.array_equal(V2, V3)


@PREC
def test_decode_step_continues_a_full_prefill(prec):
    with precision(prec):
        _decode(TOL[prec]["order"])


def _decode(tol):
    # causality: the last row of a one-shot prefill over t_0..t_T is a decode step of
    # t_T on the cache the prefill of t_0..t_{T-1} wrote (and writes the same K/V row)
    from oracle import decode_step
    w = _sharpen(cbinputs.model_weights(GQA, 11))
    m = OracleModel.from_shape(GQA, w)
    rng = np.random.default_rng(11)
    toks = rng.integers(0, GQA.vocab, size=23)
    T = 20
    ref = full_prefill(m, toks[:T + 1])
    part = full_prefill(m, toks[:T])
    L, _, H, dh = part["K"].shape
    Kb = np.zeros((L, T + 3, H, dh), dtype=part["K"].dtype)
    Vb = np.zeros_like(Kb)
    Kb[:, :T], Vb[:, :T] = part["K"], part["V"]
    lg = decode_step(m, Kb, Vb, int(toks[T]), T)
    assert _rel(lg, ref["logits"]) < tol
    assert _rel(Kb[:, T], ref["K"][:, T]) < tol and _rel(Vb[:, T], ref["V"][:, T]) < tol
    # two more steps equal the prefill over the longer sequence
    decode_step(m, Kb, Vb, int(toks[T + 1]), T + 1)
    lg2 = decode_step(m, Kb, Vb, int(toks[T + 2]), T + 2)
    assert _rel(lg2, full_prefill(m, toks[:T + 3])["logits"]) < tol
