"""Pins for the oracle's decoder pieces, deviation and top-k.

The base forward is compared with a reference assembled from torch CPU
library routines (F.rms_norm, F.linear, F.silu,
F.scaled_dot_product_attention with is_causal/enable_gqa, complex rotation via
torch.polar) -- an independent formulation of the same decoder.  Deviation and
selection are compared with brute-force loops and sorting.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import cbinputs
from oracle import (OracleModel, causal_attention, full_prefill, kv_deviation, rms_norm,
                    select_hkvd, swiglu_mlp)

SMALL = cbinputs.ModelShape("small", 2, 64, 4, 2, 16, 96, 97, 10000.0, dtype="f64")


def torch_reference_prefill(shape, weights, tokens, start):
    """Decoder forward written with torch CPU routines in float64."""
    d = torch.float64
    tok = torch.as_tensor(np.asarray(tokens), dtype=torch.long)
    x = torch.as_tensor(weights["embed"], dtype=d)[tok]
    n = len(tokens)
    pos = torch.arange(start, start + n, dtype=d)
    dh = shape.head_dim
    inv = shape.rope_theta ** (-torch.arange(0, dh, 2, dtype=d) / dh)
    rot = torch.polar(torch.ones(n, dh // 2, dtype=d), pos[:, None] * inv[None, :])

    def rope(t):  # t [n, H, dh]
        z = torch.view_as_complex(t.reshape(n, t.shape[1], dh // 2, 2).contiguous())
        return torch.view_as_real(z * rot[:, None, :]).reshape(n, t.shape[1], dh)

    Ks, Vs = [], []
    for l in range(shape.n_layers):
        w = {k: torch.as_tensor(v, dtype=d) for k, v in weights["layers"][l].items()}
        a = F.rms_norm(x, (shape.d_model,), w["attn_norm"], eps=shape.rms_eps)
        q = rope(F.linear(a, w["wq"]).reshape(n, shape.n_q_heads, dh))
        k = rope(F.linear(a, w["wk"]).reshape(n, shape.n_kv_heads, dh))
        v = F.linear(a, w["wv"]).reshape(n, shape.n_kv_heads, dh)
        Ks.append(k.numpy().copy())
        Vs.append(v.numpy().copy())
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=True, enable_gqa=True)
        o = o[0].transpose(0, 1).reshape(n, -1)
        x = x + F.linear(o, w["wo"])
        h = F.rms_norm(x, (shape.d_model,), w["mlp_norm"], eps=shape.rms_eps)
        x = x + F.linear(F.silu(F.linear(h, w["w_gate"])) * F.linear(h, w["w_up"]), w["w_down"])
    hl = F.rms_norm(x[-1:], (shape.d_model,), torch.as_tensor(weights["final_norm"], dtype=d), eps=shape.rms_eps)
    logits = F.linear(hl, torch.as_tensor(weights["lm_head"], dtype=d))[0]
    return np.stack(Ks), np.stack(Vs), logits.numpy()


def _rand_norm_gains(shape, weights, seed):
    rng = np.random.default_rng(seed)
    for lw in weights["layers"]:
        lw["attn_norm"] = 1.0 + 0.1 * rng.standard_normal(shape.d_model)
        lw["mlp_norm"] = 1.0 + 0.1 * rng.standard_normal(shape.d_model)
    weights["final_norm"] = 1.0 + 0.1 * rng.standard_normal(shape.d_model)


@pytest.mark.parametrize("start", [0, 37])
def test_full_prefill_matches_torch_functional(start):
    w = cbinputs.model_weights(SMALL, seed=11)
    _rand_norm_gains(SMALL, w, 12)   # non-unit gains so a dropped gain is caught
    # larger init so attention is not near-uniform
    for lw in w["layers"]:
        for k in ("wq", "wk"):
            lw[k] = lw[k] * 20.0
    m = OracleModel.from_shape(SMALL, w)
    tokens = np.random.default_rng(13).integers(0, SMALL.vocab, size=40)
    ours = full_prefill(m, tokens, start)
    K, V, logits = torch_reference_prefill(SMALL, w, tokens, start)
    np.testing.assert_allclose(ours["K"], K, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ours["V"], V, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ours["logits"], logits, rtol=1e-9, atol=1e-12)


def test_tiny_config_forward_matches_torch_functional():
    shape = cbinputs.SHAPES["tiny-2l-d256"].with_dtype("f64")
    w = cbinputs.model_weights(shape, seed=0)
    m = OracleModel.from_shape(shape, w)
    tokens = np.random.default_rng(0).integers(0, shape.vocab, size=96)
    ours = full_prefill(m, tokens, 0)
    K, V, logits = torch_reference_prefill(shape, w, tokens, 0)
    np.testing.assert_allclose(ours["K"], K, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ours["logits"], logits, rtol=1e-9, atol=1e-12)


def test_attention_row_subset_equals_dense_rows():
    rng = np.random.default_rng(21)
    T, Hq, Hkv, dh = 70, 8, 2, 16
    q = rng.standard_normal((T, Hq, dh)) * 3
    k = rng.standard_normal((T, Hkv, dh)) * 3
    v = rng.standard_normal((T, Hkv, dh))
    pos = np.arange(T)
    dense = causal_attention(q, pos, k, v, pos)
    rows = np.sort(rng.choice(T, size=19, replace=False))
    sub = causal_attention(q[rows], rows, k, v, pos, row_block=5)
    np.testing.assert_allclose(sub, dense[rows], rtol=1e-12, atol=1e-13)
    # dense equals torch SDPA (GQA, causal)
    ref = F.scaled_dot_product_attention(torch.as_tensor(q).transpose(0, 1)[None],
                                         torch.as_tensor(k).transpose(0, 1)[None],
                                         torch.as_tensor(v).transpose(0, 1)[None],
                                         is_causal=True, enable_gqa=True)[0].transpose(0, 1).numpy()
    np.testing.assert_allclose(dense, ref, rtol=1e-10, atol=1e-12)


def test_attention_first_row_sees_only_itself():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((5, 2, 4))
    k = rng.standard_normal((5, 1, 4))
    v = rng.standard_normal((5, 1, 4))
    o = causal_attention(q, np.arange(5), k, v, np.arange(5))
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 1], v[0, 0], rtol=0, atol=1e-15)


def test_rms_norm_and_mlp_match_torch():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((9, 32)) * 5
    g = rng.standard_normal(32)
    ref = F.rms_norm(torch.as_tensor(x), (32,), torch.as_tensor(g), eps=1e-5).numpy()
    np.testing.assert_allclose(rms_norm(x, g, 1e-5), ref, rtol=1e-12)
    wg, wu, wd = rng.standard_normal((48, 32)), rng.standard_normal((48, 32)), rng.standard_normal((32, 48))
    t = torch.as_tensor
    ref = F.linear(F.silu(F.linear(t(x), t(wg))) * F.linear(t(x), t(wu)), t(wd)).numpy()
    np.testing.assert_allclose(swiglu_mlp(x, wg, wu, wd), ref, rtol=1e-10, atol=1e-9)


def test_deviation_closed_form_and_brute_force():
    rng = np.random.default_rng(24)
    kc = rng.standard_normal((6, 2, 4))
    vc = rng.standard_normal((6, 2, 4))
    kf, vf = kc.copy(), vc.copy()
    kf[3, 1, 2] += 0.5       # one K element moved by 0.5
    vf[5, 0, 0] -= 2.0       # one V element moved by 2
    d = kv_deviation(kf, vf, kc, vc)
    np.testing.assert_allclose(d, [0, 0, 0, 0.25, 0, 4.0], rtol=0, atol=1e-15)
    kf = rng.standard_normal((6, 2, 4))
    vf = rng.standard_normal((6, 2, 4))
    d = kv_deviation(kf, vf, kc, vc)
    for j in range(6):
        s = 0.0
        for h in range(2):
            for e in range(4):
                s += (kf[j, h, e] - kc[j, h, e]) ** 2 + (vf[j, h, e] - vc[j, h, e]) ** 2
        assert d[j] == pytest.approx(s, rel=1e-13)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 6), min_size=1, max_size=60), st.data())
def test_select_matches_brute_force_sort(vals, data):
    # small integer deviations force many ties
    n = len(vals)
    dev = np.array(vals, dtype=np.float64)
    pos = np.sort(np.random.default_rng(n).choice(10 * n, size=n, replace=False))
    k = data.draw(st.integers(0, n))
    ranked = sorted(range(n), key=lambda i: (-dev[i], pos[i]))
    expect = sorted(int(pos[i]) for i in ranked[:k])
    got = select_hkvd(dev, pos, k)
    assert got.tolist() == expect
    assert np.all(np.diff(got) > 0)


def test_select_all_and_none():
    dev = np.array([3.0, 1.0, 2.0])
    pos = np.array([4, 8, 9])
    assert select_hkvd(dev, pos, 3).tolist() == [4, 8, 9]
    assert select_hkvd(dev, pos, 0).tolist() == []
    assert select_hkvd(dev, pos, 1).tolist() == [4]
    assert select_hkvd(dev, pos, 2).tolist() == [4, 9]
