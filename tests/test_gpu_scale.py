"""GPU parity at the largest shapes: the 70B width (d 8192, 64 q / 8 kv
heads, F 28672) and the 32K-token paged context of the 8B shape.

A full oracle run at these sizes takes hours on the host, so:
* cb_blend_layer is run for one selective layer at full width and full
  context; the oracle computes fresh K/V and the deviation of every candidate
  (so the whole HKVD set and every scattered row are compared), but the
  attention, O and MLP only for a sample of the kept and suffix rows, which is
  exact because a row's output depends only on its own hidden state and the
  updated cache;
* the whole 32-layer, 32K-token paged blend is checked through properties that
  hold at any size (sorted, nested sets; untouched rows keep the re-RoPE'd
  cache; changed rows are exactly the kept ones; finite logits).
Weights are drawn on the GPU by torch's seeded generator (host generation at
70B width takes about a minute per layer) and copied to the host for the
oracle before the library packs them."""
import dataclasses

import numpy as np
import pytest
import torch

import cbinputs
import oracle
from cacheblend_selective_recompute_amd import api

from gpu_helpers import (blended_cache, check_sets, fp8_close, host_layer, ints, paged_chunks, rel, say, to_dev,
                         to_np)
from oracle.blend import fp8_e4m3

pytestmark = pytest.mark.gpu


def _layer_sampled(base, N, Q, k, seed, paged, n_sample=24, kv8=None, check=True):
    """kv8 = (k_scale, v_scale): the cache holds FP8 E4M3 (oracle and GPU).
    check=False: an unchecked layer (keeps every candidate, measures nothing)."""
    shape = dataclasses.replace(base, n_layers=2, vocab=64)
    T = N + Q
    lt = cbinputs.torch_device_layer(shape, seed)
    lw = host_layer(lt, shape)
    glob = cbinputs.global_weights(shape, seed)
    m_ora = oracle.OracleModel.from_shape(shape, {"layers": [lw, lw], **glob})
    if kv8:
        m_ora.kv_storage, m_ora.k_scale, m_ora.v_scale = "fp8", kv8[0], kv8[1]
    # two shallow copies: packing replaces the matrices in each copy only
    m_gpu = api.DeviceModel(shape, [dict(lt), dict(lt)], to_dev(glob["embed"], "bf16"),
                            to_dev(glob["lm_head"], "bf16"), torch.ones(shape.d_model, device="cuda"))
    del lt
    x = cbinputs.synthetic_layer_rows(shape, T, seed=seed)
    Kc, Vc = cbinputs.synthetic_layer_cache(shape, T, seed=seed)
    if kv8:
        Kc = (fp8_e4m3(Kc / kv8[0]) * kv8[0]).astype(np.float32)
        Vc = (fp8_e4m3(Vc / kv8[1]) * kv8[1]).astype(np.float32)
        table, n_phys = cbinputs.paged_layout(T, 16, seed + 4, key=77, spare_blocks=5)
        kv = api.PagedKV(shape, T, 16, table, n_phys, fill=0.0, kv_format=api.CB_KV_FP8_E4M3, k_scale=kv8[0],
                         v_scale=kv8[1])
    else:
        kv = blended_cache(shape, T, paged=paged, seed=seed + 4, fill=0.0)
    idx = kv.slots(np.arange(T))
    if kv8:
        kv.k[1, idx] = api.fp8_encode(torch.from_numpy(Kc).cuda(), kv8[0])
        kv.v[1, idx] = api.fp8_encode(torch.from_numpy(Vc).cuda(), kv8[1])
    else:
        kv.k[1, idx] = to_dev(Kc, "bf16")
        kv.v[1, idx] = to_dev(Vc, "bf16")
    xg = torch.from_numpy(x).cuda()
    pos_out = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    dev = torch.full((N,), -1.0, device="cuda")
    api.cb_blend_layer(m_gpu, 1, kv, ints(np.arange(N)), N, Q, xg, check, k, pos_out, dev)
    torch.cuda.synchronize()
    gpos = pos_out.cpu().numpy()
    assert np.all(np.diff(gpos) > 0) and gpos[0] >= 0 and gpos[-1] < N
    if not check:
        assert np.array_equal(gpos, np.arange(N))              # every candidate, in order
        assert bool((dev == -1.0).all())                        # nothing measured
    # the oracle with the GPU's kept set imposed; its deviations are its own
    rows = np.unique(np.concatenate([np.linspace(0, k - 1, n_sample).astype(np.int64),
                                     k + np.array([0, Q // 2, Q - 1])]))
    Kl = Kc.astype(np.float64)
    Vl = Vc.astype(np.float64)
    if kv8:
        # the written rows with bf16 operands (the GPU's arithmetic): FP8 codes compared strictly
        K16, V16 = Kc.astype(np.float64), Vc.astype(np.float64)
        with oracle.operands("bf16"):
            oracle.blend_layer(m_ora, 1, K16, V16, x.astype(np.float64), np.arange(N), Q, check, k,
                               force=gpos if check else None, out_rows=rows[:1])
        # The same fresh values before rounding, with float32 and with float64 sums: the
        # GPU sums the same bf16 products in another order, so near zero (where the FP8
        # grid is finest) the two float32 results may differ by more than a grid step.
        # Each side is within about the float32-vs-float64 distance of the exact sums.
        m_ora.kv_storage = "f32"
        fresh = {}
        for prec in ("f32", "f64"):
            Kf, Vf = Kc.astype(np.float64), Vc.astype(np.float64)
            with oracle.operands("bf16"), oracle.precision(prec):
                oracle.blend_layer(m_ora, 1, Kf, Vf, x.astype(np.float64), np.arange(N), Q, check, k,
                                   force=gpos if check else None, out_rows=rows[:1])
            fresh[prec] = (Kf, Vf)
        m_ora.kv_storage = "fp8"
    x_ora, keep, dev_ora = oracle.blend_layer(m_ora, 1, Kl, Vl, x.astype(np.float64), np.arange(N), Q, check, k,
                                              force=gpos if check else None, out_rows=rows)
    if check:
        own = oracle.select_hkvd(dev_ora, np.arange(N), k)
        sc = float(np.mean(np.sum(Kc.astype(np.float64) ** 2, axis=(1, 2)) +
                           np.sum(Vc.astype(np.float64) ** 2, axis=(1, 2))))
        frac = check_sets(gpos, own, np.arange(N), dev_ora, k, sc, "layer 1")
        ed = rel(to_np(dev), dev_ora)
    else:
        frac, ed = 1.0, 0.0
    xo = to_np(xg[torch.from_numpy(rows).cuda()])
    ex = rel(xo, x_ora)
    K1, V1 = kv.logical(T)
    K1 = to_np(K1[1])
    V1 = to_np(V1[1])
    written = np.concatenate([gpos, np.arange(N, T)])
    if kv8:
        # the fresh values come from one layer's products: against the bf16-operand
        # oracle every element within one grid step plus twice the float32 summation
        # distance, 99% on the same grid point; against float32, plus how far the
        # float32 products move them
        ordK = 2 * float(np.max(np.abs(fresh["f32"][0][written] - fresh["f64"][0][written])))
        ordV = 2 * float(np.max(np.abs(fresh["f32"][1][written] - fresh["f64"][1][written])))
        say(f"  float32 summation order: up to {ordK:.2e} (K) and {ordV:.2e} (V) between two float32 results")
        fp8_close(K1[written], K16[written], kv8[0], "scattered K (bf16 operands)", extra=ordK)
        fp8_close(V1[written], V16[written], kv8[1], "scattered V (bf16 operands)", extra=ordV)
        fp8_close(K1[written], Kl[written], kv8[0], "scattered K (float32)", min_equal=0.9,
                  extra=float(np.max(np.abs(K16[written] - Kl[written]))))
        fp8_close(V1[written], Vl[written], kv8[1], "scattered V (float32)", min_equal=0.9,
                  extra=float(np.max(np.abs(V16[written] - Vl[written]))))
    ek = rel(K1[written], Kl[written])
    ev = rel(V1[written], Vl[written])
    say(f"  decision agreement {frac:.4f}, deviation rel {ed:.2e}, sampled x rows rel {ex:.2e}, "
        f"scattered K {ek:.2e} V {ev:.2e}")
    assert ed < 1e-2
    assert ex < 2e-2
    if not kv8:   # FP8: bounded element by element above (one grid step is 1/16 to 1/8 of a value)
        assert ek < 2e-2 and ev < 2e-2
    untouched = np.setdiff1d(np.arange(N), gpos)
    assert np.array_equal(K1[untouched], Kc[untouched].astype(np.float64))
    assert np.array_equal(V1[untouched], Vc[untouched].astype(np.float64))


def test_blend_layer_70b_width_sampled():
    say("cb_blend_layer: 70B width, layer 1, 4096 candidates + 64 query rows, keep 614, paged")
    _layer_sampled(cbinputs.SHAPES["llama-70b"], 4096, 64, 614, seed=5, paged=True)


def test_blend_layer_8b_width_keep_all_sampled():
    # every candidate kept: the Q/K/V product's split-K reduction takes the deviations
    # and writes the fresh K/V rows into the cache itself
    say("cb_blend_layer: 8B width, layer 1, 614 candidates + 64 query rows, keep all 614, paged")
    _layer_sampled(cbinputs.SHAPES["llama3-8b"], 614, 64, 614, seed=7, paged=True)


def test_blend_layer_8b_width_unchecked_keep_all_sampled():
    # an unchecked layer at a shape whose Q/K/V product is split: the reduction writes
    # the row maps and pos_out of every candidate and measures no deviation
    say("cb_blend_layer: 8B width, layer 1 unchecked, 614 candidates + 64 query rows, keep all 614, paged")
    _layer_sampled(cbinputs.SHAPES["llama3-8b"], 614, 64, 614, seed=9, paged=True, check=False)


def test_blend_layer_8b_width_keep_all_fp8_sampled():
    say("cb_blend_layer: 8B width, FP8 cache (scales 0.029, 0.037), layer 1 keeping all 614 candidates + 64 rows")
    _layer_sampled(cbinputs.SHAPES["llama3-8b"], 614, 64, 614, seed=8, paged=True, kv8=(0.029, 0.037))


def test_blend_layer_70b_width_fp8_sampled():
    say("cb_blend_layer: 70B width, FP8 cache (scales 0.04, 0.05), layer 1, 4096 candidates + 64 query rows, "
        "keep 614, paged")
    _layer_sampled(cbinputs.SHAPES["llama-70b"], 4096, 64, 614, seed=10, paged=True, kv8=(0.04, 0.05))


def test_blend_layer_32k_context_fp8_sampled():
    # the FP8 layer is widened to bf16 for the attention (32K keys) before the LDS-staged kernel reads it
    say("cb_blend_layer: 8B width, FP8 cache (scales 0.029, 0.037), layer 1, 32768 candidates + 128 query rows, "
        "keep 4915, paged")
    _layer_sampled(cbinputs.SHAPES["llama3-8b"], 32768, 128, 4915, seed=11, paged=True, kv8=(0.029, 0.037))


def test_blend_layer_32k_context_paged_sampled():
    say("cb_blend_layer: 8B width, layer 1, 32768 candidates + 128 query rows, keep 4915, paged")
    _layer_sampled(cbinputs.SHAPES["llama3-8b"], 32768, 128, 4915, seed=6, paged=True)


def test_blend_full_32k_paged_properties():
    say("blend: full 8B shape, 32 x 1024 + 128, paged source and destination, r 15% (properties)")
    wl = cbinputs.make_workload("8b-32x1024-q128-paged", seed=0)
    shape = wl.shape
    m = api.DeviceModel.from_tensors(shape, cbinputs.torch_device_weights(shape, 0))
    chunks = paged_chunks(shape, wl, cbinputs.torch_device_chunk_kv(shape, wl.chunk_lens, 0), 0)
    T, N = wl.n_total, wl.n_ctx
    kv = blended_cache(shape, T, paged=True, seed=3, fill=0.0)
    ks, ch = wl.schedule()
    logits = torch.empty(shape.vocab, device="cuda")
    hk = torch.full((shape.n_layers, N), -1, dtype=torch.int32, device="cuda")
    api.cb_blend_prefill(m, chunks, ints(wl.query_tokens), api.BlendParams(ks, ch), kv, logits, hk)
    torch.cuda.synchronize()
    assert torch.isfinite(logits).all()
    h = hk.cpu().numpy()
    assert np.array_equal(h[0], np.arange(N))
    prev = set(range(N))
    for l in range(1, shape.n_layers):
        s = h[l, :ks[l]]
        assert np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < N
        assert set(s.tolist()) <= prev
        prev = set(s.tolist())
    ref = blended_cache(shape, T, paged=True, seed=3, fill=0.0)
    api.cb_rerope_k(api.make_cfg(shape), chunks, ref, api.CB_COPY_V)
    torch.cuda.synchronize()
    for l in (0, 1, 16, 31):
        Kg, Vg = kv.k[l][kv.slots(np.arange(T))], kv.v[l][kv.slots(np.arange(T))]
        Kr, Vr = ref.k[l][ref.slots(np.arange(T))], ref.v[l][ref.slots(np.arange(T))]
        kept = h[l, :ks[l]] if l > 0 else np.zeros(0, dtype=np.int64)
        out = np.setdiff1d(np.arange(N), kept)
        assert torch.equal(Kg[out], Kr[out]) and torch.equal(Vg[out], Vr[out]), f"layer {l}: untouched rows changed"
        if l > 0:
            diff = (Kg[kept] != Kr[kept]).flatten(1).any(dim=1)
            assert bool(diff.all()), f"layer {l}: a kept row still holds the cached K"
        # the suffix rows hold fresh, finite K/V
        assert torch.isfinite(Kg[N:].float()).all() and (Kg[N:] != 0).flatten(1).any(dim=1).all()
