"""GPU parity with an 8-bit (FP8 E4M3) KV cache, through the C ABI.

Stored FP8 values are compared element by element with the oracle run with bf16
operands (the arithmetic the GPU performs): both round nearly the same float32
value, so every element lies within one grid step and at least 99% sit on the
same grid point.  Deeper in a blend two bf16 computations drift apart (see the
end-to-end tests), so there the bound adds the largest distance between the
bf16-operand and the float32 oracle runs of the same layer, and 97% must be
equal.  Where the input is already on the grid (re-RoPE with rotation 0, V moved
between caches with power-of-two scales) the bytes are equal.  HKVD sets: the
usual rule (99% of the keep/drop decisions equal, disagreements within the
oracle's tie band) against both oracle runs.  Deviations and logits: normwise
within 2e-2."""
import numpy as np
import pytest
import torch

import cbinputs
import oracle
from oracle.blend import fp8_e4m3
from cacheblend_selective_recompute_amd import api

from gpu_helpers import check_sets, fp8_close as _fp8_close, ints, rel, say, to_dev, to_np

pytestmark = pytest.mark.gpu

MINI8B = cbinputs.ModelShape("mini-8b-heads", 3, 1024, 8, 2, 128, 3584, 32000, 500000.0, dtype="bf16")
# head_dim 64: the attention reads the FP8 cache through the register-staged kernel
# (head_dim 128 layers are widened to bf16 first and read by the LDS-staged one)
MINI64 = cbinputs.ModelShape("mini-hd64", 3, 512, 8, 2, 64, 1792, 32000, 10000.0, dtype="bf16")
KS, VS = 2.0 ** -5, 2.0 ** -5          # grid up to 14: the K/V of unit-RMS rows fit


def _om(shape, w, ks=KS, vs=VS):
    m = oracle.OracleModel.from_shape(shape, w)
    m.kv_storage, m.k_scale, m.v_scale = "fp8", ks, vs
    return m


def _fp8_chunks(wl, kvs, ks=KS, vs=VS):
    return [api.ChunkSource(ints(wl.chunk_tokens[c]), api.fp8_encode(torch.from_numpy(K).cuda(), ks),
                            api.fp8_encode(torch.from_numpy(V).cuda(), vs), wl.old_starts[c], wl.new_starts[c],
                            kv_format=api.CB_KV_FP8_E4M3, k_scale=ks, v_scale=vs)
            for c, (K, V) in enumerate(kvs)]


def test_rerope_fp8():
    say("cb_rerope_k: FP8 chunks (scales 2^-4) into an FP8 cache (scales 2^-5, 2^-6), shuffled offsets")
    shape = MINI8B
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=4, shape=shape, chunk_len=96, n_query=8)
    rng = np.random.default_rng(4)
    kvs = []
    for ln in wl.chunk_lens:
        dims = (shape.n_layers, ln, shape.n_kv_heads, shape.head_dim)
        kvs.append((fp8_e4m3(rng.standard_normal(dims) * 2 / 2 ** -4) * 2 ** -4,
                    fp8_e4m3(rng.standard_normal(dims) * 2 / 2 ** -4) * 2 ** -4))
    chunks = _fp8_chunks(wl, [(K.astype(np.float32), V.astype(np.float32)) for K, V in kvs], 2 ** -4, 2 ** -4)
    T = wl.n_total
    dst = api.PagedKV(shape, T, 16, fill=0.0, kv_format=api.CB_KV_FP8_E4M3, k_scale=2 ** -5, v_scale=2 ** -6)
    api.cb_rerope_k(api.make_cfg(shape), chunks, dst, api.CB_COPY_V)
    torch.cuda.synchronize()
    K, V = dst.logical(T)
    K, V = to_np(K), to_np(V)
    for c, (Kc, Vc) in enumerate(kvs):
        n, p, ln = wl.new_starts[c], wl.old_starts[c], wl.chunk_lens[c]
        ref_k = oracle.rerope(Kc, n - p, shape.rope_theta, "fp8", 2 ** -5)
        _fp8_close(K[:, n:n + ln], ref_k, 2 ** -5, f"chunk {c} K (delta {n - p})", min_equal=0.995)   # one step
        # V: moved from the 2^-4 grid to the 2^-6 grid; power-of-two scales make it exact
        assert np.array_equal(V[:, n:n + ln], oracle.store_round(Vc, "fp8", 2 ** -6))
    # rotation 0 and equal scales: a byte copy
    same = api.PagedKV(shape, T, 16, fill=0.0, kv_format=api.CB_KV_FP8_E4M3, k_scale=2 ** -4, v_scale=2 ** -4)
    zero = [api.ChunkSource(c.tokens, c.k, c.v, c.new_start, c.new_start, kv_format=c.kv_format, k_scale=c.k_scale,
                            v_scale=c.v_scale) for c in chunks]
    api.cb_rerope_k(api.make_cfg(shape), zero, same, api.CB_COPY_V)
    torch.cuda.synchronize()
    for c in zero:
        rows = same.slots(np.arange(c.new_start, c.new_start + c.len))
        assert torch.equal(same.k[:, rows], c.k) and torch.equal(same.v[:, rows], c.v)


def test_deviation_fp8():
    say("cb_kv_deviation: fresh fp32 rows against an FP8 cache")
    shape = MINI8B
    rng = np.random.default_rng(5)
    T, n = 300, 200
    kvw = shape.kv_width
    cache = api.PagedKV(shape, T, 16, fill=0.0, kv_format=api.CB_KV_FP8_E4M3, k_scale=KS, v_scale=VS)
    Kc = fp8_e4m3(rng.standard_normal((T, shape.n_kv_heads, shape.head_dim)) / KS) * KS
    Vc = fp8_e4m3(rng.standard_normal((T, shape.n_kv_heads, shape.head_dim)) / VS) * VS
    idx = cache.slots(np.arange(T))
    cache.k[1, idx] = api.fp8_encode(torch.from_numpy(Kc).cuda(), KS)
    cache.v[1, idx] = api.fp8_encode(torch.from_numpy(Vc).cuda(), VS)
    pos = np.sort(rng.choice(T, size=n, replace=False))
    kf = rng.standard_normal((n, kvw)).astype(np.float32)
    vf = rng.standard_normal((n, kvw)).astype(np.float32)
    dev = torch.empty(n, device="cuda")
    api.cb_kv_deviation(api.make_cfg(shape), 1, torch.from_numpy(kf).cuda(), torch.from_numpy(vf).cuda(), ints(pos),
                        cache, dev)
    torch.cuda.synchronize()
    ref = oracle.kv_deviation(kf.reshape(n, shape.n_kv_heads, -1), vf.reshape(n, shape.n_kv_heads, -1),
                              Kc[pos], Vc[pos])
    e = rel(to_np(dev), ref)
    say(f"  deviation rel {e:.2e}")
    assert e < 1e-5


def _blend(shape, wl, w, kvs, ks, ch, seed, steps=0, kscale=KS, vscale=VS):
    m = api.DeviceModel.from_numpy(shape, w)
    T = wl.n_total
    table, n_phys = cbinputs.paged_layout(T + steps, 16, seed, key=77, spare_blocks=5)
    kv = api.PagedKV(shape, T + steps, 16, table, n_phys, fill=0.0, kv_format=api.CB_KV_FP8_E4M3, k_scale=kscale,
                     v_scale=vscale)
    logits = torch.empty(shape.vocab, device="cuda")
    N = wl.n_ctx
    hk = torch.full((shape.n_layers, N), -1, dtype=torch.int32, device="cuda")
    dv = torch.full((shape.n_layers, N), -1.0, device="cuda")
    api.cb_blend_prefill(m, _fp8_chunks(wl, kvs, kscale, vscale), ints(wl.query_tokens), api.BlendParams(ks, ch), kv,
                         logits, hk, dv)
    torch.cuda.synchronize()
    return m, kv, logits, hk.cpu().numpy(), to_np(dv)


@pytest.mark.parametrize("shape,kscale,vscale", [(MINI8B, KS, VS), (MINI8B, 0.029, 0.037), (MINI64, 0.029, 0.037)],
                         ids=["hd128-pow2", "hd128-scaled", "hd64-scaled"])
def test_blend_mini8b_fp8(shape, kscale, vscale):
    say(f"blend: {shape.name} bf16 model, FP8 cache (scales {kscale:g}, {vscale:g}), 4 chunks x 128 shuffled, q 16, r 15%")
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=6, shape=shape, chunk_len=128, n_query=16)
    w = cbinputs.model_weights(shape, 6)
    om = _om(shape, w, kscale, vscale)
    kvs = [oracle.chunk_prefill(om, t, p) for t, p in zip(wl.chunk_tokens, wl.old_starts)]
    kvs = [(K.astype(np.float32), V.astype(np.float32)) for K, V in kvs]
    ks, ch = wl.schedule()
    m, kv, logits, hk, dv = _blend(shape, wl, w, kvs, ks, ch, 6, kscale=kscale, vscale=vscale)
    force = {l: hk[l, :ks[l]] for l in range(1, shape.n_layers) if ch[l]}
    chunks = [(wl.chunk_tokens[c], kvs[c][0], kvs[c][1], wl.old_starts[c], wl.new_starts[c]) for c in range(len(kvs))]
    with oracle.operands("bf16"):
        o16 = oracle.blend_prefill(om, chunks, wl.query_tokens, ks, ch, force_sets=force)
    o32 = oracle.blend_prefill(om, chunks, wl.query_tokens, ks, ch, force_sets=force)
    for l in range(1, shape.n_layers):
        for lab, o in (("bf16 operands", o16), ("float32", o32)):
            cand, dev = o["devs"][l]
            gd = dv[l, cand]
            e = rel(gd, dev)
            say(f"  layer {l} [{lab}]: deviation rel {e:.2e}")
            assert e < 2e-2
            sc = float(np.mean(np.sum(o["K"][l, cand].astype(np.float64) ** 2, axis=(1, 2)) +
                               np.sum(o["V"][l, cand].astype(np.float64) ** 2, axis=(1, 2))))
            check_sets(hk[l, :ks[l]], oracle.select_hkvd(dev, cand, ks[l]), cand, dev, ks[l], sc, f"layer {l} [{lab}]")
    K, V = kv.logical(wl.n_total)
    K, V = to_np(K), to_np(V)
    for l in range(shape.n_layers):
        if l == 0:
            _fp8_close(K[l], o16["K"][l], kscale, f"layer {l} K")
            _fp8_close(V[l], o16["V"][l], vscale, f"layer {l} V")
        else:
            dk = float(np.max(np.abs(o16["K"][l] - o32["K"][l])))
            dvv = float(np.max(np.abs(o16["V"][l] - o32["V"][l])))
            _fp8_close(K[l], o16["K"][l], kscale, f"layer {l} K", min_equal=0.97, extra=dk)
            _fp8_close(V[l], o16["V"][l], vscale, f"layer {l} V", min_equal=0.97, extra=dvv)
    el, el32 = rel(to_np(logits), o16["logits"]), rel(to_np(logits), o32["logits"])
    say(f"  logits rel {el:.2e} (bf16 operands), {el32:.2e} (float32)")
    assert el < 2e-2 and el32 < 2e-2


def test_blend_r0_fp8_keeps_reroped_context():
    say("blend: r = 0% over an FP8 cache leaves the re-RoPE'd context untouched")
    shape = MINI8B
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=7, ratio=0.0, shape=shape, chunk_len=96, n_query=8)
    kv32 = cbinputs.synthetic_chunk_kv(shape, wl.chunk_lens, 7)
    kvs = [((fp8_e4m3(K / KS) * KS).astype(np.float32), (fp8_e4m3(V / VS) * VS).astype(np.float32)) for K, V in kv32]
    ks, ch = wl.schedule()
    w = cbinputs.model_weights(shape, 7)
    m, kv, logits, hk, dv = _blend(shape, wl, w, kvs, ks, ch, 7)
    ref = api.PagedKV(shape, wl.n_total, 16, fill=0.0, kv_format=api.CB_KV_FP8_E4M3, k_scale=KS, v_scale=VS)
    api.cb_rerope_k(api.make_cfg(shape), _fp8_chunks(wl, kvs), ref, api.CB_COPY_V)
    torch.cuda.synchronize()
    N = wl.n_ctx
    a = kv.k[:, kv.slots(np.arange(N))]
    b = ref.k[:, ref.slots(np.arange(N))]
    assert torch.equal(a, b)
    assert torch.equal(kv.v[:, kv.slots(np.arange(N))], ref.v[:, ref.slots(np.arange(N))])


def test_decode_fp8():
    say("decode: mini-8B bf16 model on an FP8 blended cache, 3 steps")
    shape = MINI8B
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=8, shape=shape, chunk_len=96, n_query=8)
    w = cbinputs.model_weights(shape, 8)
    om = _om(shape, w)
    kvs = [oracle.chunk_prefill(om, t, p) for t, p in zip(wl.chunk_tokens, wl.old_starts)]
    kvs = [(K.astype(np.float32), V.astype(np.float32)) for K, V in kvs]
    ks, ch = wl.schedule()
    steps = 3
    m, kv, logits, hk, dv = _blend(shape, wl, w, kvs, ks, ch, 8, steps=steps)
    T = wl.n_total
    K, V = kv.logical(T + steps)
    Kb, Vb = to_np(K), to_np(V)
    ws = api.Workspace(api.cb_decode_workspace_bytes(m.cfg))
    rng = np.random.default_rng(9)
    for i in range(steps):
        tok, pos = int(rng.integers(0, shape.vocab)), T + i
        api.cb_decode_step(m, kv, pos, ints([tok]), logits, ws)
        torch.cuda.synchronize()
        # both oracle runs decode on the GPU's cache (every row up to pos - 1 as stored)
        K16, V16 = Kb.copy(), Vb.copy()
        with oracle.operands("bf16"):
            lo16 = oracle.decode_step(om, K16, V16, tok, pos)
        lo = oracle.decode_step(om, Kb, Vb, tok, pos)
        K, V = kv.logical(pos + 1)
        el, el32 = rel(to_np(logits), lo16), rel(to_np(logits), lo)
        say(f"  step {i} (pos {pos}): logits {el:.2e} (bf16 operands), {el32:.2e} (float32)")
        assert el < 2e-2 and el32 < 2e-2
        # the appended row: layer 0 within one grid step of the bf16-operand oracle (99%
        # equal).  The decode kernel weights V with float32 softmax weights (the prefill
        # rounds them to bf16 for the matrix cores), so from layer 1 on a decode row is
        # about as far from either oracle run as the two runs are from each other (88%
        # of the elements on the same grid point): one grid step plus the distance
        # between the runs, and 80% equal
        gk, gv = to_np(K[:, pos]), to_np(V[:, pos])
        _fp8_close(gk[0], K16[0, pos], KS, f"step {i} K row, layer 0")
        _fp8_close(gv[0], V16[0, pos], VS, f"step {i} V row, layer 0")
        for l in range(1, shape.n_layers):
            for lab, g, o16r, o32r, sc in (("K", gk[l], K16[l, pos], Kb[l, pos], KS), ("V", gv[l], V16[l, pos], Vb[l, pos], VS)):
                say(f"  step {i} {lab} row, layer {l}: the two oracle runs share {float(np.mean(o16r == o32r)):.4f} "
                    f"of the grid points, the GPU and the float32 run {float(np.mean(g == o32r)):.4f}")
                _fp8_close(g, o16r, sc, f"step {i} {lab} row, layer {l}", min_equal=0.8,
                           extra=float(np.max(np.abs(o16r - o32r))))
        Kb[:, pos], Vb[:, pos] = gk, gv
