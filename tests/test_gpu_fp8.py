"""GPU parity with an 8-bit (FP8 E4M3) KV cache, through the C ABI.

Element rule for stored FP8 values: the GPU's stored value differs from the
oracle's by at most one grid step at that value plus the bf16 path's own
normwise error (2e-2 of the tensor's largest value, the tolerance of the bf16
cache tests: fresh values computed from bf16 activations differ from the
oracle's fp64 ones by that much in absolute terms, which small elements see
as several of their grid steps), and at least 97% of the elements are equal.  Where the input is already on the grid (re-RoPE
with rotation 0, V moved between caches with power-of-two scales) the bytes are
equal.  Logits: normwise within 5e-2 (two bf16 paths over FP8 caches whose
elements may differ by one step).  Deviations are compared normwise (2e-2);
HKVD sets by the usual rule with the tie band widened to the FP8 noise of the
deviations (section on deviation precision of the CacheBlend page: FP8 caches
make the ranking jitter)."""
import numpy as np
import pytest
import torch

import cbinputs
import oracle
from oracle.blend import fp8_e4m3
from cacheblend_selective_recompute_amd import api

from gpu_helpers import fp8_close as _fp8_close, ints, rel, say, to_dev, to_np

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
        _fp8_close(K[:, n:n + ln], ref_k, 2 ** -5, f"chunk {c} K (delta {n - p})", min_equal=0.995)
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


def _tie_band_sets(gset, cand, dev_o, dev_g, k, label):
    """Keep/drop agreement >= 97%; every disagreement lies where the GPU's and the
    oracle's deviations of the token both sit within their noise of the k-th."""
    g = set(int(x) for x in gset)
    o = set(int(x) for x in oracle.select_hkvd(dev_o, cand, k))
    assert len(g) == k
    dmap_o = {int(p): float(d) for p, d in zip(cand, dev_o)}
    dk = np.sort(np.asarray(dev_o))[::-1][k - 1]
    noise = float(np.max(np.abs(dev_g - dev_o)))
    for p in g ^ o:
        assert abs(dmap_o[p] - dk) <= 2 * noise + 1e-3 * dk, f"{label}: disagreement at {p} outside the noise band"
    frac = 1.0 - len(g ^ o) / len(cand)
    say(f"  {label}: decision agreement {frac:.4f} (deviation noise {noise / dk:.2e} of the k-th)")
    assert frac >= 0.97


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
    o = oracle.blend_prefill(om, [(wl.chunk_tokens[c], kvs[c][0], kvs[c][1], wl.old_starts[c], wl.new_starts[c])
                                  for c in range(len(kvs))], wl.query_tokens, ks, ch, force_sets=force)
    for l in range(1, shape.n_layers):
        cand, dev = o["devs"][l]
        gd = dv[l, cand]
        e = rel(gd, dev)
        say(f"  layer {l}: deviation rel {e:.2e}")
        assert e < 2e-2
        _tie_band_sets(hk[l, :ks[l]], cand, dev, gd, ks[l], f"layer {l}")
    K, V = kv.logical(wl.n_total)
    K, V = to_np(K), to_np(V)
    for l in range(shape.n_layers):
        _fp8_close(K[l], o["K"][l], kscale, f"layer {l} K")
        _fp8_close(V[l], o["V"][l], vscale, f"layer {l} V")
    el = rel(to_np(logits), o["logits"])
    say(f"  logits rel {el:.2e}")
    assert el < 5e-2


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
        lo = oracle.decode_step(om, Kb, Vb, tok, pos)
        K, V = kv.logical(pos + 1)
        el = rel(to_np(logits), lo)
        say(f"  step {i} (pos {pos}): logits {el:.2e}")
        assert el < 5e-2
        # every element of a decode row is fresh (no re-RoPE'd context to share), after
        # three bf16 layers: ~1e-2 relative difference against a 1/8 relative grid step
        # moves roughly one element in ten to a neighbouring grid value
        _fp8_close(to_np(K[:, pos]), Kb[:, pos], KS, f"step {i} K row", min_equal=0.8)
        _fp8_close(to_np(V[:, pos]), Vb[:, pos], VS, f"step {i} V row", min_equal=0.8)
        Kb[:, pos], Vb[:, pos] = to_np(K[:, pos]), to_np(V[:, pos])
