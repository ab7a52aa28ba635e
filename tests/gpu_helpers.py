"""Shared helpers for the GPU parity tests: seeded inputs -> device tensors,
oracle chunk tuples, and the comparison rules.

Tolerances (normwise, max|gpu - ref| / max|ref|):
  * bf16 models (bf16 products, fp32 accumulation): blended K/V and logits 2e-2;
  * fp32 models: 1e-4.
HKVD sets: the keep/drop decision agrees on at least 99% of the candidate
tokens, and every disagreement lies within the tie band
|Δ_j - Δ_(k)| <= 1e-3 * Δ_(k) + eps_abs of the oracle's own deviations.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import cbinputs
from cacheblend_selective_recompute_amd import api

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(g, r) -> float:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r)) if r.size else 0.0
    return float(np.max(np.abs(g - r)) / den) if den > 0 else float(np.max(np.abs(g - r), initial=0.0))


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(api.torch_dtype(dtype))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def ints(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a), dtype=np.int32)).to(DEV)


def device_chunks(shape, wl, kvs, paged_src=False, seed=0, bs=16):
    """ChunkSource list from numpy chunk K/V ([L][len][Hkv][dh] each).

    With ``paged_src`` each chunk's K/V live in a private pool of ``bs``-token
    blocks at random physical positions."""
    out = []
    keep = []
    rng = np.random.default_rng(seed + 991)
    for c, ((K, V), toks) in enumerate(zip(kvs, wl.chunk_tokens)):
        ln = len(toks)
        if not paged_src:
            out.append(api.ChunkSource(ints(toks), to_dev(K, shape.dtype), to_dev(V, shape.dtype),
                                       wl.old_starts[c], wl.new_starts[c]))
            continue
        nb = (ln + bs - 1) // bs
        n_phys = nb + 3
        ids = rng.permutation(n_phys)[:nb].astype(np.int32)
        L = K.shape[0]
        Kp = np.zeros((L, n_phys * bs) + K.shape[2:], dtype=np.float32)
        Vp = np.zeros_like(Kp)
        for b in range(nb):
            t0, t1 = b * bs, min(ln, (b + 1) * bs)
            Kp[:, ids[b] * bs: ids[b] * bs + (t1 - t0)] = K[:, t0:t1]
            Vp[:, ids[b] * bs: ids[b] * bs + (t1 - t0)] = V[:, t0:t1]
        out.append(api.ChunkSource(ints(toks), to_dev(Kp, shape.dtype), to_dev(Vp, shape.dtype),
                                   wl.old_starts[c], wl.new_starts[c], block_ids=ints(ids), block_size=bs,
                                   layer_stride=n_phys * bs * shape.kv_width))
    return out


def blended_cache(shape, n_tokens, paged=False, seed=0, fill=None, bs=16):
    if not paged:
        return api.PagedKV(shape, n_tokens, bs, fill=fill)
    table, n_phys = cbinputs.paged_layout(n_tokens, bs, seed, key=77, spare_blocks=5)
    return api.PagedKV(shape, n_tokens, bs, table, n_phys, fill=fill)


def oracle_chunks(wl, kvs):
    return [(wl.chunk_tokens[c], kvs[c][0], kvs[c][1], wl.old_starts[c], wl.new_starts[c])
            for c in range(len(kvs))]


def check_sets(gpu_set, ora_set, cand, dev_ora, k, kv_scale_sq, label=""):
    """HKVD set rule; returns the agreement fraction.

    The GPU's k kept positions must be candidates, and every position where the
    GPU and the oracle decide differently must lie in the tie band around the
    oracle's k-th largest deviation (|d - d_k| <= 1e-3 d_k + 1e-6 mean |k|^2+|v|^2).
    The keep/drop decisions must then agree on at least 99% of the candidates,
    unless more than 1% of the candidates lie in that band: then the deviations
    do not single out one set (e.g. a single chunk, whose cached K/V differ from
    fresh ones only by rounding), any top-k within the band is correct, and only
    its validity is checked."""
    g = set(int(x) for x in gpu_set)
    o = set(int(x) for x in ora_set)
    assert len(g) == k, f"{label}: GPU kept {len(g)} != {k}"
    if k == 0:
        return 1.0
    inter = len(g & o)
    cand = np.asarray(cand)
    devs = np.asarray(dev_ora, dtype=np.float64)
    dmap = {int(p): float(d) for p, d in zip(cand, devs)}
    dk = np.sort(devs)[::-1][k - 1]
    band = 1e-3 * dk + 1e-6 * kv_scale_sq
    for p in g ^ o:
        assert p in dmap, f"{label}: position {p} is not a candidate"
        assert abs(dmap[p] - dk) <= band, f"{label}: disagreement at {p}: dev {dmap[p]:.6g} vs k-th {dk:.6g}"
    frac = 1.0 - len(g ^ o) / len(cand)
    if frac >= 0.99:
        say(f"  {label}: {inter}/{k} kept positions shared, decision agreement {frac:.4f}")
    else:
        in_band = int(np.sum(np.abs(devs - dk) <= band))
        assert in_band > 0.01 * len(cand), \
            f"{label}: the keep/drop decision agrees on only {frac:.4f} of the candidates"
        say(f"  {label}: {in_band} of {len(cand)} candidates tie within the band; the GPU's set is a valid "
            f"top-{k} of them ({inter}/{k} shared with the oracle's)")
    return frac


def fp8_grid_step(x, scale):
    """Spacing of the E4M3 grid (times scale) at each |x|."""
    a = np.abs(np.asarray(x, dtype=np.float64)) / scale
    _, E = np.frexp(np.maximum(a, 2.0 ** -9))
    return np.ldexp(1.0, np.clip(E - 1, -6, 8) - 3) * scale


def fp8_close(g, o, scale, label, min_equal=0.99, extra=0.0):
    """Stored FP8 values against the oracle's: every element within one grid step
    (times scale) of the larger of the two values, plus `extra` (0 by default: both
    sides rounded the same float32 arithmetic up to the order of its sums; a caller
    comparing with a different arithmetic passes how far that arithmetic itself
    moves the values), and at least min_equal of them on the same grid point."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    d = np.abs(g - o)
    step = np.maximum(fp8_grid_step(o, scale), fp8_grid_step(g, scale))
    ok = d <= 1.0001 * step + extra
    # equal = the same grid point; the GPU side is dequantised as code x scale in fp32
    eq = float(np.mean(d <= 1e-6 * np.abs(o))) if d.size else 1.0
    say(f"  {label}: {eq:.4f} of the elements equal, the largest difference {float(np.max(d / step, initial=0.0)):.2f} "
        f"grid steps, all within the bound: {bool(ok.all())}")
    assert ok.all(), f"{label}: {int((~ok).sum())} elements beyond the bound"
    assert eq >= min_equal, f"{label}: only {eq:.4f} equal"


def host_layer(t, shape):
    """Oracle-layout fp32 host copies of a library-layout (unpacked) layer."""
    qw, kvw, F = shape.q_width, shape.kv_width, shape.d_ff
    h = lambda x: x.float().cpu().numpy()
    qkv = h(t["w_qkv"])
    gu = h(t["w_gate_up"])
    return {"wq": qkv[:qw], "wk": qkv[qw:qw + kvw], "wv": qkv[qw + kvw:], "wo": h(t["w_o"]),
            "w_gate": gu[:F], "w_up": gu[F:], "w_down": h(t["w_down"]),
            "attn_norm": h(t["attn_norm"]), "mlp_norm": h(t["mlp_norm"])}


def paged_chunks(shape, wl, kvs, seed):
    """Chunk sources whose device K/V ([L][len][Hkv][dh] each) are moved into
    private pools of 16-token blocks under random block lists."""
    out = []
    for c, (K, V) in enumerate(kvs):
        ln = wl.chunk_lens[c]
        nb = (ln + 15) // 16
        ids, n_phys = cbinputs.paged_layout(ln, 16, seed, key=1000 + c, spare_blocks=2)
        Kp = torch.zeros((shape.n_layers, n_phys * 16, shape.n_kv_heads, shape.head_dim), dtype=K.dtype, device=DEV)
        Vp = torch.zeros_like(Kp)
        rows = torch.from_numpy((np.repeat(ids.astype(np.int64), 16) * 16 + np.tile(np.arange(16), nb))[:ln]).to(DEV)
        Kp[:, rows] = K
        Vp[:, rows] = V
        out.append(api.ChunkSource(ints(wl.chunk_tokens[c]), Kp, Vp, wl.old_starts[c], wl.new_starts[c],
                                   block_ids=ints(ids), block_size=16, layer_stride=n_phys * 16 * shape.kv_width))
    return out
