"""GPU parity of the standalone entry points against the oracle:
cb_rerope_k, cb_kv_deviation, cb_select_hkvd (through the C ABI)."""
import numpy as np
import pytest
import torch

import cbinputs
import oracle
from cacheblend_selective_recompute_amd import api

from gpu_helpers import blended_cache, device_chunks, ints, rel, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _bf16_ulp(x):
    # spacing of bf16 numbers around |x| (normal range)
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 2.0 ** (e - 7)


def _rerope_case(shape, wl, paged_src, paged_dst, seed, sample=None):
    kvs = cbinputs.synthetic_chunk_kv(shape, wl.chunk_lens, seed)
    chunks = device_chunks(shape, wl, kvs, paged_src=paged_src, seed=seed)
    T = wl.n_ctx
    dst = blended_cache(shape, T, paged=paged_dst, seed=seed, fill=0.0)
    cfg = api.make_cfg(shape)
    api.cb_rerope_k(cfg, chunks, dst, api.CB_COPY_V)
    torch.cuda.synchronize()
    for c, (K, V) in enumerate(kvs):
        ln = len(wl.chunk_tokens[c])
        delta = wl.new_starts[c] - wl.old_starts[c]
        toks = np.arange(ln) if sample is None else np.unique(
            np.random.default_rng(seed + c).integers(0, ln, size=sample))
        pos = wl.new_starts[c] + toks
        idx = dst.slots(pos)
        gk = to_np(dst.k[:, idx])
        gv = to_np(dst.v[:, idx])
        ref_k = oracle.rerope(K[:, toks], delta, shape.rope_theta, shape.dtype)
        ref_v = V[:, toks].astype(np.float64)
        assert np.array_equal(gv, ref_v), f"chunk {c}: V must be copied bitwise"
        # both sides rotate with the same float32 cos/sin (float64 angle, rounded once)
        # and the same float32 operations (each product rounded, then the sum: the
        # kernel fuses no multiply-add there), then round to the storage dtype, so K is
        # bitwise the oracle's
        diff = gk != ref_k
        if shape.dtype == "bf16" and diff.any():
            say(f"  chunk {c}: {int(diff.sum())} K elements differ, largest "
                f"{float(np.max(np.abs(gk - ref_k)[diff] / _bf16_ulp(ref_k)[diff])):.1f} bf16 ulp")
        assert not diff.any(), f"chunk {c}: {int(diff.sum())} of {diff.size} K elements differ from the oracle"
        say(f"  chunk {c}: K and V bitwise equal to the oracle ({gk.size} elements)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True])
def test_rerope_small_ragged(dtype, paged):
    say(f"rerope small dtype={dtype} paged={paged}")
    shape = cbinputs.ModelShape("gqa-h128", 3, 256, 4, 2, 128, 256, 100, 500000.0, dtype=dtype)
    wl = cbinputs.make_workload("8b-16x512j-q64", seed=3, n_chunks=5, chunk_len=40, shape=shape, n_query=1)
    _rerope_case(shape, wl, paged_src=paged, paged_dst=paged, seed=3)


def test_rerope_full_8b_context_sampled():
    say("rerope 8B, 4 x 1024, 32 layers (sampled tokens)")
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=0)
    _rerope_case(wl.shape, wl, paged_src=False, paged_dst=False, seed=0, sample=64)


def test_rerope_jittered_offsets_paged():
    say("rerope 8B 16 x 512 +-25%, random stored offsets, paged (4 layers)")
    wl = cbinputs.make_workload("8b-16x512j-q64", seed=1, n_layers=4)
    _rerope_case(wl.shape, wl, paged_src=True, paged_dst=True, seed=1, sample=32)


def test_rerope_inverse_roundtrip_on_gpu():
    # rotate by delta into dst, then rotate dst back by -delta in place: identity within 1 ulp (f32: 1e-6)
    say("rerope inverse")
    shape = cbinputs.ModelShape("f32-h64", 2, 128, 2, 2, 64, 128, 10, 10000.0, dtype="f32")
    wl = cbinputs.make_workload("tiny-2x256-q32", seed=2, chunk_len=33, shape=shape, n_query=1)
    kvs = cbinputs.synthetic_chunk_kv(shape, wl.chunk_lens, 2)
    wl.old_starts = [0, 5000]
    chunks = device_chunks(shape, wl, kvs)
    dst = blended_cache(shape, wl.n_ctx, fill=0.0)
    cfg = api.make_cfg(shape)
    api.cb_rerope_k(cfg, chunks, dst, api.CB_COPY_V)
    back = [api.ChunkSource(c.tokens, dst.k[:, c.new_start:c.new_start + c.len].contiguous(),
                            dst.v[:, c.new_start:c.new_start + c.len].contiguous(), c.new_start, c.old_start)
            for c in chunks]
    out = [api.PagedKV(shape, c.len + c.new_start, 16, fill=0.0) for c in back]
    for c, o in zip(back, out):
        api.cb_rerope_k(cfg, [c], o, api.CB_COPY_V)
    torch.cuda.synchronize()
    for c, o, (K, V) in zip(back, out, kvs):
        got = to_np(o.k[:, c.new_start:c.new_start + c.len])
        assert rel(got, K) < 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deviation_matches_oracle(dtype):
    say(f"deviation dtype={dtype}")
    shape = cbinputs.SHAPES["llama3-8b"].with_dtype(dtype).with_layers(2)
    n_tok = 1000
    rng = np.random.default_rng(5)
    Kc, Vc = cbinputs.synthetic_layer_cache(shape, n_tok, seed=5)
    cache = blended_cache(shape, n_tok, paged=True, seed=5, fill=0.0)
    idx = cache.slots(np.arange(n_tok))
    cache.k[1, idx] = to_dev(Kc, dtype)
    cache.v[1, idx] = to_dev(Vc, dtype)
    pos = np.sort(rng.choice(n_tok, size=377, replace=False)).astype(np.int32)
    W = shape.kv_width
    fresh = rng.standard_normal((len(pos), 2 * W)).astype(np.float32) * 1.3
    f = torch.from_numpy(fresh).to("cuda")
    dev = torch.full((len(pos),), -1.0, device="cuda")
    api.cb_kv_deviation(api.make_cfg(shape), 1, f[:, :W], f[:, W:], ints(pos), cache, dev)
    torch.cuda.synchronize()
    ref = oracle.kv_deviation(fresh[:, :W].reshape(-1, shape.n_kv_heads, shape.head_dim),
                              fresh[:, W:].reshape(-1, shape.n_kv_heads, shape.head_dim), Kc[pos], Vc[pos])
    assert rel(to_np(dev), ref) < 1e-5
    assert np.max(np.abs(to_np(dev) - ref) / ref) < 1e-5


# up to 32768 candidates the order keys are staged in LDS; above, they are recomputed
# from the deviations on every read (40000, and a 128K context at 15%)
@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (1000, 150), (4096, 614), (4096, 4095), (32768, 4915),
                                 (32769, 4915), (40000, 6000), (131072, 19661), (5000, 0), (3000, 3000)])
def test_select_matches_oracle(n, k):
    say(f"select n={n} k={k}")
    rng = np.random.default_rng(n + k)
    dev = rng.standard_normal(n).astype(np.float32) ** 2
    if n > 10:
        dev[rng.choice(n, size=n // 5, replace=False)] = np.float32(0.5)   # a block of exact ties
        dev[rng.choice(n, size=3, replace=False)] = 0.0
    pos = np.sort(rng.choice(10 * n + 10, size=n, replace=False)).astype(np.int32)
    sel = torch.full((max(k, 1),), -7, dtype=torch.int32, device="cuda")
    slot = torch.full((max(k, 1),), -7, dtype=torch.int32, device="cuda")
    api.cb_select_hkvd(torch.from_numpy(dev).cuda(), ints(pos), k, sel, slot)
    torch.cuda.synchronize()
    ref = oracle.select_hkvd(dev.astype(np.float64), pos, k)
    if k == 0:
        assert sel.cpu().numpy()[0] == -7
        return
    got = sel.cpu().numpy()[:k]
    assert got.tolist() == ref.tolist()
    assert np.array_equal(pos[slot.cpu().numpy()[:k]], got)


def test_select_all_equal_takes_smallest_positions():
    say("select all-equal")
    n, k = 2048, 100
    dev = np.full(n, 3.0, dtype=np.float32)
    pos = np.arange(n, dtype=np.int32) * 2
    sel = torch.empty(k, dtype=torch.int32, device="cuda")
    api.cb_select_hkvd(torch.from_numpy(dev).cuda(), ints(pos), k, sel)
    torch.cuda.synchronize()
    assert sel.cpu().numpy().tolist() == (np.arange(k) * 2).tolist()


def _pack_reference(bits: np.ndarray, gate_up: bool) -> np.ndarray:
    """The packed layout as the header defines it, by index arithmetic on the host:
    32-row x 16-column blocks, element (r, c) of a block at ((c/8 % 2)*32 + r%32)*8 + c%8,
    gate/up 32-row blocks interleaved for gate_up, rows past the matrix zero."""
    R, C = bits.shape
    Rp = (R + 31) // 32 * 32
    prow = np.arange(Rp)
    if gate_up:
        F = R // 2
        blk = prow // 32
        src = np.where(blk % 2 == 1, F, 0) + (blk // 2) * 32 + prow % 32
    else:
        src = prow
    out = np.zeros(Rp * C, dtype=np.uint16)
    p, c = np.meshgrid(prow, np.arange(C), indexing="ij")
    off = ((p // 32) * (C // 16) + c // 16) * 512 + (((c // 8) % 2) * 32 + p % 32) * 8 + c % 8
    valid = src[p] < R
    out[off[valid]] = bits[src[p][valid], c[valid]]
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("rows,cols,gate_up", [(70, 48, False), (32, 16, False), (256, 4096, False),
                                               (128, 80, True), (2 * 3584, 1024, True)])
def test_pack_weight_bit_exact(rows, cols, gate_up):
    say(f"cb_pack_weight rows {rows} cols {cols} gate_up {gate_up}")
    rng = np.random.default_rng(rows * 31 + cols)
    bits = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
    w = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    got = api.cb_pack_weight(w, gate_up=gate_up)
    torch.cuda.synchronize()
    got_bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_bits, _pack_reference(bits, gate_up))
