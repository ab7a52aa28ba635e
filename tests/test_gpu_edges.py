"""GPU parity of cb_blend_prefill against the oracle on the method's degenerate
and ragged inputs ([CB] "选 token" and "位置恢复": the blend is defined for any
number of chunks of any length, any stored offset and any query length >= 1):

* a single chunk (nothing to blend; the context is one re-RoPE'd prefix);
* a one-token query (the final logits come from that row alone);
* ragged chunk lengths, a one-token chunk among them, stored at offsets both
  before and after their new positions;
* more chunks than one re-RoPE launch takes (40 > 32);
* a ratio so small that one context token is recomputed per layer, and one so
  large that all but one are;
* pages of 1, 8, 12 (not a power of two) and 32 tokens for the chunk sources and
  the blended cache: below 16 keys or off powers of two the attention reads through
  the earlier LDS-staged kernel and a decode row looks each key's page up; two decode
  steps follow each blend.

Chunk caches come from the oracle's own chunk prefill; the GPU's kept sets are
validated against the oracle's ranking and then imposed (as in test_gpu_blend)."""
import numpy as np
import pytest

import cbinputs

from gpu_helpers import say
from test_gpu_blend import MINI8B, _compare, _oracle_ref, _oracle_setup, _run_blend
from test_gpu_decode import _blend_then_decode

pytestmark = pytest.mark.gpu

TINY = cbinputs.SHAPES["tiny-2l-d256"]


def _workload(shape, lens, old, order, n_query, ratio, seed):
    """A workload with explicit chunk lengths, stored offsets and placement order."""
    rng = np.random.default_rng(seed)
    toks = [rng.integers(0, shape.vocab, size=ln).astype(np.int32) for ln in lens]
    new = [0] * len(lens)
    cur = 0
    for c in order:
        new[c] = cur
        cur += lens[c]
    q = rng.integers(0, shape.vocab, size=n_query).astype(np.int32)
    return cbinputs.Workload(name="edge", shape=shape, chunk_tokens=toks, old_starts=list(old), new_starts=new,
                             query_tokens=q, ratio=ratio, seed=seed)


def _check(shape, wl, tol, label, seed, paged=False):
    m, kvs = _oracle_setup(shape, wl, seed)
    ks, ch = wl.schedule()
    say(f"{label}: N {wl.n_ctx}, Q {wl.n_query}, {len(wl.chunk_lens)} chunks, k {ks[1:]}")
    g = _run_blend(shape, wl, kvs, ks, ch, paged=paged, paged_src=paged, seed=seed)
    _compare(shape, wl, g, _oracle_ref(m, wl, kvs, ks, ch, g), ks, tol, label)
    return g


def test_blend_single_chunk_fp32():
    wl = _workload(TINY, [300], [41], [0], n_query=5, ratio=0.15, seed=11)
    g = _check(TINY, wl, 1e-4, "single chunk", seed=11)
    # one chunk moved as a whole keeps every relative position, so its cached K/V are
    # what a fresh prefill of the prefix gives: the deviations are rounding noise
    N = wl.n_ctx
    scale = float(np.mean(np.sum(g["K"][1, :N] ** 2, axis=(1, 2)) + np.sum(g["V"][1, :N] ** 2, axis=(1, 2))))
    worst = float(np.max(g["dev"][1, :N]))
    say(f"  single chunk: largest layer-1 deviation {worst:.3g} (mean |k|^2 + |v|^2 = {scale:.3g})")
    assert worst <= 1e-6 * scale


def test_blend_one_query_token_fp32():
    wl = _workload(TINY, [100, 150, 90], [0, 512, 7], [2, 0, 1], n_query=1, ratio=0.15, seed=12)
    _check(TINY, wl, 1e-4, "one query token", seed=12)


@pytest.mark.parametrize("ratio", [0.002, 0.997])
def test_blend_one_or_all_but_one_recomputed_fp32(ratio):
    wl = _workload(TINY, [150, 150], [0, 300], [1, 0], n_query=4, ratio=ratio, seed=13)
    assert wl.k in (1, wl.n_ctx - 1)
    _check(TINY, wl, 1e-4, f"k {wl.k} of {wl.n_ctx}", seed=13)


def test_blend_ragged_chunks_bf16_paged():
    # a one-token chunk; lengths off every block size; stored before and after the new place
    lens = [1, 37, 129, 64, 200, 3]
    old = [3000, 0, 17, 2048, 5, 999]
    wl = _workload(MINI8B, lens, old, [3, 0, 5, 1, 4, 2], n_query=7, ratio=0.15, seed=14)
    _check(MINI8B, wl, 2e-2, "ragged chunks", seed=14, paged=True)


def test_blend_forty_chunks_bf16_paged():
    rng = np.random.default_rng(15)
    lens = [int(x) for x in rng.integers(10, 31, size=40)]
    old = [int(x) for x in rng.integers(0, 4096, size=40)]
    wl = _workload(MINI8B, lens, old, [int(x) for x in rng.permutation(40)], n_query=8, ratio=0.15, seed=15)
    _check(MINI8B, wl, 2e-2, "40 chunks", seed=15, paged=True)


@pytest.mark.parametrize("bs", [1, 8, 12, 32])
def test_blend_and_decode_page_sizes_bf16(bs):
    seed = 30 + bs
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=seed, shape=MINI8B, chunk_len=96, n_query=8)
    m, kvs = _oracle_setup(MINI8B, wl, seed)
    ks, ch = wl.schedule()
    say(f"pages of {bs} tokens: N {wl.n_ctx}, Q {wl.n_query}, k {ks[1:]}")
    g = _run_blend(MINI8B, wl, kvs, ks, ch, paged=True, paged_src=True, seed=seed, bs=bs)
    _compare(MINI8B, wl, g, _oracle_ref(m, wl, kvs, ks, ch, g), ks, 2e-2, f"pages of {bs}")
    _blend_then_decode(MINI8B, wl, cbinputs.model_weights(MINI8B, seed), kvs, 2, True, 2e-2, f"pages of {bs}", seed,
                       bs=bs)
