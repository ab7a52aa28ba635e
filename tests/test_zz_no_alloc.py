"""cb_rerope_k_noalloc (static per-GPU scratch, no workspace) against
cb_rerope_k (caller workspace) through the C ABI: the same kernels and the same
rotation table, so the blended caches must be bitwise equal; two calls in a
row, the second with fewer chunks and tokens, each compared with its own
cb_rerope_k run."""
import numpy as np
import pytest
import torch

import cbinputs
from cacheblend_selective_recompute_amd import api

from gpu_helpers import blended_cache, device_chunks, say

pytestmark = pytest.mark.gpu


def _case(shape, wl, seed, paged):
    kvs = cbinputs.synthetic_chunk_kv(shape, wl.chunk_lens, seed)
    chunks = device_chunks(shape, wl, kvs, paged_src=paged, seed=seed)
    T = wl.n_ctx
    cfg = api.make_cfg(shape)
    a = blended_cache(shape, T, paged=paged, seed=seed, fill=0.0)
    b = blended_cache(shape, T, paged=paged, seed=seed, fill=0.0)
    api.cb_rerope_k(cfg, chunks, a, api.CB_COPY_V)
    api.cb_rerope_k_noalloc(cfg, chunks, b, api.CB_COPY_V)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_rerope_equals_workspace_rerope_twice(dtype):
    shape = cbinputs.SHAPES["llama3-8b"].with_layers(4).with_dtype(dtype)
    # first call: 40 jittered chunks (two launch batches), paged source and destination
    say(f"cb_rerope_k_noalloc {dtype}: 40 chunks, then 3 chunks")
    wl = cbinputs.make_workload("8b-16x512j-q64", seed=11, shape=shape, n_chunks=40, chunk_len=96)
    a, b = _case(shape, wl, 11, paged=True)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert bool((a.k != 0).any())
    # second call, smaller: 3 chunks, contiguous
    wl2 = cbinputs.make_workload("8b-16x512j-q64", seed=12, shape=shape, n_chunks=3, chunk_len=40)
    a2, b2 = _case(shape, wl2, 12, paged=False)
    assert torch.equal(a2.k, b2.k) and torch.equal(a2.v, b2.v)
    assert bool((a2.k != 0).any())
