"""GPU parity of cb_blend_prefill against the oracle for every attention head
layout the bf16 path takes: query heads per KV head G = 1, 2, 4, 8, 16 at
head_dim 128 (the LDS-staged kernel) and G = 1, 4, 16 at head_dim 64 (the
register-staged kernel).  The selected tokens attend to every position up to
their own ([CB] "选 token"); GQA shares each KV head among G query heads, so
each layout stacks a different number of query rows per KV block.

Small decoders (3 layers, d_model 512) blend 4 shuffled chunks of 96 tokens
with an 8-token query at r = 15%; chunk caches come from the oracle's own chunk
prefill, and the GPU's kept sets are validated against the oracle's ranking and
then imposed (as in test_gpu_blend).  Bound: 2e-2 normwise for every layer's
blended K/V, the deviations and the logits (bf16 arithmetic).

The fp32 path (one wave per query row and head) is checked with shared KV heads
too (G = 2, 4), at 1e-4.

The same layouts then decode two tokens straight from a blended cache (the
one-row kernel at head_dim 128 with G <= 8, the general kernels otherwise),
against the oracle's decode step on a host copy of that cache (as in
test_gpu_decode)."""
import pytest

import cbinputs

from gpu_helpers import say
from test_gpu_blend import _compare, _oracle_ref, _oracle_setup, _run_blend
from test_gpu_decode import _blend_then_decode

pytestmark = pytest.mark.gpu

LAYOUTS = [  # (head_dim, query heads, KV heads, paged)
    (128, 4, 4, False),
    (128, 4, 2, True),
    (128, 16, 2, False),
    (128, 16, 1, True),
    (64, 8, 8, True),
    (64, 8, 2, False),
    (64, 16, 1, True),
]


IDS = [f"hd{h}-G{q // k}{'-paged' if p else ''}" for h, q, k, p in LAYOUTS]


def _shape(hd, nq, nkv):
    return cbinputs.ModelShape(f"hd{hd}-q{nq}-kv{nkv}", 3, 512, nq, nkv, hd, 1024, 4096, 500000.0, dtype="bf16")


@pytest.mark.parametrize("hd,nq,nkv,paged", LAYOUTS, ids=IDS)
def test_blend_head_layout_bf16(hd, nq, nkv, paged):
    shape = _shape(hd, nq, nkv)
    seed = 20 + nq + nkv + hd
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=seed, shape=shape, chunk_len=96, n_query=8)
    m, kvs = _oracle_setup(shape, wl, seed)
    ks, ch = wl.schedule()
    label = f"head_dim {hd}, G {nq // nkv} ({nq} q / {nkv} kv heads){', paged' if paged else ''}"
    say(f"{label}: N {wl.n_ctx}, Q {wl.n_query}, k {ks[1:]}")
    g = _run_blend(shape, wl, kvs, ks, ch, paged=paged, paged_src=paged, seed=seed)
    _compare(shape, wl, g, _oracle_ref(m, wl, kvs, ks, ch, g), ks, 2e-2, label)


@pytest.mark.parametrize("hd,nq,nkv,paged", LAYOUTS, ids=IDS)
def test_decode_head_layout_bf16(hd, nq, nkv, paged):
    shape = _shape(hd, nq, nkv)
    seed = 40 + nq + nkv + hd
    say(f"decode: head_dim {hd}, G {nq // nkv}{', paged' if paged else ''}, after a 4 x 96 + 8 blend, 2 steps")
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=seed, shape=shape, chunk_len=96, n_query=8)
    w = cbinputs.model_weights(shape, seed)
    kvs = cbinputs.synthetic_chunk_kv(shape, wl.chunk_lens, seed)
    _blend_then_decode(shape, wl, w, kvs, 2, paged, 2e-2, f"hd{hd} G{nq // nkv}", seed)


@pytest.mark.parametrize("nq,nkv", [(4, 2), (8, 2)], ids=["G2", "G4"])
def test_blend_gqa_fp32(nq, nkv):
    # the fp32 path's attention (one wave per query row and head) with shared KV heads
    shape = cbinputs.ModelShape(f"f32-q{nq}-kv{nkv}", 2, 256, nq, nkv, 64, 512, 1000, 10000.0, dtype="f32")
    seed = 60 + nq
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=seed, shape=shape, chunk_len=80, n_query=6)
    m, kvs = _oracle_setup(shape, wl, seed)
    ks, ch = wl.schedule()
    label = f"fp32, G {nq // nkv}"
    say(f"{label}: N {wl.n_ctx}, Q {wl.n_query}, k {ks[1:]}")
    g = _run_blend(shape, wl, kvs, ks, ch, paged=True, paged_src=True, seed=seed)
    _compare(shape, wl, g, _oracle_ref(m, wl, kvs, ks, ch, g), ks, 1e-4, label)

