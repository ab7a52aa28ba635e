"""GPU checks of the layer-pipelined prefill (cb_blend_prefill_streamed): with
the chunk caches in page-locked host memory, fed one layer at a time on a copy
stream, every output must be bitwise the one cb_blend_prefill produces from
the same caches on the device; on the tiny fp32 decoder it is also compared
with the oracle.  Models with more layers than ring slots (3) exercise the
slot reuse and its waits; two calls enqueued back to back on one stream with
one workspace exercise the wait of a call's first copies for the previous
call's use of the ring."""
import numpy as np
import pytest
import torch

import cbinputs
import oracle
from cacheblend_selective_recompute_amd import api

from gpu_helpers import blended_cache, device_chunks, ints, oracle_chunks, rel, say, to_np

pytestmark = pytest.mark.gpu

MINI8B = cbinputs.ModelShape("mini-8b-heads", 6, 1024, 8, 2, 128, 3584, 32000, 500000.0, dtype="bf16")


def _host_chunks(chunks):
    out = []
    for c in chunks:
        hk = torch.empty(c.k.shape, dtype=c.k.dtype, pin_memory=True)
        hv = torch.empty(c.v.shape, dtype=c.v.dtype, pin_memory=True)
        hk.copy_(c.k.cpu())
        hv.copy_(c.v.cpu())
        out.append(api.HostChunk(c.tokens, hk, hv, c.old_start, c.new_start))
    return out


def _both(shape, m, chunks, wl, ks, ch, paged, seed):
    T, N = wl.n_total, wl.n_ctx
    res = []
    for streamed in (False, True):
        kv = blended_cache(shape, T, paged=paged, seed=seed, fill=0.0)
        logits = torch.empty(shape.vocab, device="cuda")
        hk = torch.full((shape.n_layers, N), -1, dtype=torch.int32, device="cuda")
        dv = torch.full((shape.n_layers, N), -1.0, device="cuda")
        keep = None
        if streamed:
            host = _host_chunks(chunks)
            keep = (host, api.cb_blend_prefill_streamed(m, host, ints(wl.query_tokens), api.BlendParams(ks, ch), kv,
                                                        logits, hk, dv, copy_stream=torch.cuda.Stream()))
        else:
            api.cb_blend_prefill(m, chunks, ints(wl.query_tokens), api.BlendParams(ks, ch), kv, logits, hk, dv)
        torch.cuda.synchronize()
        del keep
        K, V = kv.logical(T)
        res.append({"K": K, "V": V, "logits": logits, "hkvd": hk, "dev": dv})
    return res


def _assert_same(a, b, label):
    for key in ("K", "V", "logits", "hkvd", "dev"):
        assert torch.equal(a[key], b[key]), f"{label}: {key} differs between the streamed and the device prefill"
    say(f"  {label}: streamed == device prefill, bitwise")


def test_streamed_equals_device_prefill_mini8b():
    say("streamed prefill: mini-8B bf16, 6 layers, 4 chunks x 128 shuffled, q 16, paged")
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=1, shape=MINI8B, chunk_len=128, n_query=16)
    m = api.DeviceModel.from_numpy(MINI8B, cbinputs.model_weights(MINI8B, 1))
    kvs = cbinputs.synthetic_chunk_kv(MINI8B, wl.chunk_lens, 1)
    chunks = device_chunks(MINI8B, wl, kvs)
    ks, ch = wl.schedule()
    a, b = _both(MINI8B, m, chunks, wl, ks, ch, True, 1)
    _assert_same(a, b, "mini-8B")


def test_streamed_tiny_fp32_matches_oracle():
    say("streamed prefill: tiny fp32, 2 chunks x 256, q 32, against the oracle")
    wl = cbinputs.make_workload("tiny-2x256-q32", seed=0)
    shape = wl.shape
    w = cbinputs.model_weights(shape, 0)
    om = oracle.OracleModel.from_shape(shape, w)
    kvs = [oracle.chunk_prefill(om, t, p) for t, p in zip(wl.chunk_tokens, wl.old_starts)]
    kvs = [(K.astype(np.float32), V.astype(np.float32)) for K, V in kvs]
    m = api.DeviceModel.from_numpy(shape, w)
    chunks = device_chunks(shape, wl, kvs)
    ks, ch = wl.schedule()
    a, b = _both(shape, m, chunks, wl, ks, ch, False, 0)
    _assert_same(a, b, "tiny")
    force = {l: b["hkvd"][l, :ks[l]].cpu().numpy() for l in range(1, shape.n_layers) if ch[l]}
    o = oracle.blend_prefill(om, oracle_chunks(wl, kvs), wl.query_tokens, ks, ch, force_sets=force)
    el = rel(to_np(b["logits"]), o["logits"])
    ek = max(rel(to_np(b["K"][l]), o["K"][l]) for l in range(shape.n_layers))
    say(f"  tiny streamed vs oracle: logits {el:.2e}, K {ek:.2e}")
    assert el < 1e-4 and ek < 1e-4


def test_streamed_equals_device_prefill_full_8b():
    say("streamed prefill: full 8B shape, 4 x 1024 + 64, r 15%, 32 layers through the 3-slot ring")
    shape = cbinputs.SHAPES["llama3-8b"]
    wl = cbinputs.make_workload("8b-4x1024-q64", seed=0)
    m = api.DeviceModel.from_tensors(shape, cbinputs.torch_device_weights(shape, 0))
    kvs = cbinputs.torch_device_chunk_kv(shape, wl.chunk_lens, 0)
    chunks = [api.ChunkSource(ints(wl.chunk_tokens[c]), kvs[c][0], kvs[c][1], wl.old_starts[c], wl.new_starts[c])
              for c in range(len(kvs))]
    ks, ch = wl.schedule()
    a, b = _both(shape, m, chunks, wl, ks, ch, True, 0)
    _assert_same(a, b, "8B")


def test_streamed_back_to_back_shared_workspace():
    say("streamed prefill: two mini-8B calls back to back on a side stream, one workspace, one copy stream")
    m = api.DeviceModel.from_numpy(MINI8B, cbinputs.model_weights(MINI8B, 21))
    cases = []
    for seed in (21, 22):
        wl = cbinputs.make_workload("8b-4x1024-q64", seed=seed, shape=MINI8B, chunk_len=128, n_query=16)
        kvs = cbinputs.synthetic_chunk_kv(MINI8B, wl.chunk_lens, seed)
        chunks = device_chunks(MINI8B, wl, kvs)
        cases.append((wl, chunks, _host_chunks(chunks), ints(wl.query_tokens)))
    wl0 = cases[0][0]
    need = api.cb_streamed_workspace_bytes(m.cfg, wl0.n_ctx, wl0.n_query, len(cases[0][1]))
    ws = api.Workspace(need)

    def outputs(wl):
        kv = blended_cache(MINI8B, wl.n_total, paged=True, seed=5, fill=0.0)
        return (kv, torch.empty(MINI8B.vocab, device="cuda"),
                torch.full((MINI8B.n_layers, wl.n_ctx), -1, dtype=torch.int32, device="cuda"),
                torch.full((MINI8B.n_layers, wl.n_ctx), -1.0, device="cuda"))

    refs = []
    for wl, chunks, _, q in cases:
        kv, lg, hk, dv = outputs(wl)
        ks, ch = wl.schedule()
        api.cb_blend_prefill(m, chunks, q, api.BlendParams(ks, ch), kv, lg, hk, dv)
        torch.cuda.synchronize()
        K, V = kv.logical(wl.n_total)
        refs.append((K.clone(), V.clone(), lg.clone(), hk.clone(), dv.clone()))
    outs = [outputs(wl) for wl, _, _, _ in cases]
    s, cs = torch.cuda.Stream(), torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    keep = []
    for (wl, _, host, q), (kv, lg, hk, dv) in zip(cases, outs):
        ks, ch = wl.schedule()
        keep.append(api.cb_blend_prefill_streamed(m, host, q, api.BlendParams(ks, ch), kv, lg, hk, dv, ws=ws,
                                                  stream=s, copy_stream=cs))
    torch.cuda.synchronize()
    del keep
    for i, ((wl, _, _, _), (kv, lg, hk, dv), ref) in enumerate(zip(cases, outs, refs)):
        K, V = kv.logical(wl.n_total)
        for name, a, b in zip(("K", "V", "logits", "hkvd", "dev"), (K, V, lg, hk, dv), ref):
            assert torch.equal(a, b), f"call {i}: {name} differs from the device prefill"
        say(f"  call {i}: streamed == device prefill, bitwise")

