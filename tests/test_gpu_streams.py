"""Two blended prefills in flight at once on two streams, each with its own
workspace, caches and outputs, give bitwise the results of the same calls run
one after the other: the library keeps no state between calls and launches
nothing outside the stream it is given (the C ABI's ownership rule).  And the
workspace's prior contents do not matter: a blend and two decode steps give the
same bits with the workspace filled with zeros and with 0xFF bytes (NaN floats,
-1 integers)."""
import pytest
import torch

import cbinputs
from cacheblend_selective_recompute_amd import api

from gpu_helpers import blended_cache, device_chunks, ints, say
from test_gpu_blend import MINI8B

pytestmark = pytest.mark.gpu


class _Case:
    def __init__(self, seed, ratio, paged):
        self.wl = cbinputs.make_workload("8b-4x1024-q64", seed=seed, ratio=ratio, shape=MINI8B, chunk_len=128,
                                         n_query=16)
        self.model = api.DeviceModel.from_numpy(MINI8B, cbinputs.model_weights(MINI8B, seed))
        kvs = cbinputs.synthetic_chunk_kv(MINI8B, self.wl.chunk_lens, seed)
        self.chunks = device_chunks(MINI8B, self.wl, kvs, paged_src=paged, seed=seed)
        self.paged, self.seed = paged, seed
        wl = self.wl
        # inputs stay alive until every call's stream has finished (the caller owns them):
        # a temporary freed at return could be handed to the other stream's next call
        # while this stream's kernels still read it
        self.q = ints(wl.query_tokens)
        self.ws = api.Workspace(api.cb_workspace_bytes(self.model.cfg, wl.n_ctx, wl.n_query, len(self.chunks)))

    def outputs(self):
        wl = self.wl
        kv = blended_cache(MINI8B, wl.n_total, paged=self.paged, seed=self.seed, fill=0.0)
        logits = torch.empty(MINI8B.vocab, device="cuda")
        hk = torch.full((MINI8B.n_layers, wl.n_ctx), -1, dtype=torch.int32, device="cuda")
        dv = torch.full((MINI8B.n_layers, wl.n_ctx), -1.0, device="cuda")
        return kv, logits, hk, dv

    def run(self, out, stream=None):
        kv, logits, hk, dv = out
        ks, ch = self.wl.schedule()
        api.cb_blend_prefill(self.model, self.chunks, self.q, api.BlendParams(ks, ch), kv,
                             logits, hk, dv, ws=self.ws, stream=stream)

    def result(self, out):
        kv, logits, hk, dv = out
        K, V = kv.logical(self.wl.n_total)
        return [K, V, logits, hk, dv]


def test_two_streams_equal_sequential_runs():
    say("two mini-8B blends (paged r 15%, contiguous r 30%) on two streams at once, three rounds")
    cases = [_Case(1, 0.15, True), _Case(2, 0.30, False)]
    ref = []
    for c in cases:                       # one after the other on the current stream
        out = c.outputs()
        c.run(out)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in c.result(out)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [c.outputs() for c in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())    # the outputs' fills come first
    for _ in range(3):                    # both in flight, no synchronisation in between
        for c, out, s in zip(cases, outs, streams):
            c.run(out, stream=s)
    torch.cuda.synchronize()
    names = ["K", "V", "logits", "hkvd", "dev"]
    for i, (c, out) in enumerate(zip(cases, outs)):
        for name, a, b in zip(names, c.result(out), ref[i]):
            assert torch.equal(a, b), f"case {i}: {name} differs from the sequential run"
        say(f"  case {i}: every output bitwise equal to the sequential run")


def test_workspace_contents_do_not_matter():
    say("a mini-8B blend and two decode steps with the workspaces filled with 0x00, then 0xFF")
    c = _Case(3, 0.15, True)
    dws = api.Workspace(api.cb_decode_workspace_bytes(c.model.cfg))
    wl = c.wl
    res = []
    for fill in (0x00, 0xFF):
        c.ws.t.fill_(fill)
        dws.t.fill_(fill)
        kv = blended_cache(MINI8B, wl.n_total + 2, paged=True, seed=3, fill=0.0)
        logits = torch.empty(MINI8B.vocab, device="cuda")
        hk = torch.full((MINI8B.n_layers, wl.n_ctx), -1, dtype=torch.int32, device="cuda")
        dv = torch.full((MINI8B.n_layers, wl.n_ctx), -1.0, device="cuda")
        c.run((kv, logits, hk, dv))
        outs = [logits.clone(), hk.clone(), dv.clone()]
        for i, tok in enumerate((17, 4242)):
            api.cb_decode_step(c.model, kv, wl.n_total + i, ints([tok]), logits, dws)
            outs.append(logits.clone())
        torch.cuda.synchronize()
        K, V = kv.logical(wl.n_total + 2)
        res.append([K, V] + outs)
    names = ["K", "V", "logits", "hkvd", "dev", "decode logits 0", "decode logits 1"]
    for name, a, b in zip(names, res[0], res[1]):
        assert torch.equal(a, b), f"{name} depends on the workspace's prior contents"
    say("  every output bitwise the same with either fill")

