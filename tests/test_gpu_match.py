"""GPU parity of fragment matching (cb_blend_match through the C ABI) with the
oracle: every match tuple and every leftmost-greedy decision is integer work,
so the comparison is exact.  Cases: the seeded request workload at two probe
strides with prefix coverage; the full-size batch the benchmark times (64
requests of the 4 x 1024 + 64 shape over an index of 65536 chunks) on a sample
of requests plus size-independent properties on all; edge cases (empty index,
empty and short requests, a tiny chunk size, output truncation, a fingerprint
taken by other content, more distinct contents than one request may match)."""
import numpy as np
import pytest
import torch

import cbinputs
from oracle import match as om
from cacheblend_selective_recompute_amd import _abi, api

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _batch(queries):
    lens = [len(q) for q in queries]
    starts = np.zeros(len(queries) + 1, dtype=np.int32)
    starts[1:] = np.cumsum(lens)
    toks = np.concatenate(queries).astype(np.int32) if sum(lens) else np.zeros(1, dtype=np.int32)
    return (torch.from_numpy(toks).cuda(), torch.from_numpy(starts).cuda(), int(starts[-1]), max(lens + [0]))


def _run(index, queries, stride=1, prefix=None, max_matches=64):
    tq, ts, total, mx = _batch(queries)
    pl = None if prefix is None else torch.from_numpy(np.asarray(prefix, dtype=np.int32)).cuda()
    out = api.cb_blend_match(index, tq, ts, total, mx, stride, pl, max_matches)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _gpu_matches(out, q):
    n = int(out["count"][q])
    m = min(n, out["chunk"].shape[1])
    return ([(int(out["chunk"][q, i]), int(out["old_st"][q, i]), int(out["cur_st"][q, i])) for i in range(m)],
            [bool(out["kept"][q, i]) for i in range(m)], n)


def _oracle_index(tokens, ids, offs, C):
    idx = om.BlendIndex(C)
    idx.add_all(tokens, ids, offs)
    return idx


def _check(idx, out, queries, stride, prefix, C, sample=None):
    for q in (range(len(queries)) if sample is None else sample):
        want = om.match(idx, queries[q], stride)
        kept = set(om.resolve_leftmost_greedy(want, C, 0 if prefix is None else int(prefix[q])))
        got, got_kept, n = _gpu_matches(out, q)
        assert n == len(want), (q, n, len(want))
        assert got == want[:len(got)], q
        assert got_kept == [m in kept for m in want[:len(got)]], q


@pytest.mark.parametrize("stride", [1, 7])
def test_match_request_workload(stride):
    w = cbinputs.fragment_workload(21, n_docs=40, chunk_size=256, n_queries=6)
    say(f"cb_blend_match: {len(w.stored_ids)} stored chunks, {len(w.queries)} requests, stride {stride}")
    index = api.BlendIndexImage(w.stored_tokens, w.stored_ids, w.stored_offsets)
    idx = _oracle_index(w.stored_tokens, w.stored_ids, w.stored_offsets, 256)
    out = _run(index, w.queries, stride, w.prefix_lens)
    _check(idx, out, w.queries, stride, w.prefix_lens, 256)
    if stride == 1:
        assert all(out["count"] >= 4)


def test_match_full_size_batch():
    C, n_docs, n_q = 256, 16384, 64
    w = cbinputs.fragment_workload(5, n_docs=n_docs, chunk_size=C, n_queries=n_q, docs_per_query=4, dup_docs=64,
                                   unknown_chunks=64)
    say(f"cb_blend_match: {len(w.stored_ids)} stored chunks, {n_q} requests of ~{np.mean([len(q) for q in w.queries]):.0f} tokens")
    index = api.BlendIndexImage(w.stored_tokens, w.stored_ids, w.stored_offsets)
    out = _run(index, w.queries, 1, w.prefix_lens, max_matches=64)
    idx = _oracle_index(w.stored_tokens, w.stored_ids, w.stored_offsets, C)
    _check(idx, out, w.queries, 1, w.prefix_lens, C, sample=[0, 13, 31, 47, 63])
    # every request: ascending starts, distinct chunks, each match's tokens equal the stored chunk's
    by_id = {int(i): (int(o), w.stored_tokens[n]) for n, (i, o) in enumerate(zip(w.stored_ids, w.stored_offsets))}
    for q in range(n_q):
        got, kept, n = _gpu_matches(out, q)
        assert n == len(got) and n >= 8
        assert [m[2] for m in got] == sorted(m[2] for m in got)
        assert len({m[0] for m in got}) == n
        for cid, old, cur in got:
            assert by_id[cid][0] == old
            assert np.array_equal(w.queries[q][cur:cur + C], by_id[cid][1])


def test_match_edge_cases():
    rng = np.random.default_rng(8)
    C = 32
    toks = rng.integers(0, 1000, size=(5, C)).astype(np.int32)
    ids, offs = np.arange(10, 15), np.arange(5) * C
    index = api.BlendIndexImage(toks, ids, offs)
    idx = _oracle_index(toks, ids, offs, C)
    queries = [np.zeros(0, dtype=np.int32), toks[0][:C - 1], toks[1].copy(),
               np.concatenate([toks[2], toks[2], toks[3]]), rng.integers(0, 1000, size=5000).astype(np.int32)]
    say("cb_blend_match: empty, short, exact, repeated and random requests")
    out = _run(index, queries, 1, [0, 0, 0, 10, 0])
    _check(idx, out, queries, 1, [0, 0, 0, 10, 0], C)
    assert list(out["count"][:3]) == [0, 0, 1]
    # truncation: more matches than the capacity
    many = np.concatenate([toks[i] for i in range(5)])
    out = _run(index, [many], 1, None, max_matches=3)
    got, kept, n = _gpu_matches(out, 0)
    assert n == 5 and got == om.match(idx, many)[:3]
    # empty index
    empty = api.BlendIndexImage(np.zeros((0, C), dtype=np.int32), np.zeros(0), np.zeros(0))
    out = _run(empty, [many], 1)
    assert out["count"][0] == 0


def test_match_taken_fingerprint_and_tiny_chunks():
    tm = np.array([bin(i).count("1") & 1 for i in range(2048)], dtype=np.int32)
    w1, w2 = np.where(tm == 0, 5, 9).astype(np.int32), np.where(tm == 0, 9, 5).astype(np.int32)
    index = api.BlendIndexImage(np.stack([w1, w2]), np.array([11, 12]), np.array([0, 0]))
    say("cb_blend_match: a fingerprint taken by other content (2048-token chunks)")
    out = _run(index, [np.concatenate([np.arange(3, dtype=np.int32), w2]),
                       np.concatenate([np.arange(3, dtype=np.int32), w1])])
    assert out["count"][0] == 0 and out["count"][1] == 1
    assert (out["chunk"][1, 0], out["old_st"][1, 0], out["cur_st"][1, 0]) == (11, 0, 3)
    # chunk_size 1: every indexed token is a content
    toks = np.arange(300, dtype=np.int32).reshape(300, 1)
    index = api.BlendIndexImage(toks, np.arange(300) + 1000, np.arange(300))
    idx = _oracle_index(toks, np.arange(300) + 1000, np.arange(300), 1)
    q = [np.random.default_rng(9).integers(0, 600, size=700).astype(np.int32)]
    out = _run(index, q, 1, None, max_matches=400)
    _check(idx, out, q, 1, None, 1)


def test_match_too_many_contents():
    n = _abi.CB_MATCH_MAX_CONTENTS + 10
    toks = np.arange(n, dtype=np.int32).reshape(n, 1)
    index = api.BlendIndexImage(toks, np.arange(n), np.arange(n))
    say(f"cb_blend_match: one request matching {n} distinct contents")
    out = _run(index, [np.arange(n, dtype=np.int32), np.arange(100, dtype=np.int32)], 1, None, max_matches=8)
    assert out["count"][0] == -1
    assert out["count"][1] == 100
