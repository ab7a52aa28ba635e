"""Pins of the fragment-matching oracle (oracle/match.py) against what the
Blend Index page and the mathematics fix, without re-using the oracle's own
hashing where the check is about hashing:

* closed forms of the polynomial hash on tiny windows, its linearity and the
  Thue-Morse collision every mod-2^64 polynomial hash with an odd base has at
  length 2048 (so the arithmetic really is mod 2^64, Horner order, odd base);
* rolling window fingerprints equal direct ones at every position;
* the page's stated behaviours: recall at any offset, near misses rejected,
  unknown offsets and wrong lengths not indexed, filter slot sharing loses
  nothing, a second content under a taken fingerprint is never matched, results
  ascending and one per chunk, the caller's leftmost-greedy resolution;
* an independent brute-force matcher (direct token comparison of every window
  with every stored chunk, no hashing, no filter) gives the same matches on the
  seeded request workload;
* the filter passes at most about 1/16 of non-indexed windows (growth 16).
"""
import numpy as np
import pytest

import cbinputs
import oracle
from oracle import match as om

B = 0x9E3779B97F4A7C15
M64 = 1 << 64


def test_fingerprint_closed_forms():
    assert oracle.POLY_BASE == B
    assert om.fingerprint([]) == 0
    assert om.fingerprint([7]) == 7
    assert om.fingerprint([0, 0, 0, 5]) == 5
    assert om.fingerprint([1, 2]) == 0x9E3779B97F4A7C17
    assert om.fingerprint([1, 0]) == 0x9E3779B97F4A7C15
    assert om.fingerprint([2, 0]) == 0x3C6EF372FE94F82A       # 2 * base wraps past 2^64


def test_fingerprint_is_linear_in_the_tokens():
    rng = np.random.default_rng(1)
    for n in (1, 3, 17, 256):
        x = rng.integers(0, 1 << 30, size=n)
        y = rng.integers(0, 1 << 30, size=n)
        assert om.fingerprint(x + y) == (om.fingerprint(x) + om.fingerprint(y)) % M64
        assert om.fingerprint(list(x) + [0]) == (om.fingerprint(x) * B) % M64


def _thue_morse(n):
    return np.array([bin(i).count("1") & 1 for i in range(n)], dtype=np.int64)


def test_thue_morse_collision_of_the_mod_2_64_hash():
    # sum over i of (-1)^tm(i) x^i = prod_j (1 - x^(2^j)); for odd x the j-th factor
    # is divisible by 2^(j+1), so 11 factors give 2^66: the hash of a Thue-Morse
    # word of length 2048 equals that of its complement mod 2^64
    tm = _thue_morse(2048)
    a, b = 5, 9
    w1 = np.where(tm == 0, a, b)
    w2 = np.where(tm == 0, b, a)
    assert om.fingerprint(w1) == om.fingerprint(w2)
    assert not np.array_equal(w1, w2)
    # the second content is never added and never matched (page 4.5)
    idx = om.BlendIndex(2048)
    assert idx.add(w1, 11, 0)
    assert not idx.add(w2, 12, 0)
    q2 = np.concatenate([np.arange(10), w2, np.arange(5)])
    assert om.match(idx, q2) == []
    q1 = np.concatenate([np.arange(10), w1, np.arange(5)])
    assert om.match(idx, q1) == [(11, 0, 10)]


def test_vectorised_fingerprints_equal_scalar():
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 1 << 31, size=(50, 37))
    assert om.fingerprints(rows) == [om.fingerprint(r) for r in rows]
    w = cbinputs.fragment_workload(2, n_docs=6, chunk_size=32, n_queries=1)
    a, b = om.BlendIndex(32), om.BlendIndex(32)
    for t, i, o in zip(w.stored_tokens, w.stored_ids, w.stored_offsets):
        a.add(t, int(i), int(o))
    b.add_all(w.stored_tokens, w.stored_ids, w.stored_offsets)
    assert a.contents == b.contents


def test_rolling_equals_direct_at_every_window():
    rng = np.random.default_rng(2)
    q = rng.integers(0, 128256, size=300)
    for C in (1, 2, 16, 64):
        direct = [om.fingerprint(q[s:s + C]) for s in range(len(q) - C + 1)]
        assert om.window_fingerprints(q, C) == direct
    assert om.window_fingerprints(q[:10], 16) == []


def test_recall_at_any_offset():
    rng = np.random.default_rng(3)
    C = 32
    idx = om.BlendIndex(C)
    chunks = [rng.integers(0, 128256, size=C) for _ in range(6)]
    for i, c in enumerate(chunks):
        assert idx.add(c, 100 + i, 1000 * i + 7)
    for trial in range(5):
        parts, want, pos = [], [], 0
        for i in rng.permutation(6):
            gap = int(rng.integers(0, 50))
            parts.append(rng.integers(0, 128256, size=gap))
            pos += gap
            parts.append(chunks[i])
            want.append((100 + int(i), 1000 * int(i) + 7, pos))
            pos += C
        got = om.match(idx, np.concatenate(parts))
        assert got == sorted(want, key=lambda t: t[2])


def test_near_miss_rejected():
    rng = np.random.default_rng(4)
    C = 64
    idx = om.BlendIndex(C)
    c = rng.integers(0, 1000, size=C)
    idx.add(c, 1, 0)
    for j in (0, 17, C - 1):
        near = c.copy()
        near[j] += 1
        assert om.match(idx, np.concatenate([[3, 4], near, [5]])) == []
    assert om.match(idx, np.concatenate([[3, 4], c, [5]])) == [(1, 0, 2)]


def test_not_indexed_unknown_offset_or_wrong_length():
    C = 8
    idx = om.BlendIndex(C)
    assert not idx.add(np.arange(C), 1, om.UNKNOWN_TOKEN_OFFSET)
    assert not idx.add(np.arange(C - 1), 2, 0)
    assert not idx.add(np.arange(C + 1), 3, 0)
    assert idx.contents == {}
    assert om.match(idx, np.arange(40)) == []
    assert idx.add(np.arange(C), 4, 0)                 # position 0 is a real position
    assert om.match(idx, np.arange(40)) == [(4, 0, 0)]


def test_filter_slot_sharing_keeps_recall():
    # 60 fingerprints in 16 slots: nearly every slot shared, all still found (page 4.4)
    rng = np.random.default_rng(5)
    C = 16
    idx = om.BlendIndex(C)
    chunks = [rng.integers(0, 128256, size=C) for _ in range(60)]
    for i, c in enumerate(chunks):
        idx.add(c, i, 3 * i)
    k, slots = idx.filter(4)
    assert sum(slots) <= 16
    got = om.match(idx, np.concatenate(chunks), slot_bits=4)
    assert got == [(i, 3 * i, C * i) for i in range(60)]


def test_equal_content_two_occupants():
    C = 16
    idx = om.BlendIndex(C)
    x = np.arange(100, 100 + C)
    assert idx.add(x, 7, 10)
    assert idx.add(x, 8, 500)                           # same content, another chunk (page 3.1)
    assert idx.add(x, 7, 10)                            # re-adding an occupant changes nothing
    assert len(idx.contents) == 1
    filler = np.array([1, 2, 3])
    assert om.match(idx, np.concatenate([filler, x])) == [(7, 10, 3)]
    two = np.concatenate([filler, x, filler, x])
    assert om.match(idx, two) == [(7, 10, 3), (8, 500, 3 + C + 3)]
    three = np.concatenate([x, x, x])
    assert om.match(idx, three) == [(7, 10, 0), (8, 500, C)]


def test_probe_stride():
    C = 8
    idx = om.BlendIndex(C)
    idx.add(np.arange(50, 58), 1, 0)
    idx.add(np.arange(60, 68), 2, 0)
    q = np.concatenate([np.zeros(4), np.arange(50, 58), np.zeros(3), np.arange(60, 68)]).astype(np.int64)
    assert om.match(idx, q, 1) == [(1, 0, 4), (2, 0, 15)]
    assert om.match(idx, q, 4) == [(1, 0, 4)]           # 15 is not a multiple of 4
    assert om.match(idx, q, 5) == [(2, 0, 15)]


def test_leftmost_greedy_resolution():
    m = [(4, 0, 300), (1, 0, 0), (2, 0, 100), (3, 0, 256)]
    assert om.resolve_leftmost_greedy(m, 256) == [(1, 0, 0), (3, 0, 256)]
    assert om.resolve_leftmost_greedy(m, 256, prefix_len=50) == [(2, 0, 100)]
    assert om.resolve_leftmost_greedy(m, 256, prefix_len=256) == [(3, 0, 256)]
    assert om.resolve_leftmost_greedy([], 256) == []


def _brute_force(w, q, stride=1):
    """Every window against every stored chunk by direct comparison, stored chunks
    in storage order, unknown offsets skipped (random data holds no fingerprint
    collision, so every other chunk is indexed); the first stored chunk with equal
    tokens that this query has not matched yet is taken."""
    C = w.chunk_size
    stored = [(int(i), int(o), w.stored_tokens[n]) for n, (i, o) in enumerate(zip(w.stored_ids, w.stored_offsets))
              if o != -1]
    seen, out = set(), []
    for s in range(0, len(q) - C + 1, stride):
        win = q[s:s + C]
        for cid, off, t in stored:
            if cid not in seen and np.array_equal(t, win):
                seen.add(cid)
                out.append((cid, off, s))
                break
    return out


@pytest.mark.parametrize("stride", [1, 7])
def test_matches_brute_force_on_request_workload(stride):
    w = cbinputs.fragment_workload(11, n_docs=12, chunk_size=64, n_queries=3, docs_per_query=3)
    idx = om.BlendIndex(w.chunk_size)
    for t, i, o in zip(w.stored_tokens, w.stored_ids, w.stored_offsets):
        idx.add(t, int(i), int(o))
    for q in w.queries:
        got = om.match(idx, q, stride)
        assert got == _brute_force(w, q, stride)
        assert [m[2] for m in got] == sorted(m[2] for m in got)
        assert len({m[0] for m in got}) == len(got)
        if stride == 1:
            assert len(got) >= 4                        # whole documents of 4 chunks were planted


def test_filter_false_positive_rate_at_growth_16():
    rng = np.random.default_rng(6)
    C = 4
    idx = om.BlendIndex(C)
    for i in range(1000):
        idx.add(rng.integers(0, 1 << 31, size=C), i, i)
    k, slots = idx.filter()
    assert (1 << k) >= 16 * 1000 and (1 << (k - 1)) < 16 * 1000
    fps = om.window_fingerprints(rng.integers(0, 1 << 31, size=100000), C)
    rate = np.mean([slots[h >> (64 - k)] for h in fps])
    assert rate <= 1 / 16 + 4 * np.sqrt((1 / 16) / len(fps))
