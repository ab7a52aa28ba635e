"""Host side of fragment matching (no GPU): the library's index builder against
the oracle's index on the seeded request workload, and the validation of
cb_blend_match (every case here fails validation, so nothing is launched)."""
import ctypes

import numpy as np
import pytest

import cbinputs
from oracle import match as om
from cacheblend_selective_recompute_amd import _abi, api


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def _oracle_index(w):
    idx = om.BlendIndex(w.chunk_size)
    for t, i, o in zip(w.stored_tokens, w.stored_ids, w.stored_offsets):
        idx.add(t, int(i), int(o))
    return idx


def _sections(info, image):
    L = {}
    off = 64

    def take(n):
        nonlocal off
        off = (off + 255) // 256 * 256
        at = off
        off += n
        return at
    L["slots"] = take(1 << info.slot_bits)
    L["tfp"] = take((1 << info.table_bits) * 8)
    L["tent"] = take((1 << info.table_bits) * 4)
    L["etok"] = take(info.n_entries * info.chunk_size * 4)
    L["eocc"] = take((info.n_entries + 1) * 4)
    L["ochunk"] = take(info.n_occupants * 8)
    L["ooff"] = take(info.n_occupants * 4)
    assert (off + 255) // 256 * 256 == info.image_bytes == image.size
    return {
        "slots": image[L["slots"]:L["slots"] + (1 << info.slot_bits)],
        "tfp": image[L["tfp"]:].view(np.uint64)[:1 << info.table_bits] if L["tfp"] % 8 == 0 else None,
        "tent": image[L["tent"]:L["tent"] + (1 << info.table_bits) * 4].view(np.int32),
        "etok": image[L["etok"]:L["etok"] + info.n_entries * info.chunk_size * 4].view(np.int32)
        .reshape(info.n_entries, info.chunk_size),
        "eocc": image[L["eocc"]:L["eocc"] + (info.n_entries + 1) * 4].view(np.int32),
        "ochunk": image[L["ochunk"]:L["ochunk"] + info.n_occupants * 8].view(np.int64),
        "ooff": image[L["ooff"]:L["ooff"] + info.n_occupants * 4].view(np.int32),
    }


@pytest.mark.parametrize("C", [64, 256])
def test_index_image_matches_oracle_index(C):
    w = cbinputs.fragment_workload(3, n_docs=20, chunk_size=C, n_queries=1)
    info, image = api.cb_blend_index_build(w.stored_tokens, w.stored_ids, w.stored_offsets)
    idx = _oracle_index(w)
    k, slots = idx.filter()
    assert info.chunk_size == C
    assert info.n_entries == len(idx.contents)
    assert info.n_occupants == sum(len(e["occupants"]) for e in idx.contents.values())
    assert info.n_skipped == int(np.sum(w.stored_offsets == -1))
    assert info.slot_bits == k
    sec = _sections(info, image)
    assert bytes(sec["slots"]) == bytes(slots)                     # the library's hashing = the oracle's
    # every content: its fingerprint in the table, its tokens and occupants in first-indexed order
    fps = list(idx.contents)
    tfp = sec["tfp"]
    for e, fp in enumerate(fps):
        at = np.nonzero((tfp == np.uint64(fp)) & (sec["tent"] >= 0))[0]
        assert len(at) == 1 and sec["tent"][at[0]] == e
        assert tuple(sec["etok"][e]) == idx.contents[fp]["tokens"]
        occ = [(int(sec["ochunk"][o]), int(sec["ooff"][o])) for o in range(sec["eocc"][e], sec["eocc"][e + 1])]
        assert occ == idx.contents[fp]["occupants"]


def test_index_build_rejects_taken_fingerprint_and_empty():
    tm = np.array([bin(i).count("1") & 1 for i in range(2048)], dtype=np.int32)
    w1, w2 = np.where(tm == 0, 5, 9), np.where(tm == 0, 9, 5)
    info, image = api.cb_blend_index_build(np.stack([w1, w2]), np.array([11, 12]), np.array([0, 0]))
    assert (info.n_entries, info.n_occupants, info.n_skipped) == (1, 1, 1)
    info, image = api.cb_blend_index_build(np.zeros((0, 256), dtype=np.int32), np.zeros(0), np.zeros(0))
    assert (info.n_entries, info.slot_bits, info.table_bits) == (0, 4, 4)


def test_index_build_validation(lib):
    info = _abi.cb_blend_index_info()
    buf = np.zeros(1 << 16, dtype=np.uint8)
    t = np.zeros((2, 16), dtype=np.int32)
    ids = np.array([1, 2], dtype=np.int64)
    off = np.array([0, 16], dtype=np.int32)
    B = lambda tt, oo, n, C, nb: lib.cb_blend_index_build(tt.ctypes.data, ids.ctypes.data, oo.ctypes.data, n, C,
                                                          buf.ctypes.data, nb, ctypes.byref(info))
    assert B(t, off, 2, 16, buf.size) == _abi.CB_OK
    assert B(t, off, -1, 16, buf.size) == _abi.CB_ERR_INVALID
    assert B(t, off, 2, 0, buf.size) == _abi.CB_ERR_INVALID
    assert B(t, np.array([0, -2], dtype=np.int32), 2, 16, buf.size) == _abi.CB_ERR_INVALID
    assert B(np.full((2, 16), -3, dtype=np.int32), off, 2, 16, buf.size) == _abi.CB_ERR_INVALID
    assert B(t, off, 2, 16, 64) == _abi.CB_ERR_WORKSPACE
    assert lib.cb_blend_index_image_bytes(-1, 16) == 0 and lib.cb_blend_index_image_bytes(4, 0) == 0


def test_match_validation(lib):
    info, image = api.cb_blend_index_build(np.arange(64, dtype=np.int32).reshape(2, 32), np.array([1, 2]),
                                           np.array([0, 32]))
    FAKE = 1 << 20
    M = lambda inf, **kw: lib.cb_blend_match(
        kw.get("img", FAKE), ctypes.byref(inf) if inf is not None else None, FAKE, FAKE, kw.get("nq", 2),
        kw.get("total", 1000), kw.get("maxlen", 600), kw.get("stride", 1), None, kw.get("mm", 8),
        kw.get("oc", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("wsb", 0), None)
    assert M(None) == _abi.CB_ERR_INVALID
    assert M(info, img=None) == _abi.CB_ERR_INVALID
    assert M(info, nq=-1) == _abi.CB_ERR_INVALID
    assert M(info, stride=0) == _abi.CB_ERR_INVALID
    assert M(info, mm=-1) == _abi.CB_ERR_INVALID
    assert M(info, oc=None) == _abi.CB_ERR_INVALID
    assert M(info, img=FAKE + 16) == _abi.CB_ERR_INVALID           # alignment
    bad = _abi.cb_blend_index_info.from_buffer_copy(info)
    bad.slot_bits += 1
    assert M(bad) == _abi.CB_ERR_INVALID
    bad = _abi.cb_blend_index_info.from_buffer_copy(info)
    bad.image_bytes += 256
    assert M(bad) == _abi.CB_ERR_INVALID
    assert M(info, wsb=16) == _abi.CB_ERR_WORKSPACE                 # 1000 tokens need 4000 bytes
    assert lib.cb_blend_match_workspace_bytes(1000) >= 4000
