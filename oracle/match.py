"""Plain oracle of blend-style fragment matching (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may use this module; the GPU library never calls it.

Source: [BI] the LMCache coordinator "Blend Index" article (nxmr.cn):
  section 3.1  an indexed chunk is keyed by the 64-bit polynomial hash of its
               chunk_size tokens with base POLY_BASE = 0x9E3779B97F4A7C15; equal
               content stored under two chunk ids is one content entry with two
               occupants, each with its own stored offset;
  section 4.1  two layers: the authoritative contents map (fingerprint -> tokens,
               occupants in first-indexed order) and a uint8 occupancy filter of
               2^k slots, a slot set when any fingerprint lands in it;
  section 4.2  matching: roll a chunk_size window over the query, test the filter
               every probe_stride positions, resolve the few survivors exactly in
               the contents map, choose the occupant, and only then compare the
               window with the stored tokens token by token; a chunk is marked
               seen only after that check passes;
  section 4.4  the filter stores no identity, so fingerprints sharing a slot are
               all still found (recall stays complete); with the growth factor
               _TABLE_GROWTH = 16 (16 slots per indexed fingerprint) the filter
               passes about 6% of non-indexed windows or fewer;
  section 4.5  a fingerprint collision means the second content is never added
               (so never matched wrongly); a window one token away is rejected;
  section 5    a chunk with an unknown stored offset (UNKNOWN_TOKEN_OFFSET = -1)
               or whose length is not chunk_size is not indexed;
  section 6.2  the result: (chunk, old_st, cur_st) tuples, old_st the re-RoPE
               source and cur_st the target, in ascending cur_st, at most one
               per chunk; they may overlap in the query, and the caller resolves
               overlaps leftmost-greedy;
  section 7    the caller first drops matches covered by the prefix, then orders
               by cur_st, and on an overlap the earlier match wins;
  section 9    configuration defaults: chunk_size 256, probe_stride 1.

Readings where the page is silent (also listed in the design notes):
  * the hash is Horner's rule over the window, h = h * POLY_BASE + token mod 2^64,
    from h = 0, token ids taken as unsigned values;
  * the filter slot of a fingerprint is its top k bits (fingerprint >> (64 - k)),
    the usual use of this multiplier; k is the smallest value >= 4 with
    2^k >= 16 * (number of fingerprints);
  * "choose the occupant" takes the first occupant, in first-indexed order, that
    this query has not matched yet, so content that occurs twice in the query
    can match two chunks that stored it;
  * "covered by the prefix" is a match that starts before the prefix length.

Parity: pinned by tests/test_oracle_match.py (closed forms and a Thue-Morse
collision of the mod-2^64 polynomial hash, brute force over every window, the
page's stated behaviours, and the filter's false-positive bound).
"""
from __future__ import annotations

POLY_BASE = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1
UNKNOWN_TOKEN_OFFSET = -1
TABLE_GROWTH = 16
DEFAULT_CHUNK_SIZE = 256
DEFAULT_PROBE_STRIDE = 1


def fingerprint(tokens) -> int:
    """64-bit polynomial hash of one window (section 3.1), Horner's rule."""
    h = 0
    for t in tokens:
        h = (h * POLY_BASE + int(t)) & MASK64
    return h


def fingerprints(rows) -> list[int]:
    """fingerprint() of every row of a [n][chunk_size] array, Horner's rule run on
    all rows at once in uint64 arithmetic (which wraps mod 2^64)."""
    import numpy as np
    a = np.asarray(rows, dtype=np.uint64)
    h = np.zeros(a.shape[0], dtype=np.uint64)
    base = np.uint64(POLY_BASE)
    with np.errstate(over="ignore"):
        for j in range(a.shape[1]):
            h = h * base + a[:, j]
    return [int(x) for x in h]


def window_fingerprints(query, chunk_size: int) -> list[int]:
    """Fingerprint of every window query[s:s+chunk_size], s = 0 .. n - chunk_size,
    rolled (section 4.2): drop the oldest token's term, shift, add the new one."""
    n = len(query)
    if n < chunk_size or chunk_size <= 0:
        return []
    top = pow(POLY_BASE, chunk_size - 1, 1 << 64)
    h = fingerprint(query[:chunk_size])
    out = [h]
    for s in range(1, n - chunk_size + 1):
        h = ((h - int(query[s - 1]) * top) * POLY_BASE + int(query[s + chunk_size - 1])) & MASK64
        out.append(h)
    return out


def slot_bits_for(n_fingerprints: int) -> int:
    """Filter size: 2^k slots, at least TABLE_GROWTH per indexed fingerprint."""
    k = 4
    while (1 << k) < TABLE_GROWTH * max(n_fingerprints, 1):
        k += 1
    return k


class BlendIndex:
    """The two layers of section 4.1 for one namespace (the fleet's namespaces,
    claims and removal paths are not modelled)."""

    def __init__(self, chunk_size: int = DEFAULT_CHUNK_SIZE):
        self.chunk_size = int(chunk_size)
        self.contents: dict[int, dict] = {}   # fingerprint -> {"tokens": tuple, "occupants": [(chunk, offset)]}

    def add(self, tokens, chunk_id: int, token_offset: int) -> bool:
        """Index one stored chunk; False when it is not indexed (sections 4.5, 5)."""
        if int(token_offset) == UNKNOWN_TOKEN_OFFSET or len(tokens) != self.chunk_size:
            return False
        return self._add(tokens, chunk_id, token_offset, fingerprint(tokens))

    def add_all(self, tokens, chunk_ids, token_offsets) -> int:
        """add() of every row in order, fingerprints computed together; returns the
        number indexed."""
        fps = fingerprints(tokens) if len(tokens) else []
        n = 0
        for t, fp, cid, off in zip(tokens, fps, chunk_ids, token_offsets):
            n += self._add(t, int(cid), int(off), fp)
        return n

    def _add(self, tokens, chunk_id: int, token_offset: int, fp: int) -> bool:
        if int(token_offset) == UNKNOWN_TOKEN_OFFSET or len(tokens) != self.chunk_size:
            return False
        toks = tuple(int(t) for t in tokens)
        entry = self.contents.get(fp)
        if entry is None:
            self.contents[fp] = {"tokens": toks, "occupants": [(int(chunk_id), int(token_offset))]}
            return True
        if entry["tokens"] != toks:
            return False                      # a different content under a taken fingerprint
        if all(c != int(chunk_id) for c, _ in entry["occupants"]):
            entry["occupants"].append((int(chunk_id), int(token_offset)))
        return True

    def filter(self, slot_bits: int | None = None) -> tuple[int, bytearray]:
        k = slot_bits_for(len(self.contents)) if slot_bits is None else int(slot_bits)
        slots = bytearray(1 << k)
        for fp in self.contents:
            slots[fp >> (64 - k)] = 1
        return k, slots


def match(index: BlendIndex, query, probe_stride: int = DEFAULT_PROBE_STRIDE,
          slot_bits: int | None = None) -> list[tuple[int, int, int]]:
    """Section 4.2: filter, resolve, choose the occupant, verify; (chunk, old_st,
    cur_st) in ascending cur_st, each chunk at most once (section 6.2)."""
    C = index.chunk_size
    k, slots = index.filter(slot_bits)
    fps = window_fingerprints(query, C)
    seen: set[int] = set()
    out = []
    for s in range(0, len(fps), max(int(probe_stride), 1)):
        h = fps[s]
        if not slots[h >> (64 - k)]:
            continue
        entry = index.contents.get(h)
        if entry is None:
            continue
        occ = next(((c, off) for c, off in entry["occupants"] if c not in seen), None)
        if occ is None:
            continue
        if tuple(int(t) for t in query[s:s + C]) != entry["tokens"]:
            continue
        seen.add(occ[0])
        out.append((occ[0], occ[1], s))
    return out


def resolve_leftmost_greedy(matches, chunk_size: int, prefix_len: int = 0) -> list[tuple[int, int, int]]:
    """Section 7: drop matches starting inside the prefix, order by cur_st, keep a
    match only if it starts at or after the end of the last kept one."""
    kept = []
    end = int(prefix_len)
    for m in sorted(matches, key=lambda t: t[2]):
        if m[2] >= end:
            kept.append(m)
            end = m[2] + int(chunk_size)
    return kept
