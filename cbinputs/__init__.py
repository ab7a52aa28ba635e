"""Seeded synthetic inputs for the blended prefill (model shapes, weights, chunk
workloads, cached KV, block tables).

This module produces inputs only.  It holds none of the method's arithmetic:
no RoPE, no attention, no deviation, no selection.  Both the CPU oracle and the
GPU path draw their inputs from here, so both see exactly the same numbers.

Conventions
-----------
* Linear weights are stored ``[out_features][in_features]`` (row-major), so a
  projection of row vectors ``a`` is ``a @ W.T``.  ``w_qkv`` stacks Q, K, V
  rows; ``w_gate_up`` stacks gate rows then up rows.
* bf16 models draw every weight in fp32 and round it to bf16 (round to nearest
  even); the values are returned as fp32 arrays holding bf16-representable
  numbers, so a consumer may upcast them without loss.
* Every tensor has its own ``SeedSequence`` stream keyed by (config seed,
  layer, tensor id), so any single layer can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "ModelShape", "Workload", "SHAPES", "WORKLOADS", "make_workload",
    "layer_weights", "global_weights", "model_weights", "synthetic_chunk_kv",
    "to_bf16_values", "bf16_bits", "recompute_count", "paged_layout",
]


# ----------------------------------------------------------------------------
# numeric storage helpers (input quantisation only)
# ----------------------------------------------------------------------------

def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# model shapes
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    rope_theta: float
    rms_eps: float = 1e-5
    dtype: str = "bf16"          # storage / compute dtype of the model: "f32" | "bf16"
    init_std: float = 0.02

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    def with_layers(self, n_layers: int) -> "ModelShape":
        return dataclasses.replace(self, n_layers=n_layers)

    def with_dtype(self, dtype: str) -> "ModelShape":
        return dataclasses.replace(self, dtype=dtype)

    def params_per_layer(self) -> int:
        d = self.d_model
        return (d * (self.q_width + 2 * self.kv_width) + self.q_width * d
                + d * 2 * self.d_ff + self.d_ff * d)

    def kv_bytes_per_token(self) -> int:
        """K and V bytes per token over all layers in the storage dtype."""
        elt = 2 if self.dtype == "bf16" else 4
        return self.n_layers * 2 * self.n_kv_heads * self.head_dim * elt


SHAPES: Dict[str, ModelShape] = {
    # tiny fp32 decoder: 2 layers, d 256, 4 x 64 MHA, MLP 1024, vocab 32000
    "tiny-2l-d256": ModelShape("tiny-2l-d256", 2, 256, 4, 4, 64, 1024, 32000,
                               10000.0, dtype="f32"),
    # Llama-3-8B-shaped decoder
    "llama3-8b": ModelShape("llama3-8b", 32, 4096, 32, 8, 128, 14336, 128256,
                            500000.0, dtype="bf16"),
    # Llama-70B-shaped decoder
    "llama-70b": ModelShape("llama-70b", 80, 8192, 64, 8, 128, 28672, 128256,
                            500000.0, dtype="bf16"),
}


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def recompute_count(ratio: float, n_ctx: int) -> int:
    """Number of context tokens recomputed per layer: floor(r * N + 0.5)."""
    return int(np.floor(ratio * n_ctx + 0.5))


@dataclass
class Workload:
    name: str
    shape: ModelShape
    chunk_tokens: List[np.ndarray]      # int32 [len_c] per chunk (storage order)
    old_starts: List[int]               # offset each chunk was prefilled at
    new_starts: List[int]               # offset each chunk is placed at
    query_tokens: np.ndarray            # int32 [Q]
    ratio: float
    seed: int
    paged: bool = False
    block_size: int = 16

    @property
    def chunk_lens(self) -> List[int]:
        return [int(len(t)) for t in self.chunk_tokens]

    @property
    def n_ctx(self) -> int:
        return int(sum(self.chunk_lens))

    @property
    def n_query(self) -> int:
        return int(len(self.query_tokens))

    @property
    def n_total(self) -> int:
        return self.n_ctx + self.n_query

    @property
    def k(self) -> int:
        return recompute_count(self.ratio, self.n_ctx)

    def schedule(self) -> Tuple[List[int], List[int]]:
        """Constant schedule: layer 0 full; every later layer checks and keeps k."""
        L = self.shape.n_layers
        ks = [self.n_ctx] + [self.k] * (L - 1)
        check = [0] + [1] * (L - 1)
        return ks, check

    def placement_order(self) -> List[int]:
        """Chunk indices sorted by new_start."""
        return sorted(range(len(self.chunk_tokens)), key=lambda c: self.new_starts[c])

    def context_tokens(self) -> np.ndarray:
        """Context tokens in placement (new position) order."""
        return np.concatenate([self.chunk_tokens[c] for c in self.placement_order()]).astype(np.int32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key)))


def _tile_offsets(lens: Sequence[int], order: Sequence[int]) -> List[int]:
    starts = [0] * len(lens)
    cur = 0
    for c in order:
        starts[c] = cur
        cur += lens[c]
    return starts


WORKLOADS = {
    # name -> (shape, description)
    "tiny-2x256-q32": "tiny fp32 decoder; 2 chunks x 256 prefilled at 0, placed at 0 and 256; 32-token query",
    "8b-4x1024-q64": "8B shape bf16; 4 chunks x 1024 prefilled at 0, shuffled placement; 64-token query",
    "8b-16x512j-q64": "8B shape bf16; 16 chunks of 512 +-25%, cached at random offsets in [0,4096), shuffled; 64-token query",
    "70b-4x1024-q64": "70B shape bf16; 4 chunks x 1024, shuffled placement; 64-token query",
    "8b-32x1024-q128-paged": "8B shape bf16; 32 chunks x 1024, shuffled; 128-token query; paged KV, 16-token blocks",
}


def make_workload(name: str, seed: int = 0, ratio: float = 0.15, *,
                  n_layers: Optional[int] = None, n_chunks: Optional[int] = None,
                  chunk_len: Optional[int] = None, n_query: Optional[int] = None,
                  shape: Optional[ModelShape] = None, paged: Optional[bool] = None) -> Workload:
    """Build one of the named workloads; keyword overrides give reduced variants.

    Chunk tokens are uniform over the vocabulary.  Placement order is a seeded
    permutation except for the tiny workload, whose placement is fixed (chunk 0
    at 0, chunk 1 at 256).
    """
    rng = _rng(seed, 7, 0)
    if name == "tiny-2x256-q32":
        shp = SHAPES["tiny-2l-d256"]
        C, ln, Q = 2, 256, 32
        lens = [ln] * (n_chunks or C) if chunk_len is None else [chunk_len] * (n_chunks or C)
        old = [0] * len(lens)
        order = list(range(len(lens)))
        is_paged = False
    elif name in ("8b-4x1024-q64", "70b-4x1024-q64"):
        shp = SHAPES["llama3-8b" if name.startswith("8b") else "llama-70b"]
        C, Q = 4, 64
        lens = [chunk_len or 1024] * (n_chunks or C)
        old = [0] * len(lens)
        order = [int(i) for i in rng.permutation(len(lens))]
        is_paged = False
    elif name == "8b-16x512j-q64":
        shp = SHAPES["llama3-8b"]
        C, Q = 16, 64
        base = chunk_len or 512
        nc = n_chunks or C
        jit = base // 4
        lens = [int(base + rng.integers(-jit, jit + 1)) for _ in range(nc)]
        old = [int(rng.integers(0, 4096)) for _ in range(nc)]
        order = [int(i) for i in rng.permutation(nc)]
        is_paged = False
    elif name == "8b-32x1024-q128-paged":
        shp = SHAPES["llama3-8b"]
        C, Q = 32, 128
        lens = [chunk_len or 1024] * (n_chunks or C)
        old = [0] * len(lens)
        order = [int(i) for i in rng.permutation(len(lens))]
        is_paged = True
    else:
        raise KeyError(f"unknown workload {name!r}")
    if shape is not None:
        shp = shape
    if n_layers is not None:
        shp = shp.with_layers(n_layers)
    if n_query is not None:
        Q = n_query
    if paged is not None:
        is_paged = paged
    trng = _rng(seed, 7, 1)
    toks = [trng.integers(0, shp.vocab, size=l, dtype=np.int64).astype(np.int32) for l in lens]
    qtok = trng.integers(0, shp.vocab, size=Q, dtype=np.int64).astype(np.int32)
    new = _tile_offsets(lens, order)
    return Workload(name=name, shape=shp, chunk_tokens=toks, old_starts=old, new_starts=new,
                    query_tokens=qtok, ratio=ratio, seed=seed, paged=is_paged)


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

_TID = {"wq": 0, "wk": 1, "wv": 2, "wo": 3, "w_gate": 4, "w_up": 5, "w_down": 6}


def _normal(shape: ModelShape, seed: int, layer_key: int, tid: int, dims) -> np.ndarray:
    g = _rng(seed, 1, layer_key, tid)
    w = g.standard_normal(size=dims, dtype=np.float32)
    w *= np.float32(shape.init_std)
    if shape.dtype == "bf16":
        w = to_bf16_values(w)
    return w


def layer_weights(shape: ModelShape, seed: int, layer: int) -> Dict[str, np.ndarray]:
    """Weights of one decoder layer; all matrices iid N(0, init_std^2), norm gains 1."""
    d, F = shape.d_model, shape.d_ff
    w = {
        "wq": _normal(shape, seed, layer + 1, _TID["wq"], (shape.q_width, d)),
        "wk": _normal(shape, seed, layer + 1, _TID["wk"], (shape.kv_width, d)),
        "wv": _normal(shape, seed, layer + 1, _TID["wv"], (shape.kv_width, d)),
        "wo": _normal(shape, seed, layer + 1, _TID["wo"], (d, shape.q_width)),
        "w_gate": _normal(shape, seed, layer + 1, _TID["w_gate"], (F, d)),
        "w_up": _normal(shape, seed, layer + 1, _TID["w_up"], (F, d)),
        "w_down": _normal(shape, seed, layer + 1, _TID["w_down"], (d, F)),
        "attn_norm": np.ones(d, dtype=np.float32),
        "mlp_norm": np.ones(d, dtype=np.float32),
    }
    return w


def global_weights(shape: ModelShape, seed: int) -> Dict[str, np.ndarray]:
    d, V = shape.d_model, shape.vocab
    return {
        "embed": _normal(shape, seed, 0, 0, (V, d)),
        "lm_head": _normal(shape, seed, 0, 1, (V, d)),
        "final_norm": np.ones(d, dtype=np.float32),
    }


def model_weights(shape: ModelShape, seed: int) -> Dict[str, object]:
    """All weights: {'layers': [per-layer dict], 'embed', 'lm_head', 'final_norm'}."""
    out: Dict[str, object] = dict(global_weights(shape, seed))
    out["layers"] = [layer_weights(shape, seed, l) for l in range(shape.n_layers)]
    return out


# ----------------------------------------------------------------------------
# cached KV and paging
# ----------------------------------------------------------------------------

def synthetic_chunk_kv(shape: ModelShape, lens: Sequence[int], seed: int,
                       scale: Optional[float] = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Stand-in cached K/V per chunk, ``[L][len][H_kv][d_h]`` each, iid normal.

    Used where a chunk prefill of the full model is too costly on the host.  The
    default scale matches a projection of a unit-RMS row by N(0, init_std^2)
    weights (std = init_std * sqrt(d_model)).
    """
    s = scale if scale is not None else shape.init_std * np.sqrt(shape.d_model)
    out = []
    for c, l in enumerate(lens):
        dims = (shape.n_layers, l, shape.n_kv_heads, shape.head_dim)
        g = _rng(seed, 3, c)
        k = g.standard_normal(size=dims, dtype=np.float32) * np.float32(s)
        v = g.standard_normal(size=dims, dtype=np.float32) * np.float32(s)
        if shape.dtype == "bf16":
            k, v = to_bf16_values(k), to_bf16_values(v)
        out.append((k, v))
    return out


def paged_layout(n_tokens: int, block_size: int, seed: int, key: int,
                 spare_blocks: int = 0) -> Tuple[np.ndarray, int]:
    """Random block table for ``n_tokens`` tokens.

    Returns (block_table int32 [ceil(n/bs)], n_physical).  Logical block b maps
    to a distinct physical block drawn from a pool of ``n_logical +
    spare_blocks`` blocks in random order.
    """
    n_log = (n_tokens + block_size - 1) // block_size
    n_phys = n_log + spare_blocks
    g = _rng(seed, 5, key)
    table = g.permutation(n_phys)[:n_log].astype(np.int32)
    return table, n_phys


def synthetic_layer_rows(shape: ModelShape, n_rows: int, seed: int, key: int = 0) -> np.ndarray:
    """Hidden rows (fp32 residual stream) for a single-layer test, iid N(0, 1)."""
    g = _rng(seed, 9, key)
    return g.standard_normal(size=(n_rows, shape.d_model), dtype=np.float32)


def synthetic_layer_cache(shape: ModelShape, n_tokens: int, seed: int, spread: float = 0.5,
                          key: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """One layer of cached K/V [n][H_kv][d_h] whose per-token scale varies
    (lognormal with sigma ``spread``), so per-token deviations are spread out."""
    g = _rng(seed, 10, key)
    s0 = shape.init_std * np.sqrt(shape.d_model)
    scale = (s0 * np.exp(spread * g.standard_normal(size=(n_tokens, 1, 1)))).astype(np.float32)
    k = g.standard_normal(size=(n_tokens, shape.n_kv_heads, shape.head_dim), dtype=np.float32) * scale
    v = g.standard_normal(size=(n_tokens, shape.n_kv_heads, shape.head_dim), dtype=np.float32) * scale
    if shape.dtype == "bf16":
        k, v = to_bf16_values(k), to_bf16_values(v)
    return k, v


def torch_device_weights(shape: ModelShape, seed: int, device="cuda") -> Dict[str, object]:
    """Seeded N(0, init_std^2) weights drawn directly on the GPU with torch's
    generator, in the library layout (w_qkv, w_o, w_gate_up, w_down; norm gains
    1).  Used where host generation of a full model would take minutes; the
    values differ from ``model_weights``."""
    import torch
    td = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    d, F = shape.d_model, shape.d_ff

    def draw(*dims):
        t = torch.randn(*dims, generator=gen, device=device, dtype=torch.float32)
        t.mul_(shape.init_std)
        return t.to(td)

    gen.manual_seed(int(seed) * 1000003 + 17)
    layers = []
    for _ in range(shape.n_layers):
        layers.append({
            "w_qkv": draw(shape.q_width + 2 * shape.kv_width, d),
            "w_o": draw(d, shape.q_width),
            "w_gate_up": draw(2 * F, d),
            "w_down": draw(d, F),
            "attn_norm": torch.ones(d, device=device, dtype=torch.float32),
            "mlp_norm": torch.ones(d, device=device, dtype=torch.float32),
        })
    return {"layers": layers, "embed": draw(shape.vocab, d), "lm_head": draw(shape.vocab, d),
            "final_norm": torch.ones(d, device=device, dtype=torch.float32)}


def torch_device_layer(shape: ModelShape, seed: int, device="cuda") -> Dict[str, object]:
    """One decoder layer's weights drawn on the GPU (library layout, as in
    ``torch_device_weights``), for single-layer tests at full width where host
    generation would take minutes."""
    import torch
    td = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 29)
    d, F = shape.d_model, shape.d_ff

    def draw(*dims):
        t = torch.randn(*dims, generator=gen, device=device, dtype=torch.float32)
        t.mul_(shape.init_std)
        return t.to(td)

    return {
        "w_qkv": draw(shape.q_width + 2 * shape.kv_width, d),
        "w_o": draw(d, shape.q_width),
        "w_gate_up": draw(2 * F, d),
        "w_down": draw(d, F),
        "attn_norm": torch.ones(d, device=device, dtype=torch.float32),
        "mlp_norm": torch.ones(d, device=device, dtype=torch.float32),
    }


def torch_device_chunk_kv(shape: ModelShape, lens: Sequence[int], seed: int, device="cuda"):
    """Stand-in cached K/V per chunk drawn on the GPU ([L][len][H_kv][d_h],
    N(0, (init_std*sqrt(d))^2)), for throughput runs."""
    import torch
    td = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 7919 + 3)
    s = shape.init_std * float(np.sqrt(shape.d_model))
    out = []
    for l in lens:
        dims = (shape.n_layers, l, shape.n_kv_heads, shape.head_dim)
        k = (torch.randn(dims, generator=gen, device=device) * s).to(td)
        v = (torch.randn(dims, generator=gen, device=device) * s).to(td)
        out.append((k, v))
    return out


@dataclass
class FragmentWorkload:
    """Stored chunks and requests for fragment matching: requests assembled from
    cached documents (whole or in part, at any alignment) plus new text, as in the
    RAG setting the pages describe.  Numbers only -- no hashing here."""
    chunk_size: int
    stored_tokens: np.ndarray      # [n_stored, chunk_size] int32
    stored_ids: np.ndarray         # [n_stored] int64 chunk ids
    stored_offsets: np.ndarray     # [n_stored] int32 stored position (-1: unknown)
    queries: List[np.ndarray]      # int32 token arrays
    prefix_lens: np.ndarray        # [n_queries] int32 prefix-cache coverage


def fragment_workload(seed: int, n_docs: int = 32, chunk_size: int = 256, chunks_per_doc: int = 4,
                      n_queries: int = 4, docs_per_query: int = 4, query_tail: int = 64,
                      vocab: int = 128256, dup_docs: int = 2, unknown_chunks: int = 2) -> FragmentWorkload:
    """Documents of chunks_per_doc chunks are stored chunk by chunk (stored offset =
    the document's start in the request that stored it + the chunk's place in the
    document); dup_docs documents are stored a second time under new ids and
    offsets; unknown_chunks chunks carry the unknown offset.  Each request: random
    filler, then docs_per_query documents (the last one truncated to a random
    length, one placed twice, one chunk copied with a token changed), random
    filler between them, and query_tail new tokens at the end; its prefix
    coverage is 0 or a random length below the first document's start."""
    rng = _rng(seed, 31, 0)
    C = int(chunk_size)
    docs = [rng.integers(0, vocab, size=chunks_per_doc * C, dtype=np.int64).astype(np.int32) for _ in range(n_docs)]
    toks, ids, offs = [], [], []
    next_id = int(rng.integers(1 << 40, 1 << 41))
    for d, doc in enumerate(docs):
        base = int(rng.integers(0, 8)) * 97
        for j in range(chunks_per_doc):
            toks.append(doc[j * C:(j + 1) * C])
            ids.append(next_id)
            offs.append(base + j * C)
            next_id += int(rng.integers(1, 1000))
    for d in rng.choice(n_docs, size=min(dup_docs, n_docs), replace=False):
        base = 5000 + int(rng.integers(0, 100))
        for j in range(chunks_per_doc):
            toks.append(docs[d][j * C:(j + 1) * C])
            ids.append(next_id)
            offs.append(base + j * C)
            next_id += 1
    for i in rng.choice(len(offs), size=min(unknown_chunks, len(offs)), replace=False):
        offs[i] = -1
    queries, prefix = [], []
    for _ in range(n_queries):
        parts = [rng.integers(0, vocab, size=int(rng.integers(0, 300)), dtype=np.int64).astype(np.int32)]
        first_start = len(parts[0])
        picks = list(rng.choice(n_docs, size=min(docs_per_query, n_docs), replace=False))
        picks.append(picks[0])                                    # one document twice
        for i, d in enumerate(picks):
            doc = docs[d]
            if i == len(picks) - 2:
                doc = doc[:int(rng.integers(C // 2, len(doc) + 1))]   # a truncated document
            parts.append(doc)
            parts.append(rng.integers(0, vocab, size=int(rng.integers(0, 40)), dtype=np.int64).astype(np.int32))
        near = docs[picks[1]][:C].copy()
        near[int(rng.integers(0, C))] ^= 1                        # one token away from a stored chunk
        parts.append(near)
        parts.append(rng.integers(0, vocab, size=query_tail, dtype=np.int64).astype(np.int32))
        queries.append(np.concatenate(parts).astype(np.int32))
        prefix.append(0 if rng.random() < 0.5 else int(rng.integers(0, first_start + 1)))
    return FragmentWorkload(C, np.stack(toks).astype(np.int32), np.array(ids, dtype=np.int64),
                            np.array(offs, dtype=np.int32), queries, np.array(prefix, dtype=np.int32))
