"""Python binding of libcacheblend: argument marshalling only.

Functions carry the C names (``cb_rerope_k``, ``cb_kv_deviation``,
``cb_select_hkvd``, ``cb_blend_layer``, ``cb_blend_prefill``,
``cb_workspace_bytes``).  They take torch tensors that already live on the GPU,
pack them into the C structs and call the library on the current torch stream.
PyTorch provides device memory and streams only; every step of the blended
prefill runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _abi
from ._abi import (CB_BF16, CB_COPY_V, CB_F32, CB_KV_FP8_E4M3, CB_KV_MODEL, CB_OK, cb_blend_params, cb_chunk, cb_host_chunk, cb_layer_w, cb_model,
                   cb_model_cfg, cb_paged_kv)


class CacheBlendError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _abi.load()
        self.status = status
        name = lib.cb_status_string(status).decode()
        detail = lib.cb_last_error().decode()
        super().__init__(f"{where}: {name}: {detail}")


def _check(st: int, where: str):
    if st != CB_OK:
        raise CacheBlendError(st, where)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream: Optional[torch.cuda.Stream] = None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def torch_dtype(dt: str) -> torch.dtype:
    return torch.bfloat16 if dt == "bf16" else torch.float32


def make_cfg(shape) -> cb_model_cfg:
    """cb_model_cfg of a cbinputs.ModelShape."""
    return cb_model_cfg(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                        shape.d_ff, shape.vocab, float(shape.rope_theta), float(shape.rms_eps),
                        CB_BF16 if shape.dtype == "bf16" else CB_F32)


# ----------------------------------------------------------------------------
# device-side containers
# ----------------------------------------------------------------------------

def cb_packed_weight_bytes(dtype: str, rows: int, cols: int) -> int:
    return int(_abi.load().cb_packed_weight_bytes(CB_BF16 if dtype == "bf16" else CB_F32, rows, cols))


def cb_pack_weight(w: torch.Tensor, gate_up: bool = False, stream=None) -> torch.Tensor:
    """Packed copy of a bf16 row-major [rows][cols] device matrix (cb_pack_weight)."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("cb_pack_weight: a contiguous 2-D bf16 tensor is required")
    rows, cols = w.shape
    nbytes = cb_packed_weight_bytes("bf16", rows, cols)
    out = torch.empty(max(nbytes // 2, 1), dtype=torch.bfloat16, device=w.device)
    _check(_abi.load().cb_pack_weight(CB_BF16, _p(w), rows, cols, 1 if gate_up else 0, _p(out), _stream(stream)),
           "cb_pack_weight")
    return out


class DeviceModel:
    """Decoder weights on the GPU in the library's layout.

    ``layers`` are dicts of torch tensors: ``w_qkv`` [(Hq+2Hkv)dh][d],
    ``w_o`` [d][Hq dh], ``w_gate_up`` [2F][d], ``w_down`` [d][F] in the model
    dtype and fp32 ``attn_norm`` / ``mlp_norm``, all row-major.  For bf16
    models the four matrices of every layer dict are replaced, in place, by
    their packed copies (cb_pack_weight) as the model is built, so the
    row-major originals can be freed; ``packed=True`` says they already are.
    """

    MATS = ("w_qkv", "w_o", "w_gate_up", "w_down")

    def __init__(self, shape, layers: List[dict], embed: torch.Tensor, lm_head: torch.Tensor,
                 final_norm: torch.Tensor, packed: bool = False):
        self.shape = shape
        self.embed = embed
        self.lm_head = lm_head
        self.final_norm = final_norm
        self.cfg = make_cfg(shape)
        self.weights_packed = 1 if shape.dtype == "bf16" else 0
        if self.weights_packed and not packed:
            for w in layers:
                for name in self.MATS:
                    w[name] = cb_pack_weight(w[name], gate_up=(name == "w_gate_up"))
        self.layers = layers
        arr = (cb_layer_w * shape.n_layers)()
        for l, w in enumerate(layers):
            arr[l] = cb_layer_w(w["w_qkv"].data_ptr(), w["w_o"].data_ptr(), w["w_gate_up"].data_ptr(),
                                w["w_down"].data_ptr(), w["attn_norm"].data_ptr(), w["mlp_norm"].data_ptr())
        self._c_layers = arr
        self.c = cb_model(self.cfg, embed.data_ptr(), final_norm.data_ptr(), lm_head.data_ptr(), arr,
                          self.weights_packed)

    @classmethod
    def from_numpy(cls, shape, weights: dict, device="cuda") -> "DeviceModel":
        """From cbinputs.model_weights (fp32 arrays holding model-dtype values)."""
        td = torch_dtype(shape.dtype)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(td)

        layers = []
        for w in weights["layers"]:
            layers.append({
                "w_qkv": up(np.concatenate([w["wq"], w["wk"], w["wv"]], axis=0)),
                "w_o": up(w["wo"]),
                "w_gate_up": up(np.concatenate([w["w_gate"], w["w_up"]], axis=0)),
                "w_down": up(w["w_down"]),
                "attn_norm": torch.from_numpy(np.asarray(w["attn_norm"], np.float32)).to(device),
                "mlp_norm": torch.from_numpy(np.asarray(w["mlp_norm"], np.float32)).to(device),
            })
        return cls(shape, layers, up(weights["embed"]), up(weights["lm_head"]),
                   torch.from_numpy(np.asarray(weights["final_norm"], np.float32)).to(device))

    @classmethod
    def from_tensors(cls, shape, t: dict) -> "DeviceModel":
        """From cbinputs.torch_device_weights output (already in the library layout)."""
        return cls(shape, t["layers"], t["embed"], t["lm_head"], t["final_norm"])


def fp8_encode(x: torch.Tensor, scale: float) -> torch.Tensor:
    """FP8 E4M3 bytes (torch.uint8) of x / scale, saturated at +-448 (input
    preparation for 8-bit caches; the library itself rounds on the GPU)."""
    y = (x.float() / float(scale)).clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def fp8_decode(b: torch.Tensor, scale: float) -> torch.Tensor:
    """fp32 values of FP8 E4M3 bytes times scale."""
    return b.view(torch.float8_e4m3fn).float() * float(scale)


class PagedKV:
    """Paged K/V pools [L][n_phys * bs][Hkv][dh] plus a block table.  With
    kv_format CB_KV_FP8_E4M3 the pools hold one FP8 E4M3 byte per element
    (torch.uint8 storage) standing for element x k_scale (K) or x v_scale (V)."""

    def __init__(self, shape, n_tokens: int, block_size: int = 16, block_table: Optional[np.ndarray] = None,
                 n_phys: Optional[int] = None, device="cuda", fill: Optional[float] = None,
                 kv_format: int = CB_KV_MODEL, k_scale: float = 1.0, v_scale: float = 1.0):
        self.shape = shape
        self.n_tokens = n_tokens
        self.block_size = block_size
        n_log = (n_tokens + block_size - 1) // block_size
        if block_table is None:
            block_table = np.arange(n_log, dtype=np.int32)
        block_table = np.asarray(block_table, dtype=np.int32)
        self.n_phys = int(n_phys if n_phys is not None else max(int(block_table.max(initial=-1)) + 1, n_log))
        self.kv_format, self.k_scale, self.v_scale = int(kv_format), float(k_scale), float(v_scale)
        fp8 = self.kv_format == CB_KV_FP8_E4M3
        td = torch.uint8 if fp8 else torch_dtype(shape.dtype)
        dims = (shape.n_layers, self.n_phys * block_size, shape.n_kv_heads, shape.head_dim)
        if fill is None:
            self.k = torch.empty(dims, dtype=td, device=device)
            self.v = torch.empty(dims, dtype=td, device=device)
        elif fp8:
            self.k = fp8_encode(torch.full(dims, fill, device=device), self.k_scale)
            self.v = fp8_encode(torch.full(dims, fill, device=device), self.v_scale)
        else:
            self.k = torch.full(dims, fill, dtype=td, device=device)
            self.v = torch.full(dims, fill, dtype=td, device=device)
        self.block_table_host = block_table
        self.block_table = torch.from_numpy(block_table).to(device)
        self.c = cb_paged_kv(self.k.data_ptr(), self.v.data_ptr(), self.block_table.data_ptr(), block_size,
                             len(block_table), self.n_phys * block_size * shape.kv_width, self.kv_format,
                             self.k_scale, self.v_scale)

    def slots(self, positions) -> torch.Tensor:
        """Physical row of each logical position (host computation on the host copy of the table)."""
        p = np.asarray(positions, dtype=np.int64)
        rows = self.block_table_host[p // self.block_size].astype(np.int64) * self.block_size + p % self.block_size
        return torch.from_numpy(rows).to(self.k.device)

    def logical(self, n: Optional[int] = None):
        """(K, V) [L][n][Hkv][dh] in logical position order (a copy; an FP8 cache is
        returned as the fp32 values it stands for)."""
        n = self.n_tokens if n is None else n
        idx = self.slots(np.arange(n))
        if self.kv_format == CB_KV_FP8_E4M3:
            return fp8_decode(self.k[:, idx], self.k_scale), fp8_decode(self.v[:, idx], self.v_scale)
        return self.k[:, idx], self.v[:, idx]


@dataclass
class ChunkSource:
    """One cached chunk on the GPU: tokens, K/V (contiguous [L][len][Hkv][dh] or a
    paged pool with block ids), the stored offset and the new offset."""
    tokens: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    old_start: int
    new_start: int
    block_ids: Optional[torch.Tensor] = None
    block_size: int = 16
    layer_stride: int = 0
    kv_format: int = CB_KV_MODEL
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def len(self) -> int:
        return int(self.tokens.numel())

    def c(self) -> cb_chunk:
        return cb_chunk(self.tokens.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                        self.block_ids.data_ptr() if self.block_ids is not None else None,
                        self.len, int(self.old_start), int(self.new_start),
                        int(self.block_size if self.block_ids is not None else 0), int(self.layer_stride),
                        int(self.kv_format), float(self.k_scale), float(self.v_scale))


@dataclass
class HostChunk:
    """One cached chunk whose K/V stay in page-locked host memory (contiguous
    [L][len][Hkv][dh] CPU tensors with pin_memory) for the layer-pipelined
    prefill; tokens are on the GPU."""
    tokens: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    old_start: int
    new_start: int

    @property
    def len(self) -> int:
        return int(self.tokens.numel())

    def c(self) -> cb_host_chunk:
        if not (self.k.is_pinned() and self.v.is_pinned() and self.k.is_contiguous() and self.v.is_contiguous()):
            raise ValueError("HostChunk: K/V must be contiguous page-locked CPU tensors")
        return cb_host_chunk(self.tokens.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.len,
                             int(self.old_start), int(self.new_start))


class LayerEvents:
    """2 x n_layers HIP events for cb_blend_prefill_streamed (created through
    torch, so they belong to the runtime the library's streams come from)."""

    def __init__(self, n_layers: int):
        self.ev = [torch.cuda.Event() for _ in range(2 * n_layers)]
        for e in self.ev:
            e.record()            # materialises the underlying event
        self.arr = (ctypes.c_void_p * len(self.ev))(*[e.cuda_event for e in self.ev])


def _chunk_array(chunks: Sequence[ChunkSource]):
    arr = (cb_chunk * max(1, len(chunks)))()
    for i, c in enumerate(chunks):
        arr[i] = c.c()
    return arr


class Workspace:
    """A reusable device workspace (uint8 tensor)."""

    def __init__(self, nbytes: int, device="cuda"):
        self.t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    @property
    def nbytes(self) -> int:
        return self.t.numel()


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def cb_workspace_bytes(cfg: cb_model_cfg, n_ctx: int, n_query: int, n_chunks: int) -> int:
    return int(_abi.load().cb_workspace_bytes(ctypes.byref(cfg), n_ctx, n_query, n_chunks))


def _ws(ws: Optional[Workspace], need: int, device, stream=None) -> Workspace:
    """The caller's workspace, or a temporary one.  A temporary workspace is freed
    when the call returns, while the kernels may still run: it is marked as used
    on the call's stream, so the caching allocator hands its memory out again only
    after that stream's work up to this point has finished."""
    if ws is None or ws.nbytes < need:
        ws = Workspace(need, device)
        if stream is not None:
            ws.t.record_stream(stream)
    return ws


def cb_rerope_k(cfg: cb_model_cfg, chunks: Sequence[ChunkSource], dst: PagedKV, flags: int = CB_COPY_V,
                ws: Optional[Workspace] = None, stream=None) -> None:
    lib = _abi.load()
    w = _ws(ws, cb_workspace_bytes(cfg, 0, 0, len(chunks)), dst.k.device, stream)
    arr = _chunk_array(chunks)
    _check(lib.cb_rerope_k(ctypes.byref(cfg), arr, len(chunks), ctypes.byref(dst.c), flags, w.ptr, w.nbytes,
                           _stream(stream)), "cb_rerope_k")


def cb_rerope_k_noalloc(cfg: cb_model_cfg, chunks: Sequence[ChunkSource], dst: PagedKV, flags: int = CB_COPY_V,
                        stream=None) -> None:
    """cb_rerope_k with the library's static per-GPU scratch instead of a workspace."""
    lib = _abi.load()
    arr = _chunk_array(chunks)
    _check(lib.cb_rerope_k_noalloc(ctypes.byref(cfg), arr, len(chunks), ctypes.byref(dst.c), flags, _stream(stream)),
           "cb_rerope_k_noalloc")


def cb_kv_deviation(cfg: cb_model_cfg, layer: int, k_fresh: torch.Tensor, v_fresh: torch.Tensor,
                    pos: torch.Tensor, cache: PagedKV, dev_out: torch.Tensor, stream=None) -> None:
    """k_fresh / v_fresh: fp32 [n][>= Hkv*dh] views sharing one row stride."""
    assert k_fresh.dtype == torch.float32 and v_fresh.dtype == torch.float32
    assert k_fresh.stride(0) == v_fresh.stride(0) and k_fresh.stride(-1) == 1
    lib = _abi.load()
    _check(lib.cb_kv_deviation(ctypes.byref(cfg), layer, _p(k_fresh), _p(v_fresh), k_fresh.stride(0), _p(pos),
                               int(pos.numel()), ctypes.byref(cache.c), _p(dev_out), _stream(stream)),
           "cb_kv_deviation")


def cb_select_hkvd(dev: torch.Tensor, pos: torch.Tensor, k: int, sel_pos: torch.Tensor,
                   sel_slot: Optional[torch.Tensor] = None, stream=None) -> None:
    lib = _abi.load()
    _check(lib.cb_select_hkvd(_p(dev), _p(pos), int(pos.numel()), int(k), _p(sel_pos), _p(sel_slot), None, 0,
                              _stream(stream)), "cb_select_hkvd")


def cb_blend_layer(model: DeviceModel, layer: int, kv: PagedKV, pos_in: torch.Tensor, n_ctx: int, n_query: int,
                   x: torch.Tensor, check_flag: bool, k_keep: int, pos_out: torch.Tensor,
                   dev_out: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None, stream=None) -> None:
    lib = _abi.load()
    w = _ws(ws, cb_workspace_bytes(model.cfg, n_ctx, n_query, 0), x.device, stream)
    _check(lib.cb_blend_layer(ctypes.byref(model.c), layer, ctypes.byref(kv.c), _p(pos_in), int(pos_in.numel()),
                              n_ctx, n_query, _p(x), int(bool(check_flag)), int(k_keep), _p(pos_out), _p(dev_out),
                              w.ptr, w.nbytes, _stream(stream)), "cb_blend_layer")


class BlendParams:
    def __init__(self, k_per_layer: Sequence[int], check: Sequence[int], flags: int = 0):
        L = len(k_per_layer)
        self._k = (ctypes.c_int32 * L)(*[int(v) for v in k_per_layer])
        self._c = (ctypes.c_uint8 * L)(*[1 if v else 0 for v in check])
        self.c = cb_blend_params(self._k, self._c, flags)


def cb_streamed_workspace_bytes(cfg: cb_model_cfg, n_ctx: int, n_query: int, n_chunks: int) -> int:
    return int(_abi.load().cb_streamed_workspace_bytes(ctypes.byref(cfg), n_ctx, n_query, n_chunks))


def cb_loading_ratio(kv_bytes_per_token: float, n_tokens: float, load_bytes_per_s: float, prefill_seconds: float,
                     r_min: float = 0.15) -> float:
    return float(_abi.load().cb_loading_ratio(float(kv_bytes_per_token), float(n_tokens), float(load_bytes_per_s),
                                              float(prefill_seconds), float(r_min)))


def cb_blend_prefill_streamed(model: DeviceModel, chunks: Sequence[HostChunk], query_tokens: torch.Tensor,
                              params: BlendParams, blended: PagedKV, logits: torch.Tensor,
                              hkvd_out: Optional[torch.Tensor] = None, dev_out: Optional[torch.Tensor] = None,
                              ws: Optional[Workspace] = None, stream=None, copy_stream=None,
                              events: Optional[LayerEvents] = None):
    """Enqueues the layer-pipelined prefill and returns (events, copy_stream, workspace):
    the caller keeps them, and the host chunks, alive until `stream` has finished."""
    lib = _abi.load()
    n_ctx = sum(c.len for c in chunks)
    w = _ws(ws, cb_streamed_workspace_bytes(model.cfg, n_ctx, int(query_tokens.numel()), len(chunks)),
            logits.device, stream)
    arr = (cb_host_chunk * max(1, len(chunks)))()
    for i, c in enumerate(chunks):
        arr[i] = c.c()
    ev = events if events is not None else LayerEvents(model.shape.n_layers)
    cs = copy_stream if copy_stream is not None else torch.cuda.Stream()
    _check(lib.cb_blend_prefill_streamed(ctypes.byref(model.c), arr, len(chunks), _p(query_tokens),
                                         int(query_tokens.numel()), ctypes.byref(params.c), ctypes.byref(blended.c),
                                         _p(logits), _p(hkvd_out), _p(dev_out), w.ptr, w.nbytes, _stream(stream),
                                         _stream(cs), ev.arr),
           "cb_blend_prefill_streamed")
    return ev, cs, w


def cb_decode_workspace_bytes(cfg: cb_model_cfg) -> int:
    return int(_abi.load().cb_decode_workspace_bytes(ctypes.byref(cfg)))


def cb_decode_step(model: DeviceModel, kv: PagedKV, pos: int, token: torch.Tensor, logits: torch.Tensor,
                   ws: Optional[Workspace] = None, stream=None) -> None:
    """One token at position `pos` through every layer over the cache [0, pos); its K/V land at pos."""
    lib = _abi.load()
    w = _ws(ws, cb_decode_workspace_bytes(model.cfg), logits.device, stream)
    _check(lib.cb_decode_step(ctypes.byref(model.c), ctypes.byref(kv.c), int(pos), _p(token), _p(logits), w.ptr,
                              w.nbytes, _stream(stream)), "cb_decode_step")


def cb_blend_prefill(model: DeviceModel, chunks: Sequence[ChunkSource], query_tokens: torch.Tensor,
                     params: BlendParams, blended: PagedKV, logits: torch.Tensor,
                     hkvd_out: Optional[torch.Tensor] = None, dev_out: Optional[torch.Tensor] = None,
                     ws: Optional[Workspace] = None, stream=None, _arr=None) -> None:
    lib = _abi.load()
    n_ctx = sum(c.len for c in chunks)
    w = _ws(ws, cb_workspace_bytes(model.cfg, n_ctx, int(query_tokens.numel()), len(chunks)), logits.device, stream)
    arr = _arr if _arr is not None else _chunk_array(chunks)
    _check(lib.cb_blend_prefill(ctypes.byref(model.c), arr, len(chunks), _p(query_tokens),
                                int(query_tokens.numel()), ctypes.byref(params.c), ctypes.byref(blended.c),
                                _p(logits), _p(hkvd_out), _p(dev_out), w.ptr, w.nbytes, _stream(stream)),
           "cb_blend_prefill")


# ----------------------------------------------------------------------------
# fragment matching
# ----------------------------------------------------------------------------

def cb_blend_index_image_bytes(n_chunks: int, chunk_size: int) -> int:
    return int(_abi.load().cb_blend_index_image_bytes(int(n_chunks), int(chunk_size)))


def cb_blend_index_build(tokens: np.ndarray, chunk_ids: np.ndarray, token_offsets: np.ndarray):
    """Host build of the index image: returns (cb_blend_index_info, uint8 host array of
    info.image_bytes)."""
    lib = _abi.load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    if tokens.ndim != 2:
        raise ValueError("tokens must be [n_chunks][chunk_size]")
    n, C = tokens.shape
    ids = np.ascontiguousarray(chunk_ids, dtype=np.int64)
    offs = np.ascontiguousarray(token_offsets, dtype=np.int32)
    if ids.shape != (n,) or offs.shape != (n,):
        raise ValueError("chunk_ids and token_offsets must have one entry per chunk")
    nbytes = cb_blend_index_image_bytes(n, C)
    image = np.zeros(max(nbytes, 1), dtype=np.uint8)
    info = _abi.cb_blend_index_info()
    _check(lib.cb_blend_index_build(tokens.ctypes.data if n else None, ids.ctypes.data if n else None,
                                    offs.ctypes.data if n else None, n, C, image.ctypes.data, nbytes,
                                    ctypes.byref(info)), "cb_blend_index_build")
    return info, image[:info.image_bytes].copy()


class BlendIndexImage:
    """An index image built on the host and copied to device memory as it is."""

    def __init__(self, tokens: np.ndarray, chunk_ids: np.ndarray, token_offsets: np.ndarray, device="cuda"):
        self.info, self.host = cb_blend_index_build(tokens, chunk_ids, token_offsets)
        self.dev = torch.empty(max(self.host.size, 256), dtype=torch.uint8, device=device)
        self.dev[:self.host.size].copy_(torch.from_numpy(self.host))


def cb_blend_match_workspace_bytes(total_tokens: int) -> int:
    return int(_abi.load().cb_blend_match_workspace_bytes(int(total_tokens)))


def cb_blend_match(index: BlendIndexImage, query_tokens: torch.Tensor, query_starts: torch.Tensor, total_tokens: int,
                   max_query_len: int, probe_stride: int = 1, prefix_lens: Optional[torch.Tensor] = None,
                   max_matches: int = 64, ws: Optional[Workspace] = None, stream=None, out: Optional[dict] = None):
    """Match a batch of requests (tokens back to back, int32 starts [n+1] on the device).
    Returns the device outputs: chunk [n][max_matches] int64, old_st / cur_st int32,
    kept uint8 and count [n] int32."""
    lib = _abi.load()
    n = int(query_starts.numel()) - 1
    dev = query_starts.device
    if out is None:
        out = {"chunk": torch.empty((n, max_matches), dtype=torch.int64, device=dev),
               "old_st": torch.empty((n, max_matches), dtype=torch.int32, device=dev),
               "cur_st": torch.empty((n, max_matches), dtype=torch.int32, device=dev),
               "kept": torch.empty((n, max_matches), dtype=torch.uint8, device=dev),
               "count": torch.empty(max(n, 0), dtype=torch.int32, device=dev)}
    w = _ws(ws, cb_blend_match_workspace_bytes(total_tokens), dev, stream)
    _check(lib.cb_blend_match(_p(index.dev), ctypes.byref(index.info), _p(query_tokens), _p(query_starts), n,
                              int(total_tokens), int(max_query_len), int(probe_stride), _p(prefix_lens),
                              int(max_matches), _p(out["chunk"]), _p(out["old_st"]), _p(out["cur_st"]),
                              _p(out["kept"]), _p(out["count"]), w.ptr, w.nbytes, _stream(stream)), "cb_blend_match")
    return out
