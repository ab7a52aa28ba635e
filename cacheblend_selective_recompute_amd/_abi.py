"""ctypes mirror of include/cacheblend.h and the loader of libcacheblend.so.

The library is the product: there is no fallback.  If the shared object is
missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint8, c_uint32, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcacheblend.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "cacheblend.h")

CB_OK = 0
CB_ERR_INVALID = -1
CB_ERR_UNSUPPORTED = -2
CB_ERR_WORKSPACE = -3
CB_ERR_DEVICE = -4
CB_F32 = 0
CB_BF16 = 1
CB_COPY_V = 1


class cb_model_cfg(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("d_ff", c_int32),
                ("vocab", c_int32), ("rope_theta", c_double), ("rms_eps", c_float), ("dtype", c_int)]


class cb_layer_w(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("w_gate_up", c_void_p),
                ("w_down", c_void_p), ("attn_norm", c_void_p), ("mlp_norm", c_void_p)]


class cb_model(ctypes.Structure):
    _fields_ = [("cfg", cb_model_cfg), ("embed", c_void_p), ("final_norm", c_void_p),
                ("lm_head", c_void_p), ("layers", POINTER(cb_layer_w)), ("weights_packed", c_int32)]


CB_KV_MODEL = 0
CB_KV_FP8_E4M3 = 1


class cb_paged_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("block_table", c_void_p),
                ("block_size", c_int32), ("n_logical", c_int32), ("layer_stride", c_int64),
                ("kv_format", c_int32), ("k_scale", c_float), ("v_scale", c_float)]


class cb_chunk(ctypes.Structure):
    _fields_ = [("tokens", c_void_p), ("k", c_void_p), ("v", c_void_p), ("block_ids", c_void_p),
                ("len", c_int32), ("old_start", c_int32), ("new_start", c_int32),
                ("block_size", c_int32), ("layer_stride", c_int64),
                ("kv_format", c_int32), ("k_scale", c_float), ("v_scale", c_float)]


class cb_host_chunk(ctypes.Structure):
    _fields_ = [("tokens", c_void_p), ("k", c_void_p), ("v", c_void_p),
                ("len", c_int32), ("old_start", c_int32), ("new_start", c_int32)]


class cb_trace(ctypes.Structure):
    _fields_ = [("events", POINTER(c_void_p)), ("capacity", c_int32), ("used", c_int32),
                ("kind_mask", c_uint32), ("kinds", POINTER(c_int32))]


class cb_blend_params(ctypes.Structure):
    _fields_ = [("k_per_layer", POINTER(c_int32)), ("check", POINTER(c_uint8)), ("flags", c_uint32),
                ("trace", POINTER(cb_trace))]


class cb_blend_index_info(ctypes.Structure):
    _fields_ = [("chunk_size", c_int32), ("n_entries", c_int32), ("n_occupants", c_int32), ("n_skipped", c_int32),
                ("slot_bits", c_int32), ("table_bits", c_int32), ("image_bytes", ctypes.c_uint64)]


CB_UNKNOWN_TOKEN_OFFSET = -1
CB_MATCH_MAX_CONTENTS = 4096


KINDS = ["rerope", "gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention", "deviation", "select",
         "scatter", "norm", "lm_head", "other"]


_PROTOS = {
    "cb_rerope_k": (c_int, [POINTER(cb_model_cfg), POINTER(cb_chunk), c_int32, POINTER(cb_paged_kv),
                            c_uint32, c_void_p, c_size_t, c_void_p]),
    "cb_rerope_k_noalloc": (c_int, [POINTER(cb_model_cfg), POINTER(cb_chunk), c_int32, POINTER(cb_paged_kv),
                                    c_uint32, c_void_p]),
    "cb_kv_deviation": (c_int, [POINTER(cb_model_cfg), c_int32, c_void_p, c_void_p, c_int64, c_void_p,
                                c_int32, POINTER(cb_paged_kv), c_void_p, c_void_p]),
    "cb_select_hkvd": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                               c_size_t, c_void_p]),
    "cb_blend_layer": (c_int, [POINTER(cb_model), c_int32, POINTER(cb_paged_kv), c_void_p, c_int32,
                               c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                               c_void_p, c_size_t, c_void_p]),
    "cb_blend_prefill": (c_int, [POINTER(cb_model), POINTER(cb_chunk), c_int32, c_void_p, c_int32,
                                 POINTER(cb_blend_params), POINTER(cb_paged_kv), c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
    "cb_blend_prefill_streamed": (c_int, [POINTER(cb_model), POINTER(cb_host_chunk), c_int32, c_void_p, c_int32,
                                          POINTER(cb_blend_params), POINTER(cb_paged_kv), c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_size_t, c_void_p, c_void_p, POINTER(c_void_p)]),
    "cb_streamed_workspace_bytes": (c_size_t, [POINTER(cb_model_cfg), c_int32, c_int32, c_int32]),
    "cb_loading_ratio": (c_double, [c_double, c_double, c_double, c_double, c_double]),
    "cb_decode_step": (c_int, [POINTER(cb_model), POINTER(cb_paged_kv), c_int32, c_void_p, c_void_p, c_void_p,
                               c_size_t, c_void_p]),
    "cb_decode_workspace_bytes": (c_size_t, [POINTER(cb_model_cfg)]),
    "cb_blend_index_image_bytes": (c_size_t, [c_int32, c_int32]),
    "cb_blend_index_build": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_size_t,
                                     POINTER(cb_blend_index_info)]),
    "cb_blend_match_workspace_bytes": (c_size_t, [c_int64]),
    "cb_blend_match": (c_int, [c_void_p, POINTER(cb_blend_index_info), c_void_p, c_void_p, c_int32, c_int64, c_int32,
                               c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_size_t, c_void_p]),
    "cb_pack_weight": (c_int, [c_int, c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p]),
    "cb_packed_weight_bytes": (c_size_t, [c_int, c_int64, c_int64]),
    "cb_workspace_bytes": (c_size_t, [POINTER(cb_model_cfg), c_int32, c_int32, c_int32]),
    "cb_status_string": (ctypes.c_char_p, [c_int32]),
    "cb_last_error": (ctypes.c_char_p, []),
    "cb_abi_version": (c_int32, []),
}

_lib = None


def header_functions() -> list:
    """Names of the functions include/cacheblend.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(cb_\w+)\s*\(", text, flags=re.M)))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m cacheblend_selective_recompute_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _PROTOS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib
