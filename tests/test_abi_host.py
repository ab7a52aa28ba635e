"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* the built library exports every function include/cacheblend.h declares;
* the ctypes mirror of every struct has the C layout (checked against a C
  program compiled with gcc from the header);
* invalid arguments are rejected before anything is enqueued, with the
  documented status codes (the fallback contract: the caller then runs a
  full prefill).
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

from cacheblend_selective_recompute_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a 16-byte-aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        from cacheblend_selective_recompute_amd import build
        build.build()
    return _abi.load()


def test_exports_every_declared_function(lib):
    names = _abi.header_functions()
    assert {"cb_rerope_k", "cb_kv_deviation", "cb_select_hkvd", "cb_blend_layer", "cb_blend_prefill",
            "cb_workspace_bytes", "cb_status_string", "cb_last_error", "cb_abi_version",
            "cb_pack_weight", "cb_packed_weight_bytes", "cb_blend_prefill_streamed",
            "cb_streamed_workspace_bytes", "cb_loading_ratio", "cb_decode_step",
            "cb_decode_workspace_bytes", "cb_blend_index_image_bytes", "cb_blend_index_build",
            "cb_blend_match_workspace_bytes", "cb_blend_match"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n


def test_struct_layout_matches_header():
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "cacheblend.h"
#define P(T) printf(#T " %zu\n", sizeof(T));
#define O(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  P(cb_model_cfg) O(cb_model_cfg, rope_theta) O(cb_model_cfg, rms_eps) O(cb_model_cfg, dtype)
  P(cb_layer_w) O(cb_layer_w, mlp_norm)
  P(cb_model) O(cb_model, embed) O(cb_model, layers) O(cb_model, weights_packed)
  P(cb_paged_kv) O(cb_paged_kv, block_size) O(cb_paged_kv, layer_stride) O(cb_paged_kv, kv_format) O(cb_paged_kv, v_scale)
  P(cb_chunk) O(cb_chunk, len) O(cb_chunk, new_start) O(cb_chunk, layer_stride) O(cb_chunk, kv_format) O(cb_chunk, v_scale)
  P(cb_blend_params) O(cb_blend_params, flags) O(cb_blend_params, trace)
  P(cb_trace) O(cb_trace, used) O(cb_trace, kinds)
  P(cb_host_chunk) O(cb_host_chunk, v) O(cb_host_chunk, len) O(cb_host_chunk, new_start)
  P(cb_blend_index_info) O(cb_blend_index_info, table_bits) O(cb_blend_index_info, image_bytes)
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "l")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.split() for l in lines if l.strip())
    for name in ("cb_model_cfg", "cb_layer_w", "cb_model", "cb_paged_kv", "cb_chunk", "cb_blend_params", "cb_trace",
                 "cb_host_chunk", "cb_blend_index_info"):
        cls = getattr(_abi, name)
        assert ctypes.sizeof(cls) == int(got[name]), name
    for key, v in got.items():
        if "." in key:
            s, f = key.split(".")
            assert getattr(getattr(_abi, s), f).offset == int(v), key


def test_status_strings_and_version(lib):
    assert lib.cb_abi_version() == 6
    for code, name in [(0, "CB_OK"), (-1, "CB_ERR_INVALID"), (-2, "CB_ERR_UNSUPPORTED"),
                       (-3, "CB_ERR_WORKSPACE"), (-4, "CB_ERR_DEVICE")]:
        assert lib.cb_status_string(code).decode() == name


def cfg8b(**kw):
    c = _abi.cb_model_cfg(32, 4096, 32, 8, 128, 14336, 128256, 500000.0, 1e-5, _abi.CB_BF16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes(lib):
    c = cfg8b()
    b = lib.cb_workspace_bytes(ctypes.byref(c), 4096, 64, 4)
    T = 4160
    # residual stream x2, activations, MLP hidden, q, o, fresh K/V (fp32): the bulk
    bulk = T * 4096 * 4 * 2 + T * 4096 * 2 + T * 14336 * 2 + T * 4096 * 2 * 2 + T * 2048 * 4
    bulk += 8 * 32768 * (128 * 4 + 8) + (32 << 20) * 4   # split-KV attention and split-K GEMM partials
    assert bulk < b < bulk * 1.05
    assert lib.cb_workspace_bytes(ctypes.byref(c), 8192, 64, 4) > b
    assert lib.cb_workspace_bytes(ctypes.byref(cfg8b(n_layers=1)), 4096, 64, 4) == 0
    assert lib.cb_workspace_bytes(ctypes.byref(c), -1, 64, 4) == 0


def _model(cfg, L=None, packed=None):
    L = L or cfg.n_layers
    layers = (_abi.cb_layer_w * L)(*[_abi.cb_layer_w(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) for _ in range(L)])
    if packed is None:
        packed = 1 if cfg.dtype == _abi.CB_BF16 else 0
    m = _abi.cb_model(cfg, FAKE, FAKE, FAKE, layers, packed)
    m._keep = layers
    return m


def _chunks(specs):
    arr = (_abi.cb_chunk * len(specs))()
    for i, (ln, old, new) in enumerate(specs):
        arr[i] = _abi.cb_chunk(FAKE, FAKE, FAKE, None, ln, old, new, 0, 0)
    return arr


def _paged(n_tokens, bs=16):
    return _abi.cb_paged_kv(FAKE, FAKE, FAKE, bs, (n_tokens + bs - 1) // bs, 0)


def _params(ks, check):
    L = len(ks)
    k = (ctypes.c_int32 * L)(*ks)
    c = (ctypes.c_uint8 * L)(*check)
    p = _abi.cb_blend_params(k, c, 0)
    p._keep = (k, c)
    return p


def _prefill(lib, cfg=None, specs=((64, 0, 0), (64, 5, 64)), nq=8, ks=None, check=None, paged=None,
             ws_bytes=None, packed=None):
    cfg = cfg or cfg8b(n_layers=3)
    m = _model(cfg, packed=packed)
    ch = _chunks(specs)
    N = sum(s[0] for s in specs)
    ks = ks or [N, 19, 19]
    check = check or [0, 1, 1]
    p = _params(ks, check)
    kv = paged or _paged(N + nq)
    need = lib.cb_workspace_bytes(ctypes.byref(cfg), N, nq, len(specs))
    ws = ws_bytes if ws_bytes is not None else need
    st = lib.cb_blend_prefill(ctypes.byref(m), ch, len(specs), FAKE, nq, ctypes.byref(p), ctypes.byref(kv),
                              FAKE, None, None, FAKE, ws, None)
    return st, lib.cb_last_error().decode()


def test_prefill_rejects_unknown_stored_offset(lib):
    st, msg = _prefill(lib, specs=((64, 0, 0), (64, -1, 64)))
    assert st == _abi.CB_ERR_INVALID and "unknown stored offset" in msg


def test_prefill_rejects_overlap_and_gap(lib):
    st, msg = _prefill(lib, specs=((64, 0, 0), (64, 0, 60)))
    assert st == _abi.CB_ERR_INVALID and "overlap" in msg
    st, msg = _prefill(lib, specs=((64, 0, 0), (64, 0, 70)))
    assert st == _abi.CB_ERR_INVALID and "gap" in msg
    st, msg = _prefill(lib, specs=((64, 0, 1), (64, 0, 65)))
    assert st == _abi.CB_ERR_INVALID and "gap" in msg


def test_prefill_rejects_bad_schedule(lib):
    st, msg = _prefill(lib, ks=[100, 19, 19])
    assert st == _abi.CB_ERR_INVALID and "layer 0 runs in full" in msg
    st, msg = _prefill(lib, ks=[128, 19, 20])
    assert st == _abi.CB_ERR_INVALID and "k_per_layer[2]" in msg
    st, msg = _prefill(lib, ks=[128, 19, 10], check=[0, 1, 0])
    assert st == _abi.CB_ERR_INVALID and "unchecked" in msg
    st, msg = _prefill(lib, ks=[128, 129, 19])
    assert st == _abi.CB_ERR_INVALID


def test_prefill_rejects_bad_shapes(lib):
    st, msg = _prefill(lib, cfg=cfg8b(n_layers=3, n_kv_heads=5))
    assert st == _abi.CB_ERR_INVALID and "multiple" in msg
    st, msg = _prefill(lib, cfg=cfg8b(n_layers=3, head_dim=127))
    assert st == _abi.CB_ERR_INVALID and "even" in msg
    st, msg = _prefill(lib, cfg=cfg8b(n_layers=1), ks=[128], check=[0])
    assert st == _abi.CB_ERR_INVALID and "n_layers" in msg
    st, msg = _prefill(lib, cfg=cfg8b(n_layers=3, head_dim=96, n_q_heads=32))
    assert st == _abi.CB_ERR_UNSUPPORTED


def test_prefill_rejects_bad_8bit_cache(lib):
    # every case fails validation (nothing is launched)
    fp8 = _paged(136)
    fp8.kv_format, fp8.k_scale, fp8.v_scale = _abi.CB_KV_FP8_E4M3, 0.0, 1.0
    st, msg = _prefill(lib, paged=fp8)
    assert st == _abi.CB_ERR_INVALID and "scales" in msg
    fp8.k_scale = 1.0
    st, msg = _prefill(lib, paged=fp8)                        # chunks in the model dtype
    assert st == _abi.CB_ERR_UNSUPPORTED and "differs" in msg
    c32 = cfg8b(n_layers=3)
    c32.dtype = _abi.CB_F32
    st, msg = _prefill(lib, cfg=c32, paged=fp8)
    assert st == _abi.CB_ERR_UNSUPPORTED and "CB_BF16" in msg
    bad = _paged(136)
    bad.kv_format = 7
    st, msg = _prefill(lib, paged=bad)
    assert st == _abi.CB_ERR_INVALID and "kv_format" in msg


def test_prefill_rejects_short_block_table_small_workspace_and_empty_query(lib):
    st, msg = _prefill(lib, paged=_paged(100))
    assert st == _abi.CB_ERR_INVALID and "block table" in msg
    st, msg = _prefill(lib, ws_bytes=1024)
    assert st == _abi.CB_ERR_WORKSPACE
    st, msg = _prefill(lib, nq=0)
    assert st == _abi.CB_ERR_INVALID and "n_query" in msg


def test_select_and_deviation_validation(lib):
    st = lib.cb_select_hkvd(FAKE, FAKE, 10, 11, FAKE, None, None, 0, None)
    assert st == _abi.CB_ERR_INVALID
    st = lib.cb_select_hkvd(FAKE, FAKE, 10, -1, FAKE, None, None, 0, None)
    assert st == _abi.CB_ERR_INVALID
    assert lib.cb_select_hkvd(None, None, 10, 0, None, None, None, 0, None) == _abi.CB_OK  # k = 0: nothing to do
    c = cfg8b()
    kv = _paged(128)
    st = lib.cb_kv_deviation(ctypes.byref(c), 40, FAKE, FAKE, 2048, FAKE, 10, ctypes.byref(kv), FAKE, None)
    assert st == _abi.CB_ERR_INVALID and "layer" in lib.cb_last_error().decode()
    st = lib.cb_kv_deviation(ctypes.byref(c), 1, FAKE, FAKE, 100, FAKE, 10, ctypes.byref(kv), FAKE, None)
    assert st == _abi.CB_ERR_INVALID and "row_stride" in lib.cb_last_error().decode()


def test_blend_layer_validation(lib):
    c = cfg8b(n_layers=3)
    m = _model(c)
    kv = _paged(200)
    ws = lib.cb_workspace_bytes(ctypes.byref(c), 128, 8, 0)
    args = lambda layer, nc, nctx, nq, chk, k: (ctypes.byref(m), layer, ctypes.byref(kv), FAKE, nc, nctx, nq, FAKE,
                                                chk, k, FAKE, None, FAKE, ws, None)
    assert lib.cb_blend_layer(*args(0, 128, 128, 8, 1, 19)) == _abi.CB_ERR_INVALID     # layer 0 is not selective
    assert lib.cb_blend_layer(*args(1, 128, 128, 8, 0, 19)) == _abi.CB_ERR_INVALID     # unchecked must keep all
    assert lib.cb_blend_layer(*args(1, 128, 128, 8, 1, 129)) == _abi.CB_ERR_INVALID    # k > candidates
    assert lib.cb_blend_layer(*args(1, 129, 128, 8, 1, 19)) == _abi.CB_ERR_INVALID     # more candidates than context
    assert lib.cb_blend_layer(*args(1, 128, 256, 8, 1, 19)) == _abi.CB_ERR_INVALID     # cache too short for 264 tokens


def test_rerope_validation(lib):
    c = cfg8b()
    kv = _paged(128)
    ch = _chunks([(64, -1, 0)])
    st = lib.cb_rerope_k(ctypes.byref(c), ch, 1, ctypes.byref(kv), 1, FAKE, 1 << 20, None)
    assert st == _abi.CB_ERR_INVALID
    ch = _chunks([(64, 0, 100)])
    st = lib.cb_rerope_k(ctypes.byref(c), ch, 1, ctypes.byref(kv), 1, FAKE, 1 << 20, None)
    assert st == _abi.CB_ERR_INVALID and "block table" in lib.cb_last_error().decode()
    ch = _chunks([(64, 0, 0)])
    st = lib.cb_rerope_k(ctypes.byref(c), ch, 1, ctypes.byref(kv), 4, FAKE, 1 << 20, None)
    assert st == _abi.CB_ERR_INVALID and "flags" in lib.cb_last_error().decode()


def test_prefill_requires_packed_bf16_weights(lib):
    st, msg = _prefill(lib, packed=0)
    assert st == _abi.CB_ERR_INVALID and "weights_packed" in msg
    c = cfg8b(n_layers=3)
    c.dtype = _abi.CB_F32
    st, msg = _prefill(lib, cfg=c, packed=1)
    assert st == _abi.CB_ERR_INVALID and "weights_packed" in msg


def test_packed_weight_bytes(lib):
    # rows are padded to whole 32-row blocks; two bytes per element
    assert lib.cb_packed_weight_bytes(_abi.CB_BF16, 6144, 4096) == 6144 * 4096 * 2
    assert lib.cb_packed_weight_bytes(_abi.CB_BF16, 70, 48) == 96 * 48 * 2
    assert lib.cb_packed_weight_bytes(_abi.CB_BF16, 1, 16) == 32 * 16 * 2
    assert lib.cb_packed_weight_bytes(_abi.CB_F32, 64, 64) == 0
    assert lib.cb_packed_weight_bytes(_abi.CB_BF16, 0, 64) == 0


def test_pack_weight_validation(lib):
    P = lib.cb_pack_weight
    big = 1 << 30
    assert P(_abi.CB_F32, FAKE, 64, 64, 0, FAKE + big, None) == _abi.CB_ERR_UNSUPPORTED
    assert P(_abi.CB_BF16, None, 64, 64, 0, FAKE, None) == _abi.CB_ERR_INVALID
    assert P(_abi.CB_BF16, FAKE, 64, 40, 0, FAKE + big, None) == _abi.CB_ERR_INVALID      # cols % 16
    assert P(_abi.CB_BF16, FAKE, 0, 64, 0, FAKE + big, None) == _abi.CB_ERR_INVALID       # rows < 1
    assert P(_abi.CB_BF16, FAKE, 96, 64, 1, FAKE + big, None) == _abi.CB_ERR_INVALID      # gate_up: 2F, F % 32
    st = P(_abi.CB_BF16, FAKE, 64, 64, 0, FAKE + 1024, None)                              # overlap
    assert st == _abi.CB_ERR_INVALID and "overlap" in lib.cb_last_error().decode()
    assert P(_abi.CB_BF16, FAKE + 8, 64, 64, 0, FAKE + big, None) == _abi.CB_ERR_INVALID  # alignment


def _streamed(lib, specs=((64, 0, 0), (64, 5, 64)), nq=8, events=True, ws_bytes=None, host_k=True, fp8=False):
    cfg = cfg8b(n_layers=3)
    m = _model(cfg)
    arr = (_abi.cb_host_chunk * len(specs))()
    for i, (ln, old, new) in enumerate(specs):
        arr[i] = _abi.cb_host_chunk(FAKE, FAKE if host_k else None, FAKE, ln, old, new)
    N = sum(s[0] for s in specs)
    p = _params([N, 19, 19], [0, 1, 1])
    kv = _paged(N + nq)
    if fp8:
        kv.kv_format, kv.k_scale, kv.v_scale = _abi.CB_KV_FP8_E4M3, 1.0, 1.0
    ev = (ctypes.c_void_p * 6)(*([FAKE] * 6)) if events else None
    need = lib.cb_streamed_workspace_bytes(ctypes.byref(cfg), N, nq, len(specs))
    ws = ws_bytes if ws_bytes is not None else need
    st = lib.cb_blend_prefill_streamed(ctypes.byref(m), arr, len(specs), FAKE, nq, ctypes.byref(p), ctypes.byref(kv),
                                       FAKE, None, None, FAKE, ws, None, None, ev)
    return st, lib.cb_last_error().decode()


def test_streamed_workspace_bytes(lib):
    c = cfg8b()
    base = lib.cb_workspace_bytes(ctypes.byref(c), 4096, 64, 4)
    # three ring slots, each one layer of every chunk's K and V (4096 x 1024 bf16 each)
    assert lib.cb_streamed_workspace_bytes(ctypes.byref(c), 4096, 64, 4) == base + 3 * 2 * 4096 * 1024 * 2
    assert lib.cb_streamed_workspace_bytes(ctypes.byref(cfg8b(n_layers=1)), 4096, 64, 4) == 0


def test_streamed_validation(lib):
    st, msg = _streamed(lib, events=False)
    assert st == _abi.CB_ERR_INVALID and "events" in msg
    st, msg = _streamed(lib, host_k=False)
    assert st == _abi.CB_ERR_INVALID and "K/V" in msg
    st, msg = _streamed(lib, specs=((64, -1, 0), (64, 5, 64)))
    assert st == _abi.CB_ERR_INVALID and "unknown stored offset" in msg
    st, msg = _streamed(lib, specs=((64, 0, 0), (64, 5, 60)))
    assert st == _abi.CB_ERR_INVALID and "overlap" in msg
    st, msg = _streamed(lib, ws_bytes=1024)
    assert st == _abi.CB_ERR_WORKSPACE
    # the layer-pipelined prefill writes caches in the model dtype only
    st, msg = _streamed(lib, fp8=True)
    assert st == _abi.CB_ERR_UNSUPPORTED and "model dtype" in msg


def test_decode_step_validation(lib):
    cfg = cfg8b(n_layers=3)
    m = _model(cfg)
    need = lib.cb_decode_workspace_bytes(ctypes.byref(cfg))
    assert need > 0 and lib.cb_decode_workspace_bytes(ctypes.byref(cfg8b(n_layers=1))) == 0
    kv = _paged(100)
    def call(pos=10, token=FAKE, kvp=kv, ws=need):
        st = lib.cb_decode_step(ctypes.byref(m), ctypes.byref(kvp), pos, token, FAKE, FAKE, ws, None)
        return st, lib.cb_last_error().decode()
    st, msg = call(pos=-1)
    assert st == _abi.CB_ERR_INVALID and "pos" in msg
    st, msg = call(token=None)
    assert st == _abi.CB_ERR_INVALID
    st, msg = call(pos=112)          # the table covers 112 tokens: position 111 is the last one
    assert st == _abi.CB_ERR_INVALID and "covers" in msg
    st, msg = call(ws=need - 256)
    assert st == _abi.CB_ERR_WORKSPACE
