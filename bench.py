#!/usr/bin/env python3
"""Blended-prefill throughput on one MI355X.

One step = one cb_blend_prefill call over a whole request: re-RoPE assembly of
the cached chunks into the blended cache, layer 0 in full, selective recompute
at every later layer (K/V projection, deviation, top-k, scatter, Q projection,
attention, O and MLP) and the final-position logits.  Chunk caches, weights and
tokens are resident in HBM before the timed region starts.

Prints one JSON line: context tokens/s (N / step time), the roofline position
of the dominant kernel (its duration measured with HIP events on the library's
stream during the timed region), a per-kind breakdown from an untimed traced
step, and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps 10] [--warmup 3] [--workload 70b-4x1024-q64] [--ratio 0.15]

The default workload is the largest that fits one GPU: the 70B-shaped decoder
(80 layers, d 8192, 64 q / 8 kv heads, F 28672) over 4 chunks x 1024 tokens
plus a 64-token query.  The 8B 4 x 1024 + 64 and the 8B 32 x 1024 + 128 paged
workloads, and the 8B blend of 16 jittered chunks (8K context at random stored
offsets) at r = 0, 5, 15, 30 and 100%, are timed after it and reported under
"other_workloads"."""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blended-prefill context tokens/s @15% recompute; % HBM / MFMA roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # fp32 vector

MFMA_KINDS = {"gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention"}


def log(msg):
    """Progress on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="70b-4x1024-q64")
    ap.add_argument("--other-workloads",
                    default="8b-4x1024-q64,8b-32x1024-q128-paged," + ",".join(
                        f"8b-16x512j-q64@{r:g}" for r in (0.0, 0.05, 0.15, 0.3, 1.0)),
                    help="comma-separated workloads timed after the main one, each optionally "
                         "name@ratio (default ratio: --ratio); empty: none")
    ap.add_argument("--other-steps", type=int, default=5)
    ap.add_argument("--ratio", type=float, default=0.15)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-runs", type=int, default=5,
                    help="extra untimed-by-contract runs, each after evicting the Infinity Cache")
    ap.add_argument("--decode-steps", type=int, default=16,
                    help="decode steps timed on the blended cache after the runs (0: skip)")
    ap.add_argument("--streamed-runs", type=int, default=3,
                    help="runs of the layer-pipelined prefill from host memory (0: skip)")
    ap.add_argument("--fp8-runs", type=int, default=5,
                    help="timed runs of the same prefill over an 8-bit (FP8) KV cache (0: skip)")
    ap.add_argument("--match-runs", type=int, default=20,
                    help="timed runs of fragment matching on a 64-request batch (0: skip)")
    ap.add_argument("--sweep", action="store_true",
                    help="only the size sweep of cb_rerope_k and cb_kv_deviation (one JSON line per size)")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the copy / library GEMM measurement of achievable peaks")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    return ap.parse_args()


class Hip:
    """hipEvent helpers straight from the HIP runtime (the library records the events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            arr[i] = e
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


def traffic_from_profile(kind, workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/<kind>_<workload>_traffic.md: FETCH_SIZE + WRITE_SIZE
    passes scaled by a plain copy of known size), or None when there is no
    summary or the kernel source changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"{kind}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            fields[k] = v
    try:
        src = os.path.join(root, fields["kernel_source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != fields["kernel_source_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def work_per_kind(shape, N, Q, ks, sets, chunk_lens, fused_keep_all=False):
    """Algorithmic FLOPs (MFMA kinds) or HBM bytes (the others) of one step.

    sets[l]: positions kept at layer l (ascending), for the attention count.
    fused_keep_all: the layers that keep every candidate took their deviations,
    wrote their fresh K/V and their (identity) top-k's row maps inside the Q/K/V
    product's split-K reduction (no deviation, select or scatter launch of their
    own), so those bytes are not counted under those kinds."""
    d, F = shape.d_model, shape.d_ff
    qw, kvw = shape.q_width, shape.kv_width
    es = 2 if shape.dtype == "bf16" else 4
    L = shape.n_layers
    T = N + Q
    w = {k: 0.0 for k in ("rerope", "gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention",
                          "deviation", "select", "scatter", "norm", "lm_head")}
    # layer 0: every row; context K/V from the cache
    w["gemm_qkv"] += 2.0 * T * d * qw + 2.0 * Q * d * 2 * kvw
    w["gemm_o"] += 2.0 * T * qw * d
    w["gemm_gate_up"] += 2.0 * T * d * 2 * F
    w["gemm_down"] += 2.0 * T * F * d
    w["attention"] += 4.0 * shape.head_dim * shape.n_q_heads * (T * (T + 1) / 2.0)
    w["scatter"] += Q * kvw * (2 * 4 + 2 * es)
    w["norm"] += T * d * (4 + es)          # layer 0 attention norm; every other layer-wide norm
    nc = N                                  # rides on the O / down projection launches
    for l in range(1, L):
        k = ks[l]
        w["gemm_qkv"] += 2.0 * (nc + Q) * d * 2 * kvw + 2.0 * (k + Q) * d * qw
        w["gemm_o"] += 2.0 * (k + Q) * qw * d
        w["gemm_gate_up"] += 2.0 * (k + Q) * d * 2 * F
        w["gemm_down"] += 2.0 * (k + Q) * F * d
        vis = float(sum(int(p) + 1 for p in sets[l])) + sum(N + i + 1 for i in range(Q))
        w["attention"] += 4.0 * shape.head_dim * shape.n_q_heads * vis
        fused = fused_keep_all and k == nc
        if not fused:
            w["deviation"] += nc * (kvw * (2 * 4 + 2 * es) + 4 + 4)
            w["scatter"] += (k + Q) * kvw * (2 * 4 + 2 * es)
            w["select"] += nc * 8 + k * 8
        if k != nc:
            w["norm"] += (k + Q) * d * (4 + es)     # the kept rows' queries, normalised apart
        nc = k
    w["norm"] += d * (4 + 4)
    w["lm_head"] += shape.vocab * d * es
    w["rerope"] += sum(chunk_lens) * L * kvw * es * 4        # K and V, read + write
    return w


MATCH_CHUNK = 256           # the pages' default chunk_size


def match_workload(seed):
    """64 requests of the 4 x 1024 + 64 shape (documents of 4 chunks of 256 tokens,
    one placed twice, new text between them) over 16448 stored documents."""
    import cbinputs
    return cbinputs.fragment_workload(seed + 5, n_docs=16384, chunk_size=MATCH_CHUNK, n_queries=64, docs_per_query=4,
                                      dup_docs=64, unknown_chunks=64)


def match_runs(torch, api, seed, runs):
    """Fragment matching of one request batch against the index: the index is
    built on the host once (timed apart), the batch sits in HBM, and `runs`
    back-to-back cb_blend_match calls are timed with events."""
    import numpy as np
    w = match_workload(seed)
    t0 = time.perf_counter()
    index = api.BlendIndexImage(w.stored_tokens, w.stored_ids, w.stored_offsets)
    build_s = time.perf_counter() - t0
    lens = [len(q) for q in w.queries]
    starts = np.zeros(len(lens) + 1, dtype=np.int32)
    starts[1:] = np.cumsum(lens)
    tq = torch.from_numpy(np.concatenate(w.queries).astype(np.int32)).cuda()
    ts = torch.from_numpy(starts).cuda()
    pl = torch.from_numpy(w.prefix_lens).cuda()
    total, mx = int(starts[-1]), max(lens)
    ws = api.Workspace(api.cb_blend_match_workspace_bytes(total))
    out = api.cb_blend_match(index, tq, ts, total, mx, 1, pl, 64, ws)
    for _ in range(3):
        api.cb_blend_match(index, tq, ts, total, mx, 1, pl, 64, ws, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(runs):
        api.cb_blend_match(index, tq, ts, total, mx, 1, pl, 64, ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / runs
    cnt = out["count"].cpu().numpy()
    kept = out["kept"].cpu().numpy()
    n_kept = sum(int(kept[q, :max(0, min(int(c), kept.shape[1]))].sum()) for q, c in enumerate(cnt))
    windows = sum(max(0, n - MATCH_CHUNK + 1) for n in lens)
    return {"requests": len(lens), "tokens": total, "windows": int(windows), "chunk_size": MATCH_CHUNK,
            "index_chunks": int(len(w.stored_ids)), "index_entries": int(index.info.n_entries),
            "image_mb": round(index.info.image_bytes / 1e6, 1), "host_index_build_s": round(build_s, 3),
            "ms_per_batch": round(ms, 4), "requests_per_s": round(len(lens) / (ms * 1e-3), 1),
            "tokens_per_s": round(total / (ms * 1e-3), 1), "windows_per_s": round(windows / (ms * 1e-3), 1),
            "matches": int(cnt.sum()), "kept": n_kept, "runs": runs}


def match_cpu_baseline(seed, n_sample=4):
    """The oracle matcher on a sample of the same request batch (host cores)."""
    from oracle import match as om
    w = match_workload(seed)
    idx = om.BlendIndex(MATCH_CHUNK)
    t0 = time.perf_counter()
    idx.add_all(w.stored_tokens, w.stored_ids, w.stored_offsets)
    build = time.perf_counter() - t0
    t0 = time.perf_counter()
    for q in w.queries[:n_sample]:
        om.resolve_leftmost_greedy(om.match(idx, q, 1), MATCH_CHUNK)
    per_req = (time.perf_counter() - t0) / n_sample
    return {"value": round(1.0 / per_req, 2), "unit": "requests/s", "cores": 1, "kind": "oracle",
            "sample": f"pure-Python oracle matcher, {n_sample} of the 64 requests ({per_req * 1e3:.0f} ms each); "
                      f"oracle index build {build:.1f} s"}


def host_layer(t, shape):
    """fp32 host copies of one library-layout (unpacked) device layer, in the
    oracle's layout."""
    qw, kvw, F = shape.q_width, shape.kv_width, shape.d_ff
    h = lambda x: x.float().cpu().numpy()
    qkv = h(t["w_qkv"])
    gu = h(t["w_gate_up"])
    return {"wq": qkv[:qw], "wk": qkv[qw:qw + kvw], "wv": qkv[qw + kvw:], "wo": h(t["w_o"]),
            "w_gate": gu[:F], "w_up": gu[F:], "w_down": h(t["w_down"]),
            "attn_norm": h(t["attn_norm"]), "mlp_norm": h(t["mlp_norm"])}


class DeviceRows:
    """Rows of a device matrix gathered on demand (the oracle reads only the
    embedding rows of the request's tokens)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, idx):
        import numpy as np
        import torch
        i = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(self.t.device)
        return self.t[i].float().cpu().numpy()


CPU_LAYERS = 5    # layers of the oracle's bounded sample (about 10 s of host work at the 70B shape)


def cpu_baseline(wl, sample):
    """The oracle (float32 NumPy, OpenBLAS sgemm on the host cores) on a bounded
    sample of the same workload, with the same weights and chunk caches as the
    GPU run (host copies of the first CPU_LAYERS layers): 3 and CPU_LAYERS layers
    timed (the difference, per layer, gives one selective layer), extrapolated to
    the full depth."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info() if p.get("internal_api") == "openblas"]
                    or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    L = wl.shape.n_layers
    n = min(CPU_LAYERS, L)
    layers, glob, kvs = sample
    m = oracle.OracleModel.from_shape(wl.shape.with_layers(n), lambda l: layers[l], glob)
    chunks = [(wl.chunk_tokens[c], kvs[c][0], kvs[c][1], wl.old_starts[c], wl.new_starts[c]) for c in range(len(kvs))]
    ks, ch = wl.schedule()
    lo = min(3, n - 1)
    times = {}
    for nl in (lo, n):
        t0 = time.perf_counter()
        oracle.blend_prefill(m, chunks, wl.query_tokens, ks[:n], ch[:n], layers_limit=nl)
        times[nl] = time.perf_counter() - t0
    per_layer = max((times[n] - times[lo]) / (n - lo), 1e-9)
    total = times[n] + (L - n) * per_layer
    return {"value": wl.n_ctx / total, "unit": "context tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"float32 NumPy oracle (sgemm), layers 0-{n - 1} of the {wl.name} blend on the GPU run's own "
                       f"weights and chunk caches, timed over {lo} and {n} layers ({times[lo] + times[n]:.1f} s of "
                       f"host work; one selective layer {per_layer:.2f} s), "
                       f"extrapolated to {L} layers ({total:.1f} s per request)")}


def measured_peaks(torch, dev):
    """What the box sustains with random data: a plain device copy (1 GiB read +
    1 GiB written) and torch's bf16 GEMM (hipBLASLt) at 8192^3, for the
    roofline fractions against measured rather than datasheet peaks."""
    a = torch.empty(256 << 20, dtype=torch.float32, device=dev).uniform_()
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    # 8192^3 with the blend's operand statistics (activations N(0, 1), weights N(0, 0.03^2);
    # the power the matrix cores draw depends on the data), in both layouts; the faster is
    # the reference (x @ w^T, the layout of [out][in] weights, on every box measured)
    n = 8192
    x = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    w = (torch.randn(n, n, device=dev) * 0.03).to(torch.bfloat16)
    rates = {}
    for layout, f in (("x @ w", lambda: x @ w), ("x @ w^T", lambda: x @ w.t())):
        for _ in range(3):
            y = f()
        e0.record()
        for _ in range(10):
            y = f()
        e1.record()
        torch.cuda.synchronize()
        rates[layout] = 10 * 2.0 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, w, y
    torch.cuda.empty_cache()
    best = max(rates, key=rates.get)
    return {"copy_gbs": round(copy_gbs, 1), "bf16_gemm_tflops": round(rates[best], 1),
            "bf16_gemm_tflops_by_layout": {k: round(v, 1) for k, v in rates.items()},
            "how": f"torch copy_ of 1 GiB fp32 (read + write); torch bf16 matmul 8192^3 (hipBLASLt), "
                   f"activations N(0,1), weights N(0,0.03^2), the faster layout ({best})"}


def kernel_sweep(torch, dev):
    """Size sweep (about 1 MB to 1 GB of algorithmic traffic) of the two
    bandwidth-bound entry points that run alone: cb_rerope_k (K rotated, V
    copied; 4 x L x H_kv x d_h x 2 B per token) and cb_kv_deviation (fresh fp32
    K/V read, cached bf16 K/V gathered; 12 KiB per row at the 8B width).  Each
    run follows a 512 MiB read that evicts the Infinity Cache (a read, so no
    dirty lines are left to write back); one JSON line per size with the median
    of 10 runs."""
    import numpy as np
    import cbinputs
    from cacheblend_selective_recompute_amd import api
    ints = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    evict = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def timed(fn, reps=10):
        ts = []
        for r in range(reps + 2):
            evict.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    shape = cbinputs.SHAPES["llama3-8b"]
    cfg = api.make_cfg(shape)
    per_tok = 4 * shape.n_layers * shape.kv_width * 2
    for n in (4, 16, 64, 256, 1024, 4096):
        gen = torch.Generator(device=dev)
        gen.manual_seed(n)
        dims = (shape.n_layers, n, shape.n_kv_heads, shape.head_dim)
        k = torch.randn(dims, generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(dims, generator=gen, device=dev).to(torch.bfloat16)
        ch = [api.ChunkSource(ints(np.zeros(n)), k, v, 0, 0)]
        dst = api.PagedKV(shape, n, 16)
        ws = api.Workspace(api.cb_workspace_bytes(cfg, 0, 0, 1), dev)
        ms = timed(lambda: api.cb_rerope_k(cfg, ch, dst, api.CB_COPY_V, ws))
        b = n * per_tok
        print(json.dumps({"sweep": "cb_rerope_k", "tokens": n, "bytes": b, "us": round(ms * 1e3, 2),
                          "gbs": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}),
              flush=True)
        del k, v, ch, dst
    sh2 = shape.with_layers(2)
    cfg2 = api.make_cfg(sh2)
    kvw = shape.kv_width
    per_row = kvw * (2 * 4 + 2 * 2) + 4 + 4
    for n in (85, 341, 1365, 5461, 21845, 87381):
        cache = api.PagedKV(sh2, n, 16, fill=0.5)
        kf = torch.randn(n, 2 * kvw, device=dev)
        pos = ints(np.arange(n))
        out = torch.empty(n, device=dev)
        ms = timed(lambda: api.cb_kv_deviation(cfg2, 1, kf[:, :kvw], kf[:, kvw:], pos, cache, out))
        b = n * per_row
        print(json.dumps({"sweep": "cb_kv_deviation", "rows": n, "bytes": b, "us": round(ms * 1e3, 2),
                          "gbs": round(b / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}),
              flush=True)
        del cache, kf, pos, out


def decode_runs(torch, api, model, shape, blended, logits, T, steps):
    """Decode steps straight on the blended cache (positions T, T+1, ...): time
    per token and the HBM rate of what one step must read (every weight matrix,
    the LM head and the cache of every layer up to the position)."""
    import numpy as np
    ws = api.Workspace(api.cb_decode_workspace_bytes(model.cfg))
    tok = torch.tensor([1234], dtype=torch.int32, device="cuda")
    if blended.n_tokens < T + steps + 1:
        return None
    api.cb_decode_step(model, blended, T, tok, logits, ws)       # warm-up (position T)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        api.cb_decode_step(model, blended, T + i, tok, logits, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    es = 2 if shape.dtype == "bf16" else 4
    d, F, qw, kvw = shape.d_model, shape.d_ff, shape.q_width, shape.kv_width
    w_bytes = shape.n_layers * (d * (qw + 2 * kvw) + qw * d + 2 * F * d + F * d) * es + shape.vocab * d * es
    kv_bytes = shape.n_layers * (T + steps / 2) * kvw * 2 * es
    gbs = (w_bytes + kv_bytes) / (ms * 1e-3) / 1e9
    return {"ms_per_token": round(ms, 4), "tokens_per_s": round(1e3 / ms, 1), "steps": steps, "from_position": T,
            "bytes_per_token": int(w_bytes + kv_bytes), "achieved_gbs": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def fp8_runs(torch, api, model, shape, chunks, qtok, params, T, N, runs):
    """The same blended prefill with 8-bit (FP8 E4M3) chunk caches and blended
    cache: one K and one V scale, max |value| / 448 over the chunk caches."""
    import numpy as np
    ks = max(float(c.k.float().abs().max()) for c in chunks) / 448.0
    vs = max(float(c.v.float().abs().max()) for c in chunks) / 448.0
    f8 = [api.ChunkSource(c.tokens, api.fp8_encode(c.k, ks), api.fp8_encode(c.v, vs), c.old_start, c.new_start,
                          block_ids=c.block_ids, block_size=c.block_size, layer_stride=c.layer_stride,
                          kv_format=api.CB_KV_FP8_E4M3, k_scale=ks, v_scale=vs) for c in chunks]
    kv = api.PagedKV(shape, T, 16, kv_format=api.CB_KV_FP8_E4M3, k_scale=ks, v_scale=vs)
    logits = torch.empty(shape.vocab, device="cuda")
    ws = api.Workspace(api.cb_workspace_bytes(model.cfg, N, int(qtok.numel()), len(f8)))
    arr = api._chunk_array(f8)
    for _ in range(2):
        api.cb_blend_prefill(model, f8, qtok, params, kv, logits, None, None, ws, _arr=arr)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(runs):
        api.cb_blend_prefill(model, f8, qtok, params, kv, logits, None, None, ws, _arr=arr)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / runs
    kv_bytes = sum(2 * c.k.numel() for c in f8)
    return {"ms_per_step": round(ms, 4), "context_tokens_per_s": round(N / (ms * 1e-3), 1),
            "chunk_kv_bytes": kv_bytes, "k_scale": ks, "v_scale": vs, "runs": runs,
            "logits_finite": bool(torch.isfinite(logits).all())}


def streamed_runs(torch, api, model, chunks, qtok, params, blended, logits, hkvd, N, runs):
    """The layer-pipelined prefill with the chunk caches in page-locked host
    memory: per-run time (host -> device copies included), the time a plain copy
    of the same bytes takes alone, and how much of it the recompute hides."""
    import numpy as np
    host = []
    for c in chunks:
        hk = torch.empty(c.k.shape, dtype=c.k.dtype, pin_memory=True)
        hv = torch.empty(c.v.shape, dtype=c.v.dtype, pin_memory=True)
        hk.copy_(c.k.cpu())
        hv.copy_(c.v.cpu())
        host.append(api.HostChunk(c.tokens, hk, hv, c.old_start, c.new_start))
    kv_bytes = sum(2 * h.k.numel() * h.k.element_size() for h in host)
    # a plain copy of the same bytes, alone
    dst = [torch.empty(h.k.shape, dtype=h.k.dtype, device="cuda") for h in host]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        e0.record()
        for h, d in zip(host, dst):
            d.copy_(h.k, non_blocking=True)
            d.copy_(h.v, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1)
    del dst
    cs = torch.cuda.Stream()
    ev = api.LayerEvents(model.shape.n_layers)
    ws = api.Workspace(api.cb_streamed_workspace_bytes(model.cfg, N, int(qtok.numel()), len(host)))
    ts = []
    for r in range(runs + 1):
        e0.record()
        api.cb_blend_prefill_streamed(model, host, qtok, params, blended, logits, hkvd, None, ws, copy_stream=cs,
                                      events=ev)
        e1.record()
        torch.cuda.synchronize()
        if r > 0:
            ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    return {"ms_per_step": round(ms, 4), "context_tokens_per_s": round(N / (ms * 1e-3), 1),
            "kv_bytes_from_host": kv_bytes, "plain_h2d_copy_ms": round(copy_ms, 4),
            "h2d_gbs": round(kv_bytes / (copy_ms * 1e-3) / 1e9, 1), "runs": runs,
            "note": "chunk caches in page-locked host memory, copied layer by layer inside the timed call"}


class Inputs:
    """One workload resident in HBM: packed model, chunk caches, blended cache,
    tokens, outputs and workspace."""

    def __init__(self, torch, api, wl, seed, dev, host_sample=False):
        import numpy as np
        import cbinputs
        shape = wl.shape
        N, Q, T = wl.n_ctx, wl.n_query, wl.n_total
        weights = cbinputs.torch_device_weights(shape, seed, dev)
        self.sample = None
        if host_sample:          # the oracle's copy of the first layers before the library packs them
            layers = [host_layer(weights["layers"][l], shape) for l in range(min(CPU_LAYERS, shape.n_layers))]
            glob = {"embed": DeviceRows(weights["embed"]), "lm_head": weights["lm_head"].float().cpu().numpy(),
                    "final_norm": weights["final_norm"].float().cpu().numpy()}
        self.model = api.DeviceModel.from_tensors(shape, weights)
        del weights
        kvs = cbinputs.torch_device_chunk_kv(shape, wl.chunk_lens, seed, dev)
        if host_sample:
            nl = min(CPU_LAYERS, shape.n_layers)
            self.sample = (layers, glob, [(k[:nl].float().cpu().numpy(), v[:nl].float().cpu().numpy()) for k, v in kvs])
        ints = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        if wl.paged:
            chunks = []
            for c, (K, V) in enumerate(kvs):
                ln = wl.chunk_lens[c]
                nb = (ln + 15) // 16
                ids, n_phys = cbinputs.paged_layout(ln, 16, seed, key=1000 + c, spare_blocks=2)
                Kp = torch.zeros((shape.n_layers, n_phys * 16, shape.n_kv_heads, shape.head_dim), dtype=K.dtype,
                                 device=dev)
                Vp = torch.zeros_like(Kp)
                rows = torch.from_numpy((np.repeat(ids.astype(np.int64), 16) * 16
                                         + np.tile(np.arange(16), nb))[:ln]).to(dev)
                Kp[:, rows] = K
                Vp[:, rows] = V
                chunks.append(api.ChunkSource(ints(wl.chunk_tokens[c]), Kp, Vp, wl.old_starts[c], wl.new_starts[c],
                                              block_ids=ints(ids), block_size=16,
                                              layer_stride=n_phys * 16 * shape.kv_width))
            del kvs
            table, n_phys = cbinputs.paged_layout(T + 64, 16, seed, key=77, spare_blocks=8)
            self.blended = api.PagedKV(shape, T + 64, 16, table, n_phys)
        else:
            chunks = [api.ChunkSource(ints(wl.chunk_tokens[c]), kvs[c][0], kvs[c][1], wl.old_starts[c],
                                      wl.new_starts[c]) for c in range(len(kvs))]
            self.blended = api.PagedKV(shape, T + 64, 16)   # room for the decode steps after the prefill
        self.chunks = chunks
        self.qtok = ints(wl.query_tokens)
        self.logits = torch.empty(shape.vocab, device=dev)
        self.hkvd = torch.empty((shape.n_layers, N), dtype=torch.int32, device=dev)
        self.ws = api.Workspace(api.cb_workspace_bytes(self.model.cfg, N, Q, len(chunks)), dev)
        self.arr = api._chunk_array(chunks)

    def run(self, api, params):
        api.cb_blend_prefill(self.model, self.chunks, self.qtok, params, self.blended, self.logits, self.hkvd, None,
                             self.ws, _arr=self.arr)


def time_blend(torch, api, _abi, hip, inp, wl, steps, warmup):
    """Warm-up (the last warm-up step traced for the per-kind breakdown), then
    `steps` timed steps with the dominant kind bracketed by events on the
    library's stream.  Returns (ms_per_step, roofline dict, breakdown, keep-all
    layer count, fused flag)."""
    shape = wl.shape
    N, Q = wl.n_ctx, wl.n_query
    ks, ch = wl.schedule()
    plain = api.BlendParams(ks, ch)
    for _ in range(max(0, warmup - 1)):
        inp.run(api, plain)
    cap = 4096 if shape.n_layers <= 40 else 8192
    ev_all = hip.events(cap)
    kinds_all = (ctypes.c_int32 * (cap // 2))()
    tr_all = _abi.cb_trace(ev_all, cap, 0, (1 << len(_abi.KINDS)) - 1, kinds_all)
    p_all = api.BlendParams(ks, ch)
    p_all.c.trace = ctypes.pointer(tr_all)
    inp.run(api, p_all)
    torch.cuda.synchronize()
    sets = {l: inp.hkvd[l, :ks[l]].cpu().numpy() for l in range(1, shape.n_layers)}
    kind_ms, kind_n = {}, {}
    for i in range(tr_all.used // 2):
        k = _abi.KINDS[kinds_all[i]]
        kind_ms[k] = kind_ms.get(k, 0.0) + hip.elapsed_ms(ev_all[2 * i], ev_all[2 * i + 1])
        kind_n[k] = kind_n.get(k, 0) + 1
    # one scatter launch per layer, except the layers that keep every candidate when
    # their Q/K/V reduction wrote the cache
    keep_all = sum(1 for l in range(1, shape.n_layers) if ks[l] == (N if l == 1 else ks[l - 1]))
    fused_keep_all = keep_all > 0 and kind_n.get("scatter", 0) == shape.n_layers - keep_all
    work = work_per_kind(shape, N, Q, ks, sets, wl.chunk_lens, fused_keep_all)
    dominant = max((k for k in kind_ms if k in work), key=lambda k: kind_ms[k])
    dom_id = _abi.KINDS.index(dominant)

    per_step = 2 * kind_n[dominant]
    ev = hip.events(per_step * steps)
    traces, params = [], []
    for s in range(steps):
        sub = ctypes.cast(ctypes.byref(ev, s * per_step * ctypes.sizeof(ctypes.c_void_p)),
                          ctypes.POINTER(ctypes.c_void_p))
        t = _abi.cb_trace(sub, per_step, 0, 1 << dom_id, None)
        p = api.BlendParams(ks, ch)
        p.c.trace = ctypes.pointer(t)
        traces.append(t)
        params.append(p)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        inp.run(api, params[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / steps
    dom_ms, launches = 0.0, 0
    for s in range(steps):
        for i in range(traces[s].used // 2):
            dom_ms += hip.elapsed_ms(ev[s * per_step + 2 * i], ev[s * per_step + 2 * i + 1])
            launches += 1
    avg_launch_ms = dom_ms / max(launches, 1)
    work_per_launch = work[dominant] / kind_n[dominant]
    if dominant in MFMA_KINDS:
        peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = work_per_launch / (avg_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "unit": "TFLOP/s"}
    else:
        peak = PEAK_HBM_GBS
        achieved = work_per_launch / (avg_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "unit": "GB/s"}
    roof.update({"kernel": dominant, "achieved": round(achieved, 2), "peak": peak, "frac": round(achieved / peak, 4),
                 "traffic": traffic_from_profile(dominant, wl.name), "launches_per_step": kind_n[dominant],
                 "avg_launch_ms": round(avg_launch_ms, 4), "work_per_launch": work_per_launch})
    breakdown = {}
    for k, ms in sorted(kind_ms.items(), key=lambda kv: -kv[1]):
        e = {"ms": round(ms, 4), "launches": kind_n[k]}
        if k in work and ms > 0:
            if k in MFMA_KINDS:
                e["tflops"] = round(work[k] / (ms * 1e-3) / 1e12, 1)
            else:
                e["gbs"] = round(work[k] / (ms * 1e-3) / 1e9, 1)
        breakdown[k] = e
    return ms_per_step, roof, breakdown, keep_all, fused_keep_all


def other_workloads(spec, main_name, main_ratio):
    """Parse --other-workloads: comma-separated `name` or `name@ratio` entries into
    {name: [ratios in the order given]}, dropping duplicates and the main run's own
    (workload, ratio) pair; a bare name takes the main run's ratio."""
    out = {}
    for item in [w.strip() for w in spec.split(",") if w.strip()]:
        name, _, r = item.partition("@")
        ratio = float(r) if r else main_ratio
        if (name, ratio) == (main_name, main_ratio):
            continue
        ratios = out.setdefault(name, [])
        if ratio not in ratios:
            ratios.append(ratio)
    return out


def config_of(wl, ratio, n_chunks):
    shape = wl.shape
    return {"workload": wl.name, "shape": f"{shape.n_layers}L d{shape.d_model} {shape.n_q_heads}q/"
                                          f"{shape.n_kv_heads}kv x{shape.head_dim} F{shape.d_ff}",
            "n_ctx": wl.n_ctx, "n_query": wl.n_query, "chunks": n_chunks, "ratio": ratio, "k": wl.k,
            "paged": bool(wl.paged), "block_size": 16}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}); the blended prefill of one "
              f"request is not sharded here, and independent requests scale by running one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import cbinputs
    from cacheblend_selective_recompute_amd import api, _abi

    torch.cuda.set_device(0)
    wl = cbinputs.make_workload(args.workload, seed=args.seed, ratio=args.ratio)
    shape = wl.shape
    N, Q, T = wl.n_ctx, wl.n_query, wl.n_total
    ks, ch = wl.schedule()
    dev = "cuda"
    if args.sweep:
        kernel_sweep(torch, dev)
        return

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    hip = Hip()
    log(f"{wl.name}: weights, chunk caches and buffers")
    inp = Inputs(torch, api, wl, args.seed, dev, host_sample=not args.no_cpu_baseline)
    log(f"{wl.name}: {args.warmup} warm-up and {args.steps} timed steps")
    ms_per_step, roof, breakdown, keep_all, fused_keep_all = time_blend(torch, api, _abi, hip, inp, wl, args.steps,
                                                                         args.warmup)
    plain = api.BlendParams(ks, ch)
    # cold runs: a 512 MiB read between runs evicts the 256 MiB Infinity Cache (the
    # chunk caches and weights then come from HBM, as for a request that just arrived)
    evict = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    cold = []
    for s in range(args.cold_runs):
        evict.sum()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        inp.run(api, plain)
        c1.record()
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    del evict
    log(f"{wl.name}: {ms_per_step:.3f} ms per step; measured peaks, decode, matching, FP8, streamed legs")
    peaks = measured_peaks(torch, dev) if args.peaks else None
    model, chunks, qtok, blended, logits, hkvd = inp.model, inp.chunks, inp.qtok, inp.blended, inp.logits, inp.hkvd
    decode = decode_runs(torch, api, model, shape, blended, logits, T, args.decode_steps) if args.decode_steps else None
    match = match_runs(torch, api, args.seed, args.match_runs) if args.match_runs > 0 else None
    fp8 = fp8_runs(torch, api, model, shape, chunks, qtok, plain, T, N, args.fp8_runs) \
        if args.fp8_runs > 0 and shape.dtype == "bf16" else None
    streamed = None
    if args.streamed_runs > 0 and not wl.paged:
        streamed = streamed_runs(torch, api, model, chunks, qtok, plain, blended, logits, hkvd, N, args.streamed_runs)
    if peaks:
        mp = peaks["bf16_gemm_tflops"] if roof["bound"] == "mfma" else peaks["copy_gbs"]
        roof["frac_of_measured_peak"] = round(roof["achieved"] / mp, 4)
    sample = inp.sample
    n_chunks = len(chunks)
    del inp, model, chunks, qtok, blended, logits, hkvd
    torch.cuda.empty_cache()

    others = {}
    for name, ratios in other_workloads(args.other_workloads, wl.name, args.ratio).items():
        log(f"{name}: setup, then {args.other_steps} timed steps at r = {', '.join(f'{r:g}' for r in ratios)}")
        oinp = Inputs(torch, api, cbinputs.make_workload(name, seed=args.seed, ratio=ratios[0]), args.seed, dev)
        for ratio in ratios:              # the inputs do not depend on the ratio; only k does
            owl = cbinputs.make_workload(name, seed=args.seed, ratio=ratio)
            oms, oroof, obd, _, _ = time_blend(torch, api, _abi, hip, oinp, owl, args.other_steps, 2)
            others[name if ratio == args.ratio else f"{name}@{ratio:g}"] = {
                "value": round(owl.n_ctx / (oms * 1e-3), 1), "unit": "context tokens/s",
                "ms_per_step": round(oms, 4), "steps": args.other_steps,
                "config": config_of(owl, ratio, len(oinp.chunks)), "roofline": oroof,
                "kernels_ms_per_step": obd}
        del oinp
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": round(N / (ms_per_step * 1e-3), 1),
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded random-init weights and chunk caches drawn on the GPU)",
        "config": config_of(wl, args.ratio, n_chunks),
        "roofline": roof,
        "kernels_ms_per_step": breakdown,
        "deviation_scatter_in_qkv_reduce": {"layers": keep_all if fused_keep_all else 0,
                                             "note": "layers keeping every candidate take their deviations, write "
                                                     "their fresh K/V and the identity top-k's row maps in the Q/K/V "
                                                     "split-K reduction (gemm_qkv)"},
        "cold_ms_per_step": ({"median": round(float(np.median(cold)), 4), "min": round(min(cold), 4), "runs": len(cold)}
                             if cold else None),
        "measured_peaks": peaks,
        "other_workloads": others,
        "streamed": streamed,
        "decode": decode,
        "match": match,
        "fp8_kv": fp8,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"{wl.name}: oracle on the host cores (layers 0-{min(CPU_LAYERS, wl.shape.n_layers) - 1})")
        out["cpu_baseline"] = cpu_baseline(wl, sample)
        if match is not None:
            out["cpu_baseline"]["match"] = match_cpu_baseline(args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
