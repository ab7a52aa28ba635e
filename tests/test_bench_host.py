"""Host-side checks of bench.py (CPU): the algorithmic work it divides by, the
one-GPU guard, and the reading of the committed traffic summary."""
import os
import subprocess
import sys

import numpy as np

import bench
import cbinputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _c2():
    shape = cbinputs.SHAPES["llama3-8b"]
    N, Q, k = 4096, 64, 614
    L = shape.n_layers
    ks = [N] + [k] * (L - 1)
    rng = np.random.default_rng(0)
    first = np.sort(rng.choice(N, size=k, replace=False))
    sets = {l: first for l in range(1, L)}
    return shape, N, Q, ks, sets, [1024] * 4


def test_projection_flops_are_two_p_per_recomputed_row():
    # a7 + a10: 2 x (parameters of a layer's projections) FLOP per recomputed row and layer
    shape, N, Q, ks, sets, lens = _c2()
    w = bench.work_per_kind(shape, N, Q, ks, sets, lens)
    d, F, qw, kvw = shape.d_model, shape.d_ff, shape.q_width, shape.kv_width
    P = d * (qw + 2 * kvw) + qw * d + 3 * d * F          # Q/K/V, O, gate/up/down
    T, R, L = N + Q, ks[1] + Q, shape.n_layers
    assert P == 218_103_808                              # the 8B shape: 218.1 M per layer
    # layer 0: every row, context K/V not recomputed; layer 1: K/V of every candidate
    l0 = 2.0 * T * (d * qw + qw * d + 3 * d * F) + 2.0 * Q * d * 2 * kvw
    rest = (L - 1) * 2.0 * R * P + 2.0 * N * d * 2 * kvw - 2.0 * ks[1] * d * 2 * kvw
    total = sum(w[k] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down"))
    assert abs(total - (l0 + rest)) <= 1e-9 * total


def test_attention_flops_count_visible_keys():
    shape, N, Q, ks, sets, lens = _c2()
    w = bench.work_per_kind(shape, N, Q, ks, sets, lens)
    T = N + Q
    per_key = 4.0 * shape.head_dim * shape.n_q_heads
    vis0 = T * (T + 1) / 2.0
    vis = float(np.sum(sets[1] + 1)) + sum(N + i + 1 for i in range(Q))
    assert abs(w["attention"] - per_key * (vis0 + (shape.n_layers - 1) * vis)) <= 1e-9 * w["attention"]


def test_fused_keep_all_layers_drop_their_own_kinds():
    # with every candidate kept after layer 1, only layer 1 launches deviation and top-k,
    # and only layers 0 and 1 launch a scatter
    shape, N, Q, ks, sets, lens = _c2()
    a = bench.work_per_kind(shape, N, Q, ks, sets, lens, fused_keep_all=False)
    b = bench.work_per_kind(shape, N, Q, ks, sets, lens, fused_keep_all=True)
    kvw, es, k = shape.kv_width, 2, ks[1]
    assert b["deviation"] == N * (kvw * (2 * 4 + 2 * es) + 8)
    assert b["select"] == N * 8 + k * 8
    assert b["scatter"] == (Q + k + Q) * kvw * (2 * 4 + 2 * es)
    assert a["deviation"] > b["deviation"] and a["select"] > b["select"] and a["scatter"] > b["scatter"]
    for kind in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention", "rerope", "lm_head", "norm"):
        assert a[kind] == b[kind]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_traffic_summary_is_read_only_for_the_unchanged_source():
    import hashlib
    for wl in ("70b-4x1024-q64", "8b-4x1024-q64"):
        path = os.path.join(ROOT, "profiles", f"gemm_gate_up_{wl}_traffic.md")
        if not os.path.exists(path):
            assert bench.traffic_from_profile("gemm_gate_up", wl) is None
            continue
        fields = dict(line[2:].strip().split(": ", 1) for line in open(path) if line.startswith("- ") and ": " in line)
        same = hashlib.sha256(open(os.path.join(ROOT, fields["kernel_source"]), "rb").read()).hexdigest() == \
            fields["kernel_source_sha256"]
        v = bench.traffic_from_profile("gemm_gate_up", wl)
        if same:
            assert v == int(fields["traffic_bytes_per_launch"]) and v > 0
        else:                        # the kernel changed since the counters were taken
            assert v is None
    assert bench.traffic_from_profile("gemm_gate_up", "no-such-workload") is None


def test_other_workloads_spec():
    spec = "8b-4x1024-q64, 70b-4x1024-q64,8b-16x512j-q64@0,8b-16x512j-q64@0.05,8b-16x512j-q64@0,8b-16x512j-q64"
    got = bench.other_workloads(spec, "70b-4x1024-q64", 0.15)
    assert got == {"8b-4x1024-q64": [0.15], "8b-16x512j-q64": [0.0, 0.05, 0.15]}
    # the main run's workload at another ratio stays; at its own ratio it is dropped
    assert bench.other_workloads("70b-4x1024-q64@1", "70b-4x1024-q64", 0.15) == {"70b-4x1024-q64": [1.0]}
    assert bench.other_workloads("", "x", 0.15) == {}
