"""Plain CPU oracle of the CacheBlend blended prefill (NumPy, float32).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark; never by the GPU library.

Method source: "CacheBlend 完全拆解" (pinghaoyang.com.cn), cited below as [CB]
with the section it comes from.  Model block: the Llama-3-shaped pre-norm
decoder that the workloads name; the pages give only Q=hW_Q, K=hW_K (then
RoPE), V=hW_V ([CB] "问题：拼接的 KV 缓存到底少了什么").

Precision: every array is float32 and every product a float32 (OpenBLAS sgemm)
product; the RoPE angles pos*theta_i and their cos/sin are evaluated in float64
and rounded once to float32, the rotation itself is float32 arithmetic.  Values
the method stores (the KV cache, in its storage dtype) are rounded from float32
to that dtype (bf16: round to nearest even) where the method writes them.
``precision("f64")`` runs the same code in float64 (cos/sin unrounded, storage
rounding straight from float64); the tests use it as an extra pin only.

``operands("bf16")`` is the arithmetic of a bf16 model computed with bf16
operands and fp32 accumulation: every operand of a matrix product is rounded
to bf16 first (the normalised rows and the SwiGLU hidden rows going into the
projections, the attention output going into W_O, the rotated queries, the
softmax weights going into the product with V, whose normaliser is the sum of
the same rounded weights), sums and everything else stay float32; the LM head
multiplies the bf16 weights by the float32 normalised row.  Weights and cached
K/V of a bf16 model are bf16 values already and are used as they are.  The
default ("f32") rounds no operand.

Readings taken where the pages are silent (all listed in the design notes):
  * layer 0 runs in full over every row; its context K/V are the re-RoPE'd
    cache (they depend on the token alone); the first checked layer is 1;
  * deviation = squared L2 over the concatenated K and V of all KV heads, K
    compared after RoPE at the new position, fresh values unrounded, summed in
    the compute precision;
  * r counts context tokens only: k = floor(r*N + 0.5); the query suffix is
    recomputed at every layer, written to the cache, never ranked;
  * ties in the top-k go to the smaller position; sets are reported ascending;
  * rows written at layer l are exactly S_l plus the suffix, before attention;
  * RoPE rotates adjacent pairs (2i, 2i+1) by pos*theta_i,
    theta_i = base^(-2i/d_h);
  * RMSNorm eps from the model, gains as given; SiLU-gated MLP; no biases;
    untied LM head after a final RMSNorm; attention scale 1/sqrt(d_h).

Parity status: every public function below is pinned by a test in
``tests/test_oracle_*.py`` against something other than itself (torch CPU
library routines, complex-number rotation, brute-force sorting, closed forms,
the method's own special cases r=0% / r=100% / single chunk).
"""
from __future__ import annotations

import contextlib
import os
from dataclasses import dataclass
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64
_CT = [np.float32]          # compute precision (one-element list: set by ``precision``)


def ct():
    """The compute dtype: numpy.float32 unless inside ``precision("f64")``."""
    return _CT[0]


@contextlib.contextmanager
def precision(name: str):
    """Run the oracle in "f32" (the default) or "f64" inside the block."""
    old = _CT[0]
    _CT[0] = {"f32": np.float32, "f64": np.float64}[name]
    try:
        yield
    finally:
        _CT[0] = old


def _a(x) -> np.ndarray:
    return np.asarray(x, dtype=ct())


_OPS = ["f32"]              # operand rounding of matrix products (set by ``operands``)


@contextlib.contextmanager
def operands(name: str):
    """Round the operands of every matrix product to bf16 ("bf16") or not ("f32",
    the default) inside the block."""
    if name not in ("f32", "bf16"):
        raise ValueError(name)
    old = _OPS[0]
    _OPS[0] = name
    try:
        yield
    finally:
        _OPS[0] = old


def _op(x) -> np.ndarray:
    """A matrix-product operand: rounded to bf16 under ``operands("bf16")``."""
    x = _a(x)
    return store_round(x, "bf16") if _OPS[0] == "bf16" else x


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------

FP8_E4M3_MAX = 448.0


def fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest value of the OCP FP8 E4M3 grid (1 sign, 4 exponent bits with bias
    7, 3 mantissa bits; subnormals down to 2^-9; largest finite 448, no
    infinities), ties to even, magnitudes beyond 448 saturated to 448.
    A value of magnitude a in binade [2^e, 2^(e+1)) (e >= -6; below that the
    subnormal spacing) sits on the grid of step 2^(e-3)."""
    x = _a(x)
    a = np.abs(x)
    _, E = np.frexp(a)                       # a = f * 2^E, f in [0.5, 1)
    e = np.clip(E - 1, -6, 8)
    step = np.ldexp(np.ones_like(a), e - 3)  # a power of two: a / step and the product are exact
    r = np.minimum(np.rint(a / step) * step, a.dtype.type(FP8_E4M3_MAX))
    return np.where(x < 0, -r, r)


def store_round(x: np.ndarray, storage: str, scale: float = 1.0) -> np.ndarray:
    """Round ``x`` to the storage dtype; the result is in the compute dtype.

    'f32' rounds to IEEE single (nearest even; nothing to do in float32);
    'bf16' keeps 7 explicit mantissa bits, rounding the compute-precision value
    directly to nearest, ties to even (normal range only, which is all this
    method produces); 'fp8' stores fp8_e4m3(x / scale) and the value it stands
    for is that times ``scale`` (one scale per cache tensor); 'f64' keeps the
    value.
    """
    x = _a(x)
    if storage == "fp8":
        s = x.dtype.type(scale)
        return fp8_e4m3(x / s) * s
    if storage == "f32":
        return x.astype(np.float32).astype(x.dtype)
    if storage == "bf16":
        if x.dtype == np.float32:
            u = np.ascontiguousarray(x).view(np.uint32).astype(np.uint64)
            lsb = (u >> np.uint64(16)) & np.uint64(1)
            r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
            return r.view(np.float32).reshape(x.shape)
        u = np.ascontiguousarray(x).view(np.uint64)
        drop = np.uint64(52 - 7)
        lsb = (u >> drop) & np.uint64(1)
        half = np.uint64((1 << 44) - 1)
        r = (u + half + lsb) & ~np.uint64((1 << 45) - 1)
        return r.view(F64).reshape(x.shape)
    if storage == "f64":
        return x
    raise ValueError(storage)


# ----------------------------------------------------------------------------
# model pieces
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm: x / sqrt(mean(x^2) + eps) * g, per row."""
    x = _a(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * _a(g)


def rope_cos_sin(pos: np.ndarray, head_dim: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin of pos * theta_i, theta_i = base^(-2i/d_h), i < d_h/2: the angle
    and its cos/sin evaluated in float64, then rounded to the compute dtype.

    [CB] "位置恢复": R_m is block diagonal with entries cos(m theta_i),
    sin(m theta_i); d/2 rotation pairs.
    """
    i = np.arange(head_dim // 2, dtype=F64)
    inv = np.power(F64(theta), -(2.0 * i) / head_dim)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv[None, :]
    return np.cos(ang).astype(ct()), np.sin(ang).astype(ct())


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Apply R_pos to every head of every row: x [n, H, d_h], pos [n].

    Pair (x_2i, x_2i+1) -> (x_2i c - x_2i+1 s, x_2i s + x_2i+1 c).
    """
    x = _a(x)
    n, H, dh = x.shape
    c, s = rope_cos_sin(pos, dh, theta)
    c = c[:, None, :]
    s = s[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rerope(k: np.ndarray, delta: int, theta: float, storage: str, scale: float = 1.0) -> np.ndarray:
    """Re-RoPE cached keys from their stored offset to the new one.

    [CB] "位置恢复": k' = R_{n-p} k_p = R_n k.  ``k`` is [..., n, H, d_h]
    (leading layer axis allowed); every token moves by the same ``delta`` =
    n - p.  The result is rounded to the storage dtype.  V is never rotated.
    """
    k = _a(k)
    shp = k.shape
    flat = k.reshape(-1, shp[-2], shp[-1])
    out = rope(flat, np.full(flat.shape[0], delta, dtype=F64), theta)
    return store_round(out.reshape(shp), storage, scale)


def _host_threads() -> int:
    """Worker threads for the per-head attention loop: the cores this process may
    use, at most 16 (the host share of one GPU on the machines this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:       # pragma: no cover - non-Linux hosts
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def causal_attention(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                     k_pos: np.ndarray, row_block: int = 1024) -> np.ndarray:
    """softmax(q k^T / sqrt(d_h)) v over keys with k_pos <= q_pos, per head.

    q [n, Hq, d_h]; k, v [P, Hkv, d_h]; GQA: q head h reads kv head
    floor(h * Hkv / Hq).  Softmax subtracts the row maximum.  Rows are taken in
    blocks of ``row_block`` (each block sees the keys up to its last row; the
    others are masked), and the (block, head) pairs, which share nothing, run on
    several threads when the problem is large; each pair's arithmetic is the
    same either way.
    """
    q = _a(q)
    k = _a(k)
    v = _a(v)
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    scale = q.dtype.type(1.0 / np.sqrt(dh))
    out = np.zeros((n, Hq, dh), dtype=q.dtype)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    blocks = []
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        qp = q_pos[r0:r1]
        # keys any row of this block may see
        kmask = k_pos <= qp.max()
        allowed = k_pos[kmask][None, :] <= qp[:, None]
        blocks.append((r0, r1, kmask, allowed))

    def one(task):
        (r0, r1, kmask, allowed), h = task
        g = (h * Hkv) // Hq
        kk = k[kmask, g, :]
        vv = v[kmask, g, :]
        s = (_op(q[r0:r1, h, :]) @ kk.T) * scale
        s = np.where(allowed, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        p = _op(np.exp(s - m))
        out[r0:r1, h, :] = (p @ vv) / np.sum(p, axis=1, keepdims=True)

    tasks = [(b, h) for b in blocks for h in range(Hq)]
    work = sum(int(b[3].size) for b in blocks) * Hq
    nt = _host_threads()
    if nt == 1 or work < (1 << 26):
        for t in tasks:
            one(t)
        return out
    # one BLAS thread per worker: the workers already fill the cores
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(one, tasks))
    return out


def swiglu_mlp(a: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """W_down (SiLU(a W_gate) * (a W_up)), SiLU(z) = z / (1 + e^-z)."""
    a = _op(a)
    g = a @ _a(w_gate).T
    u = a @ _a(w_up).T
    with np.errstate(over="ignore"):         # exp(-g) = inf for g << 0 gives SiLU = -0, its limit
        h = g / (a.dtype.type(1.0) + np.exp(-g)) * u
    return _op(h) @ _a(w_down).T


# ----------------------------------------------------------------------------
# model container
# ----------------------------------------------------------------------------

@dataclass
class OracleModel:
    """Shape + weights.  ``layer(l)`` returns the layer's weight dict
    (``wq, wk, wv, wo, w_gate, w_up, w_down`` as [out][in], ``attn_norm``,
    ``mlp_norm``); ``glob`` holds ``embed`` [V][d], ``lm_head`` [V][d],
    ``final_norm`` [d]."""
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    rope_theta: float
    rms_eps: float
    storage: str
    layer: Callable[[int], Dict[str, np.ndarray]]
    glob: Dict[str, np.ndarray]
    kv_storage: Optional[str] = None   # the KV cache's storage ('fp8' or the model dtype when None)
    k_scale: float = 1.0               # fp8 cache: stored K = k_scale * grid value
    v_scale: float = 1.0

    def store_k(self, x: np.ndarray) -> np.ndarray:
        return store_round(x, self.kv_storage or self.storage, self.k_scale)

    def store_v(self, x: np.ndarray) -> np.ndarray:
        return store_round(x, self.kv_storage or self.storage, self.v_scale)

    @classmethod
    def from_shape(cls, shape, weights_or_fn, glob=None) -> "OracleModel":
        if callable(weights_or_fn):
            fn, g = weights_or_fn, glob
        else:
            layers = weights_or_fn["layers"]
            fn = lambda l: layers[l]  # noqa: E731
            g = {k: weights_or_fn[k] for k in ("embed", "lm_head", "final_norm")}
        return cls(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads,
                   shape.head_dim, shape.d_ff, shape.vocab, shape.rope_theta,
                   shape.rms_eps, shape.dtype, fn, g)

    def heads(self, y: np.ndarray, H: int) -> np.ndarray:
        return y.reshape(y.shape[0], H, self.head_dim)


def _proj(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    return _op(a) @ _a(w).T


def _logits(m: OracleModel, x_last: np.ndarray) -> np.ndarray:
    # a matrix-vector product: the normalised row stays float32 in either operand mode
    a = rms_norm(x_last[None, :], m.glob["final_norm"], m.rms_eps)
    return (a @ _a(m.glob["lm_head"]).T)[0]


# ----------------------------------------------------------------------------
# deviation and selection
# ----------------------------------------------------------------------------

def kv_deviation(k_fresh, v_fresh, k_cached, v_cached) -> np.ndarray:
    """Per-token squared L2 distance between fresh and cached K and V.

    [CB] "核心思想", eq. Δkv: Δ[j] = || KV_i[j] - KV_i^full[j] ||, taken over
    the concatenation of K and V across every KV head; the square ranks the
    same as the norm.  Inputs [n, H_kv, d_h]; output [n] in the compute dtype.
    """
    dk = _a(k_fresh) - _a(k_cached)
    dv = _a(v_fresh) - _a(v_cached)
    ax = tuple(range(1, dk.ndim))
    return np.sum(dk * dk, axis=ax) + np.sum(dv * dv, axis=ax)


def select_hkvd(dev: np.ndarray, cand_pos: np.ndarray, k: int) -> np.ndarray:
    """The k candidates with the largest deviation (HKVD tokens).

    [CB] "选 token": rank the candidates by deviation and keep the top ones.
    Ties go to the smaller position.  Returns the positions ascending.
    """
    dev = np.asarray(dev)
    cand_pos = np.asarray(cand_pos, dtype=np.int64)
    if not (0 <= k <= len(cand_pos)):
        raise ValueError("k out of range")
    order = np.lexsort((cand_pos, -dev))      # primary: dev desc; secondary: pos asc
    return np.sort(cand_pos[order[:k]])


# ----------------------------------------------------------------------------
# one decoder layer on a set of rows
# ----------------------------------------------------------------------------

def _attn_mlp(m: OracleModel, w, x_rows, a_rows, rows_pos, Kl, Vl, k_pos):
    """Attention of the given rows over the layer cache, then O, residual, MLP."""
    q = rope(m.heads(_proj(a_rows, w["wq"]), m.n_q_heads), rows_pos, m.rope_theta)
    o = causal_attention(q, rows_pos, Kl, Vl, k_pos)
    x = x_rows + _proj(o.reshape(o.shape[0], -1), w["wo"])
    x = x + swiglu_mlp(rms_norm(x, w["mlp_norm"], m.rms_eps), w["w_gate"], w["w_up"], w["w_down"])
    return x


def full_prefill(m: OracleModel, tokens: np.ndarray, start: int = 0) -> Dict[str, np.ndarray]:
    """One-shot prefill of ``tokens`` at positions start, start+1, ...

    Returns K, V [L][n][H_kv][d_h] (storage dtype values), the final hidden
    rows and the logits of the last row.  This is the full-KV-recompute
    reference ([CB] "背景") and, with start = p, the chunk prefill that
    produces a cached chunk.
    """
    tokens = np.asarray(tokens)
    n = len(tokens)
    pos = np.arange(start, start + n)
    x = _a(m.glob["embed"][np.asarray(tokens)])
    K = np.zeros((m.n_layers, n, m.n_kv_heads, m.head_dim), dtype=ct())
    V = np.zeros_like(K)
    for l in range(m.n_layers):
        w = m.layer(l)
        a = rms_norm(x, w["attn_norm"], m.rms_eps)
        K[l] = m.store_k(rope(m.heads(_proj(a, w["wk"]), m.n_kv_heads), pos, m.rope_theta))
        V[l] = m.store_v(m.heads(_proj(a, w["wv"]), m.n_kv_heads))
        x = _attn_mlp(m, w, x, a, pos, K[l], V[l], pos)
    return {"K": K, "V": V, "x": x, "logits": _logits(m, x[-1])}


def decode_step(m: OracleModel, Kb: np.ndarray, Vb: np.ndarray, token: int, pos: int) -> np.ndarray:
    """One decoding step on a filled cache ([CB] 问题: the new token's query is
    dotted with the stored K and weights the stored V, no earlier hidden state
    is recomputed; Fig. 11: decoding starts from the fused KV).

    ``Kb``/``Vb`` [L][>= pos+1][H_kv][d_h] hold positions [0, pos); the token's
    own K/V (storage dtype) are written at ``pos`` in place, then it attends to
    [0, pos].  Returns the token's logits.
    """
    x = _a(m.glob["embed"][[int(token)]])
    p = np.array([int(pos)])
    keys = np.arange(int(pos) + 1)
    for l in range(m.n_layers):
        w = m.layer(l)
        a = rms_norm(x, w["attn_norm"], m.rms_eps)
        Kb[l, pos] = m.store_k(rope(m.heads(_proj(a, w["wk"]), m.n_kv_heads), p, m.rope_theta))[0]
        Vb[l, pos] = m.store_v(m.heads(_proj(a, w["wv"]), m.n_kv_heads))[0]
        x = _attn_mlp(m, w, x, a, p, Kb[l, :pos + 1], Vb[l, :pos + 1], keys)
    return _logits(m, x[0])


def chunk_prefill(m: OracleModel, tokens: np.ndarray, start: int) -> Tuple[np.ndarray, np.ndarray]:
    """Cached KV of one chunk prefilled alone at offset ``start``
    ([CB] "背景": each retrieved chunk is prefilled separately)."""
    r = full_prefill(m, tokens, start)
    return r["K"], r["V"]


def assemble_blended(m: OracleModel, chunks: Sequence[Tuple], n_query: int) -> Tuple[np.ndarray, np.ndarray]:
    """Concatenate cached chunks at their new offsets, re-RoPE'ing K.

    ``chunks``: sequence of (tokens, K_c, V_c, old_start, new_start).  Returns
    K_b, V_b [L][N+Q][H_kv][d_h]; query positions are left zero.
    [CB] "位置恢复"; [BI] section 6.2 (old_st = source, cur_st = target).
    """
    N = sum(len(c[0]) for c in chunks)
    T = N + n_query
    Kb = np.zeros((m.n_layers, T, m.n_kv_heads, m.head_dim), dtype=ct())
    Vb = np.zeros_like(Kb)
    for tokens, Kc, Vc, old, new in chunks:
        ln = len(tokens)
        Kb[:, new:new + ln] = rerope(Kc, new - old, m.rope_theta, m.kv_storage or m.storage, m.k_scale)
        Vb[:, new:new + ln] = m.store_v(Vc)      # a value already on the cache's grid stays as it is
    return Kb, Vb


def _context_tokens(chunks) -> np.ndarray:
    order = sorted(range(len(chunks)), key=lambda c: chunks[c][4])
    return np.concatenate([np.asarray(chunks[c][0]) for c in order])


def _check_tiling(chunks):
    order = sorted(range(len(chunks)), key=lambda c: chunks[c][4])
    cur = 0
    for c in order:
        if chunks[c][4] != cur or chunks[c][3] < 0:
            raise ValueError("chunks must tile [0, N) with known stored offsets")
        cur += len(chunks[c][0])
    return cur


def blend_layer(m: OracleModel, l: int, Kl: np.ndarray, Vl: np.ndarray, x_rows: np.ndarray,
                cand_pos: np.ndarray, n_query: int, check: bool, k_keep: int,
                force: Optional[np.ndarray] = None, out_rows: Optional[np.ndarray] = None):
    """One selective-recompute layer l >= 1 ([CB] Fig. 5 and "选 token").

    ``x_rows`` holds the hidden rows of the candidates (positions
    ``cand_pos``, ascending) followed by the ``n_query`` suffix rows at
    positions N .. N+Q-1 with N = Kl.shape[0] - n_query.  ``Kl``/``Vl`` are the
    layer's blended cache [T][H_kv][d_h] and are updated in place.

    Steps: fresh K/V for every row; if ``check``, deviation over the candidates
    and top-k_keep (or ``force``); scatter the fresh K/V of the kept rows and
    the suffix; attention of those rows over the whole cache; O, residual,
    MLP.  Returns (x_out rows for kept + suffix, kept positions, deviation or
    None).

    ``out_rows`` (indices into the kept + suffix rows) limits the attention,
    O and MLP to those rows; x_out then holds only them, in that order.  Every
    K/V row is still written first, so each returned row is exactly the one the
    full call would give: a row's output depends on its own hidden state and on
    the updated cache alone.
    """
    w = m.layer(l)
    T = Kl.shape[0]
    N = T - n_query
    nc = len(cand_pos)
    suffix = np.arange(N, T)
    rows_pos = np.concatenate([np.asarray(cand_pos, dtype=np.int64), suffix])
    a = rms_norm(x_rows, w["attn_norm"], m.rms_eps)
    kf = rope(m.heads(_proj(a, w["wk"]), m.n_kv_heads), rows_pos, m.rope_theta)
    vf = m.heads(_proj(a, w["wv"]), m.n_kv_heads)
    dev = None
    if check:
        dev = kv_deviation(kf[:nc], vf[:nc], Kl[cand_pos], Vl[cand_pos])
        keep = np.sort(np.asarray(force, dtype=np.int64)) if force is not None \
            else select_hkvd(dev, cand_pos, k_keep)
        if len(keep) != k_keep:
            raise ValueError("forced set has the wrong size")
    else:
        if k_keep != nc:
            raise ValueError("an unchecked layer keeps every candidate")
        keep = np.asarray(cand_pos, dtype=np.int64)
    slot = np.searchsorted(cand_pos, keep)
    if np.any(slot >= nc) or np.any(np.asarray(cand_pos)[np.minimum(slot, nc - 1)] != keep):
        raise ValueError("kept positions must be candidates")
    sel = np.concatenate([slot, nc + np.arange(n_query)])
    wpos = rows_pos[sel]
    # fill: fresh K/V of the kept rows and the suffix replace the cache
    Kl[wpos] = m.store_k(kf[sel])
    Vl[wpos] = m.store_v(vf[sel])
    if out_rows is not None:
        sel = sel[np.asarray(out_rows, dtype=np.int64)]
    x_out = _attn_mlp(m, w, x_rows[sel], a[sel], rows_pos[sel], Kl, Vl, np.arange(T))
    return x_out, keep, dev


def blend_prefill(m: OracleModel, chunks: Sequence[Tuple], query_tokens: np.ndarray,
                  k_sched: Sequence[int], check: Sequence[int],
                  force_sets: Optional[Dict[int, np.ndarray]] = None,
                  layers_limit: Optional[int] = None) -> Dict[str, object]:
    """CacheBlend blended prefill, gathered-rows formulation.

    ``chunks``: (tokens, K_c, V_c, old_start, new_start) per chunk; their new
    offsets tile [0, N).  ``k_sched[l]`` is |S_l| (k_sched[0] must be N),
    ``check[l]`` whether layer l re-ranks.  Layer 0 runs in full over every row
    with the context K/V taken from the re-RoPE'd cache; each later layer runs
    ``blend_layer`` on S_{l-1} plus the suffix, so S_l is a subset of S_{l-1}
    ([CB] "核心思想": sets only shrink).  Returns K, V (blended cache),
    logits of the last position, sets {l: S_l} and devs {l: (cand, Δ)}.
    ``layers_limit`` stops after that many layers (timing samples only).
    """
    N = _check_tiling(chunks)
    Q = len(query_tokens)
    T = N + Q
    L = m.n_layers
    if k_sched[0] != N:
        raise ValueError("layer 0 runs in full")
    Kb, Vb = assemble_blended(m, chunks, Q)
    tokens = np.concatenate([_context_tokens(chunks), np.asarray(query_tokens)])
    pos = np.arange(T)
    suffix = np.arange(N, T)
    # layer 0: every row; context K/V are the re-RoPE'd cache
    w = m.layer(0)
    x = _a(m.glob["embed"][np.asarray(tokens)])
    a = rms_norm(x, w["attn_norm"], m.rms_eps)
    Kb[0, suffix] = m.store_k(rope(m.heads(_proj(a[N:], w["wk"]), m.n_kv_heads), suffix, m.rope_theta))
    Vb[0, suffix] = m.store_v(m.heads(_proj(a[N:], w["wv"]), m.n_kv_heads))
    x = _attn_mlp(m, w, x, a, pos, Kb[0], Vb[0], pos)
    S = np.arange(N)
    sets = {0: S}
    devs = {}
    nl = L if layers_limit is None else min(L, layers_limit)
    for l in range(1, nl):
        if k_sched[l] > len(S):
            raise ValueError("sets may only shrink")
        force = None if force_sets is None else force_sets.get(l)
        x, S_new, dev = blend_layer(m, l, Kb[l], Vb[l], x, S, Q, bool(check[l]), int(k_sched[l]), force)
        if dev is not None:
            devs[l] = (S, dev)
        S = S_new
        sets[l] = S
    logits = _logits(m, x[-1])
    return {"K": Kb, "V": Vb, "logits": logits, "sets": sets, "devs": devs, "x_last": x[-1]}


def blend_prefill_masked(m: OracleModel, chunks: Sequence[Tuple], query_tokens: np.ndarray,
                         k_sched: Sequence[int], check: Sequence[int]) -> Dict[str, object]:
    """Masked-dense twin of ``blend_prefill``: every row is computed at every
    layer and the cache / hidden rows keep the fresh or old value by mask
    ([CB] Fig. 5 drawn literally: mask the input, fill the unselected positions
    from the cache, attend with every selected query).  It must agree with the
    gathered-rows formulation."""
    N = _check_tiling(chunks)
    Q = len(query_tokens)
    T = N + Q
    Kb, Vb = assemble_blended(m, chunks, Q)
    tokens = np.concatenate([_context_tokens(chunks), np.asarray(query_tokens)])
    pos = np.arange(T)
    x = _a(m.glob["embed"][np.asarray(tokens)])
    cand = np.ones(T, dtype=bool)
    cand[N:] = False
    is_suffix = ~cand.copy()
    is_suffix[:N] = False
    sets, devs = {}, {}
    for l in range(m.n_layers):
        w = m.layer(l)
        a = rms_norm(x, w["attn_norm"], m.rms_eps)
        kf = rope(m.heads(_proj(a, w["wk"]), m.n_kv_heads), pos, m.rope_theta)
        vf = m.heads(_proj(a, w["wv"]), m.n_kv_heads)
        if l == 0:
            keep = cand.copy()
            write = is_suffix.copy()          # context K/V of layer 0 stay cached
        else:
            if check[l]:
                d = kv_deviation(kf, vf, Kb[l], Vb[l])
                devs[l] = (np.nonzero(cand)[0], d[cand])
                # rank candidates: deviation desc, position asc
                idx = np.nonzero(cand)[0]
                ranked = sorted(idx.tolist(), key=lambda j: (-d[j], j))
                keep = np.zeros(T, dtype=bool)
                keep[ranked[:k_sched[l]]] = True
            else:
                keep = cand.copy()
            write = keep | is_suffix
        Kb[l] = np.where(write[:, None, None], m.store_k(kf), Kb[l])
        Vb[l] = np.where(write[:, None, None], m.store_v(vf), Vb[l])
        active = keep | is_suffix if l > 0 else np.ones(T, dtype=bool)
        x_new = _attn_mlp(m, w, x, a, pos, Kb[l], Vb[l], pos)
        x = np.where(active[:, None], x_new, x)
        cand = keep
        sets[l] = np.nonzero(keep)[0]
    return {"K": Kb, "V": Vb, "logits": _logits(m, x[-1]), "sets": sets, "devs": devs}


def full_reuse_prefill(m: OracleModel, Kb: np.ndarray, Vb: np.ndarray, query_tokens: np.ndarray) -> Dict[str, object]:
    """Full KV reuse ([CB] "背景", PromptCache-style): the context cache is used
    as-is at every layer and only the query suffix is computed.  ``Kb``/``Vb``
    [L][N+Q][H_kv][d_h] hold the context; suffix rows are written here."""
    Kb = Kb.copy()
    Vb = Vb.copy()
    L, T = Kb.shape[0], Kb.shape[1]
    Q = len(query_tokens)
    N = T - Q
    suffix = np.arange(N, T)
    x = _a(m.glob["embed"][np.asarray(query_tokens)])
    for l in range(L):
        w = m.layer(l)
        a = rms_norm(x, w["attn_norm"], m.rms_eps)
        Kb[l, suffix] = m.store_k(rope(m.heads(_proj(a, w["wk"]), m.n_kv_heads), suffix, m.rope_theta))
        Vb[l, suffix] = m.store_v(m.heads(_proj(a, w["wv"]), m.n_kv_heads))
        x = _attn_mlp(m, w, x, a, suffix, Kb[l], Vb[l], np.arange(T))
    return {"K": Kb, "V": Vb, "logits": _logits(m, x[-1])}


# ----------------------------------------------------------------------------
# work accounting
# ----------------------------------------------------------------------------

def flop_count(shape, n_ctx: int, n_query: int, k_sched: Sequence[int], check: Sequence[int]) -> Dict[str, float]:
    """Multiply-add FLOPs (2 per MAC) of the blend and of a full prefill of
    N+Q tokens.  Attention counts only the causally visible pairs.  Layer 0
    skips the context K/V projection (it is taken from the cache)."""
    d, Hq, Hkv, dh, F = shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff
    qw, kvw = Hq * dh, Hkv * dh
    T = n_ctx + n_query

    def attn(pos_list_sum_plus_one):  # sum over rows of (pos+1) visible keys
        return 4.0 * qw * pos_list_sum_plus_one

    def per_row_rest():   # Q, O, MLP per row
        return 2.0 * (d * qw + qw * d + 3 * d * F)

    full = 0.0
    vis_all = T * (T + 1) / 2.0
    full_layer = T * (per_row_rest() + 2.0 * d * 2 * kvw) + attn(vis_all)
    full = full_layer * shape.n_layers
    blend = 0.0
    # layer 0: Q/O/MLP on every row, K/V only for the suffix
    blend += T * per_row_rest() + n_query * 2.0 * d * 2 * kvw + attn(vis_all)
    cand = n_ctx
    for l in range(1, shape.n_layers):
        rows_kv = cand + n_query
        keep = k_sched[l]
        rows = keep + n_query
        # mean visible keys: kept context rows average (N+1)/2, suffix rows N + i + 1
        vis = keep * (n_ctx + 1) / 2.0 + sum(n_ctx + i + 1 for i in range(n_query))
        blend += rows_kv * 2.0 * d * 2 * kvw + rows * per_row_rest() + attn(vis)
        cand = keep
    return {"blend": blend, "full": full, "ratio": blend / full}
