// C ABI of libcacheblend: argument validation, workspace carving and the
// per-layer orchestration of the blended prefill.
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn):
//   * section "位置恢复": cached keys are rotated from their stored offset to
//     the new one (k' = R_{n-p} k_p); values are copied;
//   * section "核心思想" / "选 token": the first layer runs in full; each later
//     layer recomputes only the tokens kept by the previous layer, measures
//     the per-token KV deviation and keeps a top-k subset (sets only shrink);
//   * Fig. 5: the fresh K/V of the kept tokens replace the cached ones, the
//     kept queries attend to every token, only kept rows flow to the next layer;
//   * section "位置恢复、KV 存储与加载流水线": the per-layer call mirrors
//     prefill_layer(input_dict{check_flag, HKVD_indices}, KVCache).
// Everything is enqueued on the caller's stream; nothing synchronises, nothing
// allocates.  Validation runs before the first enqueue.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "cb_internal.h"

using namespace cb;

namespace {

thread_local std::string g_last_error;

cb_status fail(cb_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cb_status ok() {
  g_last_error.clear();
  return CB_OK;
}

cb_status dev_fail(hipError_t e, const char* where) {
  return fail(CB_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

#define CB_TRY(expr, where)                        \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return dev_fail(_e, where); \
  } while (0)


// Optional launch trace (cb_trace): events recorded around launches of the selected kinds.
struct Tracer {
  cb_trace* t = nullptr;
  hipStream_t s = nullptr;
  bool on(int kind) const {
    return t && t->events && ((t->kind_mask >> kind) & 1u) && t->used + 2 <= t->capacity;
  }
};

#define CB_LAUNCH(tr, kind, expr, where)                                                          \
  do {                                                                                          \
    const bool _on = (tr) != nullptr && (tr)->on(kind);                                         \
    if (_on) CB_TRY(hipEventRecord(static_cast<hipEvent_t>((tr)->t->events[(tr)->t->used]), (tr)->s), "trace"); \
    CB_TRY(expr, where);                                                                        \
    if (_on) {                                                                                  \
      CB_TRY(hipEventRecord(static_cast<hipEvent_t>((tr)->t->events[(tr)->t->used + 1]), (tr)->s), "trace"); \
      if ((tr)->t->kinds) (tr)->t->kinds[(tr)->t->used / 2] = (kind);                          \
      (tr)->t->used += 2;                                                                       \
    }                                                                                           \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize(cb_dtype dt) { return dt == CB_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
cb_status check_cfg(const cb_model_cfg* c) {
  if (!c) return fail(CB_ERR_INVALID, "cfg is NULL");
  if (c->dtype != CB_F32 && c->dtype != CB_BF16) return fail(CB_ERR_INVALID, "unknown dtype %d", (int)c->dtype);
  if (c->n_layers < 2) return fail(CB_ERR_INVALID, "n_layers must be >= 2 (got %d)", c->n_layers);
  if (c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->d_ff <= 0 ||
      c->vocab <= 0)
    return fail(CB_ERR_INVALID, "non-positive model dimension");
  if (c->head_dim % 2) return fail(CB_ERR_INVALID, "head_dim must be even (got %d)", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads)
    return fail(CB_ERR_INVALID, "n_q_heads %d not a multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
  if (!(c->rope_theta > 0.0)) return fail(CB_ERR_INVALID, "rope_theta must be > 0");
  if (!(c->rms_eps >= 0.0f)) return fail(CB_ERR_INVALID, "rms_eps must be >= 0");
  const int qw = c->n_q_heads * c->head_dim;
  const int kvw = c->n_kv_heads * c->head_dim;
  if (c->d_model % 64 || c->d_ff % 64 || qw % 64)
    return fail(CB_ERR_UNSUPPORTED, "d_model, d_ff and n_q_heads*head_dim must be multiples of 64");
  if (kvw % 8) return fail(CB_ERR_UNSUPPORTED, "n_kv_heads*head_dim must be a multiple of 8");
  if (c->d_model > 16384) return fail(CB_ERR_UNSUPPORTED, "d_model above 16384");
  if (!attention_supported(c->dtype, c->n_q_heads, c->n_kv_heads, c->head_dim))
    return fail(CB_ERR_UNSUPPORTED, "attention kernel not built for head_dim %d, %d q / %d kv heads", c->head_dim,
                c->n_q_heads, c->n_kv_heads);
  return CB_OK;
}

cb_status check_paged(const cb_model_cfg* c, const cb_paged_kv* p, int64_t n_tokens, const char* what) {
  if (!p) return fail(CB_ERR_INVALID, "%s is NULL", what);
  if (!p->k || !p->v || !p->block_table) return fail(CB_ERR_INVALID, "%s: NULL pool or block table", what);
  if (!aligned16(p->k) || !aligned16(p->v)) return fail(CB_ERR_INVALID, "%s: pools must be 16-byte aligned", what);
  if (p->block_size < 1) return fail(CB_ERR_INVALID, "%s: block_size must be >= 1", what);
  if (p->n_logical < 0) return fail(CB_ERR_INVALID, "%s: n_logical < 0", what);
  if (static_cast<int64_t>(p->n_logical) * p->block_size < n_tokens)
    return fail(CB_ERR_INVALID, "%s: block table covers %lld tokens, %lld needed", what,
                (long long)p->n_logical * p->block_size, (long long)n_tokens);
  if (p->kv_format != CB_KV_MODEL && p->kv_format != CB_KV_FP8_E4M3)
    return fail(CB_ERR_INVALID, "%s: unknown kv_format %d", what, p->kv_format);
  const bool fp8 = p->kv_format == CB_KV_FP8_E4M3;
  if (fp8 && c->dtype != CB_BF16) return fail(CB_ERR_UNSUPPORTED, "%s: an 8-bit cache needs a CB_BF16 model", what);
  if (fp8 && !(p->k_scale > 0.f && p->v_scale > 0.f && std::isfinite(p->k_scale) && std::isfinite(p->v_scale)))
    return fail(CB_ERR_INVALID, "%s: 8-bit cache scales must be positive and finite", what);
  if (fp8 && (c->n_kv_heads * c->head_dim) % 16)
    return fail(CB_ERR_UNSUPPORTED, "%s: an 8-bit cache needs n_kv_heads*head_dim a multiple of 16", what);
  const int64_t vec = fp8 ? 16 : 16 / esize(c->dtype);
  if (p->layer_stride < 0 || p->layer_stride % vec)
    return fail(CB_ERR_INVALID, "%s: layer_stride must be a non-negative multiple of %lld elements", what,
                (long long)vec);
  return CB_OK;
}

cb_status check_chunk_sources(const cb_model_cfg* c, const cb_chunk* ch, int n, bool need_tokens) {
  if (n < 0) return fail(CB_ERR_INVALID, "n_chunks < 0");
  if (n > 0 && !ch) return fail(CB_ERR_INVALID, "chunks is NULL");
  for (int i = 0; i < n; ++i) {
    const cb_chunk& x = ch[i];
    if (x.kv_format != CB_KV_MODEL && x.kv_format != CB_KV_FP8_E4M3)
      return fail(CB_ERR_INVALID, "chunk %d: unknown kv_format %d", i, x.kv_format);
    const bool fp8 = x.kv_format == CB_KV_FP8_E4M3;
    if (fp8 && !(x.k_scale > 0.f && x.v_scale > 0.f && std::isfinite(x.k_scale) && std::isfinite(x.v_scale)))
      return fail(CB_ERR_INVALID, "chunk %d: 8-bit scales must be positive and finite", i);
    const int64_t vec = fp8 ? 16 : 16 / esize(c->dtype);
    if (x.len < 0) return fail(CB_ERR_INVALID, "chunk %d: len < 0", i);
    if (x.old_start < 0)
      return fail(CB_ERR_INVALID, "chunk %d: unknown stored offset %d (a wrong position gives wrong KV)", i,
                  x.old_start);
    if (x.new_start < 0) return fail(CB_ERR_INVALID, "chunk %d: new_start < 0", i);
    if (x.len == 0) continue;
    if (!x.k || !x.v) return fail(CB_ERR_INVALID, "chunk %d: NULL K/V", i);
    if (!aligned16(x.k) || !aligned16(x.v)) return fail(CB_ERR_INVALID, "chunk %d: K/V not 16-byte aligned", i);
    if (need_tokens && !x.tokens) return fail(CB_ERR_INVALID, "chunk %d: NULL tokens", i);
    if (x.block_ids && x.block_size < 1) return fail(CB_ERR_INVALID, "chunk %d: paged source needs block_size >= 1", i);
    if (x.layer_stride < 0 || x.layer_stride % vec)
      return fail(CB_ERR_INVALID, "chunk %d: layer_stride must be a non-negative multiple of %lld", i, (long long)vec);
  }
  return CB_OK;
}

// every chunk must be stored in the destination's element format
cb_status check_chunk_formats(const cb_chunk* ch, int n, const cb_paged_kv* dst) {
  for (int i = 0; i < n; ++i)
    if (ch[i].len > 0 && ch[i].kv_format != dst->kv_format)
      return fail(CB_ERR_UNSUPPORTED, "chunk %d: kv_format %d differs from the destination's %d", i, ch[i].kv_format,
                  dst->kv_format);
  return CB_OK;
}

// new_start values must tile [0, N) exactly; returns N
cb_status check_tiling(const cb_chunk* ch, int n, int64_t* n_ctx) {
  std::vector<std::pair<int64_t, int64_t>> iv;
  iv.reserve(n);
  for (int i = 0; i < n; ++i)
    if (ch[i].len > 0) iv.emplace_back(ch[i].new_start, ch[i].len);
  std::sort(iv.begin(), iv.end());
  int64_t cur = 0;
  for (auto& e : iv) {
    if (e.first < cur) return fail(CB_ERR_INVALID, "chunks overlap at position %lld", (long long)e.first);
    if (e.first > cur) return fail(CB_ERR_INVALID, "gap in the context at position %lld", (long long)cur);
    cur += e.second;
  }
  if (cur > (int64_t)1 << 30) return fail(CB_ERR_INVALID, "context too long");
  *n_ctx = cur;
  return CB_OK;
}

cb_status check_model(const cb_model* m) {
  if (!m) return fail(CB_ERR_INVALID, "model is NULL");
  cb_status st = check_cfg(&m->cfg);
  if (st != CB_OK) return st;
  if (!m->embed || !m->final_norm || !m->lm_head || !m->layers)
    return fail(CB_ERR_INVALID, "model: NULL embed / final_norm / lm_head / layers");
  if (!aligned16(m->embed) || !aligned16(m->final_norm) || !aligned16(m->lm_head))
    return fail(CB_ERR_INVALID, "model: global tensors must be 16-byte aligned");
  if (m->weights_packed != (m->cfg.dtype == CB_BF16 ? 1 : 0))
    return fail(CB_ERR_INVALID, "model: weights_packed must be %d for this dtype (bf16 layer matrices are read packed)",
                m->cfg.dtype == CB_BF16 ? 1 : 0);
  for (int l = 0; l < m->cfg.n_layers; ++l) {
    const cb_layer_w& w = m->layers[l];
    const void* ps[6] = {w.w_qkv, w.w_o, w.w_gate_up, w.w_down, w.attn_norm, w.mlp_norm};
    for (const void* p : ps) {
      if (!p) return fail(CB_ERR_INVALID, "layer %d: NULL weight", l);
      if (!aligned16(p)) return fail(CB_ERR_INVALID, "layer %d: weight not 16-byte aligned", l);
    }
  }
  return CB_OK;
}

// ---------------------------------------------------------------------------
// workspace
// ---------------------------------------------------------------------------
struct Ws {
  float2* pos_tab;
  float2* dtab;
  int32_t* tokens;
  float* x0;
  float* x1;
  void* act;
  void* h;
  void* q;
  void* o;
  float* kvf;
  float* dev;
  int32_t* posA;
  int32_t* posB;
  int32_t* slot;
  int32_t* gmap;
  int32_t* rowpos0;
  int32_t* rowpos1;
  float* a_last;
  float* attn_o;
  float2* attn_ml;
  float* gemm_part;
};

size_t carve(const cb_model_cfg& c, int64_t N, int64_t Q, int64_t C, void* base, Ws* w) {
  const int64_t T = N + Q;
  const int64_t half = c.head_dim / 2;
  const int64_t es = esize(c.dtype);
  const int64_t qw = (int64_t)c.n_q_heads * c.head_dim;
  const int64_t kvw = (int64_t)c.n_kv_heads * c.head_dim;
  size_t off = 0;
  auto take = [&](int64_t bytes) -> void* {
    off = (off + 255) & ~size_t(255);
    void* p = base ? static_cast<char*>(base) + off : nullptr;
    off += static_cast<size_t>(std::max<int64_t>(bytes, 0));
    return p;
  };
  Ws t;
  t.pos_tab = static_cast<float2*>(take(T * half * 8));
  t.dtab = static_cast<float2*>(take(std::min<int64_t>(std::max<int64_t>(C, 1), kMaxChunksPerLaunch) * half * 8));
  t.tokens = static_cast<int32_t*>(take(T * 4));
  t.x0 = static_cast<float*>(take(T * c.d_model * 4));
  t.x1 = static_cast<float*>(take(T * c.d_model * 4));
  const int64_t TP = pk_rows(T);   // fragment-major activations hold whole 32-row blocks
  t.act = take(TP * c.d_model * es);
  t.h = take(TP * std::max(c.d_ff, c.d_model) * es);
  t.q = take(T * qw * es);
  t.o = take(TP * qw * es);
  t.kvf = static_cast<float*>(take(T * 2 * kvw * 4));
  t.dev = static_cast<float*>(take(N * 4));
  t.posA = static_cast<int32_t*>(take(N * 4));
  t.posB = static_cast<int32_t*>(take(N * 4));
  t.slot = static_cast<int32_t*>(take(N * 4));
  t.gmap = static_cast<int32_t*>(take(T * 4));
  t.rowpos0 = static_cast<int32_t*>(take(T * 4));
  t.rowpos1 = static_cast<int32_t*>(take(T * 4));
  t.a_last = static_cast<float*>(take(c.d_model * 4));
  t.attn_o = static_cast<float*>(take(T > 0 ? attn_partial_floats(c.head_dim) * 4 : 0));
  t.attn_ml = static_cast<float2*>(take(T > 0 ? kAttnPartialRows * 8 : 0));
  t.gemm_part = static_cast<float*>(take(T > 0 ? kGemmPartFloats * 4 : 0));
  if (w) *w = t;
  return (off + 255) & ~size_t(255);
}

PagedRef ref_of(const cb_paged_kv& p) {
  const bool fp8 = p.kv_format == CB_KV_FP8_E4M3;
  return PagedRef{p.k,  p.v,  p.block_table, p.block_size, p.layer_stride, block_shift(p.block_size),
                  fp8,  fp8 ? p.k_scale : 1.f, fp8 ? p.v_scale : 1.f};
}

// Chunk descriptors for one launch batch [first, first + count).
ChunkBatch make_batch(const cb_model_cfg& c, const cb_chunk* ch, int first, int count) {
  ChunkBatch b;
  std::memset(&b, 0, sizeof(b));
  const int64_t width = (int64_t)c.n_kv_heads * c.head_dim;
  int tiles = 0;
  for (int i = 0; i < count; ++i) {
    const cb_chunk& x = ch[first + i];
    ChunkDesc& d = b.d[i];
    d.k = x.k;
    d.v = x.v;
    d.blk = x.block_ids;
    d.tokens = x.tokens;
    d.layer_stride = x.layer_stride ? x.layer_stride : (int64_t)x.len * width;
    d.len = x.len;
    d.new_start = x.new_start;
    d.block_size = x.block_ids ? x.block_size : 1;
    d.delta = x.new_start - x.old_start;
    d.tile_begin = tiles;
    d.fp8 = x.kv_format == CB_KV_FP8_E4M3;
    d.ks = d.fp8 ? x.k_scale : 1.f;
    d.vs = d.fp8 ? x.v_scale : 1.f;
    tiles += c.n_layers * ((x.len + 15) / 16);
  }
  b.n = count;
  b.total_tiles = tiles;
  return b;
}

// table_ready: dtab already holds the deltas of this (single) batch of chunks
cb_status enqueue_rerope(const cb_model_cfg& c, const cb_chunk* ch, int n, const cb_paged_kv& dst, int copy_v,
                         float2* dtab, hipStream_t s, Tracer* tr, bool table_ready = false) {
  const PagedRef d = ref_of(dst);
  const int width = c.n_kv_heads * c.head_dim;
  for (int first = 0; first < n; first += kMaxChunksPerLaunch) {
    const int cnt = std::min(kMaxChunksPerLaunch, n - first);
    ChunkBatch b = make_batch(c, ch, first, cnt);
    if (!table_ready || n > kMaxChunksPerLaunch)
      CB_LAUNCH(tr, CB_KIND_OTHER, launch_rope_delta_table(dtab, b, c.head_dim, c.rope_theta, s), "rope delta table");
    CB_LAUNCH(tr, CB_KIND_REROPE, launch_rerope(c.dtype, b, d, dtab, c.n_layers, width, c.head_dim, copy_v, s), "rerope");
  }
  return CB_OK;
}

// One selective-recompute layer (l >= 1).
//   x_in rows: candidates (rowpos_in[0..nc)) then suffix; x_mid receives the
//   attention-block output of the kept rows, x_out the layer output (may equal x_mid).
struct LayerIo {
  const float* x_in;
  float* x_mid;
  float* x_out;
  const int32_t* cand_pos;
  const int32_t* rowpos_in;
  int32_t* rowpos_out;
  int32_t* pos_out;
  float* dev_slot;    // nullable [nc]
  float* dev_by_pos;  // nullable [N]
  int32_t* hkvd_row;  // nullable [k]
  bool act_ready;     // w.act already holds RMSNorm(x_in) with this layer's attn_norm
  const float* next_norm;  // nullable: attn_norm of the next layer, fused after the down projection
};

cb_status enqueue_layer(const cb_model& m, int l, const PagedRef& kv, int nc, int N, int Q, int check, int k,
                        const LayerIo& io, const Ws& w, hipStream_t s, Tracer* tr) {
  const cb_model_cfg& c = m.cfg;
  const cb_layer_w& lw = m.layers[l];
  const int d = c.d_model, F = c.d_ff;
  const int qw = c.n_q_heads * c.head_dim;
  const int kvw = c.n_kv_heads * c.head_dim;
  const int es = esize(c.dtype);
  const int rin = nc + Q;
  const int rout = k + Q;

  // fresh K (rotated at the rows' positions) and V for every candidate and suffix row
  if (!io.act_ready)
    CB_LAUNCH(tr, CB_KIND_NORM, launch_rmsnorm(c.dtype, io.x_in, nullptr, d, rin, d, lw.attn_norm, c.rms_eps, w.act, d, 0, s), "rmsnorm");
  // when every candidate is kept, the queries come from the same rows: one GEMM
  // over the whole Q/K/V weight writes Q (bf16) and the fresh K/V (fp32) at once
  const bool fused_qkv = (k == nc) && c.dtype == CB_BF16;
  GemmArgs g{};
  g.A = w.act; g.lda = d; g.a_rows = nullptr;
  g.K = d; g.M = rin;
  g.head_dim = c.head_dim; g.rope_tab = w.pos_tab; g.row_pos = io.rowpos_in;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  // with every candidate kept, a split-K reduction of that GEMM also takes the
  // deviations and writes the fresh K/V rows into the cache
  bool blend_done = false;
  if (fused_qkv) {
    g.B = lw.w_qkv; g.ldb = d;
    g.N = qw + 2 * kvw;
    g.C = w.q; g.ldc = qw; g.q_cols = qw;
    g.C2 = w.kvf; g.ldc2 = 2 * kvw; g.rope2_cols = kvw;
    g.blend = 1;
    g.blend_layer = l;
    g.blend_cache = kv;
    g.blend_nc = nc;
    g.blend_check = check;
    g.blend_dev = io.dev_slot ? io.dev_slot : w.dev;
    g.blend_dev_by_pos = io.dev_by_pos;
    g.blend_gmap = w.gmap;
    g.blend_rowpos = io.rowpos_out;
    g.blend_pos_out = io.pos_out;
    g.blend_slot = check ? w.slot : nullptr;
    g.blend_copy = io.hkvd_row;
    CB_LAUNCH(tr, CB_KIND_GEMM_QKV, launch_gemm(c.dtype, EPI_QKV, g, s, &blend_done), "qkv gemm");
  } else {
    g.B = static_cast<const char*>(lw.w_qkv) + (int64_t)qw * d * es; g.ldb = d;
    g.N = 2 * kvw;
    g.C = w.kvf; g.ldc = 2 * kvw;
    g.rope_cols = kvw;
    CB_LAUNCH(tr, CB_KIND_GEMM_QKV, launch_gemm(c.dtype, EPI_F32_ROPE, g, s), "kv gemm");
  }

  const int32_t* sel_slot = nullptr;
  const int32_t* sel_pos = io.cand_pos;
  int32_t* copy_out = io.pos_out;
  if (blend_done) {
    // the Q/K/V reduction took the deviations, wrote the cache and, the top-k of all
    // candidates being the identity, the row maps
  } else if (check) {
    // deviations of every candidate (many workgroups), then the top-k with the row
    // maps of the kept rows and the suffix (one workgroup)
    float* dev = io.dev_slot ? io.dev_slot : w.dev;
    CB_LAUNCH(tr, CB_KIND_DEVIATION, launch_deviation(c.dtype, w.kvf, w.kvf + kvw, 2 * kvw, io.cand_pos, nc, kv, l, kvw,
                                                      dev, io.dev_by_pos, s), "deviation");
    CB_LAUNCH(tr, CB_KIND_SELECT, launch_select_rows(dev, io.cand_pos, nc, k, io.pos_out, w.slot, N, Q, w.gmap,
                                                     io.rowpos_out, io.hkvd_row, s), "select");
  } else {
    // row maps of the kept rows (+ suffix); an unchecked layer keeps every candidate
    CB_LAUNCH(tr, CB_KIND_OTHER, launch_build_rows(sel_slot, sel_pos, k, nc, N, Q, w.gmap, io.rowpos_out, copy_out,
                                                   io.hkvd_row, s), "build rows");
  }

  // fill: fresh K/V of the kept rows and of the suffix replace the cache
  if (!blend_done)
    CB_LAUNCH(tr, CB_KIND_SCATTER, launch_scatter_kv(c.dtype, w.kvf, 2 * kvw, w.gmap, io.rowpos_out, rout, kv, l, kvw, s), "scatter");

  // queries of the kept rows: when the set shrank, normalise the kept rows into
  // their own (fragment-major) buffer
  const void* aq = w.act;
  if (k != nc) {
    CB_LAUNCH(tr, CB_KIND_NORM, launch_rmsnorm(c.dtype, io.x_in, w.gmap, d, rout, d, lw.attn_norm, c.rms_eps, w.h, d, 0, s),
              "rmsnorm");
    aq = w.h;
  }
  if (!fused_qkv) {
    g = GemmArgs{};
    g.A = aq; g.lda = d; g.a_rows = nullptr;
    g.B = lw.w_qkv; g.ldb = d;
    g.M = rout; g.N = qw; g.K = d;
    g.C = w.q; g.ldc = qw;
    g.rope_cols = qw; g.head_dim = c.head_dim; g.rope_tab = w.pos_tab; g.row_pos = io.rowpos_out;
    g.part = w.gemm_part;
    g.part_floats = kGemmPartFloats;
    CB_LAUNCH(tr, CB_KIND_GEMM_QKV, launch_gemm(c.dtype, EPI_STORE_ROPE, g, s), "q gemm");
  }

  AttnArgs at{};
  at.q = w.q; at.ldq = qw; at.o = w.o; at.ldo = qw; at.rowpos = io.rowpos_out; at.R = rout;
  at.cache = kv; at.layer = l; at.n_q_heads = c.n_q_heads; at.n_kv_heads = c.n_kv_heads; at.head_dim = c.head_dim;
  at.scale = 1.0f / sqrtf(static_cast<float>(c.head_dim));
  at.kv_bound = N + Q;
  at.part_o = w.attn_o;
  at.part_ml = w.attn_ml;
  // the fresh K/V rows are in the cache by now, so their buffer holds the bf16
  // copy of an FP8 layer
  at.widen = w.kvf;
  at.widen_bytes = (int64_t)(N + Q) * 2 * kvw * 4;
  CB_LAUNCH(tr, CB_KIND_ATTENTION, launch_attention(c.dtype, at, s), "attention");

  // O projection + residual (rows gathered from x_in), then the MLP
  g = GemmArgs{};
  g.A = w.o; g.lda = qw; g.B = lw.w_o; g.ldb = qw; g.M = rout; g.N = d; g.K = qw;
  g.C = io.x_mid; g.ldc = d; g.resid = io.x_in; g.resid_rows = w.gmap; g.ld_resid = d;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  g.norm_gain = lw.mlp_norm; g.norm_eps = c.rms_eps; g.norm_out = w.act;   // the MLP's RMSNorm rides on the O projection
  CB_LAUNCH(tr, CB_KIND_GEMM_O, launch_gemm(c.dtype, EPI_RESID, g, s), "o gemm");
  g = GemmArgs{};
  g.A = w.act; g.lda = d; g.B = lw.w_gate_up; g.ldb = d; g.M = rout; g.N = F; g.K = d;
  g.C = w.h; g.ldc = F; g.ff = F;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  CB_LAUNCH(tr, CB_KIND_GEMM_GATE_UP, launch_gemm(c.dtype, EPI_SWIGLU, g, s), "gate/up gemm");
  g = GemmArgs{};
  g.A = w.h; g.lda = F; g.B = lw.w_down; g.ldb = F; g.M = rout; g.N = d; g.K = F;
  g.C = io.x_out; g.ldc = d; g.resid = io.x_mid; g.resid_rows = nullptr; g.ld_resid = d;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  if (io.next_norm) { g.norm_gain = io.next_norm; g.norm_eps = c.rms_eps; g.norm_out = w.act; }
  CB_LAUNCH(tr, CB_KIND_GEMM_DOWN, launch_gemm(c.dtype, EPI_RESID, g, s), "down gemm");
  return CB_OK;
}

// Layer 0 over every row: context K/V stay the re-RoPE'd cache, suffix K/V are computed.
cb_status enqueue_layer0(const cb_model& m, const PagedRef& kv, int N, int Q, float* x, const float* next_norm,
                         const Ws& w, hipStream_t s, Tracer* tr) {
  const cb_model_cfg& c = m.cfg;
  const cb_layer_w& lw = m.layers[0];
  const int d = c.d_model, F = c.d_ff;
  const int qw = c.n_q_heads * c.head_dim;
  const int kvw = c.n_kv_heads * c.head_dim;
  const int es = esize(c.dtype);
  const int T = N + Q;
  CB_LAUNCH(tr, CB_KIND_NORM, launch_rmsnorm(c.dtype, x, nullptr, d, T, d, lw.attn_norm, c.rms_eps, w.act, d, 0, s), "rmsnorm");
  GemmArgs g{};
  g.A = w.act; g.lda = d; g.B = lw.w_qkv; g.ldb = d; g.M = T; g.N = qw; g.K = d;
  g.C = w.q; g.ldc = qw; g.rope_cols = qw; g.head_dim = c.head_dim; g.rope_tab = w.pos_tab; g.row_pos = w.rowpos0;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  CB_LAUNCH(tr, CB_KIND_GEMM_QKV, launch_gemm(c.dtype, EPI_STORE_ROPE, g, s), "q gemm");
  // suffix K/V: rows from the 32-row block holding position N (fragment-major A
  // starts on a block), the extra leading rows are computed and not scattered
  const int N32 = N & ~31;
  const int64_t a_off = (c.dtype == CB_BF16) ? pk_off(N32, 0, d) : (int64_t)N32 * d;
  g = GemmArgs{};
  g.A = static_cast<const char*>(w.act) + a_off * es; g.lda = d;
  g.B = static_cast<const char*>(lw.w_qkv) + (int64_t)qw * d * es; g.ldb = d;
  g.M = T - N32; g.N = 2 * kvw; g.K = d; g.C = w.kvf; g.ldc = 2 * kvw;
  g.rope_cols = kvw; g.head_dim = c.head_dim; g.rope_tab = w.pos_tab; g.row_pos = w.rowpos0 + N32;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  CB_LAUNCH(tr, CB_KIND_GEMM_QKV, launch_gemm(c.dtype, EPI_F32_ROPE, g, s), "suffix kv gemm");
  CB_LAUNCH(tr, CB_KIND_SCATTER, launch_scatter_kv(c.dtype, w.kvf + (int64_t)(N - N32) * 2 * kvw, 2 * kvw, nullptr, w.rowpos0 + N, Q, kv, 0, kvw, s), "suffix scatter");
  AttnArgs at{};
  at.q = w.q; at.ldq = qw; at.o = w.o; at.ldo = qw; at.rowpos = w.rowpos0; at.R = T;
  at.cache = kv; at.layer = 0; at.n_q_heads = c.n_q_heads; at.n_kv_heads = c.n_kv_heads; at.head_dim = c.head_dim;
  at.scale = 1.0f / sqrtf(static_cast<float>(c.head_dim));
  at.kv_bound = N + Q;
  at.part_o = w.attn_o;
  at.part_ml = w.attn_ml;
  // the fresh K/V rows are in the cache by now, so their buffer holds the bf16
  // copy of an FP8 layer
  at.widen = w.kvf;
  at.widen_bytes = (int64_t)(N + Q) * 2 * kvw * 4;
  CB_LAUNCH(tr, CB_KIND_ATTENTION, launch_attention(c.dtype, at, s), "attention");
  g = GemmArgs{};
  g.A = w.o; g.lda = qw; g.B = lw.w_o; g.ldb = qw; g.M = T; g.N = d; g.K = qw;
  g.C = x; g.ldc = d; g.resid = x; g.ld_resid = d;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  g.norm_gain = lw.mlp_norm; g.norm_eps = c.rms_eps; g.norm_out = w.act;
  CB_LAUNCH(tr, CB_KIND_GEMM_O, launch_gemm(c.dtype, EPI_RESID, g, s), "o gemm");
  g = GemmArgs{};
  g.A = w.act; g.lda = d; g.B = lw.w_gate_up; g.ldb = d; g.M = T; g.N = F; g.K = d; g.C = w.h; g.ldc = F; g.ff = F;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  CB_LAUNCH(tr, CB_KIND_GEMM_GATE_UP, launch_gemm(c.dtype, EPI_SWIGLU, g, s), "gate/up gemm");
  g = GemmArgs{};
  g.A = w.h; g.lda = F; g.B = lw.w_down; g.ldb = F; g.M = T; g.N = d; g.K = F;
  g.C = x; g.ldc = d; g.resid = x; g.ld_resid = d;
  g.part = w.gemm_part;
  g.part_floats = kGemmPartFloats;
  if (next_norm) { g.norm_gain = next_norm; g.norm_eps = c.rms_eps; g.norm_out = w.act; }
  CB_LAUNCH(tr, CB_KIND_GEMM_DOWN, launch_gemm(c.dtype, EPI_RESID, g, s), "down gemm");
  return CB_OK;
}

}  // namespace

namespace cb {

cb_status record_failure(cb_status st, const char* msg) { return fail(st, "%s", msg); }

size_t rerope_table_bytes(const cb_model_cfg& c, int n_chunks) {
  return static_cast<size_t>(std::min(std::max(n_chunks, 1), kMaxChunksPerLaunch)) * (c.head_dim / 2) * sizeof(float2);
}

cb_status rerope_check(const cb_model_cfg* cfg, const cb_chunk* chunks, int32_t n_chunks, const cb_paged_kv* dst,
                       uint32_t flags) {
  cb_status st = check_cfg(cfg);
  if (st != CB_OK) return st;
  if ((st = check_chunk_sources(cfg, chunks, n_chunks, false)) != CB_OK) return st;
  int64_t end = 0;
  for (int i = 0; i < n_chunks; ++i) end = std::max<int64_t>(end, (int64_t)chunks[i].new_start + chunks[i].len);
  if ((st = check_paged(cfg, dst, end, "dst")) != CB_OK) return st;
  if ((st = check_chunk_formats(chunks, n_chunks, dst)) != CB_OK) return st;
  if (flags & ~CB_COPY_V) return fail(CB_ERR_INVALID, "unknown flags 0x%x", flags);
  return CB_OK;
}

cb_status rerope_enqueue(const cb_model_cfg& c, const cb_chunk* chunks, int32_t n_chunks, const cb_paged_kv& dst,
                         uint32_t flags, float2* table, hipStream_t s) {
  cb_status st = enqueue_rerope(c, chunks, n_chunks, dst, (flags & CB_COPY_V) ? 1 : 0, table, s, nullptr);
  return st == CB_OK ? ok() : st;
}

}  // namespace cb

// ===========================================================================
// public entry points
// ===========================================================================
extern "C" {

int32_t cb_abi_version(void) { return CB_ABI_VERSION; }

const char* cb_last_error(void) { return g_last_error.c_str(); }

const char* cb_status_string(int32_t st) {
  switch (st) {
    case CB_OK: return "CB_OK";
    case CB_ERR_INVALID: return "CB_ERR_INVALID";
    case CB_ERR_UNSUPPORTED: return "CB_ERR_UNSUPPORTED";
    case CB_ERR_WORKSPACE: return "CB_ERR_WORKSPACE";
    case CB_ERR_DEVICE: return "CB_ERR_DEVICE";
    default: return "CB_UNKNOWN_STATUS";
  }
}

size_t cb_packed_weight_bytes(cb_dtype dtype, int64_t rows, int64_t cols) {
  if (dtype != CB_BF16 || rows < 1 || cols < 1) return 0;
  return static_cast<size_t>(pk_rows(rows)) * static_cast<size_t>(cols) * 2;
}

cb_status cb_pack_weight(cb_dtype dtype, const void* src, int64_t rows, int64_t cols, int32_t gate_up, void* dst,
                         cb_stream_t stream) {
  if (dtype != CB_BF16) return fail(CB_ERR_UNSUPPORTED, "only CB_BF16 matrices are packed");
  if (!src || !dst) return fail(CB_ERR_INVALID, "NULL src or dst");
  if (!aligned16(src) || !aligned16(dst)) return fail(CB_ERR_INVALID, "src and dst must be 16-byte aligned");
  if (rows < 1 || cols < 16 || cols % 16) return fail(CB_ERR_INVALID, "rows >= 1 and cols a positive multiple of 16 required");
  if (gate_up && rows % 64) return fail(CB_ERR_INVALID, "gate_up: rows = 2 F with F a multiple of 32 required");
  const size_t nb = cb_packed_weight_bytes(dtype, rows, cols);
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + nb && d0 < s0 + static_cast<size_t>(rows) * cols * 2) return fail(CB_ERR_INVALID, "src and dst overlap");
  if (launch_pack_weight(src, rows, cols, gate_up ? 1 : 0, dst, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(CB_ERR_DEVICE, "pack kernel launch failed");
  return CB_OK;
}

size_t cb_workspace_bytes(const cb_model_cfg* cfg, int32_t n_ctx, int32_t n_query, int32_t n_chunks) {
  if (check_cfg(cfg) != CB_OK || n_ctx < 0 || n_query < 0 || n_chunks < 0) return 0;
  return carve(*cfg, n_ctx, n_query, n_chunks, nullptr, nullptr);
}

cb_status cb_rerope_k(const cb_model_cfg* cfg, const cb_chunk* chunks, int32_t n_chunks, const cb_paged_kv* dst,
                      uint32_t flags, void* ws, size_t ws_bytes, cb_stream_t stream) {
  cb_status st = rerope_check(cfg, chunks, n_chunks, dst, flags);
  if (st != CB_OK) return st;
  const size_t need = cb_workspace_bytes(cfg, 0, 0, n_chunks);
  if (n_chunks > 0 && (!ws || ws_bytes < need))
    return fail(CB_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  if (ws && !aligned16(ws)) return fail(CB_ERR_INVALID, "workspace not 16-byte aligned");
  Ws w;
  carve(*cfg, 0, 0, n_chunks, ws, &w);
  return rerope_enqueue(*cfg, chunks, n_chunks, *dst, flags, w.dtab, reinterpret_cast<hipStream_t>(stream));
}

cb_status cb_kv_deviation(const cb_model_cfg* cfg, int32_t layer, const float* k_fresh, const float* v_fresh,
                          int64_t row_stride, const int32_t* pos, int32_t n_rows, const cb_paged_kv* cache,
                          float* dev_out, cb_stream_t stream) {
  cb_status st = check_cfg(cfg);
  if (st != CB_OK) return st;
  if (layer < 0 || layer >= cfg->n_layers) return fail(CB_ERR_INVALID, "layer %d out of range", layer);
  if (n_rows < 0) return fail(CB_ERR_INVALID, "n_rows < 0");
  if ((st = check_paged(cfg, cache, 0, "cache")) != CB_OK) return st;
  if (n_rows == 0) return ok();
  if (!k_fresh || !v_fresh || !pos || !dev_out) return fail(CB_ERR_INVALID, "NULL pointer");
  const int64_t kvw = (int64_t)cfg->n_kv_heads * cfg->head_dim;
  if (row_stride < kvw || row_stride % 4) return fail(CB_ERR_INVALID, "row_stride must be >= %lld and a multiple of 4", (long long)kvw);
  if (!aligned16(k_fresh) || !aligned16(v_fresh)) return fail(CB_ERR_INVALID, "fresh rows not 16-byte aligned");
  CB_TRY(launch_deviation(cfg->dtype, k_fresh, v_fresh, row_stride, pos, n_rows, ref_of(*cache), layer, (int)kvw,
                          dev_out, nullptr, reinterpret_cast<hipStream_t>(stream)),
         "deviation");
  return ok();
}

cb_status cb_select_hkvd(const float* dev, const int32_t* pos, int32_t n_cand, int32_t k, int32_t* sel_pos,
                         int32_t* sel_slot, void* ws, size_t ws_bytes, cb_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (n_cand < 0) return fail(CB_ERR_INVALID, "n_cand < 0");
  if (k < 0 || k > n_cand) return fail(CB_ERR_INVALID, "k = %d outside [0, %d]", k, n_cand);
  if (k == 0) return ok();
  if (!dev || !pos || !sel_pos) return fail(CB_ERR_INVALID, "NULL pointer");
  CB_TRY(launch_select(dev, pos, n_cand, k, sel_pos, sel_slot, reinterpret_cast<hipStream_t>(stream)), "select");
  return ok();
}

cb_status cb_blend_layer(const cb_model* model, int32_t layer, const cb_paged_kv* kv, const int32_t* pos_in,
                         int32_t n_cand, int32_t n_ctx, int32_t n_query, float* x, int32_t check_flag, int32_t k_keep,
                         int32_t* pos_out, float* dev_out, void* ws, size_t ws_bytes, cb_stream_t stream) {
  cb_status st = check_model(model);
  if (st != CB_OK) return st;
  const cb_model_cfg& c = model->cfg;
  if (layer < 1 || layer >= c.n_layers) return fail(CB_ERR_INVALID, "layer %d outside [1, %d)", layer, c.n_layers);
  if (n_cand < 0 || n_ctx < 0 || n_cand > n_ctx) return fail(CB_ERR_INVALID, "need 0 <= n_cand <= n_ctx");
  if (n_query < 1) return fail(CB_ERR_INVALID, "n_query must be >= 1");
  if (k_keep < 0 || k_keep > n_cand) return fail(CB_ERR_INVALID, "k_keep %d outside [0, %d]", k_keep, n_cand);
  if (!check_flag && k_keep != n_cand) return fail(CB_ERR_INVALID, "an unchecked layer keeps every candidate");
  if ((st = check_paged(&c, kv, (int64_t)n_ctx + n_query, "kv")) != CB_OK) return st;
  if (!x || (n_cand > 0 && !pos_in) || (k_keep > 0 && !pos_out)) return fail(CB_ERR_INVALID, "NULL pointer");
  if (!aligned16(x)) return fail(CB_ERR_INVALID, "x not 16-byte aligned");
  const size_t need = cb_workspace_bytes(&c, n_ctx, n_query, 0);
  if (!ws || ws_bytes < need) return fail(CB_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(CB_ERR_INVALID, "workspace not 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Ws w;
  carve(c, n_ctx, n_query, 0, ws, &w);
  const PagedRef r = ref_of(*kv);
  CB_TRY(launch_rope_pos_table(w.pos_tab, n_ctx + n_query, c.head_dim, c.rope_theta, s), "rope table");
  CB_TRY(launch_build_rows(nullptr, pos_in, n_cand, n_cand, n_ctx, n_query, nullptr, w.rowpos0, nullptr, nullptr, s),
         "rows");
  LayerIo io{};
  io.x_in = x;
  io.x_mid = w.x1;
  io.x_out = x;
  io.cand_pos = pos_in;
  io.rowpos_in = w.rowpos0;
  io.rowpos_out = w.rowpos1;
  io.pos_out = pos_out;
  io.dev_slot = dev_out;
  st = enqueue_layer(*model, layer, r, n_cand, n_ctx, n_query, check_flag ? 1 : 0, k_keep, io, w, s, nullptr);
  return st == CB_OK ? ok() : st;
}

namespace {

// Layer-by-layer supply of the context KV from host memory (streamed prefill):
// layer l of every chunk is copied into ring slot l % S on the copy stream, then
// re-RoPE'd into layer l of the blended cache on the compute stream.
struct StreamFeed {
  const cb_host_chunk* hc = nullptr;
  int n = 0;
  int L = 0;
  int S = 0;
  hipStream_t copy = nullptr;
  hipEvent_t* ev = nullptr;         // [2L]: copied[l], consumed[l]
  char* ring_k = nullptr;
  char* ring_v = nullptr;
  int64_t slot_bytes = 0;
  int64_t row_bytes = 0;            // one token's K (or V) row of one layer
  std::vector<int64_t> pre;         // rows of the slot before chunk i
  bool table_ready = false;
};

constexpr int kStreamSlots = 3;

int stream_slots(const cb_model_cfg& c) { return std::min(c.n_layers, kStreamSlots); }

int64_t stream_ring_bytes(const cb_model_cfg& c, int64_t n_ctx) {
  return (int64_t)stream_slots(c) * 2 * n_ctx * c.n_kv_heads * c.head_dim * esize(c.dtype);
}

cb_status feed_copy(StreamFeed& f, int l) {
  const int slot = l % f.S;
  if (l >= f.S && hipStreamWaitEvent(f.copy, f.ev[f.L + l - f.S], 0) != hipSuccess)
    return fail(CB_ERR_DEVICE, "copy stream: wait for layer %d", l - f.S);
  for (int i = 0; i < f.n; ++i) {
    const int64_t bytes = (int64_t)f.hc[i].len * f.row_bytes;
    if (bytes == 0) continue;
    const int64_t off = (int64_t)slot * f.slot_bytes + f.pre[i] * f.row_bytes;
    if (hipMemcpyAsync(f.ring_k + off, static_cast<const char*>(f.hc[i].k) + l * bytes, bytes, hipMemcpyHostToDevice,
                       f.copy) != hipSuccess ||
        hipMemcpyAsync(f.ring_v + off, static_cast<const char*>(f.hc[i].v) + l * bytes, bytes, hipMemcpyHostToDevice,
                       f.copy) != hipSuccess)
      return fail(CB_ERR_DEVICE, "host -> device copy of layer %d, chunk %d", l, i);
  }
  if (hipEventRecord(f.ev[l], f.copy) != hipSuccess) return fail(CB_ERR_DEVICE, "record copy event of layer %d", l);
  return CB_OK;
}

cb_status feed_layer(StreamFeed& f, const cb_model_cfg& c, const cb_paged_kv& blended, int l, float2* dtab,
                     hipStream_t s, Tracer* tr) {
  if (hipStreamWaitEvent(s, f.ev[l], 0) != hipSuccess) return fail(CB_ERR_DEVICE, "wait for the copy of layer %d", l);
  const int slot = l % f.S;
  std::vector<cb_chunk> ch(f.n);
  for (int i = 0; i < f.n; ++i) {
    cb_chunk& x = ch[i];
    std::memset(&x, 0, sizeof(x));
    const int64_t off = (int64_t)slot * f.slot_bytes + f.pre[i] * f.row_bytes;
    x.tokens = f.hc[i].tokens;
    x.k = f.ring_k + off;
    x.v = f.ring_v + off;
    x.len = f.hc[i].len;
    x.old_start = f.hc[i].old_start;
    x.new_start = f.hc[i].new_start;
  }
  cb_model_cfg c1 = c;
  c1.n_layers = 1;
  cb_paged_kv d = blended;
  d.k = static_cast<char*>(d.k) + (int64_t)l * d.layer_stride * esize(c.dtype);
  d.v = static_cast<char*>(d.v) + (int64_t)l * d.layer_stride * esize(c.dtype);
  cb_status st = enqueue_rerope(c1, ch.data(), f.n, d, 1, dtab, s, tr, f.table_ready);
  if (st != CB_OK) return st;
  f.table_ready = f.n <= kMaxChunksPerLaunch;   // one batch: the delta table stays valid
  if (hipEventRecord(f.ev[f.L + l], s) != hipSuccess) return fail(CB_ERR_DEVICE, "record consumed event of layer %d", l);
  return l + f.S < f.L ? feed_copy(f, l + f.S) : CB_OK;
}

// The blended prefill after validation.  feed == NULL: chunk caches on the
// device, re-RoPE'd for every layer up front; else supplied layer by layer.
cb_status blend_run(const cb_model* model, const cb_chunk* chunks, int32_t n_chunks, int N,
                    const int32_t* query_tokens, int32_t n_query, const cb_blend_params* params,
                    const cb_paged_kv* blended, float* logits, int32_t* hkvd_out, float* dev_out, void* ws,
                    hipStream_t s, StreamFeed* feed) {
  cb_status st;
  const cb_model_cfg& c = model->cfg;
  const int L = c.n_layers;
  const int Q = n_query;
  const int T = N + Q;
  Ws w;
  carve(c, N, Q, n_chunks, ws, &w);
  const PagedRef kv = ref_of(*blended);
  Tracer tracer;
  tracer.t = params->trace;
  tracer.s = s;
  if (tracer.t) tracer.t->used = 0;
  Tracer* tr = &tracer;

  // a1: assemble + re-RoPE every layer of every chunk (or start the layer feed)
  if (!feed) {
    if ((st = enqueue_rerope(c, chunks, n_chunks, *blended, 1, w.dtab, s, tr)) != CB_OK) return st;
  } else {
    // the ring may still be read by work enqueued earlier on the compute stream (a
    // previous call with the same workspace): the copy stream starts after it.  The
    // consumed event of layer 0 is free until feed_layer(0) records it again.
    if (hipEventRecord(feed->ev[feed->L], s) != hipSuccess || hipStreamWaitEvent(feed->copy, feed->ev[feed->L], 0) != hipSuccess)
      return fail(CB_ERR_DEVICE, "copy stream: wait for earlier work on the compute stream");
    for (int l = 0; l < feed->S; ++l)
      if ((st = feed_copy(*feed, l)) != CB_OK) return st;
  }
  CB_LAUNCH(tr, CB_KIND_OTHER, launch_rope_pos_table(w.pos_tab, T, c.head_dim, c.rope_theta, s), "rope table");
  // a2: tokens in new-position order, then embeddings
  {
    std::vector<cb_chunk> all(chunks, chunks + n_chunks);
    cb_chunk qc{};
    qc.tokens = query_tokens;
    qc.len = Q;
    qc.new_start = N;
    all.push_back(qc);
    for (size_t first = 0; first < all.size(); first += kMaxChunksPerLaunch) {
      const int cnt = std::min<int>(kMaxChunksPerLaunch, static_cast<int>(all.size() - first));
      ChunkBatch b = make_batch(c, all.data(), static_cast<int>(first), cnt);
      CB_LAUNCH(tr, CB_KIND_OTHER, launch_gather_tokens(b, w.tokens, s), "gather tokens");
    }
  }
  CB_LAUNCH(tr, CB_KIND_OTHER, launch_embed(c.dtype, w.tokens, T, model->embed, c.d_model, w.x0, s), "embed");
  CB_LAUNCH(tr, CB_KIND_OTHER, launch_iota(w.rowpos0, T, 0, s), "iota");
  CB_LAUNCH(tr, CB_KIND_OTHER, launch_iota(w.posA, N, 0, s), "iota");
  if (hkvd_out) CB_LAUNCH(tr, CB_KIND_OTHER, launch_iota(hkvd_out, N, 0, s), "iota");

  // a3: layer 0 in full
  if (feed && (st = feed_layer(*feed, c, *blended, 0, w.dtab, s, tr)) != CB_OK) return st;
  if ((st = enqueue_layer0(*model, kv, N, Q, w.x0, model->layers[1].attn_norm, w, s, tr)) != CB_OK) return st;

  // layers 1 .. L-1
  float* xcur = w.x0;
  float* xoth = w.x1;
  int32_t* cand = w.posA;
  int32_t* nxt = w.posB;
  int32_t* rp_in = w.rowpos0;
  int32_t* rp_out = w.rowpos1;
  int nc = N;
  for (int l = 1; l < L; ++l) {
    if (feed && (st = feed_layer(*feed, c, *blended, l, w.dtab, s, tr)) != CB_OK) return st;
    const int k = params->k_per_layer[l];
    const int chk = params->check[l] ? 1 : 0;
    LayerIo io{};
    io.x_in = xcur;
    io.x_mid = xoth;
    io.x_out = xoth;
    io.cand_pos = cand;
    io.rowpos_in = rp_in;
    io.rowpos_out = rp_out;
    io.pos_out = nxt;
    io.dev_slot = nullptr;
    io.dev_by_pos = (chk && dev_out) ? dev_out + (int64_t)l * N : nullptr;
    io.hkvd_row = hkvd_out ? hkvd_out + (int64_t)l * N : nullptr;
    io.act_ready = true;   // the previous layer's down projection normalised its output rows
    io.next_norm = (l + 1 < L) ? model->layers[l + 1].attn_norm : nullptr;
    if ((st = enqueue_layer(*model, l, kv, nc, N, Q, chk, k, io, w, s, tr)) != CB_OK) return st;
    std::swap(xcur, xoth);
    std::swap(cand, nxt);
    std::swap(rp_in, rp_out);
    nc = k;
  }

  // a12: final norm of the last position, LM head
  const int R = nc + Q;
  CB_LAUNCH(tr, CB_KIND_NORM, launch_rmsnorm(c.dtype, xcur + (int64_t)(R - 1) * c.d_model, nullptr, c.d_model, 1, c.d_model,
                        model->final_norm, c.rms_eps, w.a_last, c.d_model, 1, s), "final norm");
  CB_LAUNCH(tr, CB_KIND_LM_HEAD, launch_lmhead(c.dtype, w.a_last, model->lm_head, c.vocab, c.d_model, logits, s), "lm head");
  return ok();
}

// Validation shared by both prefills (chunk sources are checked by the caller).
cb_status check_blend_call(const cb_model* model, int N, const int32_t* query_tokens, int32_t n_query,
                           const cb_blend_params* params, const cb_paged_kv* blended, const float* logits) {
  const cb_model_cfg& c = model->cfg;
  if (n_query < 1) return fail(CB_ERR_INVALID, "n_query must be >= 1");
  if (!query_tokens || !logits) return fail(CB_ERR_INVALID, "NULL query_tokens or logits");
  if (!params || !params->k_per_layer || !params->check) return fail(CB_ERR_INVALID, "NULL params");
  if (params->flags) return fail(CB_ERR_INVALID, "unknown params flags 0x%x", params->flags);
  const int L = c.n_layers;
  if (params->k_per_layer[0] != N)
    return fail(CB_ERR_INVALID, "k_per_layer[0] = %d, layer 0 runs in full (N = %d)", params->k_per_layer[0], N);
  for (int l = 1; l < L; ++l) {
    const int k = params->k_per_layer[l], kp = params->k_per_layer[l - 1];
    if (k < 0 || k > kp)
      return fail(CB_ERR_INVALID, "k_per_layer[%d] = %d must lie in [0, k_per_layer[%d] = %d]", l, k, l - 1, kp);
    if (!params->check[l] && k != kp)
      return fail(CB_ERR_INVALID, "layer %d is unchecked but shrinks the set (%d -> %d)", l, kp, k);
  }
  cb_status st;
  if ((st = check_paged(&c, blended, (int64_t)N + n_query, "blended")) != CB_OK) return st;
  if (!aligned16(logits)) return fail(CB_ERR_INVALID, "logits not 16-byte aligned");
  return CB_OK;
}

}  // namespace

cb_status cb_blend_prefill(const cb_model* model, const cb_chunk* chunks, int32_t n_chunks,
                           const int32_t* query_tokens, int32_t n_query, const cb_blend_params* params,
                           const cb_paged_kv* blended, float* logits, int32_t* hkvd_out, float* dev_out, void* ws,
                           size_t ws_bytes, cb_stream_t stream) {
  cb_status st = check_model(model);
  if (st != CB_OK) return st;
  const cb_model_cfg& c = model->cfg;
  if ((st = check_chunk_sources(&c, chunks, n_chunks, true)) != CB_OK) return st;
  int64_t N64 = 0;
  if ((st = check_tiling(chunks, n_chunks, &N64)) != CB_OK) return st;
  const int N = static_cast<int>(N64);
  if ((st = check_blend_call(model, N, query_tokens, n_query, params, blended, logits)) != CB_OK) return st;
  if ((st = check_chunk_formats(chunks, n_chunks, blended)) != CB_OK) return st;
  const size_t need = cb_workspace_bytes(&c, N, n_query, n_chunks);
  if (!ws || ws_bytes < need) return fail(CB_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(CB_ERR_INVALID, "workspace not 16-byte aligned");
  return blend_run(model, chunks, n_chunks, N, query_tokens, n_query, params, blended, logits, hkvd_out, dev_out, ws,
                   reinterpret_cast<hipStream_t>(stream), nullptr);
}

size_t cb_streamed_workspace_bytes(const cb_model_cfg* cfg, int32_t n_ctx, int32_t n_query, int32_t n_chunks) {
  const size_t base = cb_workspace_bytes(cfg, n_ctx, n_query, n_chunks);
  if (base == 0) return 0;
  return base + static_cast<size_t>(stream_ring_bytes(*cfg, n_ctx));
}

cb_status cb_blend_prefill_streamed(const cb_model* model, const cb_host_chunk* chunks, int32_t n_chunks,
                                    const int32_t* query_tokens, int32_t n_query, const cb_blend_params* params,
                                    const cb_paged_kv* blended, float* logits, int32_t* hkvd_out, float* dev_out,
                                    void* ws, size_t ws_bytes, cb_stream_t stream, cb_stream_t copy_stream,
                                    void* const* events) {
  cb_status st = check_model(model);
  if (st != CB_OK) return st;
  const cb_model_cfg& c = model->cfg;
  if (n_chunks < 0) return fail(CB_ERR_INVALID, "n_chunks < 0");
  if (n_chunks > 0 && !chunks) return fail(CB_ERR_INVALID, "chunks is NULL");
  std::vector<cb_chunk> dev(n_chunks);
  for (int i = 0; i < n_chunks; ++i) {
    const cb_host_chunk& x = chunks[i];
    if (x.len < 0) return fail(CB_ERR_INVALID, "chunk %d: len < 0", i);
    if (x.old_start < 0)
      return fail(CB_ERR_INVALID, "chunk %d: unknown stored offset %d (a wrong position gives wrong KV)", i, x.old_start);
    if (x.new_start < 0) return fail(CB_ERR_INVALID, "chunk %d: new_start < 0", i);
    if (x.len > 0 && (!x.k || !x.v || !x.tokens)) return fail(CB_ERR_INVALID, "chunk %d: NULL tokens or host K/V", i);
    std::memset(&dev[i], 0, sizeof(cb_chunk));
    dev[i].tokens = x.tokens;
    dev[i].len = x.len;
    dev[i].old_start = x.old_start;
    dev[i].new_start = x.new_start;
  }
  int64_t N64 = 0;
  if ((st = check_tiling(dev.data(), n_chunks, &N64)) != CB_OK) return st;
  const int N = static_cast<int>(N64);
  if ((st = check_blend_call(model, N, query_tokens, n_query, params, blended, logits)) != CB_OK) return st;
  if (blended->kv_format != CB_KV_MODEL)
    return fail(CB_ERR_UNSUPPORTED, "the layer-pipelined prefill takes caches in the model dtype only");
  if (!events) return fail(CB_ERR_INVALID, "NULL events");
  for (int i = 0; i < 2 * c.n_layers; ++i)
    if (!events[i]) return fail(CB_ERR_INVALID, "event %d is NULL", i);
  const size_t base = cb_workspace_bytes(&c, N, n_query, n_chunks);
  const size_t need = cb_streamed_workspace_bytes(&c, N, n_query, n_chunks);
  if (!ws || ws_bytes < need) return fail(CB_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(CB_ERR_INVALID, "workspace not 16-byte aligned");

  StreamFeed f;
  f.hc = chunks;
  f.n = n_chunks;
  f.L = c.n_layers;
  f.S = stream_slots(c);
  f.copy = reinterpret_cast<hipStream_t>(copy_stream);
  f.ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  f.row_bytes = (int64_t)c.n_kv_heads * c.head_dim * esize(c.dtype);
  f.slot_bytes = (int64_t)N * f.row_bytes;
  f.ring_k = static_cast<char*>(ws) + base;
  f.ring_v = f.ring_k + f.S * f.slot_bytes;
  f.pre.resize(n_chunks);
  int64_t acc = 0;
  for (int i = 0; i < n_chunks; ++i) {
    f.pre[i] = acc;
    acc += chunks[i].len;
  }
  return blend_run(model, dev.data(), n_chunks, N, query_tokens, n_query, params, blended, logits, hkvd_out, dev_out,
                   ws, reinterpret_cast<hipStream_t>(stream), &f);
}

size_t cb_decode_workspace_bytes(const cb_model_cfg* cfg) {
  if (check_cfg(cfg) != CB_OK) return 0;
  return carve(*cfg, 0, 1, 0, nullptr, nullptr);
}

cb_status cb_decode_step(const cb_model* model, const cb_paged_kv* kv, int32_t pos, const int32_t* token,
                         float* logits, void* ws, size_t ws_bytes, cb_stream_t stream) {
  cb_status st = check_model(model);
  if (st != CB_OK) return st;
  const cb_model_cfg& c = model->cfg;
  if (pos < 0) return fail(CB_ERR_INVALID, "pos < 0");
  if (!token || !logits) return fail(CB_ERR_INVALID, "NULL token or logits");
  if (!aligned16(logits)) return fail(CB_ERR_INVALID, "logits not 16-byte aligned");
  if ((st = check_paged(&c, kv, (int64_t)pos + 1, "kv")) != CB_OK) return st;
  const size_t need = cb_decode_workspace_bytes(&c);
  if (!ws || ws_bytes < need) return fail(CB_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(CB_ERR_INVALID, "workspace not 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Ws w;
  carve(c, 0, 1, 0, ws, &w);
  const PagedRef r = ref_of(*kv);
  const int L = c.n_layers, d = c.d_model, F = c.d_ff;
  const int qw = c.n_q_heads * c.head_dim;
  const int kvw = c.n_kv_heads * c.head_dim;
  // one row at position pos: the GEMM epilogues rotate with a one-row table and
  // row position 0 (w.rowpos1); scatter and attention use the real position (w.rowpos0)
  CB_TRY(launch_rope_pos_table(w.pos_tab, 1, c.head_dim, c.rope_theta, s, pos), "rope table");
  CB_TRY(launch_iota(w.rowpos0, 1, pos, s), "position");
  CB_TRY(launch_iota(w.rowpos1, 1, 0, s), "table row");
  CB_TRY(launch_embed(c.dtype, token, 1, model->embed, d, w.x0, s), "embed");
  if (c.dtype == CB_BF16) {
    // matrix-vector products over the packed weights; the RMSNorms, the SwiGLU and the
    // residual adds ride on their inputs and outputs
    float* xcur = w.x0;
    float* x1 = w.x1;                                        // xcur + O projection
    float* xnext = static_cast<float*>(w.act);              // [d] fp32 (the activation block is unused here)
    bf16_t* hs = static_cast<bf16_t*>(w.h);                  // SiLU(gate) * up [F] bf16
    for (int l = 0; l < L; ++l) {
      const cb_layer_w& lw = model->layers[l];
      CB_TRY(launch_gemv_qkv(lw.w_qkv, d, xcur, lw.attn_norm, c.rms_eps, qw, kvw, c.head_dim, w.pos_tab, w.q, r, l,
                             pos, s), "qkv");
      AttnArgs at{};
      at.q = w.q; at.ldq = qw; at.o = w.o; at.ldo = qw; at.rowpos = w.rowpos0; at.R = 1;
      at.cache = r; at.layer = l; at.n_q_heads = c.n_q_heads; at.n_kv_heads = c.n_kv_heads; at.head_dim = c.head_dim;
      at.scale = 1.0f / sqrtf(static_cast<float>(c.head_dim));
      at.kv_bound = pos + 1;
      at.part_o = w.attn_o;
      at.part_ml = w.attn_ml;
      CB_TRY(launch_attention(c.dtype, at, s), "attention");
      CB_TRY(launch_gemv(0, false, lw.w_o, d, qw, w.o, nullptr, nullptr, 0.f, x1, xcur, nullptr, s), "o");
      CB_TRY(launch_gemv(1, true, lw.w_gate_up, 2 * F, d, x1, nullptr, lw.mlp_norm, c.rms_eps, hs, nullptr, nullptr,
                         s), "gate/up");
      CB_TRY(launch_gemv(2, false, lw.w_down, d, F, hs, nullptr, nullptr, 0.f, xnext, x1, nullptr, s), "down");
      std::swap(xcur, xnext);
    }
    CB_TRY(launch_rmsnorm(c.dtype, xcur, nullptr, d, 1, d, model->final_norm, c.rms_eps, w.a_last, d, 1, s),
           "final norm");
    CB_TRY(launch_lmhead(c.dtype, w.a_last, model->lm_head, c.vocab, d, logits, s), "lm head");
    return ok();
  }
  CB_TRY(launch_rmsnorm(c.dtype, w.x0, nullptr, d, 1, d, model->layers[0].attn_norm, c.rms_eps, w.act, d, 0, s),
         "rmsnorm");
  for (int l = 0; l < L; ++l) {
    const cb_layer_w& lw = model->layers[l];
    GemmArgs g{};
    g.A = w.act; g.lda = d; g.a_rows = nullptr; g.K = d; g.M = 1;
    g.head_dim = c.head_dim; g.rope_tab = w.pos_tab; g.row_pos = w.rowpos1;
    g.part = w.gemm_part; g.part_floats = kGemmPartFloats;
    if (c.dtype == CB_BF16) {
      g.B = lw.w_qkv; g.ldb = d; g.N = qw + 2 * kvw;
      g.C = w.q; g.ldc = qw; g.q_cols = qw;
      g.C2 = w.kvf; g.ldc2 = 2 * kvw; g.rope2_cols = kvw;
      CB_TRY(launch_gemm(c.dtype, EPI_QKV, g, s), "qkv gemm");
    } else {
      g.B = lw.w_qkv; g.ldb = d; g.N = qw; g.C = w.q; g.ldc = qw; g.rope_cols = qw;
      CB_TRY(launch_gemm(c.dtype, EPI_STORE_ROPE, g, s), "q gemm");
      g.B = static_cast<const char*>(lw.w_qkv) + (int64_t)qw * d * esize(c.dtype); g.N = 2 * kvw;
      g.C = w.kvf; g.ldc = 2 * kvw; g.rope_cols = kvw;
      CB_TRY(launch_gemm(c.dtype, EPI_F32_ROPE, g, s), "kv gemm");
    }
    CB_TRY(launch_scatter_kv(c.dtype, w.kvf, 2 * kvw, nullptr, w.rowpos0, 1, r, l, kvw, s), "scatter");
    AttnArgs at{};
    at.q = w.q; at.ldq = qw; at.o = w.o; at.ldo = qw; at.rowpos = w.rowpos0; at.R = 1;
    at.cache = r; at.layer = l; at.n_q_heads = c.n_q_heads; at.n_kv_heads = c.n_kv_heads; at.head_dim = c.head_dim;
    at.scale = 1.0f / sqrtf(static_cast<float>(c.head_dim));
    at.kv_bound = pos + 1;
    at.part_o = w.attn_o;
    at.part_ml = w.attn_ml;
    CB_TRY(launch_attention(c.dtype, at, s), "attention");
    g = GemmArgs{};
    g.A = w.o; g.lda = qw; g.B = lw.w_o; g.ldb = qw; g.M = 1; g.N = d; g.K = qw;
    g.C = w.x1; g.ldc = d; g.resid = w.x0; g.ld_resid = d;
    g.part = w.gemm_part; g.part_floats = kGemmPartFloats;
    g.norm_gain = lw.mlp_norm; g.norm_eps = c.rms_eps; g.norm_out = w.act;
    CB_TRY(launch_gemm(c.dtype, EPI_RESID, g, s), "o gemm");
    g = GemmArgs{};
    g.A = w.act; g.lda = d; g.B = lw.w_gate_up; g.ldb = d; g.M = 1; g.N = F; g.K = d; g.C = w.h; g.ldc = F; g.ff = F;
    g.part = w.gemm_part; g.part_floats = kGemmPartFloats;
    CB_TRY(launch_gemm(c.dtype, EPI_SWIGLU, g, s), "gate/up gemm");
    g = GemmArgs{};
    g.A = w.h; g.lda = F; g.B = lw.w_down; g.ldb = F; g.M = 1; g.N = d; g.K = F;
    g.C = w.x0; g.ldc = d; g.resid = w.x1; g.ld_resid = d;
    g.part = w.gemm_part; g.part_floats = kGemmPartFloats;
    if (l + 1 < L) { g.norm_gain = model->layers[l + 1].attn_norm; g.norm_eps = c.rms_eps; g.norm_out = w.act; }
    CB_TRY(launch_gemm(c.dtype, EPI_RESID, g, s), "down gemm");
  }
  CB_TRY(launch_rmsnorm(c.dtype, w.x0, nullptr, d, 1, d, model->final_norm, c.rms_eps, w.a_last, d, 1, s), "final norm");
  CB_TRY(launch_lmhead(c.dtype, w.a_last, model->lm_head, c.vocab, d, logits, s), "lm head");
  return ok();
}

size_t cb_blend_index_image_bytes(int32_t n_chunks, int32_t chunk_size) {
  if (n_chunks < 0 || chunk_size < 1) return 0;
  return index_layout(chunk_size, n_chunks, n_chunks, index_slot_bits(n_chunks), index_table_bits(n_chunks)).end;
}

cb_status cb_blend_index_build(const int32_t* tokens, const int64_t* chunk_ids, const int32_t* token_offsets,
                               int32_t n_chunks, int32_t chunk_size, void* image, size_t image_bytes,
                               cb_blend_index_info* info) {
  if (n_chunks < 0 || chunk_size < 1) return fail(CB_ERR_INVALID, "n_chunks %d, chunk_size %d", n_chunks, chunk_size);
  if (!image || !info || (n_chunks > 0 && (!tokens || !chunk_ids || !token_offsets)))
    return fail(CB_ERR_INVALID, "NULL pointer");
  const size_t C = static_cast<size_t>(chunk_size);
  for (int32_t i = 0; i < n_chunks; ++i) {
    if (token_offsets[i] < CB_UNKNOWN_TOKEN_OFFSET) return fail(CB_ERR_INVALID, "chunk %d: offset %d", i, token_offsets[i]);
    for (size_t t = 0; t < C; ++t)
      if (tokens[i * C + t] < 0) return fail(CB_ERR_INVALID, "chunk %d: negative token", i);
  }
  // contents in first-indexed order; occupants per content in input order
  std::unordered_map<uint64_t, int32_t> by_fp;
  std::vector<int32_t> first_chunk;                 // the chunk whose tokens an entry holds
  std::vector<uint64_t> fps;
  std::vector<std::vector<int32_t>> occ;            // chunk indices per entry
  int32_t skipped = 0;
  for (int32_t i = 0; i < n_chunks; ++i) {
    if (token_offsets[i] == CB_UNKNOWN_TOKEN_OFFSET) { ++skipped; continue; }
    const int32_t* t = tokens + i * C;
    uint64_t h = 0;
    for (size_t j = 0; j < C; ++j) h = h * kPolyBase + static_cast<uint32_t>(t[j]);
    auto it = by_fp.find(h);
    if (it == by_fp.end()) {
      by_fp.emplace(h, static_cast<int32_t>(fps.size()));
      fps.push_back(h);
      first_chunk.push_back(i);
      occ.push_back({i});
      continue;
    }
    const int32_t e = it->second;
    if (std::memcmp(tokens + first_chunk[e] * C, t, C * 4) != 0) { ++skipped; continue; }   // fingerprint taken
    bool dup = false;
    for (int32_t o : occ[e]) dup = dup || chunk_ids[o] == chunk_ids[i];
    if (!dup) occ[e].push_back(i);
  }
  const int64_t n_e = static_cast<int64_t>(fps.size());
  int64_t n_o = 0;
  for (const auto& v : occ) n_o += static_cast<int64_t>(v.size());
  const int sb = index_slot_bits(n_e), tb = index_table_bits(n_e);
  const IndexLayout L = index_layout(chunk_size, n_e, n_o, sb, tb);
  if (image_bytes < L.end) return fail(CB_ERR_WORKSPACE, "image %zu bytes, %zu needed", image_bytes, L.end);
  char* b = static_cast<char*>(image);
  std::memset(b, 0, L.end);
  const int32_t hdr[8] = {0x58494243, 1, chunk_size, static_cast<int32_t>(n_e), static_cast<int32_t>(n_o), sb, tb, 0};
  std::memcpy(b, hdr, sizeof(hdr));
  uint8_t* slots = reinterpret_cast<uint8_t*>(b + L.slots);
  uint64_t* tfp = reinterpret_cast<uint64_t*>(b + L.table_fp);
  int32_t* tent = reinterpret_cast<int32_t*>(b + L.table_entry);
  int32_t* etok = reinterpret_cast<int32_t*>(b + L.entry_tokens);
  int32_t* eocc = reinterpret_cast<int32_t*>(b + L.entry_occ);
  int64_t* ochunk = reinterpret_cast<int64_t*>(b + L.occ_chunk);
  int32_t* ooff = reinterpret_cast<int32_t*>(b + L.occ_offset);
  const uint64_t tmask = (uint64_t(1) << tb) - 1;
  for (uint64_t i = 0; i <= tmask; ++i) tent[i] = -1;
  int32_t o = 0;
  for (int64_t e = 0; e < n_e; ++e) {
    const uint64_t h = fps[e];
    slots[h >> (64 - sb)] = 1;
    uint64_t at = h >> (64 - tb);
    while (tent[at] >= 0) at = (at + 1) & tmask;
    tfp[at] = h;
    tent[at] = static_cast<int32_t>(e);
    std::memcpy(etok + e * C, tokens + first_chunk[e] * C, C * 4);
    eocc[e] = o;
    for (int32_t c : occ[e]) {
      ochunk[o] = chunk_ids[c];
      ooff[o] = token_offsets[c];
      ++o;
    }
  }
  eocc[n_e] = o;
  info->chunk_size = chunk_size;
  info->n_entries = static_cast<int32_t>(n_e);
  info->n_occupants = static_cast<int32_t>(n_o);
  info->n_skipped = skipped;
  info->slot_bits = sb;
  info->table_bits = tb;
  info->image_bytes = L.end;
  return ok();
}

size_t cb_blend_match_workspace_bytes(int64_t total_tokens) {
  if (total_tokens < 0) return 0;
  return static_cast<size_t>(((std::max<int64_t>(total_tokens, 1) * 4 + 255) / 256) * 256);
}

cb_status cb_blend_match(const void* index_image, const cb_blend_index_info* info, const int32_t* query_tokens,
                         const int32_t* query_starts, int32_t n_queries, int64_t total_tokens, int32_t max_query_len,
                         int32_t probe_stride, const int32_t* prefix_lens, int32_t max_matches, int64_t* out_chunk,
                         int32_t* out_old_st, int32_t* out_cur_st, uint8_t* out_kept, int32_t* out_count, void* ws,
                         size_t ws_bytes, cb_stream_t stream) {
  if (!index_image || !info) return fail(CB_ERR_INVALID, "NULL index image or info");
  if (n_queries < 0 || n_queries > 65535) return fail(CB_ERR_INVALID, "n_queries %d (0 .. 65535)", n_queries);
  if (probe_stride < 1) return fail(CB_ERR_INVALID, "probe_stride %d < 1", probe_stride);
  if (max_matches < 0 || total_tokens < 0 || max_query_len < 0)
    return fail(CB_ERR_INVALID, "negative max_matches, total_tokens or max_query_len");
  const cb_blend_index_info& I = *info;
  if (I.chunk_size < 1 || I.n_entries < 0 || I.n_occupants < I.n_entries || I.slot_bits != index_slot_bits(I.n_entries) ||
      I.table_bits != index_table_bits(I.n_entries))
    return fail(CB_ERR_INVALID, "index info inconsistent with its sizes");
  const IndexLayout L = index_layout(I.chunk_size, I.n_entries, I.n_occupants, I.slot_bits, I.table_bits);
  if (I.image_bytes != L.end) return fail(CB_ERR_INVALID, "index info: image_bytes %llu, layout %zu",
                                          (unsigned long long)I.image_bytes, L.end);
  if (I.chunk_size > kMatchMaxChunk)
    return fail(CB_ERR_UNSUPPORTED, "chunk_size %d above %d", I.chunk_size, kMatchMaxChunk);
  if (n_queries > 0 && (!query_starts || !out_count)) return fail(CB_ERR_INVALID, "NULL query_starts or out_count");
  if (n_queries > 0 && total_tokens > 0 && !query_tokens) return fail(CB_ERR_INVALID, "NULL query_tokens");
  if (n_queries > 0 && max_matches > 0 && (!out_chunk || !out_old_st || !out_cur_st || !out_kept))
    return fail(CB_ERR_INVALID, "NULL match outputs");
  if (reinterpret_cast<uintptr_t>(index_image) % 256 != 0) return fail(CB_ERR_INVALID, "index image not 256-byte aligned");
  const size_t need = cb_blend_match_workspace_bytes(total_tokens);
  if (!ws || ws_bytes < need) return fail(CB_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, need);
  if (n_queries == 0) return ok();
  const char* b = static_cast<const char*>(index_image);
  MatchIndexRef ix{};
  ix.slots = reinterpret_cast<const uint8_t*>(b + L.slots);
  ix.table_fp = reinterpret_cast<const uint64_t*>(b + L.table_fp);
  ix.table_entry = reinterpret_cast<const int32_t*>(b + L.table_entry);
  ix.entry_tokens = reinterpret_cast<const int32_t*>(b + L.entry_tokens);
  ix.entry_occ = reinterpret_cast<const int32_t*>(b + L.entry_occ);
  ix.occ_chunk = reinterpret_cast<const int64_t*>(b + L.occ_chunk);
  ix.occ_offset = reinterpret_cast<const int32_t*>(b + L.occ_offset);
  ix.chunk_size = I.chunk_size;
  ix.slot_bits = I.slot_bits;
  ix.table_bits = I.table_bits;
  ix.n_entries = I.n_entries;
  uint64_t pw = 1;
  for (int i = 0; i < I.chunk_size; ++i) pw *= kPolyBase;
  ix.pow_c = pw;
  const MatchOut out{out_chunk, out_old_st, out_cur_st, out_kept, out_count};
  CB_TRY(launch_blend_match(ix, query_tokens, query_starts, n_queries, total_tokens, max_query_len, probe_stride,
                            prefix_lens, max_matches, out, static_cast<int32_t*>(ws), reinterpret_cast<hipStream_t>(stream)),
         "blend match");
  return ok();
}

double cb_loading_ratio(double kv_bytes_per_token, double n_tokens, double load_bytes_per_s, double prefill_seconds,
                        double r_min) {
  if (!(prefill_seconds > 0) || !(load_bytes_per_s > 0) || kv_bytes_per_token < 0 || n_tokens < 0) return -1.0;
  const double t_load = kv_bytes_per_token * n_tokens / load_bytes_per_s;
  return std::max(r_min, std::min(1.0, t_load / prefill_seconds));
}

}  // extern "C"
