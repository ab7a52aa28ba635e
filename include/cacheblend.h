/*
 * cacheblend.h -- C ABI of the CacheBlend blended-prefill library for AMD
 * Instinct MI355X (gfx950).
 *
 * The method ("CacheBlend 完全拆解", pinghaoyang.com.cn):
 *   - chunks of context are prefilled separately and their KV cached; a request
 *     concatenates the cached chunks, rotating each cached key from the
 *     offset it was stored at to its new offset (section "位置恢复":
 *     k' = R_{n-p} k_p = R_n k; values are not rotated);
 *   - the first layer is computed in full; at every later layer only the
 *     high-KV-deviation (HKVD) tokens chosen at the previous layer are
 *     recomputed: their Q/K/V, their attention over every token, the per-token
 *     deviation between fresh and cached K/V (section "核心思想", eq. Δkv),
 *     and a top-k that keeps a shrinking subset (section "选 token", Fig. 9);
 *     the fresh K/V of the kept tokens replace the cached ones (Fig. 5);
 *   - the per-layer call mirrors the paper's prefill_layer(input_dict{check_flag,
 *     HKVD_indices}, KVCache) (section "位置恢复、KV 存储与加载流水线");
 *   - on any failure the caller falls back to a full prefill (section
 *     "工程落地清单": failures sink unconditionally to full prefill), which
 *     is cb_blend_prefill with k_per_layer[l] = N for every l.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers unless marked HOST.  The caller
 *     owns every buffer; the library never allocates or frees memory and keeps
 *     no pointer after the call returns.  Host arrays are read during the
 *     call only.
 *   - Calls are asynchronous: they validate their arguments on the host,
 *     enqueue kernels on `stream` and return.  Device buffers must stay alive
 *     until that stream work has completed.  No call synchronises the device.
 *   - Validation happens before anything is enqueued.  CB_ERR_INVALID,
 *     CB_ERR_UNSUPPORTED and CB_ERR_WORKSPACE mean nothing was written.
 *     CB_ERR_DEVICE means a launch failed; outputs are then undefined.
 *     cb_last_error() returns a thread-local description of the last failure.
 *   - Device-resident values (token ids, positions, block tables) are
 *     preconditions and are not checked: token ids in [0, vocab), candidate
 *     positions strictly ascending and < N, block-table entries inside the
 *     pools.
 *   - Pointers must be 16-byte aligned; row widths are multiples of 8 elements.
 *   - All kernels are deterministic: no floating-point atomics.
 *   - Calls on different streams with disjoint buffers may run concurrently.
 *   - Model storage dtype: CB_BF16 (bf16 weights and KV, bf16 x bf16 products
 *     with fp32 accumulation on the matrix cores) or CB_F32 (fp32 throughout).
 *     The residual stream, softmax and norm statistics are always fp32.
 */
#ifndef CACHEBLEND_H
#define CACHEBLEND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CB_ABI_VERSION 6

/* A HIP stream (hipStream_t); NULL is the null stream. */
typedef struct ihipStream_t* cb_stream_t;

typedef enum {
  CB_OK = 0,
  CB_ERR_INVALID = -1,     /* bad argument; nothing enqueued                  */
  CB_ERR_UNSUPPORTED = -2, /* shape outside the compiled kernels; nothing enqueued */
  CB_ERR_WORKSPACE = -3,   /* workspace smaller than cb_workspace_bytes()     */
  CB_ERR_DEVICE = -4       /* a kernel launch failed; outputs undefined       */
} cb_status;

typedef enum { CB_F32 = 0, CB_BF16 = 1 } cb_dtype;

/* Flags */
#define CB_COPY_V 1u /* cb_rerope_k: also copy V into the destination */

/* Decoder shape.  Llama-style pre-norm block: x += Attn(RMSNorm(x)),
 * x += W_down(SiLU(W_gate a) * W_up a) with a = RMSNorm(x); RoPE on adjacent
 * pairs (2i, 2i+1) with theta_i = rope_theta^(-2i/head_dim); GQA with q head
 * h reading kv head h / (n_q_heads / n_kv_heads); no biases. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, vocab;
  double rope_theta;
  float rms_eps;
  cb_dtype dtype;
} cb_model_cfg;

/* One decoder layer; norm gains are fp32.  Matrices [out_features][in_features]:
 * CB_F32 models pass them row-major; CB_BF16 models pass them packed by
 * cb_pack_weight (the layout the matrix-core GEMMs read), w_gate_up with
 * gate_up = 1. */
typedef struct {
  const void* w_qkv;      /* [(Hq + 2 Hkv) * dh][d]: Q heads, then K heads, then V heads */
  const void* w_o;        /* [d][Hq * dh]                                             */
  const void* w_gate_up;  /* [2 F][d]: rows [0, F) gate, rows [F, 2F) up              */
  const void* w_down;     /* [d][F]                                                   */
  const float* attn_norm; /* [d]                                                      */
  const float* mlp_norm;  /* [d]                                                      */
} cb_layer_w;

typedef struct {
  cb_model_cfg cfg;
  const void* embed;        /* [vocab][d] model dtype                  */
  const float* final_norm;  /* [d]                                      */
  const void* lm_head;      /* [vocab][d] model dtype (untied)          */
  const cb_layer_w* layers; /* HOST array [n_layers] of device pointers */
  int32_t weights_packed;   /* 1: layer matrices packed by cb_pack_weight
                               (required for CB_BF16); 0: row-major (CB_F32) */
} cb_model;

/* KV cache element formats (cb_paged_kv.kv_format, cb_chunk.kv_format).  The
 * pages run their 34B and 70B models 8-bit and note that an FP8 cache adds
 * quantisation noise to the deviation ranking ("CacheBlend 完全拆解": sections
 * 评测条件 and 偏差比较的精度); the 8-bit format here is OCP FP8 E4M3 (1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, largest finite 448), one byte
 * per element, standing for (element value) x (the tensor's scale); storing
 * rounds to nearest, ties to even, and saturates at +-448.  8-bit caches need
 * a CB_BF16 model. */
#define CB_KV_MODEL 0     /* elements in the model dtype */
#define CB_KV_FP8_E4M3 1  /* one FP8 E4M3 byte per element, scaled by k_scale / v_scale */

/* Paged KV cache: K and V pools laid out [layer][physical block][block_size]
 * [n_kv_heads][head_dim] in the element format kv_format.  Token at logical
 * position p of layer l lives at element offset
 *   l * layer_stride + (block_table[p / block_size] * block_size + p % block_size) * Hkv * dh. */
typedef struct {
  void* k;
  void* v;
  const int32_t* block_table; /* [n_logical] logical -> physical block */
  int32_t block_size;         /* tokens per block, >= 1                */
  int32_t n_logical;          /* entries in block_table                */
  int64_t layer_stride;       /* elements between layers               */
  int32_t kv_format;          /* CB_KV_MODEL or CB_KV_FP8_E4M3          */
  float k_scale, v_scale;     /* CB_KV_FP8_E4M3: value = element x scale (> 0) */
} cb_paged_kv;

/* One cached chunk: tokens and the KV it was prefilled into at old_start.
 * Source KV is either contiguous [n_layers][len][Hkv][dh] (block_ids == NULL;
 * layer_stride 0 means len * Hkv * dh) or paged like cb_paged_kv with
 * block_ids[ceil(len / block_size)] naming the chunk's physical blocks.
 * old_start is the offset the chunk was prefilled at (the re-RoPE source);
 * new_start the offset it takes in this request (the target).  An unknown
 * stored offset (-1) is rejected: a wrong position yields wrong KV. */
typedef struct {
  const int32_t* tokens;    /* [len] */
  const void* k;
  const void* v;
  const int32_t* block_ids; /* NULL = contiguous */
  int32_t len, old_start, new_start;
  int32_t block_size;       /* paged source only */
  int64_t layer_stride;     /* elements; 0 = contiguous default */
  int32_t kv_format;        /* as cb_paged_kv; must equal the destination's */
  float k_scale, v_scale;   /* CB_KV_FP8_E4M3 scales of this chunk's K and V */
} cb_chunk;

/* Launch kinds, for cb_trace. */
typedef enum {
  CB_KIND_REROPE = 0,     /* re-RoPE + assembly of the chunk caches            */
  CB_KIND_GEMM_QKV = 1,   /* Q and K/V projections (RoPE fused)                 */
  CB_KIND_GEMM_O = 2,     /* output projection + residual                      */
  CB_KIND_GEMM_GATE_UP = 3, /* gate/up projection + SiLU-gated product           */
  CB_KIND_GEMM_DOWN = 4,  /* down projection + residual                        */
  CB_KIND_ATTENTION = 5,  /* causal attention of the recomputed rows           */
  CB_KIND_DEVIATION = 6,  /* per-token KV deviation                            */
  CB_KIND_SELECT = 7,     /* top-k of the deviations                           */
  CB_KIND_SCATTER = 8,    /* fresh K/V rows into the paged cache               */
  CB_KIND_NORM = 9,       /* RMSNorm                                           */
  CB_KIND_LM_HEAD = 10,   /* final-position logits                             */
  CB_KIND_OTHER = 11      /* tables, embeddings, row maps                      */
} cb_kind;

/* Optional launch trace: the library records events[2i] / events[2i+1] on the
 * stream right before / after the i-th launch whose kind bit is set in
 * kind_mask, and stores that kind in kinds[i].  Events are hipEvent_t handles
 * the caller created; recording stops when the capacity is reached. */
typedef struct {
  void** events;      /* HOST [capacity] */
  int32_t capacity;
  int32_t used;       /* out: events recorded (an even number) */
  uint32_t kind_mask; /* bit k traces kind k */
  int32_t* kinds;     /* HOST [capacity / 2] or NULL */
} cb_trace;

/* Recompute schedule.  k_per_layer[0] must equal N (layer 0 runs in full);
 * for l >= 1, k_per_layer[l] <= k_per_layer[l-1] (sets only shrink) and
 * check[l] = 0 requires k_per_layer[l] == k_per_layer[l-1]. */
typedef struct {
  const int32_t* k_per_layer; /* HOST [n_layers] */
  const uint8_t* check;       /* HOST [n_layers]; check[0] ignored */
  uint32_t flags;             /* reserved, 0 */
  cb_trace* trace;            /* HOST, nullable: launch trace (see cb_trace) */
} cb_blend_params;

/* ---------------------------------------------------------------------------
 * cb_rerope_k -- assemble chunks into a paged blended cache, rotating K.
 * ("CacheBlend 完全拆解", section "位置恢复": k' = R_{n-p} k_p.)
 * For every chunk c, layer l and token i < len_c:
 *   dst.K[l][new_start + i] = R_{delta_c} K_c[l][i],  delta_c = new_start - old_start,
 * computed in fp32 from fp64 angles and rounded to the model dtype;
 *   dst.V[l][new_start + i] = V_c[l][i] (bitwise) when flags & CB_COPY_V.
 * dst may alias a chunk's K/V (each element is read then written by the same
 * thread).  Chunks may be given in any order and need not tile.
 * ws: at least cb_workspace_bytes(cfg, 0, 0, n_chunks) bytes.
 * Errors: CB_ERR_INVALID for null pointers, old_start < 0, new_start < 0, a
 * chunk ending beyond dst.n_logical * block_size, n_chunks < 0.
 * ------------------------------------------------------------------------- */
cb_status cb_rerope_k(const cb_model_cfg* cfg, const cb_chunk* chunks, int32_t n_chunks,
                      const cb_paged_kv* dst, uint32_t flags, void* ws, size_t ws_bytes,
                      cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * cb_rerope_k_noalloc -- cb_rerope_k without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and errors as cb_rerope_k; the rotation table it writes and the re-RoPE
 * kernel reads lives in a static device array of CB_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, which the library holds until the process ends.  The table
 * needs min(n_chunks, 32) * head_dim / 2 * 8 bytes; a larger need returns
 * CB_ERR_WORKSPACE before anything is enqueued.  The array's address on the
 * current device is looked up once per device (the stream must belong to the
 * current device).  Nothing is allocated or freed.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (on different streams,
 * or from several host threads without ordering) race on it.
 * ------------------------------------------------------------------------- */
#define CB_NOALLOC_SCRATCH_BYTES 65536
cb_status cb_rerope_k_noalloc(const cb_model_cfg* cfg, const cb_chunk* chunks, int32_t n_chunks,
                              const cb_paged_kv* dst, uint32_t flags, cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * cb_kv_deviation -- per-token KV deviation ("CacheBlend 完全拆解", section
 * "核心思想", eq. Δkv), squared L2 over the concatenated K and V of every KV head:
 *   dev_out[i] = sum_e (k_fresh[i][e] - K[layer][pos[i]][e])^2
 *              + sum_e (v_fresh[i][e] - V[layer][pos[i]][e])^2
 * k_fresh / v_fresh: fp32 rows of Hkv * dh elements, row i at offset
 * i * row_stride; k_fresh already rotated to pos[i].  Accumulated in fp32.
 * Errors: CB_ERR_INVALID for null pointers, n_rows < 0, layer out of range,
 * row_stride < Hkv * dh.
 * ------------------------------------------------------------------------- */
cb_status cb_kv_deviation(const cb_model_cfg* cfg, int32_t layer, const float* k_fresh,
                          const float* v_fresh, int64_t row_stride, const int32_t* pos,
                          int32_t n_rows, const cb_paged_kv* cache, float* dev_out,
                          cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * cb_select_hkvd -- exact top-k of the candidates by deviation (section
 * "选 token"): key = (dev descending, position ascending).  Writes the k kept
 * positions ascending to sel_pos[k] and, when sel_slot is not NULL, their
 * indices into the candidate arrays to sel_slot[k].  pos must be strictly
 * ascending.  dev values are ordered by their IEEE bit pattern (a NaN ranks
 * above +inf).  ws / ws_bytes are unused (may be NULL / 0).
 * Errors: CB_ERR_INVALID for null pointers, k < 0, k > n_cand, n_cand < 0.
 * ------------------------------------------------------------------------- */
cb_status cb_select_hkvd(const float* dev, const int32_t* pos, int32_t n_cand, int32_t k,
                         int32_t* sel_pos, int32_t* sel_slot, void* ws, size_t ws_bytes,
                         cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * cb_blend_layer -- one selective-recompute layer, layer >= 1 (Fig. 5; the
 * paper's prefill_layer(input_dict{check_flag, HKVD_indices}, KVCache)).
 *   pos_in[n_cand]: this layer's candidates (HKVD_indices from the previous
 *     layer), strictly ascending, < n_ctx.
 *   x: fp32 [(n_cand + n_query)][d]: the hidden rows of the candidates in
 *     pos_in order, then the n_query suffix rows (positions n_ctx ..
 *     n_ctx + n_query - 1).  On return the first k_keep + n_query rows hold
 *     the layer outputs of pos_out followed by the suffix (compacted in place).
 *   Steps: RMSNorm; fresh K (rotated) and V for every row; when check_flag,
 *   deviation over the candidates and top-k_keep; otherwise every candidate
 *   is kept (k_keep must equal n_cand).  The fresh K/V of the kept rows and
 *   of the suffix are written into kv at their positions; the other
 *   candidates keep the cached K/V.  Then attention of the kept rows and the
 *   suffix over positions [0, own position], O projection, residual, MLP.
 *   pos_out[k_keep]: kept positions, ascending.
 *   dev_out: NULL or fp32 [n_cand] deviations (written when check_flag).
 * kv must cover positions [0, n_ctx + n_query).
 * ws: at least cb_workspace_bytes(&model->cfg, n_ctx, n_query, 0) bytes.
 * ------------------------------------------------------------------------- */
cb_status cb_blend_layer(const cb_model* model, int32_t layer, const cb_paged_kv* kv,
                         const int32_t* pos_in, int32_t n_cand, int32_t n_ctx, int32_t n_query,
                         float* x, int32_t check_flag, int32_t k_keep, int32_t* pos_out,
                         float* dev_out, void* ws, size_t ws_bytes, cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * cb_blend_prefill -- the whole blended prefill.
 *   chunks[n_chunks]: their new_start values must tile [0, N) with no gap or
 *     overlap (overlap resolution is the caller's, leftmost-greedy as in the
 *     "Blend Index" article, section 6.2); old_start >= 0.
 *   query_tokens[n_query] (n_query >= 1) sit at positions N .. N + n_query - 1.
 *   Steps: cb_rerope_k into `blended` (K rotated, V copied); embeddings;
 *   layer 0 in full over every row (context K/V are the re-RoPE'd cache;
 *   suffix K/V computed); layers 1 .. L-1 as cb_blend_layer with
 *   params->k_per_layer / check; final RMSNorm of the last row and LM head.
 *   blended: receives every layer for positions [0, N + n_query).
 *   logits: fp32 [vocab] of the last position.
 *   hkvd_out: NULL or int32 [n_layers][N]; row l starts with S_l ascending
 *     (k_per_layer[l] entries; row 0 is 0 .. N-1).
 *   dev_out: NULL or fp32 [n_layers][N]; at a checked layer l,
 *     dev_out[l][p] = deviation of candidate position p (other entries untouched).
 * ws: at least cb_workspace_bytes(&model->cfg, N, n_query, n_chunks) bytes.
 * ------------------------------------------------------------------------- */
cb_status cb_blend_prefill(const cb_model* model, const cb_chunk* chunks, int32_t n_chunks,
                           const int32_t* query_tokens, int32_t n_query,
                           const cb_blend_params* params, const cb_paged_kv* blended,
                           float* logits, int32_t* hkvd_out, float* dev_out, void* ws,
                           size_t ws_bytes, cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * Layer-pipelined prefill from host-resident chunk caches.  The pages'
 * loading pipeline ("CacheBlend 完全拆解", section 位置恢复、KV 存储与加载流水线):
 * KV is fetched one layer at a time and the recompute of layer l overlaps the
 * loading of the layers after it; the wait between layers is per layer.
 *
 * cb_host_chunk: as cb_chunk, but k / v are HOST pointers to page-locked
 * memory (hipHostMalloc, or torch pin_memory), contiguous
 * [n_layers][len][Hkv][dh] in the model dtype; tokens stay on the device.
 * ------------------------------------------------------------------------- */
typedef struct {
  const int32_t* tokens;    /* device [len] */
  const void* k;            /* host, page-locked */
  const void* v;            /* host, page-locked */
  int32_t len, old_start, new_start;
} cb_host_chunk;

/* Workspace of cb_blend_prefill_streamed: cb_workspace_bytes plus a ring of
 * min(n_layers, 3) slots, each one layer of every chunk's K and V. */
size_t cb_streamed_workspace_bytes(const cb_model_cfg* cfg, int32_t n_ctx, int32_t n_query, int32_t n_chunks);

/* cb_blend_prefill with the chunk caches in host memory.  For every layer l,
 * each chunk's K and V of that layer are copied host -> device on copy_stream
 * into a workspace ring slot; `stream` waits for that copy (events[l]), re-RoPEs
 * the slot into layer l of `blended` and records events[n_layers + l], which the
 * copy of layer l + 3 (reusing the slot) waits for.  Every copy is enqueued
 * before the compute that needs it, so the copies of later layers run while
 * earlier layers are recomputed.
 *   events: HOST array of 2 * n_layers HIP events created by the caller
 *     (hipEventCreateWithFlags with hipEventDisableTiming is enough); they are
 *     recorded and waited on, never created or destroyed here.
 *   copy_stream: the stream for the host -> device copies (it should differ
 *     from `stream`, else nothing overlaps; the result is the same).
 * Results are bitwise those of cb_blend_prefill on the same chunk contents.
 * The host chunk memory, the events and both streams must stay valid until
 * `stream` has completed the call's work (the copies are ordered before it). 
 * Errors as cb_blend_prefill, plus CB_ERR_INVALID for a NULL host pointer or
 * event; ws: at least cb_streamed_workspace_bytes(...). */
cb_status cb_blend_prefill_streamed(const cb_model* model, const cb_host_chunk* chunks, int32_t n_chunks,
                                    const int32_t* query_tokens, int32_t n_query,
                                    const cb_blend_params* params, const cb_paged_kv* blended,
                                    float* logits, int32_t* hkvd_out, float* dev_out, void* ws,
                                    size_t ws_bytes, cb_stream_t stream, cb_stream_t copy_stream,
                                    void* const* events);

/* The loading controller of the same section: recomputing a share r of the
 * tokens costs r * prefill_seconds, loading the cache costs
 * kv_bytes_per_token * n_tokens / load_bytes_per_s; the controller takes the r
 * at which the two match, but never less than the quality floor r_min (the
 * pages use 15%).  Returns max(r_min, min(1, T_load / T_prefill)), or -1 for
 * non-positive prefill_seconds or load_bytes_per_s or negative sizes. */
double cb_loading_ratio(double kv_bytes_per_token, double n_tokens, double load_bytes_per_s,
                        double prefill_seconds, double r_min);

/* ---------------------------------------------------------------------------
 * cb_decode_step -- one decoding step straight on the blended cache ("CacheBlend
 * 完全拆解": Fig. 11, the fused KV is handed to the engine, which starts from
 * decoding; section 问题, a new token's query is dotted with the stored K and
 * weights the stored V, no earlier hidden state is recomputed).
 *   kv: positions [0, pos) of every layer are filled (e.g. by cb_blend_prefill
 *     with N + n_query = pos); the block table must cover pos + 1 tokens.
 *   token: device int32 [1], the token at position pos.
 *   Steps, for every layer: RMSNorm, Q/K/V projection with RoPE at pos, the
 *   token's K/V written at pos, causal attention over [0, pos] through the
 *   block table, O projection + residual, RMSNorm, SwiGLU MLP + residual; then
 *   the final RMSNorm and the LM head.
 *   logits: fp32 [vocab].
 * ws: at least cb_decode_workspace_bytes(&model->cfg) bytes.
 * Errors: CB_ERR_INVALID for NULL pointers, pos < 0, a short block table;
 * CB_ERR_WORKSPACE for a small workspace.
 * ------------------------------------------------------------------------- */
cb_status cb_decode_step(const cb_model* model, const cb_paged_kv* kv, int32_t pos, const int32_t* token,
                         float* logits, void* ws, size_t ws_bytes, cb_stream_t stream);

/* Workspace bytes of cb_decode_step (0 for an invalid cfg). */
size_t cb_decode_workspace_bytes(const cb_model_cfg* cfg);

/* ---------------------------------------------------------------------------
 * Fragment matching: which stored chunks a request contains, and where
 * (LMCache coordinator "Blend Index" article, nxmr.cn).  The match tuples
 * (chunk, old_st, cur_st) are the (old_start, new_start) of cb_chunk.
 * ------------------------------------------------------------------------- */
#define CB_UNKNOWN_TOKEN_OFFSET (-1)

/* Shape of an index image written by cb_blend_index_build. */
typedef struct cb_blend_index_info {
  int32_t chunk_size;   /* tokens per indexed chunk */
  int32_t n_entries;    /* distinct contents (fingerprints) indexed */
  int32_t n_occupants;  /* chunks indexed, over all entries */
  int32_t n_skipped;    /* chunks not indexed: unknown offset, or their fingerprint taken by other content */
  int32_t slot_bits;    /* occupancy filter: 2^slot_bits one-byte slots */
  int32_t table_bits;   /* fingerprint table: 2^table_bits slots (>= 4 per entry), linear probing */
  uint64_t image_bytes; /* bytes of the image actually used */
} cb_blend_index_info;

/* Bytes that suffice for the image of up to n_chunks chunks (0 for n_chunks < 0
 * or chunk_size < 1). */
size_t cb_blend_index_image_bytes(int32_t n_chunks, int32_t chunk_size);

/* cb_blend_index_build -- the index of the article's sections 3.1, 4.1 and 5,
 * built on the host into a position-independent image that the caller copies
 * to device memory as it is.
 *   tokens: host int32 [n_chunks][chunk_size] (token ids >= 0); chunk_ids: host
 *     int64 [n_chunks]; token_offsets: host int32 [n_chunks], each chunk's
 *     position in the sequence that stored it (its re-RoPE source), or
 *     CB_UNKNOWN_TOKEN_OFFSET, which is not indexed (section 5).
 *   A chunk is keyed by the 64-bit polynomial hash of its tokens, Horner's rule
 *   h = h * 0x9E3779B97F4A7C15 + token mod 2^64 from h = 0 (section 3.1).  Chunks
 *   with equal tokens become occupants of one entry, in input order; a chunk
 *   whose fingerprint is taken by different tokens is not indexed (section
 *   4.5).  The filter has 2^k slots, k the smallest value >= 4 with 2^k >= 16 x
 *   entries (growth 16, section 4.4), the slot of a fingerprint being its top k
 *   bits.
 *   image: host buffer of image_bytes >= cb_blend_index_image_bytes(n_chunks,
 *   chunk_size); info: receives the shape (needed by cb_blend_match).
 * Errors: CB_ERR_INVALID for NULL pointers (with n_chunks > 0), n_chunks < 0,
 * chunk_size < 1, a negative token or offset below -1; CB_ERR_WORKSPACE for a
 * small image.  Synchronous host code; no GPU call. */
cb_status cb_blend_index_build(const int32_t* tokens, const int64_t* chunk_ids, const int32_t* token_offsets,
                               int32_t n_chunks, int32_t chunk_size, void* image, size_t image_bytes,
                               cb_blend_index_info* info);

/* Workspace bytes of cb_blend_match for total_tokens query tokens (0 if < 0). */
size_t cb_blend_match_workspace_bytes(int64_t total_tokens);

/* Most distinct contents one query may match (more: its count is -1). */
#define CB_MATCH_MAX_CONTENTS 4096

/* cb_blend_match -- match a batch of requests against an index (section 4.2)
 * and resolve overlaps leftmost-greedy (sections 6.2, 7).
 *   index_image: device copy of the image; info: its shape (host).
 *   query_tokens: device int32, the requests back to back; query_starts: device
 *     int32 [n_queries + 1], request q is tokens [starts[q], starts[q+1]).
 *     total_tokens (host) = starts[n_queries]; max_query_len (host) bounds
 *     every request's length (longer requests are cut there; starts are
 *     clamped to [0, total_tokens]).
 *   probe_stride: windows start at 0, probe_stride, 2 probe_stride, ... (>= 1).
 *   prefix_lens: device int32 [n_queries] or NULL (0): the prefix-cache coverage.
 *   Matching: every window of chunk_size tokens at a probed start is hashed,
 *   tested against the filter, resolved exactly in the fingerprint table, and
 *   compared token by token with the entry's tokens; a verified window takes
 *   the first occupant of the entry that this request has not matched yet.
 *   Outputs per request q, in ascending cur_st (capacity max_matches each):
 *     out_chunk[q * max_matches + i] (int64 chunk id), out_old_st (int32 stored
 *     offset), out_cur_st (int32 start in the request), out_kept (uint8: 1 for
 *     the matches leftmost-greedy keeps -- drop those starting before the
 *     prefix length, then keep a match only if it starts at or after the end of
 *     the last kept one); out_count[q] = matches found (may exceed max_matches,
 *     of which the first max_matches are written), or -1 when the request
 *     matched more than CB_MATCH_MAX_CONTENTS distinct contents.
 *   ws: cb_blend_match_workspace_bytes(total_tokens) bytes.
 * Errors: CB_ERR_INVALID for NULL pointers, n_queries outside [0, 65535],
 * probe_stride < 1, max_matches < 0, an info inconsistent with its own sizes,
 * an image not 256-byte aligned; CB_ERR_UNSUPPORTED for chunk_size above
 * 4096; CB_ERR_WORKSPACE for a small workspace.  Nothing is written on error. */
cb_status cb_blend_match(const void* index_image, const cb_blend_index_info* info, const int32_t* query_tokens,
                         const int32_t* query_starts, int32_t n_queries, int64_t total_tokens, int32_t max_query_len,
                         int32_t probe_stride, const int32_t* prefix_lens, int32_t max_matches, int64_t* out_chunk,
                         int32_t* out_old_st, int32_t* out_cur_st, uint8_t* out_kept, int32_t* out_count, void* ws,
                         size_t ws_bytes, cb_stream_t stream);

/* ---------------------------------------------------------------------------
 * cb_pack_weight -- one layer matrix of a CB_BF16 model into the layout its
 * GEMM reads.  The projections are the paper's per-layer Q/K/V, O and MLP
 * matrices ("CacheBlend 完全拆解", Fig. 5); packing changes only where each
 * element is stored.
 *   src: bf16 row-major [rows][cols] (rows = out_features, cols = in_features).
 *   dst: cb_packed_weight_bytes(dtype, rows, cols) bytes.  The rows are
 *     grouped in blocks of 32 (the last block zero-padded) and the columns in
 *     blocks of 16; block (rb, cb) is 1 KiB at element offset
 *     (rb * cols / 16 + cb) * 512, and within it element (r, c) sits at
 *     ((c / 8 % 2) * 32 + r % 32) * 8 + c % 8, i.e. the order in which the
 *     64 lanes of a 32x32x16 MFMA read their 16-byte operand fragments.
 *   gate_up = 1 (w_gate_up, rows = 2 F, F a multiple of 32): packed row block
 *     2b holds gate rows 32b .. 32b+31 and block 2b+1 the up rows F+32b ..,
 *     so every gate feature and its up partner land in one GEMM tile.
 * Ownership: src and dst are the caller's and must not overlap.
 * Errors: CB_ERR_INVALID for null pointers, rows < 1, cols < 16,
 * cols % 16 != 0, gate_up with rows % 64 != 0; CB_ERR_UNSUPPORTED for a dtype
 * other than CB_BF16 (CB_F32 matrices are used row-major as they are).
 * ------------------------------------------------------------------------- */
cb_status cb_pack_weight(cb_dtype dtype, const void* src, int64_t rows, int64_t cols, int32_t gate_up,
                         void* dst, cb_stream_t stream);

/* Bytes of a packed [rows][cols] matrix: ceil(rows / 32) * 32 * cols * 2 for
 * CB_BF16; 0 for other dtypes or non-positive sizes. */
size_t cb_packed_weight_bytes(cb_dtype dtype, int64_t rows, int64_t cols);

/* Workspace bytes sufficient for every call above on a context of n_ctx
 * tokens, n_query suffix tokens and n_chunks chunks.  Returns 0 for an invalid cfg. */
size_t cb_workspace_bytes(const cb_model_cfg* cfg, int32_t n_ctx, int32_t n_query, int32_t n_chunks);

/* Static name of a status code. */
const char* cb_status_string(int32_t status);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* cb_last_error(void);

/* CB_ABI_VERSION of the built library. */
int32_t cb_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CACHEBLEND_H */
