// Internal declarations shared by the HIP translation units of libcacheblend.
// Not part of the public ABI (include/cacheblend.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cacheblend.h"

#include <algorithm>

namespace cb {

// bf16 is carried as its 16-bit pattern; arithmetic is always fp32.
using bf16_t = uint16_t;

__host__ __device__ __forceinline__ float bf2f(bf16_t u) {
  union { uint32_t i; float f; } c;
  c.i = static_cast<uint32_t>(u) << 16;
  return c.f;
}

// fp32 -> bf16, round to nearest even.
__host__ __device__ __forceinline__ bf16_t f2bf(float f) {
  union { uint32_t i; float f; } c;
  c.f = f;
  uint32_t u = c.i;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// OCP FP8 E4M3 bytes <-> fp32 through the gfx950 conversion instructions
// (nearest even); stores clamp to +-448 first so out-of-range values saturate.
using fp8_t = uint8_t;
constexpr float kFp8Max = 448.0f;
typedef float f32x2_cv __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  const f32x2_cv a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f32x2_cv b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  f[0] = a.x;
  f[1] = a.y;
  f[2] = b.x;
  f[3] = b.y;
}
__device__ __forceinline__ float fp8_clamp(float x) { return fminf(fmaxf(x, -kFp8Max), kFp8Max); }
__device__ __forceinline__ uint32_t f32_to_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(c), fp8_clamp(d), v, true);
  return static_cast<uint32_t>(v);
}
// an FP8 value has at most 4 significant bits, so its bf16 pattern is exact
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// Reference to a paged cache (see cb_paged_kv).
struct PagedRef {
  void* k;
  void* v;
  const int32_t* bt;   // block table; NULL = identity (contiguous)
  int32_t bs;          // block size
  int64_t layer_stride;
  int32_t bs_shift;    // log2(bs) when bs is a power of two, else -1
  int32_t fp8;         // 1: FP8 E4M3 elements scaled by ks / vs
  float ks, vs;
};

inline int32_t block_shift(int32_t bs) {
  int sh = 0;
  while ((1 << sh) < bs && sh < 30) ++sh;
  return (1 << sh) == bs ? sh : -1;
}

// The hardware hands workgroups of one launch to the 8 XCDs (each with its own
// L2) in round-robin order of their linear id.  xcd_remap turns a linear id into
// a logical work index such that every XCD receives one contiguous range of work
// indices, so neighbouring work (sharing operands) shares an L2.
constexpr int kXcd = 8;
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb / kXcd, r = nb % kXcd;
  const int x = b % kXcd, i = b / kXcd;
  return x * q + min(x, r) + i;
}

// Token row of logical position `pos` in one layer of a paged pool.
__device__ __forceinline__ int64_t paged_row(const int32_t* bt, int32_t bs, int32_t pos) {
  if (bt == nullptr) return pos;
  return static_cast<int64_t>(bt[pos / bs]) * bs + (pos % bs);
}
__device__ __forceinline__ int64_t paged_row(const PagedRef& r, int32_t pos) {
  if (r.bt == nullptr) return pos;
  if (r.bs_shift >= 0)
    return (static_cast<int64_t>(r.bt[pos >> r.bs_shift]) << r.bs_shift) + (pos & (r.bs - 1));
  return static_cast<int64_t>(r.bt[pos / r.bs]) * r.bs + (pos % r.bs);
}

// Fragment-major layout of bf16 GEMM A operands (activations).  A matrix of
// K columns is stored as blocks of 32 rows x 16 columns; each block is the
// 64 x 16-byte A fragment of one v_mfma_f32_32x32x16_bf16 (lane l holds row
// l % 32, columns 8 * (l / 32) .. +7), so one wave loads a fragment as a single
// contiguous 1 KiB read.  Buffers hold ceil(rows / 32) * 32 rows.
__host__ __device__ __forceinline__ int64_t pk_off(int m, int k, int K) {
  return ((static_cast<int64_t>(m >> 5) * (K >> 4) + (k >> 4)) * 64 + ((k >> 3) & 1) * 32 + (m & 31)) * 8 + (k & 7);
}
__host__ __device__ __forceinline__ int64_t pk_rows(int64_t rows) { return (rows + 31) / 32 * 32; }

// Chunk descriptors are passed by value in kernel arguments.
constexpr int kMaxChunksPerLaunch = 32;
// cb_rerope_k's validation and enqueue, shared with the entry point that keeps
// its rotation table in a static device array (cb_noalloc.hip); the table holds
// min(n_chunks, kMaxChunksPerLaunch) x head_dim / 2 (cos, sin) pairs
cb_status rerope_check(const cb_model_cfg* cfg, const cb_chunk* chunks, int32_t n_chunks, const cb_paged_kv* dst,
                       uint32_t flags);
size_t rerope_table_bytes(const cb_model_cfg& c, int n_chunks);
cb_status rerope_enqueue(const cb_model_cfg& c, const cb_chunk* chunks, int32_t n_chunks, const cb_paged_kv& dst,
                         uint32_t flags, float2* table, hipStream_t s);
// sets the thread's last-error text and returns st
cb_status record_failure(cb_status st, const char* msg);
struct ChunkDesc {
  const void* k;
  const void* v;
  const int32_t* blk;     // NULL = contiguous source
  const int32_t* tokens;
  int64_t layer_stride;   // elements
  int32_t len;
  int32_t new_start;
  int32_t block_size;
  int32_t delta;          // new_start - old_start
  int32_t tile_begin;     // first flat tile of this chunk (re-RoPE grid)
  int32_t fp8;            // 1: FP8 E4M3 source scaled by ks / vs
  float ks, vs;
  int32_t pad;
};
struct ChunkBatch {
  ChunkDesc d[kMaxChunksPerLaunch];
  int32_t n;
  int32_t total_tiles;
};

// ---------------------------------------------------------------------------
// launchers (return hipSuccess or the launch error)
// ---------------------------------------------------------------------------

// cos/sin(pos * theta_i) for pos in [0, rows): float2 [rows][dh/2]
// rows of cos/sin for positions first .. first + rows - 1
hipError_t launch_rope_pos_table(float2* out, int rows, int head_dim, double theta, hipStream_t s, int first = 0);
// cos/sin(delta_c * theta_i) per chunk of the batch: float2 [n][dh/2]
hipError_t launch_rope_delta_table(float2* out, const ChunkBatch& b, int head_dim, double theta,
                                   hipStream_t s);
// assemble + rotate: K rotated by the chunk's delta, V copied when copy_v
hipError_t launch_rerope(cb_dtype dt, const ChunkBatch& b, const PagedRef& dst, const float2* dtab,
                         int n_layers, int width, int head_dim, int copy_v, hipStream_t s);
// tokens of the batch's chunks placed at their new_start (plus any extra desc)
hipError_t launch_gather_tokens(const ChunkBatch& b, int32_t* out, hipStream_t s);
// x[t][:] = embed[tok[t]][:] (fp32 out)
hipError_t launch_embed(cb_dtype dt, const int32_t* tok, int rows, const void* embed, int d, float* x,
                        hipStream_t s);
// out[i] = RMSNorm(x[ridx ? ridx[i] : i]) * g, out in model dtype (or fp32 when out_f32);
// bf16 output is written in the fragment-major layout (K = d), fp32 output row-major
hipError_t launch_rmsnorm(cb_dtype dt, const float* x, const int32_t* ridx, int64_t ldx, int rows, int d,
                          const float* g, float eps, void* out, int64_t ldo, int out_f32, hipStream_t s);
// dev[i] = ||kf[i]-K[pos[i]]||^2 + ||vf[i]-V[pos[i]]||^2 ; optionally dev_by_pos[pos[i]] = dev[i]
hipError_t launch_deviation(cb_dtype dt, const float* kf, const float* vf, int64_t ldf, const int32_t* pos,
                            int n, const PagedRef& cache, int layer, int width, float* dev,
                            float* dev_by_pos, hipStream_t s);
// exact top-k by (dev desc, pos asc); outputs ascending
hipError_t launch_select(const float* dev, const int32_t* pos, int n, int k, int32_t* sel_pos,
                         int32_t* sel_slot, hipStream_t s);
// Decode-step matrix-vector product over a packed bf16 matrix (rows x K, K * 2
// bytes at most 64 KiB): the input is bf16 packed row 0 (in_mode 0), bf16 of
// RMSNorm(x + x2) * gain of fp32 vectors (1), or a plain bf16 vector (2).  Output
// y[r] = (r1[r] + r2[r]) + W[r] . x in fp32 (r1, r2 nullable), or with
// swiglu_out (rows a multiple of 64, row blocks alternating 32 gate and 32 up
// rows) bf16 SiLU(gate) * up of rows / 2 features.
hipError_t launch_gemv(int in_mode, bool swiglu_out, const void* w, int rows, int K, const void* x, const float* x2,
                       const float* gain, float eps, void* y, const float* r1, const float* r2, hipStream_t s);
// The fused Q/K/V product of one token (rows qw + 2 kvw, input bf16 of
// RMSNorm(x) * gain), with RoPE of Q/K by the rotation row `rot`: Q to bf16 q,
// K/V (bf16 cache) into the paged cache at `pos` of `layer`.
hipError_t launch_gemv_qkv(const void* w, int K, const void* x, const float* gain, float eps, int qw, int kvw,
                           int head_dim, const float2* rot, void* q, const PagedRef& cache, int layer, int pos,
                           hipStream_t s);

// top-k plus the layer's row maps in one launch (kept rows, then the nq suffix rows):
// gmap[i] (source row), rowpos[i] (position), for i < k + nq; copy (nullable)
// also receives the kept positions [k]
hipError_t launch_select_rows(const float* dev, const int32_t* pos, int n, int k, int32_t* sel_pos, int32_t* sel_slot,
                              int n_ctx, int nq, int32_t* gmap, int32_t* rowpos, int32_t* copy, hipStream_t s);
// the same row maps for an already selected set (copy_a / copy_b nullable)
hipError_t launch_build_rows(const int32_t* sel_slot, const int32_t* sel_pos, int k, int nc, int n_ctx,
                             int nq, int32_t* gmap, int32_t* rowpos, int32_t* copy_a, int32_t* copy_b,
                             hipStream_t s);
// cache[layer][rowpos[i]] <- model dtype of kvf[gmap ? gmap[i] : i] (K: cols [0,W), V: cols [W,2W))
hipError_t launch_scatter_kv(cb_dtype dt, const float* kvf, int64_t ldf, const int32_t* gmap,
                             const int32_t* rowpos, int n, const PagedRef& cache, int layer, int width,
                             hipStream_t s);
// logits[v] = sum_d a[d] * W[v][d]
hipError_t launch_lmhead(cb_dtype dt, const float* a, const void* w, int vocab, int d, float* logits,
                         hipStream_t s);
hipError_t launch_iota(int32_t* out, int n, int32_t base, hipStream_t s);
// bf16 row-major [rows][cols] -> the packed layout of cb_pack_weight
hipError_t launch_pack_weight(const void* src, int64_t rows, int64_t cols, int gate_up, void* dst, hipStream_t s);

// ---------------------------------------------------------------------------
// GEMM: C[M][N] = A[M][K] * B[N][K]^T with a fused epilogue.
// ---------------------------------------------------------------------------
enum GemmEpi : int {
  EPI_STORE_ROPE = 0,   // C (model dtype) = acc, RoPE on columns < rope_cols at row_pos
  EPI_F32_ROPE = 1,     // C (fp32) = acc, RoPE on columns < rope_cols at row_pos
  EPI_RESID = 2,        // C (fp32)[i] = resid[resid_rows ? resid_rows[i] : i] + acc
  EPI_SWIGLU = 3,       // C (model dtype)[i][f] = SiLU(A.Wg[f]) * (A.Wu[f])
  EPI_QKV = 4,          // columns < q_cols: C (model dtype, RoPE); the rest: C2 (fp32) at col - q_cols,
                        // RoPE on its first rope2_cols columns; both at row_pos
};
// bf16: A and B are fragment-major (pk_off, K columns); B is a packed weight
// (cb_pack_weight), for SWIGLU with gate and up 32-row blocks interleaved; the
// SWIGLU output C is fragment-major (ldc = its K).  lda / ldb / ff are unused.
// fp32: everything row-major; SWIGLU B rows [0, ff) gate, [ff, 2 ff) up.
struct GemmArgs {
  const void* A;
  int64_t lda;
  const int32_t* a_rows;   // row gather for A (fp32 path only; NULL = identity)
  const void* B;
  int64_t ldb;
  int M, N, K;             // N = output columns (features for SWIGLU)
  void* C;
  int64_t ldc;
  int rope_cols;
  int head_dim;
  const float2* rope_tab;  // [pos][head_dim/2]
  const int32_t* row_pos;  // [M]
  const float* resid;
  const int32_t* resid_rows;
  int64_t ld_resid;
  int ff;                  // fp32 SWIGLU: row offset of the up half in B
  float* part;             // split-K partial sums (fp32), may be NULL (no split)
  int64_t part_floats;     // capacity of part
  // EPI_RESID only, optional: RMSNorm of the output rows (gain norm_gain, eps
  // norm_eps) into norm_out (the next GEMM's activations: bf16 fragment-major
  // or fp32 row-major, K = N); fused into the split-K reduction when K is split
  const float* norm_gain;
  float norm_eps;
  void* norm_out;
  // EPI_QKV: second output (fp32) for the columns from q_cols on
  float* C2;
  int64_t ldc2;
  int q_cols;
  int rope2_cols;
  // EPI_QKV, optional (blend != 0; bf16 or FP8 cache): every candidate row of the
  // layer is kept.  When K is split, the reduction then also takes, if
  // blend_check, each candidate row's (rows < blend_nc) squared distance of its
  // fresh K/V from the cached row at row_pos into blend_dev[row] (and
  // blend_dev_by_pos[pos] when non-null), and writes every row's fresh K/V into
  // that row of the cache instead of into C2;
  // launch_gemm reports whether it did (if not, C2 holds them as usual).  Keeping
  // every candidate, the top-k is the identity, so the same reduction also writes
  // the layer's row maps: row r's source row (r) into blend_gmap and position into
  // blend_rowpos; for candidate rows the kept position into blend_pos_out and
  // blend_copy and the slot (r) into blend_slot (each nullable).
  int blend;
  int blend_layer;
  int blend_nc;
  int blend_check;
  PagedRef blend_cache;
  float* blend_dev;
  float* blend_dev_by_pos;
  int32_t* blend_gmap;
  int32_t* blend_rowpos;
  int32_t* blend_pos_out;
  int32_t* blend_slot;
  int32_t* blend_copy;
};
constexpr int64_t kGemmPartFloats = int64_t(32) << 20;   // 128 MiB of split-K partials
// *blend_done (nullable): set when an EPI_QKV product with a.blend did the blend's
// deviation and cache write in its reduction
hipError_t launch_gemm(cb_dtype dt, GemmEpi epi, const GemmArgs& a, hipStream_t s, bool* blend_done = nullptr);
// bf16 block tiles: 256 x 256 with 8 waves (one workgroup per CU) or 128 x 256
// with 4 waves (two per CU)
enum GemmCfg : int { GEMM_CFG_256 = 0, GEMM_CFG_128 = 1 };
// bf16 GEMM with an explicit plan: block tile, split of K, and the number of
// tile columns computed whole (the rest split; dp_cols = 0 is plain split-K,
// ignored when splits = 1)
hipError_t launch_gemm_cfg(GemmEpi epi, const GemmArgs& a, int cfg, int splits, int dp_cols, hipStream_t s);
void choose_gemm_cfg(const GemmArgs& a, int epi, int* cfg, int* splits, int* dp_cols);

// ---------------------------------------------------------------------------
// Attention of query rows over a paged cache (causal by absolute position).
// q: [R][Hq*dh] row-major in the model dtype; o: bf16 fragment-major (K = Hq*dh),
// fp32 row-major; rowpos[R] ascending.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const void* q;
  int64_t ldq;
  void* o;
  int64_t ldo;
  const int32_t* rowpos;
  int R;
  PagedRef cache;
  int layer;
  int n_q_heads, n_kv_heads, head_dim;
  float scale;
  int kv_bound;            // host-known bound: every row position is < kv_bound
  float* part_o;           // split-KV partials, attn_partial_floats(head_dim) floats
  float2* part_ml;         // split-KV (max, sum) pairs, attn_partial_rows() entries
  int n_splits_req;        // key splits to use; 0 = chosen by the launcher
  void* widen;             // nullable: room for a bf16 copy of one FP8 layer's K and V
  int64_t widen_bytes;     //   (2 x kv_bound x width x 2 bytes, each run 256-byte aligned)
};
hipError_t launch_attention(cb_dtype dt, const AttnArgs& a, hipStream_t s);
// with an explicit kernel variant: 1 / 2 register-staged K/V with 1 / 2 query groups
// of 16 rows per wave; 3 / 4 LDS-DMA staged K/V (head_dim 128) with 1 / 2 groups
hipError_t launch_attention_ng(cb_dtype dt, const AttnArgs& a, int ng, hipStream_t s);
// workspace bound of the split-KV partials
constexpr int kAttnMaxSplits = 8;
constexpr int64_t kAttnPartialRows = int64_t(kAttnMaxSplits) * 32768;   // (split, row, q head) triples
constexpr int kAttnSplitCap = 64;   // key splits of one launch (a single decode row uses many)
inline int64_t attn_partial_floats(int head_dim) { return kAttnPartialRows * head_dim; }
bool attention_supported(cb_dtype dt, int n_q_heads, int n_kv_heads, int head_dim);

// ---------------------------------------------------------------------------
// Fragment-matching index image: sections at 256-byte aligned offsets from the
// image base (a header, the occupancy filter, the fingerprint table, entry
// tokens, entry occupant ranges, occupant chunk ids and offsets).
// ---------------------------------------------------------------------------
constexpr uint64_t kPolyBase = 0x9E3779B97F4A7C15ull;
constexpr int kMatchMaxChunk = 4096;      // longest chunk_size the scan kernel stages in LDS
constexpr int kMatchMaxContents = 4096;   // distinct contents one request may match
struct IndexLayout {
  size_t slots, table_fp, table_entry, entry_tokens, entry_occ, occ_chunk, occ_offset, end;
};
inline IndexLayout index_layout(int chunk_size, int64_t n_entries, int64_t n_occ, int slot_bits, int table_bits) {
  IndexLayout L{};
  size_t off = 64;                               // header
  auto take = [&](size_t bytes) { off = (off + 255) & ~size_t(255); const size_t at = off; off += bytes; return at; };
  L.slots = take(size_t(1) << slot_bits);
  L.table_fp = take((size_t(1) << table_bits) * 8);
  L.table_entry = take((size_t(1) << table_bits) * 4);
  L.entry_tokens = take(size_t(n_entries) * chunk_size * 4);
  L.entry_occ = take(size_t(n_entries + 1) * 4);
  L.occ_chunk = take(size_t(n_occ) * 8);
  L.occ_offset = take(size_t(n_occ) * 4);
  L.end = (off + 255) & ~size_t(255);
  return L;
}
// the filter: smallest k >= 4 with 2^k >= 16 x entries; the table: load at most 1/4
inline int index_slot_bits(int64_t n_entries) {
  int k = 4;
  while ((int64_t(1) << k) < 16 * std::max<int64_t>(n_entries, 1)) ++k;
  return k;
}
inline int index_table_bits(int64_t n_entries) {
  int k = 4;
  while ((int64_t(1) << k) < 4 * std::max<int64_t>(n_entries, 1)) ++k;
  return k;
}
struct MatchIndexRef {
  const uint8_t* slots;
  const uint64_t* table_fp;
  const int32_t* table_entry;     // -1: empty slot
  const int32_t* entry_tokens;    // [n_entries][chunk_size]
  const int32_t* entry_occ;       // [n_entries + 1] occupant ranges
  const int64_t* occ_chunk;
  const int32_t* occ_offset;
  int chunk_size, slot_bits, table_bits, n_entries;
  uint64_t pow_c;                 // kPolyBase^chunk_size mod 2^64
};
struct MatchOut {
  int64_t* chunk;
  int32_t* old_st;
  int32_t* cur_st;
  uint8_t* kept;
  int32_t* count;
};
// cand: workspace int32 [total] (per token position: verified entry or -1)
hipError_t launch_blend_match(const MatchIndexRef& ix, const int32_t* tokens, const int32_t* starts, int n_queries,
                              int64_t total, int max_len, int stride, const int32_t* prefix, int max_matches,
                              const MatchOut& out, int32_t* cand, hipStream_t s);

}  // namespace cb
