// HBM-bound kernels of the blended prefill: rotation tables, re-RoPE +
// assembly, embedding, RMSNorm, KV deviation, exact top-k, row maps, the
// paged K/V scatter and the LM-head GEMV.
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn) -- section "位置恢复"
// (k' = R_{n-p} k_p, V untouched), section "核心思想" (eq. Δkv, per-token KV
// deviation), section "选 token" (keep the highest-deviation tokens, sets only
// shrink), Fig. 5 (fresh K/V of the selected tokens fill the cache).
#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// 16-byte vector helpers: 8 bf16 or 4 fp32 elements.
// 16-byte loads and stores that stream past the caches: every byte of the chunk
// caches is read once and every byte of the blended cache written once
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

template <typename T> struct V16;
template <> struct V16<bf16_t> { static constexpr int N = 8; };
template <> struct V16<float> { static constexpr int N = 4; };
template <> struct V16<fp8_t> { static constexpr int N = 16; };

__device__ __forceinline__ void unpack(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf2f(static_cast<bf16_t>(w[i] & 0xFFFFu));
    f[2 * i + 1] = bf2f(static_cast<bf16_t>(w[i] >> 16));
  }
}
__device__ __forceinline__ uint4 pack(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f2bf(f[2 * i])) | (static_cast<uint32_t>(f2bf(f[2 * i + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// A 16-byte vector of T as VN fp32 values (FP8 elements times `scale`), and back
// (FP8: times `inv_scale`, then nearest even, saturating).
template <typename T>
__device__ __forceinline__ void unpack_v(const uint4& v, float* f, float scale) {
  if constexpr (sizeof(T) == 1) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) fp8x4_to_f32(w[i], f + 4 * i);
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] *= scale;
  } else if constexpr (sizeof(T) == 2) {
    float g[8];
    unpack(v, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = g[i];
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}
template <typename T>
__device__ __forceinline__ uint4 pack_v(const float* f, float inv_scale) {
  if constexpr (sizeof(T) == 1) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = f32_to_fp8x4(f[4 * i] * inv_scale, f[4 * i + 1] * inv_scale, f[4 * i + 2] * inv_scale,
                          f[4 * i + 3] * inv_scale);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (sizeof(T) == 2) {
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = f[i];
    return pack(g);
  } else {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
}

// ---------------------------------------------------------------------------
// rotation tables: cos/sin of (multiplier * theta_i), theta_i = base^(-2i/dh),
// evaluated in fp64 and rounded once to fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 rot_entry(double mult, int i, int dh, double theta) {
  const double inv = pow(theta, -(2.0 * i) / static_cast<double>(dh));
  const double ang = mult * inv;
  double s, c;
  sincos(ang, &s, &c);
  return make_float2(static_cast<float>(c), static_cast<float>(s));
}

// row r of the table holds the rotation of position first + r
__global__ void rope_pos_table_kernel(float2* out, int rows, int first, int half, int dh, double theta) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(rows) * half) return;
  const int r = static_cast<int>(idx / half);
  const int i = static_cast<int>(idx % half);
  out[idx] = rot_entry(static_cast<double>(first) + r, i, dh, theta);
}

__global__ void rope_delta_table_kernel(float2* out, ChunkBatch b, int half, int dh, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= b.n * half) return;
  const int c = idx / half;
  const int i = idx % half;
  out[idx] = rot_entry(static_cast<double>(b.d[c].delta), i, dh, theta);
}

// ---------------------------------------------------------------------------
// re-RoPE + assembly.  One block = kTokTile tokens of one (chunk, layer);
// every thread moves 16-byte vectors, four in flight.  When a token row is a
// whole number of passes of the block (256 / vectors-per-row rows per pass) each
// thread keeps one column of the row, so its rotation entries are loaded once
// and no per-vector index division is left.
// ---------------------------------------------------------------------------
constexpr int kTokTile = 16;
constexpr int kRerope = 256;

template <typename T>
__device__ __forceinline__ void rerope_vec(uint4& kv, const float2* cs, float ks, float inv_ks) {
  constexpr int VN = V16<T>::N;
  float f[VN];
  unpack_v<T>(kv, f, ks);
#pragma unroll
  for (int j = 0; j < VN; j += 2) {
    // every product rounded to fp32 before the sum (no fused multiply-add), so the
    // rotated pair is the one plain fp32 arithmetic gives
#pragma clang fp contract(off)
    const float x0 = f[j], x1 = f[j + 1];
    f[j] = x0 * cs[j >> 1].x - x1 * cs[j >> 1].y;
    f[j + 1] = x0 * cs[j >> 1].y + x1 * cs[j >> 1].x;
  }
  kv = pack_v<T>(f, inv_ks);
}

template <typename T>
__global__ __launch_bounds__(kRerope) void rerope_kernel(ChunkBatch b, PagedRef dst, const float2* dtab,
                                                         int n_layers, int width, int dh, int copy_v) {
  constexpr int VN = V16<T>::N;
  const int tile = blockIdx.x;
  // the tile's chunk: tile_begin never decreases, so it is the number of later chunks
  // starting at or before the tile (independent comparisons, not a dependent walk)
  int c = 0;
#pragma unroll 8
  for (int i = 1; i < b.n; ++i) c += tile >= b.d[i].tile_begin ? 1 : 0;
  const ChunkDesc cd = b.d[c];
  const int ntile = (cd.len + kTokTile - 1) / kTokTile;
  const int local = tile - cd.tile_begin;
  const int layer = local / ntile;
  const int t0 = (local % ntile) * kTokTile;
  const int ntok = min(kTokTile, cd.len - t0);
  const int vpr = width / VN;                   // vectors per token row
  const int64_t src_stride = cd.layer_stride;
  const T* srck = static_cast<const T*>(cd.k) + layer * src_stride;
  const T* srcv = static_cast<const T*>(cd.v) + layer * src_stride;
  T* dk = static_cast<T*>(dst.k) + layer * dst.layer_stride;
  T* dv = static_cast<T*>(dst.v) + layer * dst.layer_stride;
  const float2* tab = dtab + static_cast<int64_t>(c) * (dh / 2);
  // FP8: source elements times the chunk's scales, stored divided by the destination's
  const float inv_ks = 1.0f / dst.ks, inv_vs = 1.0f / dst.vs;
  const bool v_requant = sizeof(T) == 1 && cd.vs != dst.vs;
  // element offsets of the tile's source and destination rows, looked up once per block
  __shared__ int64_t srow_s[kTokTile], drow_s[kTokTile];
  if (threadIdx.x < ntok) {
    const int t = t0 + threadIdx.x;
    const int64_t sr = cd.blk ? static_cast<int64_t>(cd.blk[t / cd.block_size]) * cd.block_size + t % cd.block_size
                              : static_cast<int64_t>(t);
    srow_s[threadIdx.x] = sr * width;
    drow_s[threadIdx.x] = paged_row(dst, cd.new_start + t) * width;
  }
  __syncthreads();

  auto store_v = [&](int64_t off, const uint4& raw) __attribute__((always_inline)) {
    uint4 o = raw;
    if (v_requant) {                           // FP8 V under a different scale: re-round on the new grid
      float g[VN];
      unpack_v<T>(raw, g, cd.vs);
      o = pack_v<T>(g, inv_vs);
    }
    st_stream(dv + off, o);
  };
  constexpr int U = 4;
  if (kRerope % vpr == 0) {
    // a row is a whole number of passes of the block: every thread keeps one column
    // (so its rotation entries are loaded once) and walks the tile's rows
    const int rpp = kRerope / vpr;              // rows per pass
    const int col = (threadIdx.x % vpr) * VN;
    const int r0 = threadIdx.x / vpr;
    float2 cs[VN / 2];
#pragma unroll
    for (int j = 0; j < VN; j += 2) cs[j >> 1] = tab[((col + j) % dh) >> 1];
    for (int rb = r0; rb < ntok; rb += rpp * U) {
      uint4 kv[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rb + u * rpp;
        if (r < ntok) {
          kv[u] = ld_stream(srck + srow_s[r] + col);
          if (copy_v) vv[u] = ld_stream(srcv + srow_s[r] + col);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rb + u * rpp;
        if (r >= ntok) continue;
        rerope_vec<T>(kv[u], cs, cd.ks, inv_ks);
        st_stream(dk + drow_s[r] + col, kv[u]);
        if (copy_v) store_v(drow_s[r] + col, vv[u]);
      }
    }
    return;
  }
  const int nvec = ntok * vpr;
  for (int base = threadIdx.x; base < nvec; base += kRerope * U) {
    uint4 kv[U], vv[U];
    int64_t so[U], dof[U];
    int e0[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = base + u * kRerope;
      ok[u] = v < nvec;
      const int tt = ok[u] ? v / vpr : 0;
      e0[u] = (v % vpr) * VN;
      so[u] = srow_s[tt] + e0[u];
      dof[u] = drow_s[tt] + e0[u];
      if (ok[u]) {
        kv[u] = ld_stream(srck + so[u]);
        if (copy_v) vv[u] = ld_stream(srcv + so[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      float2 cs[VN / 2];
#pragma unroll
      for (int j = 0; j < VN; j += 2) cs[j >> 1] = tab[((e0[u] + j) % dh) >> 1];
      rerope_vec<T>(kv[u], cs, cd.ks, inv_ks);
      st_stream(dk + dof[u], kv[u]);
      if (copy_v) store_v(dof[u], vv[u]);
    }
  }
}

__global__ void gather_tokens_kernel(ChunkBatch b, int32_t* out) {
  const ChunkDesc cd = b.d[blockIdx.y];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < cd.len; i += gridDim.x * blockDim.x)
    out[cd.new_start + i] = cd.tokens[i];
}

// ---------------------------------------------------------------------------
// embedding gather (fp32 residual stream)
// ---------------------------------------------------------------------------
// (d a multiple of 64: every row starts 128-byte aligned, and a thread moves 8
// elements per pass with 16-byte accesses)
template <typename T>
__global__ void embed_kernel(const int32_t* tok, const T* emb, int d, float* x) {
  const int r = blockIdx.x;
  const T* src = emb + static_cast<int64_t>(tok[r]) * d;
  float* dst = x + static_cast<int64_t>(r) * d;
  for (int e = threadIdx.x * 8; e < d; e += blockDim.x * 8) {
    float4 lo, hi;
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(src + e);
      lo = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
      hi = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
                       __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u));
    } else {
      lo = *reinterpret_cast<const float4*>(src + e);
      hi = *reinterpret_cast<const float4*>(src + e + 4);
    }
    *reinterpret_cast<float4*>(dst + e) = lo;
    *reinterpret_cast<float4*>(dst + e + 4) = hi;
  }
}

// ---------------------------------------------------------------------------
// RMSNorm: one 256-thread block per row; fp32 statistics reduced in fixed order.
// The row (d <= 16384) is read once and held in registers for the scaling pass.
// ---------------------------------------------------------------------------
template <typename TO, bool PACKED>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, const int32_t* ridx, int64_t ldx, int d,
                                                      const float* g, float eps, TO* out, int64_t ldo) {
  __shared__ float red[4];
  // neighbouring rows on one XCD, so the packed output's fragment blocks are
  // assembled in one L2 (rows of a block interleave at 16-byte granularity)
  const int r = xcd_remap(blockIdx.x, gridDim.x);
  const int src = ridx ? ridx[r] : r;
  const float* xr = x + static_cast<int64_t>(src) * ldx;
  constexpr int kChunks = 16;        // 16 x 1024 columns
  float4 row[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e = threadIdx.x * 4 + c * 1024;
    if (e < d) row[c] = *reinterpret_cast<const float4*>(xr + e);
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e = threadIdx.x * 4 + c * 1024;
    if (e < d) ss += row[c].x * row[c].x + row[c].y * row[c].y + row[c].z * row[c].z + row[c].w * row[c].w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e = threadIdx.x * 4 + c * 1024;
    if (e >= d) continue;
    const float4 v = row[c];
    const float4 gg = *reinterpret_cast<const float4*>(g + e);
    if constexpr (PACKED) {
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(v.x * inv * gg.x)) | (static_cast<uint32_t>(f2bf(v.y * inv * gg.y)) << 16);
      w.y = static_cast<uint32_t>(f2bf(v.z * inv * gg.z)) | (static_cast<uint32_t>(f2bf(v.w * inv * gg.w)) << 16);
      *reinterpret_cast<uint2*>(out + pk_off(r, e, d)) = w;
    } else {
      TO* o = out + static_cast<int64_t>(r) * ldo;
      o[e + 0] = from_f<TO>(v.x * inv * gg.x);
      o[e + 1] = from_f<TO>(v.y * inv * gg.y);
      o[e + 2] = from_f<TO>(v.z * inv * gg.z);
      o[e + 3] = from_f<TO>(v.w * inv * gg.w);
    }
  }
}

// ---------------------------------------------------------------------------
// KV deviation: one wave per row, fp32 accumulation in fixed order.  W > 0: the
// row width is known at compile time and every lane takes 8 consecutive values
// per pass (fresh: two 16-byte loads each for K and V; cached bf16: one), all of
// its loads issued before the first use.  W = 0: any width (a multiple of 4).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[8]) {
  if constexpr (sizeof(T) == 1) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    fp8x4_to_f32(u.x, f);
    fp8x4_to_f32(u.y, f + 4);
  } else if constexpr (sizeof(T) == 2) {
    unpack(*reinterpret_cast<const uint4*>(p), f);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// Squared L2 distance of one fresh K/V row (fp32) from the cached row at position p
// (K and V, every KV head), reduced over the wave in a fixed order; every lane
// returns the sum.  W = 1024: each lane takes 8 consecutive values per pass with
// all of its 16-byte loads issued first; W = 0: any width (a multiple of 4).
template <typename T, int W>
__device__ __forceinline__ float row_deviation(const float* fk, const float* fv, const PagedRef& cache, int layer,
                                               int width, int p, int lane) {
  const int64_t off = static_cast<int64_t>(layer) * cache.layer_stride + paged_row(cache, p) * width;
  const T* ck = static_cast<const T*>(cache.k) + off;
  const T* cv = static_cast<const T*>(cache.v) + off;
  float acc = 0.f;
  if constexpr (W > 0) {
    constexpr int P = W / 512;              // passes of 64 lanes x 8 values
    float a[P][8], b[P][8], c0[P][8], c1[P][8];
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int e = q * 512 + lane * 8;
      load8<float>(fk + e, a[q]);
      load8<float>(fv + e, b[q]);
      load8<T>(ck + e, c0[q]);
      load8<T>(cv + e, c1[q]);
    }
    if constexpr (sizeof(T) == 1) {          // FP8 cache: element times the tensor's scale
#pragma unroll
      for (int q = 0; q < P; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          c0[q][j] *= cache.ks;
          c1[q][j] *= cache.vs;
        }
    }
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float dk0 = a[q][j] - c0[q][j], dk1 = a[q][j + 1] - c0[q][j + 1];
        const float dv0 = b[q][j] - c1[q][j], dv1 = b[q][j + 1] - c1[q][j + 1];
        acc += (dk0 * dk0 + dk1 * dk1) + (dv0 * dv0 + dv1 * dv1);
      }
  } else {
    for (int e = lane * 4; e < width; e += 64 * 4) {
      const float4 a = *reinterpret_cast<const float4*>(fk + e);
      const float4 b = *reinterpret_cast<const float4*>(fv + e);
      float c0[4], c1[4];
      if constexpr (sizeof(T) == 1) {
        fp8x4_to_f32(*reinterpret_cast<const uint32_t*>(ck + e), c0);
        fp8x4_to_f32(*reinterpret_cast<const uint32_t*>(cv + e), c1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c0[j] *= cache.ks;
          c1[j] *= cache.vs;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c0[j] = to_f<T>(ck[e + j]);
          c1[j] = to_f<T>(cv[e + j]);
        }
      }
      const float dk0 = a.x - c0[0], dk1 = a.y - c0[1], dk2 = a.z - c0[2], dk3 = a.w - c0[3];
      const float dv0 = b.x - c1[0], dv1 = b.y - c1[1], dv2 = b.z - c1[2], dv3 = b.w - c1[3];
      acc += (dk0 * dk0 + dk1 * dk1) + (dk2 * dk2 + dk3 * dk3);
      acc += (dv0 * dv0 + dv1 * dv1) + (dv2 * dv2 + dv3 * dv3);
    }
  }
  return wave_sum(acc);
}

template <typename T, int W>
__global__ __launch_bounds__(256) void deviation_kernel(const float* kf, const float* vf, int64_t ldf,
                                                        const int32_t* pos, int n, PagedRef cache, int layer,
                                                        int width, float* dev, float* dev_by_pos) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const int p = pos[row];
  const float acc = row_deviation<T, W>(kf + static_cast<int64_t>(row) * ldf, vf + static_cast<int64_t>(row) * ldf,
                                        cache, layer, width, p, lane);
  if (lane == 0) {
    dev[row] = acc;
    if (dev_by_pos) dev_by_pos[p] = acc;
  }
}

// ---------------------------------------------------------------------------
// exact top-k by (dev descending, position ascending) over candidates given in
// ascending position order, run by one 1024-thread workgroup: radix select of
// the k-th largest order-preserving key in three passes (the top 11 bits, the
// next 11, the last 10; each pass an LDS histogram of the keys that match the
// digits found so far, the digit found by a parallel suffix scan of the bins),
// then a stable compaction in candidate order (ties: the first ones, i.e. the
// smaller positions).  Thread t takes the m = ceil(n / kSel) consecutive
// candidates [t m, t m + m), so candidate order is thread order; their order keys
// are staged in LDS, transposed (thread t's j-th key at j kSel + t, so a wave's
// reads hit distinct banks), when there are at most kSelLdsKeys candidates, else
// recomputed from dev on every read.
// ---------------------------------------------------------------------------
constexpr int kSel = 1024;
constexpr int kSelWaves = kSel / 64;
constexpr int kSelBins = 2048;
constexpr int kSelLdsKeys = 32768;     // 128 KiB of keys (LDS holds 160 KiB per CU)

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// sum of v over the threads above this one (higher thread index)
__device__ __forceinline__ int block_suffix_excl(int v, int* wsum) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl = v;                                     // v over lanes >= lane of this wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_down(incl, d, 64);
    if (lane + d < 64) incl += o;
  }
  if (lane == 0) wsum[wid] = incl;
  __syncthreads();
  int above = 0;
  for (int w = wid + 1; w < kSelWaves; ++w) above += wsum[w];
  __syncthreads();
  return above + incl - v;
}

// With rowpos set the selection also writes the layer's row maps: kept row o
// comes from candidate slot i at position pos[i]; suffix row k + j from input
// row n + j at position n_ctx + j.
struct RowMaps {
  int32_t* gmap;
  int32_t* rowpos;
  int32_t* copy;      // kept positions again (e.g. the per-layer HKVD output), or NULL
  int n_ctx, nq;
};

struct SelectSmem {
  uint32_t hist[kSelBins];
  int wsum[kSelWaves];
  int2 wsum2[kSelWaves];
  uint32_t digit, rem;
};

// Exclusive block scans (in thread order) of two counts at once; writes the totals.
__device__ __forceinline__ int2 block_scan2(int a, int b, int2* wsum2, int2* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int ia = a, ib = b;                               // inclusive within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int oa = __shfl_up(ia, d, 64), ob = __shfl_up(ib, d, 64);
    if (lane >= d) { ia += oa; ib += ob; }
  }
  if (lane == 63) wsum2[wid] = make_int2(ia, ib);
  __syncthreads();
  int2 before = make_int2(0, 0), tot = make_int2(0, 0);
  for (int w = 0; w < kSelWaves; ++w) {
    const int2 c = wsum2[w];
    if (w < wid) { before.x += c.x; before.y += c.y; }
    tot.x += c.x; tot.y += c.y;
  }
  __syncthreads();
  *total = tot;
  return make_int2(before.x + ia - a, before.y + ib - b);
}

// LDS histogram add of digit d for the lanes with `valid`: lanes of the wave that
// share a digit are counted together by one atomic (a few ballot rounds: the
// deviations of a layer often crowd into a few bins), the rest one by one.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool valid, uint32_t d) {
  const int lane = threadIdx.x & 63;
  uint64_t pending = __ballot(valid);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!pending) break;
    const int leader = __ffsll(static_cast<unsigned long long>(pending)) - 1;
    const uint32_t ld = __shfl(d, leader, 64);
    const uint64_t same = __ballot(valid && d == ld) & pending;
    if (lane == leader) atomicAdd(&hist[ld], static_cast<uint32_t>(__popcll(same)));
    pending &= ~same;
  }
  if ((pending >> lane) & 1ull) atomicAdd(&hist[d], 1u);
}

// The selection by the calling workgroup (all kSel threads) over dev[0..n); keys:
// their order keys in LDS (transposed, see above), or NULL to read dev.
__device__ void select_block(const uint32_t* keys, const float* dev, const int32_t* pos, int n, int k, int32_t* sel_pos,
                             int32_t* sel_slot, const RowMaps& rm, SelectSmem& sm) {
  const int tid = threadIdx.x;
  auto keep = [&](int o, int i) {
    const int p = pos[i];
    if (sel_pos) sel_pos[o] = p;
    if (sel_slot) sel_slot[o] = i;
    if (rm.rowpos) {
      rm.gmap[o] = i;
      rm.rowpos[o] = p;
      if (rm.copy) rm.copy[o] = p;
    }
  };
  if (rm.rowpos) {
    const int kk = max(k, 0);
    for (int j = tid; j < rm.nq; j += kSel) {
      rm.gmap[kk + j] = n + j;
      rm.rowpos[kk + j] = rm.n_ctx + j;
    }
  }
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += kSel) keep(i, i);
    return;
  }
  const int m = (n + kSel - 1) / kSel;
  const int i0 = min(n, tid * m), i1 = min(n, i0 + m);
  auto key_of = [&](int i) { return keys ? keys[(i - i0) * kSel + tid] : order_key(dev[i]); };
  uint32_t prefix = 0, mask = 0;
  uint32_t rem = static_cast<uint32_t>(k);
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kBits[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass];
    const uint32_t dmask = (1u << kBits[pass]) - 1u;
    sm.hist[2 * tid] = 0;
    sm.hist[2 * tid + 1] = 0;
    __syncthreads();
    for (int j = 0; j < m; ++j) {                    // uniform trip count: every lane takes part in the ballots
      const int i = i0 + j;
      const uint32_t key = i < i1 ? key_of(i) : 0u;
      hist_add(sm.hist, i < i1 && (key & mask) == prefix, (key >> shift) & dmask);
    }
    __syncthreads();
    // thread t owns bins 2t and 2t+1; the digit is the bin where the count of larger
    // keys first reaches rem
    const uint32_t h0 = sm.hist[2 * tid], h1 = sm.hist[2 * tid + 1];
    const uint32_t above = static_cast<uint32_t>(block_suffix_excl(static_cast<int>(h0 + h1), sm.wsum));
    if (above < rem && rem <= above + h1) {
      sm.digit = 2 * tid + 1;
      sm.rem = rem - above;
    } else if (above + h1 < rem && rem <= above + h1 + h0) {
      sm.digit = 2 * tid;
      sm.rem = rem - above - h1;
    }
    __syncthreads();
    prefix |= sm.digit << shift;
    mask |= dmask << shift;
    rem = sm.rem;
  }
  // prefix = key of the k-th largest; take every larger key and the first `rem` equal
  // ones: candidate i goes to slot (larger keys before i) + (equal keys before i)
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_of(i);
    gt += key > prefix;
    eq += key == prefix;
  }
  int2 tot;
  const int2 before = block_scan2(gt, eq, sm.wsum2, &tot);
  int g = before.x, e = before.y;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_of(i);
    if (key > prefix) {
      keep(g + min(e, static_cast<int>(rem)), i);
      ++g;
    } else if (key == prefix) {
      if (e < static_cast<int>(rem)) keep(g + e, i);
      ++e;
    }
  }
}

// Order keys of dev[0..n) into LDS, transposed, when they fit (returns them), else NULL.
__device__ __forceinline__ const uint32_t* stage_keys(const float* dev, int n, uint32_t* lds_keys) {
  if (n > kSelLdsKeys) return nullptr;
  const int m = (n + kSel - 1) / kSel;
  for (int i = threadIdx.x; i < n; i += kSel) lds_keys[(i % m) * kSel + i / m] = order_key(dev[i]);
  __syncthreads();
  return lds_keys;
}

__global__ __launch_bounds__(kSel) void select_kernel(const float* dev, const int32_t* pos, int n, int k,
                                                      int32_t* sel_pos, int32_t* sel_slot, RowMaps rm) {
  __shared__ SelectSmem sm;
  __shared__ uint32_t lds_keys[kSelLdsKeys];
  select_block(stage_keys(dev, n, lds_keys), dev, pos, n, k, sel_pos, sel_slot, rm, sm);
}

__global__ void build_rows_kernel(const int32_t* sel_slot, const int32_t* sel_pos, int k, int nc, int n_ctx, int nq,
                                  int32_t* gmap, int32_t* rowpos, int32_t* copy_a, int32_t* copy_b) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= k + nq) return;
  int g, p;
  if (i < k) {
    g = sel_slot ? sel_slot[i] : i;
    p = sel_pos[i];
    if (copy_a) copy_a[i] = p;
    if (copy_b) copy_b[i] = p;
  } else {
    g = nc + (i - k);
    p = n_ctx + (i - k);
  }
  if (gmap) gmap[i] = g;
  rowpos[i] = p;
}

// ---------------------------------------------------------------------------
// scatter fresh K/V rows (fp32) into the paged cache in the model dtype
// ---------------------------------------------------------------------------
template <typename T, int W>
__global__ __launch_bounds__(256) void scatter_kv_kernel(const float* kvf, int64_t ldf, const int32_t* gmap,
                                                         const int32_t* rowpos, int n, PagedRef cache, int layer,
                                                         int width) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const int src = gmap ? gmap[row] : row;
  const float* f = kvf + static_cast<int64_t>(src) * ldf;
  const int64_t off = static_cast<int64_t>(layer) * cache.layer_stride +
                      paged_row(cache, rowpos[row]) * width;
  T* ck = static_cast<T*>(cache.k) + off;
  T* cv = static_cast<T*>(cache.v) + off;
  if constexpr (sizeof(T) == 1) {
    // FP8: 8 values per lane and pass, divided by the tensor's scale, one 8-byte store
    const float ik = 1.0f / cache.ks, iv = 1.0f / cache.vs;
    for (int e = lane * 8; e < width; e += 512) {
      float a[8], b[8];
      load8<float>(f + e, a);
      load8<float>(f + width + e, b);
      const uint2 u = make_uint2(f32_to_fp8x4(a[0] * ik, a[1] * ik, a[2] * ik, a[3] * ik),
                                 f32_to_fp8x4(a[4] * ik, a[5] * ik, a[6] * ik, a[7] * ik));
      const uint2 w = make_uint2(f32_to_fp8x4(b[0] * iv, b[1] * iv, b[2] * iv, b[3] * iv),
                                 f32_to_fp8x4(b[4] * iv, b[5] * iv, b[6] * iv, b[7] * iv));
      *reinterpret_cast<uint2*>(ck + e) = u;
      *reinterpret_cast<uint2*>(cv + e) = w;
    }
  } else if constexpr (W > 0 && sizeof(T) == 2) {
    // 8 consecutive values per lane and pass, every load issued first, 16-byte stores
    constexpr int P = W / 512;
    float a[P][8], b[P][8];
#pragma unroll
    for (int q = 0; q < P; ++q) {
      load8<float>(f + q * 512 + lane * 8, a[q]);
      load8<float>(f + width + q * 512 + lane * 8, b[q]);
    }
#pragma unroll
    for (int q = 0; q < P; ++q) {
      *reinterpret_cast<uint4*>(ck + q * 512 + lane * 8) = pack(a[q]);
      *reinterpret_cast<uint4*>(cv + q * 512 + lane * 8) = pack(b[q]);
    }
  } else {
    for (int e = lane * 4; e < width; e += 256) {
      const float4 a = *reinterpret_cast<const float4*>(f + e);
      const float4 b = *reinterpret_cast<const float4*>(f + width + e);
      if constexpr (sizeof(T) == 2) {
        uint2 u, w;
        u.x = f2bf(a.x) | (static_cast<uint32_t>(f2bf(a.y)) << 16);
        u.y = f2bf(a.z) | (static_cast<uint32_t>(f2bf(a.w)) << 16);
        w.x = f2bf(b.x) | (static_cast<uint32_t>(f2bf(b.y)) << 16);
        w.y = f2bf(b.z) | (static_cast<uint32_t>(f2bf(b.w)) << 16);
        *reinterpret_cast<uint2*>(ck + e) = u;
        *reinterpret_cast<uint2*>(cv + e) = w;
      } else {
        *reinterpret_cast<float4*>(ck + e) = a;
        *reinterpret_cast<float4*>(cv + e) = b;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LM head GEMV: one wave per vocabulary row, 16-byte loads, fixed-order sum
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void lmhead_kernel(const float* a, const T* w, int vocab, int d, float* logits) {
  extern __shared__ float sa[];
  for (int e = threadIdx.x; e < d; e += 256) sa[e] = a[e];
  __syncthreads();
  constexpr int VN = V16<T>::N;
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * 4;
  for (int v = blockIdx.x * 4 + (threadIdx.x >> 6); v < vocab; v += waves) {
    const T* row = w + static_cast<int64_t>(v) * d;
    float acc = 0.f;
    for (int e = lane * VN; e < d; e += 64 * VN) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + e);
      if constexpr (VN == 8) {
        float f[8];
        unpack(u, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += f[j] * sa[e + j];
      } else {
        acc += __uint_as_float(u.x) * sa[e] + __uint_as_float(u.y) * sa[e + 1] +
               __uint_as_float(u.z) * sa[e + 2] + __uint_as_float(u.w) * sa[e + 3];
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[v] = acc;
  }
}

// bf16 rows of NL * 512 columns: a wave takes two rows at a time and has all
// 2 NL of its 16-byte weight loads in flight before it sums.
template <int NL>
__global__ __launch_bounds__(256) void lmhead_bf16_kernel(const float* a, const bf16_t* w, int vocab, float* logits) {
  constexpr int d = NL * 512;
  __shared__ float sa[d];
  for (int e = threadIdx.x; e < d; e += 256) sa[e] = a[e];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * 4;
  for (int v0 = 2 * (blockIdx.x * 4 + (threadIdx.x >> 6)); v0 < vocab; v0 += 2 * waves) {
    const int v1 = min(v0 + 1, vocab - 1);
    uint4 u[2][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      u[0][i] = ld_stream(reinterpret_cast<const uint4*>(w + static_cast<int64_t>(v0) * d + i * 512 + lane * 8));
      u[1][i] = ld_stream(reinterpret_cast<const uint4*>(w + static_cast<int64_t>(v1) * d + i * 512 + lane * 8));
    }
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float4 s0 = *reinterpret_cast<const float4*>(&sa[i * 512 + lane * 8]);
      const float4 s1 = *reinterpret_cast<const float4*>(&sa[i * 512 + lane * 8 + 4]);
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float f[8];
        unpack(u[r][i], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r] += f[j] * sv[j];
      }
    }
    acc[0] = wave_sum(acc[0]);
    acc[1] = wave_sum(acc[1]);
    if (lane == 0) {
      logits[v0] = acc[0];
      if (v0 + 1 < vocab) logits[v0 + 1] = acc[1];
    }
  }
}

__global__ void iota_kernel(int32_t* out, int n, int32_t base) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = base + i;
}

inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_rope_pos_table(float2* out, int rows, int head_dim, double theta, hipStream_t s, int first) {
  const int half = head_dim / 2;
  const int64_t n = static_cast<int64_t>(rows) * half;
  if (n == 0) return hipSuccess;
  rope_pos_table_kernel<<<cdiv(n, 256), 256, 0, s>>>(out, rows, first, half, head_dim, theta);
  return hipGetLastError();
}

hipError_t launch_rope_delta_table(float2* out, const ChunkBatch& b, int head_dim, double theta, hipStream_t s) {
  const int half = head_dim / 2;
  const int n = b.n * half;
  if (n == 0) return hipSuccess;
  rope_delta_table_kernel<<<cdiv(n, 256), 256, 0, s>>>(out, b, half, head_dim, theta);
  return hipGetLastError();
}

hipError_t launch_rerope(cb_dtype dt, const ChunkBatch& b, const PagedRef& dst_in, const float2* dtab, int n_layers,
                         int width, int head_dim, int copy_v, hipStream_t s) {
  if (b.total_tiles == 0) return hipSuccess;
  PagedRef dst = dst_in;
  dst.bs_shift = block_shift(dst.bs);
  if (dst.fp8)
    rerope_kernel<fp8_t><<<b.total_tiles, kRerope, 0, s>>>(b, dst, dtab, n_layers, width, head_dim, copy_v);
  else if (dt == CB_BF16)
    rerope_kernel<bf16_t><<<b.total_tiles, kRerope, 0, s>>>(b, dst, dtab, n_layers, width, head_dim, copy_v);
  else
    rerope_kernel<float><<<b.total_tiles, kRerope, 0, s>>>(b, dst, dtab, n_layers, width, head_dim, copy_v);
  return hipGetLastError();
}

hipError_t launch_gather_tokens(const ChunkBatch& b, int32_t* out, hipStream_t s) {
  if (b.n == 0) return hipSuccess;
  gather_tokens_kernel<<<dim3(8, b.n), 256, 0, s>>>(b, out);
  return hipGetLastError();
}

hipError_t launch_embed(cb_dtype dt, const int32_t* tok, int rows, const void* embed, int d, float* x, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (d % 8 != 0) return hipErrorInvalidValue;
  if (dt == CB_BF16)
    embed_kernel<bf16_t><<<rows, 256, 0, s>>>(tok, static_cast<const bf16_t*>(embed), d, x);
  else
    embed_kernel<float><<<rows, 256, 0, s>>>(tok, static_cast<const float*>(embed), d, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(cb_dtype dt, const float* x, const int32_t* ridx, int64_t ldx, int rows, int d,
                          const float* g, float eps, void* out, int64_t ldo, int out_f32, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (d % 4 != 0 || d > 16384) return hipErrorInvalidValue;
  if (out_f32 || dt == CB_F32)
    rmsnorm_kernel<float, false><<<rows, 256, 0, s>>>(x, ridx, ldx, d, g, eps, static_cast<float*>(out), ldo);
  else
    rmsnorm_kernel<bf16_t, true><<<rows, 256, 0, s>>>(x, ridx, ldx, d, g, eps, static_cast<bf16_t*>(out), ldo);
  return hipGetLastError();
}

hipError_t launch_deviation(cb_dtype dt, const float* kf, const float* vf, int64_t ldf, const int32_t* pos, int n,
                            const PagedRef& cache_in, int layer, int width, float* dev, float* dev_by_pos,
                            hipStream_t s) {
  if (n == 0) return hipSuccess;
  PagedRef cache = cache_in;
  cache.bs_shift = block_shift(cache.bs);
  const bool w1k = width == 1024 && ldf % 4 == 0;   // 8 KV heads x 128: 16-byte aligned rows
  if (cache.fp8) {
    if (w1k)
      deviation_kernel<fp8_t, 1024><<<cdiv(n, 4), 256, 0, s>>>(kf, vf, ldf, pos, n, cache, layer, width, dev, dev_by_pos);
    else
      deviation_kernel<fp8_t, 0><<<cdiv(n, 4), 256, 0, s>>>(kf, vf, ldf, pos, n, cache, layer, width, dev, dev_by_pos);
  } else if (dt == CB_BF16) {
    if (w1k)
      deviation_kernel<bf16_t, 1024><<<cdiv(n, 4), 256, 0, s>>>(kf, vf, ldf, pos, n, cache, layer, width, dev, dev_by_pos);
    else
      deviation_kernel<bf16_t, 0><<<cdiv(n, 4), 256, 0, s>>>(kf, vf, ldf, pos, n, cache, layer, width, dev, dev_by_pos);
  } else {
    if (w1k)
      deviation_kernel<float, 1024><<<cdiv(n, 4), 256, 0, s>>>(kf, vf, ldf, pos, n, cache, layer, width, dev, dev_by_pos);
    else
      deviation_kernel<float, 0><<<cdiv(n, 4), 256, 0, s>>>(kf, vf, ldf, pos, n, cache, layer, width, dev, dev_by_pos);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* dev, const int32_t* pos, int n, int k, int32_t* sel_pos, int32_t* sel_slot,
                         hipStream_t s) {
  if (k == 0 || n == 0) return hipSuccess;
  select_kernel<<<1, kSel, 0, s>>>(dev, pos, n, k, sel_pos, sel_slot, RowMaps{nullptr, nullptr, nullptr, 0, 0});
  return hipGetLastError();
}

hipError_t launch_select_rows(const float* dev, const int32_t* pos, int n, int k, int32_t* sel_pos, int32_t* sel_slot,
                              int n_ctx, int nq, int32_t* gmap, int32_t* rowpos, int32_t* copy, hipStream_t s) {
  if (k + nq == 0) return hipSuccess;
  select_kernel<<<1, kSel, 0, s>>>(dev, pos, n, k, sel_pos, sel_slot, RowMaps{gmap, rowpos, copy, n_ctx, nq});
  return hipGetLastError();
}

hipError_t launch_build_rows(const int32_t* sel_slot, const int32_t* sel_pos, int k, int nc, int n_ctx, int nq,
                             int32_t* gmap, int32_t* rowpos, int32_t* copy_a, int32_t* copy_b, hipStream_t s) {
  if (k + nq == 0) return hipSuccess;
  build_rows_kernel<<<cdiv(k + nq, 256), 256, 0, s>>>(sel_slot, sel_pos, k, nc, n_ctx, nq, gmap, rowpos, copy_a,
                                                        copy_b);
  return hipGetLastError();
}

hipError_t launch_scatter_kv(cb_dtype dt, const float* kvf, int64_t ldf, const int32_t* gmap, const int32_t* rowpos,
                             int n, const PagedRef& cache_in, int layer, int width, hipStream_t s) {
  if (n == 0) return hipSuccess;
  PagedRef cache = cache_in;
  cache.bs_shift = block_shift(cache.bs);
  if (cache.fp8)
    scatter_kv_kernel<fp8_t, 0><<<cdiv(n, 4), 256, 0, s>>>(kvf, ldf, gmap, rowpos, n, cache, layer, width);
  else if (dt == CB_BF16 && width == 1024 && ldf % 4 == 0)
    scatter_kv_kernel<bf16_t, 1024><<<cdiv(n, 4), 256, 0, s>>>(kvf, ldf, gmap, rowpos, n, cache, layer, width);
  else if (dt == CB_BF16)
    scatter_kv_kernel<bf16_t, 0><<<cdiv(n, 4), 256, 0, s>>>(kvf, ldf, gmap, rowpos, n, cache, layer, width);
  else
    scatter_kv_kernel<float, 0><<<cdiv(n, 4), 256, 0, s>>>(kvf, ldf, gmap, rowpos, n, cache, layer, width);
  return hipGetLastError();
}

hipError_t launch_lmhead(cb_dtype dt, const float* a, const void* w, int vocab, int d, float* logits, hipStream_t s) {
  const int grid = std::min(2048, cdiv(vocab, 4));
  const size_t lds = static_cast<size_t>(d) * sizeof(float);
  if (dt == CB_BF16 && d == 4096) {
    lmhead_bf16_kernel<8><<<std::min(2048, cdiv(vocab, 8)), 256, 0, s>>>(a, static_cast<const bf16_t*>(w), vocab, logits);
  } else if (dt == CB_BF16 && d == 8192) {
    lmhead_bf16_kernel<16><<<std::min(2048, cdiv(vocab, 8)), 256, 0, s>>>(a, static_cast<const bf16_t*>(w), vocab, logits);
  } else if (dt == CB_BF16)
    lmhead_kernel<bf16_t><<<grid, 256, lds, s>>>(a, static_cast<const bf16_t*>(w), vocab, d, logits);
  else
    lmhead_kernel<float><<<grid, 256, lds, s>>>(a, static_cast<const float*>(w), vocab, d, logits);
  return hipGetLastError();
}

// Weight packing: one thread per 16-byte lane chunk of the packed matrix.
// Chunk c of block (rb, cb) is lane l = c % 64: packed row rb*32 + l%32, columns
// cb*16 + (l/32)*8 .. +7.  With gate_up, packed row block 2b is gate rows
// 32b.. and block 2b+1 up rows F+32b.. (F = rows / 2).  Rows past `rows` are 0.
__global__ __launch_bounds__(256) void pack_weight_kernel(const bf16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                          int gate_up, bf16_t* __restrict__ dst, int64_t n_chunks) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= n_chunks) return;
  const int64_t cblocks = cols >> 4;
  const int64_t blk = c >> 6;
  const int l = static_cast<int>(c & 63);
  const int64_t rb = blk / cblocks, cb = blk % cblocks;
  const int64_t prow = rb * 32 + (l & 31);
  int64_t srow = prow;
  if (gate_up) {
    const int64_t F = rows >> 1;
    srow = ((rb & 1) ? F : 0) + (rb >> 1) * 32 + (l & 31);
  }
  uint4 v = make_uint4(0, 0, 0, 0);
  if (prow < rows) v = *reinterpret_cast<const uint4*>(src + srow * cols + cb * 16 + (l >> 5) * 8);
  *reinterpret_cast<uint4*>(dst + c * 8) = v;
}

hipError_t launch_pack_weight(const void* src, int64_t rows, int64_t cols, int gate_up, void* dst, hipStream_t s) {
  const int64_t n_chunks = pk_rows(rows) * cols / 8;
  const int64_t grid = (n_chunks + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  pack_weight_kernel<<<static_cast<unsigned>(grid), 256, 0, s>>>(static_cast<const bf16_t*>(src), rows, cols, gate_up,
                                                                  static_cast<bf16_t*>(dst), n_chunks);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* out, int n, int32_t base, hipStream_t s) {
  if (n == 0) return hipSuccess;
  iota_kernel<<<cdiv(n, 256), 256, 0, s>>>(out, n, base);
  return hipGetLastError();
}

}  // namespace cb
