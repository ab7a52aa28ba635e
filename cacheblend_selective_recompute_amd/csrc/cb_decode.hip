// Decoding one token on the blended cache: matrix-vector products over the
// packed layer weights, with the row-wise transforms around them folded in.
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn): Fig. 11 (the fused KV is
// handed to the engine, which starts from decoding) and section 问题 (a new
// token's query is dotted with the stored K and weights the stored V; no
// earlier hidden state is recomputed).
//
// A decode step reads every weight once, so it is bound by HBM, not by the
// matrix cores.  A packed matrix is a grid of 1 KiB blocks of 32 rows x 16
// columns; within a block, the 8-column half h of row r sits at bytes
// h * 512 + r * 16.  A workgroup owns RB consecutive rows (RB = 8, 16 or 32:
// two runs of RB * 16 bytes in every block of its row block) over all of K, so
// no partial sums cross workgroups; 32 / RB blocks go into one wave load, whose
// lanes each take 16 bytes (8 columns of one row), and the waves take the
// column blocks in turn.  Products accumulate with bf16 dot instructions
// against the input vector, which each workgroup first builds in LDS as bf16:
//   IN_PACKED  a bf16 vector in row 0 of the fragment-major activation layout
//              (element k at (k/16)*512 + ((k/8)%2)*256 + k%8), e.g. the
//              attention output;
//   IN_NORM    RMSNorm(a + b) * gain of fp32 vectors (b optional), rounded to
//              bf16 like the prefill's activations; each workgroup reduces the
//              sum of squares itself in a fixed order, so all agree bitwise;
//   IN_BF16    a plain bf16 vector.
// Outputs: fp32 y[r], or y[r] + r1[r] (+ r2[r]) for the residual stream; for
// the gate/up matrix (whose row blocks alternate 32 gate rows and their 32 up
// rows), a workgroup takes one gate block and its up block together and writes
// bf16(SiLU(gate) * up), the down projection's input; for the fused Q/K/V
// matrix, the rows of a dim pair meet in one workgroup, which applies RoPE and
// writes Q and the cache's new K/V row.
#include "cb_internal.h"

namespace cb {

namespace {

enum { IN_PACKED = 0, IN_NORM = 1, IN_BF16 = 2 };
enum { OUT_F32 = 0, OUT_SWIGLU = 1, OUT_QKV = 2 };

// Where the fused Q/K/V product of one token goes: Q, rotated, to bf16 q;
// K, rotated, and V into the paged cache at the token's position.
struct QkvOut {
  bf16_t* q;
  const float2* rot;    // rotation row of the position: (cos, sin) per dim pair
  PagedRef cache;
  int layer, pos, qw, kvw, head_dim;
};

struct GemvArgs {
  const bf16_t* w;      // packed [rows padded to 32][K]
  int rows, K;
  const void* x;        // IN_PACKED: bf16 packed row 0; IN_NORM: fp32 a; IN_BF16: bf16 vector
  const float* x2;      // IN_NORM: optional fp32 b added to a
  const float* gain;    // IN_NORM
  float eps;            // IN_NORM
  void* y;              // OUT_F32: fp32 [rows]; OUT_SWIGLU: bf16 [rows / 2]
  const float* r1;      // OUT_F32: optional residual terms added to y
  const float* r2;
  QkvOut qkv;           // OUT_QKV
};

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.x), __builtin_bit_cast(bf16x2_v, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.y), __builtin_bit_cast(bf16x2_v, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.z), __builtin_bit_cast(bf16x2_v, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w.w), __builtin_bit_cast(bf16x2_v, x.w), acc, false);
  return acc;
}

constexpr int kGemvU = 8;   // 16-byte weight loads in flight per lane

// Builds the bf16 input vector (K / 8 groups of 8) in LDS.
template <int IN, int NT>
__device__ __forceinline__ void stage_input(const GemvArgs& g, uint4* xs, float* red) {
  const int tid = threadIdx.x;
  float inv = 0.f;
  if constexpr (IN == IN_NORM) {
    const float4* a = static_cast<const float4*>(g.x);
    const float4* b = reinterpret_cast<const float4*>(g.x2);
    float ss = 0.f;
    for (int e = tid; e < (g.K >> 2); e += NT) {
      float4 v = a[e];
      if (b) { const float4 t = b[e]; v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w; }
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum_f(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < NT / 64; ++w) t += red[w];   // every thread, same order
    inv = 1.0f / sqrtf(t / static_cast<float>(g.K) + g.eps);
  }
  for (int q = tid; q < (g.K >> 3); q += NT) {
    const int c0 = q * 8;
    uint4 o;
    if constexpr (IN == IN_PACKED) {
      o = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.x) + (c0 >> 4) * 512 + ((c0 >> 3) & 1) * 256);
    } else if constexpr (IN == IN_BF16) {
      o = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(g.x) + c0);
    } else {
      const float4* a = reinterpret_cast<const float4*>(static_cast<const float*>(g.x) + c0);
      const float4* gn = reinterpret_cast<const float4*>(g.gain + c0);
      float4 a0 = a[0], a1 = a[1];
      if (g.x2) {
        const float4* b = reinterpret_cast<const float4*>(g.x2 + c0);
        const float4 b0 = b[0], b1 = b[1];
        a0.x += b0.x; a0.y += b0.y; a0.z += b0.z; a0.w += b0.w;
        a1.x += b1.x; a1.y += b1.y; a1.z += b1.z; a1.w += b1.w;
      }
      const float4 g0 = gn[0], g1 = gn[1];
      o.x = pack_bf2(a0.x * inv * g0.x, a0.y * inv * g0.y);
      o.y = pack_bf2(a0.z * inv * g0.z, a0.w * inv * g0.w);
      o.z = pack_bf2(a1.x * inv * g1.x, a1.y * inv * g1.y);
      o.w = pack_bf2(a1.z * inv * g1.z, a1.w * inv * g1.w);
    }
    xs[q] = o;
  }
  __syncthreads();
}

template <int IN, int OUT, int RB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_packed_kernel(GemvArgs g) {
  // weights are read once per token: non-temporal loads, except for the product whose
  // input is the packed attention output (O), where plain loads measured faster
  // (70B width: down 83.1 -> 73.9 us, gate/up 157.1 -> 147.9 us, Q/K/V 37.8 -> 35.6 us;
  // 8B O 8.0 -> 9.2 us with them)
  constexpr bool kStreamW = IN != IN_PACKED;
  extern __shared__ uint4 xs[];          // [K / 8] groups of 8 bf16 inputs
  constexpr int NR = OUT == OUT_SWIGLU ? 2 : 1;   // row blocks per workgroup: the gate/up pair takes two
  constexpr int NB = 32 / RB;            // column blocks per wave load
  static_assert(OUT != OUT_SWIGLU || RB == 32, "the gate/up pair takes whole row blocks");
  __shared__ float red[WAVES][32 * NR];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int kbr = g.K >> 4;
  const int j = lane / (2 * RB), hh = (lane / RB) & 1, rr = lane % RB;
  // this lane's 16 bytes in column block 0 of each owned row block
  const bf16_t* wp[NR];
  int row0;
  if constexpr (NR == 2) {
    row0 = blockIdx.x * 64;
    wp[0] = g.w + (static_cast<int64_t>(2 * blockIdx.x) * kbr) * 512 + hh * 256 + rr * 8;
    wp[1] = wp[0] + static_cast<int64_t>(kbr) * 512;
  } else {
    row0 = blockIdx.x * RB;
    const int blk = row0 >> 5, sub = (row0 & 31) / RB;
    wp[0] = g.w + (static_cast<int64_t>(blk) * kbr) * 512 + hh * 256 + (sub * RB + rr) * 8;
  }
  // wave load i of wave w covers column blocks (i * WAVES + w) * NB .. + NB - 1
  const int n_ld = (kbr + NB - 1) / NB;
  constexpr int LPB = kGemvU / NR;       // wave loads per batch
  uint4 wv[kGemvU];
  auto issue = [&](int i0) {
#pragma unroll
    for (int u = 0; u < kGemvU; ++u) {
      const int kb = ((i0 + u / NR) * WAVES + wid) * NB + j;
      if (kb < kbr) {
        const bf16_t* src = wp[u % NR] + static_cast<int64_t>(kb) * 512;
        if constexpr (kStreamW) {
          const u32x4_v t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(src));
          wv[u] = make_uint4(t.x, t.y, t.z, t.w);
        } else {
          wv[u] = *reinterpret_cast<const uint4*>(src);
        }
      }
    }
  };
  issue(0);                               // the first weights go out before the input is built
  stage_input<IN, WAVES * 64>(g, xs, &red[0][0]);

  float acc[NR] = {};
  for (int i0 = 0; i0 * WAVES + wid < n_ld; i0 += LPB) {
#pragma unroll
    for (int u = 0; u < kGemvU; ++u) {
      const int kb = ((i0 + u / NR) * WAVES + wid) * NB + j;
      if (kb < kbr) acc[u % NR] = dot8(wv[u], xs[kb * 2 + hh], acc[u % NR]);
    }
    if ((i0 + LPB) * WAVES + wid < n_ld) issue(i0 + LPB);
  }
  // lanes of one row: the NB blocks and the two column halves
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int m = RB; m < 64; m <<= 1) acc[r] += __shfl_xor(acc[r], m, 64);
  __syncthreads();                        // red[] held the norm partials
  if (lane < RB) {
#pragma unroll
    for (int r = 0; r < NR; ++r) red[wid][r * 32 + lane] = acc[r];
  }
  __syncthreads();
  if constexpr (OUT == OUT_QKV) {
    static_assert(RB % 2 == 0, "RoPE pairs stay in the workgroup");
    if (wid == 0) {
      float t = 0.f;
      if (lane < RB) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) t += red[w][lane];
      }
      const float o = __shfl_xor(t, 1, 64);   // the other row of the dim pair
      const int r = row0 + lane;
      const QkvOut& d = g.qkv;
      if (lane < RB && r < g.rows) {
        float v = t;
        if (r < d.qw + d.kvw) {                  // Q and K are rotated, V is not
          const float2 cs = d.rot[(r % d.head_dim) >> 1];
          v = (r & 1) ? o * cs.y + t * cs.x : t * cs.x - o * cs.y;
        }
        if (r < d.qw) {
          d.q[r] = f2bf(v);
        } else {
          const int e = r - d.qw;
          const bool isv = e >= d.kvw;
          const int64_t off = static_cast<int64_t>(d.layer) * d.cache.layer_stride +
                              paged_row(d.cache, d.pos) * d.kvw + (isv ? e - d.kvw : e);
          if (d.cache.fp8) {
            const float sc = isv ? d.cache.vs : d.cache.ks;
            static_cast<fp8_t*>(isv ? d.cache.v : d.cache.k)[off] =
                static_cast<fp8_t>(f32_to_fp8x4(v / sc, 0.f, 0.f, 0.f) & 0xFFu);
          } else {
            static_cast<bf16_t*>(isv ? d.cache.v : d.cache.k)[off] = f2bf(v);
          }
        }
      }
    }
  } else if (wid == 0 && lane < RB) {
    float t[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      t[r] = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) t[r] += red[w][r * 32 + lane];
    }
    if constexpr (OUT == OUT_SWIGLU) {
      // feature 32 b + lane: gate row 64 b + lane, up row 64 b + 32 + lane
      static_cast<bf16_t*>(g.y)[blockIdx.x * 32 + lane] = f2bf(silu_f(t[0]) * t[NR - 1]);
    } else {
      const int r = row0 + lane;
      if (r < g.rows) {
        // residual stream: (r1 + r2) + product, the order of the prefill's two residual adds
        float v = t[0];
        if (g.r1) v = (g.r1[r] + (g.r2 ? g.r2[r] : 0.f)) + v;
        static_cast<float*>(g.y)[r] = v;
      }
    }
  }
}

template <int IN, int OUT, int RB, int WAVES>
hipError_t gemv_launch(const GemvArgs& g, int n_wg, hipStream_t s) {
  gemv_packed_kernel<IN, OUT, RB, WAVES><<<n_wg, WAVES * 64, static_cast<size_t>(g.K) * 2, s>>>(g);
  return hipGetLastError();
}

template <int IN>
hipError_t gemv_pick(const GemvArgs& g, bool swiglu, hipStream_t s) {
  if (swiglu) return gemv_launch<IN, OUT_SWIGLU, 32, 8>(g, g.rows / 64, s);
  // the widest row share that still gives at least 512 workgroups; long rows (K >= 16384)
  // take whole 32-row blocks from 256 workgroups on (70B down product, 8192 x 28672:
  // 85.4 -> 81.5 us, 5.8 TB/s), since each workgroup then reads 1 KiB runs
  if ((g.rows + 31) / 32 >= 512) return gemv_launch<IN, OUT_F32, 32, 4>(g, (g.rows + 31) / 32, s);
  if ((g.rows + 31) / 32 >= 256 && g.K >= 16384) return gemv_launch<IN, OUT_F32, 32, 8>(g, (g.rows + 31) / 32, s);
  if ((g.rows + 15) / 16 >= 512) return gemv_launch<IN, OUT_F32, 16, 8>(g, (g.rows + 15) / 16, s);
  return gemv_launch<IN, OUT_F32, 8, 8>(g, (g.rows + 7) / 8, s);
}

}  // namespace

hipError_t launch_gemv_qkv(const void* w, int K, const void* x, const float* gain, float eps, int qw, int kvw,
                           int head_dim, const float2* rot, void* q, const PagedRef& cache_in, int layer, int pos,
                           hipStream_t s) {
  const int rows = qw + 2 * kvw;
  if (K % 16 != 0 || static_cast<int64_t>(K) * 2 > 64 * 1024 || head_dim % 8 != 0) return hipErrorInvalidValue;
  GemvArgs g{static_cast<const bf16_t*>(w), rows, K, x, nullptr, gain, eps, nullptr, nullptr, nullptr, {}};
  g.qkv = QkvOut{static_cast<bf16_t*>(q), rot, cache_in, layer, pos, qw, kvw, head_dim};
  g.qkv.cache.bs_shift = block_shift(cache_in.bs);
  // as gemv_pick: 16 rows per workgroup when that still gives 512 workgroups (70B:
  // 10240 x 8192, 46.7 -> 36.2 us: each workgroup also normalises the input vector
  // itself, so fewer, longer workgroups pay that less often)
  if ((rows + 15) / 16 >= 512) return gemv_launch<IN_NORM, OUT_QKV, 16, 8>(g, (rows + 15) / 16, s);
  return gemv_launch<IN_NORM, OUT_QKV, 8, 8>(g, (rows + 7) / 8, s);
}

hipError_t launch_gemv(int in_mode, bool swiglu_out, const void* w, int rows, int K, const void* x, const float* x2,
                       const float* gain, float eps, void* y, const float* r1, const float* r2, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % 16 != 0 || in_mode < 0 || in_mode > 2) return hipErrorInvalidValue;
  if (static_cast<int64_t>(K) * 2 > 64 * 1024) return hipErrorInvalidValue;   // the input vector must fit in LDS
  if (swiglu_out && rows % 64 != 0) return hipErrorInvalidValue;
  GemvArgs g{static_cast<const bf16_t*>(w), rows, K, x, x2, gain, eps, y, r1, r2, {}};
  switch (in_mode) {
    case 0: return gemv_pick<IN_PACKED>(g, swiglu_out, s);
    case 1: return gemv_pick<IN_NORM>(g, swiglu_out, s);
    default: return gemv_pick<IN_BF16>(g, swiglu_out, s);
  }
}

}  // namespace cb
