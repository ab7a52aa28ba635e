// Sparse-query causal attention over the paged blended cache.
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn), Fig. 5 -- the selected
// queries attend to every token: K/V of unselected positions come from the
// cache, those of the selected positions are the fresh ones already written
// there.  A query at position p sees keys at positions 0..p.
//
// bf16 path (gfx950 MFMA, v_mfma_f32_16x16x32_bf16): one workgroup = one KV
// head x a tile of query tokens; the G = Hq/Hkv query heads sharing the KV
// head are stacked so the tile has 64 query rows (64/G tokens x G heads) and
// each K/V block is read from HBM once for all of them.  Scores are computed
// transposed (S^T = K Q^T) so each lane owns one query column: the online
// softmax (fp32, exp2 with the max subtracted) needs no transpose, and the
// probabilities feed the P.V product (O^T = V^T P^T) straight from registers.
// K blocks are staged row-major in LDS, V blocks transposed.  Query tiles run
// longest-first (their rows are sorted by position).
#include "cb_internal.h"

namespace cb {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int KVB = 64;            // keys per block
constexpr int QROWS = 64;          // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int DH, int G>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int QT = QROWS / G;          // query tokens per tile
  constexpr int KP = DH + 8;             // K row pitch (bf16)
  constexpr int VP = KVB + 8;            // V^T row pitch (bf16)
  __shared__ __attribute__((aligned(16))) bf16_t Ks[KVB * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[DH * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n_tiles = (a.R + QT - 1) / QT;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x);   // longest first
  const int kvh = blockIdx.y;
  const int t0 = tile * QT;
  const int t_last = min(t0 + QT, a.R) - 1;
  const int kv_end = a.rowpos[t_last] + 1;                        // keys [0, kv_end)

  // this lane's query row: wave w owns tile rows 16w..16w+15; row r -> token r % QT, head r / QT
  const int qr = wid * 16 + (lane & 15);
  const int qtok = t0 + (qr % QT);
  const int qhead = kvh * G + qr / QT;
  const bool qvalid = qtok < a.R;
  const int qpos = qvalid ? a.rowpos[qtok] : kv_end - 1;
  const int kgrp = lane >> 4;            // 0..3

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[q][32*ks + 8*kgrp .. +7]
  bf16x8_t qf[DH / 32];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(qvalid ? qtok : t_last) * a.ldq +
                       qhead * DH + 8 * kgrp;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * ks);
  }

  f32x4_t o[DH / 16];
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;   // this lane's partial row sum
  const float sc = a.scale * kLog2e;

  const bf16_t* kbase = static_cast<const bf16_t*>(a.cache.k) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.cache.v) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const int width = a.n_kv_heads * DH;

  for (int j0 = 0; j0 < kv_end; j0 += KVB) {
    // ---- stage K (row-major) and V (transposed) for keys j0 .. j0+63 ----
    constexpr int CPR = DH / 8;              // 16-byte chunks per key row
    for (int c = tid; c < KVB * CPR; c += 256) {
      const int r = c / CPR, e = (c % CPR) * 8;
      const int p = j0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (p < kv_end) {
        const int64_t off = paged_row(a.cache.bt, a.cache.bs, p) * width + kvh * DH + e;
        kv = *reinterpret_cast<const uint4*>(kbase + off);
        vv = *reinterpret_cast<const uint4*>(vbase + off);
      }
      *reinterpret_cast<uint4*>(&Ks[r * KP + e]) = kv;
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        Vt[(e + 2 * h) * VP + r] = static_cast<bf16_t>(w[h] & 0xFFFFu);
        Vt[(e + 2 * h + 1) * VP + r] = static_cast<bf16_t>(w[h] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T tiles: 4 x (16 keys x 16 queries) ----
    f32x4_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&Ks[(16 * t + (lane & 15)) * KP + 32 * ks + 8 * kgrp]);
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[t], 0, 0, 0);
      }
    }
    // lane holds s[t][i] for key j0 + 16t + 4*kgrp + i, query column lane&15
    float mblk = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = j0 + 16 * t + 4 * kgrp + i;
        const float v = (key <= qpos) ? s[t][i] * sc : -INFINITY;
        s[t][i] = v;
        mblk = fmaxf(mblk, v);
      }
    mblk = fmaxf(mblk, __shfl_xor(mblk, 16, 64));
    mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
    const float m_new = fmaxf(m_run, mblk);          // finite: key 0 <= qpos always
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8_t pf[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s[t][i] - m_new);
        psum += p;
        pf[t >> 1][(t & 1) * 4 + i] = static_cast<__bf16>(p);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[t] *= alpha;

    // ---- O^T += V^T P^T: k-slot (kgrp, j) <-> key 32*s2 + (j<4 ? 4kgrp+j : 16+4kgrp+j-4) ----
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16_t* vr = &Vt[(16 * dt + (lane & 15)) * VP + 32 * s2 + 4 * kgrp];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
        const uint4 packed = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, packed);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[s2], o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    bf16_t* op = static_cast<bf16_t*>(a.o) + static_cast<int64_t>(qtok) * a.ldo + qhead * DH;
    // o[dt][i] = O[q][16*dt + 4*kgrp + i]
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(o[dt][0] * inv)) | (static_cast<uint32_t>(f2bf(o[dt][1] * inv)) << 16);
      w.y = static_cast<uint32_t>(f2bf(o[dt][2] * inv)) | (static_cast<uint32_t>(f2bf(o[dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + 16 * dt + 4 * kgrp) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per (query row, query head), keys in blocks of 64 with
// an online softmax; each lane owns head_dim/64 output dims (head_dim <= 256).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[256];
  __shared__ float ps[64];
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int dh = a.head_dim;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int kvh = h / G;
  const int qpos = a.rowpos[row];
  const float* q = static_cast<const float*>(a.q) + static_cast<int64_t>(row) * a.ldq + h * dh;
  for (int e = lane; e < dh; e += 64) qs[e] = q[e];
  __syncthreads();
  const int width = a.n_kv_heads * dh;
  const float* kb = static_cast<const float*>(a.cache.k) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const float* vb = static_cast<const float*>(a.cache.v) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  float m_run = -INFINITY, l_run = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 <= qpos; j0 += 64) {
    const int j = j0 + lane;
    float sv = -INFINITY;
    if (j <= qpos) {
      const float* kr = kb + paged_row(a.cache.bt, a.cache.bs, j) * width + kvh * dh;
      float d = 0.f;
      for (int e = 0; e < dh; ++e) d += qs[e] * kr[e];
      sv = d * a.scale;
    }
    float mb = sv;
    for (int m = 32; m >= 1; m >>= 1) mb = fmaxf(mb, __shfl_xor(mb, m, 64));
    const float m_new = fmaxf(m_run, mb);
    const float alpha = expf(m_run - m_new);
    const float p = (j <= qpos) ? expf(sv - m_new) : 0.f;
    float psum = p;
    for (int m = 32; m >= 1; m >>= 1) psum += __shfl_xor(psum, m, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    ps[lane] = p;
    __syncthreads();
    const int nj = min(64, qpos + 1 - j0);
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      if (e >= dh) break;
      float s = acc[c] * alpha;
      for (int jj = 0; jj < nj; ++jj) {
        const float* vr = vb + paged_row(a.cache.bt, a.cache.bs, j0 + jj) * width + kvh * dh;
        s += ps[jj] * vr[e];
      }
      acc[c] = s;
    }
    __syncthreads();
  }
  float* o = static_cast<float*>(a.o) + static_cast<int64_t>(row) * a.ldo + h * dh;
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    if (e < dh) o[e] = acc[c] / l_run;
  }
}

template <int DH, int G>
hipError_t run_bf16(const AttnArgs& a, hipStream_t s) {
  constexpr int QT = QROWS / G;
  const int n_tiles = (a.R + QT - 1) / QT;
  attn_bf16_kernel<DH, G><<<dim3(n_tiles, a.n_kv_heads), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(cb_dtype dt, int n_q_heads, int n_kv_heads, int head_dim) {
  if (n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return false;
  const int G = n_q_heads / n_kv_heads;
  if (dt == CB_F32) return head_dim <= 256 && head_dim % 2 == 0;
  return (head_dim == 64 || head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_attention(cb_dtype dt, const AttnArgs& a, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  if (dt == CB_F32) {
    attn_f32_kernel<<<dim3(a.R, a.n_q_heads), 64, 0, s>>>(a);
    return hipGetLastError();
  }
  const int G = a.n_q_heads / a.n_kv_heads;
#define CB_ATTN_CASE(D, GG) \
  if (a.head_dim == D && G == GG) return run_bf16<D, GG>(a, s);
  CB_ATTN_CASE(128, 1) CB_ATTN_CASE(128, 2) CB_ATTN_CASE(128, 4) CB_ATTN_CASE(128, 8) CB_ATTN_CASE(128, 16)
  CB_ATTN_CASE(64, 1) CB_ATTN_CASE(64, 2) CB_ATTN_CASE(64, 4) CB_ATTN_CASE(64, 8) CB_ATTN_CASE(64, 16)
#undef CB_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace cb
