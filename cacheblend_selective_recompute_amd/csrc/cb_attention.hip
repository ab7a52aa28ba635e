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
#include <algorithm>

#include "cb_internal.h"

namespace cb {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int KVB = 64;            // keys per block
constexpr int kBtCache = 4096;     // block-table entries a workgroup stages in LDS
constexpr int QROWS = 64;          // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;

template <int DH, int G, bool STAGED>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, int n_splits, int ksplit) {
  constexpr int QT = QROWS / G;          // query tokens per tile
  constexpr int KP = DH + 8;             // K row pitch (bf16): 16 rows of a fragment read hit distinct banks
  constexpr int VP = KVB + 4;            // V^T row pitch (bf16)
  constexpr int CPR = DH / 8;            // 16-byte chunks per key row
  constexpr int KCH = KVB * CPR / 256;   // K chunks per thread per block
  static_assert(KVB * CPR == 256 * KCH, "K staging");
  static_assert((KVB / 4) * CPR == 256 || (KVB / 4) * CPR == 128, "V staging");
  constexpr int VTHREADS = (KVB / 4) * CPR;    // threads that stage V (4 keys x 8 dims each)
  __shared__ __attribute__((aligned(16))) bf16_t Ks[KVB * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[DH * VP];
  __shared__ int32_t btab[kBtCache];     // block-table entries of this workgroup's key range

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n_tiles = (a.R + QT - 1) / QT;
  const int split = blockIdx.x % n_splits;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x / n_splits);   // longest first
  const int kvh = blockIdx.y;
  const int t0 = tile * QT;
  const int t_last = min(t0 + QT, a.R) - 1;
  const int kv_end = a.rowpos[t_last] + 1;                                   // keys [0, kv_end)
  const int j_begin = split * ksplit;
  const int j_end = min(kv_end, j_begin + ksplit);
  if (j_begin >= j_end) return;                                              // uniform per workgroup

  // this lane's query row: wave w owns tile rows 16w..16w+15; row r -> token r % QT, head r / QT
  const int qr = wid * 16 + (lane & 15);
  const int qtok = t0 + (qr % QT);
  const int qhead = kvh * G + qr / QT;
  const bool qvalid = qtok < a.R;
  const int qpos = qvalid ? a.rowpos[qtok] : kv_end - 1;
  const int qpos_min = a.rowpos[t0];     // rows are sorted: the tile's first row sees the fewest keys
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

  // page-table entries of keys [j_begin, j_end) staged once in LDS (the launcher
  // sizes the key splits so they fit), so K/V loads never wait on a table load
  const int bs = a.cache.bs;
  const int sh = a.cache.bs_shift;
  const int blk0 = j_begin / bs;
  const int nblk = (j_end - 1) / bs - blk0 + 1;
  if constexpr (STAGED) {
    for (int i = tid; i < nblk; i += 256) btab[i] = a.cache.bt[blk0 + i];
    __syncthreads();
  }
  auto krow = [&](int p) -> int64_t {
    const int b = sh >= 0 ? (p >> sh) : p / bs;
    const int e = STAGED ? btab[b - blk0] : a.cache.bt[b];
    return sh >= 0 ? (static_cast<int64_t>(e) << sh) + (p & (bs - 1)) : static_cast<int64_t>(e) * bs + (p - b * bs);
  };
  const bf16_t* kbase = static_cast<const bf16_t*>(a.cache.k) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.cache.v) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const int width = a.n_kv_heads * DH;

  // staging roles: K chunk c = tid + 256*u -> key c / CPR, dims (c % CPR)*8;
  // V: thread tid < VTHREADS takes keys 4*(tid % 16) .. +3, dims 8*(tid / 16) .. +7,
  // so the 16 lanes of an LDS write phase cover one V^T row's 64 keys (no bank conflicts)
  const int vkey = 4 * (tid % (KVB / 4));
  const int vdim = 8 * (tid / (KVB / 4));
  uint4 kreg[KCH], vreg[4];
  auto gload = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + 256 * u;
      const int p = j0 + c / CPR;
      kreg[u] = make_uint4(0, 0, 0, 0);
      if (p < j_end)
        kreg[u] = *reinterpret_cast<const uint4*>(kbase + krow(p) * width + kvh * DH + (c % CPR) * 8);
    }
    if (tid < VTHREADS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = j0 + vkey + i;
        vreg[i] = make_uint4(0, 0, 0, 0);
        if (p < j_end)
          vreg[i] = *reinterpret_cast<const uint4*>(vbase + krow(p) * width + kvh * DH + vdim);
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<uint4*>(&Ks[(c / CPR) * KP + (c % CPR) * 8]) = kreg[u];
    }
    if (tid < VTHREADS) {
      // V^T[vdim + e][vkey .. vkey+3] as one 8-byte word per dim
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint2 lo, hi;
        lo.x = (w0[h] & 0xFFFFu) | (w1[h] << 16);
        lo.y = (w2[h] & 0xFFFFu) | (w3[h] << 16);
        hi.x = (w0[h] >> 16) | (w1[h] & 0xFFFF0000u);
        hi.y = (w2[h] >> 16) | (w3[h] & 0xFFFF0000u);
        *reinterpret_cast<uint2*>(&Vt[(vdim + 2 * h) * VP + vkey]) = lo;
        *reinterpret_cast<uint2*>(&Vt[(vdim + 2 * h + 1) * VP + vkey]) = hi;
      }
    }
  };

  gload(j_begin);
  for (int j0 = j_begin; j0 < j_end; j0 += KVB) {
    lstore();
    __syncthreads();
    if (j0 + KVB < j_end) gload(j0 + KVB);     // next block in flight during the math

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
    // lane holds s[t][i] for key j0 + 16t + 4*kgrp + i, query column lane&15.
    // Only blocks that reach past the tile's first row or the split end need a mask.
    if (j0 + KVB - 1 > qpos_min || j0 + KVB > j_end) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j0 + 16 * t + 4 * kgrp + i;
          if (key > qpos || key >= j_end) s[t][i] = -INFINITY;
        }
    }
    float mblk = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      mblk = fmaxf(fmaxf(mblk, fmaxf(s[t][0], s[t][1])), fmaxf(s[t][2], s[t][3]));
    mblk = fmaxf(mblk, __shfl_xor(mblk, 16, 64));
    mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
    const float m_new = fmaxf(m_run, mblk * sc);             // running max in scaled log2 units
    // a row with no visible key yet keeps m = -inf; guard the exponent base
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    // rescale the output only when some row's maximum moved (wave vote)
    if (__any(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DH / 16; ++t) o[t] *= alpha;
    }
    m_run = m_new;
    float psum = 0.f;
    bf16x8_t pf[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float p4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p4[i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], sc, -m_use));
        psum += p4[i];
      }
      const bf16x2_t lo = __builtin_convertvector(f32x2_t{p4[0], p4[1]}, bf16x2_t);
      const bf16x2_t hi = __builtin_convertvector(f32x2_t{p4[2], p4[3]}, bf16x2_t);
      pf[t >> 1][(t & 1) * 4 + 0] = lo[0];
      pf[t >> 1][(t & 1) * 4 + 1] = lo[1];
      pf[t >> 1][(t & 1) * 4 + 2] = hi[0];
      pf[t >> 1][(t & 1) * 4 + 3] = hi[1];
    }
    l_run += psum;

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
  if (!qvalid) return;
  if (n_splits == 1) {
    const float inv = 1.0f / l_tot;
    bf16_t* ob = static_cast<bf16_t*>(a.o);
    const int KO = a.n_q_heads * DH;
    // o[dt][i] = O[q][16*dt + 4*kgrp + i]; written fragment-major (4 consecutive columns = 8 bytes)
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(o[dt][0] * inv)) | (static_cast<uint32_t>(f2bf(o[dt][1] * inv)) << 16);
      w.y = static_cast<uint32_t>(f2bf(o[dt][2] * inv)) | (static_cast<uint32_t>(f2bf(o[dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(ob + pk_off(qtok, qhead * DH + 16 * dt + 4 * kgrp, KO)) = w;
    }
  } else {
    // unnormalised partial for (split, row, head); m in log2 units
    const int64_t pr = (static_cast<int64_t>(split) * a.R + qtok) * a.n_q_heads + qhead;
    float* op = a.part_o + pr * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *reinterpret_cast<float4*>(op + 16 * dt + 4 * kgrp) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (kgrp == 0) a.part_ml[pr] = make_float2(m_run, l_tot);
  }
}

// Merge the split-KV partials of one (row, q head) per wave, in split order.
template <int DH>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int n_splits, int ksplit, int QT) {
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);   // row * Hq + head
  const int lane = threadIdx.x & 63;
  if (idx >= a.R * a.n_q_heads) return;
  const int row = idx / a.n_q_heads;
  const int head = idx % a.n_q_heads;
  const int t_last = min((row / QT + 1) * QT, a.R) - 1;
  const int kv_end = a.rowpos[t_last] + 1;
  const int ns = min(n_splits, (kv_end + ksplit - 1) / ksplit);
  float M = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, a.part_ml[(static_cast<int64_t>(sp) * a.R + row) * a.n_q_heads + head].x);
  constexpr int PER = DH / 64;
  float acc[PER] = {};
  float lsum = 0.f;
  for (int sp = 0; sp < ns; ++sp) {
    const int64_t pr = (static_cast<int64_t>(sp) * a.R + row) * a.n_q_heads + head;
    const float2 ml = a.part_ml[pr];
    const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
    lsum += w * ml.y;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += w * a.part_o[pr * DH + lane * PER + e];
  }
  const float inv = 1.0f / lsum;
  bf16_t* ob = static_cast<bf16_t*>(a.o);
  const int KO = a.n_q_heads * DH;
#pragma unroll
  for (int e = 0; e < PER; ++e) ob[pk_off(row, head * DH + lane * PER + e, KO)] = f2bf(acc[e] * inv);
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
  const int base = n_tiles * a.n_kv_heads;
  const int kv_blocks = (a.kv_bound + KVB - 1) / KVB;
  // split the keys only when the (tile, head) grid cannot fill the chip
  int n_splits = 1;
  if (base < 512 && a.part_o != nullptr) {
    n_splits = std::min(kAttnMaxSplits, std::max(1, (768 + base - 1) / base));
    n_splits = std::min(n_splits, kv_blocks);
    if (static_cast<int64_t>(n_splits) * a.R * a.n_q_heads > kAttnPartialRows) n_splits = 1;
  }
  const int ksplit = ((kv_blocks + n_splits - 1) / n_splits) * KVB;
  // workgroups stage the table entries of their key range in LDS when they fit
  if (ksplit / a.cache.bs + 2 <= kBtCache)
    attn_bf16_kernel<DH, G, true><<<dim3(n_tiles * n_splits, a.n_kv_heads), 256, 0, s>>>(a, n_splits, ksplit);
  else
    attn_bf16_kernel<DH, G, false><<<dim3(n_tiles * n_splits, a.n_kv_heads), 256, 0, s>>>(a, n_splits, ksplit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int pairs = a.R * a.n_q_heads;
  attn_combine_kernel<DH><<<(pairs + 3) / 4, 256, 0, s>>>(a, n_splits, ksplit, QT);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(cb_dtype dt, int n_q_heads, int n_kv_heads, int head_dim) {
  if (n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return false;
  const int G = n_q_heads / n_kv_heads;
  if (dt == CB_F32) return head_dim <= 256 && head_dim % 2 == 0;
  return (head_dim == 64 || head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_attention(cb_dtype dt, const AttnArgs& a_in, hipStream_t s) {
  if (a_in.R == 0) return hipSuccess;
  AttnArgs a = a_in;
  a.cache.bs_shift = block_shift(a.cache.bs);   // derived here so it always matches bs
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
