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
#include <type_traits>

#include "cb_internal.h"

namespace cb {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

constexpr int KVB = 64;            // keys per block
constexpr int kBtCache = 4096;     // block-table entries a workgroup stages in LDS
constexpr float kLog2e = 1.4426950408889634f;

// F8: the cache holds FP8 E4M3 elements; they widen exactly to bf16 when staged
// into LDS, the K scale joins the softmax scale and the V scale the output.
template <int DH, int G, bool STAGED, int NG, bool F8 = false>
__global__ __launch_bounds__(256, NG == 1 ? 3 : 2) void attn_bf16_kernel(AttnArgs a, int n_splits, int ksplit) {
  constexpr int QROWS = 64 * NG;         // query rows per workgroup (NG groups of 16 per wave)
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

  // this lane's query rows: group g of wave w owns tile rows 16 (w NG + g) .. +15;
  // row r -> token r % QT, head r / QT
  const int kgrp = lane >> 4;            // 0..3
  int qtok[NG], qhead[NG], qpos[NG];
  bool qvalid[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int qr = (wid * NG + g) * 16 + (lane & 15);
    qtok[g] = t0 + (qr % QT);
    qhead[g] = kvh * G + qr / QT;
    qvalid[g] = qtok[g] < a.R;
    qpos[g] = qvalid[g] ? a.rowpos[qtok[g]] : kv_end - 1;
  }
  const int qpos_min = a.rowpos[t0];     // rows are sorted: the tile's first row sees the fewest keys

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[q][32*ks + 8*kgrp .. +7]
  bf16x8_t qf[NG][DH / 32];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(qvalid[g] ? qtok[g] : t_last) * a.ldq +
                       qhead[g] * DH + 8 * kgrp;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) qf[g][ks] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * ks);
  }
  f32x4_t o[NG][DH / 16];
  float m_run[NG], l_run[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[g][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;      // this lane's partial row sum
  }
  const float sc = a.scale * kLog2e * (F8 ? a.cache.ks : 1.0f);

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
  using E = typename std::conditional<F8, fp8_t, bf16_t>::type;   // cache element
  const E* kbase = static_cast<const E*>(a.cache.k) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const E* vbase = static_cast<const E*>(a.cache.v) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const int width = a.n_kv_heads * DH;

  // staging roles: K chunk c = tid + 256*u -> key c / CPR, dims (c % CPR)*8;
  // V: thread tid < VTHREADS takes keys 4*(tid % 16) .. +3, dims 8*(tid / 16) .. +7,
  // so the 16 lanes of an LDS write phase cover one V^T row's 64 keys (no bank conflicts)
  const int vkey = 4 * (tid % (KVB / 4));
  const int vdim = 8 * (tid / (KVB / 4));
  // 8 elements per chunk: 16 bytes of bf16, or 8 bytes of FP8 widened in lstore
  using R = typename std::conditional<F8, uint2, uint4>::type;
  R kraw[KCH], vraw[4];
  uint4 kreg[KCH], vreg[4];
  auto gload = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + 256 * u;
      const int p = j0 + c / CPR;
      kraw[u] = R{};
      if (p < j_end)
        kraw[u] = *reinterpret_cast<const R*>(kbase + krow(p) * width + kvh * DH + (c % CPR) * 8);
    }
    if (tid < VTHREADS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = j0 + vkey + i;
        vraw[i] = R{};
        if (p < j_end)
          vraw[i] = *reinterpret_cast<const R*>(vbase + krow(p) * width + kvh * DH + vdim);
      }
    }
  };
  auto widen = [](const R& r) -> uint4 {
    if constexpr (F8) {
      float f[8];
      fp8x4_to_f32(r.x, f);
      fp8x4_to_f32(r.y, f + 4);
      return make_uint4(fp8x2_to_bf16x2(f[0], f[1]), fp8x2_to_bf16x2(f[2], f[3]), fp8x2_to_bf16x2(f[4], f[5]),
                        fp8x2_to_bf16x2(f[6], f[7]));
    } else {
      return r;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int u = 0; u < KCH; ++u) kreg[u] = widen(kraw[u]);
    if (tid < VTHREADS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = widen(vraw[i]);
    }
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

    // ---- S^T tiles: 4 x (16 keys x 16 queries) per group; each K fragment serves every group ----
    f32x4_t s[NG][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int g = 0; g < NG; ++g) s[g][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&Ks[(16 * t + (lane & 15)) * KP + 32 * ks + 8 * kgrp]);
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[g][ks], s[g][t], 0, 0, 0);
      }
    }
    // lane holds s[g][t][i] for key j0 + 16t + 4*kgrp + i, query column lane&15 of group g.
    // Only blocks that reach past the tile's first row or the split end need a mask.
    const bool edge = j0 + KVB - 1 > qpos_min || j0 + KVB > j_end;
    bf16x8_t pf[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (edge) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j0 + 16 * t + 4 * kgrp + i;
            if (key > qpos[g] || key >= j_end) s[g][t][i] = -INFINITY;
          }
      }
      float mblk = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        mblk = fmaxf(fmaxf(mblk, fmaxf(s[g][t][0], s[g][t][1])), fmaxf(s[g][t][2], s[g][t][3]));
      mblk = fmaxf(mblk, __shfl_xor(mblk, 16, 64));
      mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
      const float m_new = fmaxf(m_run[g], mblk * sc);          // running max in scaled log2 units
      // a row with no visible key yet keeps m = -inf; guard the exponent base
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      // rescale the output only when some row's maximum moved (wave vote)
      if (__any(m_new != m_run[g])) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_use);
        l_run[g] *= alpha;
#pragma unroll
        for (int t = 0; t < DH / 16; ++t) o[g][t] *= alpha;
      }
      m_run[g] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p4[i] = __builtin_amdgcn_exp2f(fmaf(s[g][t][i], sc, -m_use));
          psum += p4[i];
        }
        const bf16x2_t lo = __builtin_convertvector(f32x2_t{p4[0], p4[1]}, bf16x2_t);
        const bf16x2_t hi = __builtin_convertvector(f32x2_t{p4[2], p4[3]}, bf16x2_t);
        pf[g][t >> 1][(t & 1) * 4 + 0] = lo[0];
        pf[g][t >> 1][(t & 1) * 4 + 1] = lo[1];
        pf[g][t >> 1][(t & 1) * 4 + 2] = hi[0];
        pf[g][t >> 1][(t & 1) * 4 + 3] = hi[1];
      }
      l_run[g] += psum;
    }

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
#pragma unroll
        for (int g = 0; g < NG; ++g) o[g][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[g][s2], o[g][dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float l_tot = l_run[g];
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!qvalid[g]) continue;
    if (n_splits == 1 || kv_end <= ksplit) {   // the tile's keys lie in split 0: final output
      const float inv = (F8 ? a.cache.vs : 1.0f) / l_tot;
      bf16_t* ob = static_cast<bf16_t*>(a.o);
      const int KO = a.n_q_heads * DH;
      // o[g][dt][i] = O[q][16*dt + 4*kgrp + i]; written fragment-major (4 consecutive columns = 8 bytes)
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        uint2 w;
        w.x = static_cast<uint32_t>(f2bf(o[g][dt][0] * inv)) | (static_cast<uint32_t>(f2bf(o[g][dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f2bf(o[g][dt][2] * inv)) | (static_cast<uint32_t>(f2bf(o[g][dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(ob + pk_off(qtok[g], qhead[g] * DH + 16 * dt + 4 * kgrp, KO)) = w;
      }
    } else {
      // unnormalised partial for (split, row, head); m in log2 units
      const int64_t pr = (static_cast<int64_t>(split) * a.R + qtok[g]) * a.n_q_heads + qhead[g];
      float* op = a.part_o + pr * DH;
      const float vsc = F8 ? a.cache.vs : 1.0f;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        *reinterpret_cast<float4*>(op + 16 * dt + 4 * kgrp) =
            make_float4(o[g][dt][0] * vsc, o[g][dt][1] * vsc, o[g][dt][2] * vsc, o[g][dt][3] * vsc);
      if (kgrp == 0) a.part_ml[pr] = make_float2(m_run[g], l_tot);
    }
  }
}

// ---------------------------------------------------------------------------
// head_dim 128: K and V blocks are copied global -> LDS by buffer loads that
// write LDS directly (no VGPR staging), 16-byte chunks of each 256-byte key
// row placed at swizzled slots so both fragment reads are free of bank
// conflicts; V^T fragments come straight out of the key-major V block with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Two stages: block j+1 is
// in flight while block j is multiplied.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void attn_copy(uint32_t lds, __amdgpu_buffer_rsrc_t rsrc, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

template <int G, bool STAGED, int NG>
__global__ __launch_bounds__(256, NG == 1 ? 3 : 2) void attn_dma_kernel(AttnArgs a, int n_splits, int ksplit) {
  constexpr int DH = 128;
  constexpr int QROWS = 64 * NG;
  constexpr int QT = QROWS / G;
  constexpr int kBlk = KVB * DH * 2;     // bytes of one K (or V) block: 64 rows x 256 B
  constexpr int kBt = 1024;              // staged block-table entries
  __shared__ __attribute__((aligned(1024))) uint8_t kv[2][2 * kBlk];   // [stage][K | V]
  __shared__ int32_t btab[kBt];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n_tiles = (a.R + QT - 1) / QT;
  const int split = blockIdx.x % n_splits;
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x / n_splits);   // longest first
  const int kvh = blockIdx.y;
  const int t0 = tile * QT;
  const int t_last = min(t0 + QT, a.R) - 1;
  const int kv_end = a.rowpos[t_last] + 1;
  const int j_begin = split * ksplit;
  const int j_end = min(kv_end, j_begin + ksplit);
  if (j_begin >= j_end) return;

  const int kgrp = lane >> 4;
  int qtok[NG], qhead[NG], qpos[NG];
  bool qvalid[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int qr = (wid * NG + g) * 16 + (lane & 15);
    qtok[g] = t0 + (qr % QT);
    qhead[g] = kvh * G + qr / QT;
    qvalid[g] = qtok[g] < a.R;
    qpos[g] = qvalid[g] ? a.rowpos[qtok[g]] : kv_end - 1;
  }
  const int qpos_min = a.rowpos[t0];
  bf16x8_t qf[NG][DH / 32];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(qvalid[g] ? qtok[g] : t_last) * a.ldq +
                       qhead[g] * DH + 8 * kgrp;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) qf[g][ks] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * ks);
  }
  f32x4_t o[NG][DH / 16];
  float m_run[NG], l_run[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[g][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
  }
  const float sc = a.scale * kLog2e;

  const int bs = a.cache.bs;
  const int sh = a.cache.bs_shift;
  const int blk0 = j_begin / bs;
  if constexpr (STAGED) {
    const int nblk = (j_end - 1) / bs - blk0 + 1;
    for (int i = tid; i < nblk; i += 256) btab[i] = a.cache.bt[blk0 + i];
    __syncthreads();
  }
  auto krow = [&](int p) -> int {
    const int b = sh >= 0 ? (p >> sh) : p / bs;
    const int e = STAGED ? btab[b - blk0] : a.cache.bt[b];
    return sh >= 0 ? (e << sh) + (p & (bs - 1)) : e * bs + (p - b * bs);
  };
  const int width = a.n_kv_heads * DH;
  const bf16_t* kbase = static_cast<const bf16_t*>(a.cache.k) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.cache.v) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  // the launcher guarantees the layer's pool spans < 2^31 bytes
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kbase), static_cast<short>(0),
                                                                      0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vbase), static_cast<short>(0),
                                                                      0x7fffffff, 0x00020000);
  // copy u (0..3) of this wave: keys 4 (4 wid + u) + lane / 16 of the block, LDS slot lane % 16
  // of the key row; K slot p holds chunk p ^ (key % 16), V slot p chunk p ^ 2 (key % 8)
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(&kv[0][0])));
  auto issue = [&](int jb, int stage) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kr = 4 * (4 * wid + u) + (lane >> 4);
      const int key = jb + kr;
      const int slot = lane & 15;
      int ko = static_cast<int>(0x80000000u), vo = static_cast<int>(0x80000000u);   // past the range: zeros
      if (key < j_end) {
        const int rowb = krow(key) * width * 2 + kvh * DH * 2;
        ko = rowb + ((slot ^ (key & 15)) << 4);
        vo = rowb + ((slot ^ ((key & 7) << 1)) << 4);
      }
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + stage * (2 * kBlk) + (4 * wid + u) * 1024);
      attn_copy(dst, rk, ko);
      attn_copy(dst + kBlk, rv, vo);
    }
  };

  // per-lane LDS byte offsets of the fragment reads inside a stage (block-relative keys):
  // K fragment (t, ks): key 16 t + lane % 16, chunk 4 ks + kgrp at slot chunk ^ (key % 16);
  // V^T source of (dt, s2, h): key 32 s2 + 16 h + 4 kgrp + sl / 4, dims 16 dt + 4 (sl % 4)
  int koff[DH / 32], voffs[DH / 16];
  {
    const int kk = lane & 15;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) koff[ks] = kk * 256 + (((4 * ks + kgrp) ^ kk) << 4);
    const int sl = lane & 15;
    const int vkey = 4 * kgrp + (sl >> 2);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const int d = 16 * dt + 4 * (sl & 3);
      voffs[dt] = vkey * 256 + (((d >> 3) ^ ((vkey & 7) << 1)) << 4) + ((d & 7) << 1);
    }
  }
  // one 64-key block held in LDS stage `stage` (a constant at both call sites, so
  // every LDS address is a per-lane base plus an immediate offset)
  auto block = [&](int j0, int stage) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of block j0 have landed
    __syncthreads();                      // ... everyone's; block j0 - 64 is no longer read
    if (j0 + KVB < j_end) issue(j0 + KVB, stage ^ 1);
    const uint8_t* Kb = kv[stage];
    const uint8_t* Vb = kv[stage] + kBlk;

    f32x4_t s[NG][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int g = 0; g < NG; ++g) s[g][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(Kb + koff[ks] + t * (16 * 256));
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[g][ks], s[g][t], 0, 0, 0);
      }
    }
    const bool edge = j0 + KVB - 1 > qpos_min || j0 + KVB > j_end;
    bf16x8_t pf[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (edge) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j0 + 16 * t + 4 * kgrp + i;
            if (key > qpos[g] || key >= j_end) s[g][t][i] = -INFINITY;
          }
      }
      float mblk = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        mblk = fmaxf(fmaxf(mblk, fmaxf(s[g][t][0], s[g][t][1])), fmaxf(s[g][t][2], s[g][t][3]));
      mblk = fmaxf(mblk, __shfl_xor(mblk, 16, 64));
      mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
      // the reference max moves only when some row's block max exceeds it by more than
      // 2^8 in exp2 units, so exp2 of every score stays <= 256 and rescaling is rare
      const float m_blk = mblk * sc;
      if (__any(m_blk > m_run[g] + 8.f)) {
        const float m_new = fmaxf(m_run[g], m_blk);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[g] - m_new);
        l_run[g] *= alpha;
#pragma unroll
        for (int t = 0; t < DH / 16; ++t) o[g][t] *= alpha;
        m_run[g] = m_new;
      }
      const float m_use = (m_run[g] == -INFINITY) ? 0.f : m_run[g];
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p4[i] = __builtin_amdgcn_exp2f(fmaf(s[g][t][i], sc, -m_use));
          psum += p4[i];
        }
        const bf16x2_t lo = __builtin_convertvector(f32x2_t{p4[0], p4[1]}, bf16x2_t);
        const bf16x2_t hi = __builtin_convertvector(f32x2_t{p4[2], p4[3]}, bf16x2_t);
        pf[g][t >> 1][(t & 1) * 4 + 0] = lo[0];
        pf[g][t >> 1][(t & 1) * 4 + 1] = lo[1];
        pf[g][t >> 1][(t & 1) * 4 + 2] = hi[0];
        pf[g][t >> 1][(t & 1) * 4 + 3] = hi[1];
      }
      l_run[g] += psum;
    }

    // O^T += V^T P^T.  k-slot 8 kgrp + j of P^T holds key 32 s2 + 16 (j / 4) + 4 kgrp + j % 4; the
    // transposing read gives lane (group kg, index i) element e from source lane 4 e + i / 4 of
    // its 16-lane group, column i % 4, so source lane s points at key 32 s2 + 16 h + 4 kg + s / 4,
    // dims 16 dt + 4 (s % 4) .. +3
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        s16x4_t half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* src = Vb + voffs[dt] + (32 * s2 + 16 * h) * 256;
          half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(const __attribute__((address_space(3))) void*)(src));
        }
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int g = 0; g < NG; ++g) o[g][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[g][s2], o[g][dt], 0, 0, 0);
      }
    }
  };
  issue(j_begin, 0);
  for (int j0 = j_begin; j0 < j_end; j0 += 2 * KVB) {
    block(j0, 0);
    if (j0 + KVB < j_end) block(j0 + KVB, 1);
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float l_tot = l_run[g];
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!qvalid[g]) continue;
    if (n_splits == 1 || kv_end <= ksplit) {   // the tile's keys lie in split 0: final output
      const float inv = 1.0f / l_tot;
      bf16_t* ob = static_cast<bf16_t*>(a.o);
      const int KO = a.n_q_heads * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        uint2 w;
        w.x = static_cast<uint32_t>(f2bf(o[g][dt][0] * inv)) | (static_cast<uint32_t>(f2bf(o[g][dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f2bf(o[g][dt][2] * inv)) | (static_cast<uint32_t>(f2bf(o[g][dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(ob + pk_off(qtok[g], qhead[g] * DH + 16 * dt + 4 * kgrp, KO)) = w;
      }
    } else {
      const int64_t pr = (static_cast<int64_t>(split) * a.R + qtok[g]) * a.n_q_heads + qhead[g];
      float* op = a.part_o + pr * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        *reinterpret_cast<float4*>(op + 16 * dt + 4 * kgrp) = make_float4(o[g][dt][0], o[g][dt][1], o[g][dt][2], o[g][dt][3]);
      if (kgrp == 0) a.part_ml[pr] = make_float2(m_run[g], l_tot);
    }
  }
}

// Leaner variant of the LDS-DMA kernel, for pages of 16 or more keys (a power of
// two).  Per block and wave it trims the vector work that otherwise outweighs
// the matrix work:
//  * row sums of P come from the matrix cores (an all-ones A operand against the
//    same P^T fragments as the PV product), so every lane ends with the full sum
//    of its query column and no adds or shuffles are spent on them;
//  * each lane compares its own block maximum with the row's threshold
//    (reference max + 8, in score units) and the wave votes; only when some score
//    crosses it does the wave reduce the block maxima across lanes and move the
//    reference (rescaling O and the sums);
//  * the 16 keys a wave copies share a page, so one block-table entry per wave
//    and block gives every copy address, and that entry is fetched a block ahead.
// ---------------------------------------------------------------------------
// CONTIG: the keys are one contiguous bf16 run per layer (the widened copy of an
// FP8 layer, see kv_widen_fp8_kernel); the V scale of that cache then multiplies
// the output.
template <int G, int NG, bool CONTIG = false>
__global__ __launch_bounds__(256, NG == 1 ? 3 : 2) void attn_fa_kernel(AttnArgs a, int n_splits, int ksplit) {
  constexpr int DH = 128;
  constexpr int QROWS = 64 * NG;
  constexpr int QT = QROWS / G;
  constexpr int kBlk = KVB * DH * 2;     // bytes of one K (or V) block: 64 rows x 256 B
  __shared__ __attribute__((aligned(1024))) uint8_t kv[2][2 * kBlk];   // [stage][K | V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n_tiles = (a.R + QT - 1) / QT;
  // one-dimensional grid over (KV head, split, tile): each XCD takes a contiguous run
  // of work items, i.e. mostly one KV head, whose K/V stream then stays in its L2.
  // Within a head the first split of every tile (longest tile first) comes before
  // the second split of any: the later splits exist only for the longer tiles, so
  // the empty items trail and the items that run start together.
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int per_head = n_tiles * n_splits;
  const int kvh = w / per_head;
  const int split = (w % per_head) / n_tiles;
  const int tile = n_tiles - 1 - (w % per_head) % n_tiles;
  const int t0 = tile * QT;
  const int t_last = min(t0 + QT, a.R) - 1;
  const int kv_end = a.rowpos[t_last] + 1;
  const int j_begin = split * ksplit;
  const int j_end = min(kv_end, j_begin + ksplit);
  if (j_begin >= j_end) return;

  const int kgrp = lane >> 4;
  int qtok[NG], qhead[NG], qpos[NG];
  bool qvalid[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int qr = (wid * NG + g) * 16 + (lane & 15);
    qtok[g] = t0 + (qr % QT);
    qhead[g] = kvh * G + qr / QT;
    qvalid[g] = qtok[g] < a.R;
    qpos[g] = qvalid[g] ? a.rowpos[qtok[g]] : kv_end - 1;
  }
  const int qpos_min = a.rowpos[t0];
  bf16x8_t qf[NG][DH / 32];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(qvalid[g] ? qtok[g] : t_last) * a.ldq +
                       qhead[g] * DH + 8 * kgrp;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) qf[g][ks] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * ks);
  }
  f32x4_t o[NG][DH / 16];
  f32x4_t lsum[NG];                      // every element: the running sum of the lane's query column
  float m_run[NG], m_neg[NG], thr[NG];   // reference max (exp2 units), its negation (0 if none), threshold
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[g][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lsum[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[g] = -INFINITY;
    m_neg[g] = 0.f;
    thr[g] = -INFINITY;
  }
  const float sc = a.scale * kLog2e;
  const float inv_sc = 1.0f / sc;
  bf16x8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  const int sh = a.cache.bs_shift;       // >= 4: the launcher checks it
  const int width = a.n_kv_heads * DH;
  const bf16_t* kbase = static_cast<const bf16_t*>(a.cache.k) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.cache.v) + static_cast<int64_t>(a.layer) * a.cache.layer_stride;
  // the launcher guarantees the layer's pool spans < 2^31 bytes
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kbase), static_cast<short>(0),
                                                                      0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vbase), static_cast<short>(0),
                                                                      0x7fffffff, 0x00020000);
  // copy u (0..3) of this wave: key 16 wid + 4 u + lane / 16 of the block, LDS slot lane % 16 of
  // the key row; K slot p holds chunk p ^ (key % 16), V slot p chunk p ^ 2 (key % 8)
  const int sub = lane >> 4;
  const int slot = lane & 15;
  int kx[4], vx[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int kr = 4 * u + sub;          // key within the wave's 16
    kx[u] = kr * width * 2 + ((slot ^ kr) << 4);
    vx[u] = kr * width * 2 + ((slot ^ ((kr & 7) << 1)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(&kv[0][0]))) +
      wid * 4096);
  const int pmask = (1 << sh) - 1;
  // the entry is the same for the whole wave: a scalar load, counted apart from the
  // vector-memory counter that the block copies raise, so waiting for it never
  // waits for copies in flight
  // (clamped to the last key of the range, so the load is unconditional; copies past
  // the range read zeros whatever the entry)
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  const int j_last = __builtin_amdgcn_readfirstlane(j_end - 1);
  auto page_of = [&](int jb) -> int {   // block-table entry of this wave's 16 keys of block jb
    if constexpr (CONTIG) return 0;
    const int k0 = __builtin_amdgcn_readfirstlane(min(jb + 16 * wid_u, j_last));
    return a.cache.bt[k0 >> sh];
  };
  int pe = page_of(j_begin);
  auto issue = [&](int jb, int stage) {
    const int k0 = jb + 16 * wid;
    const int rowb = (CONTIG ? k0 : (pe << sh) + (k0 & pmask)) * width * 2 + kvh * DH * 2;
    pe = page_of(jb + KVB);
    if (jb + KVB <= j_end) {             // the whole block lies in the range (uniform)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t dst = ldsw + stage * (2 * kBlk) + u * 1024;
        attn_copy(dst, rk, rowb + kx[u]);
        attn_copy(dst + kBlk, rv, rowb + vx[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = k0 + 4 * u + sub < j_end;
        const int ko = ok ? rowb + kx[u] : static_cast<int>(0x80000000u);   // past the range: zeros
        const int vo = ok ? rowb + vx[u] : static_cast<int>(0x80000000u);
        const uint32_t dst = ldsw + stage * (2 * kBlk) + u * 1024;
        attn_copy(dst, rk, ko);
        attn_copy(dst + kBlk, rv, vo);
      }
    }
  };

  // per-lane LDS byte offsets of the fragment reads inside a stage (block-relative keys):
  // K fragment (t, ks): key 16 t + lane % 16, chunk 4 ks + kgrp at slot chunk ^ (key % 16);
  // V^T source of (dt, s2, h): key 32 s2 + 16 h + 4 kgrp + sl / 4, dims 16 dt + 4 (sl % 4)
  int koff[DH / 32], voffs[DH / 16];
  {
    const int kk = lane & 15;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) koff[ks] = kk * 256 + (((4 * ks + kgrp) ^ kk) << 4);
    const int sl = lane & 15;
    const int vkey = 4 * kgrp + (sl >> 2);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const int d = 16 * dt + 4 * (sl & 3);
      voffs[dt] = vkey * 256 + (((d >> 3) ^ ((vkey & 7) << 1)) << 4) + ((d & 7) << 1);
    }
  }
  auto block = [&](int j0, int stage) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of block j0 have landed
    __syncthreads();                      // ... everyone's; block j0 - 64 is no longer read
    if (j0 + KVB < j_end) issue(j0 + KVB, stage ^ 1);
    const uint8_t* Kb = kv[stage];
    const uint8_t* Vb = kv[stage] + kBlk;

    f32x4_t s[NG][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int g = 0; g < NG; ++g) s[g][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DH / 32; ++ks) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(Kb + koff[ks] + t * (16 * 256));
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[g][ks], s[g][t], 0, 0, 0);
      }
    }
    const bool edge = j0 + KVB - 1 > qpos_min || j0 + KVB > j_end;
    float mx[NG];
    bool over = false;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (edge) {
        // key j0 + 16 t + 4 kgrp + i is visible iff it is <= min(qpos, j_end - 1)
        const int lim = min(qpos[g], j_end - 1) - (j0 + 4 * kgrp);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * t + i > lim) s[g][t][i] = -INFINITY;
      }
      float m = fmaxf(fmaxf(s[g][0][0], s[g][0][1]), fmaxf(s[g][0][2], s[g][0][3]));
#pragma unroll
      for (int t = 1; t < 4; ++t) m = fmaxf(fmaxf(m, fmaxf(s[g][t][0], s[g][t][1])), fmaxf(s[g][t][2], s[g][t][3]));
      mx[g] = m;
      over |= m > thr[g];
    }
    // the reference max of a row moves only when a score exceeds it by more than 2^8 in
    // exp2 units, so every exp2 below stays <= 256 and rescaling is rare
    if (__any(over)) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float mb = mx[g];
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float m_blk = mb * sc;
        if (m_blk > m_run[g] + 8.f) {
          const float alpha = (m_run[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[g] - m_blk);
          lsum[g] *= alpha;
#pragma unroll
          for (int t = 0; t < DH / 16; ++t) o[g][t] *= alpha;
          m_run[g] = m_blk;
          m_neg[g] = -m_blk;
          thr[g] = (m_blk + 8.f) * inv_sc;
        }
      }
    }
    bf16x8_t pf[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p4[i] = __builtin_amdgcn_exp2f(fmaf(s[g][t][i], sc, m_neg[g]));
        const bf16x2_t lo = __builtin_convertvector(f32x2_t{p4[0], p4[1]}, bf16x2_t);
        const bf16x2_t hi = __builtin_convertvector(f32x2_t{p4[2], p4[3]}, bf16x2_t);
        pf[g][t >> 1][(t & 1) * 4 + 0] = lo[0];
        pf[g][t >> 1][(t & 1) * 4 + 1] = lo[1];
        pf[g][t >> 1][(t & 1) * 4 + 2] = hi[0];
        pf[g][t >> 1][(t & 1) * 4 + 3] = hi[1];
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) lsum[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[g][s2], lsum[g], 0, 0, 0);
    }

    // O^T += V^T P^T (fragment layout as in attn_dma_kernel); the V^T fragment of the
    // next step is read before this step's products issue, so LDS latency overlaps them
    auto vread = [&](int st) __attribute__((always_inline)) -> bf16x8_t {
      const int dt = st >> 1, s2 = st & 1;
      s16x4_t half[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint8_t* src = Vb + voffs[dt] + (32 * s2 + 16 * h) * 256;
        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(const __attribute__((address_space(3))) void*)(src));
      }
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int NST = 2 * (DH / 16);
    bf16x8_t vq[3];
    vq[0] = vread(0);
    vq[1] = vread(1);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + 2 < NST) vq[(st + 2) % 3] = vread(st + 2);
#pragma unroll
      for (int g = 0; g < NG; ++g)
        o[g][st >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vq[st % 3], pf[g][st & 1], o[g][st >> 1], 0, 0, 0);
      if (st + 2 < NST) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // this step's two reads (step st + 2)
        __builtin_amdgcn_sched_group_barrier(0x008, NG, 0);  // then its products
      }
    }
  };
  issue(j_begin, 0);
  for (int j0 = j_begin; j0 < j_end; j0 += 2 * KVB) {
    block(j0, 0);
    if (j0 + KVB < j_end) block(j0 + KVB, 1);
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (!qvalid[g]) continue;
    const float l_tot = lsum[g][0];
    if (n_splits == 1 || kv_end <= ksplit) {   // the tile's keys lie in split 0: final output
      const float inv = (CONTIG ? a.cache.vs : 1.0f) / l_tot;
      bf16_t* ob = static_cast<bf16_t*>(a.o);
      const int KO = a.n_q_heads * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        uint2 w;
        w.x = static_cast<uint32_t>(f2bf(o[g][dt][0] * inv)) | (static_cast<uint32_t>(f2bf(o[g][dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f2bf(o[g][dt][2] * inv)) | (static_cast<uint32_t>(f2bf(o[g][dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(ob + pk_off(qtok[g], qhead[g] * DH + 16 * dt + 4 * kgrp, KO)) = w;
      }
    } else {
      const int64_t pr = (static_cast<int64_t>(split) * a.R + qtok[g]) * a.n_q_heads + qhead[g];
      float* op = a.part_o + pr * DH;
      const float vs = CONTIG ? a.cache.vs : 1.0f;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        *reinterpret_cast<float4*>(op + 16 * dt + 4 * kgrp) =
            make_float4(o[g][dt][0] * vs, o[g][dt][1] * vs, o[g][dt][2] * vs, o[g][dt][3] * vs);
      if (kgrp == 0) a.part_ml[pr] = make_float2(m_run[g], l_tot);
    }
  }
}

// Widening of one layer of an FP8 paged cache into contiguous bf16 K and V runs
// (positions [0, rows), unscaled: every E4M3 value is exact in bf16), so the
// LDS-staged attention kernel reads it like a bf16 layer; the K scale then goes
// into the softmax scale and the V scale into the output.  One thread widens
// 16 bytes of K and of V.
__global__ __launch_bounds__(256) void kv_widen_fp8_kernel(PagedRef c, int layer, int rows, int width, bf16_t* ko,
                                                          bf16_t* vo) {
  const int per_row = width >> 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(rows) * per_row) return;
  const int pos = static_cast<int>(i / per_row);
  const int e = static_cast<int>(i % per_row) * 16;
  const int64_t src = static_cast<int64_t>(layer) * c.layer_stride + paged_row(c, pos) * width + e;
  const uint4 kw = *reinterpret_cast<const uint4*>(static_cast<const fp8_t*>(c.k) + src);
  const uint4 vw = *reinterpret_cast<const uint4*>(static_cast<const fp8_t*>(c.v) + src);
  auto widen = [](uint4 w, bf16_t* dst) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[4];
      fp8x4_to_f32(in[q], f);
      out[2 * q] = fp8x2_to_bf16x2(f[0], f[1]);
      out[2 * q + 1] = fp8x2_to_bf16x2(f[2], f[3]);
    }
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(out[0], out[1], out[2], out[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(out[4], out[5], out[6], out[7]);
  };
  const int64_t dst = static_cast<int64_t>(pos) * width + e;
  widen(kw, ko + dst);
  widen(vw, vo + dst);
}

// Merge the split-KV partials of one (row, q head) per wave.  The lanes take
// the splits' (max, sum) pairs side by side (one split per lane and pass), so a
// row with many splits (a single decode row) costs a few dependent loads, not
// one per split; the output sums then run over the splits in order, eight
// loads in flight at a time.
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
  if (ns <= 1) return;                                   // written whole by the attention kernel
  auto prow = [&](int sp) { return (static_cast<int64_t>(sp) * a.R + row) * a.n_q_heads + head; };
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) M = fmaxf(M, a.part_ml[prow(s0 + lane)].x);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  constexpr int PER = DH / 64;
  float acc[PER] = {};
  float lsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float wl = 0.f;
    if (s0 + lane < ns) {
      const float2 ml = a.part_ml[prow(s0 + lane)];
      wl = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      lsum += wl * ml.y;
    }
    const int cnt = min(64, ns - s0);
#pragma unroll 8
    for (int j = 0; j < cnt; ++j) {
      const float w = __shfl(wl, j, 64);
      const float* po = a.part_o + prow(s0 + j) * DH + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * po[e];
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) lsum += __shfl_xor(lsum, m, 64);
  const float inv = 1.0f / lsum;
  bf16_t* ob = static_cast<bf16_t*>(a.o);
  const int KO = a.n_q_heads * DH;
#pragma unroll
  for (int e = 0; e < PER; ++e) ob[pk_off(row, head * DH + lane * PER + e, KO)] = f2bf(acc[e] * inv);
}

// The same merge with whole rows: `per_row` workgroups per row, thread t of
// piece c taking CPT consecutive output columns (inside one head) from column
// (256 c + t) CPT, so every split's (max, sum) pair and partial columns are
// loaded at once; sums run in split order.  For rows of H_q x DH = 256 x CPT x
// per_row columns (CPT a multiple of 8 dividing DH).
template <int DH, int CPT>
__global__ __launch_bounds__(256) void attn_combine_wide_kernel(AttnArgs a, int n_splits, int ksplit, int QT, int per_row) {
  static_assert(CPT % 8 == 0 && DH % CPT == 0, "whole 8-column chunks inside one head");
  // groups of 8 consecutive rows on one XCD, so their 16-byte pieces of a
  // fragment-major block meet in one L2 and leave it as whole 128-byte lines;
  // successive groups go to successive XCDs, so the leading rows that need no merge
  // (their keys lie in split 0) do not all fall on the same XCDs.  The grid covers a
  // whole number of group rounds (8 x 8 rows); blocks past the last row return.
  const int grp = 8 * per_row;
  const int xi = blockIdx.x % kXcd, ii = blockIdx.x / kXcd;
  const int wi = ((ii / grp) * kXcd + xi) * grp + ii % grp;
  const int row = wi / per_row;
  if (row >= a.R) return;
  const int t_last = min((row / QT + 1) * QT, a.R) - 1;
  const int kv_end = a.rowpos[t_last] + 1;
  const int ns = min(n_splits, (kv_end + ksplit - 1) / ksplit);
  if (ns <= 1) return;                                   // written whole by the attention kernel
  const int col = ((wi % per_row) * 256 + threadIdx.x) * CPT;
  const int head = col / DH;
  auto prow = [&](int sp) { return (static_cast<int64_t>(sp) * a.R + row) * a.n_q_heads + head; };
  float M = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, a.part_ml[prow(sp)].x);
  float acc[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) acc[e] = 0.f;
  float lsum = 0.f;
#pragma unroll 2
  for (int sp = 0; sp < ns; ++sp) {
    const float2 ml = a.part_ml[prow(sp)];
    const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
    lsum += w * ml.y;
    const float4* po = reinterpret_cast<const float4*>(a.part_o + prow(sp) * DH + (col % DH));
#pragma unroll
    for (int e = 0; e < CPT / 4; ++e) {
      const float4 v = po[e];
      acc[4 * e] += w * v.x;
      acc[4 * e + 1] += w * v.y;
      acc[4 * e + 2] += w * v.z;
      acc[4 * e + 3] += w * v.w;
    }
  }
  const float inv = 1.0f / lsum;
  bf16_t* ob = static_cast<bf16_t*>(a.o);
  const int KO = a.n_q_heads * DH;
#pragma unroll
  for (int c = 0; c < CPT / 8; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f2bf(acc[8 * c + 2 * i] * inv)) |
             (static_cast<uint32_t>(f2bf(acc[8 * c + 2 * i + 1] * inv)) << 16);
    *reinterpret_cast<uint4*>(ob + pk_off(row, col + 8 * c, KO)) = make_uint4(w[0], w[1], w[2], w[3]);
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

// Key splits of the lean LDS-DMA kernel when the (tile, head) grid cannot fill the
// chip: from `from` splits up, the most whose non-empty work items still fit the
// chip's `slots` resident workgroups (two per CU, three with one query group per
// wave) at once, so none waits for a second round.  Item counts are estimated with the tiles' key ranges spread evenly up to
// the last key (sorted rows of a blend: tile t ends near (t + 1) / n_tiles of the
// keys); a wrong estimate costs time, never correctness.
int fa_splits(int from, int n_tiles, int kv_blocks, int n_kv_heads, int R, int n_q_heads, int slots) {
  int best = from;
  for (int ns = from + 1; ns <= kAttnSplitCap && ns <= kv_blocks; ++ns) {
    if (static_cast<int64_t>(ns) * R * n_q_heads > kAttnPartialRows) break;
    const int per = (kv_blocks + ns - 1) / ns;
    int64_t items = 0;
    for (int t = 0; t < n_tiles; ++t) {
      const int bt = static_cast<int>((static_cast<int64_t>(kv_blocks) * (t + 1) + n_tiles - 1) / n_tiles);
      items += (bt + per - 1) / per;
    }
    if (items * n_kv_heads > slots) break;
    best = ns;
  }
  return best;
}

// KIND 0 register-staged, 1 LDS-DMA, 2 lean LDS-DMA; CONTIG (KIND 2): keys in one contiguous run
template <int DH, int G, int NG, int KIND, bool F8 = false, bool CONTIG = false>
hipError_t run_bf16(const AttnArgs& a, hipStream_t s) {
  constexpr int QT = 64 * NG / G;
  const int n_tiles = (a.R + QT - 1) / QT;
  const int base = n_tiles * a.n_kv_heads;
  const int kv_blocks = (a.kv_bound + KVB - 1) / KVB;
  // split the keys only when the (tile, head) grid cannot fill the chip; tiles of sparse
  // rows end at spread-out positions, so only the longer tiles have keys in the later
  // splits: start from ~2 x 256 workgroups in all, and the lean kernel then takes as
  // many more splits as keep its non-empty items within one round (678 rows over 4K
  // keys, split-major order: 3 splits 60-63 us, 4 splits 54-57 us, 5 splits 64-66 us)
  int n_splits = 1;
  if (base < 512 && a.part_o != nullptr) {
    n_splits = std::min(kAttnSplitCap, std::max(1, (512 + base - 1) / base));
    n_splits = std::min(n_splits, kv_blocks);
    if (static_cast<int64_t>(n_splits) * a.R * a.n_q_heads > kAttnPartialRows) n_splits = 1;
  }
  if (a.n_splits_req > 0 && a.part_o != nullptr &&
      static_cast<int64_t>(a.n_splits_req) * a.R * a.n_q_heads <= kAttnPartialRows)
    n_splits = std::min(a.n_splits_req, kv_blocks);
  if (KIND == 2 && a.n_splits_req == 0 && n_splits > 1)
    n_splits = fa_splits(n_splits, n_tiles, kv_blocks, a.n_kv_heads, a.R, a.n_q_heads, NG == 1 ? 768 : 512);
  const int ksplit = ((kv_blocks + n_splits - 1) / n_splits) * KVB;
  const dim3 grid(n_tiles * n_splits, a.n_kv_heads);
  if constexpr (KIND == 2) {
    attn_fa_kernel<G, NG, CONTIG><<<dim3(n_tiles * n_splits * a.n_kv_heads), 256, 0, s>>>(a, n_splits, ksplit);
  } else if (KIND == 1) {
    // workgroups stage the table entries of their key range in LDS when they fit
    if (ksplit / a.cache.bs + 2 <= 1024)
      attn_dma_kernel<G, true, NG><<<grid, 256, 0, s>>>(a, n_splits, ksplit);
    else
      attn_dma_kernel<G, false, NG><<<grid, 256, 0, s>>>(a, n_splits, ksplit);
  } else if (ksplit / a.cache.bs + 2 <= kBtCache) {
    attn_bf16_kernel<DH, G, true, NG, F8><<<grid, 256, 0, s>>>(a, n_splits, ksplit);
  } else {
    attn_bf16_kernel<DH, G, false, NG, F8><<<grid, 256, 0, s>>>(a, n_splits, ksplit);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int width = a.n_q_heads * DH;
  if (width % (256 * 8) == 0) {
    // 8 columns per thread: rows of 4096 / 8192 columns take 2 / 4 workgroups each,
    // so more loads are in flight than with one workgroup per row
    const int per_row = width / (256 * 8);
    const int rows = (a.R + 8 * kXcd - 1) / (8 * kXcd) * (8 * kXcd);
    attn_combine_wide_kernel<DH, 8><<<rows * per_row, 256, 0, s>>>(a, n_splits, ksplit, QT, per_row);
  } else {
    const int pairs = a.R * a.n_q_heads;
    attn_combine_kernel<DH><<<(pairs + 3) / 4, 256, 0, s>>>(a, n_splits, ksplit, QT);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One query row (a decode step): the G query heads of a KV head read each K/V
// row once.  A workgroup takes one KV head and a range of keys, 64 per pass:
// thread t scores key t / 4 on the 32 dims (t % 4) * 32 .. +31 for all G
// heads (a quad adds its four parts), each wave redoes the pass's softmax
// update in registers (lane = key), and wave w then adds keys 16 w .. 16 w + 15
// into its lanes' two output dims per head; the V rows of the pass are loaded
// while the scores are made.  Partials (unnormalised sums, running max in
// log2 units, sum of weights) go to the split-KV buffers.
// ---------------------------------------------------------------------------
template <int DH, int G, bool RUN16, bool F8 = false>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a, int ksplit) {
  static_assert(DH == 128, "two output dims per lane");
  __shared__ uint4 qs[G][DH / 8];        // bf16 query heads, 8 dims per entry
  __shared__ float sc[G][64];
  __shared__ float red[4][G][DH];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.x % a.n_kv_heads;
  const int split = blockIdx.x / a.n_kv_heads;
  const int j_begin = split * ksplit;
  const int j_lim = min(a.kv_bound, j_begin + ksplit);          // the table covers every key below kv_bound
  if (j_begin >= j_lim) return;                                  // uniform per workgroup
  const uint4* qrow = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.q) + static_cast<int64_t>(kvh) * G * DH);
  uint4 qv = {};
  if (tid < G * DH / 8) qv = qrow[tid];   // stored to LDS once the first K/V loads are out
  const float sc_l2 = a.scale * kLog2e * (F8 ? a.cache.ks : 1.0f);
  const int width = a.n_kv_heads * DH;
  const int64_t lbase = static_cast<int64_t>(a.layer) * a.cache.layer_stride + kvh * DH;
  using E = typename std::conditional<F8, fp8_t, bf16_t>::type;   // cache element
  const E* kc = static_cast<const E*>(a.cache.k) + lbase;
  const E* vc = static_cast<const E*>(a.cache.v) + lbase;
  const int kk = tid >> 2, quarter = tid & 3;
  // loads run to j_lim without waiting for the row's position; keys past it are masked
  const int j_end = min(a.rowpos[0] + 1, j_lim);
  float m_run[G], l_run[G], acc[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.f; acc[g][0] = acc[g][1] = 0.f; }
  for (int t0 = j_begin; t0 < j_lim; t0 += 64) {
    // K: this thread's 32 dims of key t0 + kk; V: keys t0 + 16 wid + i, dims 2 lane, 2 lane + 1.
    // Both are wave w's 16 keys from t0 + 16 w, a multiple of 16: with pages of 16
    // keys or more they are 16 consecutive rows, found with one table lookup.
    // Keys at or past j_lim are clamped to j_lim - 1, so every load is in range
    // and issued unconditionally; their scores and values are masked below.
    const int key = t0 + kk;
    const int kw0 = t0 + 16 * wid;
    const int last = j_lim - 1;
    int64_t krow, vrow[16];
    if constexpr (RUN16) {
      const int g0 = min(kw0, last & ~15);                       // the 16-key run holding the clamped keys
      const int64_t rbase = paged_row(a.cache, g0);
      krow = rbase + (min(key, last) - g0);
#pragma unroll
      for (int i = 0; i < 16; ++i) vrow[i] = rbase + (min(kw0 + i, last) - g0);
    } else {
      krow = paged_row(a.cache, min(key, last));
#pragma unroll
      for (int i = 0; i < 16; ++i) vrow[i] = paged_row(a.cache, min(kw0 + i, last));
    }
    uint4 kr[4];
    const uint4* kp = reinterpret_cast<const uint4*>(kc + krow * width + quarter * 32);
    uint32_t vr[16];
    if constexpr (F8) {
      // 32 FP8 dims widen exactly to bf16 pairs; V: two FP8 dims per lane
      const uint4 k8[2] = {kp[0], kp[1]};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {k8[h].x, k8[h].y, k8[h].z, k8[h].w};
        float f[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) fp8x4_to_f32(w[i], f + 4 * i);
        kr[2 * h] = make_uint4(fp8x2_to_bf16x2(f[0], f[1]), fp8x2_to_bf16x2(f[2], f[3]), fp8x2_to_bf16x2(f[4], f[5]),
                               fp8x2_to_bf16x2(f[6], f[7]));
        kr[2 * h + 1] = make_uint4(fp8x2_to_bf16x2(f[8], f[9]), fp8x2_to_bf16x2(f[10], f[11]),
                                   fp8x2_to_bf16x2(f[12], f[13]), fp8x2_to_bf16x2(f[14], f[15]));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint16_t b2 = *reinterpret_cast<const uint16_t*>(vc + vrow[i] * width + 2 * lane);
        float f[4];
        fp8x4_to_f32(b2, f);
        vr[i] = fp8x2_to_bf16x2(f[0], f[1]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = kp[i];
#pragma unroll
      for (int i = 0; i < 16; ++i) vr[i] = *reinterpret_cast<const uint32_t*>(vc + vrow[i] * width + 2 * lane);
    }
    if (t0 == j_begin) {
      if (tid < G * DH / 8) qs[tid / (DH / 8)][tid % (DH / 8)] = qv;
      __syncthreads();
    }
    if (t0 >= j_end) break;               // no key of this pass is visible (uniform)
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s[g] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[g] = dot8_bf16(kr[i], qs[g][quarter * 4 + i], s[g]);
      s[g] += __shfl_xor(s[g], 1, 64);
      s[g] += __shfl_xor(s[g], 2, 64);
    }
    if (quarter == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g][kk] = key < j_end ? s[g] * sc_l2 : -INFINITY;
    }
    float vf[16][2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = kw0 + i < j_end;
      vf[i][0] = ok ? bf2f(static_cast<bf16_t>(vr[i] & 0xFFFFu)) : 0.f;
      vf[i][1] = ok ? bf2f(static_cast<bf16_t>(vr[i] >> 16)) : 0.f;
    }
    __syncthreads();
    // softmax update, lane = key of the pass (every wave alike)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = sc[g][lane];
      float mt = v;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) mt = fmaxf(mt, __shfl_xor(mt, m, 64));
      const float m_new = fmaxf(m_run[g], mt);                   // finite: key t0 is in range
      const float alpha = exp2f(m_run[g] - m_new);
      const float p = exp2f(v - m_new);
      float ps = p;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ps += __shfl_xor(ps, m, 64);
      l_run[g] = l_run[g] * alpha + ps;
      m_run[g] = m_new;
      float o0 = acc[g][0] * alpha, o1 = acc[g][1] * alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 16 * wid + i));
        o0 += pi * vf[i][0];
        o1 += pi * vf[i][1];
      }
      acc[g][0] = o0;
      acc[g][1] = o1;
    }
    __syncthreads();                                             // sc[] is rewritten by the next pass
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    red[wid][g][2 * lane] = acc[g][0];
    red[wid][g][2 * lane + 1] = acc[g][1];
  }
  __syncthreads();
  for (int e = tid; e < G * DH; e += 256) {
    const int g = e / DH, d = e % DH;
    const int64_t pr = static_cast<int64_t>(split) * a.n_q_heads + kvh * G + g;   // (split, row 0, head)
    a.part_o[pr * DH + d] = (((red[0][g][d] + red[1][g][d]) + red[2][g][d]) + red[3][g][d]) * (F8 ? a.cache.vs : 1.0f);
    if (d == 0) a.part_ml[pr] = make_float2(m_run[g], l_run[g]);
  }
}

// Merge many split-KV partials of one query row: one workgroup per q head;
// thread t takes dims 2 (t % 64) .. +1 of the splits t / 64, t / 64 + 4, ..., so
// all partial loads are in flight at once, and the four waves add up in LDS.
template <int DH>
__global__ __launch_bounds__(256) void attn_combine_row_kernel(AttnArgs a, int ksplit) {
  static_assert(DH == 128, "two output dims per lane");
  constexpr int PER = 16;                 // splits per wave held in registers
  __shared__ float wmax[4];
  __shared__ float red[4][DH + 1];
  const int head = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // every split below kv_bound wrote a partial (an empty one has max -inf, sum 0)
  const int ns = (a.kv_bound + ksplit - 1) / ksplit;
  float o0 = 0.f, o1 = 0.f, ls = 0.f;
  float M = -INFINITY;
  if (ns <= 4 * PER) {
    // one round of loads: wave w holds splits w, w + 4, ...
    float2 ml[PER], po[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sp = wid + 4 * i;
      if (sp < ns) {
        const int64_t pr = static_cast<int64_t>(sp) * a.n_q_heads + head;
        ml[i] = a.part_ml[pr];
        po[i] = *reinterpret_cast<const float2*>(a.part_o + pr * DH + 2 * lane);
        M = fmaxf(M, ml[i].x);
      }
    }
    if (lane == 0) wmax[wid] = M;
    __syncthreads();
    M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (wid + 4 * i < ns) {
        const float w = exp2f(ml[i].x - M);
        ls += w * ml[i].y;
        o0 += w * po[i].x;
        o1 += w * po[i].y;
      }
    }
  } else {
    for (int sp = tid; sp < ns; sp += 256) M = fmaxf(M, a.part_ml[static_cast<int64_t>(sp) * a.n_q_heads + head].x);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    if (lane == 0) wmax[wid] = M;
    __syncthreads();
    M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    for (int sp = wid; sp < ns; sp += 4) {
      const int64_t pr = static_cast<int64_t>(sp) * a.n_q_heads + head;
      const float2 ml = a.part_ml[pr];
      const float2 po = *reinterpret_cast<const float2*>(a.part_o + pr * DH + 2 * lane);
      const float w = exp2f(ml.x - M);
      ls += w * ml.y;
      o0 += w * po.x;
      o1 += w * po.y;
    }
  }
  red[wid][2 * lane] = o0;
  red[wid][2 * lane + 1] = o1;
  if (lane == 0) red[wid][DH] = ls;
  __syncthreads();
  if (wid == 0) {
    const float l = ((red[0][DH] + red[1][DH]) + red[2][DH]) + red[3][DH];
    const float inv = 1.0f / l;
    bf16_t* ob = static_cast<bf16_t*>(a.o);
    const int KO = a.n_q_heads * DH;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = 2 * lane + e;
      const float v = ((red[0][d] + red[1][d]) + red[2][d]) + red[3][d];
      ob[pk_off(0, head * DH + d, KO)] = f2bf(v * inv);
    }
  }
}

template <int G>
hipError_t run_decode(const AttnArgs& a, hipStream_t s) {
  const int kv_blocks = (a.kv_bound + KVB - 1) / KVB;
  // one 64-key pass per workgroup up to about 1024 workgroups
  int n_splits = std::max(1, std::min(kv_blocks, (1024 + a.n_kv_heads - 1) / a.n_kv_heads));
  while (static_cast<int64_t>(n_splits) * a.n_q_heads > kAttnPartialRows) --n_splits;
  const int ksplit = ((kv_blocks + n_splits - 1) / n_splits) * KVB;
  n_splits = (a.kv_bound + ksplit - 1) / ksplit;
  // pages of 16 keys or more (a power of two): a wave's 16 keys are consecutive rows
  const bool run16 = a.cache.bt == nullptr || a.cache.bs_shift >= 4;
  if (a.cache.fp8) {
    if (run16)
      attn_decode_kernel<128, G, true, true><<<n_splits * a.n_kv_heads, 256, 0, s>>>(a, ksplit);
    else
      attn_decode_kernel<128, G, false, true><<<n_splits * a.n_kv_heads, 256, 0, s>>>(a, ksplit);
  } else if (run16) {
    attn_decode_kernel<128, G, true><<<n_splits * a.n_kv_heads, 256, 0, s>>>(a, ksplit);
  } else {
    attn_decode_kernel<128, G, false><<<n_splits * a.n_kv_heads, 256, 0, s>>>(a, ksplit);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_row_kernel<128><<<a.n_q_heads, 256, 0, s>>>(a, ksplit);
  return hipGetLastError();
}

// variant: 1 / 2 = register-staged kernel with 1 / 2 query groups per wave,
// 3 / 4 = LDS-DMA kernel (head_dim 128, a layer's pool below 2 GiB) with 1 / 2,
// 5 / 6 = lean LDS-DMA kernel (as 3 / 4, pages a power of two >= 16 keys) with 1 / 2
template <int DH, int G>
hipError_t run_bf16_variant(const AttnArgs& a, int variant, hipStream_t s) {
  if (a.cache.fp8) {
    // an FP8 layer is widened into the caller's bf16 buffer when it fits there, then
    // read by the lean LDS-DMA kernel; otherwise the register-staged kernel widens it
    // while staging
    const int width = a.n_kv_heads * DH;
    const int64_t run = (static_cast<int64_t>(a.kv_bound) * width * 2 + 255) & ~int64_t(255);
    if constexpr (DH == 128) {
      if (variant >= 5 && a.widen != nullptr && 2 * run <= a.widen_bytes && run < (int64_t(1) << 31) && a.kv_bound > 0) {
        AttnArgs b = a;
        bf16_t* kw = static_cast<bf16_t*>(a.widen);
        bf16_t* vw = reinterpret_cast<bf16_t*>(static_cast<char*>(a.widen) + run);
        const int64_t threads = static_cast<int64_t>(a.kv_bound) * (width / 16);
        kv_widen_fp8_kernel<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, s>>>(a.cache, a.layer, a.kv_bound,
                                                                                          width, kw, vw);
        b.cache = PagedRef{kw, vw, nullptr, 1, 0, 0, 0, 1.f, a.cache.vs};
        b.layer = 0;
        b.scale = a.scale * a.cache.ks;
        return variant == 5 ? run_bf16<DH, G, 1, 2, false, true>(b, s) : run_bf16<DH, G, 2, 2, false, true>(b, s);
      }
    }
    return variant % 2 ? run_bf16<DH, G, 1, 0, true>(a, s) : run_bf16<DH, G, 2, 0, true>(a, s);
  }
  if constexpr (DH == 128) {
    const bool dma_ok = a.cache.layer_stride * 2 < (int64_t(1) << 31);
    const bool fa_ok = dma_ok && a.cache.bs_shift >= 4;   // pages of 16 or more keys, a power of two
    if (variant >= 5 && fa_ok) return variant == 5 ? run_bf16<DH, G, 1, 2>(a, s) : run_bf16<DH, G, 2, 2>(a, s);
    if (variant >= 3 && dma_ok) return variant % 2 ? run_bf16<DH, G, 1, 1>(a, s) : run_bf16<DH, G, 2, 1>(a, s);
  }
  // a variant whose conditions do not hold falls back to the next simpler kernel
  if (variant % 2) return run_bf16<DH, G, 1, 0>(a, s);
  return run_bf16<DH, G, 2, 0>(a, s);
}

}  // namespace

bool attention_supported(cb_dtype dt, int n_q_heads, int n_kv_heads, int head_dim) {
  if (n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return false;
  const int G = n_q_heads / n_kv_heads;
  if (dt == CB_F32) return head_dim <= 256 && head_dim % 2 == 0;
  return (head_dim == 64 || head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t launch_attention_ng(cb_dtype dt, const AttnArgs& a_in, int ng, hipStream_t s) {  // ng: variant
  if (a_in.R == 0) return hipSuccess;
  AttnArgs a = a_in;
  a.cache.bs_shift = block_shift(a.cache.bs);   // derived here so it always matches bs
  if (dt == CB_F32) {
    attn_f32_kernel<<<dim3(a.R, a.n_q_heads), 64, 0, s>>>(a);
    return hipGetLastError();
  }
  const int G = a.n_q_heads / a.n_kv_heads;
  // a single query row (a decode step) with split-KV buffers: the one-row kernel
  if (a.R == 1 && a.head_dim == 128 && a.part_o != nullptr && a.n_splits_req == 0 && (G == 1 || G == 2 || G == 4 || G == 8)) {
    if (G == 1) return run_decode<1>(a, s);
    if (G == 2) return run_decode<2>(a, s);
    if (G == 4) return run_decode<4>(a, s);
    return run_decode<8>(a, s);
  }
#define CB_ATTN_CASE(D, GG) \
  if (a.head_dim == D && G == GG) return run_bf16_variant<D, GG>(a, ng, s);
  CB_ATTN_CASE(128, 1) CB_ATTN_CASE(128, 2) CB_ATTN_CASE(128, 4) CB_ATTN_CASE(128, 8) CB_ATTN_CASE(128, 16)
  CB_ATTN_CASE(64, 1) CB_ATTN_CASE(64, 2) CB_ATTN_CASE(64, 4) CB_ATTN_CASE(64, 8) CB_ATTN_CASE(64, 16)
#undef CB_ATTN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attention(cb_dtype dt, const AttnArgs& a, hipStream_t s) {
  return launch_attention_ng(dt, a, 6, s);
}

}  // namespace cb
