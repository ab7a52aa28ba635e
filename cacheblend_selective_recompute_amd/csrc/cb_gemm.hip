// Gather-GEMM of the selected rows: C[M][N] = A[M][:] . B[n][:] with the
// epilogues the decoder block needs fused in (RoPE of Q/K at the rows'
// positions, residual add with a row gather, SiLU-gated MLP).
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn), Fig. 5 -- only the
// selected tokens go through the projections; the recompute cost is
// proportional to the selected share (section "选 token").
//
// bf16 path: v_mfma_f32_32x32x16_bf16, block tile BM x 256 with the waves in a
// (waves/2) x 2 grid and a 64 x 128 tile per wave: 256 x 256 with 8 waves (one
// workgroup per CU) or 128 x 256 with 4 waves (two per CU), so every SIMD holds
// two waves that hide each other's waits; the 256-row tile moves a third less
// global data per MFMA.  Both operands are fragment-major in memory (see pk_off:
// activations are written that way by the kernels that produce them, weights are
// packed once by cb_pack_weight), so one 32-row x 16-column block is 1 KiB laid
// out in MFMA lane order.  k advances in stages of 32 columns; each stage is
// copied global -> LDS by buffer loads that write LDS directly (one 1 KiB block
// per instruction, no VGPR staging, hardware range check returns zero past the
// last row block), into a ring of NS stages.  The copies for a stage are spread
// evenly among the MFMAs of the stages before it, so the load path is never
// flooded; the barrier that makes stage t+1 visible sits in the middle of stage
// t, so the first fragments of t+1 are read while t's last MFMAs run.  The tile
// shape and a split of K are chosen per call from a cost model so the grid fills
// the 256 CUs; split-K partials are reduced in a fixed order by a second kernel
// that also applies the epilogue.  Whole tiles are ordered M-fastest within groups
// of 8 row tiles and mapped so consecutive tiles land on the same XCD, where they
// share operand tiles in its L2.
// fp32 path: a plain LDS-tiled FMA kernel (fp32 models are small).
#include <algorithm>
#include <cmath>

#include "cb_internal.h"

namespace cb {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 32;          // k columns per stage
constexpr int BN = 256;         // block tile columns (B rows)
constexpr int kGroupM = 8;      // row tiles per group of the whole-tile order

// s_waitcnt with only the vector-memory counter constrained (n outstanding allowed)
#define CB_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Block-tile configurations (GemmCfg): 0 = 256 x 256 with 8 waves (one workgroup
// per CU), 1 = 128 x 256 with 4 waves (two per CU).  Waves form a (WV/2) x 2 grid,
// so a wave's tile is (BM / (WV/2)) x 128 = 64 x 128 in both.
template <int CFG>
struct Tile {
  static constexpr int BM = CFG == 1 ? 128 : 256;
  static constexpr int WV = CFG == 1 ? 4 : 8;     // waves per workgroup
  static constexpr int kThreads = WV * 64;
  static constexpr int FM = 2 * BM / (32 * WV);   // A fragments (32-row blocks) per wave
  static constexpr int ABLK = BM / 16;            // A blocks per stage: BM/32 row blocks x 2 k blocks
  static constexpr int kStageA = ABLK * 1024;
  static constexpr int kStage = kStageA + 16384;  // + B: 8 row blocks x 2 k blocks
  static constexpr int NS = BM == 256 ? 4 : 3;    // stages in the LDS ring
  static constexpr int DA = ABLK / WV;            // A copies per wave per stage
  static constexpr int DB = 16 / WV;              // B copies per wave per stage
  static constexpr int DQ = DA + DB;              // all copies per wave per stage
  static constexpr int H0 = DQ / 2;               // issued during the second half of a stage
  static constexpr int H1 = DQ - H0;              // ... and during the first half of the next
  static constexpr int WGS_PER_CU = BM == 256 ? 1 : 2;
  static constexpr int EP = 136;                  // epilogue staging row pitch (floats)
  static constexpr int kSmem = NS * kStage > WV * 32 * EP * 4 ? NS * kStage : WV * 32 * EP * 4;
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

// One 1 KiB fragment block global -> LDS: lane i's 16 bytes land at lds + 16 i.
__device__ __forceinline__ void copy_block(uint32_t lds, __amdgpu_buffer_rsrc_t rsrc, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// B is fragment-major with virtual rows: for SWIGLU, 32-row block 2b holds gate
// features [32b, 32b+32) and block 2b+1 the matching up features.
//
// Work of one launch: m_tiles x n_tiles output tiles.  Without SPLIT every
// workgroup computes one tile over all of K.  With SPLIT the tiles of the first
// dp_cols tile columns still do (dp_cols * m_tiles workgroups, launched first),
// and each tile of the remaining columns is cut into `splits` pieces of kps
// columns of K whose fp32 partials go to g.part as [split][M][W], W = the virtual
// columns past dp_cols * BN; a reduction kernel then sums them in split order
// and applies the epilogue.  dp_cols = 0 is plain split-K.
template <int EPI, int CFG, bool SPLIT>
__global__ __launch_bounds__(Tile<CFG>::kThreads, Tile<CFG>::WGS_PER_CU) void gemm_bf16_kernel(GemmArgs g, int splits,
                                                                                              int kps, int dp_cols) {
  using T = Tile<CFG>;
  constexpr int BM = T::BM;
  constexpr int FM = T::FM, NS = T::NS, DA = T::DA, DB = T::DB, DQ = T::DQ, H0 = T::H0, H1 = T::H1;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  const int m_tiles = (g.M + BM - 1) / BM;
  // whole tiles first, then the pieces; each range is spread over the XCDs in
  // contiguous runs so neighbouring tiles (sharing B columns) share an L2
  const int n_dp = SPLIT ? m_tiles * dp_cols : static_cast<int>(gridDim.x);
  const int b = blockIdx.x;
  const bool part = SPLIT && b >= n_dp;
  int mt, nt, split = 0;
  if (!part) {
    // groups of kGroupM row tiles, row-fastest inside a group: the workgroups an XCD
    // runs at once (32 or 64) cover 8 row tiles of 4 or 8 columns, so its L2 holds
    // 12 or 16 operand tiles per k-stage instead of every row tile of a few columns
    const int t = xcd_remap(b, n_dp);
    const int n_tiles = n_dp / m_tiles;
    const int g0 = t / (kGroupM * n_tiles), rem = t % (kGroupM * n_tiles);
    const int gm = min(kGroupM, m_tiles - g0 * kGroupM);
    mt = g0 * kGroupM + rem % gm;
    nt = rem / gm;
  } else {
    const int r = xcd_remap(b - n_dp, static_cast<int>(gridDim.x) - n_dp);
    mt = r % m_tiles;
    const int rest = r / m_tiles;
    split = rest % splits;
    nt = dp_cols + rest / splits;
  }
  const int m0 = mt * BM;
  const int n0 = nt * BN;                              // first virtual B row of the tile
  const int kbeg = part ? split * kps : 0;
  const int nk = ((part ? min(g.K, kbeg + kps) : g.K) - kbeg) / BK;   // >= 1 (host drops empty splits)

  const int kbr = g.K >> 4;                            // 16-column blocks per row block
  const int b_rows = (EPI == EPI_SWIGLU) ? 2 * g.N : g.N;
  const int mb0 = m0 >> 5, nb0 = n0 >> 5;
  const int mb_valid = (g.M + 31) >> 5, nb_valid = (b_rows + 31) >> 5;
  const int kb0 = kbeg >> 4;
  const bf16_t* A = static_cast<const bf16_t*>(g.A);
  const bf16_t* B = static_cast<const bf16_t*>(g.B);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(A + (static_cast<int64_t>(mb0) * kbr + kb0) * 512), static_cast<short>(0),
      max(0, (mb_valid - mb0) * kbr - kb0) * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(B + (static_cast<int64_t>(nb0) * kbr + kb0) * 512), static_cast<short>(0),
      max(0, (nb_valid - nb0) * kbr - kb0) * 1024, 0x00020000);

  // copy u of a stage: u < DA -> A block wid*DA+u, else B block wid*DB+u-DA;
  // block q of a stage = row block q/2, k block q%2
  int voff[DQ];
#pragma unroll
  for (int u = 0; u < DQ; ++u) {
    const int q = u < DA ? wid * DA + u : wid * DB + (u - DA);
    voff[u] = ((q >> 1) * kbr + (q & 1)) * 1024 + lane * 16;
  }
  // LDS byte address of the ring and the wave index, both wave-uniform (scalar registers)
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int wid_s = __builtin_amdgcn_readfirstlane(wid);
  // copy u of stage s into ring slot `slot` (a compile-time constant at every call)
  auto copy = [&](int s, int slot, int u) {
    const int q = u < DA ? wid_s * DA + u : wid_s * DB + (u - DA);
    const uint32_t dst = lds0 + slot * T::kStage + (u < DA ? 0 : T::kStageA) + q * 1024;
    const int soff = min(s, nk - 1) * (BK * 64);      // stages past the last re-read it into a retired slot
    if (u < DA) copy_block(dst, ra, voff[u], soff);
    else copy_block(dst, rb, voff[u], soff);
  };

  f32x16_t acc[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // per-lane fragment offsets within a slot; the slot offset is an immediate
  const uint8_t* fa = smem + (wm * FM * 2) * 1024 + lane * 16;
  const uint8_t* fb = smem + T::kStageA + (wn * 4 * 2) * 1024 + lane * 16;
  bf16x8_t af[2][FM], bfr[2][4];
  auto frag = [&](int slot, int ks, int reg) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[reg][i] = *reinterpret_cast<const bf16x8_t*>(fa + slot * T::kStage + (i * 2 + ks) * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[reg][j] = *reinterpret_cast<const bf16x8_t*>(fb + slot * T::kStage + (j * 2 + ks) * 1024);
  };
  // the MFMAs of one 16-column step, with copies u0 .. u0+cnt-1 of stage cs (slot cslot) spread among them
  auto mma = [&](int reg, int cs, int cslot, int u0, int cnt) {
    constexpr int NM = 4 * FM;
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      acc[x >> 2][x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[reg][x >> 2], bfr[reg][x & 3], acc[x >> 2][x & 3], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < cnt; ++c)
        if (x == (c * NM) / cnt + NM / cnt - 1) {
          __builtin_amdgcn_sched_barrier(0);
          copy(cs, cslot, u0 + c);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };
  // one stage: t in slot `slot`.  Copies of stage s go out during the second half of
  // stage s-NS and the first half of stage s-NS+1 (slot s % NS), i.e. after every wave
  // has read stage s-NS (its reads all precede the barrier in the middle of s-NS).
  // A wave whose 64-row slice lies wholly past the last row (the padding of a ragged
  // last row tile) only makes its share of the copies and leaves the matrix cores
  // to the other waves of its SIMD.
  const bool active = m0 + wm * (FM * 32) < g.M;
  auto stage = [&](int kt, int slot) __attribute__((always_inline)) {
    if (active) {
      frag(slot, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(0, kt + NS - 1, (slot + NS - 1) % NS, H0, H1);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int c = 0; c < H1; ++c) copy(kt + NS - 1, (slot + NS - 1) % NS, H0 + c);
    }
    CB_WAIT_VM(DQ * (NS - 2));     // this wave's copies of stage kt+1 have landed
    __syncthreads();               // ... everyone's
    if (active) {
      frag((slot + 1) % NS, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mma(1, kt + NS, slot, 0, H0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int c = 0; c < H0; ++c) copy(kt + NS, slot, c);
    }
  };

  // prologue: stages 0 .. NS-2 and the first half of stage NS-1 in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int u = 0; u < DQ; ++u) copy(s, s, u);
#pragma unroll
  for (int u = 0; u < H0; ++u) copy(NS - 1, NS - 1, u);
  CB_WAIT_VM(DQ * (NS - 2) + H0);
  __syncthreads();
  frag(0, 0, 0);
  // unrolled by NS so every ring slot is a compile-time constant
  int kt = 0;
  for (; kt + NS <= nk; kt += NS) {
#pragma unroll
    for (int r = 0; r < NS; ++r) stage(kt + r, r);
  }
#pragma unroll
  for (int r = 0; r < NS - 1; ++r)
    if (kt + r < nk) stage(kt + r, r);
  CB_WAIT_VM(0);                   // no copy may still be writing LDS when the workgroup ends

  // ---------------- epilogue ----------------
  // acc[i][j][v] holds C[row][col] with
  //   row = m0 + wm*FM*32 + i*32 + 8*(v/4) + 4*(lane/32) + v%4,  col = n0 + wn*128 + j*32 + lane%32.
  // Each 32-row slab of the wave's tile goes through the (now idle) LDS ring as a
  // row-major 32 x 128 fp32 block, so every lane then owns 4 adjacent columns:
  // RoPE pairs and SwiGLU gate/up partners are local, and rows are stored whole.
  __syncthreads();                                   // every wave is done with the ring
  constexpr int EP = T::EP;                          // row pitch (floats): the two half-waves hit different banks
  float* stg = reinterpret_cast<float*>(smem) + wid * (32 * EP);
  const int half = g.head_dim >> 1;
  const int row0 = m0 + wm * (FM * 32);
  const int col0 = n0 + wn * 128;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stg[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * EP + j * 32 + (lane & 31)] = acc[i][j][v];
    __builtin_amdgcn_wave_barrier();
    if (part) {
      const int c_part = dp_cols * BN;
      const int64_t wpart = b_rows - c_part;
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int r = p * 2 + (lane >> 5);
        const int c = (lane & 31) * 4;
        const int row = row0 + i * 32 + r;
        const int col = col0 + c;
        if (row < g.M && col < b_rows)
          *reinterpret_cast<float4*>(g.part + (static_cast<int64_t>(split) * g.M + row) * wpart + (col - c_part)) =
              *reinterpret_cast<const float4*>(stg + r * EP + c);
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      // gate columns [0,32) and [64,96) of the block pair with up columns +32
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int r = p * 4 + (lane >> 4);
        const int gc = ((lane >> 3) & 1) * 64 + (lane & 7) * 4;
        const float4 gt = *reinterpret_cast<const float4*>(stg + r * EP + gc);
        const float4 up = *reinterpret_cast<const float4*>(stg + r * EP + gc + 32);
        const int row = row0 + i * 32 + r;
        const int f = ((col0 + (gc & 64)) >> 6) * 32 + (gc & 31);
        if (row < g.M && f < g.N) {
          uint2 w;
          w.x = static_cast<uint32_t>(f2bf(silu(gt.x) * up.x)) | (static_cast<uint32_t>(f2bf(silu(gt.y) * up.y)) << 16);
          w.y = static_cast<uint32_t>(f2bf(silu(gt.z) * up.z)) | (static_cast<uint32_t>(f2bf(silu(gt.w) * up.w)) << 16);
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + pk_off(row, f, static_cast<int>(g.ldc))) = w;
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int r = p * 2 + (lane >> 5);
        const int c = (lane & 31) * 4;
        float4 x = *reinterpret_cast<const float4*>(stg + r * EP + c);
        const int row = row0 + i * 32 + r;
        const int col = col0 + c;
        if (row >= g.M || col >= g.N) continue;
        if constexpr (EPI == EPI_RESID) {
          const int rr = g.resid_rows ? g.resid_rows[row] : row;
          const float4 rv = *reinterpret_cast<const float4*>(g.resid + static_cast<int64_t>(rr) * g.ld_resid + col);
          *reinterpret_cast<float4*>(static_cast<float*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) =
              make_float4(rv.x + x.x, rv.y + x.y, rv.z + x.z, rv.w + x.w);
        } else if constexpr (EPI == EPI_QKV) {
          const int pos = g.row_pos[row];
          if (col < g.q_cols) {
            const float4 cs = *reinterpret_cast<const float4*>(g.rope_tab + static_cast<int64_t>(pos) * half + ((col % g.head_dim) >> 1));
            x = make_float4(x.x * cs.x - x.y * cs.y, x.x * cs.y + x.y * cs.x,
                            x.z * cs.z - x.w * cs.w, x.z * cs.w + x.w * cs.z);
            uint2 w;
            w.x = static_cast<uint32_t>(f2bf(x.x)) | (static_cast<uint32_t>(f2bf(x.y)) << 16);
            w.y = static_cast<uint32_t>(f2bf(x.z)) | (static_cast<uint32_t>(f2bf(x.w)) << 16);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) = w;
          } else {
            const int c2 = col - g.q_cols;
            if (c2 < g.rope2_cols) {
              const float4 cs = *reinterpret_cast<const float4*>(g.rope_tab + static_cast<int64_t>(pos) * half + ((c2 % g.head_dim) >> 1));
              x = make_float4(x.x * cs.x - x.y * cs.y, x.x * cs.y + x.y * cs.x,
                              x.z * cs.z - x.w * cs.w, x.z * cs.w + x.w * cs.z);
            }
            *reinterpret_cast<float4*>(g.C2 + static_cast<int64_t>(row) * g.ldc2 + c2) = x;
          }
        } else {   // EPI_STORE_ROPE / EPI_F32_ROPE
          if (col < g.rope_cols) {
            const int pos = g.row_pos[row];
            const float4 cs = *reinterpret_cast<const float4*>(g.rope_tab + static_cast<int64_t>(pos) * half + ((col % g.head_dim) >> 1));
            x = make_float4(x.x * cs.x - x.y * cs.y, x.x * cs.y + x.y * cs.x,
                            x.z * cs.z - x.w * cs.w, x.z * cs.w + x.w * cs.z);
          }
          if constexpr (EPI == EPI_STORE_ROPE) {
            uint2 w;
            w.x = static_cast<uint32_t>(f2bf(x.x)) | (static_cast<uint32_t>(f2bf(x.y)) << 16);
            w.y = static_cast<uint32_t>(f2bf(x.z)) | (static_cast<uint32_t>(f2bf(x.w)) << 16);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) = w;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) = x;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Split-K reduction in fixed split order, then the epilogue, over the virtual
// columns from c_part on (4 output columns per thread).  SWIGLU pairs gate
// column 64 k + j with up column 64 k + 32 + j into feature 32 k + j.
template <int EPI, int SP>   // SP > 0: the split count, known at compile time
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int splits, int c_part) {
  if constexpr (SP > 0) splits = SP;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int b_rows = (EPI == EPI_SWIGLU) ? 2 * g.N : g.N;
  const int64_t wpart = b_rows - c_part;
  if constexpr (EPI == EPI_SWIGLU) {
    const int f4 = (g.N - c_part / 2) / 4;             // output feature quads per row
    if (idx >= static_cast<int64_t>(g.M) * f4) return;
    const int row = static_cast<int>(idx / f4);
    const int fl = static_cast<int>(idx % f4) * 4;     // feature past c_part / 2
    const int gc = (fl >> 5) * 64 + (fl & 31);         // its gate column past c_part
    float4 gs = make_float4(0.f, 0.f, 0.f, 0.f), us = gs;
#pragma unroll
    for (int sp = 0; sp < splits; ++sp) {
      const float* pr = g.part + (static_cast<int64_t>(sp) * g.M + row) * wpart + gc;
      const float4 a = *reinterpret_cast<const float4*>(pr);
      const float4 u = *reinterpret_cast<const float4*>(pr + 32);
      gs.x += a.x; gs.y += a.y; gs.z += a.z; gs.w += a.w;
      us.x += u.x; us.y += u.y; us.z += u.z; us.w += u.w;
    }
    uint2 w;
    w.x = static_cast<uint32_t>(f2bf(silu(gs.x) * us.x)) | (static_cast<uint32_t>(f2bf(silu(gs.y) * us.y)) << 16);
    w.y = static_cast<uint32_t>(f2bf(silu(gs.z) * us.z)) | (static_cast<uint32_t>(f2bf(silu(gs.w) * us.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + pk_off(row, c_part / 2 + fl, static_cast<int>(g.ldc))) = w;
    return;
  }
  const int64_t n4 = wpart / 4;
  if (idx >= static_cast<int64_t>(g.M) * n4) return;
  const int row = static_cast<int>(idx / n4);
  const int lc = static_cast<int>(idx % n4) * 4;
  const int col = c_part + lc;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < splits; ++sp) {
    const float4 p = *reinterpret_cast<const float4*>(g.part + (static_cast<int64_t>(sp) * g.M + row) * wpart + lc);
    s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
  }
  float v[4] = {s.x, s.y, s.z, s.w};
  if constexpr (EPI == EPI_QKV) {
    const int p = g.row_pos[row];
    const int half = g.head_dim >> 1;
    const bool isq = col < g.q_cols;
    const int c = isq ? col : col - g.q_cols;
    if (isq || c < g.rope2_cols) {
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const float2 cs = g.rope_tab[static_cast<int64_t>(p) * half + (((c + j) % g.head_dim) >> 1)];
        const float x0 = v[j], x1 = v[j + 1];
        v[j] = x0 * cs.x - x1 * cs.y;
        v[j + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
    if (isq) {
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
      w.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + static_cast<int64_t>(row) * g.ldc + c) = w;
    } else {
      *reinterpret_cast<float4*>(g.C2 + static_cast<int64_t>(row) * g.ldc2 + c) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int rr = g.resid_rows ? g.resid_rows[row] : row;
    const float4 r = *reinterpret_cast<const float4*>(g.resid + static_cast<int64_t>(rr) * g.ld_resid + col);
    *reinterpret_cast<float4*>(static_cast<float*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) =
        make_float4(r.x + v[0], r.y + v[1], r.z + v[2], r.w + v[3]);
  } else {
    if (col < g.rope_cols) {
      const int p = g.row_pos[row];
      const int half = g.head_dim >> 1;
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const float2 cs = g.rope_tab[static_cast<int64_t>(p) * half + (((col + j) % g.head_dim) >> 1)];
        const float x0 = v[j], x1 = v[j + 1];
        v[j] = x0 * cs.x - x1 * cs.y;
        v[j + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
    if constexpr (EPI == EPI_STORE_ROPE) {
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
      w.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) = w;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(g.C) + static_cast<int64_t>(row) * g.ldc + col) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Split-K reduction of the fused Q/K/V product of a layer that keeps all of its
// candidate rows, with the blend's per-row work folded in (GemmArgs::blend): one
// workgroup per row writes the row maps of the (identity) top-k, sums the partials
// in split order, rotates Q and K at the
// row's position, stores Q (bf16), and for the K/V columns reads the cached row,
// adds the squared differences (candidate rows of a checked layer only; per
// thread in column order, then across the workgroup in a fixed order) and writes the fresh
// values over it (bf16, or FP8 divided by the tensor's scale).  T: the cache's
// element type; TPB threads per row.
template <typename T, int SP, int TPB = 256>
__global__ __launch_bounds__(TPB) void qkv_reduce_blend_kernel(GemmArgs g, int splits) {
  if constexpr (SP > 0) splits = SP;
  constexpr int NW = TPB / 64;
  __shared__ float red[NW];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int kvw = g.rope2_cols;
  const int wpart = g.q_cols + 2 * kvw;
  const int n4 = wpart >> 2;
  const int pos = g.row_pos[row];
  const int half = g.head_dim >> 1;
  const PagedRef& c = g.blend_cache;
  const int64_t off = static_cast<int64_t>(g.blend_layer) * c.layer_stride + paged_row(c, pos) * kvw;
  const bool cand = row < g.blend_nc;
  const bool measure = cand && g.blend_check;       // uniform over the workgroup
  if (tid == 0) {                                     // the row maps of an identity top-k
    if (g.blend_gmap) g.blend_gmap[row] = row;
    if (g.blend_rowpos) g.blend_rowpos[row] = pos;
    if (cand) {
      if (g.blend_pos_out) g.blend_pos_out[row] = pos;
      if (g.blend_slot) g.blend_slot[row] = row;
      if (g.blend_copy) g.blend_copy[row] = pos;
    }
  }
  float acc = 0.f;
  for (int j = tid; j < n4; j += TPB) {
    const int col = j * 4;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < splits; ++sp) {
      const float4 pv = *reinterpret_cast<const float4*>(g.part + (static_cast<int64_t>(sp) * g.M + row) * wpart + col);
      sum.x += pv.x; sum.y += pv.y; sum.z += pv.z; sum.w += pv.w;
    }
    float v[4] = {sum.x, sum.y, sum.z, sum.w};
    const bool isq = col < g.q_cols;
    const int c2 = isq ? col : col - g.q_cols;
    if (isq || c2 < kvw) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float2 cs = g.rope_tab[static_cast<int64_t>(pos) * half + (((c2 + e) % g.head_dim) >> 1)];
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs.x - x1 * cs.y;
        v[e + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
    if (isq) {
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
      w.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.C) + static_cast<int64_t>(row) * g.ldc + c2) = w;
      continue;
    }
    const bool isk = c2 < kvw;
    const int e0 = isk ? c2 : c2 - kvw;
    T* dst = static_cast<T*>(isk ? c.k : c.v) + off + e0;
    const float sc = isk ? c.ks : c.vs;
    if constexpr (sizeof(T) == 1) {
      if (measure) {
        float f[4];
        fp8x4_to_f32(*reinterpret_cast<const uint32_t*>(dst), f);
        const float d0 = v[0] - f[0] * sc, d1 = v[1] - f[1] * sc, d2 = v[2] - f[2] * sc, d3 = v[3] - f[3] * sc;
        acc += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
      }
      const float is = 1.0f / sc;
      *reinterpret_cast<uint32_t*>(dst) = f32_to_fp8x4(v[0] * is, v[1] * is, v[2] * is, v[3] * is);
    } else {
      if (measure) {
        const uint2 o = *reinterpret_cast<const uint2*>(dst);
        const float d0 = v[0] - bf2f(static_cast<bf16_t>(o.x & 0xFFFFu)), d1 = v[1] - bf2f(static_cast<bf16_t>(o.x >> 16));
        const float d2 = v[2] - bf2f(static_cast<bf16_t>(o.y & 0xFFFFu)), d3 = v[3] - bf2f(static_cast<bf16_t>(o.y >> 16));
        acc += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
      }
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(v[0])) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
      w.y = static_cast<uint32_t>(f2bf(v[2])) | (static_cast<uint32_t>(f2bf(v[3])) << 16);
      *reinterpret_cast<uint2*>(dst) = w;
    }
  }
  if (!measure) return;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float d = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) d += red[i];
    g.blend_dev[row] = d;
    if (g.blend_dev_by_pos) g.blend_dev_by_pos[pos] = d;
  }
}

template <typename T, int TPB>
hipError_t launch_qkv_reduce_blend_t(const GemmArgs& a, int eff, hipStream_t s) {
  switch (eff) {
    case 2: qkv_reduce_blend_kernel<T, 2, TPB><<<a.M, TPB, 0, s>>>(a, eff); break;
    case 3: qkv_reduce_blend_kernel<T, 3, TPB><<<a.M, TPB, 0, s>>>(a, eff); break;
    case 4: qkv_reduce_blend_kernel<T, 4, TPB><<<a.M, TPB, 0, s>>>(a, eff); break;
    default: qkv_reduce_blend_kernel<T, 0, TPB><<<a.M, TPB, 0, s>>>(a, eff); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_qkv_reduce_blend(const GemmArgs& a, int eff, hipStream_t s) {
  // wide rows (70B: 8192 Q + 2 x 1024 K/V columns) take 1024 threads, so each thread
  // has a few four-column groups instead of ten in a dependent chain
  if (a.q_cols + 2 * a.rope2_cols >= 8192) return launch_qkv_reduce_blend_t<T, 1024>(a, eff, s);
  return launch_qkv_reduce_blend_t<T, 256>(a, eff, s);
}

// Split-K reduction of a residual GEMM fused with the RMSNorm that follows it:
// one workgroup per row; x = resid + (partials summed in split order) is
// written fp32, then normalised (same reduction order as the RMSNorm kernel)
// into the fragment-major bf16 activations of the next GEMM.
constexpr int kNormChunks = 16;   // 16 x 1024 columns: d_model <= 16384

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Columns below c_part were finished by whole-tile workgroups of the same GEMM
// (resid added) and are read back from C.  NC > 0: the row is NC x 4 TPB columns
// (TPB threads, 4 columns each per chunk) and there are SP splits, all
// compile-time, so every load of the row (all partials, the residual) is issued
// before the first add; the sums keep split order.  NC = 0 (TPB 256): any width
// and split count.
template <int NC, int SP, int TPB = 256>
__global__ __launch_bounds__(TPB) void splitk_reduce_norm_kernel(GemmArgs g, int splits, int c_part) {
  static_assert(NC > 0 || TPB == 256, "the generic path runs 256 threads");
  constexpr int NW = TPB / 64;
  constexpr int CW = 4 * TPB;     // columns per chunk
  __shared__ float red[NW];
  // neighbouring rows on one XCD: their 16-byte pieces of a fragment-major block of
  // the normalised output meet in one L2 and leave it as whole lines
  const int row = xcd_remap(blockIdx.x, gridDim.x);
  const int rr = g.resid_rows ? g.resid_rows[row] : row;
  const int64_t wpart = g.N - c_part;
  constexpr int NCH = NC > 0 ? NC : kNormChunks;
  float4 v[NCH];
  float ss = 0.f;
  if constexpr (NC > 0) {
    float4 pp[NC][SP], rv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = threadIdx.x * 4 + c * CW;
      if (e < c_part) {
        v[c] = *reinterpret_cast<const float4*>(static_cast<const float*>(g.C) + static_cast<int64_t>(row) * g.ldc + e);
      } else {
#pragma unroll
        for (int sp = 0; sp < SP; ++sp)
          pp[c][sp] = *reinterpret_cast<const float4*>(g.part + (static_cast<int64_t>(sp) * g.M + row) * wpart + (e - c_part));
        rv[c] = *reinterpret_cast<const float4*>(g.resid + static_cast<int64_t>(rr) * g.ld_resid + e);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = threadIdx.x * 4 + c * CW;
      if (e >= c_part) {
        float4 sm = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sp = 0; sp < SP; ++sp) {
          sm.x += pp[c][sp].x; sm.y += pp[c][sp].y; sm.z += pp[c][sp].z; sm.w += pp[c][sp].w;
        }
        v[c] = make_float4(rv[c].x + sm.x, rv[c].y + sm.y, rv[c].z + sm.z, rv[c].w + sm.w);
        *reinterpret_cast<float4*>(static_cast<float*>(g.C) + static_cast<int64_t>(row) * g.ldc + e) = v[c];
      }
      ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < kNormChunks; ++c) {
      const int e = threadIdx.x * 4 + c * 1024;
      if (e < g.N) {
        float* cp = static_cast<float*>(g.C) + static_cast<int64_t>(row) * g.ldc + e;
        if (e < c_part) {
          v[c] = *reinterpret_cast<const float4*>(cp);
        } else {
          float4 sm = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int sp = 0; sp < splits; ++sp) {
            const float4 p = *reinterpret_cast<const float4*>(g.part + (static_cast<int64_t>(sp) * g.M + row) * wpart + (e - c_part));
            sm.x += p.x; sm.y += p.y; sm.z += p.z; sm.w += p.w;
          }
          const float4 r = *reinterpret_cast<const float4*>(g.resid + static_cast<int64_t>(rr) * g.ld_resid + e);
          v[c] = make_float4(r.x + sm.x, r.y + sm.y, r.z + sm.z, r.w + sm.w);
          *reinterpret_cast<float4*>(cp) = v[c];
        }
        ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
      }
    }
  }
  ss = wave_sum64(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float part[NW];                  // the waves' sums, added pairwise in a fixed tree
#pragma unroll
  for (int i = 0; i < NW; ++i) part[i] = red[i];
#pragma unroll
  for (int h = NW / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int i = 0; i < h; ++i) part[i] = part[2 * i] + part[2 * i + 1];
  const float tot = part[0];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(g.N) + g.norm_eps);
  bf16_t* out = static_cast<bf16_t*>(g.norm_out);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = threadIdx.x * 4 + c * (NC > 0 ? CW : 1024);
    if (NC > 0 || e < g.N) {
      const float4 gg = *reinterpret_cast<const float4*>(g.norm_gain + e);
      uint2 w;
      w.x = static_cast<uint32_t>(f2bf(v[c].x * inv * gg.x)) | (static_cast<uint32_t>(f2bf(v[c].y * inv * gg.y)) << 16);
      w.y = static_cast<uint32_t>(f2bf(v[c].z * inv * gg.z)) | (static_cast<uint32_t>(f2bf(v[c].w * inv * gg.w)) << 16);
      *reinterpret_cast<uint2*>(out + pk_off(row, e, g.N)) = w;
    }
  }
}

template <int NC, int TPB>
hipError_t launch_reduce_norm_nc(const GemmArgs& a, int eff, int c_part, hipStream_t s) {
  switch (eff) {
    case 2: splitk_reduce_norm_kernel<NC, 2, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    case 3: splitk_reduce_norm_kernel<NC, 3, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    case 4: splitk_reduce_norm_kernel<NC, 4, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    case 5: splitk_reduce_norm_kernel<NC, 5, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    case 6: splitk_reduce_norm_kernel<NC, 6, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    case 7: splitk_reduce_norm_kernel<NC, 7, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    case 8: splitk_reduce_norm_kernel<NC, 8, TPB><<<a.M, TPB, 0, s>>>(a, eff, c_part); break;
    default: splitk_reduce_norm_kernel<0, 0><<<a.M, 256, 0, s>>>(a, eff, c_part); break;
  }
  return hipGetLastError();
}

hipError_t launch_reduce_norm(const GemmArgs& a, int eff, int c_part, hipStream_t s) {
  // 8192-wide rows with more than 4 splits: 1024 threads, 8 columns of every split per
  // thread, all loads in flight at once (70B width, 678 rows: the down product's 5
  // splits 44.6 -> 34.5 us, layer 0's 8 splits 106.9 -> 81.6 us); with up to 4 splits
  // 256 threads x 32 columns stay ahead (2 splits: 24.6 against 26.2 us), as do
  // 4096-wide rows
  if (a.N == 4096) return launch_reduce_norm_nc<4, 256>(a, eff, c_part, s);
  if (a.N == 8192 && eff <= 4) return launch_reduce_norm_nc<8, 256>(a, eff, c_part, s);
  if (a.N == 8192) return launch_reduce_norm_nc<2, 1024>(a, eff, c_part, s);
  splitk_reduce_norm_kernel<0, 0><<<a.M, 256, 0, s>>>(a, eff, c_part);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64x64x16 tiles, 256 threads, 4x4 outputs per thread
// ---------------------------------------------------------------------------
constexpr int FM = 64, FN = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[FK][FM + 4];
  __shared__ float Bs[FK][FN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m_tiles = (g.M + FM - 1) / FM;
  const int t = blockIdx.x;
  const int mt = t % m_tiles, nt = t / m_tiles;
  const int m0 = mt * FM;
  const int n0 = (EPI == EPI_SWIGLU) ? nt * (FN / 2) : nt * FN;
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B);

  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const float* ap = nullptr;
  {
    const int m = m0 + lr;
    if (m < g.M) ap = A + static_cast<int64_t>(g.a_rows ? g.a_rows[m] : m) * g.lda + lk;
  }
  const float* bp = nullptr;
  {
    int r;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      const int f = n0 + (lr >> 1);
      ok = f < g.N;
      r = (lr & 1) ? g.ff + f : f;
    } else {
      r = n0 + lr;
      ok = r < g.N;
    }
    if (ok) bp = B + static_cast<int64_t>(r) * g.ldb + lk;
  }
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += FK) {
    const float4 a = ap ? *reinterpret_cast<const float4*>(ap + k0) : make_float4(0, 0, 0, 0);
    const float4 b = bp ? *reinterpret_cast<const float4*>(bp + k0) : make_float4(0, 0, 0, 0);
    As[lk + 0][lr] = a.x; As[lk + 1][lr] = a.y; As[lk + 2][lr] = a.z; As[lk + 3][lr] = a.w;
    Bs[lk + 0][lr] = b.x; Bs[lk + 1][lr] = b.y; Bs[lk + 2][lr] = b.z; Bs[lk + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
  const int half = g.head_dim >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= g.M) continue;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int f = n0 + tx * 2 + p;
        if (f < g.N)
          static_cast<float*>(g.C)[static_cast<int64_t>(row) * g.ldc + f] = silu(acc[i][2 * p]) * acc[i][2 * p + 1];
      }
    } else if constexpr (EPI == EPI_RESID) {
      const int rr = g.resid_rows ? g.resid_rows[row] : row;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < g.N)
          static_cast<float*>(g.C)[static_cast<int64_t>(row) * g.ldc + col] =
              g.resid[static_cast<int64_t>(rr) * g.ld_resid + col] + acc[i][j];
      }
    } else {
      float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      const int c0 = n0 + tx * 4;
      if (c0 < g.rope_cols) {
        const int p = g.row_pos[row];
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const float2 cs = g.rope_tab[static_cast<int64_t>(p) * half + (((c0 + j) % g.head_dim) >> 1)];
          const float x0 = v[j], x1 = v[j + 1];
          v[j] = x0 * cs.x - x1 * cs.y;
          v[j + 1] = x0 * cs.y + x1 * cs.x;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = c0 + j;
        if (col < g.N) static_cast<float*>(g.C)[static_cast<int64_t>(row) * g.ldc + col] = v[j];
      }
    }
  }
}

template <int EPI, int CFG, bool SPLIT>
hipError_t launch_cfg(int wgs, const GemmArgs& a, int splits, int kps, int dp_cols, hipStream_t s) {
  gemm_bf16_kernel<EPI, CFG, SPLIT><<<wgs, Tile<CFG>::kThreads, 0, s>>>(a, splits, kps, dp_cols);
  return hipGetLastError();
}

inline int bm_of(int cfg) { return cfg == GEMM_CFG_128 ? 128 : 256; }

inline int b_rows_of(const GemmArgs& a, int epi) { return (epi == EPI_SWIGLU) ? 2 * a.N : a.N; }
inline int m_tiles_of(const GemmArgs& a, int bm) { return (a.M + bm - 1) / bm; }
inline int n_tiles_of(const GemmArgs& a, int epi) { return (b_rows_of(a, epi) + BN - 1) / BN; }

// k columns per split (a multiple of BK) and the number of non-empty splits
inline void split_k(int K, int splits, int* kps, int* eff) {
  const int nkb = K / BK;
  const int per = (nkb + splits - 1) / splits;
  *kps = per * BK;
  *eff = (nkb + per - 1) / per;
}

// Cost model, calibrated on the GEMM microbenchmark with random bf16 data at the
// 8B blend shapes.  Workgroups run at a per-workgroup rate that rises as fewer
// CUs are busy (the chip is power-limited under MFMA load): 256-row tiles (one
// per CU) ~5.2 TFLOP/s x (256/b)^0.4 on b busy CUs; 128-row tiles two per CU ~2.6
// each, one per CU ~3.9 x (256/b)^0.4 (the gain capped at 1.25).  The fixed-order
// reduction moves the fp32 partials once (write + read) at ~8 TB/s plus a launch.
inline double busy_scale(int64_t b) { return b >= 256 ? 1.0 : fmin(1.25, pow(256.0 / static_cast<double>(b), 0.4)); }

inline double wg_rate(int bm, int64_t wgs) {   // FLOP/s of one workgroup while `wgs` run at once
  if (bm == 256) return 5.2e12 * busy_scale(std::min<int64_t>(wgs, 256));
  return wgs > 256 ? 2.6e12 : 3.9e12 * busy_scale(wgs);
}

// Whole tiles (nk k-steps each) are dispatched first, in full rounds of S
// workgroups; the r left over run beside the pieces (pk steps each), whose
// slots meanwhile take further pieces; what is left of the pieces then runs in
// rounds of S.
inline double est_time(const GemmArgs& a, int epi, int cfg, int splits, int dp_cols) {
  const int bm = bm_of(cfg);
  int kps, eff;
  split_k(a.K, splits, &kps, &eff);
  const int64_t mtl = m_tiles_of(a, bm), ntl = n_tiles_of(a, epi);
  const int64_t dpc = eff > 1 ? std::min<int64_t>(dp_cols, ntl) : ntl;
  const int64_t S = bm == 256 ? 256 : 512;
  const double sf = 2.0 * bm * BN * BK;            // FLOP of one k-step of a workgroup
  const int64_t nk = a.K / BK, pk = kps / BK;
  const int64_t n_dp = mtl * dpc, np = mtl * (ntl - dpc) * eff;
  const int64_t r = n_dp % S;
  double tm = static_cast<double>(n_dp / S) * nk * sf / wg_rate(bm, S);
  int64_t left = np;
  if (r > 0) {
    tm += nk * sf / wg_rate(bm, std::min(S, r + np));
    left -= std::min(left, (S - r) * (nk / pk));
  }
  tm += static_cast<double>(left / S) * pk * sf / wg_rate(bm, S);
  if (left % S) tm += pk * sf / wg_rate(bm, left % S);
  if (eff > 1) tm += static_cast<double>(eff) * a.M * (b_rows_of(a, epi) - dpc * BN) * 8.0 / 8e12 + 3e-6;
  return tm;
}

inline bool part_fits(const GemmArgs& a, int epi, int eff, int dp_cols) {
  return a.part != nullptr &&
         static_cast<int64_t>(eff) * a.M * (b_rows_of(a, epi) - static_cast<int64_t>(dp_cols) * BN) <= a.part_floats;
}

}  // namespace

// A hybrid plan (whole tiles plus split remainder) must beat the best plain plan
// by 10%: its short pieces and their partials cost more than the model counts
// (measured: 678 x 28672 x 4096 SwiGLU, predicted 3% faster, ran 5% slower).
void choose_gemm_cfg(const GemmArgs& a, int epi, int* cfg, int* splits, int* dp_cols) {
  *cfg = GEMM_CFG_256;
  *splits = 1;
  *dp_cols = 0;
  double best = est_time(a, epi, GEMM_CFG_256, 1, 0);
  int h_cfg = 0, h_splits = 0, h_dp = 0;
  double h_best = 0.0;
  for (int c : {GEMM_CFG_256, GEMM_CFG_128}) {
    const int bm = bm_of(c);
    const int mtl = m_tiles_of(a, bm), ntl = n_tiles_of(a, epi);
    const int64_t S = bm == 256 ? 256 : 512;
    for (int sp = 1; sp <= 8; ++sp) {
      if (sp > 1 && a.part == nullptr) break;
      if (a.K / sp < 256) break;
      int kps, eff;
      split_k(a.K, sp, &kps, &eff);
      // whole-tile column counts: none (plain split-K) or as many as fill k full rounds
      int opts[9];
      int n_opts = 0;
      if (eff == 1) {
        opts[n_opts++] = 0;
      } else {
        opts[n_opts++] = 0;
        for (int64_t k = 1; k * S <= static_cast<int64_t>(mtl) * ntl && n_opts < 9; ++k) {
          const int d = static_cast<int>(k * S / mtl);
          if (d > 0 && d < ntl) opts[n_opts++] = d;
        }
      }
      for (int o = 0; o < n_opts; ++o) {
        if (eff > 1 && !part_fits(a, epi, eff, opts[o])) continue;
        const double tm = est_time(a, epi, c, sp, opts[o]);
        if (opts[o] > 0) {
          if (h_splits == 0 || tm < h_best) {
            h_best = tm;
            h_cfg = c;
            h_splits = sp;
            h_dp = opts[o];
          }
        } else if (tm < best * 0.97) {
          best = tm;
          *cfg = c;
          *splits = sp;
        }
      }
    }
  }
  if (h_splits > 0 && h_best < 0.9 * best) {
    *cfg = h_cfg;
    *splits = h_splits;
    *dp_cols = h_dp;
  }
}

namespace {

// *normed: set when the RMSNorm of a residual GEMM's output, or the blend work of a
// Q/K/V product (GemmArgs::blend), was fused into the reduction
template <int EPI, int CFG>
hipError_t run_bm(const GemmArgs& a, int splits, int dp_cols, hipStream_t s, bool* normed) {
  constexpr int BM = Tile<CFG>::BM;
  int kps, eff;
  split_k(a.K, splits, &kps, &eff);
  const int mtl = m_tiles_of(a, BM), ntl = n_tiles_of(a, EPI);
  if (eff > 1 && dp_cols < ntl) {
    if (dp_cols < 0 || !part_fits(a, EPI, eff, dp_cols)) return hipErrorInvalidValue;
    const int wgs = mtl * dp_cols + mtl * (ntl - dp_cols) * eff;
    hipError_t e = launch_cfg<EPI, CFG, true>(wgs, a, eff, kps, dp_cols, s);
    if (e != hipSuccess) return e;
    const int c_part = dp_cols * BN;
    if (EPI == EPI_RESID && a.norm_out != nullptr && a.N <= kNormChunks * 1024) {
      e = launch_reduce_norm(a, eff, c_part, s);
      if (e != hipSuccess) return e;
      *normed = true;
    } else if (EPI == EPI_QKV && a.blend && c_part == 0) {
      e = a.blend_cache.fp8 ? launch_qkv_reduce_blend<fp8_t>(a, eff, s) : launch_qkv_reduce_blend<bf16_t>(a, eff, s);
      if (e != hipSuccess) return e;
      *normed = true;
    } else {
      const int64_t n = (EPI == EPI_SWIGLU) ? static_cast<int64_t>(a.M) * ((a.N - c_part / 2) / 4)
                                            : static_cast<int64_t>(a.M) * ((b_rows_of(a, EPI) - c_part) / 4);
      const int nb = static_cast<int>((n + 255) / 256);
      switch (eff) {
        case 2: splitk_reduce_kernel<EPI, 2><<<nb, 256, 0, s>>>(a, eff, c_part); break;
        case 3: splitk_reduce_kernel<EPI, 3><<<nb, 256, 0, s>>>(a, eff, c_part); break;
        case 4: splitk_reduce_kernel<EPI, 4><<<nb, 256, 0, s>>>(a, eff, c_part); break;
        default: splitk_reduce_kernel<EPI, 0><<<nb, 256, 0, s>>>(a, eff, c_part); break;
      }
    }
    return hipGetLastError();
  }
  return launch_cfg<EPI, CFG, false>(mtl * ntl, a, 1, a.K, ntl, s);
}

template <int EPI>
hipError_t run_cfg(const GemmArgs& a, int cfg, int splits, int dp_cols, hipStream_t s, bool* normed) {
  if (a.K % BK != 0 || a.K <= 0) return hipErrorInvalidValue;
  if (EPI == EPI_SWIGLU && a.N % 32 != 0) return hipErrorInvalidValue;
  if (splits > 1 && a.N % 4 != 0) return hipErrorInvalidValue;
  if (cfg == GEMM_CFG_256) return run_bm<EPI, GEMM_CFG_256>(a, splits, dp_cols, s, normed);
  if (cfg == GEMM_CFG_128) return run_bm<EPI, GEMM_CFG_128>(a, splits, dp_cols, s, normed);
  return hipErrorInvalidValue;
}

template <int EPI>
hipError_t run_gemm(cb_dtype dt, const GemmArgs& a, hipStream_t s, bool* blend_done) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  bool normed = false;
  hipError_t e;
  if (dt != CB_BF16) {
    if constexpr (EPI == EPI_QKV) return hipErrorInvalidValue;   // bf16 only
    const int m_tiles = (a.M + FM - 1) / FM;
    const int n_tiles = (EPI == EPI_SWIGLU) ? (a.N + FN / 2 - 1) / (FN / 2) : (a.N + FN - 1) / FN;
    gemm_f32_kernel<EPI><<<m_tiles * n_tiles, 256, 0, s>>>(a);
    e = hipGetLastError();
  } else {
    int cfg, splits, dp_cols;
    choose_gemm_cfg(a, EPI, &cfg, &splits, &dp_cols);
    e = run_cfg<EPI>(a, cfg, splits, dp_cols, s, &normed);
  }
  if (EPI == EPI_QKV && blend_done) *blend_done = e == hipSuccess && normed;
  if (e != hipSuccess || EPI != EPI_RESID || a.norm_out == nullptr || normed) return e;
  return launch_rmsnorm(dt, static_cast<const float*>(a.C), nullptr, a.ldc, a.M, a.N, a.norm_gain, a.norm_eps, a.norm_out,
                        a.N, 0, s);
}

}  // namespace

hipError_t launch_gemm_cfg(GemmEpi epi, const GemmArgs& a, int cfg, int splits, int dp_cols, hipStream_t s) {
  bool normed = false;
  switch (epi) {
    case EPI_STORE_ROPE: return run_cfg<EPI_STORE_ROPE>(a, cfg, splits, dp_cols, s, &normed);
    case EPI_F32_ROPE: return run_cfg<EPI_F32_ROPE>(a, cfg, splits, dp_cols, s, &normed);
    case EPI_RESID: return run_cfg<EPI_RESID>(a, cfg, splits, dp_cols, s, &normed);
    case EPI_SWIGLU: return run_cfg<EPI_SWIGLU>(a, cfg, splits, dp_cols, s, &normed);
    case EPI_QKV: return run_cfg<EPI_QKV>(a, cfg, splits, dp_cols, s, &normed);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(cb_dtype dt, GemmEpi epi, const GemmArgs& a, hipStream_t s, bool* blend_done) {
  if (blend_done) *blend_done = false;
  switch (epi) {
    case EPI_STORE_ROPE: return run_gemm<EPI_STORE_ROPE>(dt, a, s, nullptr);
    case EPI_F32_ROPE: return run_gemm<EPI_F32_ROPE>(dt, a, s, nullptr);
    case EPI_RESID: return run_gemm<EPI_RESID>(dt, a, s, nullptr);
    case EPI_SWIGLU: return run_gemm<EPI_SWIGLU>(dt, a, s, nullptr);
    case EPI_QKV: return run_gemm<EPI_QKV>(dt, a, s, blend_done);
  }
  return hipErrorInvalidValue;
}

}  // namespace cb
