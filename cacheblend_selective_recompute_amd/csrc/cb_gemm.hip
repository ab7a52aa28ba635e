// Gather-GEMM of the selected rows: C[M][N] = A[M][:] . B[n][:] with the
// epilogues the decoder block needs fused in (RoPE of Q/K at the rows'
// positions, residual add with a row gather, SiLU-gated MLP).
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn), Fig. 5 -- only the
// selected tokens go through the projections; the recompute cost is
// proportional to the selected share (section "选 token").
//
// bf16 path: v_mfma_f32_32x32x16_bf16, 4 waves in a 2x2 grid, block tile
// (2 WTM) x (2 WTN) x 64.  Weight tiles are staged through LDS (row pitch padded
// by 16 B so the 32 rows one fragment read touches fall in distinct banks; two
// buffers so the next tile is in flight while the current one is multiplied);
// activations arrive fragment-major (see pk_off) from the kernels that produce
// them, so each A fragment is one contiguous 1 KiB wave load straight into
// registers.  The tile shape and a split of K are chosen per call from measured
// per-configuration rates so the grid fills the 256 CUs; split-K partials are
// reduced in a fixed order by a second kernel that also applies the epilogue.
// Tiles are ordered M-fastest and mapped so consecutive tiles land on the same
// XCD, so the M tiles that share one weight tile share that XCD's L2.
// fp32 path: a plain LDS-tiled FMA kernel (fp32 models are small).
#include <algorithm>

#include "cb_internal.h"

namespace cb {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDSP = BK + 8;   // LDS row pitch in bf16 elements (144 B)
constexpr int kThreads = 256;
constexpr int kXcd = 8;

// Linear block id -> logical tile id such that the hardware's round-robin
// dispatch over XCDs gives each XCD a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb / kXcd, r = nb % kXcd;
  const int x = b % kXcd, i = b / kXcd;
  return x * q + min(x, r) + i;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Weights (B) are staged through LDS; the gathered activation rows (A) go
// straight from global memory into MFMA A-fragments: every wave owns WTM rows
// and WTN columns, waves sharing a row range read the same A lines (L1/L2 hits).
// WTM x WTN = 128 x 128 keeps 256 fp32 accumulators per lane (AGPRs) and needs
// 3/8 of the LDS bandwidth of the matrix cores per k step.
template <int EPI, int WTM, int WTN, bool SPLIT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs g, int splits, int kps) {
  constexpr int BM = 2 * WTM, BN = 2 * WTN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int NB = BN * (BK / 8) / kThreads;      // 16-byte B chunks per thread per k block
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDSP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  const int m_tiles = (g.M + BM - 1) / BM;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = t % m_tiles;
  const int rest = t / m_tiles;
  const int split = rest % splits;
  const int nt = rest / splits;
  const int m0 = mt * BM;
  const int n0 = (EPI == EPI_SWIGLU) ? nt * (BN / 2) : nt * BN;
  const int kbeg = split * kps;
  const int kend = min(g.K, kbeg + kps);
  const int nk = (kend - kbeg) / BK;

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.B);

  const int kb_per_row = g.K >> 4;
  const int mb_valid = (g.M + 31) >> 5;
  const bf16_t* arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int mb = (m0 + wm * WTM + i * 32) >> 5;
    arow[i] = (mb < mb_valid) ? A + (static_cast<int64_t>(mb) * kb_per_row * 64 + lane) * 8 : nullptr;
  }
  // B staging chunks of this thread
  const bf16_t* brow[NB];
  int lrow[NB], lcol[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int c = tid + u * kThreads;
    lrow[u] = c >> 3;
    lcol[u] = (c & 7) * 8;
    int bi;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      const int r = lrow[u];
      const int g32 = r >> 5;
      const int f = n0 + (g32 >> 1) * 32 + (r & 31);
      ok = f < g.N;
      bi = (g32 & 1) ? g.ff + f : f;
    } else {
      bi = n0 + lrow[u];
      ok = bi < g.N;
    }
    brow[u] = ok ? B + static_cast<int64_t>(bi) * g.ldb + lcol[u] : nullptr;
  }

  typedef uint4 AFrag[BK / 16][FM];
  AFrag acur, anxt;
  uint4 breg[NB];
  auto load_a = [&](AFrag& dst, int k0) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        dst[ks][i] = arow[i] ? *reinterpret_cast<const uint4*>(arow[i] + static_cast<int64_t>((k0 >> 4) + ks) * 512)
                             : make_uint4(0, 0, 0, 0);
  };
  auto load_b = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      breg[u] = brow[u] ? *reinterpret_cast<const uint4*>(brow[u] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NB; ++u) *reinterpret_cast<uint4*>(&Bs[buf][lrow[u] * LDSP + lcol[u]]) = breg[u];
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (nk > 0) {
    load_b(kbeg);
    load_a(acur, kbeg);
    store_b(0);
  }
  __syncthreads();
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const int knext = kbeg + (kt + 1) * BK;
    if (kt + 1 < nk) {
      load_b(knext);
      load_a(anxt, knext);
    }
    const bf16_t* bs = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t bfr[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&bs[(wn * WTN + j * 32 + fr) * LDSP + ks * 16 + fk]);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, acur[ks][i]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) {
      store_b(buf ^ 1);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i) acur[ks][i] = anxt[ks][i];
    }
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  // acc[i][j][v] holds C[row][col] with
  //   row = m0 + wm*WTM + i*32 + 8*(v/4) + 4*(lane/32) + v%4,  col = wn*WTN + j*32 + lane%32
  const int half = g.head_dim >> 1;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const bool rok = row < g.M;
      if constexpr (SPLIT) {
        float* prow = g.part + (static_cast<int64_t>(split) * g.M + row) * g.N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WTN + j * 32 + (lane & 31);
          if (rok && col < g.N) prow[col] = acc[i][j][v];
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < FN; j += 2) {
          const int f = n0 + wn * (WTN / 2) + (j / 2) * 32 + (lane & 31);
          if (rok && f < g.N) {
            const float h = silu(acc[i][j][v]) * acc[i][j + 1][v];
            static_cast<bf16_t*>(g.C)[pk_off(row, f, static_cast<int>(g.ldc))] = f2bf(h);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WTN + j * 32 + (lane & 31);
          float val = acc[i][j][v];
          if constexpr (EPI == EPI_STORE_ROPE || EPI == EPI_F32_ROPE) {
            const float other = __shfl_xor(val, 1, 64);
            if (rok && col < g.rope_cols) {
              const int p = g.row_pos[row];
              const float2 cs = g.rope_tab[static_cast<int64_t>(p) * half + ((col % g.head_dim) >> 1)];
              val = (col & 1) ? (other * cs.y + val * cs.x) : (val * cs.x - other * cs.y);
            }
            if (rok && col < g.N) {
              if constexpr (EPI == EPI_STORE_ROPE)
                static_cast<bf16_t*>(g.C)[static_cast<int64_t>(row) * g.ldc + col] = f2bf(val);
              else
                static_cast<float*>(g.C)[static_cast<int64_t>(row) * g.ldc + col] = val;
            }
          } else {  // EPI_RESID
            if (rok && col < g.N) {
              const int rr = g.resid_rows ? g.resid_rows[row] : row;
              const float r = g.resid[static_cast<int64_t>(rr) * g.ld_resid + col];
              static_cast<float*>(g.C)[static_cast<int64_t>(row) * g.ldc + col] = r + val;
            }
          }
        }
      }
    }
  }
}

// Split-K reduction in fixed split order, then the epilogue (4 columns per thread).
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int splits) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int n4 = g.N / 4;
  if (idx >= static_cast<int64_t>(g.M) * n4) return;
  const int row = static_cast<int>(idx / n4);
  const int col = static_cast<int>(idx % n4) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < splits; ++sp) {
    const float4 p = *reinterpret_cast<const float4*>(g.part + (static_cast<int64_t>(sp) * g.M + row) * g.N + col);
    s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
  }
  float v[4] = {s.x, s.y, s.z, s.w};
  if constexpr (EPI == EPI_RESID) {
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

template <int EPI, int WTM, int WTN, bool SPLIT>
hipError_t launch_cfg(const GemmArgs& a, int tiles, int splits, int kps, hipStream_t s) {
  gemm_bf16_kernel<EPI, WTM, WTN, SPLIT><<<tiles * splits, kThreads, 0, s>>>(a, splits, kps);
  return hipGetLastError();
}

inline int tiles_of(const GemmArgs& a, int epi, int bm, int bn) {
  const int mt = (a.M + bm - 1) / bm;
  const int nt = (epi == EPI_SWIGLU) ? (a.N + bn / 2 - 1) / (bn / 2) : (a.N + bn - 1) / bn;
  return mt * nt;
}

// Split-K cost model for the 128x128 tile, calibrated on the GEMM
// microbenchmark: a workgroup computes 2*128*128*k FLOP at ~2.2 TFLOP/s when it
// has a CU to itself and ~1.65 TFLOP/s when two share one (two fit per CU);
// workgroups run in rounds of 512; the fixed-order reduction moves the fp32
// partials once (write + read) at ~5 TB/s plus a launch.
inline double est_time_128(const GemmArgs& a, int epi, int splits) {
  const int64_t wgs = static_cast<int64_t>(tiles_of(a, epi, 128, 128)) * splits;
  const double flop_wg = 2.0 * 128 * 128 * (static_cast<double>(a.K) / splits);
  double tm;
  if (wgs <= 256) tm = flop_wg / 2.2e12;
  else tm = static_cast<double>((wgs + 511) / 512) * flop_wg / 1.65e12;
  if (splits > 1) tm += static_cast<double>(splits) * a.M * a.N * 8.0 / 5e12 + 3e-6;
  return tm;
}

}  // namespace

void choose_gemm_cfg(const GemmArgs& a, int epi, int* cfg, int* splits) {
  // the 128x128 tile (two workgroups per CU) is at least as fast per CU as the
  // larger tiles at every blend shape measured, and quantises better
  *cfg = GEMM_CFG_128x128;
  *splits = 1;
  if (epi == EPI_SWIGLU || a.part == nullptr) return;
  double best = est_time_128(a, epi, 1);
  for (int sp = 2; sp <= 8; ++sp) {
    if (a.K / sp < 512) break;
    if (static_cast<int64_t>(sp) * a.M * a.N > a.part_floats) break;
    const double tm = est_time_128(a, epi, sp);
    if (tm < best * 0.97) {
      best = tm;
      *splits = sp;
    }
  }
}

namespace {

template <int EPI>
hipError_t run_cfg(const GemmArgs& a, int cfg, int splits, hipStream_t s) {
  if (splits > 1) {
    if constexpr (EPI == EPI_SWIGLU) return hipErrorInvalidValue;
    const int t = tiles_of(a, EPI, 128, 128);
    const int kps = ((a.K / BK + splits - 1) / splits) * BK;
    hipError_t e = launch_cfg<EPI, 64, 64, true>(a, t, splits, kps, s);
    if (e != hipSuccess) return e;
    const int64_t n = static_cast<int64_t>(a.M) * (a.N / 4);
    splitk_reduce_kernel<EPI><<<static_cast<int>((n + 255) / 256), 256, 0, s>>>(a, splits);
    return hipGetLastError();
  }
  switch (cfg) {
    case GEMM_CFG_256x256: return launch_cfg<EPI, 128, 128, false>(a, tiles_of(a, EPI, 256, 256), 1, a.K, s);
    case GEMM_CFG_128x256: return launch_cfg<EPI, 64, 128, false>(a, tiles_of(a, EPI, 128, 256), 1, a.K, s);
    default: return launch_cfg<EPI, 64, 64, false>(a, tiles_of(a, EPI, 128, 128), 1, a.K, s);
  }
}

template <int EPI>
hipError_t run_gemm(cb_dtype dt, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (dt != CB_BF16) {
    const int m_tiles = (a.M + FM - 1) / FM;
    const int n_tiles = (EPI == EPI_SWIGLU) ? (a.N + FN / 2 - 1) / (FN / 2) : (a.N + FN - 1) / FN;
    gemm_f32_kernel<EPI><<<m_tiles * n_tiles, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  int cfg, splits;
  choose_gemm_cfg(a, EPI, &cfg, &splits);
  return run_cfg<EPI>(a, cfg, splits, s);
}

}  // namespace

hipError_t launch_gemm_cfg(GemmEpi epi, const GemmArgs& a, int cfg, int splits, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_ROPE: return run_cfg<EPI_STORE_ROPE>(a, cfg, splits, s);
    case EPI_F32_ROPE: return run_cfg<EPI_F32_ROPE>(a, cfg, splits, s);
    case EPI_RESID: return run_cfg<EPI_RESID>(a, cfg, splits, s);
    case EPI_SWIGLU: return run_cfg<EPI_SWIGLU>(a, cfg, splits, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(cb_dtype dt, GemmEpi epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_ROPE: return run_gemm<EPI_STORE_ROPE>(dt, a, s);
    case EPI_F32_ROPE: return run_gemm<EPI_F32_ROPE>(dt, a, s);
    case EPI_RESID: return run_gemm<EPI_RESID>(dt, a, s);
    case EPI_SWIGLU: return run_gemm<EPI_SWIGLU>(dt, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace cb
