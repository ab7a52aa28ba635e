// Gather-GEMM of the selected rows: C[M][N] = A[a_rows[m]][:] . B[n][:]
// with the epilogues the decoder block needs fused in (RoPE of Q/K at the
// rows' positions, residual add with a row gather, SiLU-gated MLP).
//
// Method: "CacheBlend 完全拆解" (pinghaoyang.com.cn), Fig. 5 -- only the
// selected tokens go through the projections; the recompute cost is
// proportional to the selected share (section "选 token").
//
// bf16 path: v_mfma_f32_32x32x16_bf16, 128x128x64 block tile, 4 waves in a
// 2x2 grid of 64x64 wave tiles, A and B tiles staged through LDS (row pitch
// padded by 16 B so the 32 rows a fragment read touches fall in distinct
// banks), two LDS buffers so the next global tile is in flight while the
// current one is multiplied.  Tiles are ordered M-fastest and mapped so that
// consecutive tiles land on the same XCD: the M tiles that share one weight
// tile then share that XCD's L2.
// fp32 path: a plain LDS-tiled FMA kernel (fp32 models are small).
#include "cb_internal.h"

namespace cb {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
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

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDSP];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDSP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  const int m_tiles = (g.M + BM - 1) / BM;
  const int nb = gridDim.x;
  const int t = xcd_remap(blockIdx.x, nb);
  const int mt = t % m_tiles, nt = t / m_tiles;
  const int m0 = mt * BM;
  // SWIGLU: a tile covers 64 features (32 gate + 32 up rows per wave column)
  const int n0 = (EPI == EPI_SWIGLU) ? nt * (BN / 2) : nt * BN;

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.B);

  // per-thread global source rows for its 4 A chunks and 4 B chunks
  const bf16_t* arow[4];
  const bf16_t* brow[4];
  int lrow[4], lcol[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + u * kThreads;  // 0..1023
    lrow[u] = c >> 3;
    lcol[u] = (c & 7) * 8;
    const int m = m0 + lrow[u];
    arow[u] = nullptr;
    if (m < g.M) {
      const int src = g.a_rows ? g.a_rows[m] : m;
      arow[u] = A + static_cast<int64_t>(src) * g.lda + lcol[u];
    }
    int brow_idx;
    bool bvalid;
    if (EPI == EPI_SWIGLU) {
      const int r = lrow[u];
      const int f = n0 + (r >> 6) * 32 + (r & 31);
      bvalid = f < g.N;
      brow_idx = ((r >> 5) & 1) ? g.ff + f : f;
    } else {
      brow_idx = n0 + lrow[u];
      bvalid = brow_idx < g.N;
    }
    brow[u] = bvalid ? B + static_cast<int64_t>(brow_idx) * g.ldb + lcol[u] : nullptr;
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = arow[u] ? *reinterpret_cast<const uint4*>(arow[u] + k0) : make_uint4(0, 0, 0, 0);
      rb[u] = brow[u] ? *reinterpret_cast<const uint4*>(brow[u] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<uint4*>(&As[buf][lrow[u] * LDSP + lcol[u]]) = ra[u];
      *reinterpret_cast<uint4*>(&Bs[buf][lrow[u] * LDSP + lcol[u]]) = rb[u];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = g.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int fr = lane & 31;          // fragment row (A) / column (B)
  const int fk = (lane >> 5) * 8;    // fragment k offset
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* as = As[buf];
    const bf16_t* bs = Bs[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&as[(wm * 64 + i * 32 + fr) * LDSP + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&bs[(wn * 64 + j * 32 + fr) * LDSP + ks * 16 + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  // acc[i][j][v] holds C[row][col] with
  //   row = m0 + wm*64 + i*32 + 8*(v/4) + 4*(lane/32) + v%4,  col = wn*64 + j*32 + lane%32
  const int half = g.head_dim >> 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const bool rok = row < g.M;
      if constexpr (EPI == EPI_SWIGLU) {
        const int f = n0 + wn * 32 + (lane & 31);
        if (rok && f < g.N) {
          const float h = silu(acc[i][0][v]) * acc[i][1][v];
          static_cast<bf16_t*>(g.C)[static_cast<int64_t>(row) * g.ldc + f] = f2bf(h);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + (lane & 31);
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

template <int EPI>
hipError_t run_gemm(cb_dtype dt, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (dt == CB_BF16) {
    const int m_tiles = (a.M + BM - 1) / BM;
    const int n_tiles = (EPI == EPI_SWIGLU) ? (a.N + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
    gemm_bf16_kernel<EPI><<<m_tiles * n_tiles, kThreads, 0, s>>>(a);
  } else {
    const int m_tiles = (a.M + FM - 1) / FM;
    const int n_tiles = (EPI == EPI_SWIGLU) ? (a.N + FN / 2 - 1) / (FN / 2) : (a.N + FN - 1) / FN;
    gemm_f32_kernel<EPI><<<m_tiles * n_tiles, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

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
