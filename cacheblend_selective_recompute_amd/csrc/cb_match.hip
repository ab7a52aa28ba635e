// Fragment matching on the GPU: which indexed chunks a batch of requests
// contains, and where.
//
// Method: the LMCache coordinator "Blend Index" article (nxmr.cn): section 3.1
// (a chunk's key is the 64-bit polynomial hash of its tokens, base
// 0x9E3779B97F4A7C15), 4.1 (occupancy filter + exact contents map), 4.2 (roll a
// chunk_size window over the request, test the filter every probe_stride
// positions, resolve survivors exactly, choose the occupant, then compare token
// by token; a chunk is seen only after that check), 6.2 and 7 (tuples in
// ascending cur_st, one per chunk; leftmost-greedy after dropping matches inside
// the prefix).
//
// Two kernels.  The scan kernel takes 1024 window starts of one request per
// workgroup: it stages the tokens they cover in LDS, forms the prefix hashes
// with a block-wide scan so every window's hash is two prefix reads and a
// multiply, gathers the filter byte of every probed window, probes the
// fingerprint table for the few survivors and compares a resolved window with
// the entry's tokens.  It writes, per token position, the verified entry or -1.  The assignment kernel
// (one workgroup per request) compacts the verified positions in order and
// lets one thread give each its entry's first occupant not yet matched by this
// request and apply the leftmost-greedy rule.
#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kRun = 4;                    // window starts per thread: t, t + 256, t + 512, t + 768
constexpr int kScanThreads = 256;
constexpr int kSpan = kScanThreads * kRun; // window starts per workgroup
constexpr int kMapSlots = 2 * kMatchMaxContents;
constexpr int kProbe = 4;                  // table slots read at once per survivor

__device__ __forceinline__ void request_range(const int32_t* starts, int q, int64_t total, int max_len, int64_t* st,
                                              int* len) {
  const int64_t a = min(max(static_cast<int64_t>(starts[q]), int64_t(0)), total);
  const int64_t b = min(max(static_cast<int64_t>(starts[q + 1]), a), total);
  *st = a;
  *len = static_cast<int>(min(b - a, static_cast<int64_t>(max_len)));
}

__device__ __forceinline__ uint64_t pow_u64(uint64_t b, int e) {
  uint64_t r = 1;
  for (; e > 0; e >>= 1, b *= b)
    if (e & 1) r *= b;
  return r;
}

// Scan: the hash of window [s, s + C) is P(s + C) - P(s) * base^C with the prefix
// hashes P(0) = 0, P(i + 1) = P(i) * base + token i of the workgroup's tokens.
// Each thread Horner-hashes G consecutive tokens (the tail padded with zeros,
// which changes no prefix that is used), a block-wide scan joins the pieces
// (x_i <- x_{i-d} * base^(G d) + x_i), and each thread then writes its G
// prefixes.  Its windows are t, t + 256, ..., so neighbouring lanes read
// neighbouring prefixes.
__global__ __launch_bounds__(kScanThreads) void match_scan_kernel(MatchIndexRef ix, const int32_t* __restrict__ tokens,
                                                                   const int32_t* __restrict__ starts, int64_t total,
                                                                   int max_len, int stride, int G,
                                                                   int32_t* __restrict__ cand) {
  extern __shared__ uint64_t P[];                              // [256 G + 1] prefixes, then 256 G tokens
  int32_t* tk = reinterpret_cast<int32_t*>(P + kScanThreads * G + 1);
  __shared__ uint64_t xs[kScanThreads];
  const int tid = threadIdx.x;
  const int q = blockIdx.y;
  int64_t st;
  int len;
  request_range(starts, q, total, max_len, &st, &len);
  const int C = ix.chunk_size;
  const int p_blk = blockIdx.x * kSpan;
  if (p_blk >= len) return;                                    // uniform per workgroup
  const int n_tok = min(kSpan + C - 1, len - p_blk);
  for (int i = tid; i < kScanThreads * G; i += kScanThreads) tk[i] = i < n_tok ? tokens[st + p_blk + i] : 0;
  __syncthreads();
  // this thread's piece: tokens [tid G, tid G + G)
  uint64_t x = 0;
  for (int j = 0; j < G; ++j) x = x * kPolyBase + static_cast<uint32_t>(tk[tid * G + j]);
  uint64_t m = pow_u64(kPolyBase, G);                          // base^(G d) for d = 1, 2, 4, ...
  for (int d = 1; d < kScanThreads; d <<= 1) {
    xs[tid] = x;
    __syncthreads();
    if (tid >= d) x = xs[tid - d] * m + x;
    __syncthreads();
    m *= m;
  }
  xs[tid] = x;
  __syncthreads();
  uint64_t h = tid > 0 ? xs[tid - 1] : 0;                      // prefix of the pieces before this one
  for (int j = 0; j < G; ++j) {
    P[tid * G + j] = h;
    h = h * kPolyBase + static_cast<uint32_t>(tk[tid * G + j]);
  }
  if (tid == kScanThreads - 1) P[kScanThreads * G] = h;
  __syncthreads();

  uint64_t hw[kRun];
  uint8_t f[kRun];
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    const int s = tid + r * kScanThreads;                      // window start in the workgroup
    hw[r] = P[s + C] - P[s] * ix.pow_c;
    const int sq = p_blk + s;                                  // ... in the request
    f[r] = (sq + C <= len && sq % stride == 0) ? ix.slots[hw[r] >> (64 - ix.slot_bits)] : 0;
  }
  // exact resolution: the first kProbe table slots of every survivor at once; the
  // table is at most a quarter full, so a longer walk (done after) is rare
  const uint32_t tmask = (1u << ix.table_bits) - 1u;
  int e_r[kRun];
  int te[kRun][kProbe];
  uint64_t tf[kRun][kProbe];
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    e_r[r] = -1;
    if (f[r]) {
      const uint32_t slot0 = static_cast<uint32_t>(hw[r] >> (64 - ix.table_bits));
#pragma unroll
      for (int k = 0; k < kProbe; ++k) {
        te[r][k] = ix.table_entry[(slot0 + k) & tmask];
        tf[r][k] = ix.table_fp[(slot0 + k) & tmask];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    if (!f[r]) continue;
    bool done = false;
#pragma unroll
    for (int k = 0; k < kProbe; ++k) {
      if (done) continue;
      if (te[r][k] < 0) done = true;
      else if (tf[r][k] == hw[r]) { e_r[r] = te[r][k]; done = true; }
    }
    if (!done) {
      // walk on past kProbe occupied slots, bounded by the table size
      uint32_t slot = (static_cast<uint32_t>(hw[r] >> (64 - ix.table_bits)) + kProbe) & tmask;
      for (uint32_t n = 0; n < tmask; ++n) {
        const int t = ix.table_entry[slot];
        if (t < 0) break;
        if (ix.table_fp[slot] == hw[r]) { e_r[r] = t; break; }
        slot = (slot + 1) & tmask;
      }
    }
  }
  // token-by-token verification, the wave's lanes together on one window at a time:
  // lane k compares tokens 4k .. 4k + 3 (+ 256 j) with 16-byte loads of the entry
  const int lane = tid & 63;
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    uint64_t pend = __ballot(e_r[r] >= 0);
    while (pend) {
      const int src = __builtin_ctzll(pend);
      pend &= pend - 1;
      const int e = __builtin_amdgcn_readlane(e_r[r], src);
      const int s = src + (tid & ~63) + r * kScanThreads;       // the source lane's window start
      const int32_t* et = ix.entry_tokens + static_cast<int64_t>(e) * C;
      bool ok = true;
      if ((C & 3) == 0) {
        for (int i = 4 * lane; i < C; i += 256) {
          const int4 v = *reinterpret_cast<const int4*>(et + i);
          ok = ok && v.x == tk[s + i] && v.y == tk[s + i + 1] && v.z == tk[s + i + 2] && v.w == tk[s + i + 3];
        }
      } else {
        for (int i = lane; i < C; i += 64) ok = ok && et[i] == tk[s + i];
      }
      const bool all_ok = __ballot(!ok) == 0;
      if (lane == src && !all_ok) e_r[r] = -1;
    }
  }
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    const int s = p_blk + tid + r * kScanThreads;
    if (s < len) cand[st + s] = e_r[r];
  }
}

// Assignment, one workgroup per request.  The positions are taken in slices of
// 256 x kPer: thread t loads kPer consecutive entries of the slice (the next
// slice's loads go out before this one is processed), a block-wide scan of the
// per-thread counts places the verified positions in order in an LDS list, and
// one thread walks the list: per entry it keeps how many of its occupants this
// request has taken (an LDS map), takes the next one if any, and applies the
// leftmost-greedy rule.  The outputs are then written in parallel.
constexpr int kPer = 16;
constexpr int kList = 1024;

__global__ __launch_bounds__(256) void match_assign_kernel(MatchIndexRef ix, const int32_t* __restrict__ starts,
                                                            int64_t total, int max_len,
                                                            const int32_t* __restrict__ prefix,
                                                            const int32_t* __restrict__ cand, int max_matches,
                                                            MatchOut out) {
  __shared__ int32_t map_key[kMapSlots];
  __shared__ int32_t map_cnt[kMapSlots];
  __shared__ int32_t l_pos[kList], l_ent[kList], l_occ0[kList], l_nocc[kList], l_take[kList], l_rank[kList];
  __shared__ uint8_t l_keep[kList];
  __shared__ int wsum[4];
  __shared__ int s_count, s_end, s_used, s_over;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int q = blockIdx.x;
  int64_t st;
  int len;
  request_range(starts, q, total, max_len, &st, &len);
  for (int i = tid; i < kMapSlots; i += 256) map_key[i] = -1;
  if (tid == 0) {
    s_count = 0;
    s_end = prefix ? prefix[q] : 0;
    s_used = 0;
    s_over = 0;
  }
  const int C = ix.chunk_size;
  constexpr int kSlice = 256 * kPer;
  int nxt[kPer];
  auto load = [&](int base, int (&v)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int pos = base + tid * kPer + j;
      v[j] = pos < len ? cand[st + pos] : -1;
    }
  };
  load(0, nxt);
  __syncthreads();
  for (int base = 0; base < len; base += kSlice) {
    int cur[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) cur[j] = nxt[j];
    if (base + kSlice < len) load(base + kSlice, nxt);
    int c = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) c += cur[j] >= 0;
    // exclusive scan of the counts over the workgroup
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int before = incl - c, n_items = 0;
    for (int w = 0; w < 4; ++w) {
      before += w < wid ? wsum[w] : 0;
      n_items += wsum[w];
    }
    __syncthreads();                                           // wsum is rewritten next slice
    if (n_items == 0) continue;                                // uniform
    for (int b0 = 0; b0 < n_items; b0 += kList) {
      // list items [b0, b0 + kList) of this slice, in position order
      int at = before;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (cur[j] < 0) continue;
        const int i = at++ - b0;
        if (i >= 0 && i < kList) {
          l_pos[i] = base + tid * kPer + j;
          l_ent[i] = cur[j];
          l_occ0[i] = ix.entry_occ[cur[j]];
          l_nocc[i] = ix.entry_occ[cur[j] + 1] - l_occ0[i];
        }
      }
      __syncthreads();
      const int nb = min(kList, n_items - b0);
      if (tid == 0) {
        int cnt = s_count, end = s_end, used = s_used, over = s_over;
        for (int i = 0; i < nb; ++i) {
          l_take[i] = -1;
          if (over) continue;
          const int ent = l_ent[i];
          uint32_t slot = (static_cast<uint32_t>(ent) * 2654435761u) & (kMapSlots - 1);
          while (map_key[slot] != -1 && map_key[slot] != ent) slot = (slot + 1) & (kMapSlots - 1);
          if (map_key[slot] == -1) {
            if (used == kMatchMaxContents) { over = 1; continue; }
            map_key[slot] = ent;
            map_cnt[slot] = 0;
            ++used;
          }
          const int u = map_cnt[slot];
          if (u >= l_nocc[i]) continue;                          // every occupant already matched here
          map_cnt[slot] = u + 1;
          const int sp = l_pos[i];
          const bool keep = sp >= end;
          if (keep) end = sp + C;
          l_take[i] = l_occ0[i] + u;
          l_rank[i] = cnt++;
          l_keep[i] = keep ? 1 : 0;
        }
        s_count = cnt;
        s_end = end;
        s_used = used;
        s_over = over;
      }
      __syncthreads();
      for (int i = tid; i < nb; i += 256) {
        if (l_take[i] < 0 || l_rank[i] >= max_matches) continue;
        const int64_t o = static_cast<int64_t>(q) * max_matches + l_rank[i];
        out.chunk[o] = ix.occ_chunk[l_take[i]];
        out.old_st[o] = ix.occ_offset[l_take[i]];
        out.cur_st[o] = l_pos[i];
        out.kept[o] = l_keep[i];
      }
      __syncthreads();                                         // the list is rewritten next
    }
    if (s_over) break;                                         // uniform after the barrier
  }
  if (tid == 0) out.count[q] = s_over ? -1 : s_count;
}

}  // namespace

hipError_t launch_blend_match(const MatchIndexRef& ix, const int32_t* tokens, const int32_t* starts, int n_queries,
                              int64_t total, int max_len, int stride, const int32_t* prefix, int max_matches,
                              const MatchOut& out, int32_t* cand, hipStream_t s) {
  if (n_queries <= 0) return hipSuccess;
  if (ix.chunk_size < 1 || ix.chunk_size > kMatchMaxChunk || n_queries > 65535) return hipErrorInvalidValue;
  if (max_len > 0) {
    const int G = (kSpan + ix.chunk_size - 1 + kScanThreads - 1) / kScanThreads;   // tokens per thread
    const size_t lds = static_cast<size_t>(kScanThreads * G + 1) * 8 + static_cast<size_t>(kScanThreads * G) * 4;
    match_scan_kernel<<<dim3((max_len + kSpan - 1) / kSpan, n_queries), kScanThreads, lds, s>>>(
        ix, tokens, starts, total, max_len, stride, G, cand);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  match_assign_kernel<<<n_queries, 256, 0, s>>>(ix, starts, total, max_len, prefix, cand, max_matches, out);
  return hipGetLastError();
}

}  // namespace cb
