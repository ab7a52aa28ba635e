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
// Two kernels.  The scan kernel gives each thread a run of kRun consecutive
// window starts of one request: it hashes the first window with Horner's rule
// from the request's tokens staged in LDS, rolls the hash to the next starts
// (drop the oldest token's term, shift, add the new token), gathers the
// filter byte of every probed window, probes the fingerprint table for the
// few survivors and compares a resolved window with the entry's tokens.  It
// writes, per token position, the verified entry or -1.  The assignment kernel
// (one workgroup per request) walks the positions in order, compacts the
// verified ones, and lets one thread give each its entry's first occupant not
// yet matched by this request (counts per entry in an LDS map) and apply the
// leftmost-greedy rule; the outputs are then written in parallel.
#include "cb_internal.h"

namespace cb {

namespace {

constexpr int kRun = 16;                   // window starts per thread
constexpr int kScanThreads = 256;
constexpr int kSpan = kScanThreads * kRun; // window starts per workgroup
constexpr int kMapSlots = 2 * kMatchMaxContents;

__device__ __forceinline__ int lds_idx(int i) { return i + (i >> 4); }   // odd stride between runs

__device__ __forceinline__ void request_range(const int32_t* starts, int q, int64_t total, int max_len, int64_t* st,
                                              int* len) {
  const int64_t a = min(max(static_cast<int64_t>(starts[q]), int64_t(0)), total);
  const int64_t b = min(max(static_cast<int64_t>(starts[q + 1]), a), total);
  *st = a;
  *len = static_cast<int>(min(b - a, static_cast<int64_t>(max_len)));
}

__global__ __launch_bounds__(kScanThreads) void match_scan_kernel(MatchIndexRef ix, const int32_t* __restrict__ tokens,
                                                                   const int32_t* __restrict__ starts, int64_t total,
                                                                   int max_len, int stride, int32_t* __restrict__ cand) {
  extern __shared__ int32_t tk[];
  const int q = blockIdx.y;
  int64_t st;
  int len;
  request_range(starts, q, total, max_len, &st, &len);
  const int C = ix.chunk_size;
  const int p_blk = blockIdx.x * kSpan;
  if (p_blk >= len) return;                                    // uniform per workgroup
  const int span = min(kSpan + C - 1, len - p_blk);
  for (int i = threadIdx.x; i < span; i += kScanThreads) tk[lds_idx(i)] = tokens[st + p_blk + i];
  __syncthreads();

  const int p0 = threadIdx.x * kRun;                           // this thread's first start, in the workgroup
  int32_t res[kRun];
#pragma unroll
  for (int j = 0; j < kRun; ++j) res[j] = -1;
  if (p_blk + p0 + C <= len) {
    // hashes of the run's windows (a window exists while start + C <= len)
    uint64_t h[kRun];
    uint64_t x = 0;
    for (int i = 0; i < C; ++i) x = x * kPolyBase + static_cast<uint32_t>(tk[lds_idx(p0 + i)]);
    h[0] = x;
#pragma unroll
    for (int j = 1; j < kRun; ++j) {
      if (p_blk + p0 + j + C <= len) {
        x = (x - static_cast<uint32_t>(tk[lds_idx(p0 + j - 1)]) * ix.top_pow) * kPolyBase +
            static_cast<uint32_t>(tk[lds_idx(p0 + j + C - 1)]);
      }
      h[j] = x;
    }
    // the filter bytes of every probed window, all loads in flight together
    uint8_t f[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const int s = p_blk + p0 + j;
      f[j] = (s + C <= len && s % stride == 0) ? ix.slots[h[j] >> (64 - ix.slot_bits)] : 0;
    }
    const uint32_t tmask = (1u << ix.table_bits) - 1u;
#pragma unroll 1
    for (int j = 0; j < kRun; ++j) {
      if (!f[j]) continue;
      // exact resolution: linear probing from the fingerprint's top bits; the table
      // is at most half full, and the walk is bounded by its size in any case
      uint32_t slot = static_cast<uint32_t>(h[j] >> (64 - ix.table_bits));
      int e = -1;
      for (uint32_t n = 0; n <= tmask; ++n) {
        const int t = ix.table_entry[slot];
        if (t < 0) break;
        if (ix.table_fp[slot] == h[j]) { e = t; break; }
        slot = (slot + 1) & tmask;
      }
      if (e < 0) continue;
      // token-by-token verification against the entry's content
      const int32_t* et = ix.entry_tokens + static_cast<int64_t>(e) * C;
      bool same = true;
      for (int i = 0; i < C && same; ++i) same = tk[lds_idx(p0 + j + i)] == et[i];
      if (same) res[j] = e;
    }
  }
#pragma unroll
  for (int j = 0; j < kRun; ++j)
    if (p_blk + p0 + j < len) cand[st + p_blk + p0 + j] = res[j];
}

__global__ __launch_bounds__(256) void match_assign_kernel(MatchIndexRef ix, const int32_t* __restrict__ starts,
                                                            int64_t total, int max_len,
                                                            const int32_t* __restrict__ prefix,
                                                            const int32_t* __restrict__ cand, int max_matches,
                                                            MatchOut out) {
  __shared__ int32_t map_key[kMapSlots];
  __shared__ int32_t map_cnt[kMapSlots];
  __shared__ int32_t l_pos[256], l_ent[256], l_occ0[256], l_nocc[256];
  __shared__ int32_t a_idx[256], a_pos[256];          // accepted this round: occupant index, start
  __shared__ uint8_t a_kept[256];
  __shared__ int wcnt[4];
  __shared__ int n_acc, s_count, s_end, s_used, s_over;
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
  __syncthreads();
  const int C = ix.chunk_size;
  for (int base = 0; base < len; base += 256) {
    const int pos = base + tid;
    const int e = pos < len ? cand[st + pos] : -1;
    // ordered compaction of the verified positions of this round
    const uint64_t m = __ballot(e >= 0);
    if (lane == 0) wcnt[wid] = __popcll(m);
    __syncthreads();
    int before = 0, n = 0;
    for (int w = 0; w < 4; ++w) {
      before += w < wid ? wcnt[w] : 0;
      n += wcnt[w];
    }
    if (e >= 0) {
      const int at = before + __popcll(m & ((uint64_t(1) << lane) - 1));
      l_pos[at] = pos;
      l_ent[at] = e;
      l_occ0[at] = ix.entry_occ[e];
      l_nocc[at] = ix.entry_occ[e + 1] - l_occ0[at];
    }
    __syncthreads();
    if (n == 0) continue;                                    // uniform
    if (tid == 0) {
      int acc = 0;
      for (int i = 0; i < n; ++i) {
        if (s_over) break;
        const int ent = l_ent[i];
        uint32_t slot = (static_cast<uint32_t>(ent) * 2654435761u) & (kMapSlots - 1);
        while (map_key[slot] != -1 && map_key[slot] != ent) slot = (slot + 1) & (kMapSlots - 1);
        if (map_key[slot] == -1) {
          if (s_used == kMatchMaxContents) { s_over = 1; break; }
          map_key[slot] = ent;
          map_cnt[slot] = 0;
          ++s_used;
        }
        const int u = map_cnt[slot];
        if (u >= l_nocc[i]) continue;                        // every occupant already matched here
        map_cnt[slot] = u + 1;
        const int s = l_pos[i];
        const bool keep = s >= s_end;
        if (keep) s_end = s + C;
        if (s_count + acc < max_matches) {
          a_idx[acc] = l_occ0[i] + u;
          a_pos[acc] = s;
          a_kept[acc] = keep ? 1 : 0;
        }
        ++acc;
      }
      n_acc = acc;
    }
    __syncthreads();
    const int na = n_acc, c0 = s_count;
    if (tid < na && c0 + tid < max_matches) {
      const int64_t o = static_cast<int64_t>(q) * max_matches + c0 + tid;
      out.chunk[o] = ix.occ_chunk[a_idx[tid]];
      out.old_st[o] = ix.occ_offset[a_idx[tid]];
      out.cur_st[o] = a_pos[tid];
      out.kept[o] = a_kept[tid];
    }
    __syncthreads();
    if (tid == 0) s_count = c0 + na;
    __syncthreads();
    if (s_over) break;                                       // uniform after the barrier
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
    const int n = kSpan + ix.chunk_size - 1;
    const size_t lds = static_cast<size_t>(n + n / 16 + 1) * 4;
    match_scan_kernel<<<dim3((max_len + kSpan - 1) / kSpan, n_queries), kScanThreads, lds, s>>>(
        ix, tokens, starts, total, max_len, stride, cand);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  match_assign_kernel<<<n_queries, 256, 0, s>>>(ix, starts, total, max_len, prefix, cand, max_matches, out);
  return hipGetLastError();
}

}  // namespace cb
