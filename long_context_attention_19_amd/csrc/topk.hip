// csa_topk_select: exact top-k of int32 indexer scores, ranked by (score desc,
// index asc), reported in ascending index order.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 item 2 (component table): CSA keeps a sparse top-k of
// the compressed entries.  The tie rule (lower index first) is this library's.
//
// Scores lie in [-2^20, 2^20), so key = score + 2^20 has 21 bits.  Two radix
// levels pin the k-th key T exactly: 2048 bins of key >> 10, then 1024 bins of
// key & 1023 within the threshold bin.  Every decision is a function of counts,
// never of arrival order, so the selection is deterministic.
//
// Kernels (grid = chunks of TK_CHUNK scores x rows):
//   hist   — LDS histogram of key >> 10, one global atomic per non-empty bin
//            (skipped when the index-score kernel already built it);
//   select — every work-group finds the threshold bin from the histogram, then
//            compacts its chunk's candidates (key bin >= threshold bin) in index
//            order into a per-chunk slot.  The last work-group of a row to
//            finish (an atomic ticket; nobody waits) resolves the row: it
//            prefix-sums the per-chunk counts, so the candidates read back in
//            index order, builds the second-level histogram, fixes T and the
//            number of T-valued entries to keep, and writes the selected indices
//            in ascending order.  It then clears the histogram and the ticket.
// Rows with n_vis <= k select every visible entry without any of this.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int TK_NT = 256;
constexpr int TK_PER_THREAD = 16;
constexpr int TK_CHUNK = TK_NT * TK_PER_THREAD;   // 4096 scores per work-group
constexpr int TK_MAX_CHUNKS = 1024;               // rows up to 4M entries
constexpr int TK_LDS_CAND = 4096;                 // candidates the resolver caches in LDS
constexpr int TK_CMP_PER_THREAD = 8;              // resolver compaction: entries per thread per block

int topk_max_chunks() { return TK_MAX_CHUNKS; }

static inline int topk_nchunks(int max_n) { return max(1, (max_n + TK_CHUNK - 1) / TK_CHUNK); }

size_t topk_ws_bytes(int rows, int max_n, int k) {
  (void)k;
  const size_t nc = (size_t)topk_nchunks(max_n);
  size_t b = align256((size_t)rows * HIST_BINS * 4);
  b += align256((size_t)rows * 4);
  b += align256((size_t)rows * nc * 4);
  b += align256((size_t)rows * nc * TK_CHUNK * 8);
  return b;
}

TopkWs topk_ws_carve(void* ws, int rows, int max_n, int k) {
  (void)k;
  TopkWs w;
  w.nchunks = topk_nchunks(max_n);
  char* p = reinterpret_cast<char*>(ws);
  w.hist = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * HIST_BINS * 4);
  w.done = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * 4);
  w.cnt = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * w.nchunks * 4);
  w.cand = reinterpret_cast<int2*>(p);
  return w;
}

// Load this thread's 16 consecutive scores of the chunk; entries >= n read as "absent".
__device__ __forceinline__ void load16(const int32_t* srow, int64_t j0, int64_t n, int32_t v[16]) {
  if (j0 + 16 <= n) {
    const i32x4* p = reinterpret_cast<const i32x4*>(srow + j0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const i32x4 x = p[q];
      v[4 * q] = x[0];
      v[4 * q + 1] = x[1];
      v[4 * q + 2] = x[2];
      v[4 * q + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = (j0 + e < n) ? srow[j0 + e] : INT32_MIN;
  }
}

__global__ __launch_bounds__(TK_NT) void topk_hist_kernel(const int32_t* __restrict__ scores,
                                                          int64_t ld, const int32_t* __restrict__ n_vis,
                                                          int max_n, int k, int32_t* __restrict__ hist) {
  __shared__ int32_t lh[HIST_BINS];
  const int row = blockIdx.y;
  const int64_t n = min(n_vis[row], max_n);
  if (n <= k) return;
  const int64_t base = (int64_t)blockIdx.x * TK_CHUNK;
  if (base >= n) return;
  const int t = threadIdx.x;
  for (int b = t; b < HIST_BINS; b += TK_NT) lh[b] = 0;
  __syncthreads();
  int32_t v[16];
  const int64_t j0 = base + (int64_t)t * TK_PER_THREAD;
  load16(scores + (int64_t)row * ld, j0, n, v);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (j0 + e < n) atomicAdd(&lh[(v[e] + KEY_BIAS) >> 10], 1);
  __syncthreads();
  int32_t* gh = hist + (int64_t)row * HIST_BINS;
  for (int b = t; b < HIST_BINS; b += TK_NT)
    if (lh[b]) atomicAdd(gh + b, lh[b]);
}

struct ResolveSmem {
  int32_t prefix[TK_MAX_CHUNKS + 1];
  int32_t fine[FINE_BINS];
  int2 cache[TK_LDS_CAND];
};

// Position p of the row's candidate sequence (index order) -> candidate.
__device__ __forceinline__ int2 cand_at(const int2* crow, const int32_t* prefix, int nch, int p) {
  int lo = 0, hi = nch;   // largest chunk c with prefix[c] <= p
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= p) lo = mid; else hi = mid;
  }
  return crow[(int64_t)lo * TK_CHUNK + (p - prefix[lo])];
}

__global__ __launch_bounds__(TK_NT) void topk_select_kernel(
    const int32_t* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_vis, int max_n,
    int k, int32_t* __restrict__ idx, int32_t* __restrict__ count, int32_t* hist, int32_t* done,
    int32_t* cnt, int2* cand, int nchunks_alloc) {
  __shared__ int32_t s_scan[TK_NT / WAVE + 1];
  __shared__ int32_t s_b[4];
  __shared__ ResolveSmem sm;

  const int row = blockIdx.y;
  const int ch = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = min(n_vis[row], max_n);   // n_vis beyond the bound is not processed
  int32_t* irow = idx + (int64_t)row * k;
  int32_t* hrow = hist + (int64_t)row * HIST_BINS;

  if (n <= k) {   // every visible entry is selected
    const int64_t p_end = min((int64_t)(ch + 1) * TK_CHUNK, (int64_t)k);
    for (int64_t p = (int64_t)ch * TK_CHUNK + t; p < p_end; p += TK_NT)
      irow[p] = p < n ? (int32_t)p : -1;
    if (ch == 0) {
      if (t == 0) count[row] = (int32_t)n;
      for (int b = t; b < HIST_BINS; b += TK_NT) hrow[b] = 0;   // a fused histogram may exist
    }
    return;
  }
  const int nch = (int)((n + TK_CHUNK - 1) / TK_CHUNK);
  if (ch >= nch) return;
  if (t < 4) s_b[t] = 0;   // defined even if a caller-supplied histogram is inconsistent
  __syncthreads();

  // ---- 1. threshold bin: thread t owns bins 2047-8t .. 2040-8t (descending)
  int32_t hv[8];
  {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(hrow + 2040 - 8 * t);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(hrow + 2044 - 8 * t);
    hv[0] = hi[3]; hv[1] = hi[2]; hv[2] = hi[1]; hv[3] = hi[0];
    hv[4] = lo[3]; hv[5] = lo[2]; hv[6] = lo[1]; hv[7] = lo[0];
  }
  int32_t hs = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) hs += hv[e];
  int32_t htot;
  const int32_t hpre = block_excl_scan<TK_NT>(hs, s_scan, &htot);
  if (hpre < k && hpre + hs >= k) {
    int32_t acc = hpre;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (acc + hv[e] >= k && acc < k) {
        s_b[0] = 2047 - 8 * t - e;
        s_b[1] = acc;
      }
      acc += hv[e];
    }
  }
  __syncthreads();
  const int bA = s_b[0];
  const int above = s_b[1];

  // ---- 2. this chunk's candidates, compacted in index order
  const int64_t j0 = (int64_t)ch * TK_CHUNK + (int64_t)t * TK_PER_THREAD;
  int32_t v[16];
  load16(scores + (int64_t)row * ld, j0, n, v);
  int32_t nc = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) nc += (j0 + e < n && ((v[e] + KEY_BIAS) >> 10) >= bA) ? 1 : 0;
  int32_t ctot;
  int32_t off = block_excl_scan<TK_NT>(nc, s_scan, &ctot);
  int2* crow = cand + (int64_t)row * nchunks_alloc * TK_CHUNK;
  int2* cslot = crow + (int64_t)ch * TK_CHUNK;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (j0 + e < n && ((v[e] + KEY_BIAS) >> 10) >= bA) cslot[off++] = make_int2((int)(j0 + e), v[e]);
  if (t == 0) cnt[(int64_t)row * nchunks_alloc + ch] = ctot;

  // ---- 3. ticket: the last work-group of this row resolves it
  __threadfence();
  __syncthreads();
  if (t == 0) s_b[2] = (atomicAdd(done + row, 1) == nch - 1) ? 1 : 0;
  __syncthreads();
  if (!s_b[2]) return;
  __threadfence();

  // prefix of per-chunk counts: thread t owns chunks 4t .. 4t+3
  {
    int32_t cv[4];
    int32_t cs = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * t + e;
      cv[e] = c < nch ? __hip_atomic_load(cnt + (int64_t)row * nchunks_alloc + c, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 0;
      cs += cv[e];
    }
    int32_t tot;
    int32_t pre = block_excl_scan<TK_NT>(cs, s_scan, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * t + e;
      if (c < nch) sm.prefix[c] = pre;
      pre += cv[e];
    }
    if (t == 0) sm.prefix[nch] = tot;
  }
  for (int b = t; b < FINE_BINS; b += TK_NT) sm.fine[b] = 0;
  __syncthreads();
  const int ctotal = sm.prefix[nch];
  const bool cached = ctotal <= TK_LDS_CAND;

  // second level: histogram of key & 1023 over candidates in the threshold bin
  for (int p = t; p < ctotal; p += TK_NT) {
    const int2 c = cand_at(crow, sm.prefix, nch, p);
    if (cached) sm.cache[p] = c;
    const int key = c.y + KEY_BIAS;
    if ((key >> 10) == bA) atomicAdd(&sm.fine[key & 1023], 1);
  }
  __syncthreads();
  const int need = k - above;   // >= 1 entries still to take from the threshold bin
  {
    int32_t fv[4];
    int32_t fs = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fv[e] = sm.fine[1023 - 4 * t - e];
      fs += fv[e];
    }
    int32_t ftot;
    const int32_t fpre = block_excl_scan<TK_NT>(fs, s_scan, &ftot);
    if (fpre < need && fpre + fs >= need) {
      int32_t acc = fpre;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (acc + fv[e] >= need && acc < need) {
          s_b[0] = 1023 - 4 * t - e;
          s_b[1] = acc;
        }
        acc += fv[e];
      }
    }
  }
  __syncthreads();
  const int T = (bA << 10) | s_b[0];          // the k-th largest key
  const int need_eq = need - s_b[1];          // entries with key == T to keep (lowest indices)

  // ---- 4. compaction in index order
  int32_t sel_before = 0, eq_before = 0;
  for (int blk = 0; blk < ctotal; blk += TK_NT * TK_CMP_PER_THREAD) {
    int2 c[TK_CMP_PER_THREAD];
    int32_t ne = 0;
#pragma unroll
    for (int e = 0; e < TK_CMP_PER_THREAD; ++e) {
      const int p = blk + t * TK_CMP_PER_THREAD + e;
      if (p < ctotal) c[e] = cached ? sm.cache[p] : cand_at(crow, sm.prefix, nch, p);
      else c[e] = make_int2(-1, INT32_MIN);
      ne += (p < ctotal && c[e].y + KEY_BIAS == T) ? 1 : 0;
    }
    int32_t etot;
    int32_t rank = eq_before + block_excl_scan<TK_NT>(ne, s_scan, &etot);
    int32_t ns = 0;
    uint32_t selmask = 0;
#pragma unroll
    for (int e = 0; e < TK_CMP_PER_THREAD; ++e) {
      const int p = blk + t * TK_CMP_PER_THREAD + e;
      const int key = c[e].y + KEY_BIAS;
      bool sel = false;
      if (p < ctotal) {
        if (key > T) sel = true;
        else if (key == T) sel = (rank++ < need_eq);
      }
      if (sel) { selmask |= 1u << e; ++ns; }
    }
    int32_t stot;
    int32_t pos = sel_before + block_excl_scan<TK_NT>(ns, s_scan, &stot);
#pragma unroll
    for (int e = 0; e < TK_CMP_PER_THREAD; ++e)
      if (selmask & (1u << e)) {
        if (pos < k) irow[pos] = c[e].x;   // exactly k are selected; the bound guards bad input
        ++pos;
      }
    sel_before += stot;
    eq_before += etot;
  }
  if (t == 0) {
    count[row] = k;
    done[row] = 0;
  }
  for (int b = t; b < HIST_BINS; b += TK_NT) hrow[b] = 0;
}

hipError_t launch_topk(const int32_t* scores, int64_t ld, int rows, int max_n, const int32_t* n_vis,
                       int k, int32_t* idx, int32_t* count, const TopkWs& w, bool hist_ready,
                       hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (!hist_ready) {
    dim3 g((unsigned)topk_nchunks(max_n), (unsigned)rows);
    hipLaunchKernelGGL(topk_hist_kernel, g, dim3(TK_NT), 0, st, scores, ld, n_vis, max_n, k,
                       w.hist);
  }
  const int span = max(max_n, k);
  dim3 g((unsigned)max(1, (span + TK_CHUNK - 1) / TK_CHUNK), (unsigned)rows);
  hipLaunchKernelGGL(topk_select_kernel, g, dim3(TK_NT), 0, st, scores, ld, n_vis, max_n, k, idx,
                     count,
                     w.hist, w.done, w.cnt, w.cand, w.nchunks);
  return hipGetLastError();
}

}  // namespace lca
