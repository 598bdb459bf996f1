// csa_topk_select: exact top-k of int32 indexer scores, ranked by (score desc,
// index asc), reported in ascending index order.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 item 2 (component table): CSA keeps a sparse top-k of
// the compressed entries.  The tie rule (lower index first) is this library's.
//
// Scores lie in [-2^20, 2^20], so key = score + 2^20 (2^20 clamped one lower, a rank
// no other reachable score takes) has 21 bits.  Two radix
// levels pin the k-th largest key T exactly: 2048 bins of key >> 10 (the coarse
// histogram), then 1024 bins of key & 1023 among the keys of the threshold bin
// (the fine histogram).  Every decision is a function of counts, never of the
// order in which work-groups run, so the selection is deterministic.
//
// Each row is cut into chunks of TK_CHUNK scores; every kernel's grid is
// (chunks x rows x layers) and work-groups never wait for one another — kernel
// boundaries order the passes, so no work-group runs a device-scope fence:
//   K1 hist  — coarse histogram (LDS, one global atomic per non-empty bin) and
//              zeroing of the row's fine histogram.  The index-score kernel can
//              do this pass while it computes the scores.
//   K2 cand  — threshold bin bA from the coarse histogram; per chunk, the keys
//              above bA (their local indices) and the keys inside bA (few: ~k/8
//              per row for Gaussian-like scores, with their low 10 bits, which
//              also go to the fine histogram), each compacted in index order.
//   K3 merge — (k <= 4096, 32 rows or more) one work-group per row: T and the quota of T-valued
//              keys from the fine histogram, then the row's candidate lists merged
//              in index order; no score is read again.  The coarse histogram is
//              cleared here.
//   K3 place — (otherwise) T and the number of T-valued keys to keep follow from the fine
//              histogram; a chunk's output offset is the number of selected keys
//              in earlier chunks: their above-bA counts plus the earlier chunks'
//              threshold-bin keys that beat T or are T-valued within the quota.
//              The chunk's own scores are then re-read and its selections written
//              in index order.  The chunk-0 group clears the coarse histogram,
//              which leaves the workspace zeroed for the next call.
// Rows with n_vis <= k select every visible entry: K2 skips them, K3 writes
// 0 .. n_vis-1 and -1 padding.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int TK_NT = 256;
constexpr int TK_PER_THREAD = 16;
constexpr int TK_CHUNK = TK_NT * TK_PER_THREAD;   // 4096 scores per work-group
constexpr int TK_MAX_CHUNKS = 1024;               // rows up to 4M entries
constexpr int TK_BATCH = 8;                       // threshold-bin keys in flight per thread

int topk_max_chunks() { return TK_MAX_CHUNKS; }

static inline int topk_nchunks(int max_n) { return max(1, (max_n + TK_CHUNK - 1) / TK_CHUNK); }

size_t topk_ws_bytes(int rows, int max_n, int k) {
  (void)k;
  const size_t nc = (size_t)topk_nchunks(max_n);
  size_t b = align256((size_t)rows * HIST_BINS * 4);        // coarse histogram
  b += align256((size_t)rows * FINE_BINS * 4);               // fine histogram
  b += align256((size_t)rows * 8);                           // (bA, above) per row
  b += 2 * align256((size_t)rows * nc * 4);                  // per-chunk counts
  b += align256((size_t)rows * nc * TK_CHUNK * 4);           // threshold-bin keys
  return b;
}

TopkWs topk_ws_carve(void* ws, int rows, int max_n, int k) {
  (void)k;
  TopkWs w;
  w.nchunks = topk_nchunks(max_n);
  char* p = reinterpret_cast<char*>(ws);
  w.hist = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * HIST_BINS * 4);
  w.fine = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * FINE_BINS * 4);
  w.rowstate = reinterpret_cast<int2*>(p);
  p += align256((size_t)rows * 8);
  w.cnt_above = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * w.nchunks * 4);
  w.cnt_bin = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * w.nchunks * 4);
  w.bin_keys = reinterpret_cast<int32_t*>(p);
  return w;
}

size_t topk_hist_region_bytes(int rows) {
  return align256((size_t)rows * HIST_BINS * 4) + align256((size_t)rows * FINE_BINS * 4);
}

// This thread's 16 consecutive scores of the chunk; entries >= n read as INT32_MIN.
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

// Threshold bin of the coarse histogram: the bin holding the k-th largest key, and
// the number of keys in higher bins.  Thread t owns bins 2047-8t .. 2040-8t.
__device__ __forceinline__ void coarse_threshold(const int32_t* hrow, int k, int32_t* s_scan,
                                                 int32_t* s_b, int& bA, int& above) {
  const int t = threadIdx.x;
  int32_t hv[8];
  const i32x4 lo = *reinterpret_cast<const i32x4*>(hrow + 2040 - 8 * t);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(hrow + 2044 - 8 * t);
  hv[0] = hi[3]; hv[1] = hi[2]; hv[2] = hi[1]; hv[3] = hi[0];
  hv[4] = lo[3]; hv[5] = lo[2]; hv[6] = lo[1]; hv[7] = lo[0];
  int32_t hs = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) hs += hv[e];
  if (t < 2) s_b[t] = 0;   // defined even for an inconsistent histogram
  int32_t htot;
  const int32_t hpre = block_excl_scan<TK_NT>(hs, s_scan, &htot);
  if (hpre < k && hpre + hs >= k) {
    int32_t acc = hpre;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (acc < k && acc + hv[e] >= k) {
        s_b[0] = 2047 - 8 * t - e;
        s_b[1] = acc;
      }
      acc += hv[e];
    }
  }
  __syncthreads();
  bA = s_b[0];
  above = s_b[1];
  __syncthreads();
}

// ------------------------------------------------------------------ K1
__global__ __launch_bounds__(TK_NT) void topk_hist_kernel(TopkBatch tb) {
  const TopkLayer& TL = tb.layer[blockIdx.z];
  const int32_t* __restrict__ scores = TL.scores;
  const int64_t ld = TL.ld;
  const int k = TL.k;
  int32_t* __restrict__ hist = TL.w.hist;
  int32_t* __restrict__ fine = TL.w.fine;
  __shared__ int32_t lh[HIST_BINS];
  const int row = blockIdx.y;
  const int64_t n = min(TL.n_vis[row], TL.max_n);
  if (n <= k) return;
  const int64_t base = (int64_t)blockIdx.x * TK_CHUNK;
  if (base >= n) return;
  const int t = threadIdx.x;
  if (blockIdx.x == 0)
    for (int b = t; b < FINE_BINS; b += TK_NT) fine[(int64_t)row * FINE_BINS + b] = 0;
  for (int b = t; b < HIST_BINS; b += TK_NT) lh[b] = 0;
  __syncthreads();
  int32_t v[16];
  const int64_t j0 = base + (int64_t)t * TK_PER_THREAD;
  load16(scores + (int64_t)row * ld, j0, n, v);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (j0 + e < n) atomicAdd(&lh[score_key(v[e]) >> 10], 1);
  __syncthreads();
  int32_t* gh = hist + (int64_t)row * HIST_BINS;
  for (int b = t; b < HIST_BINS; b += TK_NT)
    if (lh[b]) atomicAdd(gh + b, lh[b]);
}

// ------------------------------------------------------------------ K2
__global__ __launch_bounds__(TK_NT) void topk_cand_kernel(TopkBatch tb) {
  const TopkLayer& TL = tb.layer[blockIdx.z];
  const int32_t* __restrict__ scores = TL.scores;
  const int64_t ld = TL.ld;
  const int k = TL.k;
  const int max_n = TL.max_n;
  const int32_t* __restrict__ n_vis = TL.n_vis;
  const TopkWs& w = TL.w;
  __shared__ int32_t s_scan[TK_NT / WAVE + 1];
  __shared__ int32_t s_b[2];
  const int row = blockIdx.y;
  const int ch = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = min(n_vis[row], max_n);
  if (n <= k) return;
  const int nch = (int)((n + TK_CHUNK - 1) / TK_CHUNK);
  if (ch >= nch) return;

  const int64_t j0 = (int64_t)ch * TK_CHUNK + (int64_t)t * TK_PER_THREAD;
  int32_t v[16];
  load16(scores + (int64_t)row * ld, j0, n, v);   // in flight during the histogram scan
  int bA, above;
  coarse_threshold(w.hist + (int64_t)row * HIST_BINS, k, s_scan, s_b, bA, above);

  int32_t na = 0, nb = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (j0 + e < n) {
      const int bin = score_key(v[e]) >> 10;
      na += bin > bA ? 1 : 0;
      nb += bin == bA ? 1 : 0;
    }
  }
  int32_t atot, btot;
  int32_t aoff = block_excl_scan<TK_NT>(na, s_scan, &atot);
  int32_t off = block_excl_scan<TK_NT>(nb, s_scan, &btot);
  const int64_t slot = (int64_t)row * w.nchunks + ch;
  // the chunk's region: local indices of its above-bA keys, then its bA keys
  int32_t* keys = w.bin_keys + slot * TK_CHUNK;
  int32_t* frow = w.fine + (int64_t)row * FINE_BINS;
  off += atot;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (j0 + e < n) {
      const int key = score_key(v[e]);
      const int li = t * TK_PER_THREAD + e;
      if ((key >> 10) > bA) {
        keys[aoff++] = li;
      } else if ((key >> 10) == bA) {
        keys[off++] = (li << 10) | (key & 1023);
        atomicAdd(frow + (key & 1023), 1);
      }
    }
  }
  if (t == 0) {
    w.cnt_above[slot] = atot;
    w.cnt_bin[slot] = btot;
    if (ch == 0) w.rowstate[row] = make_int2(bA, above);
  }
}

// ------------------------------------------------------------------ K3
__global__ __launch_bounds__(TK_NT) void topk_place_kernel(TopkBatch tb) {
  const TopkLayer& TL = tb.layer[blockIdx.z];
  const int32_t* __restrict__ scores = TL.scores;
  const int64_t ld = TL.ld;
  const int k = TL.k;
  const int max_n = TL.max_n;
  const int32_t* __restrict__ n_vis = TL.n_vis;
  int32_t* __restrict__ idx = TL.idx;
  int32_t* __restrict__ count = TL.count;
  const TopkWs& w = TL.w;
  __shared__ int32_t s_scan[TK_NT / WAVE + 1];
  __shared__ int32_t s_b[2];
  __shared__ int32_t s_pre[TK_MAX_CHUNKS + 1];   // prefix of earlier chunks' bin counts
  __shared__ int32_t s_ca[TK_MAX_CHUNKS];        // earlier chunks' above-bA counts

  const int row = blockIdx.y;
  const int ch = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t n = min(n_vis[row], max_n);
  int32_t* irow = idx + (int64_t)row * k;

  if (ch == 0) {   // nobody reads the coarse histogram in this kernel: clear it for the next call
    int32_t* hrow = w.hist + (int64_t)row * HIST_BINS;
    for (int b = t; b < HIST_BINS; b += TK_NT) hrow[b] = 0;
    if (t == 0) count[row] = (int32_t)min(n, (int64_t)k);
  }
  if (n <= k) {   // every visible entry is selected
    const int64_t p_end = min((int64_t)(ch + 1) * TK_CHUNK, (int64_t)k);
    for (int64_t p = (int64_t)ch * TK_CHUNK + t; p < p_end; p += TK_NT)
      irow[p] = p < n ? (int32_t)p : -1;
    return;
  }
  const int nch = (int)((n + TK_CHUNK - 1) / TK_CHUNK);
  if (ch >= nch) return;

  // loads that do not depend on each other, issued together
  const int64_t j0 = (int64_t)ch * TK_CHUNK + (int64_t)t * TK_PER_THREAD;
  int32_t v[16];
  load16(scores + (int64_t)row * ld, j0, n, v);
  const int2 rs = w.rowstate[row];
  const i32x4 fq = *reinterpret_cast<const i32x4*>(w.fine + (int64_t)row * FINE_BINS + 1020 - 4 * t);
  const int64_t slot0 = (int64_t)row * w.nchunks;
  int32_t ca[4], cb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * t + e;
    ca[e] = c < ch ? w.cnt_above[slot0 + c] : 0;
    cb[e] = c < ch ? w.cnt_bin[slot0 + c] : 0;
  }
  const int bA = rs.x;
  const int need = k - rs.y;   // keys still to take from the threshold bin (>= 1)

  // fine threshold: thread t owns fine bins 1023-4t .. 1020-4t (descending)
  int32_t fv[4] = {fq[3], fq[2], fq[1], fq[0]};
  if (t < 2) s_b[t] = 0;
  int32_t fs = fv[0] + fv[1] + fv[2] + fv[3];
  int32_t ftot;
  const int32_t fpre = block_excl_scan<TK_NT>(fs, s_scan, &ftot);
  if (fpre < need && fpre + fs >= need) {
    int32_t acc = fpre;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (acc < need && acc + fv[e] >= need) {
        s_b[0] = 1023 - 4 * t - e;
        s_b[1] = acc;
      }
      acc += fv[e];
    }
  }
  __syncthreads();
  const int low_t = s_b[0];
  const int T = (bA << 10) | low_t;       // the k-th largest key
  const int need_eq = need - s_b[1];      // T-valued keys to keep, lowest indices first

  // earlier chunks: above-bA totals, and a prefix of their threshold-bin counts
  int32_t sa = ca[0] + ca[1] + ca[2] + ca[3];
  int32_t sb = cb[0] + cb[1] + cb[2] + cb[3];
  int32_t above_before;
  (void)block_excl_scan<TK_NT>(sa, s_scan, &above_before);
  int32_t bin_before;
  int32_t bpre = block_excl_scan<TK_NT>(sb, s_scan, &bin_before);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * t + e;
    if (c < ch) {
      s_pre[c] = bpre;
      s_ca[c] = ca[e];
    }
    bpre += cb[e];
  }
  if (t == 0) s_pre[ch] = bin_before;
  __syncthreads();

  // earlier chunks' threshold-bin keys: how many beat T, how many equal it
  int32_t gt = 0, eq = 0;
  for (int base = 0; base < bin_before; base += TK_NT * TK_BATCH) {
    int32_t kv[TK_BATCH];
#pragma unroll
    for (int u = 0; u < TK_BATCH; ++u) {
      const int p = base + t + TK_NT * u;
      kv[u] = -1;
      if (p < bin_before) {
        int lo = 0, hi = ch;   // chunk c with s_pre[c] <= p < s_pre[c+1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_pre[mid] <= p) lo = mid; else hi = mid;
        }
        kv[u] = w.bin_keys[(slot0 + lo) * TK_CHUNK + s_ca[lo] + (p - s_pre[lo])];
      }
    }
#pragma unroll
    for (int u = 0; u < TK_BATCH; ++u) {
      if (kv[u] >= 0) {
        const int low = kv[u] & 1023;
        gt += low > low_t ? 1 : 0;
        eq += low == low_t ? 1 : 0;
      }
    }
  }
  int32_t gt_before, eq_before;
  (void)block_excl_scan<TK_NT>(gt, s_scan, &gt_before);
  (void)block_excl_scan<TK_NT>(eq, s_scan, &eq_before);
  const int32_t sel_before = above_before + gt_before + min(eq_before, need_eq);

  // this chunk, in index order
  int32_t ne = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) ne += (j0 + e < n && score_key(v[e]) == T) ? 1 : 0;
  int32_t etot;
  int32_t rank = eq_before + block_excl_scan<TK_NT>(ne, s_scan, &etot);
  uint32_t selmask = 0;
  int32_t ns = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (j0 + e < n) {
      const int key = score_key(v[e]);
      bool sel = key > T;
      if (key == T) sel = rank++ < need_eq;
      if (sel) {
        selmask |= 1u << e;
        ++ns;
      }
    }
  }
  int32_t stot;
  int32_t pos = sel_before + block_excl_scan<TK_NT>(ns, s_scan, &stot);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (selmask & (1u << e)) {
      if (pos < k) irow[pos] = (int32_t)(j0 + e);   // exactly k in total; the bound guards bad input
      ++pos;
    }
}

// ------------------------------------------------------------------ K3' (k <= TK_MERGE_K)
// One work-group per row merges the chunks' candidate lists instead of re-reading the
// scores: the above-bA entries (all selected, fewer than k) and the bA entries that
// beat T or are T-valued within the quota, both already in index order chunk by
// chunk; an entry's output slot is its rank in its own list plus the number of
// entries of the other list with a lower index.
constexpr int TK_MERGE_K = 4096;
constexpr int TK_MNT = 1024;   // threads of the merge work-group
constexpr int TK_MERGE_MIN_ROWS = 32;
__device__ __forceinline__ int upper_le(const int32_t* a, int n, int32_t x) {   // #a[i] <= x
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int lower_lt(const int32_t* a, int n, int32_t x) {   // #a[i] < x
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(TK_MNT) void topk_merge_kernel(TopkBatch tb) {
  const TopkLayer& TL = tb.layer[blockIdx.z];
  const int k = TL.k;
  const int max_n = TL.max_n;
  const TopkWs& w = TL.w;
  __shared__ int32_t s_scan[TK_MNT / WAVE + 1];
  __shared__ int32_t s_b[2];
  __shared__ int32_t s_apre[TK_MAX_CHUNKS + 1];   // above-bA entries before chunk c
  __shared__ int32_t s_bpre[TK_MAX_CHUNKS + 1];   // bA entries before chunk c
  __shared__ int32_t s_above[TK_MERGE_K];          // global indices, ascending
  __shared__ int32_t s_sel[TK_MERGE_K];            // selected bA entries, ascending
  const int row = blockIdx.y;
  const int t = threadIdx.x;
  const int64_t n = min(TL.n_vis[row], max_n);
  int32_t* irow = TL.idx + (int64_t)row * k;
  {   // nobody reads the coarse histogram any more: clear it for the next call
    int32_t* hrow = w.hist + (int64_t)row * HIST_BINS;
    for (int b = t; b < HIST_BINS; b += TK_MNT) hrow[b] = 0;
  }
  if (t == 0) TL.count[row] = (int32_t)min(n, (int64_t)k);
  if (n <= k) {   // every visible entry is selected
    for (int p = t; p < k; p += TK_MNT) irow[p] = p < n ? p : -1;
    return;
  }
  const int nch = (int)((n + TK_CHUNK - 1) / TK_CHUNK);
  const int64_t slot0 = (int64_t)row * w.nchunks;

  // loads that do not depend on each other, issued together: thread t owns chunk t
  // and fine bin 1023 - t
  static_assert(TK_MNT == TK_MAX_CHUNKS && TK_MNT == FINE_BINS, "one chunk and one bin per thread");
  const int2 rs = w.rowstate[row];
  const int32_t fv = w.fine[(int64_t)row * FINE_BINS + 1023 - t];
  const int32_t ca = t < nch ? w.cnt_above[slot0 + t] : 0;
  const int32_t cb = t < nch ? w.cnt_bin[slot0 + t] : 0;
  const int need = k - rs.y;   // keys to take from the threshold bin (>= 1)

  // fine threshold: the bin where the descending count reaches `need`
  if (t < 2) s_b[t] = 0;
  int32_t ftot;
  const int32_t fpre = block_excl_scan<TK_MNT>(fv, s_scan, &ftot);
  if (fpre < need && fpre + fv >= need) {
    s_b[0] = 1023 - t;
    s_b[1] = fpre;
  }
  __syncthreads();
  const int low_t = s_b[0];
  const int need_eq = need - s_b[1];   // T-valued keys to keep, lowest indices first

  // chunk offsets of both lists
  int32_t a_tot, b_tot;
  const int32_t apre = block_excl_scan<TK_MNT>(ca, s_scan, &a_tot);
  const int32_t bpre = block_excl_scan<TK_MNT>(cb, s_scan, &b_tot);
  if (t < nch) {
    s_apre[t] = apre;
    s_bpre[t] = bpre;
  }
  if (t == 0) {
    s_apre[nch] = a_tot;
    s_bpre[nch] = b_tot;
  }
  __syncthreads();
  a_tot = min(a_tot, TK_MERGE_K);   // fewer than k for consistent counts; the bound guards bad input

  // gather the above-bA entries (each chunk's list is in index order), all loads in flight
  {
    constexpr int GU = TK_MERGE_K / TK_MNT;
    int32_t gc[GU], gv[GU];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int p = t + TK_MNT * u;
      gc[u] = 0;
      gv[u] = 0;
      if (p < a_tot) {
        gc[u] = upper_le(s_apre, nch, p) - 1;   // s_apre[c] <= p < s_apre[c+1]
        gv[u] = w.bin_keys[(slot0 + gc[u]) * TK_CHUNK + (p - s_apre[gc[u]])];
      }
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int p = t + TK_MNT * u;
      if (p < a_tot) s_above[p] = gc[u] * TK_CHUNK + gv[u];
    }
  }
  // threshold-bin entries in index order: those above T, and T-valued ones in order
  // until the quota is met
  int32_t eq_run = 0, sel_run = 0;
  for (int base = 0; base < b_tot; base += TK_MNT) {
    const int p = base + t;
    int gi = 0;
    bool gt = false, eq = false;
    if (p < b_tot) {
      const int c = upper_le(s_bpre, nch, p) - 1;
      const int32_t a_c = s_apre[c + 1] - s_apre[c];
      const int32_t kv = w.bin_keys[(slot0 + c) * TK_CHUNK + a_c + (p - s_bpre[c])];
      const int low = kv & 1023;
      gi = c * TK_CHUNK + (kv >> 10);
      gt = low > low_t;
      eq = low == low_t;
    }
    int32_t eq_n;
    const int32_t eq_rank = eq_run + block_excl_scan<TK_MNT>(eq ? 1 : 0, s_scan, &eq_n);
    const bool sel = gt || (eq && eq_rank < need_eq);
    int32_t sel_n;
    const int32_t q = sel_run + block_excl_scan<TK_MNT>(sel ? 1 : 0, s_scan, &sel_n);
    if (sel && q < TK_MERGE_K) s_sel[q] = gi;
    eq_run += eq_n;
    sel_run += sel_n;
  }
  __syncthreads();
  const int nsel = min(sel_run, TK_MERGE_K);
  // merge: rank in own list + entries of the other list with a lower index
  for (int p = t; p < a_tot; p += TK_MNT) {
    const int32_t x = s_above[p];
    const int pos = p + lower_lt(s_sel, nsel, x);
    if (pos < k) irow[pos] = x;
  }
  for (int q = t; q < nsel; q += TK_MNT) {
    const int32_t y = s_sel[q];
    const int pos = q + lower_lt(s_above, a_tot, y);
    if (pos < k) irow[pos] = y;
  }
}

hipError_t launch_topk(const TopkBatch& tb, int rows, bool hist_ready, hipStream_t st) {
  if (rows == 0 || tb.n == 0) return hipSuccess;
  int nch = 1, pch = 1;
  for (int l = 0; l < tb.n; ++l) {
    nch = max(nch, topk_nchunks(tb.layer[l].max_n));
    pch = max(pch, (max(tb.layer[l].max_n, tb.layer[l].k) + TK_CHUNK - 1) / TK_CHUNK);
  }
  if (!hist_ready)
    hipLaunchKernelGGL(topk_hist_kernel, dim3(nch, rows, tb.n), dim3(TK_NT), 0, st, tb);
  hipLaunchKernelGGL(topk_cand_kernel, dim3(nch, rows, tb.n), dim3(TK_NT), 0, st, tb);
  int max_k = 0;
  for (int l = 0; l < tb.n; ++l) max_k = max(max_k, tb.layer[l].k);
  // one work-group per row pays off once there are enough rows to fill the chip's
  // latency; a few rows go faster with every chunk placing its own selections
  if (max_k <= TK_MERGE_K && rows * tb.n >= TK_MERGE_MIN_ROWS)
    hipLaunchKernelGGL(topk_merge_kernel, dim3(1, rows, tb.n), dim3(TK_MNT), 0, st, tb);
  else
    hipLaunchKernelGGL(topk_place_kernel, dim3(pch, rows, tb.n), dim3(TK_NT), 0, st, tb);
  return hipGetLastError();
}

}  // namespace lca
