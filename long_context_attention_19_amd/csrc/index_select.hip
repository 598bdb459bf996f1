// csa_index_select: the indexer scores and their top-k in one kernel, for query
// batches of 16 or more tokens per sequence (prefill), without writing the scores.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 items 2 and 4: CSA scores the compressed entries with an
// indexer (its own Q.K product) and keeps a top-k of them.  The result is exactly
// that of csa_index_score followed by csa_topk_select: per query row, the top
// min(k, n_vis) entries ranked by (score desc, index asc), in ascending index
// order, then -1 padding.
//
// A prefill batch scores every query token against every key: the score matrix
// (4096 x 66,560 int32 = 1.09 GB for a 4096-token chunk at 262K context) would
// cost its write and then a read for the selection.  Here a work-group owns 16
// query tokens of one sequence and all of that sequence's entries, so it sees
// every score of its rows and never needs another work-group's counts.  It
// recomputes the scores with v_mfma_i32_16x16x64_i8 (16 entries x 16 tokens over
// the whole d_idx = 64, exact int32) in sweeps over the keys, which stream from L2
// (every row tile reads the same keys).  Usually two sweeps: the coarse
// histograms, then (when every token's threshold bin holds at most SL_BIN_CAP
// entries) the entries above the bin and inside it, collected in index order and
// resolved in LDS.  Otherwise three:
//   1. the coarse histogram, 2048 bins of key >> 10 per token, in LDS (key =
//      score + 2^20, 21 bits); from it the threshold bin bA holding the k-th
//      largest key and the count above it;
//   2. the fine histogram, 1024 bins of key & 1023 among keys in bin bA; from it
//      the k-th largest key T and how many T-valued keys to keep (lowest
//      indices first);
//   3. the selection, in index order: per round of 1024 entries each wave scans
//      its selected counts per token across its lanes, the waves' totals meet
//      in LDS (one barrier per round), and every selected entry is placed; the
//      rows build up in LDS and leave at the end as whole rows.
// Rows with n_vis <= k select every visible entry (sweeps 1 and 2 skip them).
//
// Operand layout of the MFMA (both operands: lane l supplies row l % 16 of its
// matrix and bytes 16 (l / 16) .. + 15 of it; result: lane l holds entries
// 4 (l / 16) + r, r < 4, of query token l % 16) as in the prefill scoring GEMM.
//
// FP4 indexer (query and keys packed E2M1, 32 bytes per vector): the scores come
// from v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 and unit scales.
// Lane l supplies row l % 16 and elements 32 (l / 16) .. + 31 (16 bytes) of its
// operand; d_idx = 64 fills elements 0..63, so lanes 32..63 supply zeros.  The
// result has the int8 form's layout; the fp32 sums are exact (quarter multiples far
// below 2^24) and the score is 256 x the sum, the unit of csa_index_score_fp4.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int SL_NT = 1024;                   // 16 waves: 4 per SIMD hide the latency
constexpr int SL_NW = SL_NT / WAVE;
constexpr int SL_ROWS = 16;                   // query tokens per work-group (MFMA N)
constexpr int SL_BLOCK = 64;                  // entries per wave and round: 4 MFMA tiles
constexpr int SL_STAGE_K = 2048;              // k up to this: rows are staged in LDS
constexpr int SL_BIN_CAP = 256;              // threshold-bin entries per token, two-sweep path
constexpr int SL_WT = 2 * SL_ROWS * (SL_NT / WAVE);   // wave totals, two round parities
constexpr int SL_FRONT = SL_WT + SL_ROWS * SL_BIN_CAP;   // words ahead of the staged rows
constexpr int SL_LDS = SL_FRONT + SL_ROWS * SL_STAGE_K;   // words; >= 16 x 2048 coarse bins
static_assert(SL_LDS >= SL_ROWS * HIST_BINS, "LDS region must hold the coarse histograms");
static_assert(SL_LDS >= SL_ROWS * FINE_BINS + SL_ROWS, "fine histograms and their counts");
static_assert(SL_NW <= SL_ROWS, "s_tot holds one value per wave");

// The value of lane l ^ 16 (l ^ 32): v_permlane16_swap (v_permlane32_swap) of a
// register with itself returns the lane's own value and its partner's, ordered by
// which half of the pair the lane is in.
__device__ __forceinline__ int32_t sl_partner16(int32_t x) {
  const auto v = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int32_t)((threadIdx.x & 16) ? v[0] : v[1]);
}
__device__ __forceinline__ int32_t sl_partner32(int32_t x) {
  const auto v = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int32_t)((threadIdx.x & 32) ? v[0] : v[1]);
}

__device__ __forceinline__ void sl_lds_barrier() {   // LDS traffic only: no memory fence
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Keys of one 64-entry block: tile u, lane l -> entry blk*64 + 16u + l%16, bytes
// 16 (l/16) ..; entries past N re-read entry N-1 (their scores are never used).
// Ordinary loads: the keys are shared by every row tile and should stay in L2.
// FP4 keys are 2 x 16 bytes: lanes 32..63 load nothing and hold zeros.
template <bool FP4>
__device__ __forceinline__ void sl_load(i32x4 (&kv)[4], const i32x4* __restrict__ kp, int32_t blk,
                                        int32_t N, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t j = min(blk * SL_BLOCK + 16 * u + (lane & 15), N - 1);
    if (FP4)
      kv[u] = lane < 32 ? kp[j * 2 + (lane >> 4)] : i32x4{0, 0, 0, 0};
    else
      kv[u] = kp[j * 4 + (lane >> 4)];
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The block's 16 keys (score + 2^20) of this lane's token: [tile u][r].
template <bool FP4>
__device__ __forceinline__ void sl_keys(const i32x4 (&kv)[4], const i32x4& qv, int32_t (&key)[4][4]) {
  const i32x4 zero4 = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (FP4) {
      constexpr int FP4_E2M1 = 4, UNIT_SCALE = 127;   // operand format code, E8M0 2^0
      const i32x8 ka = {kv[u][0], kv[u][1], kv[u][2], kv[u][3], 0, 0, 0, 0};
      const i32x8 qb = {qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
      const f32x4_t acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          ka, qb, f32x4_t{0.f, 0.f, 0.f, 0.f}, FP4_E2M1, FP4_E2M1, 0, UNIT_SCALE, 0, UNIT_SCALE);
#pragma unroll
      for (int r = 0; r < 4; ++r) key[u][r] = (int32_t)(acc[r] * 256.f) + KEY_BIAS;
    } else {
      const i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kv[u], qv, zero4, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) key[u][r] = acc[r] + KEY_BIAS;
    }
  }
}

// One sweep over the work-group's blocks, keys loaded two rounds ahead; `body`
// gets (keys, round, block).  Every wave runs every round (a block past the end
// has no visible entry), so bodies may hold work-group barriers.
template <bool FP4, class Body>
__device__ __forceinline__ void sl_sweep(const i32x4* __restrict__ kp, const i32x4& qv, int32_t N,
                                         int32_t nround, int w, int lane, Body&& body) {
  i32x4 ka[4], kb[4], kc[4];
  int32_t key[4][4];
  sl_load<FP4>(ka, kp, w, N, lane);
  sl_load<FP4>(kb, kp, SL_NW + w, N, lane);
  for (int32_t rd = 0; rd < nround; rd += 3) {
    sl_load<FP4>(kc, kp, (rd + 2) * SL_NW + w, N, lane);
    sl_keys<FP4>(ka, qv, key);
    body(key, rd, rd * SL_NW + w);
    sl_load<FP4>(ka, kp, (rd + 3) * SL_NW + w, N, lane);
    sl_keys<FP4>(kb, qv, key);
    body(key, rd + 1, (rd + 1) * SL_NW + w);
    sl_load<FP4>(kb, kp, (rd + 4) * SL_NW + w, N, lane);
    sl_keys<FP4>(kc, qv, key);
    body(key, rd + 2, (rd + 2) * SL_NW + w);
  }
}

// Threshold of one token's histogram (nbins bins, bin b at h[b ^ j]), by one wave:
// the bin holding the need-th largest key and the count in higher bins.  Blocks of 64
// bins from the top, lane l reading bin top - l (consecutive banks), each scanned
// across the wave until the running count reaches `need` (the caller guarantees the
// histogram holds at least that many keys).
template <int NBINS>
__device__ __forceinline__ void sl_threshold(const int32_t* h, int j, int need, int lane,
                                             int32_t* out_bin, int32_t* out_above) {
  int32_t acc = 0;   // keys in the blocks above the current one
  for (int blk = 0; blk < NBINS / WAVE; ++blk) {
    const int b = NBINS - 1 - blk * WAVE - lane;
    const int32_t c = h[b ^ j];
    const int32_t incl = wave_incl_scan(c);   // keys in this block's bins >= b
    const int32_t tot = __shfl(incl, WAVE - 1, WAVE);
    if (acc + tot >= need) {   // wave-uniform: the bin is in this block
      if (acc + incl >= need && acc + incl - c < need) {   // exactly one lane
        *out_bin = b;
        *out_above = acc + incl - c;
      }
      return;
    }
    acc += tot;
  }
}

// Two-sweep path, second sweep: each token's entries above its threshold bin bA
// (all of them selected; fewer than k) and inside bA, each list in index order
// (bA = -1 for a token that keeps every visible entry: they all count as above).
// Then one wave per token resolves the threshold inside bA by ranking the bin's
// entries (score desc, index asc), and writes the row: each entry's slot is its
// rank in its own list plus the number of selected entries of the other list
// with a lower index.
template <bool FP4>
__device__ __forceinline__ void sl_collect_finalize(
    const i32x4* __restrict__ kp, const i32x4& qv, int32_t N, int32_t nround, int w, int lane,
    int n, int grp, int32_t nv, int32_t bA, int k, int nr, int32_t* sm, int32_t* s_tot,
    int32_t* s_na, int32_t* s_nb, int32_t* __restrict__ idx0) {
  int32_t* wt = sm;                                // [2][16][waves] wave totals
  int32_t* blist = sm + SL_WT;                     // [16][SL_BIN_CAP] (index << 10 | key & 1023)
  int32_t* alist = sm + SL_FRONT;                  // [16][SL_STAGE_K] indices above bA
  int32_t a_base = 0, b_base = 0;
  __syncthreads();
  sl_sweep<FP4>(kp, qv, N, nround, w, lane, [&](const int32_t (&key)[4][4], int32_t rd, int32_t blk) __attribute__((always_inline)) {
    uint32_t ba[4], bb[4];
    int32_t ex[4];
    int32_t wtot = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ba[u] = 0;
      bb[u] = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool vis = blk * SL_BLOCK + 16 * u + 4 * grp + r < nv;
        const int32_t bin = key[u][r] >> 10;
        ba[u] |= (uint32_t)(vis && bin > bA) << r;
        bb[u] |= (uint32_t)(vis && bin == bA) << r;
      }
      const int32_t cnt = (int32_t)((__builtin_popcount(bb[u]) << 16) | __builtin_popcount(ba[u]));
      const int32_t c1 = sl_partner16(cnt);
      const int32_t pair = cnt + c1;
      const int32_t x = (grp & 1) ? pair : cnt;
      const int32_t lowpair = sl_partner32(pair);
      ex[u] = wtot + ((grp & 2) ? x + lowpair : x) - cnt;
      wtot += pair + lowpair;
    }
    int32_t* wr = wt + (rd & 1) * (SL_ROWS * SL_NW) + n * SL_NW;
    if (grp == 0) wr[w] = wtot;
    sl_lds_barrier();
    int32_t pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < SL_NW; ++i) {
      const int32_t v = wr[i];
      pre += i < w ? v : 0;
      tot += v;
    }
    // entries above bA: walk the set bits
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) m |= ba[u] << (4 * u);
    while (m) {
      const int bit = __builtin_ctz(m);
      m &= m - 1;
      const int u = bit >> 2, r = bit & 3;
      const uint32_t bau = u == 0 ? ba[0] : u == 1 ? ba[1] : u == 2 ? ba[2] : ba[3];
      const int32_t exu = u == 0 ? ex[0] : u == 1 ? ex[1] : u == 2 ? ex[2] : ex[3];
      const int32_t pos = a_base + ((pre + exu) & 0xffff) + __builtin_popcount(bau & ((1u << r) - 1));
      if (pos < SL_STAGE_K) alist[n * SL_STAGE_K + pos] = blk * SL_BLOCK + 16 * u + 4 * grp + r;
    }
    // entries inside bA (rare)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (bb[u] == 0) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (bb[u] >> r & 1) {
          const int32_t pos = b_base + ((pre + ex[u]) >> 16) + __builtin_popcount(bb[u] & ((1u << r) - 1));
          if (pos < SL_BIN_CAP)
            blist[n * SL_BIN_CAP + pos] = ((blk * SL_BLOCK + 16 * u + 4 * grp + r) << 10) | (key[u][r] & 1023);
        }
      }
    }
    a_base += tot & 0xffff;
    b_base += tot >> 16;
  });
  if (w == 0 && grp == 0) {
    s_na[n] = a_base;
    s_nb[n] = b_base;
  }
  __syncthreads();
  // one wave per token
  for (int j = w; j < nr; j += SL_NW) {
    const int32_t na = min(s_na[j], SL_STAGE_K), nb = min(s_nb[j], SL_BIN_CAP);
    const int32_t need = max(0, k - na);                // keys to take from the bin
    int32_t* bl = blist + j * SL_BIN_CAP;
    const int32_t* al = alist + j * SL_STAGE_K;
    constexpr int PB = SL_BIN_CAP / WAVE;
    int32_t e[PB], rank[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      e[u] = lane + WAVE * u < nb ? bl[lane + WAVE * u] : 0;
      rank[u] = 0;
    }
    for (int q = 0; q < nb; ++q) {   // rank by (key desc, index asc)
      const int32_t lq = bl[q] & 1023;
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int32_t li = e[u] & 1023;
        rank[u] += (lq > li || (lq == li && q < lane + WAVE * u)) ? 1 : 0;
      }
    }
    // selected bin entries, and how many of them precede each list position
    int32_t run = 0;
    int32_t sel_ex[PB];
    bool sel[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      sel[u] = lane + WAVE * u < nb && rank[u] < need;
      const uint64_t bal = __ballot(sel[u]);
      sel_ex[u] = run + __builtin_popcountll(bal & ((1ull << lane) - 1));
      run += __builtin_popcountll(bal);
    }
    const int32_t nsel = run;
#pragma unroll
    for (int u = 0; u < PB; ++u)   // keep the index, replace the key bits by the count
      if (lane + WAVE * u < nb) bl[lane + WAVE * u] = (e[u] & ~1023) | sel_ex[u];
    int32_t* orow = idx0 + (int64_t)j * k;
    for (int p = lane; p < na; p += WAVE) {   // above-bA entries
      const int32_t x = al[p];
      int lo = 0, hi = nb;                     // bin entries with a lower index
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((bl[mid] >> 10) < x) lo = mid + 1; else hi = mid;
      }
      const int32_t before = lo < nb ? (bl[lo] & 1023) : nsel;
      const int32_t pos = p + before;
      if (pos < k) orow[pos] = x;
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {            // selected bin entries
      if (!sel[u]) continue;
      const int32_t y = e[u] >> 10;
      int lo = 0, hi = na;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (al[mid] < y) lo = mid + 1; else hi = mid;
      }
      const int32_t pos = sel_ex[u] + lo;
      if (pos < k) orow[pos] = y;
    }
    for (int p = na + nsel + lane; p < k; p += WAVE) orow[p] = -1;
  }
}

template <bool STAGE, bool FP4>
__global__ __launch_bounds__(SL_NT) void index_select_kernel(SelectArgs a, int tiles_per_seq) {
  __shared__ __attribute__((aligned(16))) int32_t sm[SL_LDS];
  __shared__ int32_t s_bin[SL_ROWS], s_above[SL_ROWS], s_tot[SL_ROWS], s_flag;
  __shared__ int32_t s_na[SL_ROWS], s_nb[SL_ROWS];
  const int b = blockIdx.y / tiles_per_seq;
  const int q0 = (blockIdx.y - b * tiles_per_seq) * SL_ROWS;
  const int64_t r0 = a.q_off[b];
  const int64_t nrows = a.q_off[b + 1] - r0;
  if (q0 >= nrows) return;
  const int nr = (int)min((int64_t)SL_ROWS, nrows - q0);
  const int64_t e0 = a.ent_off[b];
  const int32_t N = (int32_t)min(a.ent_off[b + 1] - e0, (int64_t)a.max_entries);
  const int k = a.k;
  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(t / WAVE);
  const int n = lane & 15;                 // query token of this lane (tile column)
  const int grp = lane >> 4;               // lane group: entries 4 grp .. 4 grp + 3 of a tile
  const bool qok = n < nr;
  const int64_t row = r0 + q0 + (qok ? n : 0);
  const int32_t nv = qok ? (int32_t)min(a.q_pos[row] / a.c, (int64_t)N) : 0;
  const bool thr = nv > k;                 // this lane's token needs the threshold
  int32_t* __restrict__ idx0 = a.idx + (r0 + q0) * k;

  if (t == 0) s_flag = 0;
  if (t < SL_ROWS) {
    s_bin[t] = -1;
    s_above[t] = 0;
  }
  __syncthreads();
  if (t < nr) {
    const int32_t v = (int32_t)min(a.q_pos[r0 + q0 + t] / a.c, (int64_t)N);
    if (a.n_vis) a.n_vis[r0 + q0 + t] = v;
    a.count[r0 + q0 + t] = min(v, k);
  }
  if (thr) s_flag = 1;                     // benign race: every writer stores 1
  // entries visible to some token of the group: the sweeps stop there
  int32_t mx = nv;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) mx = max(mx, __shfl_xor(mx, d, WAVE));
  if (lane == 0) s_tot[w] = mx;            // s_tot doubles as scratch here
  __syncthreads();
  int32_t nvmax = 0;
  for (int i = 0; i < SL_NW; ++i) nvmax = max(nvmax, s_tot[i]);
  const bool any_thr = s_flag != 0;
  const int32_t nblk = (nvmax + SL_BLOCK - 1) / SL_BLOCK;
  const int32_t nround = (nblk + SL_NW - 1) / SL_NW;

  constexpr int VB = FP4 ? 32 : 64;        // bytes per indexer vector
  const i32x4* kp = reinterpret_cast<const i32x4*>(a.k_idx + e0 * VB);
  const i32x4 zero4 = {0, 0, 0, 0};
  const i32x4 qv = qok && 16 * grp < VB ? *reinterpret_cast<const i32x4*>(a.q_idx + row * VB + 16 * grp)
                                        : zero4;

  if (nvmax > 0 && any_thr) {
    // ---- sweep 1: coarse histograms
    for (int i = t; i < SL_ROWS * HIST_BINS; i += SL_NT) sm[i] = 0;
    __syncthreads();
    int32_t* hc = sm + n * HIST_BINS;
    sl_sweep<FP4>(kp, qv, N, nround, w, lane, [&](const int32_t (&key)[4][4], int32_t, int32_t blk) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (thr && blk * SL_BLOCK + 16 * u + 4 * grp + r < nv)
            atomicAdd(&hc[(key[u][r] >> 10) ^ n], 1);
    });
    __syncthreads();
    for (int j = w; j < nr; j += SL_NW) {
      const int32_t vj = (int32_t)min(a.q_pos[r0 + q0 + j] / a.c, (int64_t)N);
      if (vj > k) sl_threshold<HIST_BINS>(sm + j * HIST_BINS, j, k, lane, &s_bin[j], &s_above[j]);
    }
    // Two-sweep path: when every token's threshold bin holds at most SL_BIN_CAP
    // entries (the usual case: about k/20 for Gaussian-like scores), one more sweep
    // collects each token's entries above the bin and inside it, in index order,
    // and the threshold and the merge are resolved in LDS.
    if (t == 0) s_flag = (STAGE && N < (1 << 21)) ? 1 : 0;
    __syncthreads();
    if (t < nr && s_bin[t] >= 0 && sm[t * HIST_BINS + (s_bin[t] ^ t)] > SL_BIN_CAP) s_flag = 0;
    __syncthreads();
    if (s_flag) {
      sl_collect_finalize<FP4>(kp, qv, N, nround, w, lane, n, grp, nv, thr ? s_bin[n] : -1, k, nr,
                          sm, s_tot, s_na, s_nb, idx0);
      return;
    }
    // ---- sweep 2: fine histograms of the threshold bins
    const int32_t bA = s_bin[n];
    for (int i = t; i < SL_ROWS * FINE_BINS; i += SL_NT) sm[i] = 0;
    __syncthreads();
    int32_t* hf = sm + n * FINE_BINS;
    sl_sweep<FP4>(kp, qv, N, nround, w, lane, [&](const int32_t (&key)[4][4], int32_t, int32_t blk) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (thr && blk * SL_BLOCK + 16 * u + 4 * grp + r < nv && (key[u][r] >> 10) == bA)
            atomicAdd(&hf[(key[u][r] & 1023) ^ n], 1);
    });
    __syncthreads();
    if (t < SL_ROWS) {   // keep bA while the fine threshold overwrites s_bin
      s_tot[t] = s_bin[t];
    }
    __syncthreads();
    for (int j = w; j < nr; j += SL_NW) {
      const int32_t vj = (int32_t)min(a.q_pos[r0 + q0 + j] / a.c, (int64_t)N);
      if (vj > k)
        sl_threshold<FINE_BINS>(sm + j * FINE_BINS, j, k - s_above[j], lane, &s_bin[j],
                                &sm[SL_ROWS * FINE_BINS + j]);
    }
    __syncthreads();
    if (t < SL_ROWS) {
      // T = the k-th largest key; need_eq = T-valued keys to keep
      const int32_t low = s_bin[t];
      s_bin[t] = (s_tot[t] << 10) | low;
      s_above[t] = k - s_above[t] - sm[SL_ROWS * FINE_BINS + t];
    }
    __syncthreads();
  }

  // ---- sweep 3: the selection in index order
  const int32_t T = thr ? s_bin[n] : 0;
  const int32_t need_eq = thr ? s_above[n] : 0;
  int32_t* wt = sm;                               // [2][16][8] wave totals, by round parity
  int32_t* out = sm + SL_FRONT;                   // [16][k] staged rows (STAGE)
  int32_t* orow = STAGE ? out + n * k : idx0 + n * k;
  int32_t a_base = 0, e_base = 0;                 // selected-above / T-valued so far (row n)
  __syncthreads();
  if (nvmax > 0) {
    sl_sweep<FP4>(kp, qv, N, nround, w, lane, [&](const int32_t (&key)[4][4], int32_t rd, int32_t blk) __attribute__((always_inline)) {
      // Counts are packed (T-valued << 16 | above); a round adds at most 1024 to
      // either half.  Within the wave, segment (tile u, lane group g) precedes
      // (u, g') for g < g' and every segment of tiles after u: a scan over the
      // row's 4 lanes (n, n+16, n+32, n+48) per tile.
      uint32_t ba[4], be[4];
      int32_t ex[4];
      int32_t wtot = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ba[u] = 0;
        be[u] = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = blk * SL_BLOCK + 16 * u + 4 * grp + r < nv;
          const bool above = vis && (!thr || key[u][r] > T);
          const bool eq = vis && thr && key[u][r] == T;
          ba[u] |= (uint32_t)above << r;
          be[u] |= (uint32_t)eq << r;
        }
        const int32_t cnt = (int32_t)((__builtin_popcount(be[u]) << 16) | __builtin_popcount(ba[u]));
        // inclusive scan over the lane groups with two lane swaps (no LDS):
        // pair (0,1) and (2,3) sums, then the lower pair's sum for groups 2, 3
        const int32_t c1 = sl_partner16(cnt);
        const int32_t pair = cnt + c1;
        const int32_t x = (grp & 1) ? pair : cnt;
        const int32_t lowpair = sl_partner32(pair);
        ex[u] = wtot + ((grp & 2) ? x + lowpair : x) - cnt;
        wtot += pair + lowpair;
      }
      int32_t* wr = wt + (rd & 1) * (SL_ROWS * SL_NW) + n * SL_NW;
      if (grp == 0) wr[w] = wtot;
      sl_lds_barrier();   // the only barrier of the round: the totals alternate buffers
      int32_t pre = 0, tot = 0;
#pragma unroll
      for (int i = 0; i < SL_NW; ++i) {
        const int32_t v = wr[i];
        pre += i < w ? v : 0;
        tot += v;
      }
      // Placement: a selected entry's slot is the number of selected entries
      // before it (above-T ones all count, T-valued ones up to the quota).  About
      // 3% of entries are candidates, so each lane walks only its set bits.
      uint32_t m = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) m |= (ba[u] | be[u]) << (4 * u);
      while (m) {
        const int bit = __builtin_ctz(m);
        m &= m - 1;
        const int u = bit >> 2, r = bit & 3;
        const uint32_t bau = u == 0 ? ba[0] : u == 1 ? ba[1] : u == 2 ? ba[2] : ba[3];
        const uint32_t beu = u == 0 ? be[0] : u == 1 ? be[1] : u == 2 ? be[2] : be[3];
        const int32_t exu = u == 0 ? ex[0] : u == 1 ? ex[1] : u == 2 ? ex[2] : ex[3];
        const uint32_t below = (1u << r) - 1;
        const int32_t p = pre + exu;
        const int32_t ab = a_base + (p & 0xffff) + __builtin_popcount(bau & below);
        const int32_t eb = e_base + (p >> 16) + __builtin_popcount(beu & below);
        const bool isa = bau >> r & 1;
        const int32_t pos = isa ? ab + min(eb, need_eq) : ab + eb;
        if (qok && pos < k && (isa || eb < need_eq))
          orow[pos] = blk * SL_BLOCK + 16 * u + 4 * grp + r;
      }
      a_base += tot & 0xffff;
      e_base += tot >> 16;
    });
  }
  // rows leave whole (staged), with -1 past count
  if (STAGE) {
    __syncthreads();
    for (int i = t; i < nr * k; i += SL_NT) {
      const int j = i / k, p = i - j * k;
      const int32_t vj = (int32_t)min(a.q_pos[r0 + q0 + j] / a.c, (int64_t)N);
      idx0[i] = p < min(vj, k) ? out[i] : -1;
    }
  } else {
    __syncthreads();
    for (int i = t; i < nr * k; i += SL_NT) {
      const int j = i / k, p = i - j * k;
      const int32_t vj = (int32_t)min(a.q_pos[r0 + q0 + j] / a.c, (int64_t)N);
      if (p >= min(vj, k)) idx0[i] = -1;
    }
  }
}

hipError_t launch_index_select(const SelectArgs& a, int batch, hipStream_t st) {
  if (batch == 0 || a.max_q == 0) return hipSuccess;
  const int tiles = (a.max_q + SL_ROWS - 1) / SL_ROWS;
  dim3 grid(1, (unsigned)(batch * tiles));
  const bool stage = a.k <= SL_STAGE_K;
  if (a.fp4) {
    if (stage) hipLaunchKernelGGL((index_select_kernel<true, true>), grid, dim3(SL_NT), 0, st, a, tiles);
    else hipLaunchKernelGGL((index_select_kernel<false, true>), grid, dim3(SL_NT), 0, st, a, tiles);
  } else {
    if (stage) hipLaunchKernelGGL((index_select_kernel<true, false>), grid, dim3(SL_NT), 0, st, a, tiles);
    else hipLaunchKernelGGL((index_select_kernel<false, false>), grid, dim3(SL_NT), 0, st, a, tiles);
  }
  return hipGetLastError();
}

}  // namespace lca
