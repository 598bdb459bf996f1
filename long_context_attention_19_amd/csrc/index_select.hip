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
#include <type_traits>

#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int SL_NT = 1024;                   // 16 waves: 4 per SIMD hide the latency
constexpr int SL_NW = SL_NT / WAVE;
constexpr int SL_ROWS = 16;                   // query tokens per work-group (MFMA N)
constexpr int SL_BLOCK = 64;                  // entries per wave and round: 4 MFMA tiles
constexpr int SL_STAGE_K = 2048;              // k up to this: rows are staged in LDS
constexpr int SL_BIN_CAP = 448;              // threshold-bin entries per token, two-sweep path
constexpr int SL_WT = 2 * SL_ROWS * (SL_NT / WAVE);   // wave totals, two round parities
constexpr int SL_FRONT = SL_WT + SL_ROWS * SL_BIN_CAP;   // words ahead of the staged rows
constexpr int SL_LDS = SL_FRONT + SL_ROWS * SL_STAGE_K;   // words; >= 16 x 2048 coarse bins
static_assert(SL_LDS >= SL_ROWS * HIST_BINS, "LDS region must hold the coarse histograms");
static_assert(SL_LDS >= SL_ROWS * FINE_BINS + SL_ROWS, "fine histograms and their counts");
static_assert(SL_NW <= SL_ROWS, "s_tot holds one value per wave");
// Bitmap path: after the threshold-bin lists, one bit per entry for each token
// (entries above the bin, then the bin's selected ones), in the rest of the region.
constexpr int SL_BM_WORDS = (SL_LDS - SL_ROWS * SL_BIN_CAP) / SL_ROWS;   // per token
constexpr int SL_BM_MAX = SL_BM_WORDS * 32;                               // entries
static_assert(SL_BM_WORDS % 16 == 0, "a word index XOR a token (< 16) stays in the bitmap");
static_assert(SL_ROWS * SL_BIN_CAP + SL_ROWS * SL_BM_WORDS <= SL_LDS, "bitmaps fit the region");

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
// Ordinary loads: the keys are shared by every row tile and should stay in L2.  They go
// through a buffer resource over the sequence's keys: a 32-bit offset per load instead
// of a 64-bit address (the compiler keeps the first loads' addresses of every sweep
// live across the whole kernel otherwise, and spills them).
// FP4 keys are 2 x 16 bytes: lanes 32..63 load nothing and hold zeros.
template <bool FP4>
__device__ __forceinline__ void sl_load(i32x4 (&kv)[4], __amdgpu_buffer_rsrc_t rs, int32_t blk,
                                        int32_t N, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t j = min(blk * SL_BLOCK + 16 * u + (lane & 15), N - 1);
    if (FP4)
      kv[u] = lane < 32 ? __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rs, (j * 2 + (lane >> 4)) * 16, 0, 0))
                        : i32x4{0, 0, 0, 0};
    else
      kv[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, (j * 4 + (lane >> 4)) * 16, 0, 0));
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The block's 16 raw scores of this lane's token: [tile u][r] (int32; the FP4 form in its
// unit, 256 x the E2M1 dot product).  The sweeps compare raw scores against limits mapped
// from the 21-bit key space (sl_raw_limit); only the histograms form keys.
template <bool FP4>
__device__ __forceinline__ void sl_scores(const i32x4 (&kv)[4], const i32x4& qv, int us, int32_t (&sc)[4][4]) {
  const i32x4 zero4 = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (FP4) {
      constexpr int FP4_E2M1 = 4;   // operand format code; `us` holds the E8M0 unit scale 2^0
      const i32x8 ka = {kv[u][0], kv[u][1], kv[u][2], kv[u][3], 0, 0, 0, 0};
      const i32x8 qb = {qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
      const f32x4_t acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          ka, qb, f32x4_t{0.f, 0.f, 0.f, 0.f}, FP4_E2M1, FP4_E2M1, 0, us, 0, us);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[u][r] = (int32_t)(acc[r] * 256.f);
    } else {
      const i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kv[u], qv, zero4, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[u][r] = acc[r];
    }
  }
}

// score_key(s) >= lim exactly when s >= sl_raw_limit(lim): keys are min(s, 2^20 - 1) + 2^20,
// so below 2^21 the limit moves down by 2^20, and a limit past the largest key (2^21 - 1)
// admits no score (not even 2^20, whose key is clamped).
__device__ __forceinline__ int32_t sl_raw_limit(int32_t lim) {
  return lim >= (1 << 21) ? INT32_MAX : lim - KEY_BIAS;
}

// Rounds [r0, r1) of a sweep (and up to two past r1), keys loaded two rounds ahead;
// `body` gets (ALL, scores, round, block), ALL an integral constant: true when every
// entry of the round is visible to every token of the group (no per-entry test).
template <bool FP4, bool ALL, class Body>
__device__ __forceinline__ void sl_sweep_part(__amdgpu_buffer_rsrc_t kp, const i32x4& qv, int us, int32_t N,
                                              int32_t r0, int32_t r1, int w, int lane, Body& body) {
  i32x4 ka[4], kb[4], kc[4];
  int32_t sc[4][4];
  const std::integral_constant<bool, ALL> all{};
  // the part's first offsets are recomputed here, not kept from an earlier sweep (which
  // would hold them in registers across the whole kernel)
  int wv = w;
  asm volatile("" : "+s"(wv));
  sl_load<FP4>(ka, kp, r0 * SL_NW + wv, N, lane);
  sl_load<FP4>(kb, kp, (r0 + 1) * SL_NW + wv, N, lane);
  for (int32_t rd = r0; rd < r1; rd += 3) {
    sl_load<FP4>(kc, kp, (rd + 2) * SL_NW + w, N, lane);
    sl_scores<FP4>(ka, qv, us, sc);
    body(all, sc, rd, rd * SL_NW + w);
    sl_load<FP4>(ka, kp, (rd + 3) * SL_NW + w, N, lane);
    sl_scores<FP4>(kb, qv, us, sc);
    body(all, sc, rd + 1, (rd + 1) * SL_NW + w);
    sl_load<FP4>(kb, kp, (rd + 4) * SL_NW + w, N, lane);
    sl_scores<FP4>(kc, qv, us, sc);
    body(all, sc, rd + 2, (rd + 2) * SL_NW + w);
  }
}

// One sweep over the work-group's blocks: the rounds below every token's visible count
// (a multiple of 3 of them) without visibility tests, then the rest with them.  Every
// wave runs every round (a block past the end has no visible entry), so bodies may hold
// work-group barriers.
template <bool FP4, class Body>
__device__ __forceinline__ void sl_sweep(__amdgpu_buffer_rsrc_t kp, const i32x4& qv, int us, int32_t N,
                                         int32_t nround, int32_t nfull, int w, int lane, Body&& body) {
  const int32_t nf = min(nfull, nround) / 3 * 3;
  if (nf > 0) sl_sweep_part<FP4, true>(kp, qv, us, N, 0, nf, w, lane, body);
  if (nf < nround) sl_sweep_part<FP4, false>(kp, qv, us, N, nf, nround, w, lane, body);
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
// Then one wave per token resolves the threshold inside bA (the bin's largest keys,
// ties to the lower index) and writes the row: each entry's slot is its position in
// its own list plus the number of selected entries of the other list with a lower
// index.
template <bool FP4>
__device__ __forceinline__ void sl_collect_finalize(
    __amdgpu_buffer_rsrc_t kp, const i32x4& qv, int us, int32_t N, int32_t nround, int32_t nfull, int w,
    int lane, int n, int grp, bool qok, int32_t nv, int32_t bA, int k, int nr, int32_t* sm,
    int32_t* s_tot, int32_t* s_na, int32_t* s_nb, int32_t* __restrict__ idx0) {
  int32_t* wt = sm;                                // [2][16][waves] wave totals
  int32_t* blist = sm + SL_WT;                     // [16][SL_BIN_CAP] (index << 10 | key & 1023)
  int32_t* alist = sm + SL_FRONT;                  // [16][SL_STAGE_K] indices above bA
  int32_t a_base = 0, b_base = 0;
  // key limits: above the bin is key >= lim_a, inside it lim_b <= key < lim_a (bA = -1:
  // every key is above); a lane without a token takes no key
  const int32_t lim_a = sl_raw_limit(qok ? (bA + 1) << 10 : INT32_MAX);
  const int32_t lim_b = sl_raw_limit(qok ? max(bA, 0) << 10 : INT32_MAX);
  __syncthreads();
  sl_sweep<FP4>(kp, qv, us, N, nround, nfull, w, lane, [&](auto all, const int32_t (&sc)[4][4], int32_t rd, int32_t blk) __attribute__((always_inline)) {
    constexpr bool ALL = decltype(all)::value;
    uint32_t ba[4], bb[4];
    // entry e_lane + 16 u + r is visible when 16 u + r < vlim
    const int32_t e_lane = blk * SL_BLOCK + 4 * grp;
    const int32_t vlim = nv - e_lane;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t a = 0, c = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool vis = ALL || 16 * u + r < vlim;
        a |= vis && sc[u][r] >= lim_a ? 1u << r : 0u;
        c |= vis && sc[u][r] >= lim_b ? 1u << r : 0u;
      }
      ba[u] = a;
      bb[u] = c & ~a;
    }
    // List offsets within the wave: segment (tile u, lane group g) precedes (u, g') for
    // g < g' and every segment of later tiles.  The lane's four tile counts are packed one
    // byte each (at most 4); a butterfly over the token's 4 lanes (two lane swaps) gives
    // every tile's total and the lane's count of lower groups at once, and the earlier
    // tiles' totals are byte shifts of the totals: every byte stays below 64, no carries.
    auto wave_offsets = [&](const uint32_t (&m)[4], uint32_t& off, uint32_t& wsum) __attribute__((always_inline)) {
      uint32_t pk = __builtin_popcount(m[3]);
      pk = (pk << 8) + __builtin_popcount(m[2]);
      pk = (pk << 8) + __builtin_popcount(m[1]);
      pk = (pk << 8) + __builtin_popcount(m[0]);
      const uint32_t s16 = (uint32_t)sl_partner16((int32_t)pk);
      const uint32_t t1 = pk + s16;
      const uint32_t s32 = (uint32_t)sl_partner32((int32_t)t1);
      const uint32_t tall = t1 + s32;                                   // tile totals
      const uint32_t tp = (tall << 8) + (tall << 16) + (tall << 24);   // earlier tiles
      off = ((grp & 1) ? s16 : 0u) + ((grp & 2) ? s32 : 0u) + tp;
      wsum = (tp >> 24) + (tall >> 24);
    };
    uint32_t off_a, wsum_a, off_b = 0, wsum_b = 0;
    wave_offsets(ba, off_a, wsum_a);
    const bool any_b = (bb[0] | bb[1] | bb[2] | bb[3]) != 0;
    if (__builtin_amdgcn_ballot_w64(any_b)) wave_offsets(bb, off_b, wsum_b);   // rare
    int32_t* wr = wt + (rd & 1) * (SL_ROWS * SL_NW) + n * SL_NW;
    if (grp == 0) wr[w] = (int32_t)(wsum_a | wsum_b << 16);
    sl_lds_barrier();
    int32_t pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < SL_NW; ++i) {
      const int32_t v = wr[i];
      pre += i < w ? v : 0;
      tot += v;
    }
    // entries above bA: walk the lane's set bits (tile-major, so in entry order); the
    // list position is the tile's base plus the lane's earlier bits in the same tile.
    // Tile bases, 16 bits each: tiles 0 and 2 in one word, 1 and 3 in the other.
    {
      const uint32_t mall = ba[0] | ba[1] << 4 | ba[2] << 8 | ba[3] << 12;
      const uint32_t base = (uint32_t)(a_base + (pre & 0xffff));
      const uint32_t base2 = base | base << 16;
      const uint32_t bw02 = (off_a & 0x00ff00ffu) + base2, bw13 = ((off_a >> 8) & 0x00ff00ffu) + base2;
      uint32_t m = mall;
      while (m) {
        const int bit = __builtin_ctz(m);
        m &= m - 1;
        const uint32_t word = (bit & 4) ? bw13 : bw02;
        const int32_t pos = (int32_t)((word >> ((bit & 8) << 1)) & 0xffff) +
                            __builtin_popcount(__builtin_amdgcn_ubfe(mall, bit & 12, bit & 3));
        if (pos < SL_STAGE_K) alist[n * SL_STAGE_K + pos] = e_lane + (bit & 12) * 4 + (bit & 3);
      }
    }
    // entries inside bA (rare: one branch for the wave when there are none)
    if (any_b) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (bb[u] >> r & 1) {
            const int32_t pos = b_base + (pre >> 16) + (int32_t)((off_b >> (8 * u)) & 0xff) +
                                __builtin_popcount(bb[u] & ((1u << r) - 1));
            if (pos < SL_BIN_CAP)
              blist[n * SL_BIN_CAP + pos] = ((e_lane + 16 * u + r) << 10) | (score_key(sc[u][r]) & 1023);
          }
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
  const uint64_t lt_mask = (1ull << lane) - 1;   // lanes below this one
  for (int j = w; j < nr; j += SL_NW) {
    const int32_t na = min(s_na[j], SL_STAGE_K), nb = min(s_nb[j], SL_BIN_CAP);
    const int32_t need = max(0, k - na);                // keys to take from the bin
    int32_t* bl = blist + j * SL_BIN_CAP;
    const int32_t* al = alist + j * SL_STAGE_K;
    constexpr int PB = SL_BIN_CAP / WAVE;
    int32_t e[PB], kl[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const bool ok = lane + WAVE * u < nb;
      e[u] = ok ? bl[lane + WAVE * u] : 0;
      kl[u] = ok ? (e[u] & 1023) : -1;                // an empty slot takes no threshold
    }
    // The bin's `need` largest keys by (key desc, index asc): the threshold t is the
    // largest value with at least `need` low key bits >= t (a binary search over the 10
    // bits, counted by ballots); keys above t are taken, and of the keys equal to t the
    // first ones in list order (index order) up to the quota.
    auto count_ge = [&](int32_t v) __attribute__((always_inline)) {
      int32_t c = 0;
#pragma unroll
      for (int u = 0; u < PB; ++u) c += __builtin_popcountll(__ballot(kl[u] >= v));
      return c;
    };
    int32_t t, quota;
    if (need == 0) {               // wave-uniform: nothing from the bin
      t = 1024;
      quota = 0;
    } else if (need >= nb) {       // the whole bin
      t = 0;
      quota = nb;
    } else {
      int32_t lo = 0, hi = 1023;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (count_ge(mid) >= need) lo = mid; else hi = mid - 1;
      }
      t = lo;
      quota = need - count_ge(t + 1);
    }
    // selected bin entries, and how many of them precede each list position
    int32_t run = 0, run_eq = 0;
    int32_t sel_ex[PB];
    bool sel[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const uint64_t eqb = __ballot(kl[u] == t);
      const int32_t eq_rank = run_eq + __builtin_popcountll(eqb & lt_mask);
      run_eq += __builtin_popcountll(eqb);
      sel[u] = kl[u] > t || (kl[u] == t && eq_rank < quota);
      const uint64_t bal = __ballot(sel[u]);
      sel_ex[u] = run + __builtin_popcountll(bal & lt_mask);
      run += __builtin_popcountll(bal);
    }
    const int32_t nsel = run;
    // the selected bin entries' indices, compacted in order into the list's front, then
    // one per lane (nsel <= SL_BIN_CAP: up to SL_BIN_CAP / 64 registers)
#pragma unroll
    for (int u = 0; u < PB; ++u)
      if (sel[u]) bl[sel_ex[u]] = e[u] >> 10;
    int32_t sv[PB];
#pragma unroll
    for (int u = 0; u < PB; ++u) sv[u] = lane + WAVE * u < nsel ? bl[lane + WAVE * u] : INT32_MAX;
    int32_t* orow = idx0 + (int64_t)j * k;
    // above-bA entries, 64 at a time: each one's slot is its list position plus the
    // selected bin entries with a lower index, counted with ballots: those below the
    // chunk's first entry at once, the few between its first and last one by one
    for (int p0 = 0; p0 < na; p0 += WAVE) {
      const int p = p0 + lane;
      const int32_t x = p < na ? al[p] : INT32_MAX;
      const int32_t x0 = __builtin_amdgcn_readfirstlane(x);
      const int32_t xl = __builtin_amdgcn_readlane(x, min(WAVE, na - p0) - 1);
      int32_t c = 0;
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        if (WAVE * u >= nsel) break;
        c += __builtin_popcountll(__ballot(sv[u] < x0));
        uint64_t inr = __ballot(sv[u] > x0 && sv[u] < xl);
        while (inr) {
          const int l = __builtin_ctzll(inr);
          inr &= inr - 1;
          c += x > __builtin_amdgcn_readlane(sv[u], l) ? 1 : 0;
        }
      }
      const int32_t pos = p + c;
      if (p < na && pos < k) orow[pos] = x;
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {            // selected bin entries
      if (!sel[u]) continue;
      const int32_t y = e[u] >> 10;
      int lo = 0, hi = na;                     // above-bA entries with a lower index
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

// Two-sweep path over a bitmap (every token of the group sees at most SL_BM_MAX entries):
// the second sweep sets one bit per entry above each token's threshold bin bA, word
// e / 32 of the token's bitmap (bA = -1: every visible entry), and appends the bin's
// entries, unordered, to the token's list.  No order is kept during the sweep: a 64-entry
// block belongs to one wave and one round, so its two words per token are written once,
// with no barrier and no scan.  Then one wave per token resolves the threshold inside bA
// (the bin's largest keys; of the keys equal to the threshold, the lowest indices), sets
// those entries' bits, and writes the row by reading the bitmap in entry order.
template <bool FP4>
__device__ __forceinline__ void sl_bitmap_finalize(
    __amdgpu_buffer_rsrc_t kp, const i32x4& qv, int us, int32_t N, int32_t nround, int32_t nfull, int w,
    int lane, int n, int grp, bool qok, int32_t nv, int32_t bA, int k, int nr, int32_t* sm,
    const int32_t* s_above, int32_t* s_nb, const int32_t* s_nv, int32_t* __restrict__ idx0) {
  int32_t* blist = sm;                                     // [16][SL_BIN_CAP] (index << 10 | key & 1023)
  uint32_t* bm = reinterpret_cast<uint32_t*>(sm + SL_ROWS * SL_BIN_CAP);   // [16][SL_BM_WORDS]
  // word i of token j sits at j * SL_BM_WORDS + (i ^ j): the 16 tokens' words of one block
  // fall in different banks
  const int32_t lim_a = sl_raw_limit(qok ? (bA + 1) << 10 : INT32_MAX);
  const int32_t lim_b = sl_raw_limit(qok ? max(bA, 0) << 10 : INT32_MAX);
  if (threadIdx.x < SL_ROWS) s_nb[threadIdx.x] = 0;
  __syncthreads();
  uint32_t* bmn = bm + n * SL_BM_WORDS;
  int32_t* bln = blist + n * SL_BIN_CAP;
  sl_sweep<FP4>(kp, qv, us, N, nround, nfull, w, lane, [&](auto all, const int32_t (&sc)[4][4], int32_t, int32_t blk) __attribute__((always_inline)) {
    constexpr bool ALL = decltype(all)::value;
    uint32_t ba[4], bb[4];
    // entry e_lane + 16 u + r is visible when 16 u + r < vlim
    const int32_t e_lane = blk * SL_BLOCK + 4 * grp;
    const int32_t vlim = nv - e_lane;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t a = 0, c = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool vis = ALL || 16 * u + r < vlim;
        a |= vis && sc[u][r] >= lim_a ? 1u << r : 0u;
        c |= vis && sc[u][r] >= lim_b ? 1u << r : 0u;
      }
      ba[u] = a;
      bb[u] = c & ~a;
    }
    // the block's two words of this lane's token: entry 16 u + 4 g + r of the block is bit
    // (16 u + 4 g + r) % 32 of word (16 u + 4 g + r) / 32; the token's 4 lane groups OR
    // their nibbles together with two lane swaps
    const int sh = 4 * grp;
    uint32_t w0 = (ba[0] << sh) | (ba[1] << (16 + sh));
    uint32_t w1 = (ba[2] << sh) | (ba[3] << (16 + sh));
    w0 |= (uint32_t)sl_partner16((int32_t)w0);
    w1 |= (uint32_t)sl_partner16((int32_t)w1);
    w0 |= (uint32_t)sl_partner32((int32_t)w0);
    w1 |= (uint32_t)sl_partner32((int32_t)w1);
    // (the sweep runs up to two rounds past the last block, whose words would lie past
    // the bitmap: they hold no visible entry and are not stored)
    if (grp == 0 && 2 * blk < SL_BM_WORDS) {
      bmn[(2 * blk) ^ n] = w0;
      bmn[(2 * blk + 1) ^ n] = w1;
    }
    // entries inside bA (a few per wave and round): appended in any order
    if (__builtin_amdgcn_ballot_w64((bb[0] | bb[1] | bb[2] | bb[3]) != 0)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x4 su = {sc[u][0], sc[u][1], sc[u][2], sc[u][3]};
        uint32_t m = bb[u];
        while (m) {
          const int r = __builtin_ctz(m);
          m &= m - 1;
          const int32_t pos = atomicAdd(&s_nb[n], 1);
          if (pos < SL_BIN_CAP) bln[pos] = ((e_lane + 16 * u + r) << 10) | (score_key(su[r]) & 1023);
        }
      }
    }
  });
  __syncthreads();
  // one wave per token
  for (int j = w; j < nr; j += SL_NW) {
    const int32_t vj = s_nv[j];
    uint32_t* bmj = bm + j * SL_BM_WORDS;
    if (vj > k) {   // wave-uniform: the token has a threshold bin
      const int32_t nb = min(s_nb[j], SL_BIN_CAP);
      const int32_t need = k - s_above[j];   // keys to take from the bin, 1..nb
      const int32_t* bl = blist + j * SL_BIN_CAP;
      constexpr int PB = SL_BIN_CAP / WAVE;
      int32_t e[PB], kl[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const bool ok = lane + WAVE * u < nb;
        e[u] = ok ? bl[lane + WAVE * u] >> 10 : 0;
        kl[u] = ok ? (bl[lane + WAVE * u] & 1023) : -1;   // an empty slot takes no threshold
      }
      // the threshold t: the largest value with at least `need` low key bits >= t (a
      // binary search over the 10 bits, counted by ballots)
      auto count_ge = [&](int32_t v) __attribute__((always_inline)) {
        int32_t c = 0;
#pragma unroll
        for (int u = 0; u < PB; ++u) c += __builtin_popcountll(__ballot(kl[u] >= v));
        return c;
      };
      int32_t lo = 0, hi = 1023;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (count_ge(mid) >= need) lo = mid; else hi = mid - 1;
      }
      const int32_t t = lo;
      const int32_t quota = need - count_ge(t + 1);   // t-valued keys to take, lowest indices
      int32_t n_eq = 0;
#pragma unroll
      for (int u = 0; u < PB; ++u) n_eq += __builtin_popcountll(__ballot(kl[u] == t));
      // a t-valued entry's rank among the t-valued ones by index (the list is unordered):
      // only needed when some of them are left out
      int32_t rank[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) rank[u] = 0;
      if (quota < n_eq) {
#pragma unroll
        for (int v = 0; v < PB; ++v) {
          uint64_t eqb = __ballot(kl[v] == t);
          while (eqb) {
            const int l = __builtin_ctzll(eqb);
            eqb &= eqb - 1;
            const int32_t y = __builtin_amdgcn_readlane(e[v], l);
#pragma unroll
            for (int u = 0; u < PB; ++u) rank[u] += (kl[u] == t && y < e[u]) ? 1 : 0;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (kl[u] > t || (kl[u] == t && rank[u] < quota))
          atomicOr(&bmj[(e[u] >> 5) ^ j], 1u << (e[u] & 31));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the bits are in before the reads below
    }
    // the row: the set bits in entry order, 64 words at a time (lane l takes word
    // c0 + l), so the entries a round of stores writes lie close together in the row
    const int32_t nw = (vj + 31) >> 5;
    int32_t* orow = idx0 + (int64_t)j * k;
    int32_t base = 0;
    for (int32_t c0 = 0; c0 < nw; c0 += WAVE) {
      const int32_t i = c0 + lane;
      uint32_t x = i < nw ? bmj[i ^ j] : 0u;
      const int32_t cnt = __builtin_popcount(x);
      const int32_t incl = wave_incl_scan(cnt);
      int32_t pos = base + incl - cnt;
      base += __builtin_amdgcn_readlane(incl, WAVE - 1);
      while (x) {
        const int bit = __builtin_ctz(x);
        x &= x - 1;
        if (pos < k) orow[pos] = (i << 5) | bit;
        ++pos;
      }
    }
    for (int p = min(base, k) + lane; p < k; p += WAVE) orow[p] = -1;
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
  // entries visible to some token of the group: the sweeps stop there; the rounds
  // below the fewest entries visible to a token of the group need no visibility test
  int32_t mx = nv, mn = qok ? nv : INT32_MAX;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    mx = max(mx, __shfl_xor(mx, d, WAVE));
    mn = min(mn, __shfl_xor(mn, d, WAVE));
  }
  // the same in every wave (each wave's lanes n, n + 16, ... cover the group's tokens)
  const int32_t nfull = __builtin_amdgcn_readfirstlane(mn) / (SL_BLOCK * SL_NW);
  if (lane == 0) s_tot[w] = mx;            // s_tot doubles as scratch here
  __syncthreads();
  int32_t nvmax = 0;
  for (int i = 0; i < SL_NW; ++i) nvmax = max(nvmax, s_tot[i]);
  const bool any_thr = s_flag != 0;
  const int32_t nblk = (nvmax + SL_BLOCK - 1) / SL_BLOCK;
  const int32_t nround = (nblk + SL_NW - 1) / SL_NW;

  constexpr int VB = FP4 ? 32 : 64;        // bytes per indexer vector
  // the sequence's keys (N entries of VB bytes) as a buffer
  const __amdgpu_buffer_rsrc_t kp = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(a.k_idx + e0 * VB), 0, N * VB, BUF_RSRC_WORD3);
  const i32x4 zero4 = {0, 0, 0, 0};
  const i32x4 qv = qok && 16 * grp < VB ? *reinterpret_cast<const i32x4*>(a.q_idx + row * VB + 16 * grp)
                                        : zero4;
  // The E8M0 unit scale of the FP4 MFMAs in one VGPR for the whole kernel (e8m0_unit_vgpr).
  const int us = FP4 ? e8m0_unit_vgpr() : 127;

  if (nvmax > 0 && any_thr) {
    // ---- sweep 1: coarse histograms
    for (int i = t; i < SL_ROWS * HIST_BINS; i += SL_NT) sm[i] = 0;
    __syncthreads();
    int32_t* hc = sm + n * HIST_BINS;
    sl_sweep<FP4>(kp, qv, us, N, nround, nfull, w, lane, [&](auto all, const int32_t (&sc)[4][4], int32_t, int32_t blk) __attribute__((always_inline)) {
      constexpr bool ALL = decltype(all)::value;
      const int32_t vlim = nv - (blk * SL_BLOCK + 4 * grp);   // visible: 16 u + r < vlim
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (thr && (ALL || 16 * u + r < vlim))
            atomicAdd(&hc[(score_key(sc[u][r]) >> 10) ^ n], 1);
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
    if (s_flag && nvmax <= SL_BM_MAX) {
      if (t < nr) s_tot[t] = (int32_t)min(a.q_pos[r0 + q0 + t] / a.c, (int64_t)N);   // visible counts
      sl_bitmap_finalize<FP4>(kp, qv, us, N, nround, nfull, w, lane, n, grp, qok, nv,
                              thr ? s_bin[n] : -1, k, nr, sm, s_above, s_nb, s_tot, idx0);
      e8m0_keep(us);
      return;
    }
    if (s_flag) {
      sl_collect_finalize<FP4>(kp, qv, us, N, nround, nfull, w, lane, n, grp, qok, nv,
                               thr ? s_bin[n] : -1, k, nr, sm, s_tot, s_na, s_nb, idx0);
      e8m0_keep(us);
      return;
    }
    // ---- sweep 2: fine histograms of the threshold bins
    const int32_t bA = s_bin[n];
    for (int i = t; i < SL_ROWS * FINE_BINS; i += SL_NT) sm[i] = 0;
    __syncthreads();
    int32_t* hf = sm + n * FINE_BINS;
    sl_sweep<FP4>(kp, qv, us, N, nround, nfull, w, lane, [&](auto all, const int32_t (&sc)[4][4], int32_t, int32_t blk) __attribute__((always_inline)) {
      constexpr bool ALL = decltype(all)::value;
      const int32_t vlim = nv - (blk * SL_BLOCK + 4 * grp);   // visible: 16 u + r < vlim
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t key = score_key(sc[u][r]);
          if (thr && (ALL || 16 * u + r < vlim) && (key >> 10) == bA)
            atomicAdd(&hf[(key & 1023) ^ n], 1);
        }
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
    // key limits: selected-above is key >= lim_a, T-valued is lim_e <= key < lim_a (a
    // token without a threshold keeps every visible entry); a lane without a token takes none
    const int32_t lim_a = sl_raw_limit(!qok ? INT32_MAX : thr ? T + 1 : 0);
    const int32_t lim_e = sl_raw_limit(!qok ? INT32_MAX : thr ? T : 0);
    sl_sweep<FP4>(kp, qv, us, N, nround, nfull, w, lane, [&](auto all, const int32_t (&sc)[4][4], int32_t rd, int32_t blk) __attribute__((always_inline)) {
      constexpr bool ALL = decltype(all)::value;
      // Counts are packed (T-valued << 16 | above); a round adds at most 1024 to
      // either half.  Within the wave, segment (tile u, lane group g) precedes
      // (u, g') for g < g' and every segment of tiles after u: a scan over the
      // row's 4 lanes (n, n+16, n+32, n+48) per tile.
      uint32_t ba[4], be[4];
      int32_t ex[4];
      int32_t wtot = 0;
      const int32_t e_lane = blk * SL_BLOCK + 4 * grp;   // entry e_lane + 16 u + r
      const int32_t vlim = nv - e_lane;                  // visible when 16 u + r < vlim
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t x_a = 0, x_c = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = ALL || 16 * u + r < vlim;
          x_a |= vis && sc[u][r] >= lim_a ? 1u << r : 0u;
          x_c |= vis && sc[u][r] >= lim_e ? 1u << r : 0u;
        }
        ba[u] = x_a;
        be[u] = x_c & ~x_a;
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
      // 3% of entries are candidates, so each lane walks only its set bits, tile-major
      // (entry order).  The round's offsets of each tile (at most 1088, so 16 bits)
      // are packed two to a word, above-T and T-valued apart.
      const uint32_t mA = ba[0] | ba[1] << 4 | ba[2] << 8 | ba[3] << 12;
      const uint32_t mE = be[0] | be[1] << 4 | be[2] << 8 | be[3] << 12;
      uint32_t oa[2], oe[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t p0 = (uint32_t)(pre + ex[2 * h]), p1 = (uint32_t)(pre + ex[2 * h + 1]);
        oa[h] = (p0 & 0xffff) | (p1 << 16);
        oe[h] = (p0 >> 16) | (p1 & 0xffff0000u);
      }
      uint32_t m = mA | mE;
      while (m) {
        const int bit = __builtin_ctz(m);
        m &= m - 1;
        const int sh = (bit & 4) << 2;
        const bool hi = bit & 8;
        const int32_t ab = a_base + (int32_t)(((hi ? oa[1] : oa[0]) >> sh) & 0xffff) +
                           __builtin_popcount(__builtin_amdgcn_ubfe(mA, bit & 12, bit & 3));
        const int32_t eb = e_base + (int32_t)(((hi ? oe[1] : oe[0]) >> sh) & 0xffff) +
                           __builtin_popcount(__builtin_amdgcn_ubfe(mE, bit & 12, bit & 3));
        const bool isa = (mA >> bit) & 1;
        const int32_t pos = isa ? ab + min(eb, need_eq) : ab + eb;
        if (pos < k && (isa || eb < need_eq)) orow[pos] = e_lane + (bit & 12) * 4 + (bit & 3);
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
  e8m0_keep(us);
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
