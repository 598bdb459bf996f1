// Decode-time selection: indexer scores and their top-k without the score matrix.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 item 4 (the CSA indexer has its own Q.K path) and item 2
// (component table: CSA keeps a sparse top-k of the compressed entries).  The result
// is exactly that of csa_index_score followed by csa_topk_select: per query row the
// top min(k, n_vis) entries by (score desc, index asc), ascending, then -1 padding.
//
// A decode row streams 64 bytes of indexer key per entry (32 for FP4) and selects
// k of up to millions of entries.  Writing every score and reading it back costs 4
// bytes per entry and dependent passes over them; instead:
//
//   chunk launch   a work-group per DS_CHUNK entries of a row scores them into LDS,
//                  with a 2048-bin histogram of their keys (key >> 10, the coarse
//                  radix level).  From the top of that histogram it keeps whole bins
//                  until it holds `target` entries, about twice the chunk's expected
//                  share of the top-k (never more than `slot`), and writes its whole
//                  slot region: the kept entries in index order as one word each,
//                  key << 11 | entry within the chunk, then 0 (no key is 0: the lowest
//                  int8 score, -64 * 128 * 127, has key 8192, the lowest FP4 score key
//                  458752).  A group that drops entries records its cut bin.
//   select launch  a work-group per row reads the row's slot regions with coalesced
//                  loads into LDS; each thread then holds 9 consecutive slots in
//                  registers (read at an odd stride, so a thread's run starts on its
//                  own bank; longer rows in rounds) for the passes: the k-th largest
//                  key T among the candidates from the two radix levels (2048 coarse
//                  bins, then 1024 fine bins inside the threshold bin bA), then one
//                  scan of the (above T, equal to T) counts that places the selection
//                  in index order.  Every dropped entry lies below its chunk's cut bin;
//                  when every cut is at or below bA each entry of bin bA and above is a
//                  candidate, so the candidates' top-k is the row's.  Otherwise (a
//                  chunk held more than its budget at or above the threshold bin: many
//                  ties, or a top-k bunched in a few chunks) the work-group rescans the
//                  row's keys and runs the same two radix levels over every score:
//                  slower, same result.
//
// One launch with the selection in the work-group that finishes a row's last chunk
// (an agent-coherent hand-off through a per-row counter) was measured slower: each
// chunk's publish-and-count tail cost 1.5-3 us, more than the launch boundary saved
// (1M CSA decode 46.9 against 42.6 us, the hybrid stack 167.8 against 145.2 us).
//
// Every decision is a function of counts and keys, never of the order in which
// work-groups finish, so results are bitwise reproducible, and a row's result does
// not depend on the other rows of the batch.  Nothing in the workspace carries over
// between calls.
#include <algorithm>
#include <atomic>

#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int DI_NT = DS_NT;
constexpr int DI_NW = DI_NT / WAVE;
constexpr int DI_ROUNDS = 16;                                   // int8: 4 lanes per key
static_assert(DI_NT / 4 * DI_ROUNDS == DS_CHUNK, "int8 rounds cover the chunk");
constexpr int DF_ROUNDS = DS_CHUNK / (DI_NW * 32);              // FP4: 32 keys per wave and round
static_assert(DF_ROUNDS * DI_NW * 32 == DS_CHUNK, "FP4 rounds cover the chunk");
constexpr int DS_VPT = DS_SEL_VPT;
constexpr int DS_RC = DS_SEL_NT * DS_VPT;                        // slots per selection round
static_assert(DS_RC < (1 << 16), "a round's counts fit 16 bits");
static_assert(DS_MAX_CHUNKS % DS_SEL_NT == 0, "cut marks per selection thread");
static_assert(DS_VPT <= DS_MIN_SLOT, "a thread's run of slots crosses at most one chunk boundary");
static_assert(HIST_BINS % DI_NT == 0 && DS_CHUNK % DI_NT == 0, "bins and entries per thread");

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

size_t ds_cand_slots(int max_n, int k) {
  if (max_n <= k) return 0;
  const int nch = (max_n + DS_CHUNK - 1) / DS_CHUNK;
  size_t best = 0;
  for (int n = 1; n <= nch; ++n) {   // the widest slot for n chunks is at the smallest nv
    const int64_t nv = std::max<int64_t>((int64_t)(n - 1) * DS_CHUNK + 1, (int64_t)k + 1);
    if (nv > max_n) break;
    best = std::max(best, (size_t)n * (size_t)ds_budget(nv, k).slot);
  }
  return best;
}

size_t ds_ws_bytes(int rows, int max_n, int k) {
  const size_t nch = (size_t)std::max(1, (max_n + DS_CHUNK - 1) / DS_CHUNK);
  size_t b = align256((size_t)rows * 4);                         // n_vis
  b += align256((size_t)rows * 16);                              // row records
  b += align256((size_t)rows * nch * 4);                         // per-chunk cut marks
  b += align256((size_t)rows * std::max<size_t>(ds_cand_slots(max_n, k), 1) * 4);   // candidates
  return b;
}

void ds_ws_carve(void* ws, int rows, int max_n, int k, DsLayer& L) {
  const int nch = std::max(1, (max_n + DS_CHUNK - 1) / DS_CHUNK);
  const size_t slots = std::max<size_t>(ds_cand_slots(max_n, k), 1);
  char* p = reinterpret_cast<char*>(ws);
  L.n_vis = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * 4);
  L.rinfo = reinterpret_cast<int4*>(p);
  p += align256((size_t)rows * 16);
  L.dcut = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * nch * 4);
  L.cand = reinterpret_cast<int32_t*>(p);
  L.cand_slots = (int64_t)slots;
  L.nch = nch;
}

// the query row of this grid row, or false for a padding row (i beyond the sequence's
// query count)
__device__ __forceinline__ bool ds_row(const int64_t* q_off, int max_q, int64_t& row, int& b) {
  b = blockIdx.y / max_q;
  const int i = blockIdx.y - b * max_q;
  const int64_t r0 = ld_const(q_off + b);
  if (i >= ld_const(q_off + b + 1) - r0) return false;
  row = r0 + i;
  return true;
}

// word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle
constexpr int DS_RSRC_WORD3 = 0x00020000;

// The bin holding the k-th largest of the counts in hist[0 .. NB) (scanned from the
// top) and the total count of the bins above it; s_b[3] gets the histogram's total.
// Thread t owns NB / NT consecutive bins from the top.  Contains __syncthreads():
// call from all threads.
template <int NT, int NB>
__device__ __forceinline__ void ds_threshold(const int32_t* hist, int need, int32_t* s_scan,
                                             int32_t* s_b, int& bin, int& above) {
  constexpr int PER = NB / NT;
  const int t = threadIdx.x;
  int32_t hv[PER];
  int32_t hs = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    hv[e] = hist[NB - 1 - PER * t - e];
    hs += hv[e];
  }
  if (t == 0) {
    s_b[0] = 0;   // defined even when fewer than `need` are counted
    s_b[1] = 0;
  }
  int32_t htot;
  const int32_t hpre = block_excl_scan<NT>(hs, s_scan, &htot);
  if (t == 0) s_b[3] = htot;
  if (hpre < need && hpre + hs >= need) {
    int32_t acc = hpre;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (acc < need && acc + hv[e] >= need) {
        s_b[0] = NB - 1 - PER * t - e;
        s_b[1] = acc;
      }
      acc += hv[e];
    }
  }
  __syncthreads();
  bin = s_b[0];
  above = s_b[1];
  __syncthreads();
}

// An FP4 (E2M1) code's value times two, as an int8 byte: magnitudes 0, 1, 2, 3, 4, 6,
// 8, 12 for codes 0..7, the sign in bit 3 (code 8 is -0).
__device__ __forceinline__ uint32_t e2m1_x2(uint32_t nib) {
  const uint32_t mag = (uint32_t)((0x0C08060403020100ull >> (8 * (nib & 7))) & 0xffu);
  return (nib & 8) ? ((0u - mag) & 0xffu) : mag;
}
// 4 packed bytes (8 codes, element 2i in the low nibble of byte i) -> two words of
// four int8 values each, in element order
__device__ __forceinline__ void e2m1_x2_word(uint32_t w, uint32_t& d0, uint32_t& d1) {
  d0 = e2m1_x2(w & 15) | (e2m1_x2((w >> 4) & 15) << 8) | (e2m1_x2((w >> 8) & 15) << 16) |
       (e2m1_x2((w >> 12) & 15) << 24);
  d1 = e2m1_x2((w >> 16) & 15) | (e2m1_x2((w >> 20) & 15) << 8) |
       (e2m1_x2((w >> 24) & 15) << 16) | (e2m1_x2((w >> 28) & 15) << 24);
}

// The query of a row as 16 words of int8 values (FP4: the doubled code values).
template <bool FP4>
__device__ __forceinline__ void ds_query_words(const int8_t* q, int64_t row, uint32_t (&qd)[16]) {
  if constexpr (!FP4) {
    const i32x4* p = reinterpret_cast<const i32x4*>(q + row * 64);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i32x4 v = p[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) qd[4 * u + e] = (uint32_t)v[e];
    }
  } else {
    const i32x4* p = reinterpret_cast<const i32x4*>(q + row * 32);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const i32x4 v = p[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) e2m1_x2_word((uint32_t)v[e], qd[8 * u + 2 * e], qd[8 * u + 2 * e + 1]);
    }
  }
}

// One entry's score, recomputed from its key (the rescan path): int8 exactly as the
// index pass; FP4 as 64 * sum (2q)(2k) over the doubled code values = 256 * sum q k.
template <bool FP4>
__device__ __forceinline__ int32_t ds_score(const int8_t* kbase, int64_t j, const uint32_t (&qd)[16]) {
  int32_t d = 0;
  if constexpr (!FP4) {
    const i32x4* p = reinterpret_cast<const i32x4*>(kbase + j * 64);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i32x4 v = p[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_sdot4(v[e], (int)qd[4 * u + e], d, false);
    }
    return d;
  } else {
    const i32x4* p = reinterpret_cast<const i32x4*>(kbase + j * 32);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const i32x4 v = p[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t d0, d1;
        e2m1_x2_word((uint32_t)v[e], d0, d1);
        d = __builtin_amdgcn_sdot4((int)d0, (int)qd[8 * u + 2 * e], d, false);
        d = __builtin_amdgcn_sdot4((int)d1, (int)qd[8 * u + 2 * e + 1], d, false);
      }
    }
    return d * 64;
  }
}

// The exact selection over every visible entry's score, recomputed from the keys in
// three sweeps (coarse histogram, fine histogram of the threshold bin, placement in
// index order).  nv > k.  Writes k indices to irow (and to grow unless null).
template <bool FP4>
__device__ void ds_rescan(const int8_t* kbase, const uint32_t (&qd)[16], int64_t nv, int k,
                          int32_t* irow, int32_t* grow, int32_t* s_hist, int32_t* s_scan,
                          int32_t* s_b) {
  constexpr int NT = DS_SEL_NT;
  const int t = threadIdx.x;
  for (int i = t; i < HIST_BINS; i += NT) s_hist[i] = 0;
  __syncthreads();
  for (int64_t j = t; j < nv; j += NT) atomicAdd(&s_hist[score_key(ds_score<FP4>(kbase, j, qd)) >> 10], 1);
  __syncthreads();
  int bA, above;
  ds_threshold<NT, HIST_BINS>(s_hist, k, s_scan, s_b, bA, above);
  for (int i = t; i < FINE_BINS; i += NT) s_hist[i] = 0;
  __syncthreads();
  for (int64_t j = t; j < nv; j += NT) {
    const int key = score_key(ds_score<FP4>(kbase, j, qd));
    if ((key >> 10) == bA) atomicAdd(&s_hist[key & 1023], 1);
  }
  __syncthreads();
  int low_t, gt_in;
  ds_threshold<NT, FINE_BINS>(s_hist, k - above, s_scan, s_b, low_t, gt_in);
  const int T = (bA << 10) | low_t;
  const int need_eq = k - above - gt_in;   // T-valued keys to keep, lowest indices first
  int32_t eq_run = 0, sel_run = 0;
  for (int64_t base = 0; base < nv; base += NT) {
    const int64_t j = base + t;
    const int key = j < nv ? score_key(ds_score<FP4>(kbase, j, qd)) : -1;
    const bool eq = key == T;
    int32_t eq_n;
    const int32_t eq_rank = eq_run + block_excl_scan<NT>(eq ? 1 : 0, s_scan, &eq_n);
    const bool sel = key > T || (eq && eq_rank < need_eq);
    int32_t sel_n;
    const int32_t pos = sel_run + block_excl_scan<NT>(sel ? 1 : 0, s_scan, &sel_n);
    if (sel && pos < k) {
      irow[pos] = (int32_t)j;
      if (grow) grow[pos] = (int32_t)j;
    }
    eq_run += eq_n;
    sel_run += sel_n;
  }
}

// LDS of the two launches' work-groups.
struct DsSmemChunk {
  int32_t lh[HIST_BINS];                          // coarse histogram of the chunk
  __attribute__((aligned(16))) int32_t sc[DS_CHUNK];   // keys of the chunk
  int32_t out[DS_CHUNK];                          // kept slot words, compacted
};
constexpr int DS_MC = DS_RC / 2;                  // candidates at or above the threshold bin
struct DsSmemSelect {
  int32_t hist[HIST_BINS];                        // coarse, then fine histogram
  uint32_t c[DS_RC];                              // one round of candidate slots
  int32_t key[DS_MC];                             // the candidates at or above bin bA, in
  int32_t ent[DS_MC];                             // index order: key and entry
};

// The selection of one row from its candidates (all DS_SEL_NT threads of the work-group).
template <bool FP4>
__device__ void ds_select_row(const DsLayer& L, int gy, DsSmemSelect& sm, int32_t* s_scan,
                              int32_t* s_b) {
  constexpr int NT = DS_SEL_NT;
  constexpr int VPT = DS_VPT;
  constexpr int RC = DS_RC;
  constexpr int DPT = DS_MAX_CHUNKS / NT;         // cut marks per thread
  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1);
  const int k = L.k;
  // The candidate slots and cut marks of grid row gy are where the chunk launch put
  // them: their first round and the marks are loaded before the row record is back
  // (the row's own slot count, known from the record, then masks the rest).
  const int32_t* crow = L.cand + (int64_t)gy * L.cand_slots;

  // A round of slots: coalesced loads, then through LDS thread t holds its VPT
  // consecutive slots in registers (read at an odd stride: no two lanes of a read share
  // a bank); a slot word is key << 11 | entry within its chunk, 0 an empty slot.
  // Threads past the round's end hold empty slots, and their waves skip the passes.
  uint32_t ck[VPT];
  int n_in = 0;
  auto issue = [&](int rd, int vs) __attribute__((always_inline)) {
    n_in = min(RC, vs - rd * RC);
    // a buffer view of the round: loads past its end return 0, an empty slot
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(crow + rd * RC), 0, n_in * 4, DS_RSRC_WORD3);
#pragma unroll
    for (int u = 0; u < VPT; ++u) ck[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (t + NT * u) * 4, 0, 0);
  };
  auto land = [&]() __attribute__((always_inline)) {
    __syncthreads();   // the previous round's slots are no longer read
#pragma unroll
    for (int u = 0; u < VPT; ++u) sm.c[t + NT * u] = ck[u];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < VPT; ++u) ck[u] = VPT * t + u < n_in ? sm.c[VPT * t + u] : 0u;
  };

  // speculative: the first round of the slot region (all of it that one round holds) and
  // every cut mark the layer may have, beside the row record
  issue(0, (int)min((int64_t)RC, L.cand_slots));
  int32_t dc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) dc[e] = L.dcut[(int64_t)gy * L.nch + min(t + NT * e, L.nch - 1)];
  // (row, nv, sequence) from the chunk launch, as scalars: the passes below branch and
  // size their loops on it
  const int* rip = reinterpret_cast<const int*>(L.rinfo + gy);
  const int4 ri = make_int4(ld_const(rip), ld_const(rip + 1), ld_const(rip + 2), 0);
  if (ri.x < 0 || ri.y <= k) return;   // padding, or written by the chunk launch
  const int64_t row = ri.x, nv = ri.y;
  const int b = ri.z;
  if (t == 0) L.count[row] = k;
  int32_t* irow = L.idx + row * k;
  int32_t* grow = L.idx_gy ? L.idx_gy + (int64_t)gy * k : nullptr;
  const int nch = (int)((nv + DS_CHUNK - 1) / DS_CHUNK);
  const DsBudget bud = ds_budget(nv, k);
  const int vs = nch * bud.slot;   // the row's candidate slots
  const int nround = (vs + RC - 1) / RC;
  const bool one = nround == 1;
  n_in = min(RC, vs);   // the row's share of the speculative round: slots past it are not its own

  // the chunks' cut marks: the highest cut bin of a chunk that dropped entries (0: none)
  if (t == 0) s_b[2] = 0;
  int32_t dm = 0;
#pragma unroll
  for (int e = 0; e < DPT; ++e) dm = max(dm, t + NT * e < nch ? dc[e] : 0);
  dm = wave_max(dm);
  for (int i = t; i < HIST_BINS; i += NT) sm.hist[i] = 0;
  if (one)   // the fine histogram of a one-round row, in the (then unused) key list
    for (int i = t; i < FINE_BINS; i += NT) sm.key[i] = 0;
  __syncthreads();
  if (lane == 0 && dm > 0) atomicMax(&s_b[2], dm);
  land();   // round 0, the speculative one

  // coarse histogram of the candidates' keys
  for (int rd = 0; rd < nround; ++rd) {
    if (rd > 0) {
      issue(rd, vs);
      land();
    }
    if (VPT * t < n_in) {
#pragma unroll
      for (int u = 0; u < VPT; ++u)
        if (ck[u]) atomicAdd(&sm.hist[ck[u] >> 21], 1);
    }
  }
  __syncthreads();
  const int dplus = s_b[2];
  int bA, above;
  ds_threshold<NT, HIST_BINS>(sm.hist, k, s_scan, s_b, bA, above);
  const int n_cand = s_b[3];
  const int m = above + sm.hist[bA];   // candidates at or above bin bA
  __syncthreads();
  // Fewer than k candidates, or a chunk cut above the threshold bin: some entry of bin
  // bA or above may have been dropped.  Otherwise every one is a candidate.  (More
  // candidates in bin bA and above than the compacted lists hold: heavy ties.)
  const bool fast = n_cand >= k && dplus <= bA && m <= DS_MC;
  if (fast && one) {
    // A row in one round: each thread's VPT slots stay in registers for the fine
    // histogram of bin bA and for the placement (no compacted list).  Empty slots (0)
    // and threads past the round hold keys below any threshold.
    int32_t* fine = sm.key;
    if (VPT * t < n_in) {
#pragma unroll
      for (int u = 0; u < VPT; ++u)
        if ((int)(ck[u] >> 21) == bA && ck[u]) atomicAdd(&fine[(ck[u] >> 11) & 1023], 1);
    }
    __syncthreads();
    int low_t, gt_in;
    ds_threshold<NT, FINE_BINS>(fine, k - above, s_scan, s_b, low_t, gt_in);
    const int T = (bA << 10) | low_t;
    const int need_eq = k - above - gt_in;   // T-valued keys to keep, lowest indices first
    int32_t ngt = 0, neq = 0;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int key = (int)(ck[u] >> 11);
      ngt += key > T ? 1 : 0;
      neq += key == T ? 1 : 0;
    }
    int32_t tot2;
    const int32_t pre = block_excl_scan<NT>((ngt << 16) | neq, s_scan, &tot2);
    if (ngt + neq) {
      int32_t g = pre >> 16, q = pre & 0xffff;
      // this thread's run of slots crosses at most one chunk boundary, at slot u_next
      const int v0 = VPT * t;
      const int ch0 = v0 / bud.slot;
      const int u_next = (ch0 + 1) * bud.slot - v0;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int key = (int)(ck[u] >> 11);
        const bool gt = key > T;
        const bool eq = key == T;
        const int pos = g + min(q, need_eq);
        if ((gt || (eq && q < need_eq)) && pos < k) {
          const int ent = (ch0 + (u >= u_next ? 1 : 0)) * DS_CHUNK + (int)(ck[u] & 2047);
          irow[pos] = ent;
          if (grow) grow[pos] = ent;
        }
        g += gt ? 1 : 0;
        q += eq ? 1 : 0;
      }
    }
  } else if (fast) {
    // the candidates at or above bin bA, compacted in index order as (key, entry)
    int32_t run = 0;
    for (int rd = 0; rd < nround; ++rd) {
      if (!one) {
        issue(rd, vs);
        land();
      }
      int32_t nk = 0;
#pragma unroll
      for (int u = 0; u < VPT; ++u) nk += (int)(ck[u] >> 21) >= bA && ck[u] ? 1 : 0;
      int32_t tot;
      int32_t off = run + block_excl_scan<NT>(nk, s_scan, &tot);
      if (nk) {
        // this thread's first slot lies in chunk ch0; its run of VPT slots crosses at
        // most one chunk boundary (a slot region holds at least DS_MIN_SLOT words), at
        // slot u_next of the run
        const int v0 = rd * RC + VPT * t;
        const int ch0 = v0 / bud.slot;
        const int u_next = (ch0 + 1) * bud.slot - v0;
#pragma unroll
        for (int u = 0; u < VPT; ++u)
          if ((int)(ck[u] >> 21) >= bA && ck[u]) {
            const int ch = ch0 + (u >= u_next ? 1 : 0);
            sm.key[off] = (int32_t)(ck[u] >> 11);
            sm.ent[off] = ch * DS_CHUNK + (int)(ck[u] & 2047);
            ++off;
          }
      }
      run += tot;
    }
    for (int i = t; i < FINE_BINS; i += NT) sm.hist[i] = 0;
    __syncthreads();
    // thread t takes compacted candidates [IPT t, IPT t + IPT), in index order
    const int ipt = (m + NT - 1) / NT;
    const int i0 = min(ipt * t, m), i1 = min(i0 + ipt, m);
    for (int i = i0; i < i1; ++i)
      if ((sm.key[i] >> 10) == bA) atomicAdd(&sm.hist[sm.key[i] & 1023], 1);
    __syncthreads();
    int low_t, gt_in;
    ds_threshold<NT, FINE_BINS>(sm.hist, k - above, s_scan, s_b, low_t, gt_in);
    const int T = (bA << 10) | low_t;
    const int need_eq = k - above - gt_in;   // T-valued keys to keep, lowest indices first
    // one scan of (above T, equal to T) counts, 16 bits each (m < 2^16): a selected
    // candidate's place is (above-T before it) + min(T-valued before it, need_eq)
    int32_t ngt = 0, neq = 0;
    for (int i = i0; i < i1; ++i) {
      ngt += sm.key[i] > T ? 1 : 0;
      neq += sm.key[i] == T ? 1 : 0;
    }
    int32_t tot2;
    const int32_t pre = block_excl_scan<NT>((ngt << 16) | neq, s_scan, &tot2);
    int32_t g = pre >> 16, q = pre & 0xffff;
    for (int i = i0; i < i1; ++i) {
      const int key = sm.key[i];
      const bool gt = key > T;
      const bool eq = key == T;
      const int pos = g + min(q, need_eq);
      if ((gt || (eq && q < need_eq)) && pos < k) {
        irow[pos] = sm.ent[i];
        if (grow) grow[pos] = sm.ent[i];
      }
      g += gt ? 1 : 0;
      q += eq ? 1 : 0;
    }
  } else {   // uniform: every thread read the same counts and bins
    uint32_t qd[16];
    ds_query_words<FP4>(L.q_idx, row, qd);
    const int8_t* kbase = L.k_idx + L.ent_off[b] * (FP4 ? 32 : 64);
    ds_rescan<FP4>(kbase, qd, nv, k, irow, grow, sm.hist, s_scan, s_b);
  }
}

template <bool FP4>
__global__ __launch_bounds__(DI_NT) void ds_chunk_kernel(DsBatch db) {
  __shared__ DsSmemChunk sm;
  __shared__ int32_t s_scan[DI_NW + 1];
  __shared__ int32_t s_cut;
  const DsLayer& L = db.layer[blockIdx.z];
  const int t = threadIdx.x;
  // The chunk's keys are requested first, over the entries the sequence holds: the
  // row's position, and so its visible count, is two dependent loads further (the
  // query offsets, then the position).  Keys past the visible count are fetched but
  // never counted.
  const int bs = blockIdx.y / db.max_q;
  const int64_t e0 = ld_const(L.ent_off + bs);
  const int64_t N = min(ld_const(L.ent_off + bs + 1) - e0, (int64_t)L.max_entries);
  const int64_t base = (int64_t)blockIdx.x * DS_CHUNK;
  if (blockIdx.x > 0 && base >= N) return;   // no entry of the sequence (chunk 0 writes the row records)
  const int navail = (int)max(min((int64_t)DS_CHUNK, N - base), (int64_t)0);
  constexpr int VB = FP4 ? 32 : 64;          // bytes per key
  constexpr int NR = FP4 ? DF_ROUNDS : DI_ROUNDS;
  // int8: lane t takes the 16-byte piece t % 4 of key t / 4 of each 128-key round;
  // FP4: lane l of wave w takes half l / 32 of key w * 32 + l % 32 of each round
  const int w = __builtin_amdgcn_readfirstlane(t / WAVE);
  const int lane = t & (WAVE - 1);
  const int piece = FP4 ? lane >> 5 : t & 3;
  // a buffer over the chunk's keys: a load past them returns zeros, so the loads carry
  // no branches (a branch per load made the compiler wait for the first ones before
  // issuing the rest)
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(L.k_idx + (e0 + base) * VB), 0, navail * VB, BUF_RSRC_WORD3);
  i32x4 kv[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int jl = FP4 ? u * (DI_NT / WAVE * 32) + w * 32 + (lane & 31) : u * (DI_NT / 4) + (t >> 2);
    kv[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, jl * VB + piece * 16, 0, BUF_NT));
  }
  asm volatile("" ::: "memory");   // the row's loads below stay behind the key requests

  int64_t row;
  int b;
  if (!ds_row(db.q_off, db.max_q, row, b)) {
    if (blockIdx.x == 0 && t == 0) L.rinfo[blockIdx.y] = make_int4(-1, 0, 0, 0);   // padding
    return;
  }
  const int64_t nv = max(min(ld_const(db.q_pos + row) / L.c, N), (int64_t)0);
  const int k = L.k;
  if (blockIdx.x == 0 && t == 0) {
    L.n_vis[row] = (int32_t)nv;
    L.rinfo[blockIdx.y] = make_int4((int)row, (int)nv, b, 0);   // for the select launch
  }
  if (nv <= k) {   // every visible entry is selected: the first work-group writes the row
    if (blockIdx.x == 0) {
      int32_t* irow = L.idx + row * k;
      int32_t* grow = L.idx_gy ? L.idx_gy + (int64_t)blockIdx.y * k : nullptr;
      for (int p = t; p < k; p += DI_NT) {
        irow[p] = p < nv ? p : -1;
        if (grow) grow[p] = p < nv ? p : -1;
      }
      if (t == 0) L.count[row] = (int32_t)nv;
    }
    return;
  }
  if (base >= nv) return;
  const int tot = (int)min((int64_t)DS_CHUNK, nv - base);   // visible entries of the chunk
  // the chunk's candidate budget (a 64-bit division and a square root: worked out while
  // the keys are in flight, not after the scores)
  const DsBudget bud = ds_budget(nv, k);

  // The query through the constant address space: scalar loads, whose wait does not
  // hold the (in-order) key loads issued above.  Each lane keeps its 16-byte piece.
  const i32x4* qc = reinterpret_cast<const i32x4*>(L.q_idx + row * VB);
  i32x4 qv;
  if constexpr (FP4) {
    const i32x4 q0 = ld_const(qc), q1 = ld_const(qc + 1);
    qv = piece ? q1 : q0;
  } else {
    const i32x4 q0 = ld_const(qc), q1 = ld_const(qc + 1), q2 = ld_const(qc + 2), q3 = ld_const(qc + 3);
    qv = piece == 0 ? q0 : piece == 1 ? q1 : piece == 2 ? q2 : q3;
  }

  for (int i = t; i < HIST_BINS; i += DI_NT) sm.lh[i] = 0;
  __syncthreads();

  if constexpr (!FP4) {
    int32_t pd[DI_ROUNDS];
#pragma unroll
    for (int u = 0; u < DI_ROUNDS; ++u) {
      int d = __builtin_amdgcn_sdot4(kv[u][0], qv[0], 0, false);
      d = __builtin_amdgcn_sdot4(kv[u][1], qv[1], d, false);
      d = __builtin_amdgcn_sdot4(kv[u][2], qv[2], d, false);
      pd[u] = __builtin_amdgcn_sdot4(kv[u][3], qv[3], d, false);
    }
    // transpose-reduce over the 4 lanes of a key: lane `piece` ends with the whole
    // score of round 4w + piece
    const bool b0 = piece & 1, b1 = piece & 2;
#pragma unroll
    for (int w4 = 0; w4 < DI_ROUNDS / 4; ++w4) {
      const int p0 = pd[4 * w4], p1 = pd[4 * w4 + 1], p2 = pd[4 * w4 + 2], p3 = pd[4 * w4 + 3];
      const int q0 = (b0 ? p1 : p0) + __shfl_xor(b0 ? p0 : p1, 1, WAVE);
      const int q1 = (b0 ? p3 : p2) + __shfl_xor(b0 ? p2 : p3, 1, WAVE);
      const int32_t v = (b1 ? q1 : q0) + __shfl_xor(b1 ? q0 : q1, 2, WAVE);
      const int jl = (4 * w4 + piece) * (DI_NT / 4) + (t >> 2);
      const int key = score_key(v);
      sm.sc[jl] = key;
      if (jl < tot) atomicAdd(&sm.lh[key >> 10], 1);
    }
  } else {
    // FP4: v_mfma_scale_f32_32x32x64_f8f6f4, the query in every row of A (lane l
    // brings elements 32 (l / 32) .. + 31), 32 keys as the columns of B; row 0 of
    // the product, register 0 of lanes 0..31, holds the 32 scores (exact in fp32)
    constexpr int FP4_E2M1 = 4;
    const int us = e8m0_unit_vgpr();   // the E8M0 unit scale, one VGPR
    const i32x8 qa = {qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
    const f32x16 zero16 = {};
#pragma unroll
    for (int u = 0; u < DF_ROUNDS; ++u) {
      const i32x8 kb = {kv[u][0], kv[u][1], kv[u][2], kv[u][3], 0, 0, 0, 0};
      const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          qa, kb, zero16, FP4_E2M1, FP4_E2M1, 0, us, 0, us);
      if (piece == 0) {
        const int jl = u * (DI_NT / WAVE * 32) + w * 32 + (lane & 31);
        const int key = score_key((int32_t)(acc[0] * 256.0f));
        sm.sc[jl] = key;
        if (jl < tot) atomicAdd(&sm.lh[key >> 10], 1);
      }
    }
    e8m0_keep(us);
  }
  __syncthreads();

  // The cut: keep whole coarse bins from the top until `target` entries; a bin that
  // would take the count past `slot` is left out (then fewer than target are kept).
  // Thread t owns bins 2047 - BPT t .. 2048 - BPT (t + 1), highest first.
  constexpr int BPT = HIST_BINS / DI_NT;
  {
    int32_t hv[BPT];
    int32_t hs = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      hv[e] = sm.lh[HIST_BINS - 1 - BPT * t - e];
      hs += hv[e];
    }
    if (t == 0) s_cut = 0;   // the chunk fits its target: keep everything
    int32_t htot;
    const int32_t hpre = block_excl_scan<DI_NT>(hs, s_scan, &htot);
    if (tot > bud.target && hpre < bud.target && hpre + hs >= bud.target) {
      int32_t acc = hpre;
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        if (acc < bud.target && acc + hv[e] >= bud.target) {
          const int bin = HIST_BINS - 1 - BPT * t - e;
          s_cut = acc + hv[e] <= bud.slot ? bin : bin + 1;
        }
        acc += hv[e];
      }
    }
    __syncthreads();
  }
  const int cut = s_cut;

  // compaction in index order (thread t owns entries EPT t .. EPT t + EPT - 1) into LDS,
  // then the whole slot region leaves in coalesced stores, 0 past the kept ones
  constexpr int EPT = DS_CHUNK / DI_NT;
  static_assert(EPT == 4, "one 16-byte LDS read per thread");
  const i32x4 kk = *reinterpret_cast<const i32x4*>(&sm.sc[EPT * t]);
  int32_t keep = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) keep += (EPT * t + e < tot && (kk[e] >> 10) >= cut) ? 1 : 0;
  int32_t kept;
  int32_t off = block_excl_scan<DI_NT>(keep, s_scan, &kept);
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (EPT * t + e < tot && (kk[e] >> 10) >= cut)
      sm.out[off++] = (int32_t)(((uint32_t)kk[e] << 11) | (uint32_t)(EPT * t + e));
  __syncthreads();
  int32_t* cdst = L.cand + blockIdx.y * L.cand_slots + blockIdx.x * (int64_t)bud.slot;
  for (int i = t; i < bud.slot; i += DI_NT) cdst[i] = i < kept ? sm.out[i] : 0;
  if (t == 0) L.dcut[blockIdx.y * L.nch + blockIdx.x] = kept < tot ? cut : 0;   // >= 1 if dropped
}

// The selection as a kernel of its own: one work-group per row, after the chunk launch.
template <bool FP4>
__global__ __launch_bounds__(DS_SEL_NT) void ds_select_kernel(DsBatch db) {
  __shared__ DsSmemSelect sm;
  __shared__ int32_t s_scan[DS_SEL_NT / WAVE + 1];
  __shared__ int32_t s_b[4];
  const DsLayer& L = db.layer[blockIdx.z];
  ds_select_row<FP4>(L, blockIdx.y, sm, s_scan, s_b);
}

hipError_t launch_ds_chunks(const DsBatch& db, int batch, hipStream_t st) {
  if (batch == 0 || db.max_q == 0 || db.n == 0) return hipSuccess;
  int chunks = 1;
  for (int l = 0; l < db.n; ++l)
    chunks = std::max(chunks, (db.layer[l].max_entries + DS_CHUNK - 1) / DS_CHUNK);
  dim3 grid((unsigned)chunks, (unsigned)(batch * db.max_q), (unsigned)db.n);
  if (db.fp4) hipLaunchKernelGGL(ds_chunk_kernel<true>, grid, dim3(DI_NT), 0, st, db);
  else hipLaunchKernelGGL(ds_chunk_kernel<false>, grid, dim3(DI_NT), 0, st, db);
  return hipGetLastError();
}

hipError_t launch_ds_select(const DsBatch& db, int batch, hipStream_t st) {
  if (batch == 0 || db.max_q == 0 || db.n == 0) return hipSuccess;
  dim3 grid(1u, (unsigned)(batch * db.max_q), (unsigned)db.n);
  if (db.fp4) hipLaunchKernelGGL(ds_select_kernel<true>, grid, dim3(DS_SEL_NT), 0, st, db);
  else hipLaunchKernelGGL(ds_select_kernel<false>, grid, dim3(DS_SEL_NT), 0, st, db);
  return hipGetLastError();
}

// The workspace of the allocation-free selection.  In host code `scratch` names a
// host-side stand-in, never the device copy: host code uses only the address that
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) uint8_t scratch[DS_SCRATCH_BYTES];

constexpr int DS_MAX_DEVICES = 64;

hipError_t ds_scratch(void** ptr) {
  static std::atomic<void*> addr[DS_MAX_DEVICES];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= DS_MAX_DEVICES) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {   // two threads may both look it up: they find the same address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace lca
