// csa_index_score: int8 indexer scores, exact int32, one query row per grid row.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 item 4: CSA selects entries through an indexer with its
// own Q.K path.  Here query and keys are int8 vectors of width 64 and the score
// is their exact dot product.
//
// Decode streams 64 bytes of key per entry and does 16 int8 MACs per 16 bytes,
// far below the ALU ridge: the kernel is bound by HBM.  Layout of the work:
//   - a work-group owns 1024 to 4096 consecutive entries of one sequence of one layer
//     (grid z = layer: the layers of a hybrid stack are scored in one launch);
//   - in each round, lane t loads the 16-byte piece (t % 4) of key (t / 4), so a
//     wave's 128-bit loads cover 1 KiB of contiguous key rows, and IS_ROUNDS
//     such loads are in flight per thread (non-temporal: keys are read once);
//   - v_dot4 (sdot4) on each piece; a transpose-reduce over the 4 lanes of a key
//     (xor-1 then xor-2 exchanges) leaves lane p with the full score of round p
//     of each group of 4 rounds, so each store instruction writes whole 64-byte
//     segments and no lane picks a value by a dynamic index.
// Optionally the first radix level of the top-k (a 2048-bin histogram of the
// score's upper 11 bits) is built in LDS here and flushed with one global atomic
// per non-empty bin, saving the top-k a pass over the scores; the first group of
// each row also zeroes the row's second-level histogram.
#include "lca_device.h"
#include "lca_internal.h"
#include "lca.h"

namespace lca {

constexpr int IS_NT = 256;
constexpr int IS_ROUNDS = 16;
constexpr int IS_KEYS_PER_PASS = IS_NT / 4 * IS_ROUNDS;   // 1024
// Entries per work-group: IS_KEYS_PER_PASS x PASSES (1024, 2048 or 4096).  Many rows
// (IS_SMALL_CHUNK_ROWS and up) take one pass of 1024, all 16 loads issued before the
// first is used: a finer grain than 2048 evens out the ragged ends of the rows across
// the chip, and 16 loads in flight beat two passes of 8 (512 per group measured slower).
// With few rows nearly every resident group works on the same few rows, and each
// flushes its histogram into that row's bins with global atomics: groups then take
// more entries, so that a row has at most about IS_GROUPS_PER_ROW of them.
constexpr int IS_SMALL_CHUNK_ROWS = 32;
constexpr int IS_GROUPS_PER_ROW = 128;

template <bool HIST, int IS_PASSES>
__global__ __launch_bounds__(IS_NT) void index_score_kernel(IndexBatch ib) {
  constexpr int IS_CHUNK = IS_KEYS_PER_PASS * IS_PASSES;
  __shared__ int32_t lh[HIST ? HIST_BINS : 1];
  __shared__ __attribute__((aligned(16))) int32_t s_sc[IS_CHUNK];   // the group's scores
  const IndexLayer& L = ib.layer[blockIdx.z];
  const int8_t* __restrict__ q_idx = L.q_idx;
  const int8_t* __restrict__ k_idx = L.k_idx;
  int32_t* __restrict__ scores = L.scores;
  int32_t* __restrict__ hist = L.hist;
  int32_t* __restrict__ fine = L.fine;
  const int64_t ld = L.ld;
  const int c = L.c;
  const int max_q = ib.max_q;
  const int b = blockIdx.y / max_q;
  const int i = blockIdx.y - b * max_q;
  const int64_t r0 = ib.q_off[b];
  if (i >= ib.q_off[b + 1] - r0) return;
  const int64_t row = r0 + i;
  const int64_t e0 = L.ent_off[b];
  const int64_t N = min(L.ent_off[b + 1] - e0, (int64_t)L.max_entries);
  const int64_t nv = min(ib.q_pos[row] / c, N);
  const int64_t base = (int64_t)blockIdx.x * IS_CHUNK;
  if (blockIdx.x == 0 && threadIdx.x == 0) L.n_vis[row] = (int32_t)nv;
  if (base >= N) return;

  const int t = threadIdx.x;
  const int piece = t & 3;
  if (HIST) {
    if (blockIdx.x == 0)
      for (int k = t; k < FINE_BINS; k += IS_NT) fine[row * FINE_BINS + k] = 0;
    for (int k = t; k < HIST_BINS; k += IS_NT) lh[k] = 0;
    __syncthreads();
  }
  const i32x4 qv = *reinterpret_cast<const i32x4*>(q_idx + row * 64 + piece * 16);
  const i32x4* kp = reinterpret_cast<const i32x4*>(k_idx + e0 * 64);
  int32_t* srow = scores + row * ld;

  for (int pass = 0; pass < IS_PASSES; ++pass) {
    const int64_t pb = base + pass * IS_KEYS_PER_PASS;
    if (pb >= N) break;
    i32x4 kv[IS_ROUNDS];
#pragma unroll
    for (int u = 0; u < IS_ROUNDS; ++u) {
      const int64_t j = pb + u * (IS_NT / 4) + (t >> 2);
      kv[u] = (j < N) ? __builtin_nontemporal_load(kp + j * 4 + piece) : i32x4{0, 0, 0, 0};
    }
    int32_t pd[IS_ROUNDS];
#pragma unroll
    for (int u = 0; u < IS_ROUNDS; ++u) {
      int d = __builtin_amdgcn_sdot4(kv[u][0], qv[0], 0, false);
      d = __builtin_amdgcn_sdot4(kv[u][1], qv[1], d, false);
      d = __builtin_amdgcn_sdot4(kv[u][2], qv[2], d, false);
      pd[u] = __builtin_amdgcn_sdot4(kv[u][3], qv[3], d, false);
    }
    // Transpose-reduce within each group of 4 lanes: after the xor-1 and xor-2
    // steps, lane `piece` holds the full score of round 4w + piece.
    const bool b0 = piece & 1, b1 = piece & 2;
#pragma unroll
    for (int w = 0; w < IS_ROUNDS / 4; ++w) {
      const int p0 = pd[4 * w], p1 = pd[4 * w + 1], p2 = pd[4 * w + 2], p3 = pd[4 * w + 3];
      const int q0 = (b0 ? p1 : p0) + __shfl_xor(b0 ? p0 : p1, 1, WAVE);
      const int q1 = (b0 ? p3 : p2) + __shfl_xor(b0 ? p2 : p3, 1, WAVE);
      const int32_t v = (b1 ? q1 : q0) + __shfl_xor(b1 ? q0 : q1, 2, WAVE);
      const int jl = pass * IS_KEYS_PER_PASS + (4 * w + piece) * (IS_NT / 4) + (t >> 2);
      const int64_t j = base + jl;
      const bool vis = j < nv;
      s_sc[jl] = vis ? v : INT32_MIN;
      if (HIST && vis && j < N) atomicAdd(&lh[score_key(v) >> 10], 1);
    }
  }
  // the group's scores leave at the end, 16 bytes per thread per store, 4 KiB
  // contiguous per store instruction, non-temporal (measured faster for this launch
  // than ordinary stores); nothing past the sequence's last entry is written
  __syncthreads();
  {
    const int64_t cnt = min((int64_t)IS_CHUNK, N - base);
#pragma unroll
    for (int u = 0; u < (IS_CHUNK + 4 * IS_NT - 1) / (4 * IS_NT); ++u) {
      const int q = 4 * (t + IS_NT * u);
      if (q >= IS_CHUNK) break;
      if (q + 4 <= cnt) {
        __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(&s_sc[q]),
                                    reinterpret_cast<i32x4*>(srow + base + q));
      } else {
        for (int e = 0; e < 4; ++e)
          if (q + e < cnt) srow[base + q + e] = s_sc[q + e];
      }
    }
  }
  if (HIST) {
    __syncthreads();
    int32_t* gh = hist + row * HIST_BINS;
    for (int k = t; k < HIST_BINS; k += IS_NT) {
      const int32_t v = lh[k];
      if (v) atomicAdd(gh + k, v);
    }
  }
}

// ---------------------------------------------------------------- FP4 indexer
// The same scores for the FP4 indexer ("DeepSeek-V4 ... Review", section 3-2 item 4:
// the indexer's Q.K path is trained for FP4): query and keys are E2M1 codes, 32
// packed bytes per vector (element 2i in the low nibble of byte i), with one
// power-of-two scale per tensor, which cannot change the ranking and is left out.
// The score is J = 256 * sum q_d k_d: every product of two E2M1 values is a multiple
// of 1/4, so J is an exact integer with |J| <= 589,824 < 2^20.  The unit (a power of two,
// free since the tensor scales are) spreads the scores over the int8 path's key range:
// in units of 1/4 they would fill only a few of the top-k's 1024-wide coarse bins.
//
// The key stream halves (32 B per entry), and the products run on the MFMA in its
// native FP4 form: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 and unit
// scales.  Operand A is the query in every row (lane l brings bytes 16 (l / 32) ..
// + 15, i.e. elements 32 (l / 32) .. + 31), operand B holds 32 keys as columns (lane
// l brings the same elements of key l % 32), so a wave's 128-bit loads cover 32
// consecutive keys = 1 KiB.  Row 0 of the 32 x 32 result sits in register 0 of lanes
// 0..31: lane l gets key l's score.  The sums are exact in fp32 (quarter multiples
// far below 2^24), so the order in which the hardware adds them does not matter.
constexpr int IF_NT = 256;
constexpr int IF_NW = IF_NT / WAVE;
constexpr int IF_ROUNDS = 16;                                   // loads in flight per lane
constexpr int IF_KEYS_PER_PASS = IF_NW * 32 * IF_ROUNDS;         // 2048

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool HIST, int PASSES>
__global__ __launch_bounds__(IF_NT) void index_score_fp4_kernel(IndexBatch ib) {
  constexpr int CHUNK = IF_KEYS_PER_PASS * PASSES;
  constexpr int FP4_E2M1 = 4;   // MFMA operand format code
  __shared__ int32_t lh[HIST ? HIST_BINS : 1];
  __shared__ __attribute__((aligned(16))) int32_t s_sc[CHUNK];
  const IndexLayer& L = ib.layer[blockIdx.z];
  const uint8_t* __restrict__ q_fp4 = reinterpret_cast<const uint8_t*>(L.q_idx);
  const uint8_t* __restrict__ k_fp4 = reinterpret_cast<const uint8_t*>(L.k_idx);
  int32_t* __restrict__ scores = L.scores;
  int32_t* __restrict__ hist = L.hist;
  int32_t* __restrict__ fine = L.fine;
  const int64_t ld = L.ld;
  const int c = L.c;
  const int max_q = ib.max_q;
  const int b = blockIdx.y / max_q;
  const int i = blockIdx.y - b * max_q;
  const int64_t r0 = ib.q_off[b];
  if (i >= ib.q_off[b + 1] - r0) return;
  const int64_t row = r0 + i;
  const int64_t e0 = L.ent_off[b];
  const int64_t N = min(L.ent_off[b + 1] - e0, (int64_t)L.max_entries);
  const int64_t nv = min(ib.q_pos[row] / c, N);
  const int64_t base = (int64_t)blockIdx.x * CHUNK;
  if (blockIdx.x == 0 && threadIdx.x == 0) L.n_vis[row] = (int32_t)nv;
  if (base >= N) return;

  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t / WAVE);
  const int lane = t & (WAVE - 1);
  const int half = lane >> 5;   // which 32 elements of the vector this lane brings
  const int kl = lane & 31;     // which of the wave's 32 keys
  if (HIST) {
    if (blockIdx.x == 0)
      for (int k = t; k < FINE_BINS; k += IF_NT) fine[row * FINE_BINS + k] = 0;
    for (int k = t; k < HIST_BINS; k += IF_NT) lh[k] = 0;
    __syncthreads();
  }
  const i32x4 qv = *reinterpret_cast<const i32x4*>(q_fp4 + row * 32 + half * 16);
  const i32x8 qa = {qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
  const i32x4* kp = reinterpret_cast<const i32x4*>(k_fp4 + e0 * 32);   // 2 pieces per key
  int32_t* srow = scores + row * ld;
  const f32x16 zero16 = {};
  const int us = e8m0_unit_vgpr();   // the E8M0 unit scale, one VGPR for the kernel

  for (int pass = 0; pass < PASSES; ++pass) {
    const int64_t pb = base + pass * IF_KEYS_PER_PASS;
    if (pb >= N) break;
    i32x4 kv[IF_ROUNDS];
#pragma unroll
    for (int u = 0; u < IF_ROUNDS; ++u) {
      const int64_t j = pb + u * (IF_NW * 32) + w * 32 + kl;
      kv[u] = (j < N) ? __builtin_nontemporal_load(kp + j * 2 + half) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < IF_ROUNDS; ++u) {
      const i32x8 kb = {kv[u][0], kv[u][1], kv[u][2], kv[u][3], 0, 0, 0, 0};
      const f32x16 acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          qa, kb, zero16, FP4_E2M1, FP4_E2M1, 0, us, 0, us);
      if (half == 0) {   // row 0 of the product: lane kl holds key kl's score
        const int jl = pass * IF_KEYS_PER_PASS + u * (IF_NW * 32) + w * 32 + kl;
        const int64_t j = base + jl;
        const int32_t v = (int32_t)(acc[0] * 256.0f);   // exact
        const bool vis = j < nv;
        s_sc[jl] = vis ? v : INT32_MIN;
        if (HIST && vis && j < N) atomicAdd(&lh[score_key(v) >> 10], 1);
      }
    }
  }
  e8m0_keep(us);
  __syncthreads();
  {
    const int64_t cnt = min((int64_t)CHUNK, N - base);
#pragma unroll
    for (int u = 0; u < CHUNK / (4 * IF_NT); ++u) {
      const int q = 4 * (t + IF_NT * u);
      if (q + 4 <= cnt) {
        __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(&s_sc[q]),
                                    reinterpret_cast<i32x4*>(srow + base + q));
      } else {
        for (int e = 0; e < 4; ++e)
          if (q + e < cnt) srow[base + q + e] = s_sc[q + e];
      }
    }
  }
  if (HIST) {
    __syncthreads();
    int32_t* gh = hist + row * HIST_BINS;
    for (int k = t; k < HIST_BINS; k += IF_NT) {
      const int32_t v = lh[k];
      if (v) atomicAdd(gh + k, v);
    }
  }
}

static hipError_t launch_index_score_fp4(const IndexBatch& ib, int batch, int max_n, bool hist,
                                         hipStream_t st) {
  int passes = 1;
  if ((int64_t)batch * ib.max_q * ib.n < IS_SMALL_CHUNK_ROWS)
    while (passes < 4 && (int64_t)passes * IF_KEYS_PER_PASS * IS_GROUPS_PER_ROW < max_n) passes *= 2;
  const int chunk = IF_KEYS_PER_PASS * passes;
  int chunks = 1;
  for (int l = 0; l < ib.n; ++l)
    chunks = max(chunks, (ib.layer[l].max_entries + chunk - 1) / chunk);
  dim3 grid((unsigned)chunks, (unsigned)(batch * ib.max_q), (unsigned)ib.n);
#define LCA_IF_LAUNCH(P)                                                                      \
  do {                                                                                        \
    if (hist) hipLaunchKernelGGL((index_score_fp4_kernel<true, P>), grid, dim3(IF_NT), 0, st, ib); \
    else hipLaunchKernelGGL((index_score_fp4_kernel<false, P>), grid, dim3(IF_NT), 0, st, ib); \
  } while (0)
  if (passes == 1) LCA_IF_LAUNCH(1);
  else if (passes == 2) LCA_IF_LAUNCH(2);
  else LCA_IF_LAUNCH(4);
#undef LCA_IF_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------- many query rows
// With 16 or more query tokens per sequence (prefill) the scores are the int8 GEMM
// Q_idx [rows x 64] . K_idx^T [64 x N].  One v_mfma_i32_16x16x64_i8 yields the 16 x 16
// scores of 16 entries (operand A) against 16 query tokens (operand B) over the whole
// d_idx = 64, exactly, in int32.  In both operands lane l supplies row l % 16 of its
// matrix and bytes 16 (l / 16) .. 16 (l / 16) + 15 of that row, so the two operands
// agree on which byte pairs are multiplied; in the result lane l holds entries
// 4 (l / 16) + r, r < 4, of query token l % 16 — the same token whose query it loaded.
//
// A work-group owns 16 query tokens and a range of the entries (all of them when
// the grid has enough row tiles to fill the GPU).  It reads 64 B of keys per entry,
// shared by every row tile and so mostly from L2, and writes 64 B of scores per
// entry: it is bound by the HBM writes.  Those only run at full rate as long runs of
// whole lines, so each round of 8 blocks (512 entries) is staged in LDS and leaves
// as 2 KiB per token, 1 KiB per store instruction.  LDS holds, in 160 KiB:
//   - the 16 tokens' histograms, 2048 bins each, bin b of token j at b ^ j so that
//     tokens hitting the same bin use different banks;
//   - the staging tile, 16 x 512 scores, 16-byte chunk c of token j at c ^ j.
constexpr int IG_NT = 512;                   // 8 waves
constexpr int IG_NW = IG_NT / WAVE;
constexpr int IG_ROWS = 16;                  // query tokens per work-group (MFMA N)
constexpr int IG_BLOCK = 64;                 // entries per wave and round: 4 MFMA tiles
constexpr int IG_ROUND = IG_BLOCK * IG_NW;   // 512 entries per round
constexpr int IG_CHUNKS = IG_ROUND / 4;      // 16-byte chunks per staged token row

// word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle
constexpr int IG_RSRC_WORD3 = 0x00020000;
constexpr int IG_STORE_NT = 2;   // cache-policy operand of a buffer store: non-temporal

__device__ __forceinline__ void ig_lds_barrier() {   // LDS traffic only: no memory fence
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Keys of one 64-entry block: tile u, lane l -> entry blk*64 + 16u + l%16, bytes
// 16 (l/16) ..; entries past N re-read entry N-1 (their scores are dropped).  The
// keys are read by every row tile, so these loads are ordinary (kept in L2) and
// the score stores are the non-temporal ones.
__device__ __forceinline__ void ig_load(i32x4 (&kv)[4], const i32x4* __restrict__ kp, int32_t blk,
                                        int32_t N, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t j = min(blk * IG_BLOCK + 16 * u + (lane & 15), N - 1);
    kv[u] = kp[j * 4 + (lane >> 4)];
  }
}

// One round: this wave scores its block into the staging tile and the histograms,
// then the work-group writes the round's whole 16-byte chunks out, token row by
// token row.  Nothing here branches around a global memory access: on this
// architecture loads and stores share one in-order completion counter, and a store
// under a branch would make the compiler's wait for a later-issued load also wait
// for this round's stores.  So the stores are buffer stores whose range check drops
// what lies past the work-group's last whole chunk (or a whole row past the last
// token, or a round wholly past the range: `live` false); the partial last chunk of
// each row is written after the loop, from the last live round still in LDS.
template <bool HIST>
__device__ __forceinline__ void ig_round(const i32x4 (&kv)[4], const i32x4& qv, int32_t blk,
                                         int32_t rbase, int32_t cap4, int32_t nv, bool live,
                                         int64_t nr, int t, int w, int n, int grp,
                                         int32_t* __restrict__ srow0, int64_t ld,
                                         int32_t* lh, int32_t* st) {
  const i32x4 zero4 = {0, 0, 0, 0};
  i32x4 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kv[u], qv, zero4, 0, 0, 0);
    const int32_t j0 = blk * IG_BLOCK + 16 * u + 4 * grp;   // first of this lane's 4 entries
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool vis = j0 + r < nv;
      o[u][r] = vis ? acc[r] : INT32_MIN;
      if (HIST && vis) atomicAdd(&lh[n * HIST_BINS + ((score_key(acc[r]) >> 10) ^ n)], 1);
    }
  }
  if (live) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = (w * IG_BLOCK + 16 * u + 4 * grp) >> 2;   // chunk within the round
      *reinterpret_cast<i32x4*>(st + n * IG_ROUND + 4 * (c ^ n)) = o[u];
    }
  }
  ig_lds_barrier();
  // wave w writes chunks 64 (w % 2) + lane of token rows w / 2 + 4 v, 1 KiB per store
  constexpr int NV = IG_ROWS * IG_CHUNKS / IG_NT;
  const int lane = t & (WAVE - 1);
  const int c = WAVE * (w & 1) + lane;
  i32x4 ov[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int row = (w >> 1) + 4 * v;
    ov[v] = *reinterpret_cast<const i32x4*>(st + row * IG_ROUND + 4 * (c ^ row));
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int row = (w >> 1) + 4 * v;   // uniform
    const int32_t nrec = (live && row < nr) ? cap4 * 4 : 0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(srow0 + row * ld, 0, nrec, IG_RSRC_WORD3);
    __builtin_amdgcn_raw_buffer_store_b128(ov[v], rs, (rbase + 4 * c) * 4, 0, IG_STORE_NT);
  }
  ig_lds_barrier();
}

template <bool HIST>
__global__ __launch_bounds__(IG_NT) void index_gemm_kernel(IndexBatch ib, int tiles_per_seq,
                                                           int ranges) {
  __shared__ __attribute__((aligned(16))) int32_t lh[HIST ? IG_ROWS * HIST_BINS : 1];
  __shared__ __attribute__((aligned(16))) int32_t st[IG_ROWS * IG_ROUND];
  const IndexLayer& L = ib.layer[blockIdx.z];
  const int b = blockIdx.y / tiles_per_seq;
  const int q0 = (blockIdx.y - b * tiles_per_seq) * IG_ROWS;
  const int64_t r0 = ib.q_off[b];
  const int64_t nrows = ib.q_off[b + 1] - r0;
  if (q0 >= nrows) return;
  const int64_t nr = min((int64_t)IG_ROWS, nrows - q0);
  const int64_t e0 = L.ent_off[b];
  const int32_t N = (int32_t)min(L.ent_off[b + 1] - e0, (int64_t)L.max_entries);
  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(t / WAVE);
  const int n = lane & 15;                 // query token of this lane (tile column)
  const int grp = lane >> 4;               // lane group: entries 4 grp .. 4 grp + 3 of a tile
  const bool qok = n < nr;
  const int64_t row = r0 + q0 + (qok ? n : 0);
  const int32_t nv = qok ? (int32_t)min(ib.q_pos[row] / L.c, (int64_t)N) : 0;
  const int er = blockIdx.x;
  if (er == 0) {
    if (t < nr) {
      const int64_t rr = r0 + q0 + t;
      L.n_vis[rr] = (int32_t)min(ib.q_pos[rr] / L.c, (int64_t)N);
    }
    if (HIST)
      for (int i = t; i < nr * FINE_BINS; i += IG_NT) L.fine[(r0 + q0) * FINE_BINS + i] = 0;
  }
  if (N <= 0) return;
  const int32_t nblk = (N + IG_BLOCK - 1) / IG_BLOCK;
  const int32_t blk0 = (int32_t)((int64_t)nblk * er / ranges);
  const int32_t blk1 = (int32_t)((int64_t)nblk * (er + 1) / ranges);
  if (blk0 >= blk1) return;
  const int32_t cap = min(N, blk1 * IG_BLOCK);   // this work-group writes entries < cap
  const int32_t cap4 = cap & ~3;                 // ... the whole chunks of them in the loop
  const int32_t nround = (blk1 - blk0 + IG_NW - 1) / IG_NW;

  const i32x4* kp = reinterpret_cast<const i32x4*>(L.k_idx + e0 * 64);
  const i32x4 zero4 = {0, 0, 0, 0};
  const i32x4 qv = qok ? *reinterpret_cast<const i32x4*>(L.q_idx + row * 64 + 16 * grp) : zero4;
  int32_t* srow0 = L.scores + (r0 + q0) * L.ld;
  // Three key buffers: each round's block is loaded two rounds ahead, before the
  // stores of the round in between.
  i32x4 ka[4], kb[4], kc[4];
  ig_load(ka, kp, blk0 + w, N, lane);
  ig_load(kb, kp, blk0 + IG_NW + w, N, lane);
  if (HIST) {
    for (int i = t; i < IG_ROWS * HIST_BINS; i += IG_NT) lh[i] = 0;
    __syncthreads();
  }
  auto round = [&](const i32x4 (&kv)[4], int32_t rd) __attribute__((always_inline)) {
    const int32_t bb = blk0 + rd * IG_NW;
    ig_round<HIST>(kv, qv, bb + w, bb * IG_BLOCK, cap4, blk1 > bb + w ? nv : 0, rd < nround,
                   nr, t, w, n, grp, srow0, L.ld, lh, st);
  };
  for (int32_t rd = 0; rd < nround; rd += 3) {
    ig_load(kc, kp, blk0 + (rd + 2) * IG_NW + w, N, lane);
    round(ka, rd);
    ig_load(ka, kp, blk0 + (rd + 3) * IG_NW + w, N, lane);
    round(kb, rd + 1);
    ig_load(kb, kp, blk0 + (rd + 4) * IG_NW + w, N, lane);
    round(kc, rd + 2);
  }
  // the partial last chunk of each row (cap not a multiple of 4), from the staging
  // tile, which still holds the last live round
  if (cap4 < cap && t < 4 * nr) {
    const int j = t >> 2, e = t & 3;
    if (cap4 + e < cap) {
      const int32_t rl = (blk0 + (nround - 1) * IG_NW) * IG_BLOCK;   // the last round's base
      const int cc = (cap4 - rl) >> 2;
      srow0[j * L.ld + cap4 + e] = st[j * IG_ROUND + 4 * (cc ^ j) + e];
    }
  }
  if (HIST) {
    __syncthreads();
    int32_t* gh = L.hist + (r0 + q0) * HIST_BINS;
    if (ranges == 1) {   // the work-group saw every entry of its rows: plain stores
      for (int i = t; i < nr * HIST_BINS; i += IG_NT) {
        const int j = i / HIST_BINS, bin = i % HIST_BINS;
        gh[i] = lh[j * HIST_BINS + (bin ^ j)];
      }
    } else {
      for (int i = t; i < nr * HIST_BINS; i += IG_NT) {
        const int j = i / HIST_BINS, bin = i % HIST_BINS;
        const int32_t v = lh[j * HIST_BINS + (bin ^ j)];
        if (v) atomicAdd(gh + i, v);
      }
    }
  }
}

hipError_t launch_index_score(const IndexBatch& ib, int batch, hipStream_t st) {
  if (batch == 0 || ib.max_q == 0 || ib.n == 0) return hipSuccess;
  int max_n = 1;
  bool hist = false;
  for (int l = 0; l < ib.n; ++l) {
    max_n = max(max_n, ib.layer[l].max_entries);
    hist = hist || ib.layer[l].hist != nullptr;
  }
  if (ib.fp4) return launch_index_score_fp4(ib, batch, max_n, hist, st);
  if (ib.max_q >= IG_ROWS) {
    // enough query tokens per sequence for 16-wide MFMA tiles; split the entries
    // only as far as needed to give every CU a work-group
    const int tiles = (ib.max_q + IG_ROWS - 1) / IG_ROWS;
    const int64_t row_tiles = (int64_t)batch * tiles * ib.n;
    const int64_t nblk = (max_n + IG_BLOCK - 1) / IG_BLOCK;
    const int ranges = (int)std::max<int64_t>(1, std::min<int64_t>(
        nblk / (4 * IG_NW), (lca_device_cu_count() + row_tiles - 1) / row_tiles));
    dim3 grid((unsigned)ranges, (unsigned)(batch * tiles), (unsigned)ib.n);
    if (hist)
      hipLaunchKernelGGL(index_gemm_kernel<true>, grid, dim3(IG_NT), 0, st, ib, tiles, ranges);
    else
      hipLaunchKernelGGL(index_gemm_kernel<false>, grid, dim3(IG_NT), 0, st, ib, tiles, ranges);
    return hipGetLastError();
  }
  int passes = 1;
  if ((int64_t)batch * ib.max_q * ib.n < IS_SMALL_CHUNK_ROWS) {
    passes = 1;
    while (passes < 4 && (int64_t)passes * IS_KEYS_PER_PASS * IS_GROUPS_PER_ROW < max_n) passes *= 2;
  }
  const int chunk = IS_KEYS_PER_PASS * passes;
  int chunks = 1;
  for (int l = 0; l < ib.n; ++l)
    chunks = max(chunks, (ib.layer[l].max_entries + chunk - 1) / chunk);
  dim3 grid((unsigned)chunks, (unsigned)(batch * ib.max_q), (unsigned)ib.n);
#define LCA_IS_LAUNCH(P)                                                                  \
  do {                                                                                    \
    if (hist) hipLaunchKernelGGL((index_score_kernel<true, P>), grid, dim3(IS_NT), 0, st, ib); \
    else hipLaunchKernelGGL((index_score_kernel<false, P>), grid, dim3(IS_NT), 0, st, ib); \
  } while (0)
  if (passes == 1) LCA_IS_LAUNCH(1);
  else if (passes == 2) LCA_IS_LAUNCH(2);
  else LCA_IS_LAUNCH(4);
#undef LCA_IS_LAUNCH
  return hipGetLastError();
}

}  // namespace lca
