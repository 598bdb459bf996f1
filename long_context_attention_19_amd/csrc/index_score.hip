// csa_index_score: int8 indexer scores, exact int32, one query row per grid row.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 item 4: CSA selects entries through an indexer with its
// own Q.K path.  Here query and keys are int8 vectors of width 64 and the score
// is their exact dot product.
//
// Decode streams 64 bytes of key per entry and does 16 int8 MACs per 16 bytes,
// far below the ALU ridge: the kernel is bound by HBM.  Layout of the work:
//   - a work-group owns IS_CHUNK consecutive entries of one sequence of one layer
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

namespace lca {

constexpr int IS_NT = 256;
constexpr int IS_ROUNDS = 8;
constexpr int IS_KEYS_PER_PASS = IS_NT / 4 * IS_ROUNDS;   // 512
constexpr int IS_PASSES = 4;
constexpr int IS_CHUNK = IS_KEYS_PER_PASS * IS_PASSES;     // 2048 entries per work-group

template <bool HIST>
__global__ __launch_bounds__(IS_NT) void index_score_kernel(IndexBatch ib) {
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
      if (HIST && vis && j < N) atomicAdd(&lh[(v + KEY_BIAS) >> 10], 1);
    }
  }
  // the group's scores leave at the end, 16 bytes per thread per store, 8 KiB
  // contiguous; nothing past the sequence's last entry is written
  __syncthreads();
  {
    const int64_t cnt = min((int64_t)IS_CHUNK, N - base);
#pragma unroll
    for (int u = 0; u < IS_CHUNK / (4 * IS_NT); ++u) {
      const int q = 4 * (t + IS_NT * u);
      if (q + 4 <= cnt) {
        *reinterpret_cast<i32x4*>(srow + base + q) = *reinterpret_cast<const i32x4*>(&s_sc[q]);
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

hipError_t launch_index_score(const IndexBatch& ib, int batch, hipStream_t st) {
  if (batch == 0 || ib.max_q == 0 || ib.n == 0) return hipSuccess;
  int chunks = 1;
  bool hist = false;
  for (int l = 0; l < ib.n; ++l) {
    chunks = max(chunks, (ib.layer[l].max_entries + IS_CHUNK - 1) / IS_CHUNK);
    hist = hist || ib.layer[l].hist != nullptr;
  }
  dim3 grid((unsigned)chunks, (unsigned)(batch * ib.max_q), (unsigned)ib.n);
  if (hist)
    hipLaunchKernelGGL(index_score_kernel<true>, grid, dim3(IS_NT), 0, st, ib);
  else
    hipLaunchKernelGGL(index_score_kernel<false>, grid, dim3(IS_NT), 0, st, ib);
  return hipGetLastError();
}

}  // namespace lca
