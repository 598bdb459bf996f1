// Host-side interface between the C ABI (abi.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lca {

// ------------------------------------------------------------ kv_compress
hipError_t launch_kv_compress(const uint16_t* x, const int64_t* tok_off, int batch,
                              int max_tokens, int head_dim, int c, uint16_t* y,
                              const int64_t* ent_off, hipStream_t st);
// mixed rows (head_dim 128): y holds KV8_ROW_BYTES per entry
hipError_t launch_kv_compress_kv8(const uint16_t* x, const int64_t* tok_off, int batch,
                                  int max_tokens, int c, uint8_t* y, const int64_t* ent_off,
                                  hipStream_t st);

// ------------------------------------------------------------ index scores
constexpr int MAX_BATCH_LAYERS = 8;   // layers per batched launch (grid z)

// One layer of an indexer-score launch.  hist != nullptr: also build the top-k's
// coarse radix histogram (hist[rows][2048], accumulated) and zero its fine
// histogram (fine[rows][1024]); all layers of a launch either have it or not.
struct IndexLayer {
  const int8_t* q_idx;
  const int8_t* k_idx;
  const int64_t* ent_off;
  int32_t* scores;
  int64_t ld;
  int32_t* n_vis;
  int32_t* hist;
  int32_t* fine;
  int32_t c;
  int32_t max_entries;
};
struct IndexBatch {
  const int64_t* q_off;
  const int64_t* q_pos;
  int32_t max_q;
  int32_t n;
  int32_t fp4;             // q_idx / k_idx hold packed FP4 (E2M1) codes, 32 bytes per vector
  IndexLayer layer[MAX_BATCH_LAYERS];
};
hipError_t launch_index_score(const IndexBatch& ib, int batch, hipStream_t st);

// Scores and top-k in one pass over the keys, without the scores (16+ query rows
// per sequence).
struct SelectArgs {
  const int8_t* q_idx;
  const int8_t* k_idx;
  const int64_t* ent_off;
  const int64_t* q_off;
  const int64_t* q_pos;
  int32_t* idx;
  int32_t* count;
  int32_t* n_vis;   // may be null
  int32_t c;
  int32_t max_entries;
  int32_t max_q;
  int32_t k;
  int32_t fp4;      // q_idx / k_idx hold packed FP4 codes (32 bytes per vector)
};
constexpr int SELECT_MIN_Q = 16;
hipError_t launch_index_select(const SelectArgs& a, int batch, hipStream_t st);

// ------------------------------------------------------------ decode selection
// Scores and top-k without the score matrix, for decode-sized query batches: each
// work-group of a first launch scores DS_CHUNK entries of one row in LDS and keeps only
// its chunk's candidates (whole coarse bins from the top, about twice the chunk's
// expected share of the top-k); a second launch picks each row's top-k from the
// candidates, exactly, or rescans the row's keys when a chunk dropped an entry that
// could belong to it.
constexpr int DS_NT = 512;            // threads of a chunk work-group
constexpr int DS_CHUNK = 2048;        // entries per work-group
constexpr int DS_MAX_CHUNKS = 2048;   // rows up to 4M entries
constexpr int DS_SEL_NT = 1024;       // threads of a selection work-group (one per row)
constexpr int DS_SEL_VPT = 9;         // candidate slots per thread and selection round (odd:
                                      // a thread's run of LDS words starts on its own bank);
                                      // a round (9216 slots) holds a whole row up to 2^18
                                      // entries at k 2048

// A chunk's candidate budget for a row with nv > k visible entries.  E is the
// chunk's expected share of the top-k, ceil(k * DS_CHUNK / nv); the chunk keeps the
// top coarse bins until `target` entries (E plus six standard deviations of a Poisson
// count, plus 8), and never more than `slot` (target + 16), the chunk's stride in the
// candidate region.  Host and device share this rule.
struct DsBudget {
  int target;
  int slot;
};
constexpr int DS_MIN_SLOT = 31;       // the smallest slot the rule gives (E = 1)
__host__ __device__ inline DsBudget ds_budget(int64_t nv, int k) {
  int64_t e = ((int64_t)k * DS_CHUNK + nv - 1) / (nv > 0 ? nv : 1);
  if (e > DS_CHUNK) e = DS_CHUNK;
  int sq = 0;
  while ((int64_t)sq * sq < e) ++sq;
  int target = (int)e + 6 * sq + 8;
  if (target > DS_CHUNK) target = DS_CHUNK;
  int slot = target + 16;
  if (slot > DS_CHUNK) slot = DS_CHUNK;
  return DsBudget{target, slot};
}
// Candidate slots a row needs for any nv in (k, max_n]: ceil(nv / DS_CHUNK) chunks of
// ds_budget(nv, k).slot slots each; the bound is taken over every chunk count.
size_t ds_cand_slots(int max_n, int k);

struct DsLayer {
  const int8_t* q_idx;   // [rows][64] int8, or [rows][32] packed FP4
  const int8_t* k_idx;   // [ent_off[B]][64] int8, or [.][32] packed FP4
  const int64_t* ent_off;
  int32_t* n_vis;        // [rows] out
  int4* rinfo;           // [batch * max_q] per grid row: (query row or -1, nv, sequence, 0)
  int32_t* dcut;         // [batch * max_q][nch] by grid row: a chunk's cut bin if it dropped
                         // entries, else 0
  int32_t* cand;         // [batch * max_q][cand_slots] by grid row: per chunk `slot` words:
                         // (key << 11 | entry in
                         // chunk) of the kept entries in index order, then 0
  int32_t* idx;          // [rows][k] out
  int32_t* count;        // [rows] out
  int32_t* idx_gy;       // null, or [batch * max_q][k] out: idx by grid row (for the
                         // attention launch that follows, which reads it before it
                         // knows the row)
  int64_t cand_slots;
  int32_t nch;           // chunk stride of dcut
  int32_t c;
  int32_t max_entries;
  int32_t k;
};
struct DsBatch {
  const int64_t* q_off;
  const int64_t* q_pos;
  int32_t max_q;
  int32_t n;
  int32_t fp4;           // q_idx / k_idx hold packed FP4 (E2M1) codes, 32 bytes per vector
  DsLayer layer[MAX_BATCH_LAYERS];
};
size_t ds_ws_bytes(int rows, int max_n, int k);
// carve one layer's workspace: n_vis, rinfo, dcut, cand
void ds_ws_carve(void* ws, int rows, int max_n, int k, DsLayer& L);
hipError_t launch_ds_chunks(const DsBatch& db, int batch, hipStream_t st);   // candidates
hipError_t launch_ds_select(const DsBatch& db, int batch, hipStream_t st);   // the top-k
// The allocation-free form's workspace: a device array of DS_SCRATCH_BYTES, one copy
// per device.  ds_scratch returns the current device's copy (looked up on the first
// call on that device).
constexpr size_t DS_SCRATCH_BYTES = (size_t)8 << 20;
hipError_t ds_scratch(void** ptr);

// ------------------------------------------------------------ top-k
struct TopkWs {
  int32_t* hist;       // [rows][2048] coarse histogram, zero on entry and on exit
  int32_t* fine;       // [rows][1024] fine histogram, zeroed by the histogram pass
  int2* rowstate;      // [rows] (threshold bin, keys above it)
  int32_t* cnt_above;  // [rows][nchunks]
  int32_t* cnt_bin;    // [rows][nchunks]
  int32_t* bin_keys;   // [rows][nchunks][TK_CHUNK] threshold-bin keys of each chunk
  int nchunks;
};
size_t topk_ws_bytes(int rows, int max_n, int k);
size_t topk_hist_region_bytes(int rows);   // the hist + fine prefix of the workspace
TopkWs topk_ws_carve(void* ws, int rows, int max_n, int k);
int topk_max_chunks();
// One layer of a top-k launch (all layers share the row count).
struct TopkLayer {
  const int32_t* scores;
  int64_t ld;
  const int32_t* n_vis;
  int32_t* idx;
  int32_t* count;
  int32_t max_n;
  int32_t k;
  TopkWs w;
};
struct TopkBatch {
  int32_t n;
  TopkLayer layer[MAX_BATCH_LAYERS];
};
hipError_t launch_topk(const TopkBatch& tb, int rows, bool hist_ready, hipStream_t st);

// ------------------------------------------------------------ attention
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int64_t* ent_off;
  const int64_t* q_off;
  const int64_t* q_pos;    // dense only
  const int32_t* idx;      // sparse: [rows][k]; nullptr selects the dense form
  const int32_t* count;    // sparse
  const int32_t* idx_gy;   // sparse, may be null: the same ids by grid row,
                           // [batch * max_q][k], read before the row is known
  int32_t k;
  int32_t ratio;           // dense visibility ratio
  int32_t max_q;
  int32_t heads;
  int32_t splits;
  int32_t max_n;           // bound on a row's entries (k / max_entries): sets the piece size
  float scale_log2;        // scale * log2(e)
  uint16_t* out;
  float* lse;
  float* part_o;           // [batch * max_q][splits][heads][128] by grid row
  float2* part_ml;         // [batch * max_q][splits][heads]  (running max in log2 units, sum)
  int2* part_info;         // [batch * max_q] per row slot: (query row or -1, pieces),
                           // written by the piece-0 work-groups for the combine
  // Sliding-window form (dense, win_pos0 != nullptr): kc / vc / ent_off describe the
  // state buffers, whose first rows sit at absolute positions win_pos0[b]; a row at
  // position p attends the buffer's tokens at positions [p - window, p).  With
  // merge set, the result is merged by log-sum-exp into the out / lse already there
  // (the compressed branch's), one softmax over both key sets.  One piece per row.
  const int64_t* win_pos0;
  int32_t window;
  int32_t merge;
  // Attention sink: per-head logits (natural log) folded into the final result by
  // whichever kernel writes it; nullptr: none.
  const float* sink;
  // kc / vc hold mixed rows of KV8_ROW_BYTES: dims 0..63 FP8 E4M3, dims 64..127 bf16
  int32_t kv8;
};
constexpr int KV8_ROW_BYTES = 192;
// Layers of one attention launch share heads, splits and max_q.
hipError_t launch_attn_sink(uint16_t* out, float* lse, const float* sink, int64_t rows, int heads,
                            hipStream_t st);
struct AttnBatch {
  int32_t n;
  int32_t hpb;             // heads per block (one work-group's heads): 16, 32 or 64
  int32_t head_blocks;     // heads / hpb
  int32_t rows_grid;       // batch * max_q (set at launch)
  int32_t items;           // rows_grid * n * head_blocks (set at launch)
  AttnArgs a[MAX_BATCH_LAYERS];
};
inline AttnBatch attn_batch1(const AttnArgs& a) {
  AttnBatch b{};
  b.n = 1;
  b.hpb = a.heads < 64 ? a.heads : 64;
  b.head_blocks = a.heads / b.hpb;
  b.a[0] = a;
  return b;
}
// entries one sequence may hold for attention (32-bit byte offsets into its rows)
constexpr int ATTN_MAX_SEQ = 1 << 24;
int attn_auto_splits(int max_q);
size_t attn_ws_bytes(int rows, int heads, int splits);
void attn_ws_carve(void* ws, int rows, int heads, int splits, AttnArgs& a);
hipError_t launch_attention(const AttnBatch& ab, int batch, hipStream_t st);

// ------------------------------------------------------------ misc
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace lca
