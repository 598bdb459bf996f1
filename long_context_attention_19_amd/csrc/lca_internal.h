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
  int32_t k;
  int32_t ratio;           // dense visibility ratio
  int32_t max_q;
  int32_t heads;
  int32_t splits;
  int32_t max_n;           // bound on a row's entries (k / max_entries): sets the piece size
  float scale_log2;        // scale * log2(e)
  uint16_t* out;
  float* lse;
  float* part_o;           // [rows][splits][heads][128]
  float2* part_ml;         // [rows][splits][heads]  (running max in log2 units, sum)
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
  int32_t head_blocks;     // ceil(heads / 64)
  AttnArgs a[MAX_BATCH_LAYERS];
};
inline AttnBatch attn_batch1(const AttnArgs& a) {
  AttnBatch b{};
  b.n = 1;
  b.head_blocks = (a.heads + 63) / 64;
  b.a[0] = a;
  return b;
}
// entries one sequence may hold for attention (32-bit byte offsets into its rows)
constexpr int ATTN_MAX_SEQ = 1 << 24;
int attn_auto_splits(int max_q);
size_t attn_ws_bytes(int rows, int heads, int splits);
void attn_ws_carve(void* ws, int rows, int heads, int splits, AttnArgs& a);
hipError_t launch_attention(const AttnBatch& ab, int batch, hipStream_t st);

// Balanced persistent attention over the items (layer, row, 64-head block) of a batch
// of layers: G work-groups take equal runs of the items' stages end to end.
struct AttnPersist {
  int32_t* plan;           // [W + 1] stage offsets of the items, then [W] query rows
  float* part_o;           // [2G][64][128]
  float2* part_ml;         // [2G][64]
  int32_t G;               // persistent work-groups
  int32_t rows;            // rows per layer (batch * max_q)
};
constexpr int ATTN_PS_MAX_ITEMS = 256;   // layers x rows x head blocks per launch
constexpr int ATTN_PS_STAGE = 64;        // entries per stage
constexpr int ATTN_PS_MAX_RUN = 32;      // stages per work-group without re-staging ids
size_t attn_persist_ws_bytes(int G, int items);
void attn_persist_carve(void* ws, int G, int items, AttnPersist& pp);
// true when the batch can take the persistent form: 64-head blocks, few enough
// items, and a stage total (from the host bounds) that keeps runs short
bool attn_persist_fits(const AttnBatch& ab, int rows, int G);
hipError_t launch_attention_persist(const AttnBatch& ab, const AttnPersist& pp, hipStream_t st);

// ------------------------------------------------------------ misc
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace lca
