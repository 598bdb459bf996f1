// The C ABI declared in include/lca.h: argument validation, workspace carving
// and kernel enqueue.  No call allocates or synchronises; validation happens
// before any enqueue so a rejected call has no effect.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "lca.h"
#include "lca_internal.h"

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t ok() {
  g_err.clear();
  return LCA_OK;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool heads_supported(int32_t heads) {
  if (heads <= 0 || heads % 16) return false;
  if (heads < 64) return heads == 16 || heads == 32;
  return heads % 64 == 0;
}

constexpr int kTopkChunk = 4096;

// Phase-timing events of the hybrid step, created once per device on first use and
// never destroyed: [0..1] scores, [1..2] top-k, [3..4] attention.
constexpr int kMaxDevices = 64;
struct HybridTiming {
  hipEvent_t tev[5];
  bool timing = false;
  int index_reps = 1;     // launches of the index pass between events 0 and 1
  bool timed = false;     // a step recorded tev since timing was enabled
  bool has_csa = false;
  bool ready = false;
};
std::mutex g_timing_mu;
HybridTiming g_timing[kMaxDevices];

HybridTiming* hybrid_timing() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  HybridTiming& ht = g_timing[dev];
  if (!ht.ready) {
    for (int i = 0; i < 5; ++i)
      if (hipEventCreate(&ht.tev[i]) != hipSuccess) return nullptr;
    ht.ready = true;
  }
  return &ht;
}

// Piece size of the hybrid step's attention: a row's entries are cut into pieces of
// this many entries (one work-group each), merged in piece order.  It depends on the
// step's layer and query counts only, never on the batch, the layer's kind or the
// cache lengths, so a sequence's result is the same alone or inside any batch.  The
// layers of one launch share the chip, so with more layers a row takes fewer, longer
// pieces (fewer partials): kPieceRefEntries / splits entries, splits = the per-row
// split count of a single layer divided by kLayerWeight per layer.
constexpr int kLayerWeight = 2;
constexpr int kPieceRefEntries = 2048;
int hybrid_splits(int n_layers, int max_q) {
  const int base = lca::attn_auto_splits(max_q);
  const int conc = std::min(std::max(n_layers, 1) * kLayerWeight, 32);
  return std::max(1, base / conc);
}
int hybrid_piece(int n_layers, int max_q) {
  const int sp = hybrid_splits(n_layers, max_q);
  const int want = (kPieceRefEntries + sp - 1) / sp;
  return std::max(64, (want + 63) / 64 * 64);   // a multiple of every stage size
}
// Pieces of the layer's longest row (its bound: top-k, or max_entries): the grid and the
// partial workspace.
int hybrid_layer_splits(const lca_layer& L, int piece) {
  const int bound = L.kind == LCA_LAYER_CSA ? std::max(L.topk, 1) : std::max(L.max_entries, 1);
  return std::max(1, (bound + piece - 1) / piece);
}

// Attention launches of the hybrid step: up to 8 layers each, one row format per
// launch, HCA layers first (their rows hold the most pieces, so their work-groups are
// dispatched first).
std::vector<std::vector<int>> attn_groups(const lca_layer* layers, int n_layers) {
  std::vector<int> order;
  for (int kind : {LCA_LAYER_HCA, LCA_LAYER_CSA})
    for (int l = 0; l < n_layers; ++l)
      if (layers[l].kind == kind) order.push_back(l);
  std::vector<std::vector<int>> groups;
  for (int f = 0; f < 2; ++f) {
    std::vector<int> cur;
    for (int l : order) {
      if ((layers[l].kv_format == LCA_KV_MIXED ? 1 : 0) != f) continue;
      cur.push_back(l);
      if ((int)cur.size() == lca::MAX_BATCH_LAYERS) {
        groups.push_back(cur);
        cur.clear();
      }
    }
    if (!cur.empty()) groups.push_back(cur);
  }
  return groups;
}

// A CSA layer of the hybrid step: the selection's workspace, the selected ids by grid
// row (read by the attention launch before it knows the row), the attention partials.
size_t csa_layer_bytes(int rows, int max_entries, int topk, int heads, int splits) {
  return lca::ds_ws_bytes(rows, max_entries, topk) + lca::align256((size_t)rows * topk * 4) +
         lca::attn_ws_bytes(rows, heads, splits);
}

}  // namespace

extern "C" {

int32_t lca_abi_version(void) { return LCA_ABI_VERSION; }

const char* lca_last_error(void) { return g_err.c_str(); }

int32_t lca_device_cu_count(void) {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cu;
}

int32_t lca_workspace_reset(void* ws, size_t ws_bytes, void* stream) {
  if (ws_bytes == 0) return ok();
  if (!ws) return fail(LCA_ERR_NULL, "workspace_reset: ws is NULL");
  if (!al16(ws)) return fail(LCA_ERR_ALIGN, "workspace_reset: ws not 16-byte aligned");
  return hip_status(lca::launch_fill_zero(ws, ws_bytes, (hipStream_t)stream), "workspace_reset");
}

// ------------------------------------------------------------------ kv_compress
int32_t lca_kv_compress(const lca_bf16* x, const int64_t* tok_off, int32_t batch,
                        int32_t max_tokens, int32_t head_dim, int32_t c, lca_bf16* y,
                        const int64_t* ent_off, void* stream) {
  if (batch < 0 || max_tokens < 0) return fail(LCA_ERR_SHAPE, "kv_compress: negative batch or max_tokens");
  if (head_dim <= 0 || head_dim % 8) return fail(LCA_ERR_UNSUPPORTED, "kv_compress: head_dim %d not a positive multiple of 8", head_dim);
  if (c < 1 || c > 4096) return fail(LCA_ERR_SHAPE, "kv_compress: ratio c=%d outside 1..4096", c);
  if (batch == 0 || max_tokens / c == 0) return ok();
  if (!x || !tok_off || !y || !ent_off) return fail(LCA_ERR_NULL, "kv_compress: NULL pointer");
  if (!al16(x) || !al16(y)) return fail(LCA_ERR_ALIGN, "kv_compress: x / y not 16-byte aligned");
  return hip_status(lca::launch_kv_compress(x, tok_off, batch, max_tokens, head_dim, c, y, ent_off,
                                            (hipStream_t)stream),
                    "kv_compress launch");
}

int32_t lca_kv_compress_kv8(const lca_bf16* x, const int64_t* tok_off, int32_t batch,
                            int32_t max_tokens, int32_t c, uint8_t* y, const int64_t* ent_off,
                            void* stream) {
  if (batch < 0 || max_tokens < 0) return fail(LCA_ERR_SHAPE, "kv_compress_kv8: negative batch or max_tokens");
  if (c < 1 || c > 4096) return fail(LCA_ERR_SHAPE, "kv_compress_kv8: ratio c=%d outside 1..4096", c);
  if (batch == 0 || max_tokens / c == 0) return ok();
  if (!x || !tok_off || !y || !ent_off) return fail(LCA_ERR_NULL, "kv_compress_kv8: NULL pointer");
  if (!al16(x) || !al16(y)) return fail(LCA_ERR_ALIGN, "kv_compress_kv8: x / y not 16-byte aligned");
  return hip_status(lca::launch_kv_compress_kv8(x, tok_off, batch, max_tokens, c, y, ent_off,
                                                (hipStream_t)stream),
                    "kv_compress_kv8 launch");
}

// ------------------------------------------------------------------ index scores
static int32_t index_score_impl(const int8_t* q_idx, const int64_t* q_off, const int64_t* q_pos,
                            const int8_t* k_idx, const int64_t* ent_off, int32_t batch,
                            int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                            int32_t* scores, int64_t ld_scores, int32_t* n_vis, void* ws,
                            size_t ws_bytes, void* stream, bool fp4) {
  if (d_idx != 64) return fail(LCA_ERR_UNSUPPORTED, "csa_index_score: d_idx=%d (only 64)", d_idx);
  if (batch < 0 || max_q < 0 || max_entries < 0) return fail(LCA_ERR_SHAPE, "csa_index_score: negative size");
  if (c < 1) return fail(LCA_ERR_SHAPE, "csa_index_score: ratio c=%d < 1", c);
  if (ld_scores < max_entries || ld_scores % 4) return fail(LCA_ERR_SHAPE, "csa_index_score: ld_scores=%lld must be >= max_entries and a multiple of 4", (long long)ld_scores);
  if (batch == 0 || max_q == 0) return ok();
  if ((int64_t)batch * max_q > (1 << 30)) return fail(LCA_ERR_SHAPE, "csa_index_score: too many rows");
  if (!q_idx || !q_off || !q_pos || !k_idx || !ent_off || !scores || !n_vis) return fail(LCA_ERR_NULL, "csa_index_score: NULL pointer");
  if (!al16(q_idx) || !al16(k_idx) || !al16(scores)) return fail(LCA_ERR_ALIGN, "csa_index_score: q_idx / k_idx / scores not 16-byte aligned");
  lca::IndexBatch ib{};
  ib.q_off = q_off;
  ib.q_pos = q_pos;
  ib.max_q = max_q;
  ib.n = 1;
  ib.fp4 = fp4 ? 1 : 0;
  ib.layer[0] = lca::IndexLayer{q_idx, k_idx, ent_off, scores, ld_scores, n_vis, nullptr, nullptr,
                                c, max_entries};
  if (ws) {
    const int rows = batch * max_q;
    const size_t need = lca::topk_hist_region_bytes(rows);
    if (ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "csa_index_score: ws_bytes %zu < %zu", ws_bytes, need);
    if (!al16(ws)) return fail(LCA_ERR_ALIGN, "csa_index_score: ws not 16-byte aligned");
    lca::TopkWs w = lca::topk_ws_carve(ws, rows, 0, 1);   // the histograms lead the workspace
    ib.layer[0].hist = w.hist;
    ib.layer[0].fine = w.fine;
  }
  return hip_status(lca::launch_index_score(ib, batch, (hipStream_t)stream), "csa_index_score launch");
}

int32_t lca_csa_index_score(const int8_t* q_idx, const int64_t* q_off, const int64_t* q_pos,
                            const int8_t* k_idx, const int64_t* ent_off, int32_t batch,
                            int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                            int32_t* scores, int64_t ld_scores, int32_t* n_vis, void* ws,
                            size_t ws_bytes, void* stream) {
  return index_score_impl(q_idx, q_off, q_pos, k_idx, ent_off, batch, max_q, max_entries, d_idx, c,
                          scores, ld_scores, n_vis, ws, ws_bytes, stream, false);
}

int32_t lca_csa_index_score_fp4(const uint8_t* q_fp4, const int64_t* q_off, const int64_t* q_pos,
                                const uint8_t* k_fp4, const int64_t* ent_off, int32_t batch,
                                int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                                int32_t* scores, int64_t ld_scores, int32_t* n_vis, void* ws,
                                size_t ws_bytes, void* stream) {
  return index_score_impl(reinterpret_cast<const int8_t*>(q_fp4), q_off, q_pos,
                          reinterpret_cast<const int8_t*>(k_fp4), ent_off, batch, max_q,
                          max_entries, d_idx, c, scores, ld_scores, n_vis, ws, ws_bytes, stream,
                          true);
}

// ------------------------------------------------------------------ fused scores + top-k
size_t lca_csa_index_select_workspace_bytes(int32_t batch, int32_t max_q, int32_t max_entries,
                                            int32_t k) {
  if (batch <= 0 || max_q <= 0 || max_entries < 0 || k <= 0) return 0;
  if (max_q >= lca::SELECT_MIN_Q) return 0;   // the prefill form needs no workspace
  return lca::ds_ws_bytes(batch * max_q, max_entries, k);
}

static int32_t index_select_impl(const int8_t* q_idx, const int64_t* q_off, const int64_t* q_pos,
                                 const int8_t* k_idx, const int64_t* ent_off, int32_t batch,
                                 int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                                 int32_t k, int32_t* idx, int32_t* count, int32_t* n_vis,
                                 void* ws, size_t ws_bytes, void* stream, bool fp4,
                                 bool noalloc = false) {
  const char* name = noalloc ? "csa_index_select_noalloc"
                     : fp4   ? "csa_index_select_fp4"
                             : "csa_index_select";
  if (d_idx != 64) return fail(LCA_ERR_UNSUPPORTED, "%s: d_idx=%d (only 64)", name, d_idx);
  if (batch < 0 || max_q < 0 || max_entries < 0) return fail(LCA_ERR_SHAPE, "%s: negative size", name);
  if (c < 1) return fail(LCA_ERR_SHAPE, "%s: ratio c=%d < 1", name, c);
  if (k <= 0) return fail(LCA_ERR_SHAPE, "%s: k=%d must be positive", name, k);
  if (batch == 0 || max_q == 0) return ok();
  if ((int64_t)batch * max_q > (1 << 30)) return fail(LCA_ERR_SHAPE, "%s: too many rows", name);
  if ((int64_t)batch * max_q * k > ((int64_t)1 << 40)) return fail(LCA_ERR_SHAPE, "%s: output too large", name);
  if (!q_idx || !q_off || !q_pos || !k_idx || !ent_off || !idx || !count) return fail(LCA_ERR_NULL, "%s: NULL pointer", name);
  if (!al16(q_idx) || !al16(k_idx)) return fail(LCA_ERR_ALIGN, "%s: q_idx / k_idx not 16-byte aligned", name);
  if (max_q >= lca::SELECT_MIN_Q) {
    lca::SelectArgs a{q_idx, k_idx, ent_off, q_off, q_pos, idx, count, n_vis, c, max_entries,
                      max_q, k, fp4 ? 1 : 0};
    return hip_status(lca::launch_index_select(a, batch, (hipStream_t)stream), name);
  }
  // decode-sized batches: the candidate path
  if ((int64_t)max_entries > (int64_t)lca::DS_MAX_CHUNKS * lca::DS_CHUNK) return fail(LCA_ERR_UNSUPPORTED, "%s: max_entries=%d above %d", name, max_entries, lca::DS_MAX_CHUNKS * lca::DS_CHUNK);
  const int rows = batch * max_q;
  const size_t need = lca::ds_ws_bytes(rows, max_entries, k);
  if (noalloc) {
    if (need > lca::DS_SCRATCH_BYTES) return fail(LCA_ERR_WORKSPACE, "%s: the batch needs %zu bytes of workspace, above the %zu-byte scratch", name, need, lca::DS_SCRATCH_BYTES);
    const hipError_t e = lca::ds_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, name);
    ws_bytes = lca::DS_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "%s: ws_bytes %zu < %zu", name, ws_bytes, need);
  if (!al16(ws)) return fail(LCA_ERR_ALIGN, "%s: ws not 16-byte aligned", name);
  lca::DsBatch db{};
  db.q_off = q_off;
  db.q_pos = q_pos;
  db.max_q = max_q;
  db.n = 1;
  db.fp4 = fp4 ? 1 : 0;
  lca::DsLayer& L = db.layer[0];
  L.q_idx = q_idx;
  L.k_idx = k_idx;
  L.ent_off = ent_off;
  L.idx = idx;
  L.count = count;
  L.c = c;
  L.max_entries = max_entries;
  L.k = k;
  lca::ds_ws_carve(ws, rows, max_entries, k, L);
  if (n_vis) L.n_vis = n_vis;
  hipError_t e = lca::launch_ds_chunks(db, batch, (hipStream_t)stream);
  if (e == hipSuccess) e = lca::launch_ds_select(db, batch, (hipStream_t)stream);
  return hip_status(e, name);
}

int32_t lca_csa_index_select(const int8_t* q_idx, const int64_t* q_off, const int64_t* q_pos,
                             const int8_t* k_idx, const int64_t* ent_off, int32_t batch,
                             int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                             int32_t k, int32_t* idx, int32_t* count, int32_t* n_vis, void* ws,
                             size_t ws_bytes, void* stream) {
  return index_select_impl(q_idx, q_off, q_pos, k_idx, ent_off, batch, max_q, max_entries, d_idx,
                           c, k, idx, count, n_vis, ws, ws_bytes, stream, false);
}

int32_t lca_csa_index_select_noalloc(const int8_t* q_idx, const int64_t* q_off,
                                     const int64_t* q_pos, const int8_t* k_idx,
                                     const int64_t* ent_off, int32_t batch, int32_t max_q,
                                     int32_t max_entries, int32_t d_idx, int32_t c, int32_t k,
                                     int32_t* idx, int32_t* count, int32_t* n_vis,
                                     void* stream) {
  static_assert(LCA_INDEX_SELECT_SCRATCH_BYTES == lca::DS_SCRATCH_BYTES, "scratch size");
  return index_select_impl(q_idx, q_off, q_pos, k_idx, ent_off, batch, max_q, max_entries, d_idx,
                           c, k, idx, count, n_vis, nullptr, 0, stream, false, true);
}

int32_t lca_csa_index_select_fp4(const uint8_t* q_fp4, const int64_t* q_off, const int64_t* q_pos,
                                 const uint8_t* k_fp4, const int64_t* ent_off, int32_t batch,
                                 int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                                 int32_t k, int32_t* idx, int32_t* count, int32_t* n_vis,
                                 void* ws, size_t ws_bytes, void* stream) {
  return index_select_impl(reinterpret_cast<const int8_t*>(q_fp4), q_off, q_pos,
                           reinterpret_cast<const int8_t*>(k_fp4), ent_off, batch, max_q,
                           max_entries, d_idx, c, k, idx, count, n_vis, ws, ws_bytes, stream,
                           true);
}

// ------------------------------------------------------------------ top-k
size_t lca_csa_topk_workspace_bytes(int32_t rows, int32_t max_n, int32_t k) {
  if (rows <= 0 || max_n < 0 || k <= 0) return 0;
  return lca::topk_ws_bytes(rows, max_n, k);
}

int32_t lca_csa_topk_select(const int32_t* scores, int64_t ld_scores, int32_t rows,
                            int32_t max_n, const int32_t* n_vis, int32_t k, int32_t* idx,
                            int32_t* count, void* ws, size_t ws_bytes, uint32_t flags,
                            void* stream) {
  if (rows < 0 || max_n < 0) return fail(LCA_ERR_SHAPE, "csa_topk_select: negative size");
  if (k <= 0) return fail(LCA_ERR_SHAPE, "csa_topk_select: k=%d must be positive", k);
  if ((int64_t)max_n > (int64_t)lca::topk_max_chunks() * kTopkChunk) return fail(LCA_ERR_UNSUPPORTED, "csa_topk_select: max_n=%d above %d", max_n, lca::topk_max_chunks() * kTopkChunk);
  if (ld_scores < max_n || ld_scores % 4) return fail(LCA_ERR_SHAPE, "csa_topk_select: ld_scores must be >= max_n and a multiple of 4");
  if (flags & ~LCA_TOPK_HIST_READY) return fail(LCA_ERR_SHAPE, "csa_topk_select: unknown flags 0x%x", flags);
  if (rows == 0) return ok();
  if (!scores || !n_vis || !idx || !count || !ws) return fail(LCA_ERR_NULL, "csa_topk_select: NULL pointer");
  if (!al16(scores) || !al16(ws)) return fail(LCA_ERR_ALIGN, "csa_topk_select: scores / ws not 16-byte aligned");
  const size_t need = lca::topk_ws_bytes(rows, max_n, k);
  if (ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "csa_topk_select: ws_bytes %zu < %zu", ws_bytes, need);
  lca::TopkBatch tb{};
  tb.n = 1;
  tb.layer[0] = lca::TopkLayer{scores, ld_scores, n_vis, idx, count, max_n, k,
                               lca::topk_ws_carve(ws, rows, max_n, k)};
  return hip_status(lca::launch_topk(tb, rows, (flags & LCA_TOPK_HIST_READY) != 0, (hipStream_t)stream),
                    "csa_topk_select launch");
}

// ------------------------------------------------------------------ attention
size_t lca_attn_workspace_bytes(int32_t rows, int32_t heads, int32_t max_q, int32_t splits) {
  if (rows <= 0 || heads <= 0) return 0;
  const int sp = splits > 0 ? splits : lca::attn_auto_splits(max_q);
  return lca::attn_ws_bytes(rows, heads, sp);
}

static int32_t attn_common(const char* name, const lca_bf16* q, const lca_bf16* k_cmp,
                           const lca_bf16* v_cmp, const int64_t* ent_off, const int64_t* q_off,
                           int32_t batch, int32_t max_q, int32_t heads, int32_t head_dim,
                           float scale, int32_t splits, lca_bf16* out, void* ws,
                           size_t ws_bytes, lca::AttnArgs& a) {
  if (head_dim != 128) return fail(LCA_ERR_UNSUPPORTED, "%s: head_dim=%d (only 128)", name, head_dim);
  if (!heads_supported(heads)) return fail(LCA_ERR_UNSUPPORTED, "%s: heads=%d (16, 32 or a multiple of 64)", name, heads);
  if (batch < 0 || max_q < 0 || splits < 0) return fail(LCA_ERR_SHAPE, "%s: negative size", name);
  if (splits > 1024) return fail(LCA_ERR_SHAPE, "%s: splits=%d above 1024", name, splits);
  if (!std::isfinite(scale)) return fail(LCA_ERR_SHAPE, "%s: scale not finite", name);
  if ((int64_t)batch * max_q > 65535 * 1024LL) return fail(LCA_ERR_SHAPE, "%s: too many rows", name);
  if (batch == 0 || max_q == 0) return LCA_OK + 1;   // nothing to do
  if (!q || !k_cmp || !v_cmp || !ent_off || !q_off || !out) return fail(LCA_ERR_NULL, "%s: NULL pointer", name);
  if (!al16(q) || !al16(k_cmp) || !al16(v_cmp) || !al16(out)) return fail(LCA_ERR_ALIGN, "%s: q / k_cmp / v_cmp / out not 16-byte aligned", name);
  const int sp = splits > 0 ? splits : lca::attn_auto_splits(max_q);
  const int rows = batch * max_q;
  const size_t need = lca::attn_ws_bytes(rows, heads, sp);
  if (need && (!ws || ws_bytes < need)) return fail(LCA_ERR_WORKSPACE, "%s: ws_bytes %zu < %zu", name, ws_bytes, need);
  if (need && !al16(ws)) return fail(LCA_ERR_ALIGN, "%s: ws not 16-byte aligned", name);
  a = lca::AttnArgs{};
  a.q = q;
  a.kc = k_cmp;
  a.vc = v_cmp;
  a.ent_off = ent_off;
  a.q_off = q_off;
  a.max_q = max_q;
  a.heads = heads;
  a.splits = sp;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  lca::attn_ws_carve(ws, rows, heads, sp, a);
  return LCA_OK;
}

static int32_t sparse_attn_impl(const char* name, const lca_bf16* q, const lca_bf16* k_cmp,
                                const lca_bf16* v_cmp, const int64_t* ent_off, const int64_t* q_off,
                                int32_t batch, int32_t max_q, const int32_t* idx,
                                const int32_t* count, int32_t k, int32_t heads, int32_t head_dim,
                                float scale, int32_t splits, lca_bf16* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream, bool kv8) {
  if (k <= 0) return fail(LCA_ERR_SHAPE, "%s: k=%d must be positive", name, k);
  if (kv8 && heads % 64 != 0) return fail(LCA_ERR_UNSUPPORTED, "%s: heads=%d (mixed KV rows need a multiple of 64)", name, heads);
  lca::AttnArgs a;
  int32_t st = attn_common(name, q, k_cmp, v_cmp, ent_off, q_off, batch, max_q, heads,
                           head_dim, scale, splits, out, ws, ws_bytes, a);
  if (st == LCA_OK + 1) return ok();
  if (st != LCA_OK) return st;
  if (!idx || !count) return fail(LCA_ERR_NULL, "%s: idx / count NULL", name);
  a.idx = idx;
  a.count = count;
  a.k = k;
  a.max_n = k;
  a.ratio = 1;
  a.lse = lse;
  a.kv8 = kv8 ? 1 : 0;
  return hip_status(lca::launch_attention(lca::attn_batch1(a), batch, (hipStream_t)stream),
                    "sparse attention launch");
}

int32_t lca_csa_sparse_attn(const lca_bf16* q, const lca_bf16* k_cmp, const lca_bf16* v_cmp,
                            const int64_t* ent_off, const int64_t* q_off, int32_t batch,
                            int32_t max_q, const int32_t* idx, const int32_t* count, int32_t k,
                            int32_t heads, int32_t head_dim, float scale, int32_t splits,
                            lca_bf16* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return sparse_attn_impl("csa_sparse_attn", q, k_cmp, v_cmp, ent_off, q_off, batch, max_q, idx,
                          count, k, heads, head_dim, scale, splits, out, lse, ws, ws_bytes, stream,
                          false);
}

int32_t lca_csa_sparse_attn_kv8(const lca_bf16* q, const uint8_t* k_cmp, const uint8_t* v_cmp,
                                const int64_t* ent_off, const int64_t* q_off, int32_t batch,
                                int32_t max_q, const int32_t* idx, const int32_t* count, int32_t k,
                                int32_t heads, int32_t head_dim, float scale, int32_t splits,
                                lca_bf16* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
  return sparse_attn_impl("csa_sparse_attn_kv8", q, reinterpret_cast<const lca_bf16*>(k_cmp),
                          reinterpret_cast<const lca_bf16*>(v_cmp), ent_off, q_off, batch, max_q,
                          idx, count, k, heads, head_dim, scale, splits, out, lse, ws, ws_bytes,
                          stream, true);
}

static int32_t dense_attn_impl(const char* name, const lca_bf16* q, const lca_bf16* k_cmp,
                               const lca_bf16* v_cmp, const int64_t* ent_off, const int64_t* q_off,
                               const int64_t* q_pos, int32_t batch, int32_t max_q,
                               int32_t max_entries, int32_t m, int32_t heads, int32_t head_dim,
                               float scale, int32_t splits, lca_bf16* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream, bool kv8) {
  if (kv8 && heads % 64 != 0) return fail(LCA_ERR_UNSUPPORTED, "%s: heads=%d (mixed KV rows need a multiple of 64)", name, heads);
  if (m < 1) return fail(LCA_ERR_SHAPE, "%s: ratio m=%d < 1", name, m);
  if (max_entries < 0) return fail(LCA_ERR_SHAPE, "%s: negative max_entries", name);
  if (max_entries > lca::ATTN_MAX_SEQ) return fail(LCA_ERR_UNSUPPORTED, "%s: max_entries=%d above %d", name, max_entries, lca::ATTN_MAX_SEQ);
  lca::AttnArgs a;
  int32_t st = attn_common(name, q, k_cmp, v_cmp, ent_off, q_off, batch, max_q, heads,
                           head_dim, scale, splits, out, ws, ws_bytes, a);
  if (st == LCA_OK + 1) return ok();
  if (st != LCA_OK) return st;
  if (!q_pos) return fail(LCA_ERR_NULL, "%s: q_pos NULL", name);
  a.q_pos = q_pos;
  a.ratio = m;
  a.max_n = max_entries;
  a.lse = lse;
  a.kv8 = kv8 ? 1 : 0;
  return hip_status(lca::launch_attention(lca::attn_batch1(a), batch, (hipStream_t)stream),
                    "hca_dense_attn launch");
}

int32_t lca_hca_dense_attn(const lca_bf16* q, const lca_bf16* k_cmp, const lca_bf16* v_cmp,
                           const int64_t* ent_off, const int64_t* q_off, const int64_t* q_pos,
                           int32_t batch, int32_t max_q, int32_t max_entries, int32_t m,
                           int32_t heads, int32_t head_dim, float scale, int32_t splits,
                           lca_bf16* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return dense_attn_impl("hca_dense_attn", q, k_cmp, v_cmp, ent_off, q_off, q_pos, batch, max_q,
                         max_entries, m, heads, head_dim, scale, splits, out, lse, ws, ws_bytes,
                         stream, false);
}

int32_t lca_hca_dense_attn_kv8(const lca_bf16* q, const uint8_t* k_cmp, const uint8_t* v_cmp,
                               const int64_t* ent_off, const int64_t* q_off, const int64_t* q_pos,
                               int32_t batch, int32_t max_q, int32_t max_entries, int32_t m,
                               int32_t heads, int32_t head_dim, float scale, int32_t splits,
                               lca_bf16* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return dense_attn_impl("hca_dense_attn_kv8", q, reinterpret_cast<const lca_bf16*>(k_cmp),
                         reinterpret_cast<const lca_bf16*>(v_cmp), ent_off, q_off, q_pos, batch,
                         max_q, max_entries, m, heads, head_dim, scale, splits, out, lse, ws,
                         ws_bytes, stream, true);
}

// ------------------------------------------------------------------ sliding window
static lca::AttnArgs window_args(const lca_bf16* q, const lca_bf16* win_k, const lca_bf16* win_v,
                                 const int64_t* win_off, const int64_t* win_pos0,
                                 const int64_t* q_off, const int64_t* q_pos, int32_t max_q,
                                 int32_t window, int32_t heads, float scale_log2, lca_bf16* out,
                                 float* lse) {
  lca::AttnArgs a{};
  a.q = q;
  a.kc = win_k;
  a.vc = win_v;
  a.ent_off = win_off;
  a.q_off = q_off;
  a.q_pos = q_pos;
  a.max_q = max_q;
  a.heads = heads;
  a.splits = 1;
  a.ratio = 1;
  a.max_n = window;
  a.scale_log2 = scale_log2;
  a.out = out;
  a.lse = lse;
  a.win_pos0 = win_pos0;
  a.window = window;
  a.merge = 1;
  return a;
}

int32_t lca_window_attn(const lca_bf16* q, const lca_bf16* win_k, const lca_bf16* win_v,
                        const int64_t* win_off, const int64_t* win_pos0, const int64_t* q_off,
                        const int64_t* q_pos, int32_t batch, int32_t max_q, int32_t window,
                        int32_t heads, int32_t head_dim, float scale, lca_bf16* out, float* lse,
                        void* stream) {
  if (head_dim != 128) return fail(LCA_ERR_UNSUPPORTED, "window_attn: head_dim=%d (only 128)", head_dim);
  if (!heads_supported(heads)) return fail(LCA_ERR_UNSUPPORTED, "window_attn: heads=%d (16, 32 or a multiple of 64)", heads);
  if (batch < 0 || max_q < 0 || window < 0) return fail(LCA_ERR_SHAPE, "window_attn: negative size");
  if (window > lca::ATTN_MAX_SEQ) return fail(LCA_ERR_UNSUPPORTED, "window_attn: window=%d above %d", window, lca::ATTN_MAX_SEQ);
  if (!std::isfinite(scale)) return fail(LCA_ERR_SHAPE, "window_attn: scale not finite");
  if ((int64_t)batch * max_q > 65535 * 1024LL) return fail(LCA_ERR_SHAPE, "window_attn: too many rows");
  if (batch == 0 || max_q == 0 || window == 0) return ok();
  if (!q || !win_k || !win_v || !win_off || !win_pos0 || !q_off || !q_pos || !out || !lse) return fail(LCA_ERR_NULL, "window_attn: NULL pointer");
  if (!al16(q) || !al16(win_k) || !al16(win_v) || !al16(out)) return fail(LCA_ERR_ALIGN, "window_attn: q / win_k / win_v / out not 16-byte aligned");
  const lca::AttnArgs a = window_args(q, win_k, win_v, win_off, win_pos0, q_off, q_pos, max_q,
                                      window, heads, scale * 1.4426950408889634f, out, lse);
  return hip_status(lca::launch_attention(lca::attn_batch1(a), batch, (hipStream_t)stream),
                    "window_attn launch");
}

int32_t lca_attn_sink(lca_bf16* out, float* lse, const float* sink, int64_t rows, int32_t heads,
                      int32_t head_dim, void* stream) {
  if (head_dim != 128) return fail(LCA_ERR_UNSUPPORTED, "attn_sink: head_dim=%d (only 128)", head_dim);
  if (rows < 0 || heads <= 0) return fail(LCA_ERR_SHAPE, "attn_sink: rows=%lld heads=%d", (long long)rows, heads);
  if (rows * heads > ((int64_t)1 << 27)) return fail(LCA_ERR_SHAPE, "attn_sink: rows x heads above 2^27");
  if (rows == 0) return ok();
  if (!out || !lse || !sink) return fail(LCA_ERR_NULL, "attn_sink: NULL pointer");
  if (!al16(out)) return fail(LCA_ERR_ALIGN, "attn_sink: out not 16-byte aligned");
  return hip_status(lca::launch_attn_sink(out, lse, sink, rows, heads, (hipStream_t)stream),
                    "attn_sink launch");
}

// ------------------------------------------------------------------ hybrid step
size_t lca_hybrid_workspace_bytes(const lca_layer* layers, int32_t n_layers, int32_t batch,
                                  int32_t max_q, int32_t heads) {
  if (!layers || n_layers <= 0 || batch <= 0 || max_q <= 0 || heads <= 0) return 0;
  const int rows = batch * max_q;
  size_t b = 0;
  for (int l = 0; l < n_layers; ++l) {
    const int sp = hybrid_layer_splits(layers[l], hybrid_piece(n_layers, max_q));
    if (layers[l].kind == LCA_LAYER_CSA)
      b += csa_layer_bytes(rows, std::max(layers[l].max_entries, 0), std::max(layers[l].topk, 1),
                           heads, sp);
    else
      b += lca::attn_ws_bytes(rows, heads, sp);
  }
  return b;
}

int32_t lca_hybrid_layer_step(const lca_layer* layers, int32_t n_layers, const int64_t* q_off,
                              const int64_t* q_pos, int32_t batch, int32_t max_q, int32_t heads,
                              int32_t head_dim, float scale, void* ws, size_t ws_bytes,
                              void* stream) {
  if (n_layers < 0 || batch < 0 || max_q < 0) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: negative size");
  if (n_layers == 0 || batch == 0 || max_q == 0) return ok();
  if (!layers || !q_off || !q_pos) return fail(LCA_ERR_NULL, "hybrid_layer_step: NULL pointer");
  const size_t need = lca_hybrid_workspace_bytes(layers, n_layers, batch, max_q, heads);
  if (need && (!ws || ws_bytes < need)) return fail(LCA_ERR_WORKSPACE, "hybrid_layer_step: ws_bytes %zu < %zu", ws_bytes, need);
  if (need && !al16(ws)) return fail(LCA_ERR_ALIGN, "hybrid_layer_step: ws not 16-byte aligned");
  // validate every layer before enqueueing anything
  for (int l = 0; l < n_layers; ++l) {
    const lca_layer& L = layers[l];
    if (L.kind != LCA_LAYER_CSA && L.kind != LCA_LAYER_HCA) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: layer %d has unknown kind %d", l, L.kind);
    if (L.ratio < 1 || L.max_entries < 0) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: layer %d ratio/max_entries", l);
    if (L.max_entries > lca::ATTN_MAX_SEQ) return fail(LCA_ERR_UNSUPPORTED, "hybrid_layer_step: layer %d max_entries above %d", l, lca::ATTN_MAX_SEQ);
    if (!L.q || !L.k_cmp || !L.v_cmp || !L.ent_off || !L.out) return fail(LCA_ERR_NULL, "hybrid_layer_step: layer %d NULL pointer", l);
    if (L.kind == LCA_LAYER_CSA) {
      if (L.topk <= 0) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: layer %d topk=%d", l, L.topk);
      if (!L.q_idx || !L.k_idx || !L.idx || !L.count) return fail(LCA_ERR_NULL, "hybrid_layer_step: CSA layer %d NULL pointer", l);
      if (!al16(L.q_idx) || !al16(L.k_idx)) return fail(LCA_ERR_ALIGN, "hybrid_layer_step: layer %d indexer not aligned", l);
      if (L.idx_format != LCA_IDX_INT8 && L.idx_format != LCA_IDX_FP4) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: layer %d idx_format=%d", l, L.idx_format);
      if ((int64_t)L.max_entries > (int64_t)lca::DS_MAX_CHUNKS * lca::DS_CHUNK) return fail(LCA_ERR_UNSUPPORTED, "hybrid_layer_step: layer %d max_entries too large", l);
    }
    if (head_dim != 128) return fail(LCA_ERR_UNSUPPORTED, "hybrid_layer_step: head_dim=%d (only 128)", head_dim);
    if (!heads_supported(heads)) return fail(LCA_ERR_UNSUPPORTED, "hybrid_layer_step: heads=%d", heads);
    if (!al16(L.q) || !al16(L.k_cmp) || !al16(L.v_cmp) || !al16(L.out)) return fail(LCA_ERR_ALIGN, "hybrid_layer_step: layer %d tensors not aligned", l);
    if (L.window < 0 || L.window > lca::ATTN_MAX_SEQ) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: layer %d window=%d", l, L.window);
    if (L.kv_format != LCA_KV_BF16 && L.kv_format != LCA_KV_MIXED) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: layer %d kv_format=%d", l, L.kv_format);
    if (L.kv_format == LCA_KV_MIXED && heads % 64 != 0) return fail(LCA_ERR_UNSUPPORTED, "hybrid_layer_step: layer %d mixed KV rows need heads a multiple of 64", l);
    if (L.window > 0) {
      if (!L.win_k || !L.win_v || !L.win_off || !L.win_pos0 || !L.lse) return fail(LCA_ERR_NULL, "hybrid_layer_step: layer %d window buffers / lse NULL", l);
      if (!al16(L.win_k) || !al16(L.win_v)) return fail(LCA_ERR_ALIGN, "hybrid_layer_step: layer %d window buffers not aligned", l);
    }
  }
  if (!std::isfinite(scale)) return fail(LCA_ERR_SHAPE, "hybrid_layer_step: scale not finite");
  const hipStream_t caller = (hipStream_t)stream;
  const int rows = batch * max_q;
  const float scale_log2 = scale * 1.4426950408889634f;

  // carve each layer's workspace region (layer order, as lca_hybrid_workspace_bytes sizes it)
  std::vector<lca::DsLayer> il;
  std::vector<int> il_fp4;   // per CSA layer: FP4 indexer codes
  std::vector<lca::AttnArgs> args((size_t)n_layers);
  bool has_csa = false;
  char* p = reinterpret_cast<char*>(ws);
  for (int l = 0; l < n_layers; ++l) {
    const lca_layer& L = layers[l];
    const int piece = hybrid_piece(n_layers, max_q);
    const int sp = hybrid_layer_splits(L, piece);
    lca::AttnArgs a{};
    a.q = L.q;
    a.kc = L.k_cmp;
    a.vc = L.v_cmp;
    a.ent_off = L.ent_off;
    a.q_off = q_off;
    a.max_q = max_q;
    a.heads = heads;
    a.splits = sp;
    a.scale_log2 = scale_log2;
    a.out = L.out;
    a.lse = L.lse;
    a.sink = L.window > 0 ? nullptr : L.sink;   // else the window branch writes last
    a.kv8 = L.kv_format == LCA_KV_MIXED ? 1 : 0;
    if (L.kind == LCA_LAYER_CSA) {
      lca::DsLayer d{};
      d.q_idx = L.q_idx;
      d.k_idx = L.k_idx;
      d.ent_off = L.ent_off;
      d.idx = L.idx;
      d.count = L.count;
      d.c = L.ratio;
      d.max_entries = L.max_entries;
      d.k = L.topk;
      lca::ds_ws_carve(p, rows, L.max_entries, L.topk, d);
      p += lca::ds_ws_bytes(rows, L.max_entries, L.topk);
      d.idx_gy = reinterpret_cast<int32_t*>(p);
      p += lca::align256((size_t)rows * L.topk * 4);
      il.push_back(d);
      il_fp4.push_back(L.idx_format == LCA_IDX_FP4 ? 1 : 0);
      a.idx = L.idx;
      a.idx_gy = d.idx_gy;
      a.count = L.count;
      a.k = L.topk;
      a.max_n = piece * sp;   // every row's piece: ceil(max_n / splits) = piece
      a.ratio = 1;
      lca::attn_ws_carve(p, rows, heads, sp, a);
      p += lca::attn_ws_bytes(rows, heads, sp);
      has_csa = true;
    } else {
      a.q_pos = q_pos;
      a.ratio = L.ratio;
      a.max_n = piece * sp;
      lca::attn_ws_carve(p, rows, heads, sp, a);
      p += lca::attn_ws_bytes(rows, heads, sp);
    }
    args[l] = a;
  }

  // One stream, three phases: the CSA layers' scores and selections (batched, up to 8
  // layers per launch), then the attention of every layer, CSA and HCA together in
  // launches of up to 8 layers.  Everything is bound by HBM bandwidth except the
  // selection, and one attention launch for all layers pays the pipeline start and
  // drain once instead of per kind.
  HybridTiming* ls = hybrid_timing();
  hipError_t e = hipSuccess;
  const int hb64 = (heads + 63) / 64;   // 64-head blocks
  const bool timing = ls && ls->timing;
  if (timing) {
    ls->has_csa = has_csa;
    ls->timed = true;
  }
  auto mark = [&](int i) {
    if (timing && e == hipSuccess) e = hipEventRecord(ls->tev[i], caller);
  };
  // index launches group the CSA layers by indexer format, up to 8 layers each
  std::vector<std::vector<int>> groups;
  for (int f = 0; f < 2; ++f) {
    std::vector<int> cur;
    for (size_t l = 0; l < il.size(); ++l) {
      if (il_fp4[l] != f) continue;
      cur.push_back((int)l);
      if ((int)cur.size() == lca::MAX_BATCH_LAYERS) {
        groups.push_back(cur);
        cur.clear();
      }
    }
    if (!cur.empty()) groups.push_back(cur);
  }
  for (size_t gi = 0; gi < groups.size() && e == hipSuccess; ++gi) {
    const std::vector<int>& grp = groups[gi];
    const int n = (int)grp.size();
    lca::DsBatch db{};
    db.q_off = q_off;
    db.q_pos = q_pos;
    db.max_q = max_q;
    db.n = n;
    db.fp4 = il_fp4[grp[0]];
    for (int i = 0; i < n; ++i) db.layer[i] = il[grp[i]];
    const bool first = gi == 0;
    if (first) mark(0);
    e = lca::launch_ds_chunks(db, batch, caller);
    // timed steps may repeat the index pass back to back (identical results): event 1
    // minus event 0 over the count is then the launch's own duration, without the
    // dispatch gap after an event
    for (int r = 1; first && timing && r < ls->index_reps && e == hipSuccess; ++r)
      e = lca::launch_ds_chunks(db, batch, caller);
    if (first) mark(1);
    if (e == hipSuccess) e = lca::launch_ds_select(db, batch, caller);
    if (first) mark(2);
  }
  mark(3);
  for (const std::vector<int>& grp : attn_groups(layers, n_layers)) {
    if (e != hipSuccess) break;
    lca::AttnBatch ab{};
    ab.n = (int)grp.size();
    ab.hpb = std::min(heads, 64);
    ab.head_blocks = hb64;
    for (int i = 0; i < ab.n; ++i) ab.a[i] = args[grp[i]];
    e = lca::launch_attention(ab, batch, caller);
  }
  // sliding-window branches, merged into each layer's result (one launch per 8 layers)
  std::vector<lca::AttnArgs> win_a;
  for (int l = 0; l < n_layers; ++l) {
    const lca_layer& L = layers[l];
    if (L.window > 0) {
      win_a.push_back(window_args(L.q, L.win_k, L.win_v, L.win_off, L.win_pos0, q_off, q_pos,
                                  max_q, L.window, heads, scale_log2, L.out, L.lse));
      win_a.back().sink = L.sink;
    }
  }
  for (size_t c0 = 0; c0 < win_a.size() && e == hipSuccess; c0 += lca::MAX_BATCH_LAYERS) {
    const int n = (int)std::min<size_t>(lca::MAX_BATCH_LAYERS, win_a.size() - c0);
    lca::AttnBatch ab{};
    ab.n = n;
    ab.hpb = std::min(heads, 64);
    ab.head_blocks = hb64;
    for (int i = 0; i < n; ++i) ab.a[i] = win_a[c0 + i];
    e = lca::launch_attention(ab, batch, caller);
  }
  mark(4);
  if (e != hipSuccess) return fail(LCA_ERR_HIP, "hybrid_layer_step: %s", hipGetErrorString(e));
  return ok();
}

int32_t lca_hybrid_timing_enable(int32_t enable) {
  HybridTiming* ls = hybrid_timing();
  if (!ls) return fail(LCA_ERR_HIP, "hybrid_timing_enable: no timing events");
  ls->timing = enable != 0;
  ls->index_reps = std::max(1, std::min(enable, 1000));
  ls->timed = false;
  return ok();
}

int32_t lca_hybrid_timing_read(float* ms, int32_t n) {
  if (!ms || n < 0) return fail(LCA_ERR_NULL, "hybrid_timing_read: ms NULL");
  HybridTiming* ls = hybrid_timing();
  if (!ls) return fail(LCA_ERR_HIP, "hybrid_timing_read: no timing events");
  if (!ls->timing || !ls->timed) return fail(LCA_ERR_SHAPE, "hybrid_timing_read: no timed step");
  float t[LCA_HYBRID_PHASES] = {0.f, 0.f, 0.f};
  const int pairs[LCA_HYBRID_PHASES][2] = {{0, 1}, {1, 2}, {3, 4}};
  for (int p = 0; p < LCA_HYBRID_PHASES; ++p) {
    const bool present = p < 2 ? ls->has_csa : true;
    if (!present) continue;
    if (hipEventSynchronize(ls->tev[pairs[p][1]]) != hipSuccess ||
        hipEventElapsedTime(&t[p], ls->tev[pairs[p][0]], ls->tev[pairs[p][1]]) != hipSuccess)
      return fail(LCA_ERR_HIP, "hybrid_timing_read: event query");
  }
  t[0] /= (float)ls->index_reps;
  for (int p = 0; p < n && p < LCA_HYBRID_PHASES; ++p) ms[p] = t[p];
  return ok();
}

}  // extern "C"
