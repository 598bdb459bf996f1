/*
 * lca.h — C ABI of the CSA / HCA compressed-KV attention library for gfx950.
 *
 * The operations follow "DeepSeek-V4: Towards Highly Efficient Million-Token
 * Context Intelligence Review" (dimensionstp.github.io):
 *   - section 2-1 and section 3-2 item 2 (component table): CSA compresses the KV
 *     sequence 4 tokens per entry and runs sparse attention over a top-k of the
 *     entries; HCA compresses 128 tokens per entry and attends densely; both
 *     ratios are the same in both model sizes; CSA and HCA layers are interleaved.
 *   - section 3-2 item 4: CSA's indexer has its own Q.K path; the compressed
 *     cache is kept apart from a state cache holding the sliding window and the
 *     tokens not yet ready for compression.
 * The page leaves the pooling operator, the indexer form and the sizes open.
 * This library implements mean pooling, an int8 indexer (d_idx = 64, exact
 * int32 dot products), a top-k ranked by (score desc, index asc), and softmax
 * attention with fp32 accumulation over bf16 K/V (head_dim = 128).
 *
 * Conventions shared by every call
 *   Memory.   Every tensor pointer is DEVICE memory owned by the caller.  The
 *             library allocates no device memory.  Its only state is a
 *             per-thread error string and, once lca_hybrid_layer_step or its
 *             timing calls have run on a device, 5 timing events for that device
 *             (created on first use, kept until exit).  Every call runs on the
 *             caller's stream only.  Tensors are dense
 *             and row-major.  bf16 values are
 *             passed as uint16_t bit patterns.  K/V/query rows and indexer rows
 *             must be 16-byte aligned (else LCA_ERR_ALIGN).
 *   Batches.  Sequences are packed.  ent_off[B+1] (device, int64) gives each
 *             sequence's first compressed entry; q_off[B+1] (device, int64) its
 *             first query row; q_pos[rows] (device, int64) the absolute token
 *             position of each query row (a decoding query after L tokens sits at
 *             L).  Host scalars max_q / max_entries bound the per-sequence counts
 *             and size the launch grids; values beyond them are not processed.
 *   Visibility. A query at position p sees entry j of a cache compressed at
 *             ratio r iff the entry's block has ended before p: (j+1)*r <= p.
 *   Streams.  `stream` is a hipStream_t passed as void* (NULL = default
 *             stream).  Calls validate, enqueue and return; none synchronises.
 *   Errors.   Every call returns an int32 status (below).  Validation happens
 *             before anything is enqueued, so a failed call has no effect.
 *             lca_last_error() returns a per-thread message for the last failure.
 *             Faults inside a kernel surface at the caller's next synchronisation.
 *   Workspace. Calls that need scratch memory take (ws, ws_bytes); the size comes
 *             from the matching lca_*_workspace_bytes query.  A workspace must be
 *             ZERO-FILLED by the caller before its first use; every call returns
 *             it to that state (the kernels that consume counters and histograms
 *             clear them), so one zeroed workspace serves any number of calls in
 *             stream order.  Calls that share a workspace must not run
 *             concurrently.  lca_workspace_reset() re-zeroes one on a stream.
 *   Determinism. Every output is bitwise reproducible: no result depends on the
 *             order in which work-groups finish.  Batch invariance: a query row's
 *             result depends only on its own inputs and on the size arguments that
 *             fix how a row is cut into pieces (the single-layer attention calls:
 *             splits with k or max_entries; lca_hybrid_layer_step: the layer and
 *             query counts), never on the other rows of the batch.  So a sequence
 *             gives the same bits alone or inside any batch of the hybrid step,
 *             and inside any batch of a single call made with the same splits and
 *             bound.
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCA_ABI_VERSION 8

enum lca_status {
  LCA_OK = 0,
  LCA_ERR_NULL = -1,        /* a required pointer is NULL */
  LCA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or inconsistent */
  LCA_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  LCA_ERR_UNSUPPORTED = -4, /* head_dim != 128, d_idx != 64, heads % 16 != 0, ... */
  LCA_ERR_WORKSPACE = -5,   /* ws_bytes smaller than the query returned */
  LCA_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  LCA_ERR_INTERNAL = -7
};

typedef uint16_t lca_bf16;

int32_t lca_abi_version(void);
const char* lca_last_error(void);
/* Number of compute units of the current device (for callers sizing work); -1 on error. */
int32_t lca_device_cu_count(void);
/* Re-zero a workspace on `stream` (a fill kernel, not a memset node). */
int32_t lca_workspace_reset(void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kv_compress — mean pooling of complete blocks of c tokens.
 * Page section 3-2 item 2 (component table): CSA maps every 4 tokens to one
 * compressed entry, HCA every 128; the pooling operator is the mean here.
 *
 *   x        [tok_off[B], head_dim] bf16 raw tokens, sequence b in rows
 *            tok_off[b] .. tok_off[b+1]-1.
 *   y        [*, head_dim] bf16; sequence b writes n_b = min(floor(T_b / c),
 *            ent_off[b+1] - ent_off[b]) entries at rows ent_off[b] .. .
 *            Entry j = mean of tokens j*c .. j*c+c-1 of its sequence, summed in
 *            fp64 and rounded once to bf16 (to nearest, ties to even).  The
 *            T_b mod c tail tokens form no entry.
 *   max_tokens  host bound on T_b; head_dim % 8 == 0; 1 <= c <= 4096.
 * ------------------------------------------------------------------------- */
int32_t lca_kv_compress(const lca_bf16* x, const int64_t* tok_off, int32_t batch,
                        int32_t max_tokens, int32_t head_dim, int32_t c, lca_bf16* y,
                        const int64_t* ent_off, void* stream);

/* kv_compress_kv8 — the same pooling into mixed KV rows (head_dim 128), the row
 * format the _kv8 attention calls read (page section 3-2 item 2, component table:
 * the cache keeps the RoPE dims in BF16, the rest in FP8; the last 64 dims are taken
 * as the RoPE dims).
 *   y        [*, 192] bytes, 16-byte aligned; entry rows at ent_off[b] .. as in
 *            lca_kv_compress.  Bytes 0..63 of a row: dims 0..63 of the fp64 mean,
 *            each rounded once to an FP8 E4M3 code (nearest, ties to the even code,
 *            magnitudes above 448 clamped to 448, the sign kept); bytes 64..191:
 *            dims 64..127 rounded once to bf16 (little-endian).
 *   Other arguments and errors as lca_kv_compress (head_dim is 128).
 */
int32_t lca_kv_compress_kv8(const lca_bf16* x, const int64_t* tok_off, int32_t batch,
                            int32_t max_tokens, int32_t c, uint8_t* y, const int64_t* ent_off,
                            void* stream);

/* ---------------------------------------------------------------------------
 * csa_index_score — indexer scores of every query row against its sequence's
 * indexer keys.  Page section 3-2 item 4: CSA's indexer scores entries through
 * a Q.K product of its own.  Here: int8 x int8 products summed exactly in
 * int32, in [-2^20, 2^20]: 64 * (-128)^2 = 2^20 is reached only by a query and a
 * key of all -128 codes; every other score is at most 2^20 - 128.
 *
 *   q_idx    [rows, d_idx] int8, one indexer query per query row.
 *   k_idx    [ent_off[B], d_idx] int8 indexer keys, one per compressed entry.
 *   scores   [rows, ld_scores] int32; row r of sequence b gets N_b values:
 *            entries j < n_vis[r] hold the score, entries n_vis[r] <= j < N_b
 *            hold INT32_MIN; columns >= N_b are not written.
 *   n_vis    [rows] int32 out: min(floor(q_pos[r] / c), N_b).
 *   ws       optional top-k workspace, sized by lca_csa_topk_workspace_bytes(
 *            batch * max_q, max_entries, k).  When given, the first radix pass
 *            of the following lca_csa_topk_select (rows = batch * max_q) is fused
 *            here; that call must then pass LCA_TOPK_HIST_READY with the same
 *            workspace.
 *   rows     = q_off[B] must not exceed batch * max_q.
 *   d_idx == 64; ld_scores >= max_entries.
 * ------------------------------------------------------------------------- */
int32_t lca_csa_index_score(const int8_t* q_idx, const int64_t* q_off, const int64_t* q_pos,
                            const int8_t* k_idx, const int64_t* ent_off, int32_t batch,
                            int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                            int32_t* scores, int64_t ld_scores, int32_t* n_vis, void* ws,
                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * csa_index_score_fp4 — the indexer scores with FP4 query and keys.  Page section
 * 3-2 item 4: the indexer's Q.K path is trained with FP4 quantisation-aware
 * training.  Reading: E2M1 codes (the OCP Microscaling FP4 element: sign, 2
 * exponent bits with bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 * their negatives), d_idx = 64 codes packed two per byte (element 2i in the low
 * nibble of byte i), 32 bytes per vector, with one power-of-two scale per tensor,
 * which cannot change the ranking and is left out.  score = 256 * sum_d q_d k_d, an
 * exact integer (a multiple of 64) in [-589824, 589824]: inside the int8 scores'
 * range (|score| < 2^20) and spread over it, so lca_csa_topk_select and its fused
 * histogram apply unchanged and their 2048 coarse bins resolve it.
 *
 *   q_fp4    [rows, 32] uint8, k_fp4 [ent_off[B], 32] uint8; 16-byte aligned.
 *   Every other argument as lca_csa_index_score (d_idx == 64).  Query batches of
 *   any size run the same per-row kernel; for prefill-sized batches
 *   lca_csa_index_select_fp4 selects without writing the scores.
 * ------------------------------------------------------------------------- */
int32_t lca_csa_index_score_fp4(const uint8_t* q_fp4, const int64_t* q_off, const int64_t* q_pos,
                                const uint8_t* k_fp4, const int64_t* ent_off, int32_t batch,
                                int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                                int32_t* scores, int64_t ld_scores, int32_t* n_vis, void* ws,
                                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * csa_index_select — csa_index_score and csa_topk_select in one call, without
 * the score matrix: idx, count and n_vis are exactly what those two calls give.
 * Page section 3-2 items 2 and 4 (indexer scores, then a sparse top-k).
 *
 * Decode-sized batches (max_q < 16 query rows per sequence) take the candidate
 * path and need a workspace: one work-group per 2048 entries of a row scores them
 * in LDS and keeps the chunk's top coarse bins (about twice its expected share of
 * the top-k, in index order); one work-group per row then selects the top-k from
 * the candidates, exactly.  When a chunk held more than its share at or above the
 * row's threshold bin (heavy ties, or a top-k bunched in a few chunks), that row's
 * selection rescans its keys instead: the same result, more time.
 * Prefill-sized batches (max_q >= 16): a work-group owns 16 query tokens of a
 * sequence and all its entries and recomputes the int8 scores (MFMA) in sweeps
 * over the keys: the coarse histogram, then (when every token's threshold bin
 * holds at most 448 entries) one sweep collecting the entries above and inside
 * that bin, resolved in LDS; otherwise the fine histogram of the threshold bin and
 * a third sweep placing the selection in index order.  No workspace.
 *   q_idx, q_off, q_pos, k_idx, ent_off, batch, max_q, max_entries, d_idx, c
 *            as for lca_csa_index_score.
 *   k        entries kept per query row (>= 1).
 *   idx      [rows, k] int32 out: selected entry indices in ascending order,
 *            then -1 padding.    count [rows] int32 out: min(k, n_vis[r]).
 *   n_vis    [rows] int32 out, or NULL: min(floor(q_pos[r] / c), N_b).
 *   ws       workspace of lca_csa_index_select_workspace_bytes(batch, max_q,
 *            max_entries, k) bytes (0 for prefill-sized batches: ws may be NULL),
 *            16-byte aligned; its contents on entry do not matter (every call
 *            writes whatever it reads back), so calls sharing one ws must not
 *            overlap in time.
 *   Decode-sized batches: max_entries <= 4,194,304 (else LCA_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */
size_t lca_csa_index_select_workspace_bytes(int32_t batch, int32_t max_q, int32_t max_entries,
                                            int32_t k);
int32_t lca_csa_index_select(const int8_t* q_idx, const int64_t* q_off, const int64_t* q_pos,
                             const int8_t* k_idx, const int64_t* ent_off, int32_t batch,
                             int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                             int32_t k, int32_t* idx, int32_t* count, int32_t* n_vis, void* ws,
                             size_t ws_bytes, void* stream);

/* csa_index_select_fp4 — the same selection over FP4 indexer codes (page section 3-2
 * item 4: the indexer's Q.K path trained with FP4 quantisation-aware training; the code
 * format and score unit as lca_csa_index_score_fp4): exactly what
 * lca_csa_index_score_fp4 followed by lca_csa_topk_select gives.  Scores come from the
 * FP4 MFMA (E2M1 operands, unit scales); the workspace is the int8 form's.
 *   q_fp4 [rows, 32], k_fp4 [ent_off[B], 32] packed E2M1 codes as for
 *   lca_csa_index_score_fp4; every other argument and error as lca_csa_index_select.
 */
int32_t lca_csa_index_select_fp4(const uint8_t* q_fp4, const int64_t* q_off, const int64_t* q_pos,
                                 const uint8_t* k_fp4, const int64_t* ent_off, int32_t batch,
                                 int32_t max_q, int32_t max_entries, int32_t d_idx, int32_t c,
                                 int32_t k, int32_t* idx, int32_t* count, int32_t* n_vis,
                                 void* ws, size_t ws_bytes, void* stream);

/* csa_index_select_noalloc — lca_csa_index_select for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without ws / ws_bytes and the same result.
 * The workspace of the decode-sized form is a device array inside the library of
 * LCA_INDEX_SELECT_SCRATCH_BYTES bytes, one per GPU, held until the process ends;
 * the first call on a GPU looks up that GPU's copy (hipGetSymbolAddress), so make
 * it before any capture.  The call allocates nothing.
 *   Errors: as lca_csa_index_select, and LCA_ERR_WORKSPACE when the batch needs
 *   more than LCA_INDEX_SELECT_SCRATCH_BYTES, i.e. when
 *   lca_csa_index_select_workspace_bytes(batch, max_q, max_entries, k) exceeds it
 *   (8 MiB holds 26 rows of 4,194,304 entries, or 227 rows of 262,144, at k 2048).
 *   Every call on one GPU uses that GPU's one array: calls that overlap in time on
 *   one GPU (two streams, or two threads) race and give undefined results.  Nothing
 *   in it needs clearing between calls.
 */
#define LCA_INDEX_SELECT_SCRATCH_BYTES ((size_t)8 << 20)
int32_t lca_csa_index_select_noalloc(const int8_t* q_idx, const int64_t* q_off,
                                     const int64_t* q_pos, const int8_t* k_idx,
                                     const int64_t* ent_off, int32_t batch, int32_t max_q,
                                     int32_t max_entries, int32_t d_idx, int32_t c, int32_t k,
                                     int32_t* idx, int32_t* count, int32_t* n_vis,
                                     void* stream);

/* ---------------------------------------------------------------------------
 * csa_topk_select — per row, the top min(k, n_vis[r]) entries of
 * scores[r, 0 .. n_vis[r]) ranked by (score desc, index asc).
 * Page section 3-2 item 2 (component table): CSA keeps a sparse top-k of the
 * compressed entries.  The tie rule (lower index first) is this library's.
 *
 *   scores   [rows, ld_scores] int32, values in [-2^20, 2^20] (what the int8
 *            indexer with d_idx = 64 produces; others give unspecified sets).  The
 *            radix key clamps 2^20 to 2^20 - 1, a value no other int8 score reaches.
 *   n_vis    [rows] int32 visible entries per row (<= max_n).
 *   idx      [rows, k] int32 out: selected entry indices in ascending order,
 *            then -1 padding.    count [rows] int32 out: min(k, n_vis[r]).
 *   flags    LCA_TOPK_HIST_READY if lca_csa_index_score already ran with ws.
 *   Radix select over a 21-bit key in two levels (2048 then 1024 bins); each
 *   chunk of 4096 scores places its selections from counts of the earlier
 *   chunks, so ties resolve deterministically and no work-group waits on another.
 * ------------------------------------------------------------------------- */
#define LCA_TOPK_HIST_READY 1u
size_t lca_csa_topk_workspace_bytes(int32_t rows, int32_t max_n, int32_t k);
int32_t lca_csa_topk_select(const int32_t* scores, int64_t ld_scores, int32_t rows,
                            int32_t max_n, const int32_t* n_vis, int32_t k, int32_t* idx,
                            int32_t* count, void* ws, size_t ws_bytes, uint32_t flags,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Attention over compressed entries (one shared KV head, H query heads).
 * Page sections 2-1 and 3-2 item 2: CSA attends the selected entries, HCA all
 * visible ones.  For each head h: logits = scale * q_h . K_j, p = softmax,
 * o_h = sum_j p_j V_j; lse_h = log sum_j exp(logits_j).  bf16 inputs, fp32
 * logits / softmax / accumulation, bf16 output (to nearest, ties to even).
 * A row with no entries gets o = 0 and lse = -inf.
 *
 *   q        [rows, heads, 128] bf16;  out [rows, heads, 128] bf16
 *   lse      [rows, heads] fp32 (nullable)
 *   k_cmp, v_cmp  [ent_off[B], 128] bf16 compressed cache; a sequence may hold
 *            at most 2^24 entries (max_entries above that is LCA_ERR_UNSUPPORTED;
 *            sparse indices are clamped into the first 2^24 entries).
 *   heads % 16 == 0, head_dim == 128.
 *   splits   work-groups per (row, 64 heads) along the entries for a row at the
 *            bound (k for CSA, max_entries for HCA); shorter rows take
 *            proportionally fewer.  0 = automatic (32 when max_q == 1, fewer as
 *            max_q grows, 1 from max_q >= 32).  The split of a row depends only on
 *            its own entry count, the bound and `splits`, so a row's result does not
 *            depend on the other rows of the batch.
 * ------------------------------------------------------------------------- */
size_t lca_attn_workspace_bytes(int32_t rows, int32_t heads, int32_t max_q, int32_t splits);

/* Sparse (CSA): row r attends entries ent_off[b] + idx[r, j] for j < count[r]. */
int32_t lca_csa_sparse_attn(const lca_bf16* q, const lca_bf16* k_cmp, const lca_bf16* v_cmp,
                            const int64_t* ent_off, const int64_t* q_off, int32_t batch,
                            int32_t max_q, const int32_t* idx, const int32_t* count, int32_t k,
                            int32_t heads, int32_t head_dim, float scale, int32_t splits,
                            lca_bf16* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Dense (HCA): row r attends entries 0 .. min(floor(q_pos[r] / m), N_b) - 1. */
int32_t lca_hca_dense_attn(const lca_bf16* q, const lca_bf16* k_cmp, const lca_bf16* v_cmp,
                           const int64_t* ent_off, const int64_t* q_off, const int64_t* q_pos,
                           int32_t batch, int32_t max_q, int32_t max_entries, int32_t m,
                           int32_t heads, int32_t head_dim, float scale, int32_t splits,
                           lca_bf16* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Mixed KV storage.  Page section 3-2 item 2 (component table): the KV cache keeps the
 * RoPE dims in BF16 and the rest in FP8.  Reading: of the 128 dims of a compressed
 * entry the last 64 are the RoPE dims; a row of KV8 (192 bytes, 16-byte aligned)
 * holds dims 0..63 as FP8 E4M3 codes (OCP E4M3: bias 7, no infinities, largest 448;
 * one scale per tensor, 1) in bytes 0..63 and dims 64..127 as bf16 in bytes 64..191.
 * The K and the V cache use the same row format.  The _kv8 calls take k_cmp / v_cmp
 * [ent_off[B], 192] uint8 in that format and are otherwise the calls above; heads must
 * be a multiple of 64 (LCA_ERR_UNSUPPORTED otherwise).  The FP8 dims are widened to
 * bf16 exactly (every E4M3 value is a bf16 value) and the arithmetic is the same. */
int32_t lca_csa_sparse_attn_kv8(const lca_bf16* q, const uint8_t* k_cmp, const uint8_t* v_cmp,
                                const int64_t* ent_off, const int64_t* q_off, int32_t batch,
                                int32_t max_q, const int32_t* idx, const int32_t* count, int32_t k,
                                int32_t heads, int32_t head_dim, float scale, int32_t splits,
                                lca_bf16* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream);
int32_t lca_hca_dense_attn_kv8(const lca_bf16* q, const uint8_t* k_cmp, const uint8_t* v_cmp,
                               const int64_t* ent_off, const int64_t* q_off, const int64_t* q_pos,
                               int32_t batch, int32_t max_q, int32_t max_entries, int32_t m,
                               int32_t heads, int32_t head_dim, float scale, int32_t splits,
                               lca_bf16* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * window_attn — the sliding-window branch, merged into a compressed branch's result.
 * Page section 3-2 item 2: CSA and HCA both add a branch over the most recent tokens
 * uncompressed (window 128 in the config table); section 3-2 item 4: those tokens
 * live in a state cache beside the compressed cache.  Reading: the window is the
 * `window` raw tokens strictly before the query (positions [p - window, p)), and
 * the branch adds its keys to the same softmax as the compressed entries.
 *
 *   win_k, win_v  [win_off[B], head_dim] bf16 raw tokens of each sequence's state
 *            buffer; buffer b's first row is the token at absolute position
 *            win_pos0[b] (device int64 [B]).  Tokens of the window missing from the
 *            buffer are not attended.
 *   q, q_off, q_pos, batch, max_q, heads, head_dim, scale  as for the attention calls.
 *   out, lse in: the compressed branch's result for every row (lse natural log,
 *            -inf with out = 0 for a row that attended nothing); out: the result
 *            of one softmax over both key sets (log-sum-exp merge).  lse required.
 *   window >= 0 (0: nothing to do).  No workspace.
 *
 * Decode with the state cache (page section 3-2 item 4: the window and the tokens not
 * yet ready for compression are kept apart from the compressed cache).  Per layer of
 * compression ratio r and window w, for a sequence of L tokens (query at position L):
 *   - the compressed cache holds the floor(L / r) complete blocks; it may be laid out
 *     with room for later entries (ent_off spaced by capacity): the attention and the
 *     selection see only min(floor(q_pos / r), N_b) entries, so rows not yet written
 *     are never read;
 *   - the state buffer holds at least the tokens [min(L - w, floor(L / r) * r), L):
 *     the window and the incomplete block's tail (up to r - 1 tokens); win_pos0 is
 *     the position of its row 0, and rows past position L - 1 are never read;
 *   - after the step the new token (position L) is appended to the buffer; when
 *     L + 1 is a multiple of r the block [L + 1 - r, L + 1) is complete:
 *     lca_kv_compress over those r buffered tokens (tok_off {0, r}, batch 1, ent_off
 *     {0, 1}, y = the sequence's next cache row) appends its entry (for CSA the
 *     indexer key of the new entry is written beside it), and the buffer may drop
 *     the tokens before L + 1 - w (moving win_pos0 up).
 * ------------------------------------------------------------------------- */
int32_t lca_window_attn(const lca_bf16* q, const lca_bf16* win_k, const lca_bf16* win_v,
                        const int64_t* win_off, const int64_t* win_pos0, const int64_t* q_off,
                        const int64_t* q_pos, int32_t batch, int32_t max_q, int32_t window,
                        int32_t heads, int32_t head_dim, float scale, lca_bf16* out, float* lse,
                        void* stream);

/* ---------------------------------------------------------------------------
 * attn_sink — fold an attention sink into a finished attention result, in place.
 * Page section 3-2 item 2 lists an attention sink among the parts of the CSA / HCA
 * attention without defining it.  Reading: head h has a scalar logit sink[h]
 * (natural-log units, like the scaled q.K logits) that joins the softmax
 * normalisation as one more key with a zero value row:
 *     p_j = e^(l_j) / (e^(sink_h) + sum_i e^(l_i)),   o_h = sum_j p_j V_j.
 * Applied to a result (o, lse) of the attention calls (after lca_window_attn when
 * the window branch is used, so that the sink joins that one softmax once):
 *     o <- o / (1 + e^(sink_h - lse)),   lse <- log(e^lse + e^(sink_h)).
 * A row that attended nothing (o = 0, lse = -inf) gets lse = sink_h; sink_h = -inf
 * leaves the row unchanged.
 *   out   [rows, heads, head_dim] bf16, in / out.
 *   lse   [rows, heads] fp32 natural log, in / out (required).
 *   sink  [heads] fp32 device.
 *   rows >= 0 query rows (0: nothing to do); head_dim 128.  No workspace.
 * ------------------------------------------------------------------------- */
int32_t lca_attn_sink(lca_bf16* out, float* lse, const float* sink, int64_t rows, int32_t heads,
                      int32_t head_dim, void* stream);

/* ---------------------------------------------------------------------------
 * hybrid_layer_step — a stack of independent attention layers over the same
 * batch, CSA and HCA interleaved (page section 3-2 item 2).  Each layer has its
 * own cache and queries; a CSA layer runs the selection of lca_csa_index_select
 * (its decode form: candidates, then the top-k) -> sparse_attn, an HCA layer
 * dense_attn, with the same kernels as the single calls.  Layers are independent
 * and each has its own workspace region.  All work is enqueued on `stream` in
 * three phases: the CSA layers' candidate index pass and their top-k selection
 * (up to 8 layers per launch), then the attention of every
 * layer, CSA and HCA in the same launches (up to 8 layers each), followed by the
 * sliding-window branch of every layer that has one (window > 0).  A layer's sink
 * (sink != NULL, as lca_attn_sink) is folded in by the kernel that writes the
 * layer's final result, after the window branch.  The attention cuts every
 * row, CSA or HCA, into pieces of P entries, one work-group each, merged in
 * piece order: P = 2048 / s rounded up to a multiple of 64, s = max(1, S / min(2L,
 * 32)) for L layers, where S = 32 for one query row per sequence, 32 / max_q for
 * up to 31 and 1 from 32 (8 layers of decode: P = 1024).  P depends on L and
 * max_q only, so the step is batch invariant (see Determinism).
 * ------------------------------------------------------------------------- */
enum lca_layer_kind { LCA_LAYER_CSA = 0, LCA_LAYER_HCA = 1 };
enum lca_idx_format { LCA_IDX_INT8 = 0, LCA_IDX_FP4 = 1 };
enum lca_kv_format { LCA_KV_BF16 = 0, LCA_KV_MIXED = 1 };

typedef struct lca_layer {
  int32_t kind;          /* LCA_LAYER_CSA or LCA_LAYER_HCA */
  int32_t ratio;         /* compression ratio: c (CSA) or m (HCA) */
  int32_t topk;          /* CSA only */
  int32_t max_entries;   /* host bound on entries per sequence in this layer */
  const lca_bf16* q;     /* [rows, heads, 128] */
  const int8_t* q_idx;   /* CSA: [rows, 64] */
  const lca_bf16* k_cmp; /* [ent_off[B], 128] */
  const lca_bf16* v_cmp; /* [ent_off[B], 128] */
  const int8_t* k_idx;   /* CSA: [ent_off[B], 64] */
  const int64_t* ent_off;/* [B+1] device */
  lca_bf16* out;         /* [rows, heads, 128] */
  float* lse;            /* [rows, heads] or NULL */
  int32_t* idx;          /* CSA out: [rows, topk] */
  int32_t* count;        /* CSA out: [rows] */
  /* optional sliding-window branch (window = 0: none), as lca_window_attn; needs lse */
  const lca_bf16* win_k; /* [win_off[B], 128] raw tokens of the state cache */
  const lca_bf16* win_v;
  const int64_t* win_off;  /* [B+1] device */
  const int64_t* win_pos0; /* [B] device: absolute position of each buffer's first row */
  int32_t window;
  const float* sink;     /* optional [heads] per-head sink logits (NULL: none), as lca_attn_sink */
  int32_t idx_format;    /* CSA: LCA_IDX_INT8, or LCA_IDX_FP4 (q_idx [rows, 32] / k_idx
                            [ent_off[B], 32] hold packed FP4 codes, as lca_csa_index_score_fp4) */
  int32_t kv_format;     /* LCA_KV_BF16, or LCA_KV_MIXED (k_cmp / v_cmp hold 192-byte mixed
                            rows, as lca_csa_sparse_attn_kv8; heads a multiple of 64) */
} lca_layer;

size_t lca_hybrid_workspace_bytes(const lca_layer* layers, int32_t n_layers, int32_t batch,
                                  int32_t max_q, int32_t heads);
int32_t lca_hybrid_layer_step(const lca_layer* layers, int32_t n_layers, const int64_t* q_off,
                              const int64_t* q_pos, int32_t batch, int32_t max_q, int32_t heads,
                              int32_t head_dim, float scale, void* ws, size_t ws_bytes,
                              void* stream);

/* ---------------------------------------------------------------------------
 * Phase timing of lca_hybrid_layer_step, for measurement.  While enabled, each
 * hybrid step on the current device records HIP events around its phases on the
 * caller's stream (not for use under graph capture).
 *   lca_hybrid_timing_enable(r / 0) switches it on / off for the current device; with
 *   r > 1 (at most 1000) a timed step launches its first index pass r times back to
 *   back (the same result each time), so that [0] below is that launch's own
 *   duration rather than one launch plus the dispatch gap after an event.
 *   lca_hybrid_timing_read(ms, n) waits for the last timed step and writes up to
 *   n durations in milliseconds: [0] the index pass (scores and candidates) of the
 *   first batch of CSA layers (per launch, the average of the r launches), [1] their
 *   top-k selection, [2] the attention of all
 *   layers with the split combine and the sliding-window branches (0 for a phase
 *   the step did not have).
 *   LCA_ERR_SHAPE if no timed step ran since enabling.
 * ------------------------------------------------------------------------- */
#define LCA_HYBRID_PHASES 3
int32_t lca_hybrid_timing_enable(int32_t enable);
int32_t lca_hybrid_timing_read(float* ms, int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* LCA_H */
