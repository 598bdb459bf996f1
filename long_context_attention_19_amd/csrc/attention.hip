// Softmax attention of H query heads over compressed entries of one shared KV
// head (head_dim 128): the sparse form for CSA (entries listed by the top-k) and
// the dense form for HCA (every visible entry).
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", sections 2-1 and 3-2 item 2: CSA attends a top-k of the compressed
// entries, HCA every compressed entry; both are softmax attention.
//
// All H heads of a query token read the same K/V rows, so a work-group holds up
// to 64 heads (the MFMA N dimension) and streams the entries once.  The
// contraction runs transposed, with entries / head dims as the MFMA M
// dimension and heads as N, using v_mfma_f32_16x16x32_bf16:
//     S^T[e][h] = sum_d K[e][d] Q[h][d]       (A = K tile from LDS, B = Q in VGPRs)
//     O^T[d][h] += sum_e V^T[d][e] P^T[e][h]  (A = V^T tile from LDS, B = P^T)
// In this form each lane holds one head: the row max of the online softmax needs
// only two cross-lane steps, the rescale factor is one scalar per lane, and the
// S^T accumulator already sits in the lanes that feed P^T to the second product
// (entries 4g..4g+3 of each 16-row block go to K-slots 8g..8g+7), so P never
// leaves registers.
//
// Per work-group: 256 threads = 4 waves.  With HG = min(H, 64)/16 head groups,
// wave w takes head group w % HG and entry sub-group w / HG.  A stage of 64
// entries (128 for H = 16) is copied from HBM into LDS by the waves' DMA while
// the previous stage is in use; softmax is fp32 in log2 units, P is rounded to
// bf16 for the MFMA and the running sum uses the rounded values.
//
// Splitting: a row's entries are cut into pieces of one size per launch, a multiple
// of the stage chosen so that a row at the host's bound (k for CSA, max_entries for
// HCA) takes `splits` pieces; each piece is a work-group and shorter rows take fewer.
// A single piece writes the final output; otherwise each writes (O, max, sum)
// partials and the combine kernel merges them in piece order.  The cut depends on
// the row's own entry count, the bound and `splits` only, never on other rows.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int AT_NT = 256;
constexpr int HD = 128;            // head_dim

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

int attn_auto_splits(int max_q) {
  if (max_q <= 1) return 32;
  if (max_q >= 32) return 1;
  return max(1, 32 / max_q);
}

size_t attn_ws_bytes(int rows, int heads, int splits) {
  if (splits <= 1) return 0;
  return align256((size_t)rows * splits * heads * HD * 4) +
         align256((size_t)rows * splits * heads * 8) + align256((size_t)rows * 8);
}

void attn_ws_carve(void* ws, int rows, int heads, int splits, AttnArgs& a) {
  if (splits <= 1 || ws == nullptr) {
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.part_info = nullptr;
    return;
  }
  char* p = reinterpret_cast<char*>(ws);
  a.part_o = reinterpret_cast<float*>(p);
  p += align256((size_t)rows * splits * heads * HD * 4);
  a.part_ml = reinterpret_cast<float2*>(p);
  p += align256((size_t)rows * splits * heads * 8);
  a.part_info = reinterpret_cast<int2*>(p);
}

// One piece size for every row of the launch, from the host's bound on the entry
// count: shorter rows get proportionally fewer pieces (a row beyond the bound widens
// its own pieces so that it still fits in `splits`).
__device__ __forceinline__ int piece_size(int n, int max_n, int splits, int stage) {
  const int want = (max(n, max_n) + splits - 1) / splits;
  return max(stage, (want + stage - 1) / stage * stage);
}

// ---------------------------------------------------------------------------------
// The K and V rows go from HBM straight into
// LDS with global_load_lds_dwordx4 (no register staging, no LDS stores issued by the
// waves), into two stage buffers: while one super-tile is in use the next one is in
// flight.  V is kept row-major in LDS and the V^T operand is read with
// ds_read_b64_tr_b16, which transposes 16-bit elements across each group of 16 lanes:
// lane i of the group receives element i % 4 of the 8-byte reads of lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4.  So lane 4e + q of group g points at
// entry 4g + e, dims 16db + 4q .. +3, and lane i then holds dim 16db + i of entries
// 4g .. 4g + 3: the V^T fragment of the same entry order as P^T.
//
// LDS layout: a 256-byte row is 16 slots of 16 bytes; one DMA instruction fills 4
// rows (64 lanes x 16 bytes, contiguous), so rows are not padded and the slots are
// permuted instead: K row r keeps dims 8c..8c+7 in slot c ^ (r & 15) (the 16 rows a
// K-fragment read touches land in 16 distinct slots), V row r in slot c ^ 2(r & 7)
// (the 8 rows x 32 bytes of a transposed read's half-wave are distinct slots).
//
// The DMA is issued from inline assembly so that the compiler does not order LDS
// reads behind it: the transposed reads carry no alias information and the compiler
// would otherwise wait for every DMA in flight, the next stage's included.  The
// waits are explicit (vmcnt), and no compiler-visible global load is in flight while
// the pipeline runs: the sparse form copies a chunk of entry ids to LDS first.
constexpr int AT_SUB64 = 2;        // 64 heads: 32-entry sub-tiles per wave per stage
constexpr int AT_NB64 = 2;         // 64 heads: stage buffers
constexpr int AT_IDS = 2048;       // entry ids staged in LDS per chunk (sparse form)

// MODE: 0 dense (HCA), 1 sparse (CSA), 2 either, per layer of the launch
template <int ST, int NB, int MODE, int KV>
struct AttnDmaSmem {
  alignas(256) i32x4 k[NB][ST * 16];   // 256-byte aligned: attn_stage XORs slot bits
  alignas(256) i32x4 v[NB][ST * 16];
  int ids[MODE != 0 ? AT_IDS : 1];
};
// Mixed KV rows (dims 0..63 FP8, 64..127 bf16): per stage buffer the FP8 halves as
// fetched (64 B rows) and the bf16 halves (128 B rows, slots permuted as the bf16
// tiles); the FP8 halves are converted once per stage into one bf16 tile (128 B rows).
template <int ST, int NB, int MODE>
struct AttnDmaSmem<ST, NB, MODE, 1> {
  alignas(256) i32x4 k8[NB][ST * 4];
  alignas(256) i32x4 v8[NB][ST * 4];
  alignas(256) i32x4 khi[NB][ST * 8];
  alignas(256) i32x4 vhi[NB][ST * 8];
  alignas(256) i32x4 klo[ST * 8];
  alignas(256) i32x4 vlo[ST * 8];
  int ids[MODE != 0 ? AT_IDS : 1];
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// 64 lanes x 16 bytes from seq + voff (per lane) into LDS at lds .. lds + 1023.
// seq and lds are the same in every lane; they are read from the first lane so that
// the compiler keeps them in scalar registers.
__device__ __forceinline__ void dma16(const void* seq_any, uint32_t voff, uint32_t lds_any) {
  const uint64_t sp = reinterpret_cast<uint64_t>(seq_any);
  // readfirstlane returns int: convert through uint32_t so the low half is not
  // sign-extended into the high half
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sp >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sp);
  const uint64_t su = ((uint64_t)hi << 32) | (uint64_t)lo;
  const void* seq = reinterpret_cast<const void*>(su);
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_any);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(seq), "s"(lds)
      : "memory");
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS reads done and work-group barrier, also a compiler barrier for memory
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// max / sum over the 4 lanes that share l16 (lanes l16, l16+16, l16+32, l16+48):
// v_permlane32_swap exchanges the two 32-lane halves, v_permlane16_swap the odd and
// even 16-lane rows, both without LDS
__device__ __forceinline__ float lanes4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lanes4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Attention sink ("DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence Review", section 3-2 item 2 names one; reading: a per-head logit z
// in the softmax normalisation with a zero value).  Folded into a finished result
// whose log-sum-exp is lse (natural log): the output is multiplied by the returned
// 1 / (1 + e^(z - lse)) and lse becomes log(e^lse + e^z).
__device__ __forceinline__ float sink_fold(float lse, float z, float* lse_out) {
  const float mx = fmaxf(lse, z);
  if (mx == -INFINITY) {   // nothing attended and no sink
    *lse_out = -INFINITY;
    return 0.f;
  }
  *lse_out = mx + log1pf(__expf(-fabsf(lse - z)));
  return 1.f / (1.f + __expf(z - lse));   // z - lse = +inf gives 0, -inf gives 1
}

// The running max of the online softmax moves only when a block's max exceeds it
// by more than this (log2 units): until then the weights are taken against the
// stale max, so they stay below 2^8, and the rescale of O and the sum (32 + 1
// multiplies per lane) is skipped.  O, the sum and the max stay consistent, so the
// result and the log-sum-exp are those of the exact max.
constexpr float AT_MAX_SLACK = 8.f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One stage of the online softmax attention for the 16 heads of this wave (head
// l16 of the lane) over its SUB 32-entry sub-tiles starting at stage row el_base
// (a multiple of 32), treated as one block of 32*SUB entries: S^T = K Q^T for every
// sub-tile first (independent MFMA chains), one running-max update for the block,
// then O^T += V^T P^T with the V^T operand read transposed from the stage's V tile.
// Entries at or past e1 are masked (their rows were fetched but hold repeats; their
// weights are exactly 0).  The caller guarantees the block's first entry is valid.
// The running max is kept in scaled log2 units; the exponent is one fma, v_exp_f32
// without range fix-up (a weight below 2^-126 flushes to 0, as it would in bf16).
// The lane's share of the sum adds the bf16-rounded weights in pairs (v_dot2 with
// ones).
//
// LDS addresses: both stage buffers start on 256-byte boundaries, so the slot
// permutation of a row (bits 4..7 of the address) is an XOR on a per-lane base:
// K fragment ks of row r sits at base_k ^ (ks << 6), V^T fragment db at
// base_v ^ (db << 5), and the sub-tile / half offsets are instruction immediates.
template <int SUB>
__device__ __forceinline__ void attn_stage(const i32x4* kb, const char* vbase, int el_base, int tb,
                                           int e1, const bf16x8 (&qf)[4], f32x4 (&o)[8],
                                           float& m_run, float& l_run, float scale_log2, int l16,
                                           int g) {
  typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  // K: row el_base + 32 sub + 16 rb + l16 keeps dims 8(4ks + g) .. in slot (4ks + g) ^ l16
  const uint32_t base_k = lds_addr(kb) + (uint32_t)(el_base + l16) * 256u + ((uint32_t)(g ^ l16) << 4);
  f32x4 sacc[SUB][2];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) sacc[sub][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t ak = base_k ^ ((uint32_t)ks << 6);
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(lds_i32x4*)(size_t)(ak + (sub * 32 + rb * 16) * 256));
        sacc[sub][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[sub][rb], 0, 0, 0);
      }
  }
  float x[SUB * 8];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[sub * 8 + rb * 4 + i] = sacc[sub][rb][i];
  const int ev0 = tb + el_base;
  if (ev0 + 32 * SUB > e1) {   // the block crosses the end: mask entries >= e1
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (ev0 + sub * 32 + rb * 16 + 4 * g + i >= e1) x[sub * 8 + rb * 4 + i] = -INFINITY;
  }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < SUB * 8; ++i) mx = __builtin_elementwise_maximum(mx, x[i]);
  mx = lanes4_max(mx) * scale_log2;            // scale > 0: max commutes with it
  // finite: the block has a valid entry; true on the first block (m_run = -inf)
  const bool raise = mx > m_run + AT_MAX_SLACK;
  if (__any(raise)) {
    const float m_new = raise ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 first, 1 if kept
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;
    l_run *= alpha;
    m_run = m_new;
  }
  const float m_use = m_run;
  bf16x8 pf[SUB];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pf[sub][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(x[sub * 8 + i], scale_log2, -m_use));
  const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
  float psum = l_run;
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[sub][2 * i], pf[sub][2 * i + 1]}, one2, psum,
                                             false);
  l_run = psum;
  // V: row r = el_base + 32 sub + 16 hh + 4g + (l16 >> 2), r & 7 = (4g + (l16 >> 2)) & 7,
  // keeps dims 8c .. in slot c ^ 2(r & 7); lane q = l16 & 3 reads dims 16db + 4q .. +3
  const int r7 = (4 * g + (l16 >> 2)) & 7;
  const int q = l16 & 3;
  const uint32_t base_v = lds_addr(vbase) + (uint32_t)(el_base + 4 * g + (l16 >> 2)) * 256u +
                          ((uint32_t)r7 << 5) + ((uint32_t)(q >> 1) << 4) + (uint32_t)(q & 1) * 8u;
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t av = (base_v ^ ((uint32_t)db << 5)) + (uint32_t)sub * 32u * 256u;
      const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)av);
      const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(av + 16 * 256));
      const bf16x8 vf = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[sub], o[db], 0, 0, 0);
    }
}

// Mixed KV rows: 128-byte half rows (dims 0..63 converted from FP8 in `lo`, dims
// 64..127 as fetched in `hi`, both bf16).  Slot permutations of a half row (8 slots of
// 16 bytes): K row r keeps dims 8c .. 8c+7 of its half in slot c ^ ((r >> 1) & 7), so
// the 16 rows of a K-fragment read cover both row parities x 8 slots (every bank once);
// V row r in slot c ^ 2((r >> 1) & 3), so the 8 rows x 32 bytes of a transposed read's
// half-wave land on distinct banks.
__device__ __forceinline__ uint32_t kv8_kslot(int r, int c) { return (uint32_t)(c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ uint32_t kv8_vslot(int r, int c) { return (uint32_t)(c ^ (((r >> 1) & 3) << 1)); }

// attn_stage over mixed KV rows: the same arithmetic, with K fragments ks = 0, 1 and
// V^T fragments db = 0..3 read from the `lo` tiles and the others from the `hi` tiles.
template <int SUB>
__device__ __forceinline__ void attn_stage_kv8(const i32x4* klo, const i32x4* khi,
                                               const i32x4* vlo, const i32x4* vhi, int el_base,
                                               int tb, int e1, const bf16x8 (&qf)[4],
                                               f32x4 (&o)[8], float& m_run, float& l_run,
                                               float scale_log2, int l16, int g) {
  typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  // K row el_base + 32 sub + 16 rb + l16: (row >> 1) & 7 = (l16 >> 1) & 7
  const uint32_t koff = (uint32_t)(el_base + l16) * 128u + ((uint32_t)(g ^ ((l16 >> 1) & 7)) << 4);
  const uint32_t bk[2] = {lds_addr(klo) + koff, lds_addr(khi) + koff};
  f32x4 sacc[SUB][2];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) sacc[sub][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t ak = bk[ks >> 1] ^ ((uint32_t)(ks & 1) << 6);
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(lds_i32x4*)(size_t)(ak + (sub * 32 + rb * 16) * 128));
        sacc[sub][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[sub][rb], 0, 0, 0);
      }
  }
  float x[SUB * 8];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[sub * 8 + rb * 4 + i] = sacc[sub][rb][i];
  const int ev0 = tb + el_base;
  if (ev0 + 32 * SUB > e1) {
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (ev0 + sub * 32 + rb * 16 + 4 * g + i >= e1) x[sub * 8 + rb * 4 + i] = -INFINITY;
  }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < SUB * 8; ++i) mx = __builtin_elementwise_maximum(mx, x[i]);
  mx = lanes4_max(mx) * scale_log2;
  const bool raise = mx > m_run + AT_MAX_SLACK;
  if (__any(raise)) {
    const float m_new = raise ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;
    l_run *= alpha;
    m_run = m_new;
  }
  const float m_use = m_run;
  bf16x8 pf[SUB];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pf[sub][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(x[sub * 8 + i], scale_log2, -m_use));
  const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
  float psum = l_run;
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[sub][2 * i], pf[sub][2 * i + 1]}, one2, psum,
                                             false);
  l_run = psum;
  // V row R = el_base + 32 sub + 16 hh + 4g + (l16 >> 2): (R >> 1) & 3 = (2g + (l16 >> 3)) & 3
  const int m2 = (2 * g + (l16 >> 3)) & 3;
  const int q = l16 & 3;
  const uint32_t voff = (uint32_t)(el_base + 4 * g + (l16 >> 2)) * 128u + ((uint32_t)m2 << 5) +
                        ((uint32_t)(q >> 1) << 4) + (uint32_t)(q & 1) * 8u;
  const uint32_t bv[2] = {lds_addr(vlo) + voff, lds_addr(vhi) + voff};
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t av = (bv[db >> 2] ^ ((uint32_t)(db & 3) << 5)) + (uint32_t)sub * 32u * 128u;
      const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)av);
      const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(av + 16 * 128));
      const bf16x8 vf = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[sub], o[db], 0, 0, 0);
    }
}

// The K and V row pieces of one DMA instruction: lane (r, slot l16) of instruction
// u fetches row r's 16-byte chunk l16 ^ (r & 15) for K and l16 ^ 2(r & 7) for V.
__device__ __forceinline__ void attn_issue_rows(const char* kseq, const char* vseq,
                                                uint32_t row_off, int r, int l16, uint32_t k_lds,
                                                uint32_t v_lds) {
  const uint32_t ck = (uint32_t)(l16 ^ (r & 15)) << 4;
  const uint32_t cv = (uint32_t)(l16 ^ ((r & 7) << 1)) << 4;
  dma16(kseq, row_off + ck, k_lds);
  dma16(vseq, row_off + cv, v_lds);
}

// ES entry sub-groups of waves; each wave takes SUB consecutive 32-entry sub-tiles of
// every stage, so a stage covers 32*ES*SUB entries.  KV = 1: mixed KV rows (dims
// 0..63 FP8 E4M3, 64..127 bf16, 192 bytes); each stage's FP8 halves are converted to
// bf16 in LDS by the whole work-group before the waves use the stage.
template <int ES, int SUB, int NB, int MODE, int KV>
__global__ __launch_bounds__(AT_NT) void attn_dma_kernel(AttnBatch ab) {
  // grid x = item (query row slot, then layer x head block), padded to an odd count;
  // grid y = piece.  Consecutive work-groups go to the XCDs in turn, so with an odd
  // item count the pieces of one item land on different XCDs, and the work-groups of
  // the first pieces (present in every row) are dispatched before the later ones.
  const int item = blockIdx.x;
  if (item >= ab.items) return;
  const int lz = item / ab.rows_grid;            // layer x head block
  const int gy = item - lz * ab.rows_grid;       // query row slot
  const AttnArgs& a = ab.a[lz / ab.head_blocks];
  const int s = blockIdx.y;
  if (s >= a.splits) return;                     // a layer with fewer pieces per row
  const bool sparse = MODE == 2 ? a.idx != nullptr : MODE == 1;   // uniform
  constexpr int ST = 32 * ES * SUB;             // entries per super-tile (stage)
  constexpr int IPT = AT_IDS / AT_NT;           // entry ids per thread and chunk
  const int t = threadIdx.x;
  const int kk = a.k;
  // the piece as far as it is known before the entry count: exact when the count is
  // within the bound (always for the sparse form)
  const int per_g = piece_size(0, a.max_n, a.splits, ST);
  const int e0_g = s * per_g;
  // Sparse rows whose ids are also stored by grid row: the first chunk of ids is
  // requested now, before the row bounds (a row's ids by row would wait for them).
  int idv[MODE != 0 ? IPT : 1];
  const bool ids_gy = MODE != 0 && sparse && a.idx_gy != nullptr;   // uniform
  if (ids_gy) {
    const int cnt = min(min(e0_g + per_g, kk), e0_g + AT_IDS) - e0_g;
    const int* src = a.idx_gy + (int64_t)gy * kk + e0_g;
    if (cnt > 0) {
#pragma unroll
      for (int u = 0; u < IPT; ++u) idv[u] = src[min(t + AT_NT * u, cnt - 1)];
    }
  }
  constexpr int HG = 4 / ES;                    // head groups of 16 per work-group
  constexpr int NU = ST / 16;                   // DMA instructions per wave per matrix
  static_assert(NU >= 1 && NU <= 8 && AT_IDS % ST == 0, "stage size");
  static_assert(KV == 0 || (ES == 1 && ST == 64), "mixed KV rows: 64-entry stages, 64 heads");
  // DMA instructions per wave per stage: bf16 rows 2 x NU; mixed rows, per matrix, one
  // for the 16 FP8 half rows of the wave and two for its 16 bf16 half rows
  constexpr int DPS = KV ? 6 : 2 * NU;
  constexpr int D = NB - 1;                     // stages in flight ahead of the one in use
  static_assert(NB >= 2 && D * DPS < 64, "pipeline depth");
  __shared__ AttnDmaSmem<ST, NB, MODE, KV> sm;

  // The loads that set up a work-group form a short dependency chain; the query,
  // the first entry ids and the first stages' rows are issued as soon as their
  // addresses are known, before the row's entry count (and so the exact end of the
  // piece) is back.  Rows past the end are read but masked in the softmax.
  const int b = gy / a.max_q;
  const int qi = gy - b * a.max_q;
  // row bounds and counts as scalar loads: a vector load here would be waited for
  // with the entry ids and the query
  const int64_t r0 = ld_const(a.q_off + b), r1 = ld_const(a.q_off + b + 1);
  int64_t e_base = ld_const(a.ent_off + b);
  const int64_t e_end = ld_const(a.ent_off + b + 1);
  // both pairs in flight together (otherwise the entry range is requested only after
  // the padding test below)
  asm volatile("" ::"s"(r0), "s"(r1), "s"(e_base), "s"(e_end));
  const int64_t nq = r1 - r0;
  int64_t n_seq = e_end - e_base;
  if (qi >= nq) {   // a padding row slot: nothing for the combine either
    if (s == 0 && threadIdx.x == 0 && a.part_info) a.part_info[gy] = make_int2(-1, 0);
    return;
  }
  // a piece that starts past the sequence's entries (or past k) exists for no row of
  // the sequence: leave before the row's count is read (pieces only widen beyond the bound)
  if (s > 0 && (int64_t)s * piece_size(0, a.max_n, a.splits, ST) >=
                   (sparse ? min(n_seq, (int64_t)a.k) : n_seq))
    return;
  const int64_t row = r0 + qi;
  // the row's entry count: only needed after the first DMAs are issued
  int n_raw = sparse ? ld_const(a.count + row) : (int)min(ld_const(a.q_pos + row) / a.ratio, (int64_t)INT32_MAX);
  if (MODE == 0 && a.win_pos0 != nullptr) {
    // sliding window: the buffer's tokens at positions [p - window, p), as buffer
    // rows [lo, hi); the rows before lo are skipped by moving the sequence base
    const int64_t p = ld_const(a.q_pos + row), pos0 = ld_const(a.win_pos0 + b);
    const int64_t lo = min(max(p - a.window, pos0) - pos0, max(n_seq, (int64_t)0));
    const int64_t hi = max(min(p, pos0 + n_seq) - pos0, lo);
    e_base += lo;
    n_seq -= lo;
    n_raw = (int)(hi - lo);
  }
  const int max_n = a.max_n;
  const int splits = a.splits;
  const int h0 = (lz % ab.head_blocks) * ab.hpb;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int hg = w % HG;
  const int es = w / HG;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int head = h0 + hg * 16 + l16;
  // kernel arguments used inside the pipeline are read once: the asm memory clobbers
  // would otherwise make the compiler reload them
  const float scale_log2 = a.scale_log2;

  bf16x8 qf[4];
  {
    const i32x4* qp = reinterpret_cast<const i32x4*>(a.q + (row * a.heads + head) * HD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qp[ks * 4 + g]);
  }
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // wave w fills rows w*ST/4 .. +ST/4 of a stage; DMA instruction u covers 4 of them
  const int wrow0 = w * (ST / 4);
  const int my_row = lane >> 4;
  const int id_max = (int)min(n_seq, (int64_t)ATTN_MAX_SEQ) - 1;
  const int64_t row_bytes = KV ? KV8_ROW_BYTES : HD * 2;
  const char* kseq = reinterpret_cast<const char*>(a.kc) + e_base * row_bytes;
  const char* vseq = reinterpret_cast<const char*>(a.vc) + e_base * row_bytes;
  uint32_t k_lds0, v_lds0;
  if constexpr (KV) {   // FP8 half rows of this wave; the bf16 half rows are offset below
    k_lds0 = lds_addr(&sm.k8[0][wrow0 * 4]);
    v_lds0 = lds_addr(&sm.v8[0][wrow0 * 4]);
  } else {
    k_lds0 = lds_addr(&sm.k[0][wrow0 * 16]);
    v_lds0 = lds_addr(&sm.v[0][wrow0 * 16]);
  }
  constexpr uint32_t BUF_BYTES = ST * 256;

  // the end of the piece as far as it is known before the entry count: where reads
  // stay valid
  const int end_g = n_seq <= 0 ? e0_g   // an empty sequence: nothing to fetch
                    : sparse ? min(e0_g + per_g, kk)
                             : (int)min((int64_t)e0_g + per_g, (int64_t)id_max + 1);

  // issue the DMA of the stage starting at entry tb into buffer buf; rows past
  // e_last repeat row e_last (cached, and masked in the softmax)
  auto row_id = [&](int r, int tb, int cbase, int e_last) __attribute__((always_inline)) {
    // sparse: the staged ids are clamped and run on past the chunk's end (load_ids)
    if (MODE != 0 && sparse) return (uint32_t)sm.ids[tb + r - cbase];
    return (uint32_t)min(max(min(tb + r, e_last), 0), id_max);
  };
  // Every row id of the stage is read first (LDS, one wait), then the DMAs are issued:
  // the DMA's inline assembly clobbers memory, so an id read placed after one would
  // wait on its own.
  auto issue = [&](int buf, int tb, int cbase, int e_last) __attribute__((always_inline)) {
    if constexpr (KV) {
      // FP8 halves: 16 rows of 64 bytes, lane -> (row lane / 4, chunk lane % 4);
      // bf16 halves: 2 x 8 rows of 128 bytes, lane -> (row lane / 8, slot lane % 8)
      const uint32_t rid0 = row_id(wrow0 + (lane >> 2), tb, cbase, e_last);
      uint32_t rid[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) rid[u] = row_id(wrow0 + 8 * u + (lane >> 3), tb, cbase, e_last);
      {
        const uint32_t off = rid0 * KV8_ROW_BYTES + (uint32_t)(lane & 3) * 16u;
        dma16(kseq, off, k_lds0 + buf * (ST * 64));
        dma16(vseq, off, v_lds0 + buf * (ST * 64));
      }
      const uint32_t khi0 = lds_addr(&sm.khi[buf][0]), vhi0 = lds_addr(&sm.vhi[buf][0]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = wrow0 + 8 * u + (lane >> 3);
        const uint32_t base = rid[u] * KV8_ROW_BYTES + 64u;
        const int sl = lane & 7;
        dma16(kseq, base + kv8_kslot(r, sl) * 16u, khi0 + (uint32_t)(wrow0 + 8 * u) * 128u);
        dma16(vseq, base + kv8_vslot(r, sl) * 16u, vhi0 + (uint32_t)(wrow0 + 8 * u) * 128u);
      }
    } else {
      uint32_t rid[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) rid[u] = row_id(wrow0 + 4 * u + my_row, tb, cbase, e_last);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int r = wrow0 + 4 * u + my_row;
        attn_issue_rows(kseq, vseq, rid[u] * 256u, r, l16,
                        k_lds0 + buf * BUF_BYTES + u * 1024, v_lds0 + buf * BUF_BYTES + u * 1024);
      }
    }
  };
  // copy the entry ids [cbase, cend) to LDS (sparse form; nothing else in flight),
  // clamped to the sequence's rows (a padding id reads row 0, masked in the softmax),
  // and the slots past cend repeat the last id: a stage's rows then need no clamp
  auto store_ids = [&](int (&v)[MODE != 0 ? IPT : 1]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < IPT; ++u) v[u] = min(max(v[u], 0), id_max);
    __syncthreads();   // the previous chunk's ids are no longer read
#pragma unroll
    for (int u = 0; u < IPT; ++u) sm.ids[t + AT_NT * u] = v[u];
    __syncthreads();
  };
  auto load_ids = [&](int cbase, int cend) __attribute__((always_inline)) {
    const int* src = ids_gy ? a.idx_gy + (int64_t)gy * kk + cbase : a.idx + row * kk + cbase;
    const int cnt = cend - cbase;   // >= 1
    int v[MODE != 0 ? IPT : 1];
#pragma unroll
    for (int u = 0; u < IPT; ++u) v[u] = src[min(t + AT_NT * u, cnt - 1)];   // all in flight
    store_ids(v);
  };
  // first stages of a chunk, one per buffer; returns the number issued
  auto prologue = [&](int cbase, int cend) __attribute__((always_inline)) {
    const int nst = (cend - cbase + ST - 1) / ST;
    const int p = min(NB, nst);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j < p) issue(j, cbase + j * ST, cbase, cend - 1);
    return p;
  };

  int issued = 0;
  int cb0 = e0_g;
  const int cend0 = sparse ? min(end_g, e0_g + AT_IDS) : end_g;
  if (cend0 > e0_g) {
    if (MODE != 0 && sparse) {
      if (ids_gy) store_ids(idv);   // requested at the start
      else load_ids(e0_g, cend0);
    }
    issued = prologue(e0_g, cend0);
  }
  // the query is needed now: the compiler's wait for it lands here, behind the DMAs
  asm volatile("" : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]));

  const int n = n_seq <= 0 ? 0 : sparse ? max(0, min(n_raw, kk)) : (int)min((int64_t)n_raw, n_seq);
  const int per = piece_size(n, max_n, splits, ST);
  const int nsp = n > 0 ? (n + per - 1) / per : 1;
  if (s == 0 && t == 0 && a.part_info) a.part_info[gy] = make_int2((int)row, nsp);
  if (s >= nsp || per != per_g) {
    // outside the row, or a row beyond the bound: drop what was fetched speculatively
    wait_vm<0>();
    lds_barrier();
    issued = 0;
    if (s >= nsp) return;
  }
  const int e0 = s * per;
  const int e1 = min(e0 + per, n);

  auto compute = [&](int buf, int tb) __attribute__((always_inline)) {
    if constexpr (KV) {
      // the stage's FP8 halves to bf16, once for all waves: thread t converts the 16
      // dims 16 (t % 4) .. of K and V row t / 4 into two slots of the lo tiles
      const int r = t >> 2, ch = t & 3;
      const i32x4 k8 = sm.k8[buf][r * 4 + ch];
      const i32x4 v8 = sm.v8[buf][r * 4 + ch];
      i32x4 klo[2], vlo[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const int word = 2 * h + d;
          klo[h][2 * d] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k8[word], 1.f, false));
          klo[h][2 * d + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k8[word], 1.f, true));
          vlo[h][2 * d] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v8[word], 1.f, false));
          vlo[h][2 * d + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v8[word], 1.f, true));
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sm.klo[r * 8 + kv8_kslot(r, 2 * ch + h)] = klo[h];
        sm.vlo[r * 8 + kv8_vslot(r, 2 * ch + h)] = vlo[h];
      }
      lds_barrier();
      if (tb < e1)
        attn_stage_kv8<SUB>(sm.klo, sm.khi[buf], sm.vlo, sm.vhi[buf], 0, tb, e1, qf, o, m_run,
                            l_run, scale_log2, l16, g);
    } else {
      if (tb + es * SUB * 32 < e1)   // this wave's block has a valid entry
        attn_stage<SUB>(sm.k[buf], reinterpret_cast<const char*>(sm.v[buf]), es * SUB * 32, tb,
                        e1, qf, o, m_run, l_run, scale_log2, l16, g);
    }
  };

  // Per stage: wait for this stage's DMA (the later stages' may stay outstanding),
  // barrier, compute, barrier, then reuse the buffer for the stage NB ahead.
  for (int cbase = e0; cbase < e1; cbase += (sparse ? AT_IDS : (1 << 30))) {
    const int cend = sparse ? min(cbase + AT_IDS, e1) : e1;
    const int nst = (cend - cbase + ST - 1) / ST;
    if (cbase != cb0 || issued == 0) {
      wait_vm<0>();
      if (MODE != 0 && sparse) load_ids(cbase, cend);
      else lds_barrier();
      issued = prologue(cbase, cend);
      cb0 = cbase;
    }
    // stage j uses buffer j % NB; unrolled by NB so that the buffer (and with it every
    // LDS address of the stage) is a compile-time constant
    for (int j0 = 0; j0 < nst; j0 += NB) {
#pragma unroll
      for (int buf = 0; buf < NB; ++buf) {
        const int j = j0 + buf;
        if (j < nst) {
          const int ahead = issued - 1 - j;   // stages issued after stage j
          if (NB > 3 && ahead >= 3) wait_vm<(NB > 3 ? 3 : 0) * DPS>();
          else if (NB > 2 && ahead == 2) wait_vm<(NB > 2 ? 2 : 0) * DPS>();
          else if (ahead == 1) wait_vm<DPS>();
          else wait_vm<0>();
          lds_barrier();
          compute(buf, cbase + j * ST);
          lds_barrier();
          if (j + NB < nst) {
            issue(buf, cbase + (j + NB) * ST, cbase, cend - 1);
            issued = j + NB + 1;
          }
        }
      }
    }
  }
  wait_vm<0>();   // stages fetched past the end

  l_run = lanes4_sum(l_run);

  if constexpr (ES > 1) {
    // merge the ES entry sub-groups of each head group; the stage buffers are free
    static_assert(sizeof(sm.k) >= 4 * 16 * HD * 4, "merge buffer");
    float* merge_o = reinterpret_cast<float*>(sm.k[0]);        // [4][16][HD]
    float* merge_ml = reinterpret_cast<float*>(sm.v[0]);       // [4][16][2]
    __syncthreads();
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f32x4*>(&merge_o[(w * 16 + l16) * HD + db * 16 + 4 * g]) = o[db];
    if (g == 0) {
      merge_ml[(w * 16 + l16) * 2] = m_run;
      merge_ml[(w * 16 + l16) * 2 + 1] = l_run;
    }
    __syncthreads();
    if (es != 0) return;
    float mm = -INFINITY;
#pragma unroll
    for (int q = 0; q < ES; ++q) mm = fmaxf(mm, merge_ml[((hg + q * HG) * 16 + l16) * 2]);
    float ll = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < ES; ++q) {
      const int wq = hg + q * HG;
      const float mq = merge_ml[(wq * 16 + l16) * 2];
      const float f = (mq == -INFINITY) ? 0.f : exp2f(mq - mm);
      ll += merge_ml[(wq * 16 + l16) * 2 + 1] * f;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        o[db] += *reinterpret_cast<const f32x4*>(&merge_o[(wq * 16 + l16) * HD + db * 16 + 4 * g]) * f;
    }
    m_run = mm;
    l_run = ll;
  }

  if (nsp == 1 && MODE == 0 && a.merge) {
    // one softmax over this result and the one already in out / lse: weights
    // exp(lse - max) of the two normalised outputs
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse_w = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
    uint16_t* op = a.out + (row * a.heads + head) * HD;
    float* lp = a.lse + row * a.heads + head;
    const float lse_c = *lp;
    const float mx = fmaxf(lse_c, lse_w);
    const float wc = mx == -INFINITY ? 0.f : __expf(lse_c - mx);
    const float ww = mx == -INFINITY ? 0.f : __expf(lse_w - mx);
    const float den = wc + ww;
    float rden = den > 0.f ? 1.f / den : 0.f;
    float lse_new = den > 0.f ? mx + __logf(den) : -INFINITY;
    if (a.sink) rden *= sink_fold(lse_new, a.sink[head], &lse_new);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint2 ck = *reinterpret_cast<const uint2*>(op + db * 16 + 4 * g);
      const float c0 = bf16_bits_to_f32(ck.x & 0xffffu), c1 = bf16_bits_to_f32(ck.x >> 16);
      const float c2 = bf16_bits_to_f32(ck.y & 0xffffu), c3 = bf16_bits_to_f32(ck.y >> 16);
      uint2 pk;
      pk.x = f32_to_bf16_bits((wc * c0 + ww * o[db][0] * inv) * rden) |
             (f32_to_bf16_bits((wc * c1 + ww * o[db][1] * inv) * rden) << 16);
      pk.y = f32_to_bf16_bits((wc * c2 + ww * o[db][2] * inv) * rden) |
             (f32_to_bf16_bits((wc * c3 + ww * o[db][3] * inv) * rden) << 16);
      *reinterpret_cast<uint2*>(op + db * 16 + 4 * g) = pk;
    }
    if (g == 0) *lp = lse_new;
  } else if (nsp == 1) {
    float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float lse_v = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
    if (a.sink) inv *= sink_fold(lse_v, a.sink[head], &lse_v);
    uint16_t* op = a.out + (row * a.heads + head) * HD;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(o[db][0] * inv) | (f32_to_bf16_bits(o[db][1] * inv) << 16);
      pk.y = f32_to_bf16_bits(o[db][2] * inv) | (f32_to_bf16_bits(o[db][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + db * 16 + 4 * g) = pk;
    }
    if (a.lse && g == 0) a.lse[row * a.heads + head] = lse_v;
  } else {
    const int64_t slot = ((int64_t)gy * a.splits + s) * a.heads + head;   // by grid row
    float* pp = a.part_o + slot * HD;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(pp + db * 16 + 4 * g) = o[db];
    if (g == 0) a.part_ml[slot] = make_float2(m_run, l_run);
  }
}

// Merge split partials: a work-group per (row slot, layer x head block, 8 heads), the
// item numbering of the attention grid times the 8-head groups of a block.  The row and
// its piece count come from a record the attention's piece-0 work-groups wrote.  The
// partials sit by grid row, so a sparse layer's pieces (as many as its launch has, up to
// U; a full row has them all) are requested beside the record; a dense layer's rows
// hold fewer pieces the shorter they are, so its pieces are requested once the count is
// known.  A work-group takes H heads (8, or 2 when the launch has few rows, so that
// its groups spread over more CUs: each group's loads are then a quarter as many).
// Thread t takes head t / 32 of the group and dims 4 (t % 32) .. +3, and loads
// the (max, sum) and O of U pieces at a time, all in flight together; the pieces are
// added in piece order against a running maximum, so the result does not depend on
// load timing, nor on H.
template <int U, int H>
__global__ __launch_bounds__(32 * H) void attn_combine_kernel(AttnBatch ab, int groups) {
  const int item = blockIdx.x / groups;
  const int hgrp = blockIdx.x - item * groups;
  if (item >= ab.items) return;
  const int lz = item / ab.rows_grid;
  const int gy = item - lz * ab.rows_grid;
  const AttnArgs& a = ab.a[lz / ab.head_blocks];
  if (a.splits <= 1 || a.part_info == nullptr) return;
  const int t = threadIdx.x;
  const int head = (lz % ab.head_blocks) * ab.hpb + hgrp * H + t / 32;
  const int d0 = (t % 32) * 4;
  const int64_t base = (int64_t)gy * a.splits * a.heads + head;
  float2 ml[U];
  f32x4 ov[U];
  // pieces j0 .. j0 + U - 1, those below `lim` (past it: not loaded, masked below)
  auto fetch = [&](int j0, int lim) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < lim) {
        const int64_t slot = base + (int64_t)(j0 + u) * a.heads;
        ml[u] = a.part_ml[slot];
        ov[u] = *reinterpret_cast<const f32x4*>(a.part_o + slot * HD + d0);
      }
    }
  };
  const bool spec = a.idx != nullptr;   // uniform
  if (spec) fetch(0, a.splits);
  const int2 info = a.part_info[gy];
  const int nsp = info.y;
  if (nsp <= 1) return;
  const int64_t row = info.x;
  float mt = -INFINITY, lt = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nsp; j0 += U) {
    if (j0 > 0 || !spec) fetch(j0, nsp);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u >= nsp) {   // a piece the row does not have
        ml[u] = make_float2(-INFINITY, 0.f);
        ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    float mb = mt;   // piece j0 exists and holds an entry: mb is finite
#pragma unroll
    for (int u = 0; u < U; ++u) mb = fmaxf(mb, ml[u].x);
    const float r = exp2f(mt - mb);   // 0 on the first round
    lt *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = exp2f(ml[u].x - mb);   // 0 for pieces past the end
      lt += ml[u].y * f;
      acc += ov[u] * f;
    }
    mt = mb;
  }
  float inv = 1.f / lt;
  float lse_v = (mt + log2f(lt)) * 0.69314718055994530942f;
  if (a.sink) inv *= sink_fold(lse_v, a.sink[head], &lse_v);
  uint2 pk;
  pk.x = f32_to_bf16_bits(acc[0] * inv) | (f32_to_bf16_bits(acc[1] * inv) << 16);
  pk.y = f32_to_bf16_bits(acc[2] * inv) | (f32_to_bf16_bits(acc[3] * inv) << 16);
  *reinterpret_cast<uint2*>(a.out + (row * a.heads + head) * HD + d0) = pk;
  if (a.lse && d0 == 0) a.lse[row * a.heads + head] = lse_v;
}

// lca_attn_sink: the sink folded into a finished result, in place.  A thread takes
// 8 dims of one (row, head); 16 threads per (row, head).
__global__ __launch_bounds__(256) void attn_sink_kernel(uint16_t* __restrict__ out,
                                                        float* __restrict__ lse,
                                                        const float* __restrict__ sink,
                                                        int64_t rows, int heads) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = t >> 4;   // (row, head)
  if (rh >= rows * heads) return;
  const int head = (int)(rh % heads);
  float lse_v;
  const float f = sink_fold(lse[rh], sink[head], &lse_v);
  uint4* op = reinterpret_cast<uint4*>(out + rh * HD) + (t & 15);
  const uint4 v = *op;
  uint4 r;
  r.x = f32_to_bf16_bits(bf16_bits_to_f32(v.x & 0xffffu) * f) | (f32_to_bf16_bits(bf16_bits_to_f32(v.x >> 16) * f) << 16);
  r.y = f32_to_bf16_bits(bf16_bits_to_f32(v.y & 0xffffu) * f) | (f32_to_bf16_bits(bf16_bits_to_f32(v.y >> 16) * f) << 16);
  r.z = f32_to_bf16_bits(bf16_bits_to_f32(v.z & 0xffffu) * f) | (f32_to_bf16_bits(bf16_bits_to_f32(v.z >> 16) * f) << 16);
  r.w = f32_to_bf16_bits(bf16_bits_to_f32(v.w & 0xffffu) * f) | (f32_to_bf16_bits(bf16_bits_to_f32(v.w >> 16) * f) << 16);
  *op = r;
  // every thread of the (row, head) read lse before any writes it: the 16 threads sit
  // in one wave (t & 15 spans an aligned group of 16 lanes)
  if ((t & 15) == 0) lse[rh] = lse_v;
}

hipError_t launch_attn_sink(uint16_t* out, float* lse, const float* sink, int64_t rows, int heads,
                            hipStream_t st) {
  const int64_t threads = rows * heads * 16;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sink_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     out, lse, sink, rows, heads);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnBatch& ab_in, int batch, hipStream_t st) {
  if (batch == 0 || ab_in.n == 0) return hipSuccess;
  AttnBatch ab = ab_in;
  const AttnArgs& a0 = ab.a[0];   // heads and max_q are shared by the batch
  if (a0.max_q == 0) return hipSuccess;
  int max_splits = 1;               // each layer has its own split count
  for (int l = 0; l < ab.n; ++l) max_splits = max(max_splits, ab.a[l].splits);
  if (max_splits > 65535) return hipErrorInvalidValue;
  const int hg = ab.hpb / 16;                     // 1, 2 or 4
  const unsigned rows_grid = (unsigned)(batch * a0.max_q);
  const int64_t items = (int64_t)rows_grid * ab.n * ab.head_blocks;
  if (items >= INT32_MAX) return hipErrorInvalidValue;
  ab.rows_grid = (int)rows_grid;
  ab.items = (int)items;
  dim3 grid((unsigned)(items | 1), (unsigned)max_splits, 1u);
  int n_sparse = 0;
  for (int l = 0; l < ab.n; ++l) n_sparse += ab.a[l].idx != nullptr;
  const int mode = n_sparse == 0 ? 0 : n_sparse == ab.n ? 1 : 2;
#define LCA_ATTN_LAUNCH_KV(ES, SUB, NB, KV)                                                   \
  do {                                                                                        \
    if (mode == 0) hipLaunchKernelGGL((attn_dma_kernel<ES, SUB, NB, 0, KV>), grid, dim3(AT_NT), 0, st, ab); \
    else if (mode == 1) hipLaunchKernelGGL((attn_dma_kernel<ES, SUB, NB, 1, KV>), grid, dim3(AT_NT), 0, st, ab); \
    else hipLaunchKernelGGL((attn_dma_kernel<ES, SUB, NB, 2, KV>), grid, dim3(AT_NT), 0, st, ab); \
  } while (0)
#define LCA_ATTN_LAUNCH(ES, SUB, NB) LCA_ATTN_LAUNCH_KV(ES, SUB, NB, 0)
  // mixed KV rows (every layer of the batch; 64-head blocks): 64-entry stages
  // 64 heads: 64-entry stages, except for sparse prefill-sized query batches, which
  // run 32-entry stages (more groups resident per CU; measured 4 % faster there,
  // slower for dense rows)
  if (a0.kv8) {
    if (hg != 4) return hipErrorInvalidValue;
    LCA_ATTN_LAUNCH_KV(1, 2, 2, 1);
  } else if (hg == 4 && mode == 1 && a0.max_q >= 16) LCA_ATTN_LAUNCH(1, 1, 2);
  else if (hg == 4) LCA_ATTN_LAUNCH(1, AT_SUB64, AT_NB64);
  else if (hg == 2) LCA_ATTN_LAUNCH(2, 1, 2);
  else LCA_ATTN_LAUNCH(4, 1, 2);
#undef LCA_ATTN_LAUNCH
#undef LCA_ATTN_LAUNCH_KV
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_splits <= 1) return e;
  // 8-head groups of a block of 16, 32 or 64 heads; 2-head groups when 8-head ones
  // would not give every CU a group
  const bool narrow = items * (ab.hpb / 8) < 256;
  const int groups = ab.hpb / (narrow ? 2 : 8);
  if ((int64_t)items * groups >= INT32_MAX) return hipErrorInvalidValue;
  const dim3 cgrid((unsigned)(items * groups));
  // rounds of 16 pieces for launches of sparse layers only with more than 8 pieces per
  // row (one round for a 16-piece row), else of 8
  const bool u16 = mode == 1 && max_splits > 8;
  if (narrow && u16) hipLaunchKernelGGL((attn_combine_kernel<16, 2>), cgrid, dim3(64), 0, st, ab, groups);
  else if (narrow) hipLaunchKernelGGL((attn_combine_kernel<8, 2>), cgrid, dim3(64), 0, st, ab, groups);
  else if (u16) hipLaunchKernelGGL((attn_combine_kernel<16, 8>), cgrid, dim3(256), 0, st, ab, groups);
  else hipLaunchKernelGGL((attn_combine_kernel<8, 8>), cgrid, dim3(256), 0, st, ab, groups);
  return hipGetLastError();
}

}  // namespace lca
