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
         align256((size_t)rows * splits * heads * 8);
}

void attn_ws_carve(void* ws, int rows, int heads, int splits, AttnArgs& a) {
  if (splits <= 1 || ws == nullptr) {
    a.part_o = nullptr;
    a.part_ml = nullptr;
    return;
  }
  char* p = reinterpret_cast<char*>(ws);
  a.part_o = reinterpret_cast<float*>(p);
  p += align256((size_t)rows * splits * heads * HD * 4);
  a.part_ml = reinterpret_cast<float2*>(p);
}

struct RowInfo {
  int64_t row;       // global query row
  int64_t e_base;    // first entry of the sequence
  int64_t n_seq;     // entries the sequence holds
  int n;             // entries this row attends
  int per;           // entries per split piece
  int nsp;           // split pieces actually used
};

// One piece size for every row of the launch, from the host's bound on the entry
// count: shorter rows get proportionally fewer pieces (a row beyond the bound widens
// its own pieces so that it still fits in `splits`).
__device__ __forceinline__ int piece_size(int n, int max_n, int splits, int stage) {
  const int want = (max(n, max_n) + splits - 1) / splits;
  return max(stage, (want + stage - 1) / stage * stage);
}

// Shared by the attention and combine kernels so both cut a row identically.
__device__ __forceinline__ bool row_info(const AttnArgs& a, int supertile, RowInfo& ri) {
  const int b = blockIdx.y / a.max_q;
  const int i = blockIdx.y - b * a.max_q;
  const int64_t r0 = a.q_off[b];
  if (i >= a.q_off[b + 1] - r0) return false;
  ri.row = r0 + i;
  ri.e_base = a.ent_off[b];
  const int64_t N = a.ent_off[b + 1] - ri.e_base;
  ri.n_seq = N;
  if (N <= 0) ri.n = 0;
  else if (a.idx) ri.n = max(0, min(a.count[ri.row], a.k));
  else ri.n = (int)min(a.q_pos[ri.row] / a.ratio, N);
  ri.per = piece_size(ri.n, a.max_n, a.splits, supertile);
  ri.nsp = ri.n > 0 ? (ri.n + ri.per - 1) / ri.per : 1;
  return true;
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
#ifndef AT_SUB64
#define AT_SUB64 2          // 64 heads: 32-entry sub-tiles per wave per stage
#endif
#ifndef AT_NB64
#define AT_NB64 2           // 64 heads: stage buffers
#endif
constexpr int AT_IDS = 2048;       // entry ids staged in LDS per chunk (sparse form)

template <int ST, int NB, bool SPARSE>
struct AttnDmaSmem {
  i32x4 k[NB][ST * 16];
  i32x4 v[NB][ST * 16];
  int ids[SPARSE ? AT_IDS : 1];
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

// ES entry sub-groups of waves; each wave takes SUB consecutive 32-entry sub-tiles of
// every stage, so a stage covers 32*ES*SUB entries.
template <int ES, int SUB, int NB, bool SPARSE>
__global__ __launch_bounds__(AT_NT) void attn_dma_kernel(AttnBatch ab) {
  const AttnArgs& a = ab.a[blockIdx.z / ab.head_blocks];   // grid z = layer x head block
  constexpr int ST = 32 * ES * SUB;             // entries per super-tile (stage)
  constexpr int HG = 4 / ES;                    // head groups of 16 per work-group
  constexpr int NU = ST / 16;                   // DMA instructions per wave per matrix
  static_assert(NU >= 1 && NU <= 8 && AT_IDS % ST == 0, "stage size");
  constexpr int D = NB - 1;                     // stages in flight ahead of the one in use
  static_assert(NB >= 2 && D * 2 * NU < 64, "pipeline depth");
  __shared__ AttnDmaSmem<ST, NB, SPARSE> sm;

  // The loads that set up a work-group form a short dependency chain; the query,
  // the first entry ids and the first stages' rows are issued as soon as their
  // addresses are known, before the row's entry count (and so the exact end of the
  // piece) is back.  Rows past the end are read but masked in the softmax.
  const int b = blockIdx.y / a.max_q;
  const int qi = blockIdx.y - b * a.max_q;
  const int64_t r0 = a.q_off[b];
  const int64_t nq = a.q_off[b + 1] - r0;
  const int64_t e_base = a.ent_off[b];
  const int64_t n_seq = a.ent_off[b + 1] - e_base;
  if (qi >= nq) return;
  const int64_t row = r0 + qi;
  const int s = blockIdx.x;
  // the row's entry count: only needed after the first DMAs are issued
  const int n_raw = SPARSE ? a.count[row] : (int)min(a.q_pos[row] / a.ratio, (int64_t)INT32_MAX);
  const int max_n = a.max_n;
  const int splits = a.splits;
  const int kk = a.k;
  const int h0 = (blockIdx.z % ab.head_blocks) * 64;
  const int t = threadIdx.x;
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
  const char* kseq = reinterpret_cast<const char*>(a.kc + e_base * HD);
  const char* vseq = reinterpret_cast<const char*>(a.vc + e_base * HD);
  const uint32_t k_lds0 = lds_addr(&sm.k[0][wrow0 * 16]);
  const uint32_t v_lds0 = lds_addr(&sm.v[0][wrow0 * 16]);
  constexpr uint32_t BUF_BYTES = ST * 256;

  // the piece as far as it is known before the entry count: exact when the count is
  // within the bound (always for the sparse form); its end is where reads stay valid
  const int per_g = piece_size(0, max_n, splits, ST);
  const int e0_g = s * per_g;
  const int end_g = n_seq <= 0 ? e0_g   // an empty sequence: nothing to fetch
                    : SPARSE ? min(e0_g + per_g, kk)
                             : (int)min((int64_t)e0_g + per_g, (int64_t)id_max + 1);

  // issue the DMA of the stage starting at entry tb into buffer buf; rows past
  // e_last repeat row e_last (cached, and masked in the softmax)
  auto issue = [&](int buf, int tb, int cbase, int e_last) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = wrow0 + 4 * u + my_row;
      const int e = min(tb + r, e_last);
      int id = SPARSE ? sm.ids[e - cbase] : e;
      id = min(max(id, 0), id_max);
      const uint32_t row_off = (uint32_t)id * 256u;
      const uint32_t ck = (uint32_t)(l16 ^ (r & 15)) << 4;
      const uint32_t cv = (uint32_t)(l16 ^ ((r & 7) << 1)) << 4;
      dma16(kseq, row_off + ck, k_lds0 + buf * BUF_BYTES + u * 1024);
      dma16(vseq, row_off + cv, v_lds0 + buf * BUF_BYTES + u * 1024);
    }
  };
  // copy the entry ids [cbase, cend) to LDS (sparse form; nothing else in flight)
  auto load_ids = [&](int cbase, int cend) __attribute__((always_inline)) {
    const int* src = a.idx + row * kk + cbase;
    const int cnt = cend - cbase;
    int v[AT_IDS / AT_NT];
#pragma unroll
    for (int u = 0; u < AT_IDS / AT_NT; ++u) {   // all loads in flight, then the stores
      const int j = t + AT_NT * u;
      v[u] = j < cnt ? src[j] : 0;
    }
    __syncthreads();   // the previous chunk's ids are no longer read
#pragma unroll
    for (int u = 0; u < AT_IDS / AT_NT; ++u) sm.ids[t + AT_NT * u] = v[u];
    __syncthreads();
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
  const int cend0 = SPARSE ? min(end_g, e0_g + AT_IDS) : end_g;
  if (cend0 > e0_g) {
    if constexpr (SPARSE) load_ids(e0_g, cend0);
    issued = prologue(e0_g, cend0);
  }
  // the query is needed now: the compiler's wait for it lands here, behind the DMAs
  asm volatile("" : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]));

  // as row_info computes it for the combine kernel
  const int n = n_seq <= 0 ? 0 : SPARSE ? max(0, min(n_raw, kk)) : (int)min((int64_t)n_raw, n_seq);
  const int per = piece_size(n, max_n, splits, ST);
  const int nsp = n > 0 ? (n + per - 1) / per : 1;
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
    const i32x4* kb = sm.k[buf];
    const char* vbase = reinterpret_cast<const char*>(sm.v[buf]);
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub) {
      const int el0 = (es * SUB + sub) * 32;   // this wave's 32 entries of the stage
      const int ev0 = tb + el0;
      if (ev0 < e1) {
        f32x4 sacc[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int r = el0 + rb * 16 + l16;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, kb[r * 16 + ((4 * ks + g) ^ (r & 15))]);
            sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[rb], 0, 0, 0);
          }
        }
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = ev0 + rb * 16 + 4 * g + i;
            const float v = (e < e1) ? sacc[rb][i] * scale_log2 : -INFINITY;
            x[rb * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
        const float m_new = fmaxf(m_run, mx);       // finite: the wave has a valid entry
        const float alpha = exp2f(m_run - m_new);   // 0 on the first tile, 1 if unchanged
        bf16x8 pf;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const __bf16 pb = (__bf16)exp2f(x[i] - m_new);
          pf[i] = pb;
          psum += (float)pb;
        }
        l_run = l_run * alpha + psum;
        if (__any(m_new > m_run)) {                 // otherwise every factor is exactly 1
#pragma unroll
          for (int db = 0; db < 8; ++db) o[db] *= alpha;
        }
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          bf16x4 half[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int r = el0 + 16 * hh + 4 * g + (l16 >> 2);
            const int q = l16 & 3;
            const int off = r * 256 + (((2 * db + (q >> 1)) ^ ((r & 7) << 1)) << 4) + (q & 1) * 8;
            half[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(vbase + off));
          }
          const bf16x8 vf = {half[0][0], half[0][1], half[0][2], half[0][3],
                             half[1][0], half[1][1], half[1][2], half[1][3]};
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }
  };


  // Per stage: wait for this stage's DMA (the later stages' may stay outstanding),
  // barrier, compute, barrier, then reuse the buffer for the stage NB ahead.
  for (int cbase = e0; cbase < e1; cbase += (SPARSE ? AT_IDS : (1 << 30))) {
    const int cend = SPARSE ? min(cbase + AT_IDS, e1) : e1;
    const int nst = (cend - cbase + ST - 1) / ST;
    if (cbase != cb0 || issued == 0) {
      wait_vm<0>();
      if constexpr (SPARSE) load_ids(cbase, cend);
      else lds_barrier();
      issued = prologue(cbase, cend);
      cb0 = cbase;
    }
    int buf = 0;
    for (int j = 0; j < nst; ++j) {
      const int ahead = issued - 1 - j;   // stages issued after stage j
      if (NB > 3 && ahead >= 3) wait_vm<(NB > 3 ? 3 : 0) * 2 * NU>();
      else if (NB > 2 && ahead == 2) wait_vm<(NB > 2 ? 2 : 0) * 2 * NU>();
      else if (ahead == 1) wait_vm<2 * NU>();
      else wait_vm<0>();
      lds_barrier();
      compute(buf, cbase + j * ST);
      lds_barrier();
      if (j + NB < nst) {
        issue(buf, cbase + (j + NB) * ST, cbase, cend - 1);
        issued = j + NB + 1;
      }
      buf = buf + 1 == NB ? 0 : buf + 1;
    }
  }
  wait_vm<0>();   // stages fetched past the end

  l_run += __shfl_xor(l_run, 16, WAVE);
  l_run += __shfl_xor(l_run, 32, WAVE);

  if (ES > 1) {
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

  if (nsp == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* op = a.out + (row * a.heads + head) * HD;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(o[db][0] * inv) | (f32_to_bf16_bits(o[db][1] * inv) << 16);
      pk.y = f32_to_bf16_bits(o[db][2] * inv) | (f32_to_bf16_bits(o[db][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + db * 16 + 4 * g) = pk;
    }
    if (a.lse && g == 0)
      a.lse[row * a.heads + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
  } else {
    const int64_t slot = (row * a.splits + s) * a.heads + head;
    float* pp = a.part_o + slot * HD;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(pp + db * 16 + 4 * g) = o[db];
    if (g == 0) a.part_ml[slot] = make_float2(m_run, l_run);
  }
}

// Merge split partials: a work-group takes 2 heads of one row; per head, 32 dim
// groups (4 dims, one 16-byte load per piece) x 4 piece groups (pieces g, g+4, ...).
// Each thread merges its pieces in order with a running maximum, up to CB pieces per
// round of loads, then piece group 0 merges the 4 groups' results in group order.
// The result therefore does not depend on load timing.
constexpr int CMB_HEADS = 2;
constexpr int CMB_PG = 4;
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnBatch ab, int stage) {
  const AttnArgs& a = ab.a[blockIdx.z];   // grid z = layer
  constexpr int CB = 8;
  __shared__ float red[CMB_HEADS][CMB_PG][32][6];
  RowInfo ri;
  if (!row_info(a, stage, ri)) return;
  if (ri.nsp <= 1) return;
  const int hl = threadIdx.x >> 7;
  const int head = blockIdx.x * CMB_HEADS + hl;   // heads is a multiple of CMB_HEADS
  const int pg = (threadIdx.x >> 5) & (CMB_PG - 1);
  const int dg = threadIdx.x & 31;
  const int64_t base = ri.row * a.splits * a.heads + head;
  float mm = -INFINITY, ll = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = pg; s0 < ri.nsp; s0 += CB * CMB_PG) {
    float2 ml[CB];
    f32x4 ov[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int sp = s0 + u * CMB_PG;
      const bool in = sp < ri.nsp;
      const int64_t slot = base + (int64_t)(in ? sp : s0) * a.heads;
      ml[u] = a.part_ml[slot];
      ov[u] = *reinterpret_cast<const f32x4*>(a.part_o + slot * HD + dg * 4);
      if (!in) ml[u] = make_float2(-INFINITY, 0.f);
    }
    float mb = mm;
#pragma unroll
    for (int u = 0; u < CB; ++u) mb = fmaxf(mb, ml[u].x);
    const float r = exp2f(mm - mb);   // 0 on the first round
    ll *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float f = exp2f(ml[u].x - mb);   // 0 for pieces past the end
      ll += ml[u].y * f;
      acc += ov[u] * f;
    }
    mm = mb;
  }
  float* my = red[hl][pg][dg];
  my[0] = mm;
  my[1] = ll;
  my[2] = acc[0];
  my[3] = acc[1];
  my[4] = acc[2];
  my[5] = acc[3];
  __syncthreads();
  if (pg != 0) return;
  float mt = -INFINITY;
#pragma unroll
  for (int q = 0; q < CMB_PG; ++q) mt = fmaxf(mt, red[hl][q][dg][0]);   // pg 0 holds piece 0
  float lt = 0.f;
  f32x4 at = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < CMB_PG; ++q) {
    const float* o = red[hl][q][dg];
    const float f = o[0] == -INFINITY ? 0.f : exp2f(o[0] - mt);
    lt += o[1] * f;
    at += f32x4{o[2], o[3], o[4], o[5]} * f;
  }
  const float inv = 1.f / lt;
  uint2 pk;
  pk.x = f32_to_bf16_bits(at[0] * inv) | (f32_to_bf16_bits(at[1] * inv) << 16);
  pk.y = f32_to_bf16_bits(at[2] * inv) | (f32_to_bf16_bits(at[3] * inv) << 16);
  *reinterpret_cast<uint2*>(a.out + (ri.row * a.heads + head) * HD + dg * 4) = pk;
  if (a.lse && dg == 0) a.lse[ri.row * a.heads + head] = (mt + log2f(lt)) * 0.69314718055994530942f;
}

hipError_t launch_attention(const AttnBatch& ab, int batch, hipStream_t st) {
  if (batch == 0 || ab.n == 0) return hipSuccess;
  const AttnArgs& a0 = ab.a[0];   // heads, splits and max_q are shared by the batch
  if (a0.max_q == 0) return hipSuccess;
  const int hg = min(a0.heads, 64) / 16;          // 1, 2 or 4
  const unsigned rows_grid = (unsigned)(batch * a0.max_q);
  dim3 grid((unsigned)a0.splits, rows_grid, (unsigned)(ab.n * ab.head_blocks));
  const bool sparse = a0.idx != nullptr;         // a batch holds one kind of layer
  int st_size;
  if (hg == 4) {
    if (sparse) hipLaunchKernelGGL((attn_dma_kernel<1, AT_SUB64, AT_NB64, true>), grid, dim3(AT_NT), 0, st, ab);
    else hipLaunchKernelGGL((attn_dma_kernel<1, AT_SUB64, AT_NB64, false>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 32 * AT_SUB64;
  } else if (hg == 2) {
    if (sparse) hipLaunchKernelGGL((attn_dma_kernel<2, 1, 2, true>), grid, dim3(AT_NT), 0, st, ab);
    else hipLaunchKernelGGL((attn_dma_kernel<2, 1, 2, false>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 64;
  } else {
    if (sparse) hipLaunchKernelGGL((attn_dma_kernel<4, 1, 2, true>), grid, dim3(AT_NT), 0, st, ab);
    else hipLaunchKernelGGL((attn_dma_kernel<4, 1, 2, false>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 128;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a0.splits <= 1) return e;
  dim3 cgrid((unsigned)((a0.heads + CMB_HEADS - 1) / CMB_HEADS), rows_grid, (unsigned)ab.n);
  hipLaunchKernelGGL(attn_combine_kernel, cgrid, dim3(256), 0, st, ab, st_size);
  return hipGetLastError();
}

}  // namespace lca
