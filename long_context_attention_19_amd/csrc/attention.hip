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
// Splitting: a row's entries are cut into at most `splits` pieces of a multiple
// of the stage; each piece is a work-group.  A single piece writes the final
// output; otherwise each writes (O, max, sum) partials and the combine kernel
// merges them in piece order.  The cut depends only on the row's own entry
// count, so a row's bits do not depend on the rest of the batch.
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
  const int want = (ri.n + a.splits - 1) / a.splits;
  ri.per = max(supertile, (want + supertile - 1) / supertile * supertile);
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
constexpr int AT_IDS = 2048;       // entry ids staged in LDS per chunk (sparse form)

template <int ST, bool SPARSE>
struct AttnDmaSmem {
  i32x4 k[2][ST * 16];
  i32x4 v[2][ST * 16];
  int ids[SPARSE ? AT_IDS : 1];
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// 64 lanes x 16 bytes from seq + voff (per lane) into LDS at lds .. lds + 1023
__device__ __forceinline__ void dma16(const void* seq, uint32_t voff, uint32_t lds) {
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
template <int ES, int SUB, bool SPARSE>
__global__ __launch_bounds__(AT_NT) void attn_dma_kernel(AttnBatch ab) {
  const AttnArgs& a = ab.a[blockIdx.z / ab.head_blocks];   // grid z = layer x head block
  constexpr int ST = 32 * ES * SUB;             // entries per super-tile (stage)
  constexpr int HG = 4 / ES;                    // head groups of 16 per work-group
  constexpr int NU = ST / 16;                   // DMA instructions per wave per matrix
  static_assert(NU >= 1 && NU <= 8 && AT_IDS % ST == 0, "stage size");
  __shared__ AttnDmaSmem<ST, SPARSE> sm;

  RowInfo ri;
  if (!row_info(a, ST, ri)) return;
  const int s = blockIdx.x;
  if (s >= ri.nsp) return;
  const int h0 = (blockIdx.z % ab.head_blocks) * 64;
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int hg = w % HG;
  const int es = w / HG;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int head = h0 + hg * 16 + l16;
  const int e0 = s * ri.per;
  const int e1 = min(e0 + ri.per, ri.n);
  // kernel arguments used inside the pipeline are read once: the asm memory clobbers
  // would otherwise make the compiler reload them
  const float scale_log2 = a.scale_log2;

  bf16x8 qf[4];
  {
    const i32x4* qp = reinterpret_cast<const i32x4*>(a.q + (ri.row * a.heads + head) * HD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qp[ks * 4 + g]);
    // take the compiler's wait for the query here, before any DMA is in flight
    asm volatile("" : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]));
  }
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // wave w fills rows w*ST/4 .. +ST/4 of a stage; DMA instruction u covers 4 of them
  const int wrow0 = w * (ST / 4);
  const int my_row = lane >> 4;
  const int id_max = (int)min(ri.n_seq, (int64_t)ATTN_MAX_SEQ) - 1;
  const char* kseq = reinterpret_cast<const char*>(a.kc + ri.e_base * HD);
  const char* vseq = reinterpret_cast<const char*>(a.vc + ri.e_base * HD);
  const uint32_t k_lds0 = lds_addr(&sm.k[0][wrow0 * 16]);
  const uint32_t v_lds0 = lds_addr(&sm.v[0][wrow0 * 16]);
  constexpr uint32_t BUF_BYTES = ST * 256;

  // issue the DMA of the stage starting at entry tb into buffer buf; rows past
  // e_last repeat row e_last (cached, and masked in the softmax)
  auto issue = [&](int buf, int tb, int cbase, int e_last) {
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
  auto compute = [&](int buf, int tb) {
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

  // Per stage: issue the next stage's DMA into the other buffer, wait for this
  // stage's own DMA (the next stage's 2*NU operations may stay outstanding), barrier,
  // compute, barrier (the buffer is then free for the DMA two stages ahead).
  for (int cbase = e0; cbase < e1; cbase += (SPARSE ? AT_IDS : (1 << 30))) {
    const int cend = SPARSE ? min(cbase + AT_IDS, e1) : e1;
    const int e_last = cend - 1;
    if constexpr (SPARSE) {
      __syncthreads();   // the previous chunk's ids are no longer read
      const int* src = a.idx + ri.row * a.k + cbase;
      const int cnt = cend - cbase;
      int v[AT_IDS / AT_NT];
#pragma unroll
      for (int u = 0; u < AT_IDS / AT_NT; ++u) {   // all loads in flight, then the stores
        const int j = t + AT_NT * u;
        v[u] = j < cnt ? src[j] : 0;
      }
#pragma unroll
      for (int u = 0; u < AT_IDS / AT_NT; ++u) sm.ids[t + AT_NT * u] = v[u];
      __syncthreads();
    }
    int buf = 0;
    issue(0, cbase, cbase, e_last);
    for (int tb = cbase; tb < cend; tb += ST) {
      if (tb + ST < cend) {
        issue(buf ^ 1, tb + ST, cbase, e_last);
        wait_vm<2 * NU>();
      } else {
        wait_vm<0>();
      }
      lds_barrier();
      compute(buf, tb);
      lds_barrier();
      buf ^= 1;
    }
  }

  l_run += __shfl_xor(l_run, 16, WAVE);
  l_run += __shfl_xor(l_run, 32, WAVE);

  if (ES > 1) {
    // merge the ES entry sub-groups of each head group; the stage buffers are free
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

  if (ri.nsp == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* op = a.out + (ri.row * a.heads + head) * HD;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(o[db][0] * inv) | (f32_to_bf16_bits(o[db][1] * inv) << 16);
      pk.y = f32_to_bf16_bits(o[db][2] * inv) | (f32_to_bf16_bits(o[db][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + db * 16 + 4 * g) = pk;
    }
    if (a.lse && g == 0)
      a.lse[ri.row * a.heads + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
  } else {
    const int64_t slot = (ri.row * a.splits + s) * a.heads + head;
    float* pp = a.part_o + slot * HD;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(pp + db * 16 + 4 * g) = o[db];
    if (g == 0) a.part_ml[slot] = make_float2(m_run, l_run);
  }
}

// Merge split partials: thread = (head, dim).  Up to CB pieces are loaded at once
// (all of them for the default split count), then merged in piece order with a
// running maximum, so the result does not depend on load timing.
template <int ST>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnBatch ab) {
  const AttnArgs& a = ab.a[blockIdx.z];   // grid z = layer
  constexpr int CB = 32;
  RowInfo ri;
  if (!row_info(a, ST, ri)) return;
  if (ri.nsp <= 1) return;
  const int head = blockIdx.x * 2 + (threadIdx.x >> 7);
  if (head >= a.heads) return;
  const int d = threadIdx.x & 127;
  const int64_t base = ri.row * a.splits * a.heads + head;
  float mm = -INFINITY, ll = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < ri.nsp; s0 += CB) {
    float2 ml[CB];
    float ov[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const bool in = s0 + u < ri.nsp;
      const int64_t slot = base + (int64_t)(s0 + u) * a.heads;
      ml[u] = in ? a.part_ml[slot] : make_float2(-INFINITY, 0.f);
      ov[u] = in ? a.part_o[slot * HD + d] : 0.f;
    }
    float mb = mm;
#pragma unroll
    for (int u = 0; u < CB; ++u) mb = fmaxf(mb, ml[u].x);
    const float r = exp2f(mm - mb);   // 0 on the first batch
    ll *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float f = exp2f(ml[u].x - mb);
      ll += ml[u].y * f;
      acc += ov[u] * f;
    }
    mm = mb;
  }
  a.out[(ri.row * a.heads + head) * HD + d] = (uint16_t)f32_to_bf16_bits(acc / ll);
  if (a.lse && d == 0) a.lse[ri.row * a.heads + head] = (mm + log2f(ll)) * 0.69314718055994530942f;
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
    if (sparse) hipLaunchKernelGGL((attn_dma_kernel<1, 2, true>), grid, dim3(AT_NT), 0, st, ab);
    else hipLaunchKernelGGL((attn_dma_kernel<1, 2, false>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 64;
  } else if (hg == 2) {
    if (sparse) hipLaunchKernelGGL((attn_dma_kernel<2, 1, true>), grid, dim3(AT_NT), 0, st, ab);
    else hipLaunchKernelGGL((attn_dma_kernel<2, 1, false>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 64;
  } else {
    if (sparse) hipLaunchKernelGGL((attn_dma_kernel<4, 1, true>), grid, dim3(AT_NT), 0, st, ab);
    else hipLaunchKernelGGL((attn_dma_kernel<4, 1, false>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 128;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a0.splits <= 1) return e;
  dim3 cgrid((unsigned)((a0.heads + 1) / 2), rows_grid, (unsigned)ab.n);
  if (st_size == 64) hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(256), 0, st, ab);
  else hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(256), 0, st, ab);
  return hipGetLastError();
}

}  // namespace lca
