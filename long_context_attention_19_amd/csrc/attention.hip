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
// leaves registers.  V is stored transposed in LDS when staged, so the V^T
// operand is two 8-byte LDS reads per MFMA.
//
// Per work-group: 256 threads = 4 waves.  With HG = min(H, 64)/16 head groups,
// wave w takes head group w % HG and entry sub-group w / HG; a super-tile of 64
// entries (128 for H = 16) is gathered with 128-bit loads (one 256-byte row per
// 16 lanes), K row-major and V transposed into LDS, while the next two
// super-tiles' rows are already in flight in registers.  Softmax is fp32 in log2 units;
// P is rounded to bf16 for the MFMA and the running sum uses the rounded values.
//
// Splitting: a row's entries are cut into at most `splits` pieces of a multiple
// of the super-tile; each piece is a work-group.  A single piece writes the
// final output; otherwise each writes (O, max, sum) partials and the combine
// kernel merges them in piece order.  The cut depends only on the row's own
// entry count, so a row's bits do not depend on the rest of the batch.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int AT_NT = 256;
constexpr int HD = 128;            // head_dim
constexpr int KSTR = HD + 8;       // K row stride in LDS (bf16 elements): 272 B, spreads banks

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

template <int ES, int SUB>
struct AttnSmem {
  static constexpr int ST = 32 * ES * SUB;      // entries per super-tile
  static constexpr int VSTR = ST + 4;           // V^T row stride (bf16 elements)
  union {
    struct {
      uint16_t k[ST * KSTR];
      uint16_t vt[HD * VSTR];
    } tile;
    float merge_o[ES > 1 ? 4 : 1][ES > 1 ? 16 * HD : 1];   // per-wave O for the ES merge
  };
  float merge_ml[ES > 1 ? 4 : 1][16][2];
};

// ES entry sub-groups of waves; each wave takes SUB consecutive 32-entry sub-tiles
// of every super-tile, so one super-tile (one gather round trip) covers 32*ES*SUB rows.
template <int ES, int SUB>
__global__ __launch_bounds__(AT_NT) void attn_kernel(AttnBatch ab) {
  const AttnArgs& a = ab.a[blockIdx.z / ab.head_blocks];   // grid z = layer x head block
  constexpr int ST = AttnSmem<ES, SUB>::ST;
  constexpr int VSTR = AttnSmem<ES, SUB>::VSTR;
  constexpr int NPT = ST * 16 / AT_NT;          // 16-byte row pieces per thread per matrix
  constexpr int HG = 4 / ES;                    // head groups of 16 per work-group
  __shared__ AttnSmem<ES, SUB> sm;

  RowInfo ri;
  if (!row_info(a, ST, ri)) return;
  const int s = blockIdx.x;
  if (s >= ri.nsp) return;
  const int h0 = (blockIdx.z % ab.head_blocks) * 64;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & 63;
  const int hg = w % HG;
  const int es = w / HG;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int head = h0 + hg * 16 + l16;
  const int e0 = s * ri.per;
  const int e1 = min(e0 + ri.per, ri.n);

  // Q^T fragments (B operand of S^T): head `head`, dims 32ks + 8g .. +7
  bf16x8 qf[4];
  {
    const i32x4* qp = reinterpret_cast<const i32x4*>(a.q + (ri.row * a.heads + head) * HD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qp[ks * 4 + g]);
  }

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Staging: piece p = t + 256*u covers entry p/16, dims 8*(p%16) .. +7.  The loads
  // form a fixed, branch-free sequence so the compiler can wait on exact load counts:
  // the entry ids of a super-tile are fetched one stage before its K/V rows, and two
  // super-tiles of K/V rows are in flight while the current one is in use.  Pieces
  // past the split's end read the split's last row (already cached) and are zeroed
  // when staged.
  i32x4 kA[NPT], vA[NPT], kB[NPT], vB[NPT];
  int idA[NPT], idB[NPT];
  const int e_last = e1 - 1;
  auto load_ids = [&](int* ids, int tb) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int e = min(tb + ((t + AT_NT * u) >> 4), e_last);
      ids[u] = a.idx ? a.idx[ri.row * a.k + e] : e;
    }
  };
  auto gather = [&](const int* ids, i32x4* kr, i32x4* vr) {
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int col = (t + AT_NT * u) & 15;
      int64_t id = ids[u];
      id = id < 0 ? 0 : (id >= ri.n_seq ? ri.n_seq - 1 : id);   // stay inside the sequence
      const int64_t ent = ri.e_base + id;
      kr[u] = reinterpret_cast<const i32x4*>(a.kc + ent * HD)[col];
      vr[u] = reinterpret_cast<const i32x4*>(a.vc + ent * HD)[col];
    }
  };
  auto stage = [&](const i32x4* kr, const i32x4* vr, int tb) {
    __syncthreads();   // previous super-tile fully consumed
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int p = t + AT_NT * u;
      const int el = p >> 4;
      const int col = p & 15;
      const bool valid = tb + el < e1;
      const i32x4 kz = valid ? kr[u] : i32x4{0, 0, 0, 0};
      const i32x4 vz = valid ? vr[u] : i32x4{0, 0, 0, 0};
      *reinterpret_cast<i32x4*>(&sm.tile.k[el * KSTR + col * 8]) = kz;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t word = (uint32_t)vz[q];
        sm.tile.vt[(col * 8 + 2 * q) * VSTR + el] = (uint16_t)(word & 0xffffu);
        sm.tile.vt[(col * 8 + 2 * q + 1) * VSTR + el] = (uint16_t)(word >> 16);
      }
    }
    __syncthreads();
  };
  auto compute = [&](int tb) {
#pragma unroll
    for (int sub = 0; sub < SUB; ++sub) {
      const int el0 = (es * SUB + sub) * 32;   // this wave's 32 entries of the super-tile
      const int ev0 = tb + el0;                // their first entry number
      if (ev0 < e1) {
        // S^T for two 16-entry blocks
        f32x4 sacc[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
          const uint16_t* krow = &sm.tile.k[(el0 + rb * 16 + l16) * KSTR + 8 * g];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kf =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(krow + 32 * ks));
            sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[rb], 0, 0, 0);
          }
        }
        // online softmax (log2 units); lane holds head l16, entries 16rb + 4g + i
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = ev0 + rb * 16 + 4 * g + i;
            const float v = (e < e1) ? sacc[rb][i] * a.scale_log2 : -INFINITY;
            x[rb * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
        const float m_new = fmaxf(m_run, mx);       // finite: the wave has a valid entry
        const float alpha = exp2f(m_run - m_new);   // 0 on the first tile
        bf16x8 pf;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const __bf16 pb = (__bf16)exp2f(x[i] - m_new);
          pf[i] = pb;
          psum += (float)pb;
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          o[db] *= alpha;
          const uint16_t* vrow = &sm.tile.vt[(db * 16 + l16) * VSTR + el0 + 4 * g];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 16);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[db], 0, 0, 0);
        }
        m_run = m_new;
      }
    }
  };

  if (e1 > e0) {
    load_ids(idA, e0);
    load_ids(idB, e0 + ST);
    gather(idA, kA, vA);
    load_ids(idA, e0 + 2 * ST);
    gather(idB, kB, vB);
    load_ids(idB, e0 + 3 * ST);
    for (int tb = e0; tb < e1; tb += 2 * ST) {
      stage(kA, vA, tb);
      gather(idA, kA, vA);               // rows of super-tile tb + 2*ST
      load_ids(idA, tb + 4 * ST);
      compute(tb);
      stage(kB, vB, tb + ST);
      gather(idB, kB, vB);               // rows of super-tile tb + 3*ST
      load_ids(idB, tb + 5 * ST);
      compute(tb + ST);                  // no-op past the end
    }
  }

  // total of the per-lane-group partial sums for this lane's head
  l_run += __shfl_xor(l_run, 16, WAVE);
  l_run += __shfl_xor(l_run, 32, WAVE);

  if (ES > 1) {
    // merge the ES entry sub-tiles of each head group through LDS
    __syncthreads();
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.merge_o[w][l16 * HD + db * 16 + 4 * g + i] = o[db][i];
    if (g == 0) {
      sm.merge_ml[w][l16][0] = m_run;
      sm.merge_ml[w][l16][1] = l_run;
    }
    __syncthreads();
    if (es != 0) return;
    float mm = -INFINITY;
#pragma unroll
    for (int q = 0; q < ES; ++q) mm = fmaxf(mm, sm.merge_ml[hg + q * HG][l16][0]);
    float ll = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < ES; ++q) {
      const int wq = hg + q * HG;
      const float mq = sm.merge_ml[wq][l16][0];
      const float f = (mq == -INFINITY) ? 0.f : exp2f(mq - mm);
      ll += sm.merge_ml[wq][l16][1] * f;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] += sm.merge_o[wq][l16 * HD + db * 16 + 4 * g + i] * f;
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
  int st_size;
  if (hg == 4) {
    hipLaunchKernelGGL((attn_kernel<1, 2>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 64;
  } else if (hg == 2) {
    hipLaunchKernelGGL((attn_kernel<2, 1>), grid, dim3(AT_NT), 0, st, ab);
    st_size = 64;
  } else {
    hipLaunchKernelGGL((attn_kernel<4, 1>), grid, dim3(AT_NT), 0, st, ab);
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
