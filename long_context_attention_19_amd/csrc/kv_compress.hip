// kv_compress: mean pooling of complete c-token blocks into compressed entries.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
// Review", section 3-2 item 2 (component table): CSA keeps one entry per 4
// tokens, HCA one per 128.  The mean is the pooling operator used here.
//
// Each thread owns one 16-byte column slice (8 dims) of one output entry and
// walks the entry's c tokens; loads are 128-bit and a wave covers whole
// 256-byte rows.  Sums run in fp64 in token order: every bf16 has 8 significant
// bits, so for any realistic spread of magnitudes the sum is exact, and the mean
// is rounded once to bf16 (ties to even) — the same value the plain definition
// gives.  HBM-bound: 2*c*D bytes read and 2*D written per entry.
//
// The mixed-row form (D = 128) writes 192-byte rows instead: dims 0..63 of the mean
// as FP8 E4M3 codes (bytes 0..63), dims 64..127 as bf16 (bytes 64..191); the page's
// component table keeps the RoPE dims of the KV cache in BF16 and the rest in FP8,
// and the last 64 dims are taken as the RoPE dims.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int KC_NT = 256;
constexpr int KC_KV8_DIM = 128;   // head_dim of a mixed row

// double -> FP8 E4M3 code with a single rounding: nearest value, ties to the even
// code, magnitudes above the largest finite value (448 = 1.75 * 2^8) clamped to it,
// the sign kept (also on zero).  Normal range (|x| >= 2^-6): E4M3 keeps 3 of the 52
// stored mantissa bits, so add the rounding bias below bit 49 of the fp64 encoding
// and clear those bits; the rounded value's exponent and top 3 mantissa bits are the
// code.  Below 2^-6 the codes are the multiples m * 2^-9 (m = 0..7; m = 8 is the
// first normal code, 0x08, so the code is m either way).  NaN inputs give 0x7F.
__device__ __forceinline__ uint32_t f64_to_e4m3_code(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 56) & 0x80u;
  uint64_t a = u & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return 0x7fu;                          // NaN
  if (a < 0x3f90000000000000ull)                                         // |x| < 2^-6
    return sign | (uint32_t)rint(__longlong_as_double((long long)a) * 0x1p9);
  a += 0x0000ffffffffffffull + ((a >> 49) & 1ull);
  a &= ~0x0001ffffffffffffull;
  if (a > 0x407c000000000000ull) return sign | 0x7eu;                    // above 448
  const uint32_t e = (uint32_t)(a >> 52) - 1023u + 7u;                   // 1 .. 15
  return sign | (e << 3) | (uint32_t)((a >> 49) & 7u);
}

template <bool KV8>
__global__ __launch_bounds__(KC_NT) void kv_compress_kernel(const uint16_t* __restrict__ x,
                                                            const int64_t* __restrict__ tok_off,
                                                            const int64_t* __restrict__ ent_off,
                                                            int D, int c, void* __restrict__ y) {
  const int b = blockIdx.y;
  const int64_t t0 = tok_off[b];
  const int64_t T = tok_off[b + 1] - t0;
  const int64_t e0 = ent_off[b];
  const int64_t cap = ent_off[b + 1] - e0;
  const int64_t n = min(T / c, cap);
  const int vpr = D >> 3;                       // 16-byte slices per row
  const int64_t gid = (int64_t)blockIdx.x * KC_NT + threadIdx.x;
  if (gid >= n * vpr) return;
  const int64_t j = gid / vpr;
  const int v = (int)(gid - j * vpr);

  const i32x4* src = reinterpret_cast<const i32x4*>(x + (t0 + j * c) * D) + v;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;

  int t = 0;
  for (; t + 4 <= c; t += 4) {
    i32x4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = __builtin_nontemporal_load(src + (int64_t)(t + u) * vpr);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = (uint32_t)r[u][w];
        acc[2 * w] += (double)bf16_bits_to_f32(word & 0xffffu);
        acc[2 * w + 1] += (double)bf16_bits_to_f32(word >> 16);
      }
    }
  }
  for (; t < c; ++t) {
    const i32x4 r = __builtin_nontemporal_load(src + (int64_t)t * vpr);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t word = (uint32_t)r[w];
      acc[2 * w] += (double)bf16_bits_to_f32(word & 0xffffu);
      acc[2 * w + 1] += (double)bf16_bits_to_f32(word >> 16);
    }
  }
  if (KV8 && v < 8) {   // dims 8v .. 8v+7 of the FP8 half: bytes 8v .. 8v+7 of the row
    uint32_t w2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w2[h] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) w2[h] |= f64_to_e4m3_code(acc[4 * h + i] / (double)c) << (8 * i);
    }
    *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(y) + (e0 + j) * KV8_ROW_BYTES + 8 * v) =
        make_uint2(w2[0], w2[1]);
    return;
  }
  i32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = f64_to_bf16_bits(acc[2 * w] / (double)c);
    const uint32_t hi = f64_to_bf16_bits(acc[2 * w + 1] / (double)c);
    o[w] = (int)(lo | (hi << 16));
  }
  if (KV8)   // the bf16 half: bytes 64 + 16 (v - 8) ..
    *reinterpret_cast<i32x4*>(reinterpret_cast<uint8_t*>(y) + (e0 + j) * KV8_ROW_BYTES + 64 +
                              16 * (v - 8)) = o;
  else
    reinterpret_cast<i32x4*>(reinterpret_cast<uint16_t*>(y) + (e0 + j) * D)[v] = o;
}

hipError_t launch_kv_compress(const uint16_t* x, const int64_t* tok_off, int batch, int max_tokens,
                              int head_dim, int c, uint16_t* y, const int64_t* ent_off,
                              hipStream_t st) {
  const int64_t max_out = (int64_t)(max_tokens / c) * (head_dim / 8);
  if (max_out == 0 || batch == 0) return hipSuccess;
  dim3 grid((unsigned)((max_out + KC_NT - 1) / KC_NT), (unsigned)batch);
  hipLaunchKernelGGL(kv_compress_kernel<false>, grid, dim3(KC_NT), 0, st, x, tok_off, ent_off,
                     head_dim, c, (void*)y);
  return hipGetLastError();
}

hipError_t launch_kv_compress_kv8(const uint16_t* x, const int64_t* tok_off, int batch,
                                  int max_tokens, int c, uint8_t* y, const int64_t* ent_off,
                                  hipStream_t st) {
  const int64_t max_out = (int64_t)(max_tokens / c) * (KC_KV8_DIM / 8);
  if (max_out == 0 || batch == 0) return hipSuccess;
  dim3 grid((unsigned)((max_out + KC_NT - 1) / KC_NT), (unsigned)batch);
  hipLaunchKernelGGL(kv_compress_kernel<true>, grid, dim3(KC_NT), 0, st, x, tok_off, ent_off,
                     KC_KV8_DIM, c, (void*)y);
  return hipGetLastError();
}

// Zero-fill used to reset workspaces without a memset node.
__global__ __launch_bounds__(256) void fill_zero_kernel(i32x4* p, size_t n16, uint8_t* tail,
                                                        size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = i32x4{0, 0, 0, 0};
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  const size_t want = (n16 + 255) / 256 + 1;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st,
                     reinterpret_cast<i32x4*>(p), n16, reinterpret_cast<uint8_t*>(p) + n16 * 16,
                     ntail);
  return hipGetLastError();
}

}  // namespace lca
