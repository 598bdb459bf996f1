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
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

constexpr int KC_NT = 256;

__global__ __launch_bounds__(KC_NT) void kv_compress_kernel(const uint16_t* __restrict__ x,
                                                            const int64_t* __restrict__ tok_off,
                                                            const int64_t* __restrict__ ent_off,
                                                            int D, int c, uint16_t* __restrict__ y) {
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
  i32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = f64_to_bf16_bits(acc[2 * w] / (double)c);
    const uint32_t hi = f64_to_bf16_bits(acc[2 * w + 1] / (double)c);
    o[w] = (int)(lo | (hi << 16));
  }
  reinterpret_cast<i32x4*>(y + (e0 + j) * D)[v] = o;
}

hipError_t launch_kv_compress(const uint16_t* x, const int64_t* tok_off, int batch, int max_tokens,
                              int head_dim, int c, uint16_t* y, const int64_t* ent_off,
                              hipStream_t st) {
  const int64_t max_out = (int64_t)(max_tokens / c) * (head_dim / 8);
  if (max_out == 0 || batch == 0) return hipSuccess;
  dim3 grid((unsigned)((max_out + KC_NT - 1) / KC_NT), (unsigned)batch);
  hipLaunchKernelGGL(kv_compress_kernel, grid, dim3(KC_NT), 0, st, x, tok_off, ent_off, head_dim,
                     c, y);
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
