// Device helpers shared by the gfx950 kernels: bf16 conversions, wave and
// work-group scans.  All code targets 64-lane wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int KEY_BIAS = 1 << 20;        // indexer scores lie in [-2^20, 2^20)
constexpr int HIST_BINS = 2048;          // first radix level: key >> 10
constexpr int FINE_BINS = 1024;          // second radix level: key & 1023

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// double -> bf16 with a single rounding (to nearest, ties to even).
// Normal range: add the rounding bias below bit 45 of the fp64 encoding (bf16 keeps
// 7 of the 52 stored mantissa bits), clear those bits, then narrow exactly to fp32.
// Below 2^-126 bf16 spacing is fixed at 2^-133: scale, round to integer, scale back.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint64_t a = u & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return 0x7fc0u;                       // NaN
  if (a < 0x3810000000000000ull) {                                    // |x| < 2^-126
    double r = rint(x * 0x1p133) * 0x1p-133;
    return __float_as_uint((float)r) >> 16;
  }
  u += 0x00000fffffffffffull + ((u >> 45) & 1ull);
  u &= ~0x00001fffffffffffull;
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;   // >= 2^128 -> inf
}

// ---------------------------------------------------------------- scans

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    T o = __shfl_up(v, d, WAVE);
    if (lane >= d) v += o;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = WAVE / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

// Exclusive scan across a work-group of NT threads (NT a multiple of 64, <= 1024).
// `tmp` is LDS scratch of NT/64 + 1 elements.  Returns the exclusive prefix and
// writes the total to *total.  Contains __syncthreads(): call from all threads.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* tmp, T* total) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE;
  T inc = wave_incl_scan(v);
  if (lane == WAVE - 1) tmp[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    T run = 0;
    for (int i = 0; i < NW; ++i) {
      T t = tmp[i];
      tmp[i] = run;
      run += t;
    }
    tmp[NW] = run;
  }
  __syncthreads();
  T res = inc - v + tmp[w];
  *total = tmp[NW];
  __syncthreads();
  return res;
}

}  // namespace lca
