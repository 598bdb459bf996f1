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
constexpr int KEY_BIAS = 1 << 20;        // indexer scores lie in [-2^20, 2^20]
// word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle (loads past
// the resource's byte range return zeros)
constexpr int BUF_RSRC_WORD3 = 0x00020000;
constexpr int BUF_NT = 2;                  // cache-policy bit of a buffer load: nontemporal

// A value no kernel of the launch writes, read through the constant address space: a
// scalar load for a uniform address, whose wait does not hold the in-order vector loads.
template <class T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(size_t)p;
}
constexpr int HIST_BINS = 2048;          // first radix level: key >> 10
constexpr int FINE_BINS = 1024;          // second radix level: key & 1023

// The 21-bit radix key of an indexer score.  int8 scores lie in [-2^20, 2^20]; the top
// value 2^20 = 64 * (-128)^2 needs a query and a key of all -128 codes, and the next
// reachable score is 63 * 2^14 + 128 * 127 = 2^20 - 128.  Clamping 2^20 to 2^20 - 1
// therefore keeps every reachable score's rank, and the key stays below 2^21.
__device__ __forceinline__ int score_key(int32_t s) { return min(s, KEY_BIAS - 1) + KEY_BIAS; }

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

// The E8M0 unit scale (2^0, code 127) of the scaled (FP4) MFMAs, held in one VGPR that a
// kernel defines once and keeps to its end (e8m0_keep after its last MFMA).  Left to the
// compiler, the constant is rematerialised into a short-lived VGPR that the very next VALU
// instruction may overwrite while the multi-pass MFMA reading it as its scale is still in
// flight; rows of huge scores were seen with such code.  An asm definition cannot be
// rematerialised, and while it is live no other value is allocated to it.
__device__ __forceinline__ int e8m0_unit_vgpr() {
  int s;
  asm volatile("v_mov_b32 %0, 127" : "=v"(s));
  return s;
}
__device__ __forceinline__ void e8m0_keep(int s) { asm volatile("" ::"v"(s)); }

// ---------------------------------------------------------------- scans

// Inclusive prefix sum over the 64 lanes of a wave with DPP: a Hillis-Steele scan
// inside each row of 16 lanes (row_shr 1, 2, 4, 8; lanes past the row's start read
// 0), then row 15's lane added into rows 1 and 3 (row_bcast:15) and lane 31 into
// rows 2 and 3 (row_bcast:31).  Rows left out by the row mask add 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = WAVE / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = WAVE / 2; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, WAVE));
  return v;
}

// Exclusive prefix sum across a work-group of NT threads (NT a multiple of 64, at most
// 1024) in thread order.  `tmp` is LDS scratch of NT/64 + 1 ints.  Returns the exclusive
// prefix and writes the total to *total.  The waves scan their lanes; the first wave
// scans the wave totals.  Contains __syncthreads(): call from all threads.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / WAVE;
  static_assert(NW >= 1 && NW <= WAVE, "work-group size");
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE;
  const int inc = wave_incl_scan(v);
  if (lane == WAVE - 1) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int x = lane < NW ? tmp[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < NW) tmp[lane] = xi - x;
    if (lane == NW - 1) tmp[NW] = xi;
  }
  __syncthreads();
  const int res = inc - v + tmp[w];
  *total = tmp[NW];
  __syncthreads();
  return res;
}

}  // namespace lca
