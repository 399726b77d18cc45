// Device helpers for gfx950 (CDNA4, 64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace l3 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(16))) float floatx16;
// Native 16-byte vector: unlike the struct-based uint4, arrays of it stay in
// registers (the struct type made the compiler keep staging arrays in
// scratch memory).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even: gfx950 converts in
// hardware (v_cvt_pk_bf16_f32, two values an instruction).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values into one word, lo in the low half.
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element access for the two storage types.
template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf2f(p[i]);
}

template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, int64_t i, float v) {
  p[i] = v;
}
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, int64_t i,
                                             float v) {
  p[i] = f2bf(v);
}

// 16x16x32 bf16 MFMA: lane l supplies row (l & 15) of A and column (l & 15)
// of B, eight consecutive k values from group (l >> 4); the 16x16 float
// result lands as rows 4*(l >> 4) + i, column l & 15 in element i.
__device__ __forceinline__ floatx4 mfma_bf16(const uint4& a, const uint4& b,
                                             floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}
// 32x32x16 bf16 MFMA: lane l supplies row (l & 31) of A and column (l & 31)
// of B, eight consecutive k values from half (l >> 5); element e of the
// 32x32 float result is row 8*(e/4) + 4*(l >> 5) + (e % 4), column l & 31.
__device__ __forceinline__ floatx16 mfma32_bf16(const u32x4& a,
                                                const u32x4& b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}
// 16x16x4 float32 MFMA, same output layout; lane l supplies one k value
// (group l >> 4) of row / column l & 15.
__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Cross-lane reductions on DPP moves (no trip through the LDS crossbar).
// Controls (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140, row_bcast15 = 0x142,
// row_bcast31 = 0x143.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                         __builtin_bit_cast(int, v), CTRL,
                                         ROW_MASK, 0xF, false));
}
// Every lane of each 16-lane row gets the row's sum / maximum: after the two
// quad permutations each quad holds its total, the half mirror pairs the two
// quads of each 8 lanes, the mirror pairs the two halves of the row.
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_f<0xB1>(v, v);
  v += dpp_f<0x4E>(v, v);
  v += dpp_f<0x141>(v, v);
  v += dpp_f<0x140>(v, v);
  return v;
}
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v, v));
  v = fmaxf(v, dpp_f<0x4E>(v, v));
  v = fmaxf(v, dpp_f<0x141>(v, v));
  v = fmaxf(v, dpp_f<0x140>(v, v));
  return v;
}
// 32-lane groups (lanes 0-31, 32-63): the total lands in lanes 16-31 and
// 48-63 (row 1 / row 3 receive lane 15 of the row below).
__device__ __forceinline__ float group32_sum_hi(float v) {
  v = group16_sum(v);
  return v + dpp_f<0x142, 0xA>(0.f, v);
}
__device__ __forceinline__ float group32_max_hi(float v) {
  v = group16_max(v);
  return fmaxf(v, dpp_f<0x142, 0xA>(-INFINITY, v));
}
// Whole-wave reductions, result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = group32_sum_hi(v);
  v = v + dpp_f<0x143, 0xC>(0.f, v);
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = group32_max_hi(v);
  v = fmaxf(v, dpp_f<0x143, 0xC>(-INFINITY, v));
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Inclusive prefix sum over a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64).
// `tmp` must hold NT/64 + 1 ints. Returns the thread's exclusive prefix and
// writes the block total to *total. Contains __syncthreads().
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = wave_incl_scan(v, lane);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < NT / 64; ++i) {
      int t = tmp[i];
      tmp[i] = run;
      run += t;
    }
    tmp[NT / 64] = run;
  }
  __syncthreads();
  int res = tmp[w] + inc - v;
  *total = tmp[NT / 64];
  __syncthreads();
  return res;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) {
  return (a + b - 1) / b;
}

}  // namespace l3
