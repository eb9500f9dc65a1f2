// Row access helpers shared by the gather/reduce kernels: a row is read and
// written in units of 8 elements (one 16-byte vector of bf16, two of fp32),
// widened to fp32, and rounded back to nearest-even once.  Internal header.
#pragma once

#include "moe_internal.h"

namespace moe {

// 8 elements of a row as fp32.
template <bool BF16>
struct Unit;

template <>
struct Unit<true> {  // 8 bf16 = one 16-byte vector
  u32x4 v;
  __device__ __forceinline__ void load(const char *row, int i) {
    v = __builtin_nontemporal_load((const u32x4 *)(row + (size_t)i * 16));
  }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t w = v[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

template <>
struct Unit<false> {  // 8 fp32 = two 16-byte vectors
  u32x4 a, b;
  __device__ __forceinline__ void load(const char *row, int i) {
    const u32x4 *p = (const u32x4 *)(row + (size_t)i * 32);
    a = __builtin_nontemporal_load(p);
    b = __builtin_nontemporal_load(p + 1);
  }
  __device__ __forceinline__ float get(int j) const {
    return __uint_as_float(j < 4 ? a[j] : b[j - 4]);
  }
};

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 fp32 values rounded into out's unit layout: one 16-byte vector of bf16
// (v[0]) or two of fp32 (v[0], v[1]).
template <bool OBF16>
__device__ __forceinline__ void pack_unit(const float *a, u32x4 *v) {
  if constexpr (OBF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[0][j] = bf16_rne(a[2 * j]) | (bf16_rne(a[2 * j + 1]) << 16);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[0][j] = __float_as_uint(a[j]);
      v[1][j] = __float_as_uint(a[4 + j]);
    }
  }
}

template <bool OBF16>
__device__ __forceinline__ void store_unit(char *row, int i, const float *a) {
  if constexpr (OBF16) {
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = bf16_rne(a[2 * j]) | (bf16_rne(a[2 * j + 1]) << 16);
    __builtin_nontemporal_store(v, (u32x4 *)(row + (size_t)i * 16));
  } else {
    u32x4 v0, v1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v0[j] = __float_as_uint(a[j]);
      v1[j] = __float_as_uint(a[4 + j]);
    }
    u32x4 *p = (u32x4 *)(row + (size_t)i * 32);
    __builtin_nontemporal_store(v0, p);
    __builtin_nontemporal_store(v1, p + 1);
  }
}

}  // namespace moe
