// hsa_common.h -- device helpers shared by the HSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

constexpr int kWave = 64;
constexpr int kMaxK = 16;   // largest top-K the kernels support
constexpr int kMaxG = 16;   // largest number of query heads per KV group
constexpr int kChunk = 64;  // chunk size S the kernels are written for

// bf16 storage: the upper half of an IEEE fp32.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float((uint32_t)x.bits << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return bf16{f32_to_bf16_bits(x)}; }

// fp64 -> storage type with a single rounding (nearest, ties to even).  For bf16 the value
// is first narrowed to fp32 with round-to-odd (truncate, then force the last bit when
// inexact); fp32 keeps more than two extra bits, so the second rounding is exact.
template <typename T>
__device__ __forceinline__ T from_f64(double x);
template <>
__device__ __forceinline__ float from_f64<float>(double x) { return (float)x; }
template <>
__device__ __forceinline__ bf16 from_f64<bf16>(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x && x == x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return bf16{f32_to_bf16_bits(f)};
}

// Eight consecutive elements -> fp32 (p 16-byte aligned for bf16, 32-byte for fp32 rows).
__device__ __forceinline__ void load8(const bf16* p, float* o) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// ---- wave64 reductions (butterfly over all 64 lanes) ----------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = (uint64_t)__shfl_xor((unsigned long long)v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// ---- rank keys ----------------------------------------------------------------------
// A candidate (score s, chunk c) becomes one 64-bit key whose unsigned order is the rank
// order: larger score first, then lower chunk index.  NaN ranks as -inf; -0 as +0.  Key 0
// never occurs for a real candidate and marks "no candidate".
__device__ __forceinline__ uint64_t rank_key(float s, int c) {
  if (s != s) s = -__builtin_inff();
  if (s == 0.0f) s = 0.0f;
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (uint32_t)c);
}
__device__ __forceinline__ float key_score(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u ^ 0x80000000u) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ int key_chunk(uint64_t k) {
  return (int)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
}

// Insert key into a descending list of length n (n <= kMaxK), dropping the smallest.
__device__ __forceinline__ void topk_insert(uint64_t (&top)[kMaxK], uint64_t key, int n) {
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) {
    if (i < n && key > top[i]) {
      uint64_t t = top[i];
      top[i] = key;
      key = t;
    }
  }
}
__device__ __forceinline__ void topk_pop(uint64_t (&top)[kMaxK]) {
#pragma unroll
  for (int i = 0; i < kMaxK - 1; ++i) top[i] = top[i + 1];
  top[kMaxK - 1] = 0;
}

// Stick-breaking over `n` ranked scores in double: w_k = p_k * prod_{j<k}(1 - p_j).
__device__ __forceinline__ double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

}  // namespace hsa
