// mfma_common.h -- CDNA4 (gfx950) matrix-core helpers for the bf16 kernels.
//
// v_mfma_f32_16x16x32_bf16: D[16x16] = A[16x32] * B[32x16] + C, fp32 accumulate.
//   A: lane l holds row l%16, 8 consecutive k of block l/16 (16 bytes)
//   B: lane l holds column l%16, 8 consecutive k of block l/16
//   D: lane l holds column l%16, rows 4*(l/16) .. 4*(l/16)+3
// Only the D layout matters to callers: the contraction pairs the same (lane block, element)
// slots of A and B, so any k order that A and B share gives the same sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Eight fp32 -> bf16 (round to nearest even, hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(f32x4 lo, f32x4 hi) {
  f32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Key order used by the P.V contraction (64 keys in two steps of 32).  The logits tile
// t (keys 16t..16t+15) leaves lane l with keys 16t + 4*(l/16) + i; step s pairs tiles 2s and
// 2s+1, so the B operand of lane l, element e, holds key perm_key(s, l/16, e).  The value
// operand must list its keys in the same order: the transposed value layout Vt stores
// position p = 32s + 8*(l/16) + e at key perm_key(s, l/16, e).
__host__ __device__ __forceinline__ int perm_key(int s, int block, int e) {
  return 32 * s + 16 * (e / 4) + 4 * block + (e % 4);
}

}  // namespace hsa
