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

#include "hsa_common.h"

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

// ---- 16x16x16 operands, transposing LDS reads, wave-local LDS ordering ----------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 pack_bf16x4(f32x4 v) {
  return __builtin_bit_cast(s16x4, __builtin_convertvector(v, bf16x4));
}
// Orders this wave's earlier LDS accesses before its later ones that touch other lanes' data
// (the LDS serves one wave's instructions in order; the wait and the compiler barrier keep
// both the hardware and the compiler from moving accesses across this point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ bf16x8 cat_bf16x8(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}
// gfx950 transposing LDS read of four 16-bit elements: in each group of 16 lanes, lane j
// receives element j%4 of the 8-byte word that lane 4*i + j/4 addresses, for i = 0..3.
// With lane m of group `blk` addressing row 4*blk + m/4, column c0 + 4*(m%4) of a row-major
// LDS matrix, lane j gets column c0 + j of rows 4*blk .. 4*blk+3: the 16x16x16 MFMA
// A operand of the transposed matrix.  p must point into LDS.
__device__ __forceinline__ s16x4 lds_read_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// E consecutive bf16 values (E = 4, 8 or 16; 2E-byte aligned): raw load, fp32 accumulation,
// and the RNE store of E fp32 values
template <int E>
__device__ __forceinline__ void load_raw(const bf16* p, uint32_t (&u)[E / 2]) {
  if constexpr (E == 4) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    u[0] = x.x;
    u[1] = x.y;
  } else {
#pragma unroll
    for (int h = 0; h < E / 8; ++h) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + 8 * h);
      u[4 * h] = x.x;
      u[4 * h + 1] = x.y;
      u[4 * h + 2] = x.z;
      u[4 * h + 3] = x.w;
    }
  }
}
template <int E>
__device__ __forceinline__ void add_raw(float (&acc)[E], const uint32_t (&u)[E / 2], bool on) {
#pragma unroll
  for (int j = 0; j < E / 2; ++j) {
    acc[2 * j] += on ? __uint_as_float(u[j] << 16) : 0.0f;
    acc[2 * j + 1] += on ? __uint_as_float(u[j] & 0xffff0000u) : 0.0f;
  }
}
template <int E>
__device__ __forceinline__ void store_row(bf16* p, const float (&v)[E]) {
#pragma unroll
  for (int j = 0; j < E / 4; ++j)
    *reinterpret_cast<s16x4*>(p + 4 * j) =
        pack_bf16x4(f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]});
}

}  // namespace hsa
