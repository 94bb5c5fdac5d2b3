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

// ---- four-element operands, transposing LDS reads, wave-local LDS ordering -------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Four fp32 values to bf16 (RNE), as two pair conversions: written per pair, the compiler
// keeps one v_cvt_pk_bf16_f32 per pair where the whole-vector form was sometimes split into
// four single conversions and two permutes.
__device__ __forceinline__ s16x4 pack_bf16x4(f32x4 v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
  const uint2 u = {__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
  return __builtin_bit_cast(s16x4, u);
}
// ---- 32x32x16 products over 16 rows ------------------------------------------------------
// v_mfma_f32_32x32x16_bf16: D[32x32] = A[32x16] * B[16x32] + C, fp32 accumulate, at the full
// matrix-core rate with a contraction only 16 deep (the legacy 16x16x16 form issues at the
// 16x16x32 form's rate, so it delivers half the flops).
//   A: lane l holds row l%32, k = 8*(l/32) .. +7;  B: lane l holds column l%32, the same k
//   D: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4 in element i (i = 0..15)
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The B operand of a 32x32x16 product whose contraction runs over the 16 rows of two 16x16
// output tiles: lo covers columns 32g .. 32g+15, hi columns 32g+16 .. 32g+31, each packed to
// bf16 (lane (c, blk) holds rows 4*blk .. 4*blk+3 of column c).  One swap with the
// neighbouring 16-lane row leaves lane l with rows 8*(l/32) .. +7 of column 32g + l%32, in
// row order: the lane of an even row keeps its lo rows and takes its partner's lo rows, the
// lane of an odd row takes its partner's hi rows and keeps its own.
__device__ __forceinline__ bf16x8 tiles_to_b32(uint2 lo, uint2 hi) {
  const auto p0 = __builtin_amdgcn_permlane16_swap(lo.x, hi.x, false, false);
  const auto p1 = __builtin_amdgcn_permlane16_swap(lo.y, hi.y, false, false);
  const uint4 v = {p0[0], p1[0], p0[1], p1[1]};
  return __builtin_bit_cast(bf16x8, v);
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
// LDS matrix, lane j gets column c0 + j of rows 4*blk .. 4*blk+3 of that matrix.  p must
// point into LDS.
__device__ __forceinline__ s16x4 lds_read_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}
// The A operand of a 32x32x16 product that matches tiles_to_b32: rows d0 .. d0+31 of the
// transpose of a row-major LDS matrix m (16 rows, row stride `stride` elements), i.e. lane l
// gets column d0 + l%32 of rows 8*(l/32) .. +7, by two transposing reads.  Lane
// l = 16*blk + col of group blk = 2h + u addresses row 8h + col/4 (then 4 rows further),
// columns d0 + 16u + 4*(col%4).
__device__ __forceinline__ bf16x8 lds_read_tr8_rows(const uint16_t* m, int stride, int d0, int lane) {
  const int col = lane % 16, blk = lane / 16;
  const uint16_t* p = m + (8 * (blk / 2) + col / 4) * stride + d0 + 16 * (blk % 2) + 4 * (col % 4);
  return cat_bf16x8(lds_read_tr4(p), lds_read_tr4(p + 4 * stride));
}

// Output tiles of a 16x16 MFMA with rows d and columns the 16 query rows: lane (col, blk)
// holds d = 16 dt + 4 blk .. +3 of query row col for each of the DT tiles (DT even).  The
// values are packed to bf16 and regrouped across the four 16-lane rows, a swap with the row
// two away (permlane32) and then with the neighbouring row (permlane16), so that afterwards
// lane blk holds d = 32 j + 8 blk .. +7 in u[2j] (first four) and u[2j+1] (next four): a
// 16-byte store per j then writes 64 contiguous bytes of every query row, the four lanes of
// the row side by side, instead of four 8-byte pieces 32 bytes apart.
template <int DT>
__device__ __forceinline__ void regroup_rows_bf16(const f32x4 (&o)[DT], uint32_t (&u)[DT][2]) {
  static_assert(DT % 2 == 0, "d-tiles come in pairs");
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const uint2 pk = __builtin_bit_cast(uint2, pack_bf16x4(o[dt]));
    u[dt][0] = pk.x;
    u[dt][1] = pk.y;
  }
#pragma unroll
  for (int i = 0; i < DT / 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto p = __builtin_amdgcn_permlane32_swap(u[2 * i][h], u[2 * i + 1][h], false, false);
      u[2 * i][h] = p[0];
      u[2 * i + 1][h] = p[1];
    }
#pragma unroll
  for (int i = 0; i < DT / 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto p = __builtin_amdgcn_permlane16_swap(u[2 * i][h], u[2 * i + 1][h], false, false);
      u[2 * i][h] = p[0];
      u[2 * i + 1][h] = p[1];
    }
}
// Stores the regrouped values of one query row: dst points at the row's d = 8 blk.
template <int DT, bool NT>
__device__ __forceinline__ void store_regrouped(bf16* dst, const uint32_t (&u)[DT][2]) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int j = 0; j < DT / 2; ++j) {
    const u32x4 v = {u[2 * j][0], u[2 * j][1], u[2 * j + 1][0], u[2 * j + 1][1]};
    if (NT)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + 32 * j));
    else
      *reinterpret_cast<u32x4*>(dst + 32 * j) = v;
  }
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
// The same load with the non-temporal hint, for partials that are read exactly once: the
// token phases measured faster with it (fwd_16k forward token phase 0.270 -> 0.225 ms).
template <int E>
__device__ __forceinline__ void load_raw_nt(const bf16* p, uint32_t (&u)[E / 2]) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (E == 4) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    u[0] = x[0];
    u[1] = x[1];
  } else {
#pragma unroll
    for (int h = 0; h < E / 8; ++h) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 8 * h));
      u[4 * h] = x[0];
      u[4 * h + 1] = x[1];
      u[4 * h + 2] = x[2];
      u[4 * h + 3] = x[3];
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
