// bwd_mfma.hip -- bf16 backward on the matrix cores (gfx950), in two phases.
//
// "Hardware-aligned Hierarchical Sparse Attention ...", papernotes.org note, 方法详解 ›
// 硬件对齐 Kernel: the backward first accumulates the gradients of the queries and of the chunk
// weights per token, then the gradients of keys and values per chunk over every token that
// selected it; the chunk weights pass gradient on into the selection scores (same note,
// 层次化稀疏注意力（HSA）, 端到端学习).
//
// The gradients of queries, keys, values, chunk weights and selection scores are the same as
// that two-phase plan's; the order of the work differs.  The chunk phase does all the per-edge
// work.  Per segment of a chunk's selector list (the chunk -> (token, slot) index) and job of
// 16 query rows:
//   S = Q K_c^T, dP = dO V_c^T; P = softmax1(S); D = sum_keys P.dP; dS = w P (dP - D)
//   dV^T += dO^T (w P), dK^T += Q^T dS     (MFMA, registers, fp32 partial per segment)
//   dQ_k^T = K_c^T dS^T                     (MFMA, one bf16 partial per selection edge)
//   dw_edge = sum over the edge's heads of D
// For D = 64 the two waves of a segment take alternate jobs over all 64 keys; for D = 128
// they split the keys and share each job.  A token phase sums each token's dQ partials in
// slot order and applies the stick-breaking chain rule for ds and dQs; a segment pass forms
// dKslc = sum ds * Qs; a fixed-order reduction sums the segments' partials per chunk.
#include "hsa_common.h"
#include "hsa_launch.h"
#include "mfma_common.h"
#include "tile_common.h"  // row reductions

namespace hsa {

// ---- chunk phase, then token phase ----------------------------------------------------------

// dw of the job's edges from the row sums D of rows 4*blk + i (i = 0..3; row r belongs to
// selector r / G): one lane per edge writes the sum of its G rows.  For G >= 4 a selector's
// rows span G/4 lane blocks (added across them, 16 and 32 lanes apart); for G < 4 a lane
// block holds 4/G selectors.
template <int G>
__device__ __forceinline__ void edge_dw(const float (&dr)[4], int blk, int col, int n_here,
                                        int ej, const int64_t* eo_l, float* __restrict__ dw_out) {
  if constexpr (G >= 4) {
    float dsel = (dr[0] + dr[1]) + (dr[2] + dr[3]);
    if (G >= 8) dsel += __shfl_xor(dsel, 16);
    if (G == 16) dsel += __shfl_xor(dsel, 32);
    const int s = (4 * blk) / G;
    if (col == 0 && (4 * blk) % G == 0 && s < n_here) dw_out[eo_l[ej + s]] = dsel;
  } else {
#pragma unroll
    for (int j = 0; j < 4 / G; ++j) {
      const float dsel = G == 2 ? dr[2 * j] + dr[2 * j + 1] : dr[j];
      const int s = (4 * blk) / G + j;
      if (col == 0 && s < n_here) dw_out[eo_l[ej + s]] = dsel;
    }
  }
}

// Chunk phase for D = 64: one block of two waves per segment of a chunk's selector list.  The
// chunk's keys and values sit in LDS; a job takes 16/G selectors (16 query rows, row
// q = selector * G + head), and the two waves take alternate jobs:
//   S = Q K_c^T, dP = dO V_c^T                               (MFMA 16x16x32)
//   P = exp(S - lse), with lse the forward's normaliser (HL) or computed here over the
//   chunk's 64 keys; D = rowsum(P * dP); dS = w P (dP - D)
//   dV^T += dO^T (w P), dK^T += Q^T dS                       (MFMA 32x32x16, registers)
//   dQ_k^T = K_c^T dS^T                                      (MFMA 16x16x32, per edge)
//   dw_edge = sum over the edge's G heads of D
// Every selection edge belongs to exactly one segment, so the edge's dQ contribution (bf16,
// unscaled) and dw are stored once; the segment's dK/dV are fp32 partials that a fixed-order
// reduction sums per chunk.
template <int G, bool HL>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
k_bwd_chunk_mfma(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ w, const bf16* __restrict__ dO, const float* __restrict__ lse_in,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ entries,
    const int32_t* __restrict__ seg_start, const int32_t* __restrict__ seg_chunk,
    const int32_t* __restrict__ n_seg,
    const int32_t* __restrict__ seg_order, float* __restrict__ part_dk, float* __restrict__ part_dv,
    bf16* __restrict__ dq_part, float* __restrict__ dw_out, int L, int Hq, int Hkv, int Kn,
    int nC, int seg, int64_t max_seg, float c2, float sm_scale) {
  // two waves share the segment's chunk in LDS and take alternate jobs; their dK/dV sums
  // meet in LDS at the end
  constexpr int D = 64, TPJ = 16 / G, KS = D / 32, DT = D / 16, NW = 2, NT = 64 * NW;
  // rows of D + 16 elements keep the 16-byte operand reads and the transposing reads free
  // of LDS bank conflicts; the dS^T tile is swizzled as the forward's P~^T tile
  constexpr int KROW = D + 16, WREGION = 2 * 16 * KROW + 64 * 16;
  __shared__ __attribute__((aligned(16))) uint16_t sm[2 * 64 * KROW + NW * WREGION];
  __shared__ int tok_l[kBwdSeg];
  __shared__ int64_t eo_l[kBwdSeg];  // the entry's (b, t, g, slot) index
  __shared__ float w_l[kBwdSeg];
  const int64_t slot = blockIdx.x % max_seg;
  const int bg = (int)(blockIdx.x / max_seg);
  if (slot >= n_seg[bg]) return;  // whole block
  const int64_t sidx = seg_order[(size_t)bg * max_seg + slot];  // segments in token order
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int c = seg_chunk[(size_t)bg * max_seg + sidx];
  const int32_t* off = offsets + (size_t)bg * (nC + 1);
  const int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  const int e0 = off[c] + (int)(sidx - ss[c]) * seg;
  const int ne = min(off[c + 1], e0 + seg) - e0;  // <= seg = kBwdSeg
  const int32_t* ent = entries + (size_t)bg * L * Kn + e0;
  const int tid = threadIdx.x, lane = tid % 64, col = lane % 16, blk = lane / 16;
  const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
  uint16_t (*kl)[KROW] = reinterpret_cast<uint16_t (*)[KROW]>(sm);
  uint16_t (*vl)[KROW] = reinterpret_cast<uint16_t (*)[KROW]>(sm + 64 * KROW);
  uint16_t* wreg = sm + 2 * 64 * KROW + wv * WREGION;  // this wave's job staging
  uint16_t (*ql)[KROW] = reinterpret_cast<uint16_t (*)[KROW]>(wreg);
  uint16_t (*dl)[KROW] = reinterpret_cast<uint16_t (*)[KROW]>(wreg + 16 * KROW);
  uint16_t (*sdl)[16] = reinterpret_cast<uint16_t (*)[16]>(wreg + 32 * KROW);  // dS^T
  const size_t kvrow = (size_t)Hkv * D;
  const size_t cb = ((b * L + (size_t)c * 64) * Hkv + g) * D;
  for (int i = tid; i < ne; i += NT) {
    const int val = ent[i];
    const int t = val / Kn, k = val % Kn;
    const int64_t eo = ((int64_t)(b * L + t) * Hkv + g) * Kn + k;
    tok_l[i] = t;
    eo_l[i] = eo;
    w_l[i] = w[eo];
  }
  for (int i = tid; i < 64 * (D / 8); i += NT) {
    const int key = i / (D / 8), d = (i % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(&kl[key][d]) = *reinterpret_cast<const uint4*>(K + cb + key * kvrow + d);
    *reinterpret_cast<uint4*>(&vl[key][d]) = *reinterpret_cast<const uint4*>(V + cb + key * kvrow + d);
  }
  // dK^T and dV^T as 32x32 tiles: [d2][k2] holds d = 32*d2 + 8*(i/4) + 4*(lane/32) + i%4,
  // keys 32*k2 + lane%32
  f32x16 dk[2][2], dv[2][2];
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dk[d2][k2][i] = 0.0f;
        dv[d2][k2][i] = 0.0f;
      }
  const int qs_sel = col / G, qs_head = col % G;  // this lane's A-operand row -> selector, head
  __syncthreads();

  // this lane's query row of job j (a padding row repeats the job's first selector) and, with
  // HL, the forward's normaliser of the lane's four output rows 4*blk + i: four consecutive
  // heads of one selector for G >= 4 (one 16-byte load), one load per row otherwise
  const size_t row_off = (b * L * Hq + (size_t)g * G + qs_head) * D + 8 * blk;
  const size_t tok_stride = (size_t)Hq * D;
  auto load_rows = [&](int ej, bf16x8 (&qa)[KS], bf16x8 (&da)[KS], float (&le)[4]) {
    const int n_here = min(TPJ, ne - ej);
    const size_t qoff = row_off + (size_t)tok_l[ej + (qs_sel < n_here ? qs_sel : 0)] * tok_stride;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = ld_bf16x8(Q + qoff + 32 * ks);
      da[ks] = ld_bf16x8(dO + qoff + 32 * ks);
    }
    if (HL) {
      if constexpr (G >= 4) {
        const int s2 = (4 * blk) / G, e = ej + (s2 < n_here ? s2 : 0);
        const float4 v = *reinterpret_cast<const float4*>(lse_in + eo_l[e] * G + (4 * blk) % G);
        le[0] = v.x;
        le[1] = v.y;
        le[2] = v.z;
        le[3] = v.w;
      } else {  // the four rows belong to 4/G selectors
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s2 = (4 * blk + i) / G, e = ej + (s2 < n_here ? s2 : 0);
          le[i] = lse_in[eo_l[e] * G + (4 * blk + i) % G];
        }
      }
    }
  };
  bf16x8 qn[KS], dn[KS];
  float len[4] = {0.f, 0.f, 0.f, 0.f};
  if (wv * TPJ < ne) load_rows(wv * TPJ, qn, dn, len);
  for (int ej = wv * TPJ; ej < ne; ej += NW * TPJ) {
    const int n_here = min(TPJ, ne - ej);
    bf16x8 qa[KS], da[KS];
    float lse[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = qn[ks];
      da[ks] = dn[ks];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lse[i] = len[i];
    if (ej + NW * TPJ < ne) load_rows(ej + NW * TPJ, qn, dn, len);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      *reinterpret_cast<bf16x8*>(&ql[col][32 * ks + 8 * blk]) = qa[ks];
      *reinterpret_cast<bf16x8*>(&dl[col][32 * ks + 8 * blk]) = da[ks];
    }
    wave_lds_sync();  // ql/dl are read transposed below
    // S = Q K_c^T, dP = dO V_c^T (rows: the 16 query rows; columns: keys 16*t4 + col)
    f32x4 sa[4], pa[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      sa[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
      pa[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&kl[16 * t4 + col][32 * ks + 8 * blk]);
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&vl[16 * t4 + col][32 * ks + 8 * blk]);
        sa[t4] = mfma_16x16x32(qa[ks], kb, sa[t4]);
        pa[t4] = mfma_16x16x32(da[ks], vb, pa[t4]);
      }
    }
    if (!HL) {  // softmax1 normaliser of each row over the chunk's 64 keys (log2 domain)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) m = fmaxf(m, sa[t4][i] * c2);
        m = row16_max(m);
        float sum = 0.0f;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) sum += exp2_fast(sa[t4][i] * c2 - m);
        sum = row16_sum(sum);
        lse[i] = m + __builtin_amdgcn_logf(exp2_fast(-m) + sum);
      }
    }
    // P, and per row r = 4*blk + i: D = sum over keys of P dP, the selector's weight
    float wr[4], dr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = (4 * blk + i) / G;
      float dsum = 0.0f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        sa[t4][i] = exp2_fast(sa[t4][i] * c2 - lse[i]);
        dsum += sa[t4][i] * pa[t4][i];
      }
      dr[i] = row16_sum(dsum);
      wr[i] = s < n_here ? w_l[ej + s] : 0.0f;
    }
    // dw of each edge: its G rows' D (rows 4*blk .. 4*blk+3 per lane block)
    edge_dw<G>(dr, blk, col, n_here, ej, eo_l, dw_out);
    // dV^T += dO^T (w P), dK^T += Q^T dS on the 32x32x16 product, whose contraction is the
    // job's 16 query rows: A = 32 dimensions of dO^T or Q^T (transposing reads), B = the
    // w P or dS tiles of 32 keys brought to the same rows by one lane swap; dS^T also goes
    // to LDS for dQ
    bf16x8 doT[2], qT[2];
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
      doT[d2] = lds_read_tr8_rows(&dl[0][0], KROW, 32 * d2, lane);
      qT[d2] = lds_read_tr8_rows(&ql[0][0], KROW, 32 * d2, lane);
    }
    const int trow = 4 * blk + col / 4, tcol = 4 * (col % 4);
    const int pcol = 4 * ((col % 4) ^ blk);  // tcol in the swizzled dS^T rows 4*blk + col/4
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      uint2 wpu[2], dsu[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t4 = 2 * k2 + h;
        f32x4 wp, dsv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wp[i] = wr[i] * sa[t4][i];
          dsv[i] = wr[i] * sa[t4][i] * (pa[t4][i] - dr[i]);
        }
        const s16x4 dsb = pack_bf16x4(dsv);
        *reinterpret_cast<s16x4*>(&sdl[16 * t4 + col][4 * (blk ^ (col / 4))]) = dsb;
        wpu[h] = __builtin_bit_cast(uint2, pack_bf16x4(wp));
        dsu[h] = __builtin_bit_cast(uint2, dsb);
      }
      const bf16x8 wpb = tiles_to_b32(wpu[0], wpu[1]), dsb = tiles_to_b32(dsu[0], dsu[1]);
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
        dv[d2][k2] = mfma_32x32x16(doT[d2], wpb, dv[d2][k2]);
        dk[d2][k2] = mfma_32x32x16(qT[d2], dsb, dk[d2][k2]);
      }
    }
    wave_lds_sync();  // sdl is read transposed below
    // dQ^T (rows d, columns the 16 query rows) = K_c^T dS^T over the chunk's keys, 32 keys
    // per product: lane block blk takes keys 32*kk + 4*blk + i and 32*kk + 16 + 4*blk + i in
    // both operands
    f32x4 dq[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 dsT = cat_bf16x8(lds_read_tr4(&sdl[32 * kk + trow][pcol]),
                                    lds_read_tr4(&sdl[32 * kk + 16 + trow][pcol]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dq[dt] = mfma_16x16x32(cat_bf16x8(lds_read_tr4(&kl[32 * kk + trow][16 * dt + tcol]),
                                          lds_read_tr4(&kl[32 * kk + 16 + trow][16 * dt + tcol])),
                               dsT, dq[dt]);
    }
    // the per-edge partials are stored non-temporally: they are read once, by the token
    // phase, and measured faster that way (for the forward's partials it was slower)
    // (regrouped across the lanes first, so that each store writes 64 contiguous bytes of a
    // query row; all lanes take part in the swaps)
    uint32_t u[DT][2];
    regroup_rows_bf16<DT>(dq, u);
    if (qs_sel < n_here)  // lane column = query row col: its edge's partial
      store_regrouped<DT, true>(dq_part + (eo_l[ej + qs_sel] * G + qs_head) * D + 8 * blk, u);
    wave_lds_sync();  // ql/dl/sdl reuse by the next job
  }
  // wave 1's sums meet wave 0's in LDS (dK, then dV); wave 0 stores the segment's partials
  __syncthreads();  // every job is done: the chunk and staging areas are free
  f32x4* xs = reinterpret_cast<f32x4*>(sm);  // 16 x 64 lanes x 16 bytes
  const size_t pb = (size_t)bg * max_seg + sidx;
  // four consecutive d of one key: elements 4j .. 4j+3 of a 32x32 tile
  auto quad = [](const f32x16& v, int j) {
    return f32x4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
  };
  if (wv == 1) {
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) xs[((d2 * 2 + k2) * 4 + j) * 64 + lane] = quad(dk[d2][k2], j);
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 32 * k2 + lane % 32, d = 32 * d2 + 8 * j + 4 * (lane / 32);
          *reinterpret_cast<f32x4*>(part_dk + (pb * 64 + key) * D + d) =
              (quad(dk[d2][k2], j) + xs[((d2 * 2 + k2) * 4 + j) * 64 + lane]) * sm_scale;
        }
  }
  __syncthreads();
  if (wv == 1) {
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) xs[((d2 * 2 + k2) * 4 + j) * 64 + lane] = quad(dv[d2][k2], j);
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 32 * k2 + lane % 32, d = 32 * d2 + 8 * j + 4 * (lane / 32);
          *reinterpret_cast<f32x4*>(part_dv + (pb * 64 + key) * D + d) =
              quad(dv[d2][k2], j) + xs[((d2 * 2 + k2) * 4 + j) * 64 + lane];
        }
  }
}

// Chunk phase for D = 128: two waves per segment split the chunk's 64 keys (wave w owns keys
// 32w .. 32w+31, their dK/dV sums in 128 registers and their value rows as dP's B operand in
// 32 more) and work through the jobs together.
// Per job of 16 query rows (16/G selectors x G heads):
//   the rows of Q and dO are staged once in LDS for both waves;
//   each wave: S and dP over its 32 keys, P (from the forward's normaliser, or its own over
//   the chunk's keys: the row maxima and sums of the two halves meet in LDS), its half of
//   D = sum over keys of P dP (the halves meet in LDS, added in key order), dS over its keys,
//   dV^T and dK^T of its keys, dS^T of its keys to a shared LDS tile;
//   then each wave forms dQ^T = K_c^T dS^T for half of the 128 dimensions, over all 64 keys.
// Each wave stores its keys' segment partials of dK and dV at the end.
template <int G, bool HL>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
k_bwd_chunk_keys(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ w, const bf16* __restrict__ dO, const float* __restrict__ lse_in,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ entries,
    const int32_t* __restrict__ seg_start, const int32_t* __restrict__ seg_chunk,
    const int32_t* __restrict__ n_seg,
    const int32_t* __restrict__ seg_order, float* __restrict__ part_dk, float* __restrict__ part_dv,
    bf16* __restrict__ dq_part, float* __restrict__ dw_out, int L, int Hq, int Hkv, int Kn,
    int nC, int seg, int64_t max_seg, float c2, float sm_scale) {
  constexpr int D = 128, TPJ = 16 / G, KS = D / 32, NT = 128;
  // rows of D + 16 elements: no LDS bank conflicts in the operand and transposing reads
  constexpr int KROW = D + 16;
  __shared__ __attribute__((aligned(16))) uint16_t kl[64][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t ql[16][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t dl[16][KROW];
  // dS^T of the job; column group j of row r sits at group j ^ ((r / 4) % 4), so that the
  // 8-byte stores and the transposing reads both spread over the banks
  __shared__ __attribute__((aligned(16))) uint16_t sdl[64][16];
  __shared__ float xl[3][2][16];  // per wave and row: D half; without HL also max, sum
  __shared__ int tok_l[kBwdSeg];
  __shared__ int64_t eo_l[kBwdSeg];  // the entry's (b, t, g, slot) index
  __shared__ float w_l[kBwdSeg];
  const int64_t slot = blockIdx.x % max_seg;
  const int bg = (int)(blockIdx.x / max_seg);
  if (slot >= n_seg[bg]) return;  // whole block
  const int64_t sidx = seg_order[(size_t)bg * max_seg + slot];  // segments in token order
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int c = seg_chunk[(size_t)bg * max_seg + sidx];
  const int32_t* off = offsets + (size_t)bg * (nC + 1);
  const int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  const int e0 = off[c] + (int)(sidx - ss[c]) * seg;
  const int ne = min(off[c + 1], e0 + seg) - e0;  // <= seg = kBwdSeg
  const int32_t* ent = entries + (size_t)bg * L * Kn + e0;
  const int tid = threadIdx.x, lane = tid % 64, col = lane % 16, blk = lane / 16;
  const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
  const size_t kvrow = (size_t)Hkv * D;
  const size_t cb = ((b * L + (size_t)c * 64) * Hkv + g) * D;
  for (int i = tid; i < ne; i += NT) {
    const int val = ent[i];
    const int t = val / Kn, k = val % Kn;
    const int64_t eo = ((int64_t)(b * L + t) * Hkv + g) * Kn + k;
    tok_l[i] = t;
    eo_l[i] = eo;
    w_l[i] = w[eo];
  }
  for (int i = tid; i < 64 * (D / 8); i += NT) {
    const int key = i / (D / 8), d = (i % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(&kl[key][d]) = *reinterpret_cast<const uint4*>(K + cb + key * kvrow + d);
  }
  // the value rows of this wave's keys stay in registers as dP's B operand
  bf16x8 vb[2][KS];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      vb[t2][ks] = ld_bf16x8(V + cb + (32 * wv + 16 * t2 + col) * kvrow + 32 * ks + 8 * blk);
  // dK^T and dV^T of this wave's keys as 32x32 tiles: [d4] holds keys 32*wv + lane%32,
  // d = 32*d4 + 8*(i/4) + 4*(lane/32) + i%4
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[d4][i] = 0.0f;
      dv[d4][i] = 0.0f;
    }
  const int qs_sel = col / G, qs_head = col % G;  // this lane's query row -> selector, head
  const int trow = 4 * blk + col / 4, tcol = 4 * (col % 4);
  const int pcol = 4 * ((col % 4) ^ blk);  // tcol in the swizzled dS^T rows 4*blk + col/4
  // staging of job j: thread tid copies 32 bytes of row tid/8 of Q and of dO (a padding row
  // repeats the job's first selector)
  const int srow = tid / 8, spc = tid % 8;
  const size_t srow_off = (b * L * Hq + (size_t)g * G + srow % G) * D + 16 * spc;
  const size_t tok_stride = (size_t)Hq * D;
  // the rows of job ej, returned by value so that they stay in registers
  struct JobRows {
    uint4 q0, q1, d0, d1;
    float4 le;
  };
  auto fetch = [&](int ej) {
    JobRows r;
    const int n_here = min(TPJ, ne - ej);
    const int s2 = srow / G;
    const size_t qoff = srow_off + (size_t)tok_l[ej + (s2 < n_here ? s2 : 0)] * tok_stride;
    r.q0 = *reinterpret_cast<const uint4*>(Q + qoff);
    r.q1 = *reinterpret_cast<const uint4*>(Q + qoff + 8);
    r.d0 = *reinterpret_cast<const uint4*>(dO + qoff);
    r.d1 = *reinterpret_cast<const uint4*>(dO + qoff + 8);
    r.le = float4{0.f, 0.f, 0.f, 0.f};
    if (HL) {  // the normaliser of this lane's four output rows 4*blk .. 4*blk+3
      if constexpr (G >= 4) {
        const int s3 = (4 * blk) / G, e = ej + (s3 < n_here ? s3 : 0);
        r.le = *reinterpret_cast<const float4*>(lse_in + eo_l[e] * G + (4 * blk) % G);
      } else {  // the four rows belong to 4/G selectors
        float le[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s3 = (4 * blk + i) / G, e = ej + (s3 < n_here ? s3 : 0);
          le[i] = lse_in[eo_l[e] * G + (4 * blk + i) % G];
        }
        r.le = float4{le[0], le[1], le[2], le[3]};
      }
    }
    return r;
  };
  __syncthreads();
  JobRows nxt = {};
  if (ne > 0) nxt = fetch(0);
  for (int ej = 0; ej < ne; ej += TPJ) {
    const int n_here = min(TPJ, ne - ej);
    float lse[4] = {nxt.le.x, nxt.le.y, nxt.le.z, nxt.le.w};
    *reinterpret_cast<uint4*>(&ql[srow][16 * spc]) = nxt.q0;
    *reinterpret_cast<uint4*>(&ql[srow][16 * spc + 8]) = nxt.q1;
    *reinterpret_cast<uint4*>(&dl[srow][16 * spc]) = nxt.d0;
    *reinterpret_cast<uint4*>(&dl[srow][16 * spc + 8]) = nxt.d1;
    __syncthreads();  // the job's rows are staged
    if (ej + TPJ < ne) nxt = fetch(ej + TPJ);
    // S = Q K^T, dP = dO V^T over this wave's keys 32*wv + 16*t2 + col (rows: the 16 query
    // rows, four per lane block)
    f32x4 sa[2], pa[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      sa[t2] = f32x4{0.f, 0.f, 0.f, 0.f};
      pa[t2] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&ql[col][32 * ks + 8 * blk]);
      const bf16x8 da = *reinterpret_cast<const bf16x8*>(&dl[col][32 * ks + 8 * blk]);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int key = 32 * wv + 16 * t2 + col;
        sa[t2] = mfma_16x16x32(qa, *reinterpret_cast<const bf16x8*>(&kl[key][32 * ks + 8 * blk]),
                               sa[t2]);
        pa[t2] = mfma_16x16x32(da, vb[t2][ks], pa[t2]);
      }
    }
    if (!HL) {  // softmax1 normaliser of each row over the chunk's 64 keys (log2 domain)
      float mh[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) m = fmaxf(m, sa[t2][i] * c2);
        mh[i] = row16_max(m);
        if (col == 0) xl[1][wv][4 * blk + i] = mh[i];
      }
      __syncthreads();
      float sh[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mh[i] = fmaxf(xl[1][0][4 * blk + i], xl[1][1][4 * blk + i]);
        float sum = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) sum += exp2_fast(sa[t2][i] * c2 - mh[i]);
        sh[i] = row16_sum(sum);
        if (col == 0) xl[2][wv][4 * blk + i] = sh[i];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sum = xl[2][0][4 * blk + i] + xl[2][1][4 * blk + i];
        lse[i] = mh[i] + __builtin_amdgcn_logf(exp2_fast(-mh[i]) + sum);
      }
    }
    // P; this wave's half of D = sum over keys of P dP per row r = 4*blk + i
    float wr[4], dr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = (4 * blk + i) / G;
      float dsum = 0.0f;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        sa[t2][i] = exp2_fast(sa[t2][i] * c2 - lse[i]);
        dsum += sa[t2][i] * pa[t2][i];
      }
      dsum = row16_sum(dsum);
      if (col == 0) xl[0][wv][4 * blk + i] = dsum;
      wr[i] = s < n_here ? w_l[ej + s] : 0.0f;
    }
    __syncthreads();  // both halves of D
#pragma unroll
    for (int i = 0; i < 4; ++i) dr[i] = xl[0][0][4 * blk + i] + xl[0][1][4 * blk + i];
    if (wv == 0) edge_dw<G>(dr, blk, col, n_here, ej, eo_l, dw_out);  // each edge: its G rows' D
    // dV^T += dO^T (w P), dK^T += Q^T dS over this wave's 32 keys on the 32x32x16 product
    // (contraction: the job's 16 query rows; the B operands brought to the A operands' rows
    // by one lane swap); dS^T of its keys to the shared tile
    uint2 wpu[2], dsu[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      f32x4 wp, dsv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wp[i] = wr[i] * sa[t2][i];
        dsv[i] = wr[i] * sa[t2][i] * (pa[t2][i] - dr[i]);
      }
      const s16x4 dsb = pack_bf16x4(dsv);
      *reinterpret_cast<s16x4*>(&sdl[32 * wv + 16 * t2 + col][4 * (blk ^ (col / 4))]) = dsb;
      wpu[t2] = __builtin_bit_cast(uint2, pack_bf16x4(wp));
      dsu[t2] = __builtin_bit_cast(uint2, dsb);
    }
    {
      const bf16x8 wpb = tiles_to_b32(wpu[0], wpu[1]), dsb = tiles_to_b32(dsu[0], dsu[1]);
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        dv[d4] = mfma_32x32x16(lds_read_tr8_rows(&dl[0][0], KROW, 32 * d4, lane), wpb, dv[d4]);
        dk[d4] = mfma_32x32x16(lds_read_tr8_rows(&ql[0][0], KROW, 32 * d4, lane), dsb, dk[d4]);
      }
    }
    __syncthreads();  // the shared dS^T tile is complete
    // dQ^T rows d = 64*wv .. 64*wv+63 (columns: the 16 query rows) = K_c^T dS^T over the 64
    // keys, 32 keys per product: lane block blk takes keys 32*kk + 4*blk + i and
    // 32*kk + 16 + 4*blk + i in both operands
    f32x4 dq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 dsT = cat_bf16x8(lds_read_tr4(&sdl[32 * kk + trow][pcol]),
                                    lds_read_tr4(&sdl[32 * kk + 16 + trow][pcol]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 64 * wv + 16 * j;
        dq[j] = mfma_16x16x32(cat_bf16x8(lds_read_tr4(&kl[32 * kk + trow][d0 + tcol]),
                                         lds_read_tr4(&kl[32 * kk + 16 + trow][d0 + tcol])),
                              dsT, dq[j]);
      }
    }
    // this wave's half of the edge's partial, regrouped across the lanes and stored
    // non-temporally, as in the d = 64 chunk phase
    uint32_t u[4][2];
    regroup_rows_bf16<4>(dq, u);
    if (qs_sel < n_here)  // lane column = query row col
      store_regrouped<4, true>(dq_part + (eo_l[ej + qs_sel] * G + qs_head) * D + 64 * wv + 8 * blk,
                               u);
    // no barrier here: the next job restages Q and dO after the dK/dV barrier above, and
    // rewrites dS^T and the row exchange only after its own exchange barrier
  }
  const size_t pb = (size_t)bg * max_seg + sidx;
  const int key = 32 * wv + lane % 32;
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * d4 + 8 * j + 4 * (lane / 32);
      *reinterpret_cast<f32x4*>(part_dk + (pb * 64 + key) * D + d) =
          f32x4{dk[d4][4 * j], dk[d4][4 * j + 1], dk[d4][4 * j + 2], dk[d4][4 * j + 3]} * sm_scale;
      *reinterpret_cast<f32x4*>(part_dv + (pb * 64 + key) * D + d) =
          f32x4{dv[d4][4 * j], dv[d4][4 * j + 1], dv[d4][4 * j + 2], dv[d4][4 * j + 3]};
    }
}

// Token phase: one wave per (b, t, g) row.  dQ = sm_scale * the sum of the chunk
// phase's partials over the token's valid slots in slot order; ds by the stick-breaking chain
// rule from the edges' dw (fp64, newest slot first); dQs = sel_scale * sum_k ds_k Kslc[c_k].
// The slot data and every slot's partial are loaded together: a slot that is not valid has no
// partial or dw (its workspace bytes are stale) and is masked out by selection.
template <int D, int G>
__global__ void __launch_bounds__(256) k_bwd_tok(
    const bf16* __restrict__ dq_part, const float* __restrict__ dw_in,
    const int32_t* __restrict__ idx, const float* __restrict__ score,
    const float* __restrict__ w, const bf16* __restrict__ Kslc, bf16* __restrict__ dQ,
    bf16* __restrict__ dQs, float* __restrict__ ds_out, int L, int Hkv, int Kn, int nC,
    int64_t rows, float sm_scale, float sel_scale, int softmax_w) {
  // elements of the row's G x D block per lane: at least four (8-byte pieces), so rows of
  // fewer than 256 values (G < 4 at d = 64, G = 1 at d = 128) leave the upper lanes idle
  constexpr int E = G * D / 64 >= 4 ? G * D / 64 : 4;
  constexpr int LANES = G * D / E;
  constexpr int F = D / 64;  // features of dQs per lane: lane + 64 f
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // (b * L + t) * Hkv + g
  if (row >= rows) return;  // whole wave
  const int g = (int)(row % Hkv);
  const int64_t bt = row / Hkv;
  const int64_t b = bt / L;
  const size_t o = (size_t)row * Kn;
  int c = -1;
  float wk = 0.0f, sk = 0.0f, dwk = 0.0f;
  if (lane < Kn) {
    c = idx[o + lane];
    wk = w[o + lane];
    sk = score[o + lane];
    dwk = dw_in[o + lane];
  }
  const bool valid = c >= 0 && c < nC;
  const bool dq_lane = LANES == 64 || lane < LANES;
  const bf16* src = dq_part + o * (size_t)(G * D) + (size_t)(dq_lane ? lane : 0) * E;
  float acc[E];
#pragma unroll
  for (int j = 0; j < E; ++j) acc[j] = 0.0f;
  const uint64_t vmask = __ballot(valid);
  for (int k0 = 0; dq_lane && k0 < Kn; k0 += 8) {
    uint32_t v[8][E / 2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u < Kn) {
        if constexpr (D == 64)  // measured: faster at d = 64, slower at d = 128
          load_raw_nt<E>(src + (size_t)(k0 + u) * G * D, v[u]);
        else
          load_raw<E>(src + (size_t)(k0 + u) * G * D, v[u]);
      } else {
#pragma unroll
        for (int j = 0; j < E / 2; ++j) v[u][j] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) add_raw<E>(acc, v[u], k0 + u < Kn && ((vmask >> (k0 + u)) & 1));
  }
#pragma unroll
  for (int j = 0; j < E; ++j) acc[j] *= sm_scale;
  if (dq_lane)
    store_row<E>(dQ + bt * (int64_t)Hkv * G * D + (size_t)g * G * D + (size_t)lane * E, acc);
  // stick-breaking: ds_k = dw_k w_k (1 - p_k) - p_k * sum_{k' > k} dw_k' w_k'  (fp64, suffix
  // from the last slot); softmax weights: ds_k = w_k (dw_k - sum_j w_j dw_j)  (fp64, slot order)
  const double dww = valid ? (double)dwk * (double)wk : 0.0;
  const int2 dwi = __builtin_bit_cast(int2, dww);
  double suffix = 0.0, mean = 0.0;
  if (softmax_w) {
    for (int k2 = 0; k2 < Kn; ++k2)
      mean += __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(dwi.x, k2),
                                                   __builtin_amdgcn_readlane(dwi.y, k2)));
  } else {
    for (int k2 = Kn - 1; k2 >= 0; --k2) {
      const int2 vi = make_int2(__builtin_amdgcn_readlane(dwi.x, k2),
                                __builtin_amdgcn_readlane(dwi.y, k2));
      if (k2 > lane) suffix += __builtin_bit_cast(double, vi);
    }
  }
  float dsk = 0.0f;
  if (valid) {
    if (softmax_w) {
      dsk = (float)((double)wk * ((double)dwk - mean));
    } else {
      const double p = sigmoid_d((double)sk);
      dsk = (float)(dww * (1.0 - p) - p * suffix);
    }
  }
  if (lane < Kn) ds_out[o + lane] = dsk;
  // dQs (features lane + 64 f), slots in order; the rows of the valid slots load together
  float a[F];
#pragma unroll
  for (int f = 0; f < F; ++f) a[f] = 0.0f;
  if (nC > 0) {
    const int cv = valid ? c : 0;
    for (int k0 = 0; k0 < Kn; k0 += 8) {
      float kv[8][F];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ck = __builtin_amdgcn_readlane(cv, min(k0 + u, Kn - 1));
#pragma unroll
        for (int f = 0; f < F; ++f)
          kv[u][f] = to_f32(Kslc[((b * nC + ck) * Hkv + g) * D + lane + 64 * f]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        const float dsv = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dsk), min(k, Kn - 1)));
        if (k < Kn && ((vmask >> k) & 1)) {
#pragma unroll
          for (int f = 0; f < F; ++f) a[f] += dsv * kv[u][f];
        }
      }
    }
  }
#pragma unroll
  for (int f = 0; f < F; ++f) dQs[row * D + lane + 64 * f] = from_f32<bf16>(a[f] * sel_scale);
}

// dKslc partial of one segment of a chunk's selector list (features lane + 64 f per lane):
// sel_scale * sum over the segment's selectors of ds * Qs.  Four waves take a quarter of the
// list each, in list order; their sums are added in wave order.
template <int D>
__global__ void __launch_bounds__(256) k_bwd_dks(
    const bf16* __restrict__ Qs, const float* __restrict__ ds, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ seg_chunk, const int32_t* __restrict__ n_seg,
    float* __restrict__ part_dks, int L, int Hkv, int Kn, int nC, int seg, int64_t max_seg,
    float sel_scale) {
  constexpr int NW = 4, F = D / 64;
  __shared__ int tok_l[kBwdSeg];
  __shared__ float ds_l[kBwdSeg];
  __shared__ float wsum[NW][D];
  const int64_t sidx = blockIdx.x % max_seg;
  const int bg = (int)(blockIdx.x / max_seg);
  if (sidx >= n_seg[bg]) return;  // whole block
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int c = seg_chunk[(size_t)bg * max_seg + sidx];
  const int32_t* off = offsets + (size_t)bg * (nC + 1);
  const int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  const int e0 = off[c] + (int)(sidx - ss[c]) * seg;
  const int ne = min(off[c + 1], e0 + seg) - e0;
  const int32_t* ent = entries + (size_t)bg * L * Kn + e0;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  for (int i = tid; i < ne; i += 64 * NW) {
    const int val = ent[i];
    const int t = val / Kn, k = val % Kn;
    tok_l[i] = t;
    ds_l[i] = ds[((b * L + t) * Hkv + g) * Kn + k];
  }
  __syncthreads();
  const bf16* qs = Qs + (b * L * Hkv + g) * D + lane;
  const size_t tstride = (size_t)Hkv * D;
  const int i0 = ne * wave / NW, i1 = ne * (wave + 1) / NW;
  float a[F];
#pragma unroll
  for (int f = 0; f < F; ++f) a[f] = 0.0f;
  int i = i0;
  for (; i + 8 <= i1; i += 8) {  // eight rows in flight, summed in list order
    float v[8][F];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int f = 0; f < F; ++f) v[u][f] = to_f32(qs[(size_t)tok_l[i + u] * tstride + 64 * f]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int f = 0; f < F; ++f) a[f] += ds_l[i + u] * v[u][f];
  }
  for (; i < i1; ++i)
#pragma unroll
    for (int f = 0; f < F; ++f) a[f] += ds_l[i] * to_f32(qs[(size_t)tok_l[i] * tstride + 64 * f]);
#pragma unroll
  for (int f = 0; f < F; ++f) wsum[wave][lane + 64 * f] = a[f];
  __syncthreads();
  if (wave == 0)
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int e = lane + 64 * f;
      part_dks[((size_t)bg * max_seg + sidx) * D + e] =
          (((wsum[0][e] + wsum[1][e]) + wsum[2][e]) + wsum[3][e]) * sel_scale;
    }
}

bool bwd_mfma_supported(const Dims& d) {
  return d.dtype == 1 && (d.D == 64 || d.D == 128) &&
         (d.G == 1 || d.G == 2 || d.G == 4 || d.G == 8 || d.G == 16) && d.nC < 32768 &&
         !(d.flags & 1u);
}

// Chunk phase, token phase (+ dKslc partials), reduction.
static hipError_t launch_bwd_fused(const Dims& d, const BwdLayout& lay, const void* Q,
                                   const void* K, const void* V, const void* Qs,
                                   const void* Kslc, const int32_t* idx, const float* score,
                                   const float* w, const void* dO, void* dQ, void* dK, void* dV,
                                   void* dQs, float* dKslc, bool fold, bool after_fwd, char* ws,
                                   hipStream_t s) {
  const int BG = d.B * d.Hkv;
  const float c2 = (float)(d.sm_scale * 1.4426950408889634);
  if (d.nC > 0) {
    dim3 grid((unsigned)(BG * lay.max_seg));
    auto go = [&](auto kern) {
      Timed tm(HSA_KERNEL_BWD_P2, s);
      kern<<<grid, 128, 0, s>>>((const bf16*)Q, (const bf16*)K, (const bf16*)V, w,
                               (const bf16*)dO, (const float*)(ws + lay.lse),
                               (const int32_t*)(ws + lay.offsets),
                               (const int32_t*)(ws + lay.entries),
                               (const int32_t*)(ws + lay.seg_start),
                               (const int32_t*)(ws + lay.seg_chunk),
                               (const int32_t*)(ws + lay.n_seg),
                               (const int32_t*)(ws + lay.seg_order), (float*)(ws + lay.part_dk),
                               (float*)(ws + lay.part_dv), (bf16*)(ws + lay.dq_part),
                               (float*)(ws + lay.dw), d.L, d.Hq, d.Hkv, d.K, d.nC, lay.seg,
                               lay.max_seg, c2, (float)d.sm_scale);
    };
    if (d.D == 64) {
      if (d.G == 1) after_fwd ? go(k_bwd_chunk_mfma<1, true>) : go(k_bwd_chunk_mfma<1, false>);
      else if (d.G == 2) after_fwd ? go(k_bwd_chunk_mfma<2, true>) : go(k_bwd_chunk_mfma<2, false>);
      else if (d.G == 4) after_fwd ? go(k_bwd_chunk_mfma<4, true>) : go(k_bwd_chunk_mfma<4, false>);
      else if (d.G == 8) after_fwd ? go(k_bwd_chunk_mfma<8, true>) : go(k_bwd_chunk_mfma<8, false>);
      else after_fwd ? go(k_bwd_chunk_mfma<16, true>) : go(k_bwd_chunk_mfma<16, false>);
    } else {
      if (d.G == 1) after_fwd ? go(k_bwd_chunk_keys<1, true>) : go(k_bwd_chunk_keys<1, false>);
      else if (d.G == 2) after_fwd ? go(k_bwd_chunk_keys<2, true>) : go(k_bwd_chunk_keys<2, false>);
      else if (d.G == 4) after_fwd ? go(k_bwd_chunk_keys<4, true>) : go(k_bwd_chunk_keys<4, false>);
      else if (d.G == 8) after_fwd ? go(k_bwd_chunk_keys<8, true>) : go(k_bwd_chunk_keys<8, false>);
      else after_fwd ? go(k_bwd_chunk_keys<16, true>) : go(k_bwd_chunk_keys<16, false>);
    }
  }
  {
    Timed tm(HSA_KERNEL_BWD_P1, s);
    const int64_t rows = (int64_t)d.B * d.L * d.Hkv;
    auto go = [&](auto kern) {
      kern<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(
          (const bf16*)(ws + lay.dq_part), (const float*)(ws + lay.dw), idx, score, w,
          (const bf16*)Kslc, (bf16*)dQ, (bf16*)dQs, (float*)(ws + lay.ds), d.L, d.Hkv, d.K,
          d.nC, rows, (float)d.sm_scale, (float)d.sel_scale, softmax_w(d));
    };
    if (d.D == 64) {
      if (d.G == 1) go(k_bwd_tok<64, 1>);
      else if (d.G == 2) go(k_bwd_tok<64, 2>);
      else if (d.G == 4) go(k_bwd_tok<64, 4>);
      else if (d.G == 8) go(k_bwd_tok<64, 8>);
      else go(k_bwd_tok<64, 16>);
    } else {
      if (d.G == 1) go(k_bwd_tok<128, 1>);
      else if (d.G == 2) go(k_bwd_tok<128, 2>);
      else if (d.G == 4) go(k_bwd_tok<128, 4>);
      else if (d.G == 8) go(k_bwd_tok<128, 8>);
      else go(k_bwd_tok<128, 16>);
    }
    auto dks = d.D == 64 ? k_bwd_dks<64> : k_bwd_dks<128>;
    if (d.nC > 0)
      dks<<<dim3((unsigned)(BG * lay.max_seg)), 256, 0, s>>>(
          (const bf16*)Qs, (const float*)(ws + lay.ds), (const int32_t*)(ws + lay.offsets),
          (const int32_t*)(ws + lay.entries), (const int32_t*)(ws + lay.seg_start),
          (const int32_t*)(ws + lay.seg_chunk), (const int32_t*)(ws + lay.n_seg),
          (float*)(ws + lay.part_dks), d.L, d.Hkv, d.K, d.nC, lay.seg, lay.max_seg,
          (float)d.sel_scale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(d, lay, dK, dV, dKslc, fold, ws, s);
}

hipError_t launch_bwd_mfma(const Dims& d, const BwdLayout& lay, const void* Q, const void* K,
                           const void* V, const void* Qs, const void* Kslc, const int32_t* idx,
                           const float* score, const float* w, const float* lse,
                           const void* dO, void* dQ, void* dK, void* dV, void* dQs,
                           float* dKslc, bool fold, bool after_fwd, char* ws, hipStream_t s) {
  // after the chunk-major forward the index of this selection is in place
  if (!(after_fwd && fwd_chunked(d))) {
    hipError_t e = launch_invidx(d, lay, idx, ws, s);
    if (e != hipSuccess) return e;
  }
  if (lse) {  // the caller's normalisers replace whatever the state holds
    hipError_t e = launch_lse_import(d, lse, (float*)(ws + lay.lse), s);
    if (e != hipSuccess) return e;
  }
  return launch_bwd_fused(d, lay, Q, K, V, Qs, Kslc, idx, score, w, dO, dQ, dK, dV, dQs, dKslc,
                          fold, after_fwd || lse != nullptr, ws, s);
}

}  // namespace hsa
