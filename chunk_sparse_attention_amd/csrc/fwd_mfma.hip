// fwd_mfma.hip -- bf16 forward on the matrix cores (gfx950).
//
// Token-level softmax-off-by-one attention inside each selected chunk fused with the
// stick-breaking chunk weights ("Hardware-aligned Hierarchical Sparse Attention ...",
// papernotes.org note, 方法详解 › 层次化稀疏注意力（HSA） 第一阶段/第二阶段, 硬件对齐 Kernel).
//
// Two designs.  The chunk-major one (below k_fwd_tile) runs whenever the inverse index fits
// (at most 16384 chunks), for G = 1, 2, 4, 8 and 16; the token-tile one covers longer
// sequences for G = 4, 8 and 16.
//
// Token tiles: one workgroup owns a tile of TT consecutive tokens of one (batch, group) and keeps their
// fp32 outputs in LDS.  The tile's (token, slot) edges are sorted by chunk; each wave takes a
// contiguous range of 16-column jobs (16/G tokens of one chunk, G heads each), holds that
// chunk's key and transposed value operands in registers while its jobs share the chunk, and
// per job computes
//   S^T = K_c Q^T            (keys x columns, MFMA)
//   P   = w * softmax1(S)    (per column, fp32, exp2 with the logit scale folded in)
//   O^T += V_c^T P^T         (MFMA), added into the tile's LDS accumulators.
// Jobs are coloured into rounds in which no token appears twice; the waves of a round add
// into LDS with plain read-add-write and a barrier separates rounds, so the result does not
// depend on wave timing.
#include "hsa_common.h"
#include "hsa_launch.h"
#include "mfma_common.h"
#include "tile_common.h"

namespace hsa {

// Chunk operands in the order one wave's MFMA operand loads consume them, so every load is
// one contiguous 1 KB block (64 lanes x 16 bytes) per chunk, tile and step.
//   ROWS (A operand [key x d], for S^T = K Q^T or dP^T = V dO^T), per chunk:
//     out[((t4 * (D/32) + ks) * 64 + lane) * 8 + e] = src[16*t4 + lane%16][32*ks + 8*(lane/16) + e]
//   TRANS (A operand [d x key], for O^T = V^T P^T or dQ^T = K^T dS^T), per chunk:
//     out[((dt * 2 + s) * 64 + lane) * 8 + e] = src[perm_key(s, lane/16, e)][16*dt + lane%16]
// src is one KV group of a [B, L, Hkv, D] tensor; out is [B*Hkv][nC][64*D].
template <bool TRANS>
__global__ void __launch_bounds__(256) k_prep_ops(const bf16* __restrict__ src, bf16* __restrict__ out,
                                                  int L, int Hkv, int D, int nC) {
  __shared__ uint16_t tile[64][136];
  const int c = blockIdx.x % nC;
  const int bg = blockIdx.x / nC;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const bf16* s0 = src + ((b * L + (size_t)c * 64) * Hkv + g) * D;
  for (int i = threadIdx.x; i < 64 * D / 8; i += 256) {
    const int key = i / (D / 8), d = (i % (D / 8)) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(s0 + (size_t)key * Hkv * D + d);
    *reinterpret_cast<uint4*>(&tile[key][d]) = v;
  }
  __syncthreads();
  bf16* dst = out + ((size_t)bg * nC + c) * 64 * D;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int e = i % 8, lane = (i / 8) % 64, step = i / 512;  // step = t4*KS+ks or dt*2+s
    const int col = lane % 16, blk = lane / 16;
    uint16_t v;
    if (!TRANS) {
      const int ks_n = D / 32, t4 = step / ks_n, ks = step % ks_n;
      v = tile[16 * t4 + col][32 * ks + 8 * blk + e];
    } else {
      const int dt = step / 2, s = step % 2;
      v = tile[perm_key(s, blk, e)][16 * dt + col];
    }
    dst[i].bits = v;
  }
}

template <int D, int TT, int G>
__global__ void __launch_bounds__(512) k_fwd_tile(
    const bf16* __restrict__ Q, const bf16* __restrict__ Kop, const bf16* __restrict__ Vt,
    const int32_t* __restrict__ idx, const float* __restrict__ w,
    const uint32_t* __restrict__ prep, bf16* __restrict__ O, float* __restrict__ lse_out, int L,
    int Hq, int Hkv, int Kt, int nC, int BG, float c2) {
  constexpr int NT = 512, NW = NT / 64;
  constexpr int DP = D + 1;    // padded accumulator row
  constexpr int KS = D / 32;   // k-steps of S^T
  constexpr int DT = D / 16;   // d-tiles of O^T
  constexpr int NMAX = TT * 16;
  __shared__ float acc[TT * G * DP];
  __shared__ uint32_t keys[NMAX];
  __shared__ uint32_t order[NMAX];
  __shared__ int roff[65];
  __shared__ float wsh[TT * 16];
  __shared__ int hdr[3];

  const int bg = blockIdx.x % BG;  // consecutive blocks: different (b, g), XCD-interleaved
  const int tile = blockIdx.x / BG;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int t0 = tile * TT;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;

  // 1. the tile's prepared edges, jobs and rounds; weights; zeroed accumulators
  load_prep<NT, TT>(prep + (size_t)blockIdx.x * prep_words(TT), keys, order, roff, hdr);
  for (int i = tid; i < TT * Kt; i += NT) {
    const int tl = i / Kt, k = i % Kt, t = t0 + tl;
    if (t < L) wsh[tl * 16 + k] = w[((b * L + t) * Hkv + g) * Kt + k];
  }
  for (int i = tid; i < TT * G * DP; i += NT) acc[i] = 0.0f;
  __syncthreads();
  const int n_rounds = hdr[2];

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // this wave's share of round r: [rb(r), re(r))
  auto rb = [&](int r) {
    const int a = roff[r], n = roff[r + 1] - a;
    return a + (int)((long)n * wv / NW);
  };
  auto re = [&](int r) {
    const int a = roff[r], n = roff[r + 1] - a;
    return a + (int)((long)n * (wv + 1) / NW);
  };
  // next job of this wave after job j of round r (or -1): uniform scalar work
  auto next_job = [&](int r, int j) {
    if (j + 1 < re(r)) return j + 1;
    for (int r2 = r + 1; r2 < n_rounds; ++r2)
      if (rb(r2) < re(r2)) return rb(r2);
    return -1;
  };
  const int col = lane % 16, blk = lane / 16;
  const int slot = col / G, head = col % G;
  // D=64: the next chunk's keys and values are prefetched into a second register set.
  // D=128 has no registers to spare for that; its chunk operands load when the chunk changes.
  constexpr bool kPrefetchKV = (D == 64);
  bf16x8 ka[4][KS], kn[4][KS];           // K_c rows (A operand of S^T): current, next
  bf16x8 va[DT][2], vn[DT][2];           // V_c^T rows (A operand of O^T): current, next
  bf16x8 qb[KS], qn[KS];                 // Q^T columns (B operand of S^T): current, next
  int tl_c = 0, k_c = 0, tl_n = 0, k_n = 0;
  bool valid_c = false, valid_n = false;

  auto chunk_of = [&](int j) {
    return __builtin_amdgcn_readfirstlane(edge_chunk(keys[order[j] & 0xffff]));
  };
  auto load_k = [&](bf16x8 (&dst)[4][KS], int c) {
    const bf16* kc = Kop + ((size_t)bg * nC + c) * D * 64 + lane * 8;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[kt][ks] = ld_bf16x8(kc + (kt * KS + ks) * 512);
  };
  auto load_v = [&](bf16x8 (&dst)[DT][2], int c) {
    const bf16* vt = Vt + ((size_t)bg * nC + c) * D * 64 + lane * 8;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < 2; ++s) dst[dt][s] = ld_bf16x8(vt + (dt * 2 + s) * 512);
  };
  auto load_q = [&](bf16x8 (&dst)[KS], int j, int& tl, int& k, bool& valid) {
    const uint32_t job = __builtin_amdgcn_readfirstlane(order[j]);
    const int e0 = (int)(job & 0xffff), cnt = (int)(job >> 16);
    valid = slot < cnt;
    // a padding column reads the job's first token: its weight factor is 0 and nothing of it
    // is stored, and an unconditional load keeps the prefetch free of branches and waits
    const uint32_t ek = keys[e0 + (valid ? slot : 0)];
    tl = edge_token(ek);
    k = edge_slot(ek);
    const bf16* qrow = Q + ((b * L + t0 + tl) * Hq + (size_t)g * G + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = ld_bf16x8(qrow + 32 * ks + 8 * blk);
  };

  // The loads for a wave's next job are issued before its current job is computed; at the
  // top of each job the prefetched registers move into the working set, so the matrix work
  // only waits for loads issued a whole job earlier.  Loads may cross a round barrier: only
  // the LDS accumulation is ordered by rounds.
  int cur = -1, nxt = -1;
  int jn = -1;
  for (int r = 0; r < n_rounds && jn < 0; ++r)
    if (rb(r) < re(r)) jn = rb(r);
  if (jn >= 0) {
    nxt = chunk_of(jn);
    if (kPrefetchKV) {
      load_k(kn, nxt);
      load_v(vn, nxt);
    }
    load_q(qn, jn, tl_n, k_n, valid_n);
  }
  for (int r = 0; r < n_rounds; ++r) {
  const int jr1 = re(r);
  for (int j = rb(r); j < jr1; ++j) {
    if (nxt != cur) {
      if (kPrefetchKV) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) ka[kt][ks] = kn[kt][ks];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int s = 0; s < 2; ++s) va[dt][s] = vn[dt][s];
      } else {
        load_k(ka, nxt);
        load_v(va, nxt);
      }
      cur = nxt;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = qn[ks];
    tl_c = tl_n;
    k_c = k_n;
    valid_c = valid_n;
    jn = next_job(r, j);
    if (jn >= 0) {
      nxt = chunk_of(jn);
      if (kPrefetchKV && nxt != cur) {
        load_k(kn, nxt);
        load_v(vn, nxt);
      }
      load_q(qn, jn, tl_n, k_n, valid_n);
    }
    // S^T = K_c Q^T
    f32x4 s_acc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s_acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s_acc[kt] = mfma_16x16x32(ka[kt][ks], qb[ks], s_acc[kt]);
    }
    // softmax-off-by-one over the 64 keys of this column (4 lanes x 16 values)
    float m = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_acc[kt][i] *= c2;
        m = fmaxf(m, s_acc[kt][i]);
      }
    m = rows4_max(m);
    float sum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_acc[kt][i] = exp2_fast(s_acc[kt][i] - m);
        sum += s_acc[kt][i];
      }
    sum = rows4_sum(sum);
    const float den = exp2_fast(-m) + sum;
    if (valid_c && blk == 0)  // the normaliser, kept for a backward over the same selection
      __builtin_nontemporal_store(m + __builtin_amdgcn_logf(den),
                                  lse_out + (((b * L + t0 + tl_c) * Hkv + g) * Kt + k_c) * G + head);
    const float f = valid_c ? wsh[tl_c * 16 + k_c] / den : 0.0f;
    bf16x8 pb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) pb[s] = pack_bf16x8(s_acc[2 * s] * f, s_acc[2 * s + 1] * f);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      o = mfma_16x16x32(va[dt][0], pb[0], o);
      o = mfma_16x16x32(va[dt][1], pb[1], o);
      if (valid_c) {
        float* dst = acc + (tl_c * G + head) * DP + 16 * dt + 4 * blk;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] += o[i];
      }
    }
  }
  __syncthreads();  // end of round r
  }

  // 5. outputs (rows past L skipped; tokens with no chunk stay 0)
  for (int i = tid; i < TT * G * D / 8; i += NT) {
    const int e = i * 8;
    const int tl = e / (G * D), h = (e / D) % G, d = e % D;
    const int t = t0 + tl;
    if (t >= L) continue;
    const float* src = acc + (tl * G + h) * DP + d;
    f32x4 lo = {src[0], src[1], src[2], src[3]};
    f32x4 hi = {src[4], src[5], src[6], src[7]};
    *reinterpret_cast<bf16x8*>(O + ((b * L + t) * Hq + (size_t)g * G + h) * D + d) = pack_bf16x8(lo, hi);
  }
}

// ---- chunk-major forward ------------------------------------------------------------------
// One block of NW waves per segment of a chunk's selector list (the chunk -> (token, slot)
// index); the chunk's keys and values sit in LDS and the waves take turns at jobs of 16
// query rows (16/G selectors x G heads, row q = selector * G + head):
//   S = Q K_c^T                                  (MFMA; lane: key column, four query rows)
//   softmax-off-by-one over the chunk's 64 keys  (row statistics across 16 lanes)
//   P~ = w P, packed to bf16, to LDS as P~^T
//   O_k^T = V_c^T P~^T                           (MFMA, both operands by transposing reads)
// Each selection edge lies in exactly one segment: its weighted output (bf16, G x D) and the
// normaliser of each of its heads are stored once; a token phase sums the edges of a token.
template <int D, int G, int NW>
__global__ void __launch_bounds__(64 * NW) k_fwd_chunk(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const float* __restrict__ w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ seg_chunk, const int32_t* __restrict__ n_seg,
    const int32_t* __restrict__ seg_order,
    bf16* __restrict__ o_part, float* __restrict__ lse_out, int L, int Hq, int Hkv, int Kn,
    int nC, int seg, int64_t max_seg, float c2) {
  constexpr int TPJ = 16 / G, KS = D / 32, DT = D / 16, NT = 64 * NW;
  // Rows of D + 16 elements (a stride of 8 banks) keep both the 16-byte key reads and the
  // transposing value reads free of LDS bank conflicts.
  constexpr int KROW = D + 16;
  __shared__ __attribute__((aligned(16))) uint16_t kl[64][KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vl[64][KROW];
  // P~^T of a wave's job, 64 key rows of 16 query columns.  Column group j (four columns,
  // 8 bytes) of row r sits at group j ^ ((r / 4) % 4): the 8-byte stores (16 rows at one
  // group) and the transposing reads (4 rows at all groups) then both spread over the banks.
  __shared__ __attribute__((aligned(16))) uint16_t pl[NW][64][16];
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
    *reinterpret_cast<uint4*>(&vl[key][d]) = *reinterpret_cast<const uint4*>(V + cb + key * kvrow + d);
  }
  __syncthreads();
  const int qs_sel = col / G, qs_head = col % G;  // this lane's A-operand row -> selector, head
  const int trow = 4 * blk + col / 4, tcol = 4 * (col % 4);
  const int pcol = 4 * ((col % 4) ^ blk);  // tcol in the swizzled P~^T rows 4*blk + col/4
  const bf16* qbase = Q + ((b * L * Hq + (size_t)g * G + qs_head) * D + 8 * blk);
  const size_t qstride = (size_t)Hq * D;  // per token
  // this lane's query row of job j (a padding row repeats the job's first selector)
  auto load_q = [&](int ej, bf16x8 (&qa)[KS]) {
    const int n_here = min(TPJ, ne - ej);
    const bf16* qr = qbase + (size_t)tok_l[ej + (qs_sel < n_here ? qs_sel : 0)] * qstride;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = ld_bf16x8(qr + 32 * ks);
  };
  bf16x8 qn[KS];
  if (wv * TPJ < ne) load_q(wv * TPJ, qn);
  for (int ej = wv * TPJ; ej < ne; ej += NW * TPJ) {
    const int n_here = min(TPJ, ne - ej);
    bf16x8 qa[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = qn[ks];
    if (ej + NW * TPJ < ne) load_q(ej + NW * TPJ, qn);
    f32x4 sa[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      sa[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sa[t4] = mfma_16x16x32(
            qa[ks], *reinterpret_cast<const bf16x8*>(&kl[16 * t4 + col][32 * ks + 8 * blk]),
            sa[t4]);
    }
    // z = logit * log2(e).  Softmax-off-by-one of a row: P = exp2(z - lse) with
    // lse = log2(1 + sum exp2(z)), evaluated with a shift m as m + log2(exp2(-m) + sum
    // exp2(z - m)).  Any m gives the same value; m = max(0, max z) is needed only when some
    // exp2(z) could overflow, so m = 0 unless a logit of the job exceeds 64.
    float lmax = 0.0f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[t4][i] *= c2;
        lmax = fmaxf(lmax, sa[t4][i]);
      }
    float m[4] = {0.f, 0.f, 0.f, 0.f};
    if (__ballot(lmax > 64.0f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mi = 0.0f;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) mi = fmaxf(mi, sa[t4][i]);
        m[i] = row16_max(mi);
      }
    }
    float lse[4], f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = (4 * blk + i) / G;
      float sum = 0.0f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        sa[t4][i] = exp2_fast(sa[t4][i] - m[i]);
        sum += sa[t4][i];
      }
      const float den = exp2_fast(-m[i]) + row16_sum(sum);
      lse[i] = m[i] + __builtin_amdgcn_logf(den);
      f[i] = s < n_here ? w_l[ej + s] * __builtin_amdgcn_rcpf(den) : 0.0f;
    }
    {  // the normaliser of row 4*blk + col (lanes col < 4), kept for a backward
      const int r = 4 * blk + col, s = r / G;
      const float v = col == 0 ? lse[0] : col == 1 ? lse[1] : col == 2 ? lse[2] : lse[3];
      if (col < 4 && s < n_here)
        __builtin_nontemporal_store(v, lse_out + eo_l[ej + s] * G + r % G);
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[t4][i] *= f[i];
      *reinterpret_cast<s16x4*>(&pl[wv][16 * t4 + col][4 * (blk ^ (col / 4))]) =
          pack_bf16x4(sa[t4]);
    }
    wave_lds_sync();  // P~^T is read transposed below
    // O^T (rows d, columns the 16 query rows) = V_c^T P~^T, 32 keys per product: lane block
    // blk takes keys 32*kk + 4*blk + i and 32*kk + 16 + 4*blk + i in both operands
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pT = cat_bf16x8(lds_read_tr4(&pl[wv][32 * kk + trow][pcol]),
                                   lds_read_tr4(&pl[wv][32 * kk + 16 + trow][pcol]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = mfma_16x16x32(cat_bf16x8(lds_read_tr4(&vl[32 * kk + trow][16 * dt + tcol]),
                                         lds_read_tr4(&vl[32 * kk + 16 + trow][16 * dt + tcol])),
                              pT, o[dt]);
    }
    // regrouped so that each store writes 64 contiguous bytes of every query row (all lanes
    // take part in the cross-lane swaps); measured: chunk phase 1.05 -> 0.83 ms at fwd_64k.
    // At D = 128 the partials are stored non-temporally: the chunk phase loses less than the
    // token phase that reads them gains (at D = 64 the two even out).
    uint32_t u[DT][2];
    regroup_rows_bf16<DT>(o, u);
    if (qs_sel < n_here)  // lane column = query row col: its edge's output
      store_regrouped<DT, D == 128>(o_part + (eo_l[ej + qs_sel] * G + qs_head) * D + 8 * blk, u);
    wave_lds_sync();  // pl reuse by the next job
  }
}

// Token phase of the chunk-major forward: SPLIT waves per (b, t, g) row, each owning a
// contiguous 1/SPLIT of the row's G x D outputs; O = the sum of the row's valid slots'
// weighted outputs in slot order (fp32), rounded once.  Slots that are not valid have no
// partial (their workspace bytes are stale) and are masked out by selection.  The partials
// are read once, with the non-temporal hint; rows of more than 512 outputs are split so that
// a wave keeps at most eight 16-byte loads in flight per slot (measured: d = 128, G = 8
// token phase 0.50 -> 0.465 ms at L = 64K).
template <int D, int G, int SPLIT>
__global__ void __launch_bounds__(256) k_fwd_tok(const bf16* __restrict__ o_part,
                                                 const int32_t* __restrict__ idx,
                                                 bf16* __restrict__ O, int L, int Hkv, int Kn,
                                                 int nC, int64_t rows) {
  // elements of the row's G x D block per lane: at least four (8-byte pieces), so rows of
  // fewer than 256 outputs (G < 4 at d = 64, G = 1 at d = 128) leave the upper lanes idle
  constexpr int E = G * D / 64 / SPLIT >= 4 ? G * D / 64 / SPLIT : 4;
  constexpr int LANES = G * D / SPLIT / E;
  static_assert(LANES >= 1 && LANES <= 64, "one wave covers its part of the row");
  const int lane = threadIdx.x % 64;
  const int64_t wid = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int64_t row = wid / SPLIT;  // (b * L + t) * Hkv + g
  const int part = (int)(wid % SPLIT);
  if (row >= rows) return;  // whole wave
  const int g = (int)(row % Hkv);
  const int64_t bt = row / Hkv;
  const size_t o = (size_t)row * Kn;
  const int c = lane < Kn ? idx[o + lane] : -1;
  const uint64_t vmask = __ballot(c >= 0 && c < nC);
  if (LANES < 64 && lane >= LANES) return;  // after the ballot
  const size_t off = (size_t)part * (G * D / SPLIT) + (size_t)lane * E;
  const bf16* src = o_part + o * (size_t)(G * D) + off;
  float acc[E];
#pragma unroll
  for (int j = 0; j < E; ++j) acc[j] = 0.0f;
  for (int k0 = 0; k0 < Kn; k0 += 8) {
    uint32_t v[8][E / 2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u < Kn) {
        load_raw_nt<E>(src + (size_t)(k0 + u) * G * D, v[u]);
      } else {
#pragma unroll
        for (int j = 0; j < E / 2; ++j) v[u][j] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) add_raw<E>(acc, v[u], k0 + u < Kn && ((vmask >> (k0 + u)) & 1));
  }
  store_row<E>(O + bt * (int64_t)Hkv * G * D + (size_t)g * G * D + off, acc);
}

int tile_tokens(const Dims& d) { return (d.D == 64 ? 64 : 32) / (d.G == 16 ? 2 : 1); }

size_t tile_prep_bytes(const Dims& d) {
  const int tt = tile_tokens(d);
  const size_t tiles = (size_t)d.B * d.Hkv * ((d.L + tt - 1) / tt);
  return (tiles * prep_words(tt) * sizeof(uint32_t) + 255) & ~(size_t)255;
}

template <int TT>
static void launch_prep_tt(const Dims& d, const int32_t* idx, uint32_t* prep, hipStream_t s) {
  const int BG = d.B * d.Hkv;
  const int n_tiles = (d.L + TT - 1) / TT;
  Timed tm(HSA_KERNEL_TILE_PREP, s);
  k_tile_prep<256, TT><<<dim3(BG * n_tiles), 256, 0, s>>>(idx, prep, d.L, d.Hkv, d.K, d.nC, BG,
                                                          16 / d.G);
}

void launch_tile_prep(const Dims& d, const int32_t* idx, void* prep, hipStream_t s) {
  switch (tile_tokens(d)) {
    case 64: launch_prep_tt<64>(d, idx, (uint32_t*)prep, s); break;
    case 32: launch_prep_tt<32>(d, idx, (uint32_t*)prep, s); break;
    default: launch_prep_tt<16>(d, idx, (uint32_t*)prep, s); break;
  }
}

template <int D, int TT, int G>
static void launch_fwd_tile(const Dims& d, const void* Q, const void* K, const void* Vt,
                            const int32_t* idx, const float* w, const void* prep, void* O,
                            float* lse, hipStream_t s) {
  const int BG = d.B * d.Hkv;
  const int n_tiles = (d.L + TT - 1) / TT;
  const float c2 = (float)(d.sm_scale * 1.4426950408889634);  // logit scale * log2(e)
  Timed tm(HSA_KERNEL_FWD, s);
  k_fwd_tile<D, TT, G><<<dim3(BG * n_tiles), 512, 0, s>>>(
      (const bf16*)Q, (const bf16*)K, (const bf16*)Vt, idx, w, (const uint32_t*)prep, (bf16*)O,
      lse, d.L, d.Hq, d.Hkv, d.K, d.nC, BG, c2);
}

template <int D, int TT>
static bool launch_fwd_tile_g(const Dims& d, const void* Q, const void* K, const void* Vt,
                              const int32_t* idx, const float* w, const void* prep, void* O,
                              float* lse, hipStream_t s) {
  switch (d.G) {
    case 4: launch_fwd_tile<D, TT, 4>(d, Q, K, Vt, idx, w, prep, O, lse, s); return true;
    case 8: launch_fwd_tile<D, TT, 8>(d, Q, K, Vt, idx, w, prep, O, lse, s); return true;
    case 16: launch_fwd_tile<D, TT / 2, 16>(d, Q, K, Vt, idx, w, prep, O, lse, s); return true;
  }
  return false;
}

bool fwd_mfma_supported(const Dims& d) {
  // G = 1 and 2 run chunk-major only (the token tiles past 16384 chunks need G >= 4)
  return d.dtype == 1 && (d.D == 64 || d.D == 128) && !(d.flags & 1u) &&
         (((d.G == 4 || d.G == 8 || d.G == 16) && d.nC < 32768) ||
          ((d.G == 1 || d.G == 2) && d.nC <= 16384));
}

bool fwd_chunked(const Dims& d) { return fwd_mfma_supported(d) && d.nC <= 16384; }

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FwdState fwd_state(const Dims& d) {
  FwdState st{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  st.lse = take(sizeof(float) * (size_t)d.B * d.L * d.Hq * d.K);
  if (fwd_chunked(d)) {
    st.ix = index_layout(d, o);
    st.part = take(sizeof(uint16_t) * (size_t)d.B * d.L * d.Hq * d.K * d.D);
  } else {
    st.prep = take(tile_prep_bytes(d));
    st.kop = take(chunk_ops_bytes(d));
  }
  st.total = o;
  return st;
}

size_t fwd_mfma_ws(const Dims& d) {
  return fwd_chunked(d) ? fwd_state(d).total : fwd_state(d).total + chunk_ops_bytes(d);
}

void launch_prep_ops(const Dims& d, const void* src, void* dst, bool trans, hipStream_t s) {
  if (d.nC == 0) return;
  dim3 grid(d.B * d.Hkv * d.nC);
  Timed tm(HSA_KERNEL_PREP_OPS, s);
  if (trans)
    k_prep_ops<true><<<grid, 256, 0, s>>>((const bf16*)src, (bf16*)dst, d.L, d.Hkv, d.D, d.nC);
  else
    k_prep_ops<false><<<grid, 256, 0, s>>>((const bf16*)src, (bf16*)dst, d.L, d.Hkv, d.D, d.nC);
}

size_t chunk_ops_bytes(const Dims& d) {
  return ((size_t)d.B * d.Hkv * d.nC * 64 * d.D * sizeof(uint16_t) + 255) & ~(size_t)255;
}

// waves per segment block of the chunk-major forward (they share the chunk in LDS)
constexpr int kFwdWaves = 8;
constexpr int kFwdWaves128 = 6;  // d = 128: three blocks of six waves fit a CU's LDS

static hipError_t launch_fwd_chunked(const Dims& d, const FwdState& st, const void* Q,
                                     const void* K, const void* V, const int32_t* idx,
                                     const float* w, void* O, char* ws, hipStream_t s,
                                     bool index_ready = false) {
  if (!index_ready) {  // the index of this selection is not in ws yet
    hipError_t e = launch_invidx(d, st.ix, idx, ws, s);
    if (e != hipSuccess) return e;
  }
  const int BG = d.B * d.Hkv;
  const float c2 = (float)(d.sm_scale * 1.4426950408889634);  // logit scale * log2(e)
  if (d.nC > 0) {
    Timed tm(HSA_KERNEL_FWD, s);
    auto go = [&](auto kern, int nw) {
      kern<<<dim3((unsigned)(BG * st.ix.max_seg)), 64 * nw, 0, s>>>(
          (const bf16*)Q, (const bf16*)K, (const bf16*)V, w,
          (const int32_t*)(ws + st.ix.offsets), (const int32_t*)(ws + st.ix.entries),
          (const int32_t*)(ws + st.ix.seg_start), (const int32_t*)(ws + st.ix.seg_chunk),
          (const int32_t*)(ws + st.ix.n_seg), (const int32_t*)(ws + st.ix.seg_order),
          (bf16*)(ws + st.part), (float*)(ws + st.lse),
          d.L, d.Hq, d.Hkv, d.K, d.nC, st.ix.seg, st.ix.max_seg, c2);
    };
    if (d.D == 64) {
      if (d.G == 1) go(k_fwd_chunk<64, 1, kFwdWaves>, kFwdWaves);
      else if (d.G == 2) go(k_fwd_chunk<64, 2, kFwdWaves>, kFwdWaves);
      else if (d.G == 4) go(k_fwd_chunk<64, 4, kFwdWaves>, kFwdWaves);
      else if (d.G == 8) go(k_fwd_chunk<64, 8, kFwdWaves>, kFwdWaves);
      else go(k_fwd_chunk<64, 16, kFwdWaves>, kFwdWaves);
    } else {
      if (d.G == 1) go(k_fwd_chunk<128, 1, kFwdWaves128>, kFwdWaves128);
      else if (d.G == 2) go(k_fwd_chunk<128, 2, kFwdWaves128>, kFwdWaves128);
      else if (d.G == 4) go(k_fwd_chunk<128, 4, kFwdWaves128>, kFwdWaves128);
      else if (d.G == 8) go(k_fwd_chunk<128, 8, kFwdWaves128>, kFwdWaves128);
      else go(k_fwd_chunk<128, 16, kFwdWaves128>, kFwdWaves128);
    }
  }
  {
    Timed tm(HSA_KERNEL_FWD_TOKEN, s);
    const int64_t rows = (int64_t)d.B * d.L * d.Hkv;
    auto go = [&](auto kern, int split) {
      kern<<<dim3((unsigned)((rows * split + 3) / 4)), 256, 0, s>>>(
          (const bf16*)(ws + st.part), idx, (bf16*)O, d.L, d.Hkv, d.K, d.nC, rows);
    };
    if (d.D == 64) {
      if (d.G == 1) go(k_fwd_tok<64, 1, 1>, 1);
      else if (d.G == 2) go(k_fwd_tok<64, 2, 1>, 1);
      else if (d.G == 4) go(k_fwd_tok<64, 4, 1>, 1);
      else if (d.G == 8) go(k_fwd_tok<64, 8, 1>, 1);
      else go(k_fwd_tok<64, 16, 2>, 2);
    } else {
      if (d.G == 1) go(k_fwd_tok<128, 1, 1>, 1);
      else if (d.G == 2) go(k_fwd_tok<128, 2, 1>, 1);
      else if (d.G == 4) go(k_fwd_tok<128, 4, 1>, 1);
      else if (d.G == 8) go(k_fwd_tok<128, 8, 2>, 2);
      else go(k_fwd_tok<128, 16, 4>, 4);
    }
  }
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const Dims& d, const void* Q, const void* K, const void* V,
                           const int32_t* idx, const float* w, void* O, char* ws, hipStream_t s,
                           bool index_ready) {
  const FwdState st = fwd_state(d);
  if (fwd_chunked(d)) return launch_fwd_chunked(d, st, Q, K, V, idx, w, O, ws, s, index_ready);
  char* kop = ws + st.kop;
  char* prep = ws + st.prep;
  float* lse = (float*)(ws + st.lse);
  char* vt = ws + st.total;
  launch_prep_ops(d, K, kop, false, s);
  launch_prep_ops(d, V, vt, true, s);
  if (!index_ready) launch_tile_prep(d, idx, prep, s);
  if (d.D == 64)
    launch_fwd_tile_g<64, 64>(d, Q, kop, vt, idx, w, prep, O, lse, s);
  else
    launch_fwd_tile_g<128, 32>(d, Q, kop, vt, idx, w, prep, O, lse, s);
  return hipGetLastError();
}

}  // namespace hsa
