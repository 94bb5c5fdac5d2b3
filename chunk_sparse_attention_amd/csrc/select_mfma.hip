// select_mfma.hip -- top-K chunk selection for bf16 inputs: a matrix-core candidate filter
// followed by exact rescoring of the few candidates that can matter.
//
// Chunk selection ("Hardware-aligned Hierarchical Sparse Attention ...", papernotes.org note,
// 方法详解 › 层次化稀疏注意力（HSA）, Chunk Selection): every token scores each earlier chunk's
// pooled key with its selection query and keeps the top-K, per query group; the chunk
// weights are stick-breaking over the sigmoid of the ranked scores (same section, 第二阶段).
//
// The result is the exact one: scores are the fp64 dot products of the stored values,
// rounded once to fp32, ranked by (score desc, chunk asc).  Only the work is reduced.
//   1. Every candidate's sign(scale) * q.k, which orders the chunks as their scores do, is
//      computed approximately on the matrix cores (bf16 products are exact in fp32, so the
//      fp32 sum is off by at most E = |q| * max|k| * (D+8) * 2^-24; a factor 2 of headroom
//      is added, which also covers two chunks whose scores round to the same fp32 value).
//   2. T = the K-th largest approximate value of the token.  Every chunk of the exact top-K
//      has an approximate value >= T - 2E: if V is the exact K-th largest value, then T <=
//      V + E (else K chunks would lie above V exactly) and each member lies >= V - E.
//      The four lanes of a token keep only their KP largest approximate scores, and T is
//      taken as the K-th largest of those 4 KP values: a subset's K-th largest is at most
//      the whole set's, so the bound still holds (a lane holding more than KP of the top-K
//      only lowers T and adds candidates).
//   3. The chunks at or above T - 2E (about K per token) are rescored exactly in fp64 and
//      ranked; a token with more than kSelCap such chunks, or any non-finite value, is
//      scored exactly over all its candidates instead.
#include "hsa_common.h"
#include "hsa_launch.h"
#include "mfma_common.h"
#include "tile_common.h"

namespace hsa {

constexpr int kSelCap = 48;  // chunks rescored exactly per token

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of squares of eight bf16 values (four bf16 pair dot products; only bounds use it, and
// its rounding is far inside their headroom).
__device__ __forceinline__ float sq8(bf16x8 v) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = __builtin_bit_cast(bf16x2, w[i]);
    s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
  }
  return s;
}

// Keeps the KP largest values seen in top[] (descending): the new list is the top KP of
// the old one and v, each entry the median of its old neighbours and v.
template <int KP>
__device__ __forceinline__ void keep_top(float (&top)[KP], float v) {
  float old[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) old[j] = top[j];
  top[0] = __builtin_amdgcn_fmed3f(old[0], v, __builtin_inff());
#pragma unroll
  for (int j = 1; j < KP; ++j) top[j] = __builtin_amdgcn_fmed3f(old[j - 1], old[j], v);
}

// Order-preserving 32-bit image of a float (NaN never reaches it).
__device__ __forceinline__ uint32_t ord_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Output slot k of one (token, group) row from its ranked key (0: a masked slot), with the
// stick-breaking weight: the sigmoid of the score times the stick left by slots < k.
__device__ __forceinline__ void write_slot(uint64_t key, int k, size_t o, double& rem,
                                           int32_t* idx, float* score, float* w) {
  if (key == 0) {
    idx[o + k] = -1;
    score[o + k] = -__builtin_inff();
    w[o + k] = 0.0f;
  } else {
    const float sc = key_score(key);
    const double p = sigmoid_d((double)sc);
    idx[o + k] = key_chunk(key);
    score[o + k] = sc;
    w[o + k] = (float)(p * rem);
    rem *= 1.0 - p;
  }
}

// Value of lane j (0..3, the same in every lane) of each quad of lanes, in every lane of it.
__device__ __forceinline__ double quad_bcast_f64(double x, int j) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int src = (__lane_id() & ~3) | j;
  const int lo = __builtin_amdgcn_ds_bpermute(src * 4, (int)(uint32_t)u);
  const int hi = __builtin_amdgcn_ds_bpermute(src * 4, (int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Inserts key into a descending list of N keys (the smallest falls off).
template <int N>
__device__ __forceinline__ void insert_key(uint64_t (&tk)[N], uint64_t key) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (key > tk[i]) {
      const uint64_t x = tk[i];
      tk[i] = key;
      key = x;
    }
}

template <int D, int KL, int KP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) k_select_mfma(const bf16* __restrict__ Qs,
                                                     const bf16* __restrict__ Kslc,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ score,
                                                     float* __restrict__ w, int L, int Hkv,
                                                     int Kt, int nC, int BG, double sel_scale) {
  constexpr int KS = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t kl[64][D + 8];  // a group of 64 chunks
  __shared__ int cnt[64];
  __shared__ int fall[64];
  __shared__ int candl[64][kSelCap];
  const int bg = blockIdx.x % BG;
  // query chunk of the tile (its tokens see chunks < q); a tile's work grows with q, so the
  // grid hands out the last tiles first and the short ones fill in behind them
  const int q = (int)(gridDim.x / BG) - 1 - (int)(blockIdx.x / BG);
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int t0 = q * 64;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int col = lane % 16, blk = lane / 16;
  const int m = min(q, nC);
  const int tl = 16 * wave + col;  // this lane's token in the tile (MFMA column)
  const int t = t0 + tl;
  const float sel_f = (float)sel_scale;
  const bf16* kbase = Kslc + (b * nC * Hkv + g) * (size_t)D;  // chunk c row: + c * Hkv * D

  if (tid < 64) {
    cnt[tid] = 0;
    fall[tid] = 0;
  }
  __syncthreads();

  // B operand: this lane's token column, 8 dimensions per k-step, read from the token's
  // Qs row (zero past the sequence); |q|^2 over the 4 lanes.  The filter works on
  // sign(scale) * q.k, which orders the chunks as the scaled scores do: with a negative
  // scale q enters negated (exact in bf16), and the scale's magnitude is left out.
  bf16x8 qb[KS];
  float q2 = 0.0f;
  const bf16* qrow = Qs + ((b * L + (size_t)t) * Hkv + g) * D;
  const uint32_t qsign = sel_scale < 0.0 ? 0x80008000u : 0u;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qb[ks] = t < L ? ld_bf16x8(qrow + 32 * ks + 8 * blk) : zero_bf16x8();
    q2 += sq8(qb[ks]);
    uint4 u = __builtin_bit_cast(uint4, qb[ks]);
    u.x ^= qsign;
    u.y ^= qsign;
    u.z ^= qsign;
    u.w ^= qsign;
    qb[ks] = __builtin_bit_cast(bf16x8, u);
  }
  q2 = rows4_sum(q2);

  // The block stages each group of 64 chunk keys in LDS; every thread holds D/32 16-byte
  // pieces of the next group in registers while the current one is scored.
  constexpr int NP = D / 32;
  uint4 pre[NP];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), e = (i % (D / 8)) * 8;
      pre[u] = c0 + r < m ? *reinterpret_cast<const uint4*>(kbase + (size_t)(c0 + r) * Hkv * D + e)
                          : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&]() {  // between two block barriers
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = tid + 256 * u, r = i / (D / 8), e = (i % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&kl[r][e]) = pre[u];
    }
  };
  // |k|^2 of the staged rows, each row's D/8 pieces summed across the D/8 consecutive
  // threads that hold them, folded into a running maximum (pass 1 only; rows past m were
  // loaded as zeros)
  float k2run = 0.0f;
  bool kbad = false;  // a staged row with a NaN or infinite |k|^2 (fmaxf would drop a NaN)
  auto k2_of_staged = [&]() {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const float k2 = group_sum<D / 8>(sq8(__builtin_bit_cast(bf16x8, pre[u])));
      k2run = fmaxf(k2run, k2);
      kbad = kbad || !(k2 <= 3.0e38f);
    }
  };

  // approximate scores of chunks c0 .. c0+63 (staged) against the wave's 16 tokens: lane
  // holds chunks c0 + 16*t4 + 4*blk + i of its token
  auto approx = [&](f32x4 (&sacc)[4]) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      sacc[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&kl[16 * t4 + col][32 * ks + 8 * blk]);
        sacc[t4] = mfma_16x16x32(ka, qb[ks], sacc[t4]);
      }
    }
  };

  // 1. the KP largest approximate values of this lane's share (4 KP >= K), kept sorted by
  //    keep_top.  Non-finite values are caught once, from |q|^2 and |k|^2, below: when
  //    every norm is finite and sel |q| max|k| and |q| max|k| stay far below the fp32 range,
  //    no partial sum of any approximate score can overflow (Cauchy-Schwarz)
  static_assert(4 * KP >= KL, "the token's four lists must hold K scores");
  float top[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) top[i] = -__builtin_inff();
  if (m > 0) fetch(0);
  for (int c0 = 0; c0 < m; c0 += 64) {
    __syncthreads();  // the previous group is no longer read
    stage();
    k2_of_staged();
    __syncthreads();
    if (c0 + 64 < m) fetch(c0 + 64);
    f32x4 sacc[4];
    approx(sacc);
    if (c0 + 64 <= m) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) keep_top(top, sacc[t4][i]);
    } else {  // the last group: rows past m were staged as zeros
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          keep_top(top, c0 + 16 * t4 + 4 * blk + i < m ? sacc[t4][i] : -__builtin_inff());
    }
  }
  // max |k|^2 over every candidate chunk, and whether any was not finite: over the wave,
  // then over the block's waves
  __shared__ float k2w[4];
  __shared__ int kbadw[4];
  {
    const float k2wave = rows4_max(row16_max(k2run));
    const bool kb = __ballot(kbad) != 0;
    if (lane == 0) {
      k2w[wave] = k2wave;
      kbadw[wave] = kb ? 1 : 0;
    }
  }
  __syncthreads();
  const float k2max = fmaxf(fmaxf(k2w[0], k2w[1]), fmaxf(k2w[2], k2w[3]));
  const float qk = sqrtf(q2) * sqrtf(k2max);  // bounds |q.k| and its partial sums
  // Besides non-finite values and overflow, two cases of tiny magnitudes go to the exact
  // path: scores so small that fp32's subnormal spacing exceeds the headroom below
  // (|scale| |q| max|k| (D+8) < 2^-125, a zero scale among them), where rounding ties
  // chunks the filter keeps apart; and |q| max|k| < 2^-60 (its fp32 norms may underflow,
  // and subnormal products in the approximate sums would no longer be inside the bound).
  // A tile with no earlier chunk has nothing to rank.
  bool bad = !(q2 <= 3.0e38f) || (kbadw[0] | kbadw[1] | kbadw[2] | kbadw[3]) != 0 ||
             !(qk < 1.0e37f) || !(fabsf(sel_f) * qk < 1.0e37f) ||
             (m > 0 && !(qk >= 0x1p-60f && fabsf(sel_f) * qk * (float)(D + 8) >= 0x1p-125f));
  // T = K-th largest over the token's 4 lanes (lane order breaks equal values apart)
  float T = -__builtin_inff();
  for (int k = 0; k < Kt; ++k) {
    const uint64_t key = ((uint64_t)ord_f32(top[0]) << 2) | (uint64_t)blk;
    const uint64_t best = rows4_max_key(key);
    if (best == key) {
#pragma unroll
      for (int j = 0; j + 1 < KP; ++j) top[j] = top[j + 1];
      top[KP - 1] = -__builtin_inff();
    }
    const uint32_t bo = (uint32_t)(best >> 2);
    T = __uint_as_float((bo & 0x80000000u) ? (bo ^ 0x80000000u) : ~bo);
  }
  // the approximate values' error bound, with a factor 2 of headroom (in units of q.k)
  const float E = 2.0f * qk * (float)(D + 8) * 5.9604645e-8f;
  bad = bad || (__float_as_uint(E) & 0x7f800000u) == 0x7f800000u;
  const float thr = T == -__builtin_inff() ? -__builtin_inff() : T - 2.0f * E;
  const uint64_t badmask = __ballot(bad);
  if (blk == 0 && ((badmask >> col) & 0x0001000100010001ull)) fall[tl] = 1;

  // 2. collect the chunks at or above the threshold
  if (m > 0) fetch(0);
  for (int c0 = 0; c0 < m; c0 += 64) {
    __syncthreads();  // the previous group is no longer read
    stage();
    __syncthreads();
    if (c0 + 64 < m) fetch(c0 + 64);
    f32x4 sacc[4];
    approx(sacc);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 16 * t4 + 4 * blk + i;
        if (c < m && sacc[t4][i] >= thr) {
          const int pos = atomicAdd(&cnt[tl], 1);
          if (pos < kSelCap) candl[tl][pos] = c;
        }
      }
  }
  __syncthreads();

  // 3. exact scores of the candidates: four consecutive lanes per token, each rescoring
  //    every fourth candidate (two at a time, so two independent fp64 chains are in flight)
  //    into its own ranked list of KL >= K keys; the four lists merge by quad maxima, and
  //    lane s of the quad forms the weights of slots s, s + 4, ...
  {
    const int tj = 16 * wave + lane / 4, sub = lane % 4, tt = t0 + tj;
    const bool fb = fall[tj] || cnt[tj] > kSelCap;
    const int n = (fb || tt >= L) ? 0 : cnt[tj];  // rows past the sequence read nothing
    const bf16* qr = Qs + ((b * L + (size_t)tt) * Hkv + g) * D;
    uint64_t tk[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) tk[i] = 0;
    for (int r = sub; r < n; r += 8) {
      const bool two = r + 4 < n;
      const int c1 = candl[tj][r], c2 = two ? candl[tj][r + 4] : c1;
      const bf16* k1 = kbase + (size_t)c1 * Hkv * D;
      const bf16* k2 = kbase + (size_t)c2 * Hkv * D;
      double d1 = 0.0, d2 = 0.0;
#pragma unroll 2
      for (int e = 0; e < D; e += 8) {
        const uint4 qv = *reinterpret_cast<const uint4*>(qr + e);
        const uint4 kv1 = *reinterpret_cast<const uint4*>(k1 + e);
        const uint4 kv2 = *reinterpret_cast<const uint4*>(k2 + e);
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
        const uint32_t kw1[4] = {kv1.x, kv1.y, kv1.z, kv1.w}, kw2[4] = {kv2.x, kv2.y, kv2.z, kv2.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const double qlo = (double)bf16_lo(qw[h]), qhi = (double)bf16_hi(qw[h]);
          d1 = fma(qlo, (double)bf16_lo(kw1[h]), d1);
          d2 = fma(qlo, (double)bf16_lo(kw2[h]), d2);
          d1 = fma(qhi, (double)bf16_hi(kw1[h]), d1);
          d2 = fma(qhi, (double)bf16_hi(kw2[h]), d2);
        }
      }
      insert_key(tk, rank_key((float)(sel_scale * d1), c1));
      if (two) insert_key(tk, rank_key((float)(sel_scale * d2), c2));
    }
    // K rounds of the quad maximum; every lane of the quad sees each slot's key and keeps
    // those of its own slots
    constexpr int NS = (KL + 3) / 4;
    uint64_t mine[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) mine[j] = 0;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      if (k < Kt) {
        const uint64_t best = dpp_max_key<0x4E>(dpp_max_key<0xB1>(tk[0]));  // over the quad
        if (best != 0 && tk[0] == best) {
#pragma unroll
          for (int i = 0; i + 1 < KL; ++i) tk[i] = tk[i + 1];
          tk[KL - 1] = 0;
        }
        if ((k & 3) == sub) mine[k >> 2] = best;
      }
    }
    // slot k's weight is sigmoid(s_k) times the stick left by slots < k; the sigmoids are
    // formed in parallel, the stick passes along the quad in slot order
    double p[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) p[j] = mine[j] ? sigmoid_d((double)key_score(mine[j])) : 0.0;
    const bool writes = tt < L && !fb;  // a token without candidates: all masked
    const size_t o = ((b * L + tt) * Hkv + g) * Kt;
    double rem = 1.0;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      if (k < Kt) {
        const double pk = quad_bcast_f64(p[k >> 2], k & 3);
        if (writes && (k & 3) == sub) {
          const uint64_t key = mine[k >> 2];
          idx[o + k] = key ? key_chunk(key) : -1;
          score[o + k] = key ? key_score(key) : -__builtin_inff();
          w[o + k] = key ? (float)(pk * rem) : 0.0f;
        }
        rem *= 1.0 - pk;
      }
    }
  }
  // tokens for the exact path over all their candidates, one token at a time per wave
  for (int j = 0; j < 16; ++j) {
    const int tj = 16 * wave + j, tt = t0 + tj;
    if (tt >= L || !(fall[tj] || cnt[tj] > kSelCap)) continue;  // uniform over the wave
    uint64_t tk[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) tk[i] = 0;
    const bf16* qr = Qs + ((b * L + (size_t)tt) * Hkv + g) * D;
    for (int c = lane; c < m; c += 64) {
      const bf16* kr = kbase + (size_t)c * Hkv * D;
      double dot = 0.0;
      for (int e = 0; e < D; ++e) dot = fma((double)to_f32(qr[e]), (double)to_f32(kr[e]), dot);
      insert_key(tk, rank_key((float)(sel_scale * dot), c));
    }
    // the wave's ranked top-K: K rounds of the maximum over the lanes' list heads
    const size_t o = ((b * L + tt) * Hkv + g) * Kt;
    double rem = 1.0;
    for (int k = 0; k < Kt; ++k) {
      const uint64_t best = wave_max_key(tk[0]);
      if (best != 0 && tk[0] == best) {
#pragma unroll
        for (int i = 0; i + 1 < KL; ++i) tk[i] = tk[i + 1];
        tk[KL - 1] = 0;
      }
      if (lane == 0) write_slot(best, k, o, rem, idx, score, w);
    }
  }
}

bool select_mfma_supported(const Dims& d) { return d.dtype == 1 && !(d.flags & 1u); }

hipError_t launch_select_mfma(const Dims& d, const void* Qs, const void* Kslc, int32_t* idx,
                              float* score, float* w, hipStream_t s) {
  const int BG = d.B * d.Hkv;
  const int n_tiles = (d.L + 63) / 64;
  Timed tm(HSA_KERNEL_SELECT, s);
  auto go = [&](auto kern) {
    kern<<<dim3(BG * n_tiles), 256, 0, s>>>((const bf16*)Qs, (const bf16*)Kslc, idx, score, w,
                                            d.L, d.Hkv, d.K, d.nC, BG, d.sel_scale);
  };
  // KP = K/4 + 2 scores per lane in the filter's first pass
  if (d.D == 64) {
    if (d.K <= 8) go(k_select_mfma<64, 8, 4>);
    else go(k_select_mfma<64, 16, 6>);
  } else {
    if (d.K <= 8) go(k_select_mfma<128, 8, 4>);
    else go(k_select_mfma<128, 16, 6>);
  }
  return hipGetLastError();
}

}  // namespace hsa
