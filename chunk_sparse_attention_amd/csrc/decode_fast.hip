// decode_fast.hip -- one decode step per sequence, bandwidth-shaped (fp32 and bf16).
//
// At inference only the compact chunk-key table is scanned for selection, and each step
// reads only the selected chunks' key/value rows ("Hardware-aligned Hierarchical Sparse
// Attention ...", papernotes.org note, 方法详解 › 训练与推理优化, KV Cache Offloading).  The
// step has two kernels:
//   scan    streams the chunk-key table once.  Every lane scores kScanPer chunks with an
//           fp64 dot product in dimension order (exact products, so each score is the
//           correctly rounded definition); the block reduces its candidates to a ranked
//           top-K that it writes to the workspace.
//   attend  one block per (sequence, group, quarter of the group's heads) with one wave per
//           kept slot, so a (sequence, group) spreads over up to four CUs.  Each wave merges
//           the scan's candidates itself (so no wave waits on another), forms the
//           stick-breaking weights, and runs softmax-off-by-one attention of the block's heads
//           over its slot's chunk: lane j holds key row j for the logits, and the value rows
//           are read as independent 16-byte pieces so that all of a chunk's loads are in
//           flight at once.  The K weighted slot outputs meet in LDS and are summed in slot
//           order.
#include <algorithm>
#include <type_traits>

#include "hsa_common.h"
#include "hsa_launch.h"
#include "mfma_common.h"
#include "tile_common.h"

namespace hsa {

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 1;                                   // chunks per lane
constexpr int kScanChunks = kScanThreads * kScanPer;          // chunks per scan block
constexpr int kScanWaves = kScanThreads / kWave;

// Raw row of D elements kept as loaded (16-byte pieces), converted when used.
template <typename T, int D>
struct RawRow;
template <int D>
struct RawRow<bf16, D> {
  uint4 v[D / 8];
  __device__ __forceinline__ void load(const bf16* p) {
#pragma unroll
    for (int i = 0; i < D / 8; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ float get(int e) const {
    const uint4 q = v[e / 8];
    const uint32_t w = (e % 8) < 2 ? q.x : (e % 8) < 4 ? q.y : (e % 8) < 6 ? q.z : q.w;
    return (e % 2) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <int D>
struct RawRow<float, D> {
  float4 v[D / 4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) v[i] = reinterpret_cast<const float4*>(p)[i];
  }
  __device__ __forceinline__ float get(int e) const {
    const float4 q = v[e / 4];
    return (e % 4) == 0 ? q.x : (e % 4) == 1 ? q.y : (e % 4) == 2 ? q.z : q.w;
  }
};

// Workspace: the scan blocks' candidate keys.
struct DecFastLayout {
  int n_blocks;
  size_t cand, total;
};
static DecFastLayout dec_fast_layout(const Dims& d) {
  DecFastLayout l{};
  l.n_blocks = d.nC > 0 ? (d.nC + kScanChunks - 1) / kScanChunks : 0;
  l.cand = 0;
  l.total = (sizeof(uint64_t) * (size_t)d.B * d.Hkv * l.n_blocks * d.K + 255) & ~(size_t)255;
  return l;
}
size_t dec_fast_ws(const Dims& d) { return dec_fast_layout(d).total; }

template <typename T, int D>
__global__ void __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(4)))
k_dec_scan_fast(const T* __restrict__ qs, const T* __restrict__ Kslc,
                uint64_t* __restrict__ cand, int Hkv, int K, int nC, int n_blocks,
                double sel_scale, const int32_t* __restrict__ ctx_lens) {
  __shared__ double qsh[D];
  const int blk = blockIdx.x % n_blocks;
  const int bg = blockIdx.x / n_blocks;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // chunks this sequence may select: all nC of the table, or those below its own length
  const int nCb = ctx_lens ? min(nC, max(0, ctx_lens[b]) / kChunk) : nC;
  for (int e = tid; e < D; e += kScanThreads)
    qsh[e] = (double)to_f32(qs[((size_t)b * Hkv + g) * D + e]);

  // bf16 rows are taken whole; fp32 rows in parts of 32 values, one after the other and
  // still summed in dimension order, so that the 1024-thread block stays within 128
  // registers per lane
  constexpr int DP = sizeof(T) == 2 ? D : 32;
  int cs[kScanPer];
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) cs[i] = blk * kScanChunks + i * kScanThreads + tid;
  double dot[kScanPer];
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) dot[i] = 0.0;
#pragma unroll 1
  for (int d0 = 0; d0 < D; d0 += DP) {
    RawRow<T, DP> row[kScanPer];
#pragma unroll
    for (int i = 0; i < kScanPer; ++i)
      if (cs[i] < nCb) row[i].load(Kslc + ((b * nC + cs[i]) * Hkv + g) * D + d0);
    if (d0 == 0) __syncthreads();  // qsh ready
    // the dimension loop is outermost so that only eight query values are live at a time
#pragma unroll
    for (int e0 = 0; e0 < DP; e0 += 8) {
      double qv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = qsh[d0 + e0 + e];
#pragma unroll
      for (int i = 0; i < kScanPer; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) dot[i] = fma(qv[e], (double)row[i].get(e0 + e), dot[i]);
    }
  }
  static_assert(kScanPer == 1 && kScanWaves <= kWave && kScanWaves >= kMaxK,
                "one chunk per lane; the wave maxima fill one wave and bound every K");
  const uint64_t key = cs[0] < nCb ? rank_key((float)(sel_scale * dot[0]), cs[0]) : 0;
  uint64_t* out = cand + ((size_t)bg * n_blocks + blk) * K;
  // The block's top-K all have a score (the key's upper half, 0 = no chunk) of at least
  // thr, the K-th largest of the waves' maximum scores: those are the scores of K keys of
  // the block.  Usually only about K keys do; they are gathered, and each one's rank is the
  // number of gathered keys above it (keys are distinct apart from 0).
  __shared__ uint32_t wmax[kScanWaves];
  __shared__ uint64_t clist[kWave];
  __shared__ int ccount;
  const uint32_t sc = (uint32_t)(key >> 32);
  const uint32_t mw = wave_max_u32(sc);
  if (lane == 0) wmax[wave] = mw;
  if (tid == 0) ccount = 0;
  __syncthreads();
  uint32_t thr;
  {
    const uint32_t mine = lane < kScanWaves ? wmax[lane] : 0;
    int n_ge = 0;  // wave maxima at or above this lane's
#pragma unroll
    for (int j = 0; j < kScanWaves; ++j) n_ge += wmax[j] >= mine ? 1 : 0;
    thr = wave_max_u32(n_ge >= K ? mine : 0);
  }
  const bool is_c = key != 0 && sc >= thr;
  const uint64_t bal = __ballot(is_c);
  int base = 0;
  if (lane == 0 && bal) base = atomicAdd(&ccount, __popcll(bal));
  base = __shfl(base, 0);
  const int pos = base + __popcll(bal & ((1ull << lane) - 1));
  if (is_c && pos < kWave) clist[pos] = key;
  __syncthreads();
  const int nc = ccount;  // uniform
  if (nc <= kWave) {
    if (wave == 0) {
      const uint64_t v = lane < nc ? clist[lane] : 0;
      int r = 0;
      for (int j = 0; j < nc; ++j) r += clist[j] > v ? 1 : 0;
      if (lane < nc && r < K) out[r] = v;
      if (lane >= nc && lane < K) out[lane] = 0;  // fewer chunks than K: masked slots
    }
    return;
  }
  // many keys at thr or above (equal scores): K rounds of a wave
  // maximum in every wave, then the block's ranked top-K from the waves' lists (at most
  // 16 x 16 keys, four per lane)
  __shared__ uint64_t wtop[kScanWaves][kMaxK];
  {
    uint64_t v = key;
    for (int k = 0; k < K; ++k) {
      const uint64_t best = wave_max_key(v);
      if (best != 0 && v == best) v = 0;
      if (lane == 0) wtop[wave][k] = best;
    }
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = lane + kWave * i;
      v[i] = j < kScanWaves * K ? wtop[j / K][j % K] : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = i + 1; j < 4; ++j)
        if (v[j] > v[i]) {
          const uint64_t t = v[i];
          v[i] = v[j];
          v[j] = t;
        }
    for (int k = 0; k < K; ++k) {
      const uint64_t best = wave_max_key(v[0]);
      if (best != 0 && v[0] == best) {
        v[0] = v[1];
        v[1] = v[2];
        v[2] = v[3];
        v[3] = 0;
      }
      if (lane == 0) out[k] = best;
    }
  }
}

__device__ __forceinline__ float wave_sum_f(float v) { return rows4_sum(row16_sum(v)); }
__device__ __forceinline__ float wave_max_f(float v) { return rows4_max(row16_max(v)); }

// Ranked top-K of the scan's candidates (n_cand / K ranked lists of K keys, one per scan
// block) in every wave; lane k < K returns slot k's key.  lds: kWave + K keys of LDS that
// only this wave uses.
//   The top-K all score at least thr, the K-th largest of the lists' first scores (those
//   are K of the keys).  Usually only about K keys do: they are gathered, and each one's
//   slot is the number of gathered keys above it (keys are distinct apart from 0).
__device__ __forceinline__ uint64_t rank_candidates(const uint64_t* __restrict__ cb, int n_cand,
                                                    int K, int lane, uint64_t* lds) {
  const int nl = n_cand / K;
  if (nl <= kWave) {
    // With at most two keys per lane every key is loaded at once and the list heads are
    // taken from the lanes that hold them, so that the ranking waits for one round trip.
    const bool two = n_cand <= 2 * kWave;
    uint64_t ka = 0, kb = 0;
    uint32_t mine;
    if (two) {
      ka = lane < n_cand ? cb[lane] : 0;
      kb = lane + kWave < n_cand ? cb[lane + kWave] : 0;
      const int h = lane * K;  // this lane's list head (lanes < nl)
      const uint64_t ha = __shfl(ka, h % kWave), hb = __shfl(kb, h % kWave);
      mine = lane < nl ? (uint32_t)((h < kWave ? ha : hb) >> 32) : 0;
    } else {
      mine = lane < nl ? (uint32_t)(cb[lane * K] >> 32) : 0;
    }
    lds[lane] = mine;
    wave_lds_sync();
    int n_ge = 0;  // lists whose first score is at least this lane's
    for (int j = 0; j < nl; ++j) n_ge += (uint32_t)lds[j] >= mine ? 1 : 0;
    const uint32_t thr = wave_max_u32(n_ge >= K ? mine : 0);
    wave_lds_sync();  // lds is reused below
    int nc = 0;
    for (int i0 = 0; i0 < n_cand; i0 += kWave) {
      const int i = i0 + lane;
      const uint64_t k = two ? (i0 == 0 ? ka : kb) : (i < n_cand ? cb[i] : 0);
      const bool c = k != 0 && (uint32_t)(k >> 32) >= thr;
      const uint64_t bal = __ballot(c);
      const int pos = nc + __popcll(bal & ((1ull << lane) - 1));
      if (c && pos < kWave) lds[pos] = k;
      nc += __popcll(bal);
    }
    if (nc <= kWave) {
      wave_lds_sync();
      const uint64_t v = lane < nc ? lds[lane] : 0;
      int r = 0;
      for (int j = 0; j < nc; ++j) r += lds[j] > v ? 1 : 0;
      if (lane < nc && r < K) lds[kWave + r] = v;
      if (lane >= nc && lane < K) lds[kWave + lane] = 0;  // fewer keys than K: masked slots
      wave_lds_sync();
      return lane < K ? lds[kWave + lane] : 0;
    }
  }
  // many keys at thr or above (equal scores): K rounds of a wave maximum
  uint64_t mykey = 0;
  if (n_cand <= 2 * kWave) {
    // at most two keys per lane: a sorted pair
    uint64_t a = lane < n_cand ? cb[lane] : 0;
    uint64_t c = lane + kWave < n_cand ? cb[lane + kWave] : 0;
    if (c > a) {
      const uint64_t t = a;
      a = c;
      c = t;
    }
    for (int k = 0; k < K; ++k) {
      const uint64_t best = wave_max_key(a);
      if (best != 0 && a == best) {
        a = c;
        c = 0;
      }
      if (lane == k) mykey = best;
    }
  } else {
    uint64_t top[kMaxK];
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) top[i] = 0;
    for (int i = lane; i < n_cand; i += kWave) topk_insert(top, cb[i], K);
    for (int k = 0; k < K; ++k) {
      const uint64_t best = wave_max_key(top[0]);
      if (best != 0 && top[0] == best) topk_pop(top);
      if (lane == k) mykey = best;
    }
  }
  return mykey;
}

// One block per (b, g, head group): a head group is HW of the group's G query heads, and the
// block has one wave per kept slot.  D elements per row = P pieces of 8; the 64 lanes of a
// wave form JG = 64/P groups of P lanes, and group jg reads rows jg, jg+JG, ... of the chunk
// in the value product.  Every wave merges the scan's candidates itself (so no wave waits on
// another) and forms the stick-breaking weights; the slots' weighted outputs meet in LDS and
// are summed in rank order.
template <typename T, int D, int ZH, int NT>
__global__ void __launch_bounds__(NT) k_dec_attend_heads(
    const T* __restrict__ q, const T* __restrict__ Kc, const T* __restrict__ Vc,
    const uint64_t* __restrict__ cand, T* __restrict__ O, int32_t* __restrict__ idx,
    float* __restrict__ score, float* __restrict__ w, int ctx, int Hq, int Hkv, int K, int G,
    int HW, int n_hg, int n_cand, float c2, int softmax_w, const int32_t* __restrict__ sel_idx,
    const float* __restrict__ sel_w, size_t q_lstride, size_t kv_lstride) {
  constexpr int P = D / 8;
  constexpr int JG = kWave / P;
  constexpr int RPL = kChunk / JG;  // rows per lane in the value product
  constexpr int NS = NT / kWave;    // slots (waves) per block
  __shared__ float qsh[ZH][D];
  __shared__ float ash[NS][ZH][kChunk];
  __shared__ float osh[NS][ZH][D];
  __shared__ uint64_t rk[NS][kWave + kMaxK];  // each wave's candidate ranking
  const int tid = threadIdx.x, lane = tid % kWave, slot = tid / kWave;
  const int hg = blockIdx.x % n_hg, bg = blockIdx.x / n_hg;
  // layer blockIdx.y of a stack of layers that share one selection (strides 0 otherwise)
  const size_t layer = blockIdx.y;
  q += layer * q_lstride;
  O += layer * q_lstride;
  Kc += layer * kv_lstride;
  Vc += layer * kv_lstride;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int h_lo = hg * HW, nh = min(G, h_lo + HW) - h_lo;
  const size_t qbase = ((size_t)b * Hq + (size_t)g * G + h_lo) * D;
  for (int i = tid; i < nh * D; i += blockDim.x) qsh[i / D][i % D] = to_f32(q[qbase + i]);

  int my_c = -1;       // lane k < K: slot k's chunk (-1 = masked)
  double wslot = 0.0;  // and its weight
  uint64_t mykey = 0;
  if (sel_idx) {
    // a selection made before (an earlier layer's): the slots' chunks and weights as given
    if (lane < K) {
      my_c = sel_idx[(size_t)bg * K + lane];
      if (my_c >= ctx / kChunk) my_c = -1;  // an index past the cache is a masked slot
      wslot = my_c >= 0 ? (double)sel_w[(size_t)bg * K + lane] : 0.0;
    }
  } else {
    mykey =
        n_cand > 0 ? rank_candidates(cand + (size_t)bg * n_cand, n_cand, K, lane, rk[slot]) : 0;
    my_c = mykey != 0 ? key_chunk(mykey) : -1;
  }
  // this wave's slot, read from lane `slot`
  const int mine = __builtin_amdgcn_readlane(my_c, slot);
  const size_t kvstride = (size_t)Hkv * D;
  const size_t cbase = ((b * ctx + (size_t)(mine >= 0 ? mine : 0) * kChunk) * Hkv + g) * D;
  const int p8 = lane % P, jg = lane / P;
  // key row j in lane j; the value pieces are requested at the same time where the
  // register budget holds both (otherwise after the logits)
  constexpr bool kEarlyV = sizeof(T) == 2 && (NT <= 512 || D == 64);
  // with 128 registers per lane a D = 128 key row is taken in two halves, one after the
  // other (the logits still accumulate in dimension order)
  constexpr int KP = (NT > 512 && D == 128) ? 2 : 1;
  constexpr int DK = D / KP;
  // fp32 d = 128 value rows in 1024-thread blocks are taken in two parts (128 registers per
  // lane would not hold them all)
  constexpr int VP = (sizeof(T) == 4 && NT > 512 && D == 128) ? 2 : 1;
  constexpr int RPV = RPL / VP;
  RawRow<T, 8> vp[RPV];
  auto load_v = [&](int part) {
#pragma unroll
    for (int i = 0; i < RPV; ++i)
      vp[i].load(Vc + cbase + (size_t)(jg + JG * (part * RPV + i)) * kvstride + 8 * p8);
  };
  // the slot's key row (the whole row, or its first half) and, where they fit, its value
  // pieces are requested before the weights are formed, whose work then overlaps their
  // latency (not for fp32 rows in 1024-thread blocks, whose 128 registers per lane would
  // not hold them across the weights)
  constexpr bool kEarlyK = sizeof(T) == 2 || NT <= 512;
  RawRow<T, DK> kr0;
  if (kEarlyK && mine >= 0) {
    kr0.load(Kc + cbase + (size_t)lane * kvstride);
    if (kEarlyV) load_v(0);
  }
  if (!sel_idx) {
    if (softmax_w) {
      // softmax of the valid slots' scores (lanes 0..K-1), shifted by their maximum and
      // summed in slot order
      const double sc = mykey != 0 ? (double)key_score(mykey) : -__builtin_inf();
      double m = -__builtin_inf();
      for (int j = 0; j < K; ++j) m = fmax(m, __shfl(sc, j));
      const double e = (mykey != 0 && m != -__builtin_inf()) ? exp(sc - m) : 0.0;
      double den = 0.0;
      for (int j = 0; j < K; ++j) den += __shfl(e, j);
      wslot = den > 0.0 ? e / den : 0.0;
    } else {
      // stick-breaking in rank order: slot k needs p_k * prod_{j<k} (1 - p_j), a prefix
      // product over lanes 0..K-1 (masked slots have p = 0 and come last)
      const double p = mykey != 0 ? sigmoid_d((double)key_score(mykey)) : 0.0;
      double keep = 1.0 - p;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const double x = __shfl_up(keep, o, 16);
        if ((lane & 15) >= o) keep *= x;
      }
      double excl = __shfl_up(keep, 1, 16);
      if ((lane & 15) == 0) excl = 1.0;
      wslot = p * excl;
    }
    if (hg == 0 && slot == 0 && lane < K) {
      const size_t o = (size_t)bg * K + lane;
      if (mykey == 0) {
        idx[o] = -1;
        if (score) score[o] = -__builtin_inff();
        w[o] = 0.0f;
      } else {
        idx[o] = key_chunk(mykey);
        if (score) score[o] = key_score(mykey);
        w[o] = (float)wslot;
      }
    }
  }
  // the valid slots (the first ones, in what the scan ranks; in a given selection, any)
  const uint64_t vmask = __ballot(lane < K && my_c >= 0);
  const float wf = __shfl((float)wslot, slot);
  __syncthreads();  // qsh ready

  if (mine >= 0) {
    float z[ZH];
#pragma unroll
    for (int h = 0; h < ZH; ++h) z[h] = 0.0f;
#pragma unroll 1
    for (int kp = 0; kp < KP; ++kp) {
      RawRow<T, DK> kr;
      if (kEarlyK && kp == 0)
        kr = kr0;
      else
        kr.load(Kc + cbase + (size_t)lane * kvstride + kp * DK);
      if (!kEarlyK && kEarlyV && kp == 0) load_v(0);
#pragma unroll
      for (int h = 0; h < ZH; ++h) {
        if (h < nh) {
#pragma unroll
          for (int e0 = 0; e0 < DK; e0 += 8) {
            int off = h * D + kp * DK + e0;  // the empty asm keeps the query reads in the loop
            asm volatile("" : "+v"(off));
            const float4 qa = *reinterpret_cast<const float4*>(&qsh[0][0] + off);
            const float4 qb = *reinterpret_cast<const float4*>(&qsh[0][0] + off + 4);
            const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) z[h] = fmaf(qv[e], kr.get(e0 + e), z[h]);
          }
        }
      }
    }
    // softmax-off-by-one of each head (log2 domain), scaled by the slot weight
#pragma unroll
    for (int h = 0; h < ZH; ++h) {
      float aw = 0.0f;
      if (h < nh) {
        const float zz = z[h] * c2;
        const float m = fmaxf(0.0f, wave_max_f(zz));
        const float ex = exp2f(zz - m);
        aw = wf * ex / (exp2f(-m) + wave_sum_f(ex));
      }
      ash[slot][h][lane] = aw;
    }
    // value product: lane (jg, p8) accumulates rows jg + JG*i of piece p8, in row order
    float acc[ZH][8];
#pragma unroll
    for (int h = 0; h < ZH; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
#pragma unroll
    for (int part = 0; part < VP; ++part) {
      if (!kEarlyV) load_v(part);
#pragma unroll
      for (int i = 0; i < RPV; ++i) {
        const int j = jg + JG * (part * RPV + i);
#pragma unroll
        for (int h = 0; h < ZH; ++h) {
          if (h >= nh) continue;
          const float aw = ash[slot][h][j];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(aw, vp[i].get(e), acc[h][e]);
        }
      }
    }
    // sum over the JG row groups: lanes p8 + P*jg
#pragma unroll
    for (int h = 0; h < ZH; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (h >= nh) continue;
        float sum = acc[h][e];
        if (P == 8) sum += dppc<0x128>(sum);  // row_ror:8 pairs lanes l and l^8 in a row
        acc[h][e] = rows4_sum(sum);
      }
    if (jg == 0) {
#pragma unroll
      for (int h = 0; h < ZH; ++h)
        if (h < nh) {
#pragma unroll
          for (int e = 0; e < 8; ++e) osh[slot][h][8 * p8 + e] = acc[h][e];
        }
    }
  }
  __syncthreads();
  // O = sum over the valid slots in slot order
  for (int i = tid; i < nh * D; i += blockDim.x) {
    float sum = 0.0f;
    for (int k = 0; k < K; ++k)
      if ((vmask >> k) & 1) sum += osh[k][i / D][i % D];
    O[qbase + i] = from_f32<T>(sum);
  }
}

template <typename T, int D>
static void launch_dec_fast_t(const Dims& d, const void* q, const void* qs, const void* Kc,
                              const void* Vc, const void* Kslc, void* O, int32_t* idx,
                              float* score, float* w, bool host_kv, const int32_t* ctx_lens,
                              char* ws, hipStream_t s) {
  const int bg = d.B * d.Hkv;
  const DecFastLayout lay = dec_fast_layout(d);
  const int n_blocks = lay.n_blocks;
  uint64_t* cand = (uint64_t*)(ws + lay.cand);
  if (n_blocks > 0) {
    Timed tm(HSA_KERNEL_DECODE_SCAN, s);
    k_dec_scan_fast<T, D><<<dim3(bg * n_blocks), kScanThreads, 0, s>>>(
        (const T*)qs, (const T*)Kslc, cand, d.Hkv, d.K, d.nC, n_blocks, d.sel_scale, ctx_lens);
  }
  const float c2 = (float)(d.sm_scale * 1.4426950408889634);
  Timed tm(HSA_KERNEL_DECODE_ATTEND, s);
  // one block per (b, g, head group) of HW <= ZH heads, one wave per kept slot.  With the
  // caches in device memory a group's heads spread over up to four blocks (more CUs); with
  // them in host memory one block takes up to eight heads, so that each selected chunk
  // crosses the host link once per eight heads.
  // The launch bound sets the register budget: 256 VGPRs up to 8 slots, 128 above.
  auto go = [&](auto kern, int zh) {
    const int n_hg0 = (d.G + zh - 1) / zh;
    const int HW = host_kv ? (d.G + n_hg0 - 1) / n_hg0 : (d.G + 3) / 4;
    const int n_hg = (d.G + HW - 1) / HW;
    kern<<<dim3(bg * n_hg), kWave * d.K, 0, s>>>((const T*)q, (const T*)Kc, (const T*)Vc, cand,
                                                 (T*)O, idx, score, w, d.L, d.Hq, d.Hkv, d.K,
                                                 d.G, HW, n_hg, n_blocks * d.K, c2,
                                                 softmax_w(d), nullptr, nullptr, 0, 0);
  };
  constexpr int ZW = 8;  // heads per block for host caches, up to 8 slots
  if (d.K > 8) go(k_dec_attend_heads<T, D, 4, 1024>, 4);
  else if (host_kv) go(k_dec_attend_heads<T, D, ZW, 512>, ZW);
  else if ((d.G + 3) / 4 <= 2) go(k_dec_attend_heads<T, D, 2, 512>, 2);
  else go(k_dec_attend_heads<T, D, 4, 512>, 4);
}

// A stack of n_layers layers attending with one given selection (attend kernel only).
template <typename T, int D>
static void launch_dec_shared_t(const Dims& d, int n_layers, const void* q, const void* Kc,
                                const void* Vc, const int32_t* sel_idx, const float* sel_w,
                                void* O, bool host_kv, hipStream_t s) {
  const int bg = d.B * d.Hkv;
  const float c2 = (float)(d.sm_scale * 1.4426950408889634);
  const size_t q_ls = (size_t)d.B * d.Hq * D, kv_ls = (size_t)d.B * d.L * d.Hkv * D;
  Timed tm(HSA_KERNEL_DECODE_ATTEND, s);
  // head groups as in launch_dec_fast_t: quarters of the group's heads for device caches,
  // up to eight heads per block for host caches
  auto go = [&](auto kern, int zh) {
    const int n_hg0 = (d.G + zh - 1) / zh;
    const int HW = host_kv ? (d.G + n_hg0 - 1) / n_hg0 : (d.G + 3) / 4;
    const int n_hg = (d.G + HW - 1) / HW;
    kern<<<dim3(bg * n_hg, n_layers), kWave * d.K, 0, s>>>(
        (const T*)q, (const T*)Kc, (const T*)Vc, nullptr, (T*)O, nullptr, nullptr, nullptr,
        d.L, d.Hq, d.Hkv, d.K, d.G, HW, n_hg, 0, c2, 0, sel_idx, sel_w, q_ls, kv_ls);
  };
  if (d.K > 8) go(k_dec_attend_heads<T, D, 4, 1024>, 4);
  else if (host_kv) go(k_dec_attend_heads<T, D, 8, 512>, 8);
  else if ((d.G + 3) / 4 <= 2) go(k_dec_attend_heads<T, D, 2, 512>, 2);
  else go(k_dec_attend_heads<T, D, 4, 512>, 4);
}

hipError_t launch_decode_shared(const Dims& d, int n_layers, const void* q, const void* Kc,
                                const void* Vc, const int32_t* sel_idx, const float* sel_w,
                                void* O, bool host_kv, hipStream_t s) {
  if (d.B * d.Hkv == 0) return hipSuccess;
  auto go = [&](auto tag, auto dim) {
    using T = decltype(tag);
    launch_dec_shared_t<T, decltype(dim)::value>(d, n_layers, q, Kc, Vc, sel_idx, sel_w, O,
                                                 host_kv, s);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (d.dtype == 1) {
    if (d.D == 64) go(bf16{}, D64{});
    else go(bf16{}, D128{});
  } else {
    if (d.D == 64) go(float{}, D64{});
    else go(float{}, D128{});
  }
  return hipGetLastError();
}

hipError_t launch_decode_fast(const Dims& d, const void* q, const void* qs, const void* Kc,
                              const void* Vc, const void* Kslc, void* O, int32_t* idx,
                              float* score, float* w, bool host_kv, const int32_t* ctx_lens,
                              char* ws, hipStream_t s) {
  if (d.B * d.Hkv == 0) return hipSuccess;
  auto go = [&](auto tag, auto dim) {
    using T = decltype(tag);
    launch_dec_fast_t<T, decltype(dim)::value>(d, q, qs, Kc, Vc, Kslc, O, idx, score, w,
                                               host_kv, ctx_lens, ws, s);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (d.dtype == 1) {
    if (d.D == 64) go(bf16{}, D64{});
    else go(bf16{}, D128{});
  } else {
    if (d.D == 64) go(float{}, D64{});
    else go(float{}, D128{});
  }
  return hipGetLastError();
}

}  // namespace hsa
