// select_generic.hip -- chunk-key pooling and the plain vector-ALU selection kernel.
//
// Chunk selection ("Hardware-aligned Hierarchical Sparse Attention ...", papernotes.org note,
// 方法详解 › 层次化稀疏注意力（HSA）, Chunk Selection): each chunk is keyed by the mean of its
// keys; each token scores the earlier chunks with its selection query and keeps the top-K,
// per query group.  The chunk weights are stick-breaking over the sigmoid of the ranked
// scores (same section, 第二阶段).
#include "hsa_common.h"
#include "hsa_launch.h"

namespace hsa {

// Kslc[b,c,g,e] = mean_j K[b, c*S+j, g, e] (S = 64): one thread per output element; the sum
// runs in fp64 in row order so the result is the exact mean for any bf16/fp32 chunk in
// practice, rounded once to the storage type.  Consecutive threads read consecutive e
// (coalesced), and sixteen rows' loads are in flight at a time.
// Feature e of the chunk key of (b, chunk c, group g): the mean of the chunk's S key rows,
// summed in row order in fp64 and rounded once.
template <typename T>
__device__ __forceinline__ T pool_one(const T* __restrict__ K, int L, int Hkv, int D, size_t b,
                                      int c, int g, int e) {
  const T* src = K + ((b * L + (size_t)c * kChunk) * Hkv + g) * D + e;
  const size_t stride = (size_t)Hkv * D;
  // sixteen rows' loads in flight at a time; the sum stays in row order
  double sum = 0.0;
  for (int j0 = 0; j0 < kChunk; j0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = to_f32(src[(size_t)(j0 + u) * stride]);
#pragma unroll
    for (int u = 0; u < 16; ++u) sum += (double)v[u];
  }
  return from_f64<T>(sum / kChunk);
}

template <typename T>
__global__ void __launch_bounds__(256) k_pool(const T* __restrict__ K, T* __restrict__ Kslc,
                                              int L, int Hkv, int D, int S, int nC,
                                              size_t total) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  int e = (int)(i % D);
  size_t r = i / D;
  int g = (int)(r % Hkv);
  r /= Hkv;
  int c = (int)(r % nC);
  size_t b = r / nC;
  Kslc[i] = pool_one(K, L, Hkv, D, b, c, g, e);
}

hipError_t launch_pool(const Dims& d, const void* K, void* Kslc, hipStream_t s) {
  size_t total = (size_t)d.B * d.nC * d.Hkv * d.D;
  if (total == 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  Timed tm(HSA_KERNEL_POOL, s);
  if (d.dtype == 1)
    k_pool<bf16><<<grid, 256, 0, s>>>((const bf16*)K, (bf16*)Kslc, d.L, d.Hkv, d.D, d.S, d.nC,
                                      total);
  else
    k_pool<float><<<grid, 256, 0, s>>>((const float*)K, (float*)Kslc, d.L, d.Hkv, d.D, d.S,
                                       d.nC, total);
  return hipGetLastError();
}

// The chunk keys of listed chunks only (a decoder appends the chunk its sequence just
// completed): one thread per (b, listed entry, g, feature), the same arithmetic as k_pool.
template <typename T>
__global__ void __launch_bounds__(256) k_pool_chunks(const T* __restrict__ K, T* __restrict__ Kslc,
                                                     const int32_t* __restrict__ chunk_ids,
                                                     int n_ids, int L, int Hkv, int D, int nC,
                                                     size_t total) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int e = (int)(i % D);
  size_t r = i / D;
  const int g = (int)(r % Hkv);
  r /= Hkv;  // b * n_ids + j
  const size_t b = r / n_ids;
  const int c = chunk_ids[r];
  if (c < 0 || c >= nC) return;
  Kslc[((b * nC + c) * Hkv + g) * D + e] = pool_one(K, L, Hkv, D, b, c, g, e);
}

hipError_t launch_pool_chunks(const Dims& d, const void* K, void* Kslc, const int32_t* chunk_ids,
                              int n_ids, hipStream_t s) {
  const size_t total = (size_t)d.B * n_ids * d.Hkv * d.D;
  if (total == 0 || d.nC == 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  Timed tm(HSA_KERNEL_POOL, s);
  if (d.dtype == 1)
    k_pool_chunks<bf16><<<grid, 256, 0, s>>>((const bf16*)K, (bf16*)Kslc, chunk_ids, n_ids, d.L,
                                             d.Hkv, d.D, d.nC, total);
  else
    k_pool_chunks<float><<<grid, 256, 0, s>>>((const float*)K, (float*)Kslc, chunk_ids, n_ids,
                                              d.L, d.Hkv, d.D, d.nC, total);
  return hipGetLastError();
}

// Selection, one wave per (b, t, g) row.  Lane l scores chunks l, l+64, ... with an fp64
// dot product of the stored values (exact products, sequential sum), keeps a private
// ranked list, and the wave merges the lists K times by a 64-bit max.  Lane 0 then forms
// the stick-breaking weights in fp64 and writes the K slots.
template <typename T>
__global__ void __launch_bounds__(64) k_select_generic(const T* __restrict__ Qs,
                                                       const T* __restrict__ Kslc,
                                                       int32_t* __restrict__ idx,
                                                       float* __restrict__ score,
                                                       float* __restrict__ w, int L, int Hkv,
                                                       int D, int S, int K, int nC,
                                                       double sel_scale) {
  __shared__ double qsh[128];
  __shared__ uint64_t chosen[kMaxK];
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;  // (b*L + t)*Hkv + g
  const int g = (int)(row % Hkv);
  const size_t bt = row / Hkv;
  const int t = (int)(bt % L);
  const size_t b = bt / L;
  int n_avail = t / S;
  if (n_avail > nC) n_avail = nC;

  for (int e = lane; e < D; e += kWave) qsh[e] = (double)to_f32(Qs[row * D + e]);
  __syncthreads();

  uint64_t top[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) top[i] = 0;
  for (int c = lane; c < n_avail; c += kWave) {
    const T* kr = Kslc + ((b * nC + c) * Hkv + g) * D;
    double dot = 0.0;
    for (int e = 0; e < D; e += 8) {
      float kv[8];
      load8(kr + e, kv);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += qsh[e + i] * (double)kv[i];
    }
    float s = (float)(sel_scale * dot);
    topk_insert(top, rank_key(s, c), K);
  }
  for (int k = 0; k < K; ++k) {
    uint64_t best = wave_max_u64(top[0]);
    if (best != 0 && top[0] == best) topk_pop(top);
    if (lane == 0) chosen[k] = best;
  }
  __syncthreads();
  if (lane == 0) {
    double remaining = 1.0;
    size_t o = row * K;
    for (int k = 0; k < K; ++k) {
      uint64_t key = chosen[k];
      if (key == 0) {
        idx[o + k] = -1;
        score[o + k] = -__builtin_inff();
        w[o + k] = 0.0f;
      } else {
        float s = key_score(key);
        double p = sigmoid_d((double)s);
        idx[o + k] = key_chunk(key);
        score[o + k] = s;
        w[o + k] = (float)(p * remaining);
        remaining *= 1.0 - p;
      }
    }
  }
}

// Softmax chunk weights of one (token, group) row per thread from its written scores: with
// m the largest valid score, w_k = exp(s_k - m) / sum_j exp(s_j - m) over the valid slots
// (fp64, summed in slot order); masked slots, and rows whose scores are all -inf, get 0.
__global__ void __launch_bounds__(256) k_softmax_weights(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ score,
                                                         float* __restrict__ w, int64_t rows,
                                                         int K) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const int64_t o = row * K;
  double m = -__builtin_inf();
  for (int k = 0; k < K; ++k)
    if (idx[o + k] >= 0) m = fmax(m, (double)score[o + k]);
  const bool any = m != -__builtin_inf();
  double den = 0.0;
  for (int k = 0; k < K; ++k)
    if (idx[o + k] >= 0 && any) den += exp((double)score[o + k] - m);
  for (int k = 0; k < K; ++k)
    w[o + k] = (idx[o + k] >= 0 && den > 0.0) ? (float)(exp((double)score[o + k] - m) / den)
                                              : 0.0f;
}

hipError_t launch_softmax_weights(const Dims& d, const int32_t* idx, const float* score,
                                  float* w, hipStream_t s) {
  const int64_t rows = (int64_t)d.B * d.L * d.Hkv;
  if (rows == 0) return hipSuccess;
  Timed tm(HSA_KERNEL_SELECT, s);
  k_softmax_weights<<<dim3((unsigned)((rows + 255) / 256)), 256, 0, s>>>(idx, score, w, rows,
                                                                          d.K);
  return hipGetLastError();
}

hipError_t launch_select_generic(const Dims& d, const void* Qs, const void* Kslc, int32_t* idx,
                                 float* score, float* w, hipStream_t s) {
  size_t rows = (size_t)d.B * d.L * d.Hkv;
  if (rows == 0) return hipSuccess;
  Timed tm(HSA_KERNEL_SELECT, s);
  if (d.dtype == 1)
    k_select_generic<bf16><<<dim3((unsigned)rows), 64, 0, s>>>(
        (const bf16*)Qs, (const bf16*)Kslc, idx, score, w, d.L, d.Hkv, d.D, d.S, d.K, d.nC,
        d.sel_scale);
  else
    k_select_generic<float><<<dim3((unsigned)rows), 64, 0, s>>>(
        (const float*)Qs, (const float*)Kslc, idx, score, w, d.L, d.Hkv, d.D, d.S, d.K, d.nC,
        d.sel_scale);
  return hipGetLastError();
}

}  // namespace hsa
