// decode_generic.hip -- one decode step per sequence (fp32 and bf16).
//
// At inference only the compact chunk-key table stays resident for selection, and each step
// reads only the selected chunks' key/value rows ("Hardware-aligned Hierarchical Sparse
// Attention ...", papernotes.org note, 方法详解 › 训练与推理优化, KV Cache Offloading).  The
// scan of the chunk table is the memory-bound part: it is split over many blocks, each
// keeping its own top-K, and a second kernel merges the candidates, forms the
// stick-breaking weights and attends over the K selected chunks.
#include "hsa_common.h"
#include "hsa_launch.h"

namespace hsa {

constexpr int kDecChunksPerBlock = 256;

DecLayout dec_layout(const Dims& d) {
  DecLayout l{};
  l.chunks_per_block = kDecChunksPerBlock;
  l.n_blocks = d.nC > 0 ? (d.nC + kDecChunksPerBlock - 1) / kDecChunksPerBlock : 1;
  l.cand = 0;
  l.total = sizeof(uint64_t) * (size_t)d.B * d.Hkv * l.n_blocks * d.K;
  l.total = (l.total + 255) & ~(size_t)255;
  return l;
}

// Scan: one thread per chunk; block-local top-K by repeated 64-bit maxima.
template <typename T>
__global__ void __launch_bounds__(256) k_dec_scan(const T* __restrict__ qs,
                                                  const T* __restrict__ Kslc,
                                                  uint64_t* __restrict__ cand, int Hkv, int D,
                                                  int K, int nC, int n_blocks,
                                                  double sel_scale,
                                                  const int32_t* __restrict__ ctx_lens) {
  __shared__ double qsh[128];
  __shared__ uint64_t wbest[4][kMaxK];
  const int blk = blockIdx.x % n_blocks;
  const int bg = blockIdx.x / n_blocks;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  for (int e = tid; e < D; e += blockDim.x) qsh[e] = (double)to_f32(qs[((size_t)b * Hkv + g) * D + e]);
  __syncthreads();
  const int c = blk * kDecChunksPerBlock + tid;
  // chunks this sequence may select: all nC of the table, or those below its own length
  const int nCb = ctx_lens ? min(nC, max(0, ctx_lens[b]) / kChunk) : nC;
  uint64_t key = 0;
  if (c < nCb) {
    const T* kr = Kslc + ((b * nC + c) * Hkv + g) * D;
    double dot = 0.0;
    for (int e = 0; e < D; e += 8) {
      float kv[8];
      load8(kr + e, kv);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += qsh[e + i] * (double)kv[i];
    }
    key = rank_key((float)(sel_scale * dot), c);
  }
  for (int k = 0; k < K; ++k) {
    uint64_t best = wave_max_u64(key);
    if (key == best) key = 0;
    if (lane == 0) wbest[wave][k] = best;
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t v = (lane < 4 * K) ? wbest[lane / K][lane % K] : 0;
    for (int k = 0; k < K; ++k) {
      uint64_t best = wave_max_u64(v);
      if (v == best) v = 0;
      if (lane == 0) cand[((size_t)bg * n_blocks + blk) * K + k] = best;
    }
  }
}

// Merge + weights + attention, one wave per (sequence, group).
template <typename T>
__global__ void __launch_bounds__(64) k_dec_attend(
    const T* __restrict__ q, const T* __restrict__ Kc, const T* __restrict__ Vc,
    const uint64_t* __restrict__ cand, T* __restrict__ O, int32_t* __restrict__ idx,
    float* __restrict__ score, float* __restrict__ w, int ctx, int Hq, int Hkv, int D, int S,
    int K, int G, int nC, int n_blocks, float sm_scale, int softmax_w) {
  __shared__ float qsh[kMaxG][128];
  __shared__ float ash[kMaxG][kChunk];
  __shared__ int sidx[kMaxK];
  __shared__ float sw[kMaxK];
  const int lane = threadIdx.x;
  const int bg = blockIdx.x;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  uint64_t top[kMaxK];
#pragma unroll
  for (int i = 0; i < kMaxK; ++i) top[i] = 0;
  const int n_cand = n_blocks * K;
  for (int i = lane; i < n_cand; i += kWave) topk_insert(top, cand[(size_t)bg * n_cand + i], K);
  __shared__ uint64_t skey[kMaxK];
  for (int k = 0; k < K; ++k) {
    uint64_t best = wave_max_u64(top[0]);
    if (best != 0 && top[0] == best) topk_pop(top);
    if (lane == 0) skey[k] = best;
  }
  __syncthreads();
  if (lane == 0) {
    // softmax weights: the valid slots' largest score and the sum of their exponentials
    double m = -__builtin_inf(), den = 0.0;
    if (softmax_w) {
      for (int k = 0; k < K; ++k)
        if (skey[k] != 0) m = fmax(m, (double)key_score(skey[k]));
      for (int k = 0; k < K; ++k)
        if (skey[k] != 0 && m != -__builtin_inf()) den += exp((double)key_score(skey[k]) - m);
    }
    double remaining = 1.0;
    for (int k = 0; k < K; ++k) {
      const uint64_t key = skey[k];
      const size_t o = (size_t)bg * K + k;
      if (key == 0) {
        sidx[k] = -1;
        sw[k] = 0.0f;
        idx[o] = -1;
        if (score) score[o] = -__builtin_inff();
        w[o] = 0.0f;
      } else {
        const float s = key_score(key);
        float wk;
        if (softmax_w) {
          wk = den > 0.0 ? (float)(exp((double)s - m) / den) : 0.0f;
        } else {
          const double p = sigmoid_d((double)s);
          wk = (float)(p * remaining);
          remaining *= 1.0 - p;
        }
        sidx[k] = key_chunk(key);
        sw[k] = wk;
        idx[o] = key_chunk(key);
        if (score) score[o] = s;
        w[o] = wk;
      }
    }
  }
  const size_t qbase = ((size_t)b * Hq + (size_t)g * G) * D;
  for (int i = lane; i < G * D; i += kWave) qsh[i / D][i % D] = to_f32(q[qbase + i]);
  __syncthreads();

  float acc[kMaxG][2];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) acc[h][0] = acc[h][1] = 0.0f;
  const size_t kvstride = (size_t)Hkv * D;
  for (int k = 0; k < K; ++k) {
    const int c = sidx[k];
    if (c < 0) continue;
    const float wk = sw[k];
    const size_t cbase = ((b * ctx + (size_t)c * S) * Hkv + g) * D;
    float z[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) z[h] = 0.0f;
    const T* kr = Kc + cbase + (size_t)lane * kvstride;
    for (int e = 0; e < D; e += 8) {
      float kv[8];
      load8(kr + e, kv);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h)
        if (h < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) z[h] += qsh[h][e + i] * kv[i];
        }
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float zz = z[h] * sm_scale;
        float m = fmaxf(0.0f, wave_max(zz));
        float ex = __expf(zz - m);
        ash[h][lane] = wk * ex / (__expf(-m) + wave_sum(ex));
      }
    }
    __syncthreads();
    const T* vr = Vc + cbase;
    for (int j = 0; j < kChunk; ++j) {
      float v0 = to_f32(vr[(size_t)j * kvstride + lane]);
      float v1 = (D > 64) ? to_f32(vr[(size_t)j * kvstride + 64 + lane]) : 0.0f;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h)
        if (h < G) {
          acc[h][0] += ash[h][j] * v0;
          acc[h][1] += ash[h][j] * v1;
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      O[qbase + (size_t)h * D + lane] = from_f32<T>(acc[h][0]);
      if (D > 64) O[qbase + (size_t)h * D + 64 + lane] = from_f32<T>(acc[h][1]);
    }
  }
}

hipError_t launch_decode_generic(const Dims& d, const DecLayout& lay, const void* q,
                                 const void* qs, const void* Kc, const void* Vc,
                                 const void* Kslc, void* O, int32_t* idx, float* score,
                                 float* w, const int32_t* ctx_lens, char* ws, hipStream_t s) {
  const int bg = d.B * d.Hkv;
  if (bg == 0) return hipSuccess;
  uint64_t* cand = (uint64_t*)(ws + lay.cand);
  float sm = (float)d.sm_scale;
  // d.L is the context length; the new token may select every complete chunk.
  if (d.dtype == 1) {
    {
      Timed tm(HSA_KERNEL_DECODE_SCAN, s);
      k_dec_scan<bf16><<<dim3(bg * lay.n_blocks), 256, 0, s>>>(
          (const bf16*)qs, (const bf16*)Kslc, cand, d.Hkv, d.D, d.K, d.nC, lay.n_blocks,
          d.sel_scale, ctx_lens);
    }
    Timed tm(HSA_KERNEL_DECODE_ATTEND, s);
    k_dec_attend<bf16><<<dim3(bg), 64, 0, s>>>((const bf16*)q, (const bf16*)Kc, (const bf16*)Vc,
                                               cand, (bf16*)O, idx, score, w, d.L, d.Hq, d.Hkv,
                                               d.D, d.S, d.K, d.G, d.nC, lay.n_blocks, sm,
                                               softmax_w(d));
  } else {
    {
      Timed tm(HSA_KERNEL_DECODE_SCAN, s);
      k_dec_scan<float><<<dim3(bg * lay.n_blocks), 256, 0, s>>>(
          (const float*)qs, (const float*)Kslc, cand, d.Hkv, d.D, d.K, d.nC, lay.n_blocks,
          d.sel_scale, ctx_lens);
    }
    Timed tm(HSA_KERNEL_DECODE_ATTEND, s);
    k_dec_attend<float><<<dim3(bg), 64, 0, s>>>(
        (const float*)q, (const float*)Kc, (const float*)Vc, cand, (float*)O, idx, score, w,
        d.L, d.Hq, d.Hkv, d.D, d.S, d.K, d.G, d.nC, lay.n_blocks, sm, softmax_w(d));
  }
  return hipGetLastError();
}

}  // namespace hsa
