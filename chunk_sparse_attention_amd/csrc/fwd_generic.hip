// fwd_generic.hip -- plain vector-ALU forward (any supported shape, fp32 and bf16).
//
// Token-level attention inside each selected chunk, normalised with softmax-off-by-one
// ("Hardware-aligned Hierarchical Sparse Attention ...", papernotes.org note, 方法详解 ›
// 层次化稀疏注意力（HSA） 第一阶段 and 硬件对齐 Kernel), fused with the stick-breaking chunk
// weights (same note, 第二阶段): O_t = sum_k w_k softmax1(q K_c^T) V_c.
#include "hsa_common.h"
#include "hsa_launch.h"

namespace hsa {

// One wave per (b, t, g) row.  Lane j owns key j of the current chunk for the logits; lane
// e owns output columns e and e+64 for the weighted sum over the chunk's values.
template <typename T>
__global__ void __launch_bounds__(64) k_fwd_generic(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const float* __restrict__ w, T* __restrict__ O,
    float* __restrict__ lse, int L, int Hq, int Hkv, int D, int S, int Kt, int G, int nC,
    float sm_scale) {
  __shared__ float qsh[kMaxG][128];
  __shared__ float ash[kMaxG][kChunk];
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;  // (b*L + t)*Hkv + g
  const int g = (int)(row % Hkv);
  const size_t bt = row / Hkv;
  const size_t b = bt / L;
  const size_t qbase = (bt * Hq + (size_t)g * G) * D;  // first head of the group

  for (int i = lane; i < G * D; i += kWave) qsh[i / D][i % D] = to_f32(Q[qbase + i]);
  float acc[kMaxG][2];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) acc[h][0] = acc[h][1] = 0.0f;
  __syncthreads();

  const size_t kvstride = (size_t)Hkv * D;
  for (int k = 0; k < Kt; ++k) {
    const int c = idx[row * Kt + k];
    if (c < 0 || c >= nC) {  // masked slot (or out-of-range index): adds nothing
      if (lse)
        for (int h = lane; h < G; h += kWave) lse[(bt * Hq + (size_t)g * G + h) * Kt + k] = 0.0f;
      continue;
    }
    const float wk = w[row * Kt + k];
    const size_t cbase = ((b * L + (size_t)c * S) * Hkv + g) * D;
    // logits of lane j's key for every head of the group
    float z[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) z[h] = 0.0f;
    const T* kr = K + cbase + (size_t)lane * kvstride;
    for (int e = 0; e < D; e += 8) {
      float kv[8];
      load8(kr + e, kv);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) z[h] += qsh[h][e + i] * kv[i];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float zz = z[h] * sm_scale;
        float m = fmaxf(0.0f, wave_max(zz));
        float ex = __expf(zz - m);
        float den = __expf(-m) + wave_sum(ex);
        ash[h][lane] = wk * ex / den;
        if (lse && lane == 0) lse[(bt * Hq + (size_t)g * G + h) * Kt + k] = m + logf(den);
      }
    }
    __syncthreads();
    const T* vr = V + cbase;
    for (int j = 0; j < kChunk; ++j) {
      float v0 = to_f32(vr[(size_t)j * kvstride + lane]);
      float v1 = (D > 64) ? to_f32(vr[(size_t)j * kvstride + 64 + lane]) : 0.0f;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          float a = ash[h][j];
          acc[h][0] += a * v0;
          acc[h][1] += a * v1;
        }
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

hipError_t launch_fwd_generic(const Dims& d, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* w, void* O, float* lse,
                              hipStream_t s) {
  size_t rows = (size_t)d.B * d.L * d.Hkv;
  if (rows == 0) return hipSuccess;
  float sm = (float)d.sm_scale;
  Timed tm(HSA_KERNEL_FWD, s);
  if (d.dtype == 1)
    k_fwd_generic<bf16><<<dim3((unsigned)rows), 64, 0, s>>>(
        (const bf16*)Q, (const bf16*)K, (const bf16*)V, idx, w, (bf16*)O, lse, d.L, d.Hq, d.Hkv, d.D,
        d.S, d.K, d.G, d.nC, sm);
  else
    k_fwd_generic<float><<<dim3((unsigned)rows), 64, 0, s>>>(
        (const float*)Q, (const float*)K, (const float*)V, idx, w, (float*)O, lse, d.L, d.Hq, d.Hkv,
        d.D, d.S, d.K, d.G, d.nC, sm);
  return hipGetLastError();
}

}  // namespace hsa
