// lse.hip -- the softmax-off-by-one normalisers at the boundary.
//
// Inside the library the matrix-core forward keeps, per (token, group, slot), the G heads'
// normalisers next to each other in the log2 domain (z scaled by log2 e):
//   state[((b*L + t)*Hkv + g)*K + k)*G + h] = log2(1 + sum_j 2^(z_j log2 e)).
// At the C ABI they are the natural-log values in the layout of the queries, one per
// (token, head, slot): lse[((b*L + t)*Hq + g*G + h)*K + k] = log(1 + sum_j exp(z_j)), 0 for a
// masked slot ("Hardware-aligned Hierarchical Sparse Attention ...", papernotes.org note,
// 方法详解 › 硬件对齐 Kernel: softmax-off-by-one inside each selected chunk).
#include "hsa_common.h"
#include "hsa_launch.h"

namespace hsa {

// One thread per lse element (the ABI layout); masked slots get 0.
__global__ void __launch_bounds__(256) k_lse_export(const float* __restrict__ state,
                                                    const int32_t* __restrict__ idx,
                                                    float* __restrict__ lse, int Hq, int Hkv,
                                                    int Kt, int nC, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int k = (int)(i % Kt);
  const int hq = (int)((i / Kt) % Hq);
  const int64_t bt = i / ((int64_t)Kt * Hq);
  const int G = Hq / Hkv, g = hq / G, h = hq % G;
  const int64_t so = (bt * Hkv + g) * Kt + k;
  const int c = idx[so];
  lse[i] = (c >= 0 && c < nC) ? state[so * G + h] * 0.69314718055994531f : 0.0f;
}

// The inverse: the ABI values into the state layout (log2 domain).
__global__ void __launch_bounds__(256) k_lse_import(const float* __restrict__ lse,
                                                    float* __restrict__ state, int Hq, int Hkv,
                                                    int Kt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // state index
  if (i >= n) return;
  const int G = Hq / Hkv;
  const int h = (int)(i % G);
  const int64_t so = i / G;
  const int k = (int)(so % Kt);
  const int64_t btg = so / Kt;
  const int g = (int)(btg % Hkv);
  const int64_t bt = btg / Hkv;
  state[i] = lse[(bt * Hq + (int64_t)g * G + h) * Kt + k] * 1.4426950408889634f;
}

hipError_t launch_lse_export(const Dims& d, const float* state, const int32_t* idx, float* lse,
                             hipStream_t s) {
  const int64_t n = (int64_t)d.B * d.L * d.Hq * d.K;
  if (n == 0) return hipSuccess;
  k_lse_export<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(state, idx, lse, d.Hq, d.Hkv,
                                                                  d.K, d.nC, n);
  return hipGetLastError();
}

hipError_t launch_lse_import(const Dims& d, const float* lse, float* state, hipStream_t s) {
  const int64_t n = (int64_t)d.B * d.L * d.Hq * d.K;
  if (n == 0) return hipSuccess;
  k_lse_import<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(lse, state, d.Hq, d.Hkv, d.K,
                                                                  n);
  return hipGetLastError();
}

}  // namespace hsa
