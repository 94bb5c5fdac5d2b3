// select_tile.hip -- tiled top-K chunk selection (fp32 and bf16 inputs).
//
// Chunk selection ("Hardware-aligned Hierarchical Sparse Attention ...", papernotes.org note,
// 方法详解 › 层次化稀疏注意力（HSA）, Chunk Selection): every token scores each earlier chunk's
// pooled key with its selection query and keeps the top-K, per query group; the chunk
// weights are stick-breaking over the sigmoid of the ranked scores (same section, 第二阶段).
//
// The 64 tokens of one query chunk share their candidate set (all chunks before it), so a
// block scores a 64-token tile against blocks of 64 chunks staged in LDS.  Thread (tr, tc)
// owns tokens 4tr..4tr+3 and chunks 4tc..4tc+3 of each block and accumulates those 16 dot
// products in fp64 in dimension order (the products of stored bf16/fp32 values are exact in
// fp64, so each score is the correctly rounded definition); it keeps a running top-K per
// token over its chunks, and the 16 threads of a token merge their lists at the end.
#include "hsa_common.h"
#include "hsa_launch.h"
#include "tile_common.h"

namespace hsa {

template <typename T, int D>
__global__ void __launch_bounds__(256) k_select_tile(const T* __restrict__ Qs,
                                                     const T* __restrict__ Kslc,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ score,
                                                     float* __restrict__ w, int L, int Hkv,
                                                     int Kt, int nC, int BG, double sel_scale) {
  __shared__ float qt[D][64];   // Qs tile, transposed: [dim][token]
  __shared__ float kb[D][64];   // chunk-key block, transposed: [dim][chunk]
  const int bg = blockIdx.x % BG;
  const int q = blockIdx.x / BG;  // query chunk of the tile
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int t0 = q * 64;
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  const int m = min(q, nC);  // candidates of every token in the tile

  // fills: lane = token (or chunk), 8 consecutive dimensions per load, conflict-free LDS rows
  for (int i = tid; i < 64 * D / 8; i += 256) {
    const int tl = i % 64, e0 = (i / 64) * 8, t = t0 + tl;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (t < L) load8(Qs + ((b * L + t) * Hkv + g) * D + e0, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) qt[e0 + j][tl] = v[j];
  }
  uint64_t top[4][kMaxK];
  uint64_t thr[4];  // smallest kept key per token (0 while the list is not full)
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    thr[a] = 0;
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) top[a][i] = 0;
  }

  for (int c0 = 0; c0 < m; c0 += 64) {
    __syncthreads();
    for (int i = tid; i < 64 * D / 8; i += 256) {
      const int cl = i % 64, e0 = (i / 64) * 8, c = c0 + cl;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (c < m) load8(Kslc + ((b * nC + c) * Hkv + g) * D + e0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) kb[e0 + j][cl] = v[j];
    }
    __syncthreads();
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[a][j] = 0.0;
    for (int e = 0; e < D; ++e) {
      const float4 qv = *reinterpret_cast<const float4*>(&qt[e][4 * tr]);
      const float4 kv = *reinterpret_cast<const float4*>(&kb[e][4 * tc]);
      const double qd[4] = {qv.x, qv.y, qv.z, qv.w};
      const double kd[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[a][j] = fma(qd[a], kd[j], acc[a][j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + 4 * tc + j;
      if (c < m) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint64_t key = rank_key((float)(sel_scale * acc[a][j]), c);
          if (key > thr[a]) {
            topk_insert(top[a], key, Kt);
#pragma unroll
            for (int i = 0; i < kMaxK; ++i)
              if (i == Kt - 1) thr[a] = top[a][i];
          }
        }
      }
    }
  }

  // merge the 16 lists of each token (the 16 lanes of one row) and write the slots
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int tl = 4 * tr + a, t = t0 + tl;
    uint64_t mine = 0;  // lane tc keeps the key of slot tc
    for (int k = 0; k < Kt; ++k) {
      const uint64_t best = row16_max_key(top[a][0]);
      if (best != 0 && top[a][0] == best) topk_pop(top[a]);
      if (tc == k) mine = best;
    }
    // stick-breaking in rank order: lane tc needs prod_{j<tc} (1 - p_j), a row prefix product
    double p = 0.0;
    if (tc < Kt && mine != 0) p = sigmoid_d((double)key_score(mine));
    double keep = 1.0 - p;
    double excl = 1.0;  // product of (1 - p_j) over j < tc
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const double x = __shfl_up(keep, o, 16);
      if (tc >= o) keep *= x;
    }
    excl = __shfl_up(keep, 1, 16);
    if (tc == 0) excl = 1.0;
    if (t < L && tc < Kt) {
      const size_t o = ((b * L + t) * Hkv + g) * Kt + tc;
      if (mine == 0) {
        idx[o] = -1;
        score[o] = -__builtin_inff();
        w[o] = 0.0f;
      } else {
        idx[o] = key_chunk(mine);
        score[o] = key_score(mine);
        w[o] = (float)(p * excl);
      }
    }
  }
}

bool select_tile_supported(const Dims& d) { return !(d.flags & 1u); }

hipError_t launch_select_tile(const Dims& d, const void* Qs, const void* Kslc, int32_t* idx,
                              float* score, float* w, hipStream_t s) {
  const int BG = d.B * d.Hkv;
  const int n_tiles = (d.L + 63) / 64;
  dim3 grid((unsigned)(BG * n_tiles));
  auto go = [&](auto kern, auto* qs, auto* ks) {
    Timed tm(HSA_KERNEL_SELECT, s);
    kern<<<grid, 256, 0, s>>>(qs, ks, idx, score, w, d.L, d.Hkv, d.K, d.nC, BG, d.sel_scale);
  };
  if (d.dtype == 1) {
    if (d.D == 64) go(k_select_tile<bf16, 64>, (const bf16*)Qs, (const bf16*)Kslc);
    else go(k_select_tile<bf16, 128>, (const bf16*)Qs, (const bf16*)Kslc);
  } else {
    if (d.D == 64) go(k_select_tile<float, 64>, (const float*)Qs, (const float*)Kslc);
    else go(k_select_tile<float, 128>, (const float*)Qs, (const float*)Kslc);
  }
  return hipGetLastError();
}

}  // namespace hsa
