// tile_common.h -- per-tile edge lists for the token-tile MFMA kernels.
//
// A tile is a run of consecutive tokens of one (batch, KV group).  Its (token, slot)
// selections are its edges.  The kernels group the edges by chunk so that one wave can hold
// a chunk's key/value operands in registers while it serves every token of the tile that
// selected it; consecutive tokens of one chunk are packed into 16-column MFMA jobs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

constexpr uint32_t kNoEdge = 0xffffffffu;

// Edge key: chunk in the high 16 bits, then token-in-tile (6 bits) and slot (4 bits), so an
// ascending sort groups edges by chunk and keeps token order inside a chunk.
__device__ __forceinline__ uint32_t edge_key(int c, int tl, int k) {
  return ((uint32_t)c << 16) | ((uint32_t)tl << 4) | (uint32_t)k;
}
__device__ __forceinline__ int edge_chunk(uint32_t key) { return (int)(key >> 16); }
__device__ __forceinline__ int edge_token(uint32_t key) { return (int)((key >> 4) & 63); }
__device__ __forceinline__ int edge_slot(uint32_t key) { return (int)(key & 15); }

// Ascending bitonic sort of N (power of two) keys in LDS by the whole block.
template <int NT>
__device__ void block_bitonic_sort(uint32_t* keys, int N) {
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N; i += NT) {
        int p = i ^ j;
        if (p > i) {
          uint32_t a = keys[i], b = keys[p];
          bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Inclusive scan of N ints in LDS (Hillis-Steele), op 0 = sum, 1 = max.
template <int NT>
__device__ void block_inclusive_scan(int* a, int* tmp, int N, int op) {
  for (int off = 1; off < N; off <<= 1) {
    for (int i = threadIdx.x; i < N; i += NT) {
      int v = a[i];
      if (i >= off) v = op == 0 ? v + a[i - off] : max(v, a[i - off]);
      tmp[i] = v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += NT) a[i] = tmp[i];
    __syncthreads();
  }
}

// From sorted keys[0..N): the number of valid edges and the job list.  A job is up to
// `tpj` consecutive edges of one chunk; jobs[j] = first edge | (edge count << 16).
// Scratch arrays rs and tmp hold N ints each.  Returns through *n_valid / *n_jobs (LDS).
template <int NT>
__device__ void build_jobs(const uint32_t* keys, int N, int tpj, int* rs, int* tmp,
                           uint32_t* jobs, int* n_valid, int* n_jobs) {
  for (int i = threadIdx.x; i < N; i += NT) {
    bool v = keys[i] != kNoEdge;
    if (v && (i + 1 == N || keys[i + 1] == kNoEdge)) *n_valid = i + 1;
    if (i == 0 && !v) *n_valid = 0;
  }
  __syncthreads();
  const int nv = *n_valid;
  for (int i = threadIdx.x; i < N; i += NT) {
    bool start = i < nv && (i == 0 || edge_chunk(keys[i]) != edge_chunk(keys[i - 1]));
    rs[i] = start ? i : -1;
  }
  __syncthreads();
  block_inclusive_scan<NT>(rs, tmp, N, 1);  // rs[i] = first edge of i's chunk run
  int* jf = tmp + N;                        // second scratch half
  for (int i = threadIdx.x; i < N; i += NT) jf[i] = (i < nv && (i - rs[i]) % tpj == 0) ? 1 : 0;
  __syncthreads();
  block_inclusive_scan<NT>(jf, tmp, N, 0);
  if (threadIdx.x == 0) *n_jobs = nv > 0 ? jf[nv - 1] : 0;
  for (int i = threadIdx.x; i < nv; i += NT) {
    if ((i - rs[i]) % tpj == 0) {
      int cnt = 1;
      const int c = edge_chunk(keys[i]);
      while (cnt < tpj && i + cnt < nv && edge_chunk(keys[i + cnt]) == c) ++cnt;
      jobs[jf[i] - 1] = (uint32_t)i | ((uint32_t)cnt << 16);
    }
  }
  __syncthreads();
}

// Conflict-free rounds.  Jobs of one round touch disjoint tokens, so the waves of a round
// can update the tile's LDS accumulators with plain read-add-write (LDS float atomics are
// slow on this part).  Greedy colouring in job order: a job takes the lowest round none of
// its tokens is in yet.  A token has at most 16 edges and a job at most 4 tokens, so no job
// needs a round above 4*15 = 60.  Wave 0 does the colouring with the per-token round masks
// in registers (lane tl holds token tl's mask) so the sequential loop has no memory latency.
// In: jobs[0..n_jobs), keys.  Out: order[] = jobs grouped by round (job order kept inside a
// round), roff[0..n_rounds] = round offsets, *n_rounds.  Scratch: jround[n_jobs] (int).
template <int NT>
__device__ void build_rounds(const uint32_t* keys, const uint32_t* jobs, int n_jobs,
                             int* jround, int* roff, uint32_t* order, int* n_rounds) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint64_t tmask = 0;   // rounds used by token `lane`
    uint32_t count = 0;   // jobs in round `lane`
    int rmax = -1;
    for (int jb = 0; jb < n_jobs; jb += 64) {
      // lane i fetches job jb+i: its tokens packed 6 bits each, count in the top bits
      uint32_t packed = 0;
      if (jb + lane < n_jobs) {
        const uint32_t job = jobs[jb + lane];
        const int e0 = (int)(job & 0xffff), cnt = (int)(job >> 16);
        packed = (uint32_t)cnt << 24;
        for (int i = 0; i < cnt; ++i) packed |= (uint32_t)edge_token(keys[e0 + i]) << (6 * i);
      }
      int myr = 0;
      const int nb = min(64, n_jobs - jb);
      for (int i = 0; i < nb; ++i) {
        const uint32_t pk = __builtin_amdgcn_readlane(packed, i);
        const int cnt = (int)(pk >> 24);
        uint64_t used = 0;
        bool mine = false;
        for (int q = 0; q < cnt; ++q) {
          const int tl = (int)((pk >> (6 * q)) & 63);
          used |= ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(tmask >> 32), tl) << 32) |
                  (uint64_t)__builtin_amdgcn_readlane((uint32_t)tmask, tl);
          mine |= lane == tl;
        }
        const int r = __builtin_ctzll(~used);
        if (mine) tmask |= 1ull << r;
        if (lane == r) ++count;
        if (lane == i) myr = r;
        rmax = max(rmax, r);
      }
      if (jb + lane < n_jobs) jround[jb + lane] = myr;
    }
    // exclusive scan of the round sizes (lane r holds round r's size)
    uint32_t incl = count;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    uint32_t next = incl - count;  // start of round `lane`, advanced as jobs are placed
    if (lane <= rmax) roff[lane] = (int)next;
    if (lane == 0) {
      roff[rmax + 1] = n_jobs;
      *n_rounds = rmax + 1;
    }
    // stable placement in job order
    for (int jb = 0; jb < n_jobs; jb += 64) {
      const int myr = jb + lane < n_jobs ? jround[jb + lane] : 0;
      const uint32_t myjob = jb + lane < n_jobs ? jobs[jb + lane] : 0u;
      const int nb = min(64, n_jobs - jb);
      for (int i = 0; i < nb; ++i) {
        const int r = __builtin_amdgcn_readlane(myr, i);
        const uint32_t pos = __builtin_amdgcn_readlane(next, r);
        if (lane == r) ++next;
        if (lane == i) order[pos] = myjob;
      }
    }
  }
  __syncthreads();
}

// ---- prepared tiles ------------------------------------------------------------------------
// A tile-prep kernel sorts each tile's edges, builds its jobs and colours them into rounds,
// and stores the result; the attention kernels then only copy it into LDS.  Per tile:
//   [0] n_valid, [1] n_jobs, [2] n_rounds, [3..3+65) round offsets,
//   [68 .. 68+TT*16) sorted edge keys, [68+TT*16 .. 68+2*TT*16) jobs grouped by round.
__host__ __device__ constexpr int prep_words(int tt) { return 68 + 2 * tt * 16; }

template <int NT, int TT>
__global__ void __launch_bounds__(NT) k_tile_prep(const int32_t* __restrict__ idx,
                                                  uint32_t* __restrict__ prep, int L, int Hkv,
                                                  int Kt, int nC, int BG, int tpj) {
  constexpr int NMAX = TT * 16;
  __shared__ uint32_t keys[NMAX];
  __shared__ uint32_t jobs[NMAX];
  __shared__ int scratch[3 * NMAX];
  __shared__ int n_valid_sh, n_jobs_sh, n_rounds_sh;
  const int bg = blockIdx.x % BG;
  const int tile = blockIdx.x / BG;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int t0 = tile * TT;
  int N = 1;
  while (N < TT * Kt) N <<= 1;
  for (int i = threadIdx.x; i < N; i += NT) {
    uint32_t key = kNoEdge;
    if (i < TT * Kt) {
      const int tl = i / Kt, k = i % Kt, t = t0 + tl;
      if (t < L) {
        const int c = idx[((b * L + t) * Hkv + g) * Kt + k];
        if (c >= 0 && c < nC) key = edge_key(c, tl, k);
      }
    }
    keys[i] = key;
  }
  __syncthreads();
  block_bitonic_sort<NT>(keys, N);
  build_jobs<NT>(keys, N, tpj, scratch, scratch + NMAX, jobs, &n_valid_sh, &n_jobs_sh);
  const int n_jobs = n_jobs_sh;
  uint32_t* order = reinterpret_cast<uint32_t*>(scratch + NMAX);
  int* roff = scratch + 2 * NMAX;
  build_rounds<NT>(keys, jobs, n_jobs, scratch, roff, order, &n_rounds_sh);
  uint32_t* out = prep + (size_t)blockIdx.x * prep_words(TT);
  const int nv = n_valid_sh, nr = n_rounds_sh;
  if (threadIdx.x == 0) {
    out[0] = (uint32_t)nv;
    out[1] = (uint32_t)n_jobs;
    out[2] = (uint32_t)nr;
  }
  for (int i = threadIdx.x; i <= nr; i += NT) out[3 + i] = (uint32_t)roff[i];
  for (int i = threadIdx.x; i < nv; i += NT) out[68 + i] = keys[i];
  for (int i = threadIdx.x; i < n_jobs; i += NT) out[68 + NMAX + i] = order[i];
}

// Copy a prepared tile into LDS; returns n_jobs and n_rounds through the pointers (uniform).
template <int NT, int TT>
__device__ void load_prep(const uint32_t* __restrict__ src, uint32_t* keys, uint32_t* order,
                          int* roff, int* hdr) {
  constexpr int NMAX = TT * 16;
  if (threadIdx.x < 3) hdr[threadIdx.x] = (int)src[threadIdx.x];
  __syncthreads();
  const int nv = hdr[0], nj = hdr[1], nr = hdr[2];
  for (int i = threadIdx.x; i <= nr; i += NT) roff[i] = (int)src[3 + i];
  for (int i = threadIdx.x; i < nv; i += NT) keys[i] = src[68 + i];
  for (int i = threadIdx.x; i < nj; i += NT) order[i] = src[68 + NMAX + i];
}

// ---- cross-lane reductions without LDS ----------------------------------------------------
// Over the 16 lanes of a row (DPP butterfly: xor 1, xor 2, half-row mirror, row mirror).
template <int CTRL>
__device__ __forceinline__ float dppc(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppc<0xB1>(v);
  v += dppc<0x4E>(v);
  v += dppc<0x141>(v);
  v += dppc<0x140>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dppc<0xB1>(v));
  v = fmaxf(v, dppc<0x4E>(v));
  v = fmaxf(v, dppc<0x141>(v));
  v = fmaxf(v, dppc<0x140>(v));
  return v;
}
// Sum over aligned groups of N lanes inside a row (N = 2, 4, 8 or 16).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += dppc<0xB1>(v);
  if (N >= 4) v += dppc<0x4E>(v);
  if (N >= 8) v += dppc<0x141>(v);
  if (N >= 16) v += dppc<0x140>(v);
  return v;
}
// Across the four 16-lane rows at the same position (lanes l, l^16, l^32, l^48), with the
// gfx950 row-swap instructions.  Both inputs of a swap are the same value; the empty asm
// keeps the compiler from treating the two swapped results as one (it folds them otherwise).
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  unsigned p0 = p[0], p1 = p[1];
  asm volatile("" : "+v"(p0), "+v"(p1));
  a = __builtin_bit_cast(float, p0);
  b = __builtin_bit_cast(float, p1);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  unsigned p0 = p[0], p1 = p[1];
  asm volatile("" : "+v"(p0), "+v"(p1));
  a = __builtin_bit_cast(float, p0);
  b = __builtin_bit_cast(float, p1);
}
__device__ __forceinline__ float rows4_sum(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(a + b, a, b);
  return a + b;
}
__device__ __forceinline__ float rows4_max(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

}  // namespace hsa
