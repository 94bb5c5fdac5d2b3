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
// slow on this part).  Greedy colouring in job order by one thread: a job takes the lowest
// round none of its tokens is in yet.  A token has at most 16 edges, so with at most 4
// tokens per job no job needs a round above 4*15 = 60.
// In: jobs[0..n_jobs), keys.  Out: order[] = jobs grouped by round (job order kept inside
// a round), roff[0..n_rounds] = round offsets, *n_rounds.  Scratch: tmask[TT] (uint64),
// jround[n_jobs] (int).
template <int NT, int TT>
__device__ void build_rounds(const uint32_t* keys, const uint32_t* jobs, int n_jobs,
                             uint64_t* tmask, int* jround, int* roff, uint32_t* order,
                             int* n_rounds) {
  for (int i = threadIdx.x; i < TT; i += NT) tmask[i] = 0;
  for (int i = threadIdx.x; i <= 64; i += NT) roff[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    int rmax = -1;
    for (int j = 0; j < n_jobs; ++j) {
      const uint32_t job = jobs[j];
      const int e0 = (int)(job & 0xffff), cnt = (int)(job >> 16);
      uint64_t used = 0;
      for (int i = 0; i < cnt; ++i) used |= tmask[edge_token(keys[e0 + i])];
      const int r = __builtin_ctzll(~used);
      for (int i = 0; i < cnt; ++i) tmask[edge_token(keys[e0 + i])] |= 1ull << r;
      jround[j] = r;
      roff[r + 1] += 1;
      rmax = max(rmax, r);
    }
    int run = 0;
    for (int r = 0; r <= rmax; ++r) {
      run += roff[r + 1];
      roff[r + 1] = run;
    }
    *n_rounds = rmax + 1;
    // stable placement: position = round offset + number of earlier jobs of that round
    for (int j = 0; j < n_jobs; ++j) order[roff[jround[j]]++] = jobs[j];
    for (int r = rmax; r >= 1; --r) roff[r] = roff[r - 1];
    roff[0] = 0;
  }
  __syncthreads();
}

}  // namespace hsa
