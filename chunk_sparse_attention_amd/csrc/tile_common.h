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
// Tokens per scheduling piece (see build_jobs); a piece of one job when equal to the jobs'
// tokens.
constexpr int kPieceTokens = 2;

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

// Inclusive scan of N ints in LDS (N a power of two, at most 4*NT), op 0 = sum, 1 = max
// (values >= -1).  Each thread scans up to four consecutive elements in registers, the
// waves scan the thread totals with shuffles, and wtot (NT/64 ints) carries the wave totals.
template <int NT>
__device__ void block_inclusive_scan(int* a, int* wtot, int N, int op) {
  const int ident = op == 0 ? 0 : -1;
  const int P = N > NT ? N / NT : 1;
  const int base = threadIdx.x * P;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int v[4];
  int acc = ident;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    v[p] = ident;
    if (p < P && base + p < N) {
      const int x = a[base + p];
      acc = op == 0 ? acc + x : max(acc, x);
      v[p] = acc;
    }
  }
  int x = acc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x = op == 0 ? x + y : max(x, y);
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int pre = ident;
  for (int w = 0; w < wave; ++w) pre = op == 0 ? pre + wtot[w] : max(pre, wtot[w]);
  const int below = __shfl_up(x, 1, 64);
  if (lane > 0) pre = op == 0 ? pre + below : max(pre, below);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    if (p < P && base + p < N) a[base + p] = op == 0 ? pre + v[p] : max(pre, v[p]);
  __syncthreads();
}

// From sorted keys[0..N): the number of valid edges and the job list.  A job is up to
// `tpj` consecutive edges of one chunk; jobs[j] = first edge | (edge count << 16).  Up to
// 4/tpj consecutive jobs of one chunk form a piece (at most four tokens) that is scheduled as
// a unit, so one wave serves them with one load of the chunk's operands; phead[j] = the
// piece's first job.
// Scratch arrays rs and tmp hold N ints each (tmp also holds the scan's wave totals).
// Returns through *n_valid / *n_jobs (LDS).
template <int NT>
__device__ void build_jobs(const uint32_t* keys, int N, int tpj, int* rs, int* tmp,
                           uint32_t* jobs, int* phead, int* n_valid, int* n_jobs) {
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
  int* jf = tmp + 64;
  for (int i = threadIdx.x; i < N; i += NT) jf[i] = (i < nv && (i - rs[i]) % tpj == 0) ? 1 : 0;
  __syncthreads();
  block_inclusive_scan<NT>(jf, tmp, N, 0);
  if (threadIdx.x == 0) *n_jobs = nv > 0 ? jf[nv - 1] : 0;
  for (int i = threadIdx.x; i < nv; i += NT) {
    if ((i - rs[i]) % tpj == 0) {
      int cnt = 1;
      const int c = edge_chunk(keys[i]);
      while (cnt < tpj && i + cnt < nv && edge_chunk(keys[i + cnt]) == c) ++cnt;
      const int j = jf[i] - 1;
      const int pj = max(1, kPieceTokens / tpj);    // jobs per piece
      const int first = jf[rs[i]] - 1;              // first job of the chunk's run
      jobs[j] = (uint32_t)i | ((uint32_t)cnt << 16);
      phead[j] = first + (j - first) / pj * pj;
    }
  }
  __syncthreads();
}

// Conflict-free rounds.  Jobs of one round touch disjoint tokens, so the waves of a round
// can update the tile's LDS accumulators with plain read-add-write (LDS float atomics are
// slow on this part).  Pieces (see build_jobs) are coloured as units by the greedy rule in
// piece order -- a piece takes the lowest round that no earlier piece sharing one of its
// tokens has -- computed in parallel: a piece picks its round as soon as all those earlier
// pieces have theirs, which gives the same rounds as colouring the pieces one by one, in as
// many steps as the longest chain of such dependencies (about 20 for random top-8
// selections).  A piece has at most 4 tokens and a token at most 16 edges, so no round
// exceeds 4*15 = 60.  Every job takes its piece's round, and a piece's jobs stay adjacent.
// In: jobs[0..n_jobs), phead, keys.  Out: order[] = jobs grouped by round, roff[0..n_rounds]
// = round offsets, *n_rounds.  Within a round no token repeats, so the order inside a round
// does not change any token's accumulation order.  Scratch: colour[n_jobs], jl[TT*16],
// cnt[64] (ints), tmask[TT].
template <int NT, int TT>
__device__ void build_rounds(const uint32_t* keys, const uint32_t* jobs, const int* phead,
                             int n_jobs, int Kt, int* colour, int* jl, int* cnt,
                             unsigned long long* tmask, int* roff, uint32_t* order,
                             int* n_rounds) {
  constexpr int kNone = 0x7fffffff;
  static_assert(TT * 16 % 4 == 0, "token lists are read as 16-byte words");
  for (int i = threadIdx.x; i < TT * 16; i += NT) jl[i] = kNone;
  for (int i = threadIdx.x; i < 64; i += NT) cnt[i] = 0;
  for (int i = threadIdx.x; i < TT; i += NT) tmask[i] = 0;
  __syncthreads();
  // token -> its pieces (every (token, slot) edge lies in exactly one job, hence one piece)
  for (int j = threadIdx.x; j < n_jobs; j += NT) {
    const uint32_t job = jobs[j];
    const int e0 = (int)(job & 0xffff), c = (int)(job >> 16);
    for (int i = 0; i < c; ++i) {
      const uint32_t k = keys[e0 + i];
      jl[edge_token(k) * 16 + edge_slot(k)] = phead[j];
    }
    colour[j] = -1;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < TT; t += NT) {  // ascending piece order per token
    int v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = q < Kt ? jl[t * 16 + q] : kNone;
#pragma unroll
    for (int a = 1; a < 16; ++a)
#pragma unroll
      for (int q = a; q > 0; --q)
        if (v[q] < v[q - 1]) {
          const int tmp = v[q];
          v[q] = v[q - 1];
          v[q - 1] = tmp;
        }
#pragma unroll
    for (int q = 0; q < 16; ++q) jl[t * 16 + q] = v[q];
  }
  __syncthreads();
  // rounds of the piece heads.  The earlier pieces of one token form a chain (each waits
  // for the one before it), so a piece is ready exactly when the latest earlier piece of
  // each of its tokens has a round.  Each lane takes its heads (j = lane + s*NT) in
  // ascending order and re-checks its current one until it is ready; the smallest head
  // without a round is always some lane's current one and is ready, so the waves make
  // progress without block barriers.  tmask[t] collects the rounds of t's pieces so far
  // (its earlier pieces); a piece adds its round there before it publishes the round.
  {
    constexpr int kJpt = 4;  // jobs per lane: n_jobs <= TT*16 <= 4*NT
    // colour and tmask are written by other waves while this loop spins: both are read
    // through volatile pointers, so every read is a fresh LDS load issued in program order
    // (a piece's tmask reads come after the colour reads that found it ready)
    const volatile int* vcol = colour;
    const volatile unsigned long long* vmask = tmask;
    int nts[kJpt], prevs[kJpt][4], tks[kJpt][4];
#pragma unroll
    for (int s = 0; s < kJpt; ++s) {  // every head's tokens and latest earlier pieces
      const int j = threadIdx.x + s * NT;
      nts[s] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        prevs[s][i] = -1;
        tks[s][i] = 0;
      }
      if (j < n_jobs && phead[j] == j) {
        int n = 0;
        for (int jj = j; jj < n_jobs && phead[jj] == j; ++jj) {
          const uint32_t job = jobs[jj];
          const int e0 = (int)(job & 0xffff), c = (int)(job >> 16);
          for (int i = 0; i < c; ++i) {
            const int t = edge_token(keys[e0 + i]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (q == n) tks[s][q] = t;
            ++n;
          }
        }
        nts[s] = n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < n) {
            const int4* l4 = reinterpret_cast<const int4*>(jl + tks[s][i] * 16);
            int pv = -1;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int4 x = l4[w];
              pv = x.x < j ? max(pv, x.x) : pv;
              pv = x.y < j ? max(pv, x.y) : pv;
              pv = x.z < j ? max(pv, x.z) : pv;
              pv = x.w < j ? max(pv, x.w) : pv;
            }
            prevs[s][i] = pv;
          }
        }
      }
    }
    int cur = 0;
    for (;;) {
      // the current head: the next slot with a piece (slots without one are skipped)
      int nt = 0, prev[4], tk[4], jcur = 0;
#pragma unroll
      for (int s = kJpt - 1; s >= 0; --s)
        if (s >= cur && nts[s] > 0) {
          nt = nts[s];
          jcur = threadIdx.x + s * NT;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            prev[i] = prevs[s][i];
            tk[i] = tks[s][i];
          }
        }
      if (!__ballot(nt > 0)) break;
      if (nt > 0) {
        bool ready = true;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nt && prev[i] >= 0 && vcol[prev[i]] < 0) ready = false;
        if (ready) {
          uint64_t u = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < nt) u |= vmask[tk[i]];
          const int r = __builtin_ctzll(~u);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < nt) atomicOr(&tmask[tk[i]], 1ull << r);
          __threadfence_block();
          colour[jcur] = r;
          cur = (jcur - threadIdx.x) / NT + 1;
        }
      }
    }
    __syncthreads();
  }
  // every job takes its piece's round; round sizes, offsets (rounds used are
  // 0..n_rounds-1); then each head places its piece's jobs adjacently
  for (int j = threadIdx.x; j < n_jobs; j += NT) {
    const int r = colour[phead[j]];
    atomicAdd(&cnt[r], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int size = cnt[lane];
    int incl = size;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const uint64_t nz = __ballot(size > 0);
    const int nr = nz ? 64 - __builtin_clzll(nz) : 0;
    if (lane <= nr) roff[lane] = incl - size;
    if (lane == 0) *n_rounds = nr;
    cnt[lane] = incl - size;  // placement cursor of round `lane`
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n_jobs; j += NT) {
    if (phead[j] != j) continue;
    int sz = 1;
    while (j + sz < n_jobs && phead[j + sz] == j) ++sz;
    const int pos = atomicAdd(&cnt[colour[j]], sz);
    for (int i = 0; i < sz; ++i) order[pos + i] = jobs[j + i];
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
  __shared__ __attribute__((aligned(16))) int jl[TT * 16];
  __shared__ int phead[NMAX];
  __shared__ int cnt[64];
  __shared__ unsigned long long tmask[TT];
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
  build_jobs<NT>(keys, N, tpj, scratch, scratch + NMAX, jobs, phead, &n_valid_sh, &n_jobs_sh);
  const int n_jobs = n_jobs_sh;
  uint32_t* order = reinterpret_cast<uint32_t*>(scratch + NMAX);
  int* roff = scratch + 2 * NMAX;
  build_rounds<NT, TT>(keys, jobs, phead, n_jobs, Kt, scratch, jl, cnt, tmask, roff, order,
                       &n_rounds_sh);
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

// Maximum of unsigned values over the whole wave, in every lane (0 is the identity).
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dppu<0xB1>(v));
  v = max(v, dppu<0x4E>(v));
  v = max(v, dppu<0x141>(v));
  v = max(v, dppu<0x140>(v));
  auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  unsigned p0 = p[0], p1 = p[1];
  asm volatile("" : "+v"(p0), "+v"(p1));
  v = max(p0, p1);
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  unsigned r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  return max(r0, r1);
}

// ---- 64-bit rank keys across lanes ---------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_key(uint64_t v) {
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, 0xF, 0xF, true);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
  const uint64_t o = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
  return o > v ? o : v;
}
// Maximum over the 16 lanes of a row, in every lane of the row.
__device__ __forceinline__ uint64_t row16_max_key(uint64_t v) {
  v = dpp_max_key<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_key<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_key<0x141>(v);  // row_half_mirror
  return dpp_max_key<0x140>(v);  // row_mirror
}
// Maximum of v and its partner 16 (rows32 = false) or 32 (true) lanes away; the halves of a
// key travel together through the swap, and the empty asm keeps the two results apart.
__device__ __forceinline__ uint64_t swap_max_key(uint64_t v, bool rows32) {
  const unsigned hi = (unsigned)(v >> 32), lo = (unsigned)v;
  unsigned h0, h1, l0, l1;
  if (rows32) {
    auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    h0 = ph[0]; h1 = ph[1]; l0 = pl[0]; l1 = pl[1];
  } else {
    auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    h0 = ph[0]; h1 = ph[1]; l0 = pl[0]; l1 = pl[1];
  }
  asm volatile("" : "+v"(h0), "+v"(h1), "+v"(l0), "+v"(l1));
  const uint64_t a = ((uint64_t)h0 << 32) | l0, b = ((uint64_t)h1 << 32) | l1;
  return a > b ? a : b;
}
// Maximum over lanes l, l^16, l^32, l^48 (the four rows at one position).
__device__ __forceinline__ uint64_t rows4_max_key(uint64_t v) {
  return swap_max_key(swap_max_key(v, false), true);
}
// Maximum over the whole wave, in every lane.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  return rows4_max_key(row16_max_key(v));
}

}  // namespace hsa
