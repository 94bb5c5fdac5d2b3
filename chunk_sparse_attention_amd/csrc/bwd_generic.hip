// bwd_generic.hip -- chunk->token inverse index and the plain vector-ALU backward.
//
// The backward runs in two phases ("Hardware-aligned Hierarchical Sparse Attention ...",
// papernotes.org note, 方法详解 › 硬件对齐 Kernel): per token the gradients of the queries and
// of the chunk weights; then per chunk, over every token that selected it, the gradients of
// the keys and values.  The weight gradient flows on into the selection scores and from
// there into the selection query and the pooled chunk key (same note, 层次化稀疏注意力（HSA）
// 端到端学习).  Phase 2 reads a chunk -> (token, slot) index built without atomics contention:
// per-tile histograms, an exclusive scan, and a stable scatter in (token, slot) order.
#include "hsa_common.h"
#include "hsa_launch.h"

namespace hsa {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IndexLayout index_layout(const Dims& d, size_t& o) {
  IndexLayout x{};
  int tt = 64;
  while ((d.L + tt - 1) / tt > 256) tt *= 2;
  x.tile_tokens = tt;
  x.n_tiles = (d.L + tt - 1) / tt;
  x.seg = (fwd_chunked(d) || bwd_mfma_supported(d)) ? kBwdSeg : 128;
  const int64_t bg = (int64_t)d.B * d.Hkv;
  const int64_t E = (int64_t)d.L * d.K;  // entry capacity per (b, g)
  x.max_seg = (E + x.seg - 1) / x.seg + d.nC;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  // per (b, g, chunk, tile): the tile's count of the chunk, then its exclusive prefix
  x.tile_counts = take(sizeof(int32_t) * bg * x.n_tiles * d.nC);
  x.offsets = take(sizeof(int32_t) * bg * (d.nC + 1));
  x.entries = take(sizeof(int32_t) * bg * E);
  x.seg_start = take(sizeof(int32_t) * bg * (d.nC + 1));
  x.seg_chunk = take(sizeof(int32_t) * bg * x.max_seg);
  x.n_seg = take(sizeof(int32_t) * bg);
  x.seg_order = take(sizeof(int32_t) * bg * x.max_seg);
  return x;
}

BwdLayout bwd_layout(const Dims& d) {
  BwdLayout l{};
  const FwdState st = fwd_state(d);  // the forward's state comes first
  l.lse = st.lse;
  size_t o = st.total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const bool chunked = fwd_chunked(d);
  // the chunk-major forward builds the index in its state; otherwise it follows the state
  static_cast<IndexLayout&>(l) = chunked ? st.ix : index_layout(d, o);
  const int64_t bg = (int64_t)d.B * d.Hkv;
  const int64_t E = (int64_t)d.L * d.K;
  l.ds = take(sizeof(float) * bg * E);
  l.dw = take(sizeof(float) * bg * E);
  l.part_dk = take(sizeof(float) * bg * l.max_seg * kChunk * d.D);
  l.part_dv = take(sizeof(float) * bg * l.max_seg * kChunk * d.D);
  l.part_dks = take(sizeof(float) * bg * l.max_seg * d.D);
  if (bwd_mfma_supported(d)) {
    // per (token, group, slot, head): the edge's dQ contribution (the chunk-major forward's
    // partials' buffer, free once the forward has summed them)
    l.dq_part = chunked ? st.part : take(sizeof(uint16_t) * bg * E * d.G * d.D);
  }
  l.total = o;
  return l;
}

// ---- inverse index ---------------------------------------------------------------------

// The counting and scattering blocks keep one LDS counter per chunk; past kIndexPart chunks
// the chunks are split into parts of that many, one block per (b, g, tile, part), each
// handling only the entries whose chunk lies in its part.
constexpr int kIndexPart = 16384;

// Per (b, g, tile, part): how many of the tile's (token, slot) entries chose each chunk of
// the part, stored chunk-major: tile_counts[(bg * nC + c) * n_tiles + tile].
__global__ void __launch_bounds__(256) k_inv_count(const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ tile_counts, int L,
                                                   int Hkv, int K, int nC, int tile_tokens,
                                                   int n_tiles, int n_parts) {
  extern __shared__ int32_t cnt[];
  const int part = blockIdx.x % n_parts;
  const int tile = (blockIdx.x / n_parts) % n_tiles;
  const int bg = blockIdx.x / n_parts / n_tiles;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int c_lo = part * kIndexPart, nCp = min(nC - c_lo, kIndexPart);
  for (int c = threadIdx.x; c < nCp; c += blockDim.x) cnt[c] = 0;
  __syncthreads();
  const int t0 = tile * tile_tokens;
  const int n = (min(L, t0 + tile_tokens) - t0) * K;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int t = t0 + i / K, k = i % K;
    const int c = idx[((b * L + t) * Hkv + g) * K + k] - c_lo;
    if (c >= 0 && c < nCp) atomicAdd(&cnt[c], 1);
  }
  __syncthreads();
  int32_t* out = tile_counts + ((size_t)bg * nC + c_lo) * n_tiles + tile;
  for (int c = threadIdx.x; c < nCp; c += blockDim.x) out[(size_t)c * n_tiles] = cnt[c];
}

// One wave per (b, g, chunk): exclusive prefix of the chunk's tile counts over the tiles
// (n_tiles <= 256, four per lane), written in place; the chunk's total entries go to
// offsets[c] and its segment count to seg_start[c] (both scanned over chunks next).
__global__ void __launch_bounds__(256) k_inv_colscan(int32_t* __restrict__ tile_counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ seg_start, int nC,
                                                     int n_tiles, int seg, int n_rows) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;  // bg * nC + c
  if (row >= n_rows) return;  // whole wave
  const int lane = threadIdx.x % kWave;
  const int bg = row / nC, c = row % nC;
  int32_t* tc = tile_counts + (size_t)row * n_tiles;
  int32_t v[4], s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // lane takes tiles 4*lane .. 4*lane+3
    const int tile = 4 * lane + j;
    v[j] = tile < n_tiles ? tc[tile] : 0;
    s += v[j];
  }
  int32_t incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  int32_t run = incl - s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tile = 4 * lane + j;
    if (tile < n_tiles) tc[tile] = run;
    run += v[j];
  }
  if (lane == kWave - 1) {
    offsets[(size_t)bg * (nC + 1) + c] = incl;
    seg_start[(size_t)bg * (nC + 1) + c] = (incl + seg - 1) / seg;
  }
}

// Exclusive scan of n ints in place (one block of 1024 threads; thread-contiguous runs):
// per-thread run sums, a shuffle scan inside each wave, then the wave totals.
__device__ void block_exclusive_scan(int32_t* a, int n, int32_t* total_out) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, tid * per);
  const int hi = min(n, lo + per);
  int32_t s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  int32_t incl = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int32_t run = incl - s;
  int32_t total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) run += wsum[w];
    total += wsum[w];
  }
  if (tid == 0) *total_out = total;
  for (int i = lo; i < hi; ++i) {
    int32_t v = a[i];
    a[i] = run;
    run += v;
  }
  __syncthreads();
}

// Per (b, g): chunk offsets and the segments (ceil(n_c / seg) per chunk) with their chunk
// ids, from the per-chunk totals and segment counts.
__global__ void __launch_bounds__(1024) k_inv_scan(int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ seg_start,
                                                   int32_t* __restrict__ seg_chunk,
                                                   int32_t* __restrict__ n_seg, int nC,
                                                   int64_t max_seg) {
  __shared__ int32_t total_e, total_s;
  const int bg = blockIdx.x;
  int32_t* off = offsets + (size_t)bg * (nC + 1);
  int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  block_exclusive_scan(off, nC, &total_e);
  block_exclusive_scan(ss, nC, &total_s);
  if (threadIdx.x == 0) {
    off[nC] = total_e;
    ss[nC] = total_s;
    n_seg[bg] = total_s;
  }
  __syncthreads();
  int32_t* sc = seg_chunk + (size_t)bg * max_seg;
  for (int c = threadIdx.x; c < nC; c += blockDim.x)
    for (int s = ss[c]; s < ss[c + 1]; ++s) sc[s] = c;
}

// Per (b, g), one block: the segments ordered by the token of their first entry (a counting
// sort over kOrderBuckets token ranges; the order inside a range is whatever the LDS atomics
// give, which no result depends on: every segment writes its own partials).  Blocks of the
// chunk-major kernels that run together then gather the Q (and dO) rows of nearby tokens,
// which the last-level cache can hold, instead of rows from the whole sequence.
constexpr int kOrderBuckets = 1024;
__global__ void __launch_bounds__(1024) k_inv_order(const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ seg_start,
                                                    const int32_t* __restrict__ seg_chunk,
                                                    const int32_t* __restrict__ n_seg,
                                                    const int32_t* __restrict__ entries,
                                                    int32_t* __restrict__ seg_order, int L,
                                                    int K, int nC, int seg, int64_t max_seg) {
  __shared__ int32_t hist[kOrderBuckets];
  __shared__ int32_t total;
  const int bg = blockIdx.x;
  const int ns = n_seg[bg];
  const int32_t* off = offsets + (size_t)bg * (nC + 1);
  const int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  const int32_t* sc = seg_chunk + (size_t)bg * max_seg;
  const int32_t* ent = entries + (size_t)bg * L * K;
  int32_t* order = seg_order + (size_t)bg * max_seg;
  auto bucket = [&](int s) {
    const int c = sc[s];
    const int t = ent[off[c] + (s - ss[c]) * seg] / K;
    return (int)((int64_t)t * kOrderBuckets / L);
  };
  for (int i = threadIdx.x; i < kOrderBuckets; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < ns; s += blockDim.x) atomicAdd(&hist[bucket(s)], 1);
  __syncthreads();
  block_exclusive_scan(hist, kOrderBuckets, &total);
  for (int s = threadIdx.x; s < ns; s += blockDim.x) order[atomicAdd(&hist[bucket(s)], 1)] = s;
}

// Per (b, g, tile, part): place the tile's entries whose chunk lies in the part, a chunk's
// entries in token order from offsets[c] + the tile's prefix for c.
//   Bitmap path (W > 0: a single part, the tile's tokens fit W 64-bit words, and the block's
//   LDS holds a word row per chunk): each chunk's row marks the tile's tokens that chose it, and an
//   entry's place among the chunk's entries of the tile is the number of marked tokens before
//   its own, so every entry is placed in parallel.  This needs each row's chunks distinct.
//   Walk path (W = 0, or a row that repeats a chunk): wave 0 walks the tile's tokens in order
//   and lane k places slot k.  A selection from hsa_select never repeats a chunk within a
//   row, but a caller's may: such slots are given consecutive entries in slot order (rank r
//   among the row's equal slots goes to the counter's value + r, and the first of them
//   advances the counter past all), which is the count k_inv_count made for them, so every
//   entry is written exactly once.
// Tokens are staged in LDS kScatterBatch at a time (the bitmap path takes the whole tile:
// W * 64 <= kScatterBatch).
constexpr int kScatterBatch = 256;
constexpr int kScatterThreads = 256;
__global__ void __launch_bounds__(kScatterThreads) k_inv_scatter(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ tile_prefix,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ entries, int L, int Hkv, int K,
    int nC, int tile_tokens, int n_tiles, int n_parts, int W) {
  // the part's counters, then (bitmap path) nC * W mask words
  extern __shared__ int32_t cnt[];
  __shared__ int32_t sel[kScatterBatch * kMaxK];
  __shared__ uint16_t dup[kScatterBatch * kMaxK];  // rank among equal slots | their number << 8
  const int part = blockIdx.x % n_parts;
  const int tile = (blockIdx.x / n_parts) % n_tiles;
  const int bg = blockIdx.x / n_parts / n_tiles;
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int c_lo = part * kIndexPart, nCp = min(nC - c_lo, kIndexPart);
  const int32_t* tp = tile_prefix + ((size_t)bg * nC + c_lo) * n_tiles + tile;
  const int32_t* off = offsets + (size_t)bg * (nC + 1) + c_lo;
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(cnt + ((nCp + 1) & ~1));
  for (int c = tid; c < nCp; c += kScatterThreads) cnt[c] = off[c] + tp[(size_t)c * n_tiles];
  for (int i = tid; i < nCp * W; i += kScatterThreads) mask[i] = 0;
  int32_t* ent = entries + (size_t)bg * L * K;
  const int t0 = tile * tile_tokens;
  const int t1 = min(L, t0 + tile_tokens);
  for (int tb0 = t0; tb0 < t1; tb0 += kScatterBatch) {
    const int nt = min(kScatterBatch, t1 - tb0);
    __syncthreads();
    for (int i = tid; i < nt * K; i += kScatterThreads)
      sel[i] = idx[((b * L + tb0 + i / K) * Hkv + g) * K + i % K];
    __syncthreads();
    bool rep = false;  // some row of the batch repeats a chunk
    for (int tt = tid; tt < nt; tt += kScatterThreads) {  // one token per thread
      int cv[kMaxK];
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) cv[j] = j < K ? sel[tt * K + j] : 0;
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        if (k < K) {
          int rank = 0, n = 0;
#pragma unroll
          for (int j = 0; j < kMaxK; ++j) {
            const bool eq = j < K && cv[j] == cv[k];
            rank += (j < k && eq) ? 1 : 0;
            n += eq ? 1 : 0;
          }
          dup[tt * K + k] = (uint16_t)(rank | (n << 8));
          rep = rep || (n > 1 && cv[k] >= 0 && cv[k] < nC);
        }
      }
    }
    if (!__syncthreads_or(rep) && W > 0) {
      for (int i = tid; i < nt * K; i += kScatterThreads) {
        const int c = sel[i] - c_lo;
        if (c >= 0 && c < nCp) {
          const int tt = i / K;
          atomicOr(&mask[c * W + tt / 64], 1ull << (tt % 64));
        }
      }
      __syncthreads();
      for (int i = tid; i < nt * K; i += kScatterThreads) {
        const int c = sel[i] - c_lo;
        if (c >= 0 && c < nCp) {
          const int tt = i / K;
          const unsigned long long* m = mask + c * W;
          int r = __popcll(m[tt / 64] & ((1ull << (tt % 64)) - 1));
          for (int w = 0; w < tt / 64; ++w) r += __popcll(m[w]);
          ent[cnt[c] + r] = (tb0 + tt) * K + i % K;
        }
      }
      continue;  // W * 64 >= tile_tokens: this was the tile's only batch
    }
    if (tid < kWave) {
      for (int tt = 0; tt < nt; ++tt) {
        if (lane < K) {
          const int c = sel[tt * K + lane] - c_lo;
          if (c >= 0 && c < nCp) {
            const int r = dup[tt * K + lane];
            const int pos = cnt[c] + (r & 0xff);  // every lane reads before any lane writes
            if ((r & 0xff) == 0) cnt[c] = pos + (r >> 8);
            ent[pos] = (tb0 + tt) * K + lane;
          }
        }
      }
    }
  }
}

hipError_t launch_invidx(const Dims& d, const IndexLayout& lay, const int32_t* idx, char* ws,
                         hipStream_t s) {
  const int bg = d.B * d.Hkv;
  if (bg == 0 || d.nC == 0) return hipSuccess;
  int32_t* tc = (int32_t*)(ws + lay.tile_counts);
  const int n_parts = (d.nC + kIndexPart - 1) / kIndexPart;
  const size_t lds = sizeof(int32_t) * (d.nC < kIndexPart ? d.nC : kIndexPart);
  Timed tm(HSA_KERNEL_INVIDX, s);
  k_inv_count<<<dim3(bg * lay.n_tiles * n_parts), 256, lds, s>>>(
      idx, tc, d.L, d.Hkv, d.K, d.nC, lay.tile_tokens, lay.n_tiles, n_parts);
  const int rows = bg * d.nC;
  k_inv_colscan<<<dim3((rows + 3) / 4), 256, 0, s>>>(tc, (int32_t*)(ws + lay.offsets),
                                                     (int32_t*)(ws + lay.seg_start), d.nC,
                                                     lay.n_tiles, lay.seg, rows);
  k_inv_scan<<<dim3(bg), 1024, 0, s>>>((int32_t*)(ws + lay.offsets),
                                       (int32_t*)(ws + lay.seg_start),
                                       (int32_t*)(ws + lay.seg_chunk),
                                       (int32_t*)(ws + lay.n_seg), d.nC, lay.max_seg);
  // the bitmap path when the tile's tokens fit four words and the masks 48 KB of LDS (which
  // also keeps it to a single part)
  const int W = (lay.tile_tokens + 63) / 64;
  const size_t lds_bm = sizeof(int32_t) * ((d.nC + 1) & ~1) + sizeof(uint64_t) * (size_t)d.nC * W;
  const bool bm = n_parts == 1 && W <= 4 && W * 64 <= kScatterBatch && lds_bm <= 48 * 1024;
  k_inv_scatter<<<dim3(bg * lay.n_tiles * n_parts), kScatterThreads, bm ? lds_bm : lds, s>>>(
      idx, tc, (const int32_t*)(ws + lay.offsets), (int32_t*)(ws + lay.entries), d.L, d.Hkv,
      d.K, d.nC, lay.tile_tokens, lay.n_tiles, n_parts, bm ? W : 0);
  k_inv_order<<<dim3(bg), 1024, 0, s>>>((const int32_t*)(ws + lay.offsets),
                                        (const int32_t*)(ws + lay.seg_start),
                                        (const int32_t*)(ws + lay.seg_chunk),
                                        (const int32_t*)(ws + lay.n_seg),
                                        (const int32_t*)(ws + lay.entries),
                                        (int32_t*)(ws + lay.seg_order), d.L, d.K, d.nC, lay.seg,
                                        lay.max_seg);
  return hipGetLastError();
}

// ---- phase 1: per token ----------------------------------------------------------------

// One wave per (b, t, g) row: recompute each selected chunk's probabilities, accumulate
// dQ, the weight gradients dw_k = sum_h <dO_h, O_{t,h,k}>, the score gradients ds through
// the stick-breaking chain, and dQs.
template <typename T>
__global__ void __launch_bounds__(64) k_bwd_p1_generic(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ Kslc, const int32_t* __restrict__ idx,
    const float* __restrict__ score, const float* __restrict__ w, const T* __restrict__ dO,
    T* __restrict__ dQ, T* __restrict__ dQs, float* __restrict__ ds_out,
    float* __restrict__ dw_out, int L, int Hq, int Hkv, int D, int S, int Kt, int G, int nC,
    float sm_scale, float sel_scale, int softmax_w) {
  __shared__ float qsh[kMaxG][128];
  __shared__ float dosh[kMaxG][128];
  __shared__ float dzsh[kMaxG][kChunk];
  __shared__ float dwsh[kMaxK];
  __shared__ float dssh[kMaxK];
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;
  const int g = (int)(row % Hkv);
  const size_t bt = row / Hkv;
  const size_t b = bt / L;
  const size_t qbase = (bt * Hq + (size_t)g * G) * D;
  for (int i = lane; i < G * D; i += kWave) {
    qsh[i / D][i % D] = to_f32(Q[qbase + i]);
    dosh[i / D][i % D] = to_f32(dO[qbase + i]);
  }
  float dq[kMaxG][2];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) dq[h][0] = dq[h][1] = 0.0f;
  __syncthreads();

  const size_t kvstride = (size_t)Hkv * D;
  for (int k = 0; k < Kt; ++k) {
    const int c = idx[row * Kt + k];
    if (c < 0 || c >= nC) {
      if (lane == 0) dwsh[k] = 0.0f;
      continue;
    }
    const float wk = w[row * Kt + k];
    const size_t cbase = ((b * L + (size_t)c * S) * Hkv + g) * D;
    float z[kMaxG], da[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) z[h] = da[h] = 0.0f;
    const T* kr = K + cbase + (size_t)lane * kvstride;
    const T* vr = V + cbase + (size_t)lane * kvstride;
    for (int e = 0; e < D; e += 8) {
      float kv[8], vv[8];
      load8(kr + e, kv);
      load8(vr + e, vv);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            z[h] += qsh[h][e + i] * kv[i];
            da[h] += dosh[h][e + i] * vv[i];
          }
        }
      }
    }
    float dwk = 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float zz = z[h] * sm_scale;
        float m = fmaxf(0.0f, wave_max(zz));
        float ex = __expf(zz - m);
        float a = ex / (__expf(-m) + wave_sum(ex));
        float Dh = wave_sum(a * da[h]);
        dzsh[h][lane] = wk * a * (da[h] - Dh);
        dwk += Dh;
      }
    }
    if (lane == 0) dwsh[k] = dwk;
    __syncthreads();
    const T* kc = K + cbase;
    for (int j = 0; j < kChunk; ++j) {
      float k0 = to_f32(kc[(size_t)j * kvstride + lane]);
      float k1 = (D > 64) ? to_f32(kc[(size_t)j * kvstride + 64 + lane]) : 0.0f;
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
          float dz = dzsh[h][j];
          dq[h][0] += dz * k0;
          dq[h][1] += dz * k1;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      dQ[qbase + (size_t)h * D + lane] = from_f32<T>(dq[h][0] * sm_scale);
      if (D > 64) dQ[qbase + (size_t)h * D + 64 + lane] = from_f32<T>(dq[h][1] * sm_scale);
    }
  }
  // softmax weights: ds_k = w_k (dw_k - sum_j w_j dw_j) over the valid slots (slot order)
  if (lane == 0 && softmax_w) {
    double mean = 0.0;
    for (int k = 0; k < Kt; ++k) {
      const int c = idx[row * Kt + k];
      if (c >= 0 && c < nC) mean += (double)dwsh[k] * (double)w[row * Kt + k];
    }
    for (int k = 0; k < Kt; ++k) {
      const int c = idx[row * Kt + k];
      const bool ok = c >= 0 && c < nC;
      const double dsk = ok ? (double)w[row * Kt + k] * ((double)dwsh[k] - mean) : 0.0;
      dssh[k] = (float)dsk;
      ds_out[row * Kt + k] = (float)dsk;
      dw_out[row * Kt + k] = ok ? dwsh[k] : 0.0f;
    }
  }
  // stick-breaking chain rule over the valid prefix, newest slot first:
  // ds_k = dw_k w_k (1 - p_k) - p_k * sum_{k' > k} dw_k' w_k'
  if (lane == 0 && !softmax_w) {
    double suffix = 0.0;
    for (int k = Kt - 1; k >= 0; --k) {
      int c = idx[row * Kt + k];
      double dsk = 0.0;
      if (c >= 0 && c < nC) {
        double p = sigmoid_d((double)score[row * Kt + k]);
        double dwk = (double)dwsh[k], wk = (double)w[row * Kt + k];
        dsk = dwk * wk * (1.0 - p) - p * suffix;
        suffix += dwk * wk;
      }
      dssh[k] = (float)dsk;
      ds_out[row * Kt + k] = (float)dsk;
      dw_out[row * Kt + k] = (c >= 0 && c < nC) ? dwsh[k] : 0.0f;
    }
  }
  __syncthreads();
  const size_t qsrow = row * D;
  for (int e = lane; e < D; e += kWave) {
    float acc = 0.0f;
    for (int k = 0; k < Kt; ++k) {
      int c = idx[row * Kt + k];
      if (c < 0 || c >= nC) continue;
      acc += dssh[k] * to_f32(Kslc[((b * nC + c) * Hkv + g) * D + e]);
    }
    dQs[qsrow + e] = from_f32<T>(acc * sel_scale);
  }
}

// ---- phase 2: per chunk segment ----------------------------------------------------------

// One block of two waves per segment of a chunk's selector list.  Lane j of wave 0 keeps
// row j of the segment's partial dK in registers, lane j of wave 1 row j of dV; wave 1
// also sums the segment's partial dKslc.  Partials are reduced in segment order later.
template <typename T, int D>
__global__ void __launch_bounds__(128) k_bwd_p2_seg(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ Qs, const float* __restrict__ w, const T* __restrict__ dO,
    const float* __restrict__ ds_in, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ seg_chunk, const int32_t* __restrict__ n_seg,
    float* __restrict__ part_dk, float* __restrict__ part_dv, float* __restrict__ part_dks,
    int L, int Hq, int Hkv, int S, int Kt, int G, int nC, int seg, int64_t max_seg,
    float sm_scale, float sel_scale) {
  __shared__ float qsh[kMaxG][D];
  __shared__ float dosh[kMaxG][D];
  __shared__ float qssh[D];
  const int64_t sidx = blockIdx.x % max_seg;
  const int bg = (int)(blockIdx.x / max_seg);
  if (sidx >= n_seg[bg]) return;  // uniform for the whole block
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const int c = seg_chunk[(size_t)bg * max_seg + sidx];
  const int32_t* off = offsets + (size_t)bg * (nC + 1);
  const int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  const int e0 = off[c] + (int)(sidx - ss[c]) * seg;
  const int e1 = min(off[c + 1], e0 + seg);
  const int32_t* ent = entries + (size_t)bg * L * Kt;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const size_t kvstride = (size_t)Hkv * D;
  const size_t cbase = ((b * L + (size_t)c * S) * Hkv + g) * D;
  const T* krow = K + cbase + (size_t)lane * kvstride;  // this lane's key row
  const T* vrow = V + cbase + (size_t)lane * kvstride;  // and value row
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.0f;
  float dks0 = 0.0f, dks1 = 0.0f;

  for (int ei = e0; ei < e1; ++ei) {
    const int val = ent[ei];
    if (val < 0 || val >= L * Kt) continue;  // only an invalid selection leaves a hole here
    const int t = val / Kt;
    const int k = val % Kt;
    const size_t srow = ((b * L + t) * Hkv + g);
    const float wk = w[srow * Kt + k];
    const float dsk = ds_in[srow * Kt + k];
    const size_t qbase = ((b * L + t) * Hq + (size_t)g * G) * D;
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += 2 * kWave) {
      qsh[i / D][i % D] = to_f32(Q[qbase + i]);
      dosh[i / D][i % D] = to_f32(dO[qbase + i]);
    }
    for (int i = threadIdx.x; i < D; i += 2 * kWave) qssh[i] = to_f32(Qs[srow * D + i]);
    __syncthreads();
    float z[kMaxG], da[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) z[h] = da[h] = 0.0f;
    for (int e = 0; e < D; e += 8) {
      float kv[8], vv[8];
      load8(krow + e, kv);
      load8(vrow + e, vv);
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            z[h] += qsh[h][e + i] * kv[i];
            da[h] += dosh[h][e + i] * vv[i];
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float zz = z[h] * sm_scale;
        float m = fmaxf(0.0f, wave_max(zz));
        float ex = __expf(zz - m);
        float a = ex / (__expf(-m) + wave_sum(ex));
        if (wave == 0) {
          float Dh = wave_sum(a * da[h]);
          float dz = wk * a * (da[h] - Dh) * sm_scale;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] += dz * qsh[h][e];
        } else {
          float wa = wk * a;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] += wa * dosh[h][e];
        }
      }
    }
    if (wave == 1) {
      dks0 += dsk * qssh[lane];
      if (D > 64) dks1 += dsk * qssh[(lane + 64) % D];
    }
  }
  const size_t pbase = ((size_t)bg * max_seg + sidx);
  float* dst = (wave == 0 ? part_dk : part_dv) + (pbase * kChunk + lane) * D;
  for (int e = 0; e < D; e += 4) {
    *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
  if (wave == 1) {
    part_dks[pbase * D + lane] = dks0 * sel_scale;
    if (D > 64) part_dks[pbase * D + 64 + lane] = dks1 * sel_scale;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// One block per (b, g, chunk, group of 1024/D key rows), the incomplete tail chunk included
// (its rows get zero): dK and dV = the sums of the chunk's segment partials in segment order,
// dKslc the same over the dKslc partials; with fold, dK rows also get dKslc / S.  Each thread
// owns four features of one key row, keeps eight segments' loads in flight and sums the dKslc
// partials of its features itself, so no phase waits for another.
template <typename T>
__global__ void __launch_bounds__(256) k_bwd_p2_reduce(
    const float* __restrict__ part_dk, const float* __restrict__ part_dv,
    const float* __restrict__ part_dks, const int32_t* __restrict__ seg_start, T* __restrict__ dK,
    T* __restrict__ dV, float* __restrict__ dKslc, int L, int Hkv, int D, int S, int nC,
    int n_chunks_all, int64_t max_seg, int fold) {
  const int n_rg = D / 16;  // row groups per chunk: 64 rows / (1024 / D)
  const int rg = blockIdx.x % n_rg;
  const int c = (blockIdx.x / n_rg) % n_chunks_all;
  const int bg = blockIdx.x / (n_rg * n_chunks_all);
  const int g = bg % Hkv;
  const size_t b = bg / Hkv;
  const size_t kvstride = (size_t)Hkv * D;
  const size_t cbase = ((b * L + (size_t)c * S) * Hkv + g) * D;
  const int j = rg * (1024 / D) + threadIdx.x / (D / 4), e = 4 * (threadIdx.x % (D / 4));
  if (c >= nC) {  // incomplete tail chunk: never selectable
    if ((size_t)c * S + j < (size_t)L) {
      store4<T>(dK + cbase + j * kvstride + e, make_float4(0.f, 0.f, 0.f, 0.f));
      store4<T>(dV + cbase + j * kvstride + e, make_float4(0.f, 0.f, 0.f, 0.f));
    }
    return;
  }
  const int32_t* ss = seg_start + (size_t)bg * (nC + 1);
  const int s0 = ss[c], s1 = ss[c + 1], ns = s1 - s0;
  const size_t pb = (size_t)bg * max_seg;
  const size_t step = (size_t)kChunk * D;
  const float* pk = part_dk + ((pb + s0) * kChunk + j) * D + e;
  const float* pv = part_dv + ((pb + s0) * kChunk + j) * D + e;
  const float* ps = part_dks + (pb + s0) * D + e;
  auto add = [](float4& a, const float4& v) {
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  };
  float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak, as = ak;
  int s = 0;
  for (; s + 8 <= ns; s += 8) {  // eight segments' loads in flight, summed in segment order
    float4 k8[8], v8[8], d8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      k8[u] = *reinterpret_cast<const float4*>(pk + (size_t)(s + u) * step);
      v8[u] = *reinterpret_cast<const float4*>(pv + (size_t)(s + u) * step);
      d8[u] = *reinterpret_cast<const float4*>(ps + (size_t)(s + u) * D);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      add(ak, k8[u]);
      add(av, v8[u]);
      add(as, d8[u]);
    }
  }
  for (; s < ns; ++s) {
    add(ak, *reinterpret_cast<const float4*>(pk + (size_t)s * step));
    add(av, *reinterpret_cast<const float4*>(pv + (size_t)s * step));
    add(as, *reinterpret_cast<const float4*>(ps + (size_t)s * D));
  }
  if (j == 0 && dKslc)
    *reinterpret_cast<float4*>(dKslc + ((b * nC + c) * Hkv + g) * D + e) = as;
  if (fold) {
    ak.x += as.x / (float)S;
    ak.y += as.y / (float)S;
    ak.z += as.z / (float)S;
    ak.w += as.w / (float)S;
  }
  store4<T>(dK + cbase + j * kvstride + e, ak);
  store4<T>(dV + cbase + j * kvstride + e, av);
}

template <typename T>
static void launch_p1_generic(const Dims& d, const BwdLayout& lay, const void* Q, const void* K,
                              const void* V, const void* Kslc, const int32_t* idx,
                              const float* score, const float* w, const void* dO, void* dQ,
                              void* dQs, char* ws, hipStream_t s) {
  const size_t rows = (size_t)d.B * d.L * d.Hkv;
  Timed tm(HSA_KERNEL_BWD_P1, s);
  k_bwd_p1_generic<T><<<dim3((unsigned)rows), 64, 0, s>>>(
      (const T*)Q, (const T*)K, (const T*)V, (const T*)Kslc, idx, score, w, (const T*)dO,
      (T*)dQ, (T*)dQs, (float*)(ws + lay.ds), (float*)(ws + lay.dw), d.L, d.Hq, d.Hkv, d.D, d.S,
      d.K, d.G, d.nC, (float)d.sm_scale, (float)d.sel_scale, softmax_w(d));
}

template <typename T>
static void launch_p2_generic(const Dims& d, const BwdLayout& lay, const void* Q, const void* K,
                              const void* V, const void* Qs, const float* w, const void* dO,
                              char* ws, hipStream_t s) {
  const int bg = d.B * d.Hkv;
  const float sm = (float)d.sm_scale, sel = (float)d.sel_scale;
  dim3 grid((unsigned)(bg * lay.max_seg));
  auto args = [&](auto kern) {
    Timed tm(HSA_KERNEL_BWD_P2, s);
    kern<<<grid, 128, 0, s>>>((const T*)Q, (const T*)K, (const T*)V, (const T*)Qs, w,
                              (const T*)dO, (const float*)(ws + lay.ds),
                              (const int32_t*)(ws + lay.offsets),
                              (const int32_t*)(ws + lay.entries),
                              (const int32_t*)(ws + lay.seg_start),
                              (const int32_t*)(ws + lay.seg_chunk),
                              (const int32_t*)(ws + lay.n_seg), (float*)(ws + lay.part_dk),
                              (float*)(ws + lay.part_dv), (float*)(ws + lay.part_dks), d.L, d.Hq,
                              d.Hkv, d.S, d.K, d.G, d.nC, lay.seg, lay.max_seg, sm, sel);
  };
  if (d.D == 64)
    args(k_bwd_p2_seg<T, 64>);
  else
    args(k_bwd_p2_seg<T, 128>);
}

hipError_t launch_bwd_generic_p2(const Dims& d, const BwdLayout& lay, const void* Q,
                                 const void* K, const void* V, const void* Qs, const float* w,
                                 const void* dO, char* ws, hipStream_t s) {
  if (d.nC == 0) return hipSuccess;
  if (d.dtype == 1)
    launch_p2_generic<bf16>(d, lay, Q, K, V, Qs, w, dO, ws, s);
  else
    launch_p2_generic<float>(d, lay, Q, K, V, Qs, w, dO, ws, s);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const Dims& d, const BwdLayout& lay, void* dK, void* dV,
                             float* dKslc, bool fold, char* ws, hipStream_t s) {
  const int bg = d.B * d.Hkv;
  const int n_all = (d.L + d.S - 1) / d.S;
  auto go = [&](auto kern, auto* dk, auto* dv) {
    Timed tm(HSA_KERNEL_BWD_REDUCE, s);
    kern<<<dim3((unsigned)(bg * n_all * (d.D / 16))), 256, 0, s>>>(
        (const float*)(ws + lay.part_dk), (const float*)(ws + lay.part_dv),
        (const float*)(ws + lay.part_dks), (const int32_t*)(ws + lay.seg_start), dk, dv, dKslc,
        d.L, d.Hkv, d.D, d.S, d.nC, n_all, lay.max_seg, fold ? 1 : 0);
  };
  if (d.dtype == 1)
    go(k_bwd_p2_reduce<bf16>, (bf16*)dK, (bf16*)dV);
  else
    go(k_bwd_p2_reduce<float>, (float*)dK, (float*)dV);
  return hipGetLastError();
}

hipError_t launch_bwd_generic(const Dims& d, const BwdLayout& lay, const void* Q, const void* K,
                              const void* V, const void* Qs, const void* Kslc,
                              const int32_t* idx, const float* score, const float* w,
                              const void* dO, void* dQ, void* dK, void* dV, void* dQs,
                              float* dKslc, bool fold, char* ws, hipStream_t s) {
  hipError_t e = launch_invidx(d, lay, idx, ws, s);
  if (e != hipSuccess) return e;
  if (d.dtype == 1)
    launch_p1_generic<bf16>(d, lay, Q, K, V, Kslc, idx, score, w, dO, dQ, dQs, ws, s);
  else
    launch_p1_generic<float>(d, lay, Q, K, V, Kslc, idx, score, w, dO, dQ, dQs, ws, s);
  e = launch_bwd_generic_p2(d, lay, Q, K, V, Qs, w, dO, ws, s);
  if (e != hipSuccess) return e;
  return launch_bwd_reduce(d, lay, dK, dV, dKslc, fold, ws, s);
}

}  // namespace hsa
