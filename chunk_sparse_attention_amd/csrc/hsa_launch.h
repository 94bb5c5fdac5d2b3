// hsa_launch.h -- host-side launchers behind the C ABI (internal to libhsa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hsa.h"

namespace hsa {

// Brackets the launches made during its lifetime with HIP events when kernel timing is on
// (kc is an hsa_kernel_t class); does nothing otherwise.
class Timed {
 public:
  Timed(int kc, hipStream_t s);
  ~Timed();
  Timed(const Timed&) = delete;
  Timed& operator=(const Timed&) = delete;

 private:
  int kc_, slot_;
  hipStream_t s_;
};

// Validated problem, with derived sizes and the scales resolved in double.
struct Dims {
  int B, L, Hq, Hkv, D, S, K;
  int nC;  // complete chunks floor(L/S)
  int G;   // query heads per group
  double sm_scale, sel_scale;
  int dtype;  // 0 fp32, 1 bf16
  unsigned flags;
};

// The chunk -> (token, slot) inverse index: per (b, g), entries grouped by chunk and cut into
// segments of `seg` entries (byte offsets into a workspace).
struct IndexLayout {
  int tile_tokens;  // tokens per tile of the index build
  int n_tiles;      // tiles per (b, g)
  int seg;          // entries per segment
  int64_t max_seg;  // segment capacity per (b, g)
  size_t tile_counts, offsets, entries, seg_start, seg_chunk, n_seg;
  // the segments of each (b, g) in the order the chunk-major kernels take them: by the token
  // of their first entry, so that the blocks in flight gather the rows of nearby tokens
  size_t seg_order;
};
// Entries per chunk segment of the chunk-major kernels (two waves of 16-row jobs).
constexpr int kBwdSeg = 256;
// Lays the index out from byte offset o (advanced past it).
IndexLayout index_layout(const Dims& d, size_t& o);

// State the forward leaves at the start of its workspace for a backward over the same
// selection: per (token, group, slot, head) the softmax-off-by-one normaliser in the log2
// domain, and either (chunk-major forward) the inverse index and the per-edge partials'
// buffer, or (token-tile forward) the tiles' job lists and the key rows in MFMA operand
// order.  The backward's workspace starts with the same regions.
struct FwdState {
  size_t lse;
  IndexLayout ix;      // chunk-major forward
  size_t part;         // chunk-major forward: per-edge bf16 partials, G*D per (t, g, slot)
  size_t prep, kop;    // token-tile forward
  size_t total;
};
FwdState fwd_state(const Dims& d);

// Backward workspace carve-up (byte offsets into the caller's workspace).
struct BwdLayout : IndexLayout {
  size_t ds, dw, part_dk, part_dv, part_dks, lse, dq_part, total;
};
BwdLayout bwd_layout(const Dims& d);

// Decode workspace: per (b, g) the candidate keys of every scan block.
struct DecLayout {
  int chunks_per_block;
  int n_blocks;  // scan blocks per (b, g)
  size_t cand, total;
};
DecLayout dec_layout(const Dims& d);

// 1 when the chunk weights are the softmax of the selected scores (HSA_FLAG_SOFTMAX_WEIGHTS).
inline int softmax_w(const Dims& d) { return (d.flags & HSA_FLAG_SOFTMAX_WEIGHTS) ? 1 : 0; }
// Rewrites w of every (token, group) row as the softmax of its valid slots' scores.
hipError_t launch_softmax_weights(const Dims& d, const int32_t* idx, const float* score,
                                  float* w, hipStream_t s);

// F1 pooling (both dtypes).
hipError_t launch_pool(const Dims& d, const void* K, void* Kslc, hipStream_t s);
// Pooling of listed chunks only: chunk_ids [B, n_ids] (device); entries outside [0, nC) skip.
hipError_t launch_pool_chunks(const Dims& d, const void* K, void* Kslc, const int32_t* chunk_ids,
                              int n_ids, hipStream_t s);

// Generic vector-ALU kernels (fp32 and bf16).
hipError_t launch_select_generic(const Dims& d, const void* Qs, const void* Kslc, int32_t* idx,
                                 float* score, float* w, hipStream_t s);
// lse (optional, [B, L, Hq, K], natural log, 0 for masked slots): the normalisers.
hipError_t launch_fwd_generic(const Dims& d, const void* Q, const void* K, const void* V,
                              const int32_t* idx, const float* w, void* O, float* lse,
                              hipStream_t s);
// The forward state's normalisers (log2 domain, [B, L, Hkv, K, G]) to the ABI's lse
// ([B, L, Hq, K], natural log, 0 for masked slots) and back.
hipError_t launch_lse_export(const Dims& d, const float* state, const int32_t* idx, float* lse,
                             hipStream_t s);
hipError_t launch_lse_import(const Dims& d, const float* lse, float* state, hipStream_t s);
hipError_t launch_invidx(const Dims& d, const IndexLayout& lay, const int32_t* idx, char* ws,
                         hipStream_t s);
hipError_t launch_bwd_generic(const Dims& d, const BwdLayout& lay, const void* Q, const void* K,
                              const void* V, const void* Qs, const void* Kslc,
                              const int32_t* idx, const float* score, const float* w,
                              const void* dO, void* dQ, void* dK, void* dV, void* dQs,
                              float* dKslc, bool fold, char* ws, hipStream_t s);
hipError_t launch_bwd_generic_p2(const Dims& d, const BwdLayout& lay, const void* Q,
                                 const void* K, const void* V, const void* Qs, const float* w,
                                 const void* dO, char* ws, hipStream_t s);
hipError_t launch_bwd_reduce(const Dims& d, const BwdLayout& lay, void* dK, void* dV,
                             float* dKslc, bool fold, char* ws, hipStream_t s);

// Tiled selection (exact fp64 scores, any dtype).
bool select_tile_supported(const Dims& d);
hipError_t launch_select_tile(const Dims& d, const void* Qs, const void* Kslc, int32_t* idx,
                              float* score, float* w, hipStream_t s);

// Selection for bf16: matrix-core candidate filter, exact rescoring (same results).
bool select_mfma_supported(const Dims& d);
hipError_t launch_select_mfma(const Dims& d, const void* Qs, const void* Kslc, int32_t* idx,
                              float* score, float* w, hipStream_t s);

// Matrix-core (MFMA) kernels for bf16.
// Per-chunk operand copies for the matrix-core kernels (layouts in fwd_mfma.hip):
// trans = false: key rows in A-operand order; trans = true: transposed, P.V key order.
void launch_prep_ops(const Dims& d, const void* src, void* dst, bool trans, hipStream_t s);
size_t chunk_ops_bytes(const Dims& d);
// Token tiles of the matrix-core kernels: tokens per tile, and the prepared job lists.
int tile_tokens(const Dims& d);
size_t tile_prep_bytes(const Dims& d);
void launch_tile_prep(const Dims& d, const int32_t* idx, void* prep, hipStream_t s);
// On the matrix cores the chunk phase also yields per-edge dQ partials, which a token phase
// sums.
bool bwd_mfma_supported(const Dims& d);
// after_fwd: ws still holds the forward's state for this problem, Q, K, idx and w (see
// FwdState): its index and normalisers are reused.  lse (optional, the ABI layout): the
// normalisers to use, copied into the state first.
hipError_t launch_bwd_mfma(const Dims& d, const BwdLayout& lay, const void* Q, const void* K,
                           const void* V, const void* Qs, const void* Kslc, const int32_t* idx,
                           const float* score, const float* w, const float* lse,
                           const void* dO, void* dQ, void* dK, void* dV, void* dQs,
                           float* dKslc, bool fold, bool after_fwd, char* ws, hipStream_t s);
bool fwd_mfma_supported(const Dims& d);
// bf16 up to 16384 chunks: the forward runs chunk-major (inverse index, per-edge partials,
// token sums); beyond, on token tiles (G >= 4; fwd_mfma_supported is false there for G < 4).
bool fwd_chunked(const Dims& d);
size_t fwd_mfma_ws(const Dims& d);
// index_ready: ws already holds the inverse index (or the token tiles' job lists) of this
// selection, built by the previous call on the same workspace and idx.
hipError_t launch_fwd_mfma(const Dims& d, const void* Q, const void* K, const void* V,
                           const int32_t* idx, const float* w, void* O, char* ws, hipStream_t s,
                           bool index_ready = false);

// Decode with a bandwidth-shaped scan and one wave per kept slot (both dtypes).
size_t dec_fast_ws(const Dims& d);
// host_kv: Kc and Vc are the device's view of page-locked host memory.  ctx_lens (device,
// [B], or NULL): sequence b may select only chunks below ctx_lens[b] / S.
hipError_t launch_decode_fast(const Dims& d, const void* q, const void* qs, const void* Kc,
                              const void* Vc, const void* Kslc, void* O, int32_t* idx,
                              float* score, float* w, bool host_kv, const int32_t* ctx_lens,
                              char* ws, hipStream_t s);
// n_layers layers attending with one given selection (idx/w [B, Hkv, K]); q, O
// [n_layers, B, Hq, D], caches [n_layers, B, L, Hkv, D] (host_kv: the device's view of
// page-locked host memory).
hipError_t launch_decode_shared(const Dims& d, int n_layers, const void* q, const void* Kc,
                                const void* Vc, const int32_t* sel_idx, const float* sel_w,
                                void* O, bool host_kv, hipStream_t s);
hipError_t launch_decode_generic(const Dims& d, const DecLayout& lay, const void* q,
                                 const void* qs, const void* Kc, const void* Vc,
                                 const void* Kslc, void* O, int32_t* idx, float* score,
                                 float* w, const int32_t* ctx_lens, char* ws, hipStream_t s);

}  // namespace hsa
