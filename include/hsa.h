/*
 * hsa.h -- C ABI of libhsa.so, Hierarchical Sparse Attention (HSA) on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (from "Hardware-aligned Hierarchical Sparse Attention for Efficient
 * Long-term Memory Access", papernotes.org note, section 方法详解 › 层次化稀疏注意力（HSA）,
 * and the atlas.scime.ai summary of the same paper, section "Approach"):
 *   1. Chunk selection: the sequence is cut into chunks of S tokens; every chunk is keyed by
 *      the mean of its key rows; every token scores each earlier chunk with its own selection
 *      query and keeps the top-K chunks, separately for each query group (KV head).
 *   2. Token level: inside each selected chunk, ordinary attention of the token's query over
 *      the chunk's S keys, normalised with softmax-off-by-one (note section 硬件对齐 Kernel).
 *   3. Chunk level: the K per-chunk outputs are fused with stick-breaking weights computed
 *      from the sigmoid of the selection scores, with no positional term.
 *   The backward runs in two phases (note section 硬件对齐 Kernel): per token the query and
 *   chunk-weight gradients, then per chunk the key and value gradients over every token that
 *   selected it.  The gradient also flows through the weights into the selection scores.
 *   Decode (note section 训练与推理优化, KV Cache Offloading): one new token per sequence is
 *   scored against the resident chunk-key table and reads only the selected chunks' K/V.
 *
 * Definitions used where the pages are silent (the numbers refer to no page):
 *   nC        = floor(L / S) complete chunks; a trailing partial chunk is never selectable.
 *   Kslc      [b,c,g,:] = mean_{j<S} K[b, c*S+j, g, :], summed in fp64 in row order and
 *             rounded once (nearest, ties to even) to the storage dtype.
 *   score     s = sel_scale * <Qs[b,t,g,:], Kslc[b,c,g,:]>, for c < min(floor(t/S), nC),
 *             taken in fp32; NaN counts as -inf.
 *   ranking   score descending, ties to the lower chunk index; slots past the number of
 *             candidates are masked: idx -1, score -inf, w 0.
 *   weights   w_k = sigmoid(s_k) * prod_{j<k} (1 - sigmoid(s_j)) over the valid slots.
 *   attention z_j = sm_scale * <Q[b,t,h,:], K[b,c*S+j,g,:]>,
 *             a_j = exp(z_j) / (1 + sum_i exp(z_i)), O_{t,h,k} = sum_j a_j V[b,c*S+j,g,:],
 *             O[b,t,h,:] = sum_k w_k O_{t,h,k} (0 when no slot is valid).
 *   groups    query head h belongs to KV group g = floor(h / (Hq/Hkv)).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers to dense row-major arrays in the layouts given
 *     below ("BSHD": [batch, token, head, dim]), 16-byte aligned.  Inputs are read only.
 *   - The caller owns all memory.  The library never allocates, frees or synchronises;
 *     scratch memory comes from the caller's workspace `ws` of at least
 *     hsa_workspace_size() bytes (256-byte aligned; may be NULL when that size is 0).
 *   - Outputs are fully overwritten, never accumulated.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without waiting.  Asynchronous faults surface at the caller's next sync.
 *   - Arguments are validated before anything is enqueued; on a nonzero status nothing was
 *     launched and nothing was written.  hsa_last_error() then describes the problem.
 *   - Calls are reentrant; concurrent calls must use distinct workspaces.
 *
 * Supported envelope: S = 64; D in {64, 128}; 1 <= K <= 16; Hq % Hkv == 0 with
 * 1 <= Hq/Hkv <= 16; dtype fp32 or bf16; L*K < 2^31; hsa_bwd at most 32767 chunks (L/S).
 * Anything else returns HSA_ERR_UNSUPPORTED.
 */
#ifndef HSA_H_
#define HSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSA_OK = 0,
  HSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, bad scale */
  HSA_ERR_UNSUPPORTED = 2, /* outside the supported envelope above */
  HSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than hsa_workspace_size() */
  HSA_ERR_HIP = 4          /* a HIP launch failed; see hsa_last_error() */
} hsa_status_t;

typedef enum { HSA_F32 = 0, HSA_BF16 = 1 } hsa_dtype_t;

typedef enum { HSA_OP_SELECT = 0, HSA_OP_FWD = 1, HSA_OP_BWD = 2, HSA_OP_DECODE = 3 } hsa_op_t;

/* hsa_problem_t.flags */
#define HSA_FLAG_GENERIC 0x1u /* use the plain vector-ALU kernels even where MFMA kernels exist */
/* Chunk weights as a softmax of the valid slots' selection scores instead of stick-breaking
 * (the variant of the pages' weights ablation: atlas summary, measured effects; note
 * section 亮点): hsa_select and hsa_decode write them, hsa_bwd differentiates them
 * (ds_k = w_k (dw_k - sum_j w_j dw_j)); hsa_fwd takes whatever w it is given.  Give the same
 * flag to the select and the backward of one step. */
#define HSA_FLAG_SOFTMAX_WEIGHTS 0x2u

/* hsa_bwd flags */
#define HSA_BWD_FOLD_KSLC 0x1u /* add dKslc/S into every key row of the chunk (Kslc = mean K) */
#define HSA_BWD_AFTER_FWD 0x2u /* reuse what hsa_fwd left in ws for this problem, Q, K, idx
                                  and w, when the library can confirm it (see hsa_bwd) */

typedef struct hsa_problem {
  int32_t B;        /* batch (decode: number of sequences) */
  int32_t L;        /* tokens per sequence (decode: context length already cached) */
  int32_t Hq;       /* query heads */
  int32_t Hkv;      /* KV heads = query groups */
  int32_t D;        /* head dimension */
  int32_t S;        /* chunk size */
  int32_t K;        /* chunks kept per (token, group) */
  float sm_scale;   /* token-level logit scale; 0 => 1/sqrt(D) (taken in double) */
  float sel_scale;  /* selection score scale; 0 => 1/sqrt(D) (taken in double) */
  int32_t dtype;    /* hsa_dtype_t of Q, K, V, Qs, Kslc, dO and of O and the gradients */
  uint32_t flags;   /* HSA_FLAG_* */
} hsa_problem_t;

typedef void* hsa_stream_t; /* hipStream_t */

/* Human-readable name of a status code (static string). */
const char* hsa_status_string(hsa_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* hsa_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* hsa_version(void);

/* Workspace bytes the entry point `op` (hsa_op_t) needs for problem *p.  Writes *bytes;
 * returns the same validation status the entry point itself would. */
hsa_status_t hsa_workspace_size(int op, const hsa_problem_t* p, size_t* bytes);

/* Chunk-key pooling and top-K selection with stick-breaking weights
 * (note section 层次化稀疏注意力（HSA）: Chunk Selection and 第二阶段).
 *   Qs    [B, L, Hkv, D] dtype  selection queries; NULL => pool only
 *   K     [B, L, Hkv, D] dtype  keys
 *   Kslc  [B, nC, Hkv, D] dtype out: chunk keys (mean of each chunk's key rows)
 *   idx   [B, L, Hkv, K] int32 out: selected chunks in rank order, -1 = masked
 *   score [B, L, Hkv, K] fp32  out: their scores, -inf = masked
 *   w     [B, L, Hkv, K] fp32  out: stick-breaking weights (softmax weights with
 *                                 HSA_FLAG_SOFTMAX_WEIGHTS), 0 = masked
 * With Qs == NULL only Kslc is written and idx/score/w may be NULL (used to build the
 * resident chunk table for decode); otherwise all must be non-NULL. */
hsa_status_t hsa_select(const hsa_problem_t* p, const void* Qs, const void* K, void* Kslc,
                        int32_t* idx, float* score, float* w, void* ws, size_t ws_bytes,
                        hsa_stream_t stream);

/* Token-level softmax-off-by-one attention inside the selected chunks, fused with the
 * chunk weights (note sections 层次化稀疏注意力（HSA） 第一阶段/第二阶段 and 硬件对齐 Kernel).
 *   Q   [B, L, Hq, D] dtype;  K, V [B, L, Hkv, D] dtype
 *   idx [B, L, Hkv, K] int32 and w [B, L, Hkv, K] fp32 as written by hsa_select (any valid
 *       selection works: valid slots first, each chunk < min(floor(t/S), nC), -1 after, the
 *       chunks of one row distinct).  A slot whose chunk is negative or not below nC adds
 *       nothing.  A row that repeats a chunk is outside that contract; up to 16384 chunks
 *       each repeated slot still adds its own term (as hsa_bwd differentiates it), beyond
 *       (the token-tile kernels) only one of a row's equal slots adds its term.
 *   O   [B, L, Hq, D] dtype out
 *   lse [B, L, Hq, K] fp32 out, optional (NULL: not written): the softmax-off-by-one
 *       normaliser of every (token, head, slot), lse = log(1 + sum_j exp(z_j)) in the natural
 *       log, with z_j the slot's S logits; 0 for a masked slot.  hsa_bwd can take it back.
 * The forward also leaves state in ws that a backward over the same problem, Q, K, idx and
 * w can reuse (HSA_BWD_AFTER_FWD). */
hsa_status_t hsa_fwd(const hsa_problem_t* p, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* w, void* O, float* lse, void* ws,
                     size_t ws_bytes, hsa_stream_t stream);

/* Backward of hsa_select's scores/weights and hsa_fwd with the selection held fixed
 * (note section 硬件对齐 Kernel: two phases; section 层次化稀疏注意力（HSA）: end-to-end
 * gradients through the chunk weights).  Inputs as in hsa_select / hsa_fwd plus
 *   Kslc [B, nC, Hkv, D] dtype (the chunk keys the scores were computed from)
 *   lse  [B, L, Hq, K] fp32, optional: the normalisers hsa_fwd wrote for this problem, Q, K
 *        and idx; NULL => recomputed (from the workspace state under HSA_BWD_AFTER_FWD, see
 *        below, else from Q and K).  The plain vector-ALU kernels (fp32, HSA_FLAG_GENERIC, or
 *        shapes outside the matrix-core kernels) always recompute it.
 *   dO   [B, L, Hq, D] dtype  upstream gradient of O
 * Outputs (all fully written):
 *   dQ [B, L, Hq, D], dK, dV, dQs [B, L, Hkv, D] dtype
 *   dKslc [B, nC, Hkv, D] fp32, gradient with respect to Kslc (may be NULL)
 * flags: HSA_BWD_FOLD_KSLC adds dKslc[c]/S to dK of every row of chunk c, which is the
 * complete key gradient when Kslc was pooled from K.
 * HSA_BWD_AFTER_FWD asks to reuse the state the last hsa_fwd (or hsa_fwd_layers, for its last
 * layer) left in this same workspace (sized for hsa_bwd, which is at least the forward's
 * size): the chunk -> (token, slot) inverse index, or the token tiles' job lists, and every
 * softmax normaliser.  The library keeps, per workspace pointer and device, a record of the
 * forward that last filled it (problem, Q, K, idx, w); the state is reused only when that
 * record matches this call and no other entry point has used the workspace since (hsa_bwd
 * calls that reused it leave it intact).  Otherwise the backward rebuilds what it needs, so
 * the flag never changes the result beyond fp32 rounding.  The record cannot see the
 * contents: the caller must not change Q, K, idx, w or the workspace bytes in between. */
hsa_status_t hsa_bwd(const hsa_problem_t* p, const void* Q, const void* K, const void* V,
                     const void* Qs, const void* Kslc, const int32_t* idx, const float* score,
                     const float* w, const float* lse, const void* dO, void* dQ, void* dK,
                     void* dV, void* dQs, float* dKslc, uint32_t flags, void* ws,
                     size_t ws_bytes, hsa_stream_t stream);

/* One decode step for B sequences with L = ctx tokens already cached (note section
 * 训练与推理优化: only the chunk-key table is scanned; only the selected chunks' K/V are read).
 * The new token sits at position ctx and may select chunks c < floor(ctx/S).
 *   q  [B, Hq, D] dtype;  qs [B, Hkv, D] dtype
 *   Kcache, Vcache [B, ctx, Hkv, D] dtype;  Kslc [B, floor(ctx/S), Hkv, D] dtype
 *   O  [B, Hq, D] dtype out;  idx [B, Hkv, K] int32 out;  w [B, Hkv, K] fp32 out;
 *   score [B, Hkv, K] fp32 out (may be NULL) */
hsa_status_t hsa_decode(const hsa_problem_t* p, const void* q, const void* qs,
                        const void* Kcache, const void* Vcache, const void* Kslc, void* O,
                        int32_t* idx, float* score, float* w, void* ws, size_t ws_bytes,
                        hsa_stream_t stream);

/* hsa_decode for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments, results and errors without
 * `ws`.  Its scratch (the scan blocks' candidate keys, 8 * B * Hkv * ceil(ctx/(64*1024)) * K
 * bytes on the default kernels) lives in a device array of 4 MiB inside the library, one
 * copy per device, held until the process ends; a
 * problem that needs more returns HSA_ERR_UNSUPPORTED before anything is enqueued.  The call
 * allocates nothing and frees nothing.  Every call on one device uses that device's copy,
 * and each call rewrites all of the scratch it reads, so successive calls need no clearing;
 * calls that overlap in time on one device (other streams, other threads) race on it and
 * must be ordered by the caller. */
hsa_status_t hsa_decode_noalloc(const hsa_problem_t* p, const void* q, const void* qs,
                                const void* Kcache, const void* Vcache, const void* Kslc,
                                void* O, int32_t* idx, float* score, float* w,
                                hsa_stream_t stream);

/* One decode step with the token K/V cache left in host memory (note section 训练与推理优化,
 * KV cache offloading: the chunk-key table stays on the device for selection and each step
 * moves only the selected chunks; 局限与展望: that exchange is g x dh x K x S values per
 * sequence and group).  Arguments, results and errors are those of hsa_decode, except:
 *   Kcache, Vcache [B, ctx, Hkv, D] dtype: page-locked host memory mapped for the device
 *   (hipHostMalloc, or a pinned torch tensor), owned by the caller and read in place: the
 *   step reads the K selected chunks' 64 rows of K and V per (sequence, group) across the
 *   host link and nothing else of them.  q, qs, Kslc, O, idx, score, w and ws are device
 *   memory as for hsa_decode.
 * Each cache pointer is checked with hipPointerGetAttributes before anything is enqueued:
 * memory that is not host memory mapped for the device (pageable host memory, or device
 * memory, which hsa_decode takes) gives HSA_ERR_INVALID_ARG. */
hsa_status_t hsa_decode_host_kv(const hsa_problem_t* p, const void* q, const void* qs,
                                const void* Kcache, const void* Vcache, const void* Kslc,
                                void* O, int32_t* idx, float* score, float* w, void* ws,
                                size_t ws_bytes, hsa_stream_t stream);

/* One decode step for B sequences of different lengths in one cache (note section
 * 训练与推理优化: decode scans the chunk-key table and reads only the selected chunks).
 * p->L is the cache capacity: Kcache, Vcache [B, L, Hkv, D], Kslc [B, floor(L/S), Hkv, D],
 * as for hsa_decode.  ctx_lens [B] int32 (device memory): sequence b's new token sits at
 * position ctx_lens[b] and may select chunks c < min(floor(ctx_lens[b]/S), floor(L/S))
 * (values below 0 count as 0), so its result equals hsa_decode's on that sequence's first
 * ctx_lens[b] tokens.  Other arguments, results and errors as for hsa_decode. */
hsa_status_t hsa_decode_ragged(const hsa_problem_t* p, const int32_t* ctx_lens, const void* q,
                               const void* qs, const void* Kcache, const void* Vcache,
                               const void* Kslc, void* O, int32_t* idx, float* score, float* w,
                               void* ws, size_t ws_bytes, hsa_stream_t stream);

/* Chunk keys of listed chunks only, for a decoder that appends the chunk its sequence has
 * just completed (note section 训练与推理优化: the chunk-key table stays resident and grows by
 * one chunk every S tokens).  p->L is the cache capacity; K [B, L, Hkv, D] dtype.
 * chunk_ids [B, n_ids] int32 (device memory): for every entry c with 0 <= c < floor(L/S),
 * Kslc[b, c] is recomputed from rows cS .. cS+S-1 of sequence b, with the same arithmetic
 * as hsa_select's pooling (so the result equals a full pooling bit for bit); other entries
 * (e.g. -1) are skipped.  1 <= n_ids <= max(floor(L/S), 1), else HSA_ERR_INVALID_ARG. */
hsa_status_t hsa_pool_chunks(const hsa_problem_t* p, const void* K, void* Kslc,
                             const int32_t* chunk_ids, int n_ids, hsa_stream_t stream);

/* ---- Layers that share one selection ------------------------------------------------
 * The pages' model shares the chunk selection across its HSA layers (atlas summary,
 * measured effects: removing that sharing slows offloaded decoding): the selection is made
 * once and the layers attend with it.  Both calls take a stack of n_layers layers in one
 * contiguous tensor per operand, layer-major.
 *
 * hsa_fwd for each layer: Q, O [n_layers, B, L, Hq, D], K, V [n_layers, B, L, Hkv, D], one
 * idx/w [B, L, Hkv, K] for all layers (as for hsa_fwd).  The inverse index (or the token
 * tiles' job lists) is built once for the stack.  ws as for hsa_fwd with the same problem
 * (the layers run one after the other on it); afterwards it holds the last layer's forward
 * state, so HSA_BWD_AFTER_FWD applies to a backward of the last layer only.  n_layers >= 1. */
hsa_status_t hsa_fwd_layers(const hsa_problem_t* p, int n_layers, const void* Q, const void* K,
                            const void* V, const int32_t* idx, const float* w, void* O,
                            void* ws, size_t ws_bytes, hsa_stream_t stream);

/* Decode attention of a stack of layers with a selection made before (by hsa_decode,
 * hsa_decode_ragged or hsa_decode_host_kv for one layer): nothing is scanned.
 *   q [n_layers, B, Hq, D];  Kcache, Vcache [n_layers, B, L, Hkv, D] (L = context length);
 *   idx [B, Hkv, K] int32, w [B, Hkv, K] fp32 as those calls write them (a slot whose
 *   index is -1, or not below floor(L/S), adds nothing);  O [n_layers, B, Hq, D] out.
 * All device memory; one launch covers the stack.  1 <= n_layers <= 65535. */
hsa_status_t hsa_decode_shared(const hsa_problem_t* p, int n_layers, const void* q,
                               const void* Kcache, const void* Vcache, const int32_t* idx,
                               const float* w, void* O, hsa_stream_t stream);

/* hsa_decode_shared with the layers' token K/V caches in page-locked host memory (as for
 * hsa_decode_host_kv: each cache pointer is checked with hipPointerGetAttributes first, and
 * memory that is not host memory mapped for the device gives HSA_ERR_INVALID_ARG); only the
 * selected chunks' rows cross the host link, once per layer and eight heads. */
hsa_status_t hsa_decode_shared_host_kv(const hsa_problem_t* p, int n_layers, const void* q,
                                       const void* Kcache, const void* Vcache,
                                       const int32_t* idx, const float* w, void* O,
                                       hsa_stream_t stream);

/* ---- Kernel timing (measurement aid; not part of the operation) ----------------------
 * The entry points above each enqueue a short sequence of kernels.  To price one kernel
 * against the device's roofline, the library can bracket every launch of a kernel class
 * with a pair of HIP events recorded on that launch's stream.  Timing is off by default;
 * when on, each recorded launch adds two event records to its stream and a little host
 * work, and up to 4096 launches per class are recorded (later ones are not).  The state is
 * process-wide and shared by all threads and devices; events come from the current device
 * of the first launch that needs them, so time one device per enable. */
typedef enum {
  HSA_KERNEL_POOL = 0,       /* chunk-key mean pooling */
  HSA_KERNEL_SELECT = 1,     /* scoring, top-K and stick-breaking weights */
  HSA_KERNEL_TILE_PREP = 2,  /* per-token-tile job lists of the matrix-core kernels */
  HSA_KERNEL_PREP_OPS = 3,   /* per-chunk operand copies of the matrix-core kernels */
  HSA_KERNEL_FWD = 4,        /* token-level attention fused with the chunk weights */
  HSA_KERNEL_INVIDX = 5,     /* chunk -> (token, slot) inverse index (count, scan, scatter) */
  HSA_KERNEL_BWD_P1 = 6,     /* backward, token phase: per token dQ, ds, dQs (matrix-core
                                path: the sum of the chunk phase's per-edge dQ partials, then
                                the dKslc partials per segment; plain kernels: one wave per
                                token row that also forms dw) */
  HSA_KERNEL_BWD_P2 = 7,     /* backward, chunk phase: per chunk segment dK, dV partials
                                (matrix-core path: also the per-edge dQ partials and dw; runs
                                first) */
  HSA_KERNEL_BWD_REDUCE = 8, /* backward: fixed-order reduction of the segment partials */
  HSA_KERNEL_DECODE_SCAN = 9,    /* decode: scan of the chunk-key table, per-block top-K */
  HSA_KERNEL_DECODE_ATTEND = 10, /* decode: merge, weights and attention over the kept chunks */
  HSA_KERNEL_FWD_TOKEN = 11, /* chunk-major forward (bf16, up to 16384 chunks): per token sum
                                of the edges' weighted outputs */
  HSA_KERNEL_COUNT = 12
} hsa_kernel_t;

/* enable != 0: forget earlier records and start recording; enable == 0: stop recording
 * (records are kept for hsa_timer_read).  Always returns HSA_OK. */
hsa_status_t hsa_timer_enable(int enable);

/* Number of recorded launches of class `kernel` (hsa_kernel_t) since the last enable and
 * the sum of their durations in milliseconds.  Waits for the recorded events to complete
 * (the one call of this library that synchronises).  HSA_ERR_INVALID_ARG for an unknown
 * class or NULL outputs; HSA_ERR_HIP if an event cannot be read. */
hsa_status_t hsa_timer_read(int kernel, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* HSA_H_ */
