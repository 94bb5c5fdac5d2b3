// hsa_api.hip -- the C ABI of libhsa.so: validation, workspace sizing and dispatch.
//
// Every entry point validates its arguments before enqueuing anything; on failure it
// returns a status, records a message for hsa_last_error(), launches nothing and writes
// nothing.  The library never allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "hsa.h"
#include "hsa_common.h"
#include "hsa_launch.h"

#define HSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

hsa_status_t fail(hsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hsa_status_t ok() {
  g_last_error.clear();
  return HSA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Common shape checks.  `op` decides which limits apply.
hsa_status_t check_problem(int op, const hsa_problem_t* p, hsa::Dims* d) {
  if (!p) return fail(HSA_ERR_INVALID_ARG, "problem pointer is NULL");
  if (op < HSA_OP_SELECT || op > HSA_OP_DECODE)
    return fail(HSA_ERR_INVALID_ARG, "unknown op %d", op);
  if (p->B < 1 || p->L < 1 || p->Hq < 1 || p->Hkv < 1 || p->D < 1 || p->S < 1 || p->K < 1)
    return fail(HSA_ERR_INVALID_ARG, "sizes must be positive (B=%d L=%d Hq=%d Hkv=%d D=%d S=%d K=%d)",
                p->B, p->L, p->Hq, p->Hkv, p->D, p->S, p->K);
  if (p->dtype != HSA_F32 && p->dtype != HSA_BF16)
    return fail(HSA_ERR_UNSUPPORTED, "dtype %d is not fp32 (0) or bf16 (1)", p->dtype);
  if (p->Hq % p->Hkv != 0)
    return fail(HSA_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->Hq / p->Hkv > hsa::kMaxG)
    return fail(HSA_ERR_UNSUPPORTED, "Hq/Hkv=%d exceeds %d", p->Hq / p->Hkv, hsa::kMaxG);
  if (p->S != hsa::kChunk) return fail(HSA_ERR_UNSUPPORTED, "chunk size S=%d (only 64)", p->S);
  if (p->D != 64 && p->D != 128)
    return fail(HSA_ERR_UNSUPPORTED, "head dim D=%d (only 64 or 128)", p->D);
  if (p->K > hsa::kMaxK) return fail(HSA_ERR_UNSUPPORTED, "K=%d exceeds %d", p->K, hsa::kMaxK);
  if ((int64_t)p->L * p->K >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "L*K=%lld does not fit int32", (long long)p->L * p->K);
  if ((int64_t)p->B * p->L * p->Hkv >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "B*L*Hkv rows exceed the grid limit");
  if (p->flags & ~(HSA_FLAG_GENERIC | HSA_FLAG_SOFTMAX_WEIGHTS))
    return fail(HSA_ERR_INVALID_ARG, "unknown problem flags 0x%x", p->flags);
  if (!isfinite(p->sm_scale) || !isfinite(p->sel_scale))
    return fail(HSA_ERR_INVALID_ARG, "scales must be finite");
  const int nC = p->L / p->S;
  if (op == HSA_OP_BWD && nC > 32767)
    return fail(HSA_ERR_UNSUPPORTED, "backward supports at most 32767 chunks (nC=%d)", nC);
  d->B = p->B;
  d->L = p->L;
  d->Hq = p->Hq;
  d->Hkv = p->Hkv;
  d->D = p->D;
  d->S = p->S;
  d->K = p->K;
  d->nC = nC;
  d->G = p->Hq / p->Hkv;
  d->sm_scale = p->sm_scale != 0.0f ? (double)p->sm_scale : 1.0 / sqrt((double)p->D);
  d->sel_scale = p->sel_scale != 0.0f ? (double)p->sel_scale : 1.0 / sqrt((double)p->D);
  d->dtype = p->dtype;
  d->flags = p->flags;
  return HSA_OK;
}

hsa_status_t need_tensor(const void* ptr, const char* name) {
  if (!ptr) return fail(HSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(HSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return HSA_OK;
}

hsa_status_t need_small(const void* ptr, const char* name) {
  if (!ptr) return fail(HSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, 4)) return fail(HSA_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
  return HSA_OK;
}

size_t ws_bytes_for(int op, const hsa::Dims& d) {
  switch (op) {
    case HSA_OP_BWD:
      return hsa::bwd_layout(d).total;
    case HSA_OP_DECODE:
      return (d.flags & HSA_FLAG_GENERIC) ? hsa::dec_layout(d).total : hsa::dec_fast_ws(d);
    case HSA_OP_FWD:
      return hsa::fwd_mfma_supported(d) ? hsa::fwd_mfma_ws(d) : 0;
    default:
      return 0;
  }
}

hsa_status_t check_ws(int op, const hsa::Dims& d, const void* ws, size_t ws_bytes) {
  size_t need = ws_bytes_for(op, d);
  if (need == 0) return HSA_OK;
  if (!ws || ws_bytes < need)
    return fail(HSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                ws ? "" : " (NULL)");
  if (!aligned(ws, 256)) return fail(HSA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return HSA_OK;
}

// Refuse to enqueue behind an unreported failure of earlier work.
hsa_status_t check_pending() {
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess)
    return fail(HSA_ERR_HIP, "a HIP error is pending from earlier work: %s", hipGetErrorString(e));
  return HSA_OK;
}

hsa_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define TRY(x)                          \
  do {                                  \
    hsa_status_t st_ = (x);             \
    if (st_ != HSA_OK) return st_;      \
  } while (0)

// ---- forward-state records ------------------------------------------------------------
// The forward leaves, at the start of its workspace, state a backward over the same
// selection can reuse (the inverse index or token-tile job lists, and the normalisers).  The
// library records, per (workspace pointer, device), which forward filled it; any other call
// that writes into a workspace drops that workspace's record.  hsa_bwd reuses the state
// only when the record names this very problem and these Q, K, idx and w.
struct FwdRecord {
  const void* ws;
  int device;
  hsa_problem_t p;
  const void *Q, *K, *idx, *w;
};
constexpr int kMaxRecords = 64;
std::mutex g_rec_mu;
FwdRecord g_rec[kMaxRecords];
int g_n_rec = 0, g_next_rec = 0;

int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = -1;
  }
  return dev;
}

// The fields the forward's state depends on (the selection scale and the weighting rule
// do not enter it).
bool same_problem(const hsa_problem_t& a, const hsa_problem_t& b) {
  return a.B == b.B && a.L == b.L && a.Hq == b.Hq && a.Hkv == b.Hkv && a.D == b.D &&
         a.S == b.S && a.K == b.K && a.sm_scale == b.sm_scale && a.dtype == b.dtype &&
         (a.flags & HSA_FLAG_GENERIC) == (b.flags & HSA_FLAG_GENERIC);
}

int find_record(const void* ws, int dev) {
  for (int i = 0; i < g_n_rec; ++i)
    if (g_rec[i].ws == ws && g_rec[i].device == dev) return i;
  return -1;
}

void forget_state(const void* ws) {
  if (!ws) return;
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_rec_mu);
  const int i = find_record(ws, dev);
  if (i >= 0) g_rec[i].ws = nullptr;
}

void record_state(const void* ws, const hsa_problem_t* p, const void* Q, const void* K,
                  const void* idx, const void* w) {
  if (!ws) return;
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_rec_mu);
  int i = find_record(ws, dev);
  if (i < 0) {
    for (int j = 0; j < g_n_rec && i < 0; ++j)
      if (!g_rec[j].ws) i = j;  // a dropped record's place
  }
  if (i < 0) {
    if (g_n_rec < kMaxRecords) {
      i = g_n_rec++;
    } else {
      i = g_next_rec;
      g_next_rec = (g_next_rec + 1) % kMaxRecords;
    }
  }
  g_rec[i] = FwdRecord{ws, dev, *p, Q, K, idx, w};
}

bool state_matches(const void* ws, const hsa_problem_t* p, const void* Q, const void* K,
                   const void* idx, const void* w) {
  if (!ws) return false;
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_rec_mu);
  const int i = find_record(ws, dev);
  if (i < 0) return false;
  const FwdRecord& r = g_rec[i];
  return same_problem(r.p, *p) && r.Q == Q && r.K == K && r.idx == idx && r.w == w;
}

}  // namespace

HSA_EXPORT const char* hsa_status_string(hsa_status_t s) {
  switch (s) {
    case HSA_OK:
      return "HSA_OK";
    case HSA_ERR_INVALID_ARG:
      return "HSA_ERR_INVALID_ARG";
    case HSA_ERR_UNSUPPORTED:
      return "HSA_ERR_UNSUPPORTED";
    case HSA_ERR_WORKSPACE:
      return "HSA_ERR_WORKSPACE";
    case HSA_ERR_HIP:
      return "HSA_ERR_HIP";
  }
  return "HSA_ERR_UNKNOWN";
}

HSA_EXPORT const char* hsa_last_error(void) { return g_last_error.c_str(); }

HSA_EXPORT const char* hsa_version(void) { return "0.1.0"; }

HSA_EXPORT hsa_status_t hsa_workspace_size(int op, const hsa_problem_t* p, size_t* bytes) {
  hsa::Dims d;
  if (!bytes) return fail(HSA_ERR_INVALID_ARG, "bytes pointer is NULL");
  TRY(check_problem(op, p, &d));
  *bytes = ws_bytes_for(op, d);
  return ok();
}

HSA_EXPORT hsa_status_t hsa_select(const hsa_problem_t* p, const void* Qs, const void* K,
                                   void* Kslc, int32_t* idx, float* score, float* w, void* ws,
                                   size_t ws_bytes, hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_SELECT, p, &d));
  TRY(need_tensor(K, "K"));
  if (d.nC > 0) TRY(need_tensor(Kslc, "Kslc"));
  if (Qs) {
    TRY(need_tensor(Qs, "Qs"));
    TRY(need_small(idx, "idx"));
    TRY(need_small(score, "score"));
    TRY(need_small(w, "w"));
  }
  TRY(check_ws(HSA_OP_SELECT, d, ws, ws_bytes));
  TRY(check_pending());
  forget_state(ws);
  hipStream_t s = (hipStream_t)stream;
  if (d.nC > 0) {
    hipError_t e = hsa::launch_pool(d, K, Kslc, s);
    if (e != hipSuccess) return launched(e, "pool");
  }
  if (!Qs) return ok();
  hipError_t e;
  if (hsa::select_mfma_supported(d))
    e = hsa::launch_select_mfma(d, Qs, Kslc, idx, score, w, s);
  else if (hsa::select_tile_supported(d))
    e = hsa::launch_select_tile(d, Qs, Kslc, idx, score, w, s);
  else
    e = hsa::launch_select_generic(d, Qs, Kslc, idx, score, w, s);
  if (e == hipSuccess && hsa::softmax_w(d)) e = hsa::launch_softmax_weights(d, idx, score, w, s);
  return launched(e, "select");
}

HSA_EXPORT hsa_status_t hsa_fwd(const hsa_problem_t* p, const void* Q, const void* K,
                                const void* V, const int32_t* idx, const float* w, void* O,
                                float* lse, void* ws, size_t ws_bytes, hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_FWD, p, &d));
  TRY(need_tensor(Q, "Q"));
  TRY(need_tensor(K, "K"));
  TRY(need_tensor(V, "V"));
  TRY(need_small(idx, "idx"));
  TRY(need_small(w, "w"));
  TRY(need_tensor(O, "O"));
  if (lse && !aligned(lse, 4)) return fail(HSA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  TRY(check_ws(HSA_OP_FWD, d, ws, ws_bytes));
  TRY(check_pending());
  hipStream_t s = (hipStream_t)stream;
  forget_state(ws);
  if (!hsa::fwd_mfma_supported(d))
    return launched(hsa::launch_fwd_generic(d, Q, K, V, idx, w, O, lse, s), "fwd");
  hipError_t e = hsa::launch_fwd_mfma(d, Q, K, V, idx, w, O, (char*)ws, s);
  if (e == hipSuccess && lse)
    e = hsa::launch_lse_export(d, (const float*)((const char*)ws + hsa::fwd_state(d).lse), idx,
                               lse, s);
  if (e == hipSuccess) record_state(ws, p, Q, K, idx, w);
  return launched(e, "fwd");
}

HSA_EXPORT hsa_status_t hsa_bwd(const hsa_problem_t* p, const void* Q, const void* K,
                                const void* V, const void* Qs, const void* Kslc,
                                const int32_t* idx, const float* score, const float* w,
                                const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                                void* dQs, float* dKslc, uint32_t flags, void* ws,
                                size_t ws_bytes, hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_BWD, p, &d));
  TRY(need_tensor(Q, "Q"));
  TRY(need_tensor(K, "K"));
  TRY(need_tensor(V, "V"));
  TRY(need_tensor(Qs, "Qs"));
  if (d.nC > 0) TRY(need_tensor(Kslc, "Kslc"));
  TRY(need_small(idx, "idx"));
  TRY(need_small(score, "score"));
  TRY(need_small(w, "w"));
  if (lse && !aligned(lse, 4)) return fail(HSA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  TRY(need_tensor(dO, "dO"));
  TRY(need_tensor(dQ, "dQ"));
  TRY(need_tensor(dK, "dK"));
  TRY(need_tensor(dV, "dV"));
  TRY(need_tensor(dQs, "dQs"));
  if (dKslc && !aligned(dKslc, 16)) return fail(HSA_ERR_INVALID_ARG, "dKslc is not 16-byte aligned");
  if (flags & ~(uint32_t)(HSA_BWD_FOLD_KSLC | HSA_BWD_AFTER_FWD))
    return fail(HSA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  TRY(check_ws(HSA_OP_BWD, d, ws, ws_bytes));
  TRY(check_pending());
  hipStream_t s = (hipStream_t)stream;
  hsa::BwdLayout lay = hsa::bwd_layout(d);
  const bool fold = (flags & HSA_BWD_FOLD_KSLC) != 0;
  if (!hsa::bwd_mfma_supported(d)) {
    forget_state(ws);
    return launched(hsa::launch_bwd_generic(d, lay, Q, K, V, Qs, Kslc, idx, score, w, dO, dQ,
                                            dK, dV, dQs, dKslc, fold, (char*)ws, s),
                    "bwd");
  }
  // the forward's state is reused only when the record of this workspace confirms it
  const bool reuse = (flags & HSA_BWD_AFTER_FWD) && hsa::fwd_mfma_supported(d) &&
                     state_matches(ws, p, Q, K, idx, w);
  // a backward that rebuilds the index or copies the caller's normalisers into the state
  // leaves a state that no forward made
  if (!reuse || lse) forget_state(ws);
  return launched(hsa::launch_bwd_mfma(d, lay, Q, K, V, Qs, Kslc, idx, score, w, lse, dO, dQ,
                                       dK, dV, dQs, dKslc, fold, reuse, (char*)ws, s),
                  "bwd");
}

namespace {

// The device's view of page-locked host memory, or an error for anything else.
hsa_status_t host_view(const void* p, const char* name, const void** dev) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // the query's own error is not a failure of enqueued work
    return fail(HSA_ERR_INVALID_ARG, "%s is not page-locked host memory (%s)", name,
                hipGetErrorString(e));
  }
  if (a.type != hipMemoryTypeHost || !a.devicePointer)
    return fail(HSA_ERR_INVALID_ARG, "%s is not host memory mapped for the device", name);
  *dev = a.devicePointer;
  return HSA_OK;
}

}  // namespace

namespace {

hsa_status_t decode_impl(const hsa_problem_t* p, const void* q, const void* qs,
                         const void* Kcache, const void* Vcache, const void* Kslc, void* O,
                         int32_t* idx, float* score, float* w, void* ws, size_t ws_bytes,
                         hsa_stream_t stream, bool host_kv, const int32_t* ctx_lens) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_DECODE, p, &d));
  TRY(need_tensor(q, "q"));
  TRY(need_tensor(qs, "qs"));
  TRY(need_tensor(Kcache, "Kcache"));
  TRY(need_tensor(Vcache, "Vcache"));
  if (d.nC > 0) TRY(need_tensor(Kslc, "Kslc"));
  TRY(need_tensor(O, "O"));
  TRY(need_small(idx, "idx"));
  TRY(need_small(w, "w"));
  if (score && !aligned(score, 4)) return fail(HSA_ERR_INVALID_ARG, "score is not 4-byte aligned");
  TRY(check_ws(HSA_OP_DECODE, d, ws, ws_bytes));
  TRY(check_pending());
  forget_state(ws);
  hipStream_t s = (hipStream_t)stream;
  if (!(d.flags & HSA_FLAG_GENERIC))
    return launched(hsa::launch_decode_fast(d, q, qs, Kcache, Vcache, Kslc, O, idx, score, w,
                                            host_kv, ctx_lens, (char*)ws, s),
                    "decode");
  hsa::DecLayout lay = hsa::dec_layout(d);
  return launched(hsa::launch_decode_generic(d, lay, q, qs, Kcache, Vcache, Kslc, O, idx, score,
                                             w, ctx_lens, (char*)ws, s),
                  "decode");
}

}  // namespace

HSA_EXPORT hsa_status_t hsa_decode(const hsa_problem_t* p, const void* q, const void* qs,
                                   const void* Kcache, const void* Vcache, const void* Kslc,
                                   void* O, int32_t* idx, float* score, float* w, void* ws,
                                   size_t ws_bytes, hsa_stream_t stream) {
  return decode_impl(p, q, qs, Kcache, Vcache, Kslc, O, idx, score, w, ws, ws_bytes, stream,
                     false, nullptr);
}

// ---- decode without a caller workspace ---------------------------------------------------
// Scratch of hsa_decode_noalloc: the scan blocks' candidate keys, in a file-scope device
// array.  Each device that runs the library holds its own copy until the process ends.  In
// host code the array's name is not a device address: the address of this device's copy
// comes from hipGetSymbolAddress, taken once per device and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (nullptr and a message on failure).
hsa_status_t scratch_for_current_device(void** out) {
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HSA_ERR_HIP, "no current HIP device in [0, %d) (got %d)", kMaxDevices, dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(HSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HSA_OK;
}

}  // namespace

HSA_EXPORT hsa_status_t hsa_decode_noalloc(const hsa_problem_t* p, const void* q,
                                           const void* qs, const void* Kcache,
                                           const void* Vcache, const void* Kslc, void* O,
                                           int32_t* idx, float* score, float* w,
                                           hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_DECODE, p, &d));
  const size_t need = ws_bytes_for(HSA_OP_DECODE, d);
  if (need > kNoAllocScratchBytes)
    return fail(HSA_ERR_UNSUPPORTED,
                "decode needs %zu bytes of scratch, more than the %zu hsa_decode_noalloc holds "
                "(use hsa_decode with a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) TRY(scratch_for_current_device(&ws));
  return decode_impl(p, q, qs, Kcache, Vcache, Kslc, O, idx, score, w, ws,
                     ws ? kNoAllocScratchBytes : 0, stream, false, nullptr);
}

HSA_EXPORT hsa_status_t hsa_decode_host_kv(const hsa_problem_t* p, const void* q,
                                           const void* qs, const void* Kcache,
                                           const void* Vcache, const void* Kslc, void* O,
                                           int32_t* idx, float* score, float* w, void* ws,
                                           size_t ws_bytes, hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_DECODE, p, &d));
  TRY(need_tensor(Kcache, "Kcache"));
  TRY(need_tensor(Vcache, "Vcache"));
  const void *kd = nullptr, *vd = nullptr;
  TRY(host_view(Kcache, "Kcache", &kd));
  TRY(host_view(Vcache, "Vcache", &vd));
  if (!aligned(kd, 16) || !aligned(vd, 16))
    return fail(HSA_ERR_INVALID_ARG, "the device view of the caches is not 16-byte aligned");
  return decode_impl(p, q, qs, kd, vd, Kslc, O, idx, score, w, ws, ws_bytes, stream, true,
                     nullptr);
}

HSA_EXPORT hsa_status_t hsa_decode_ragged(const hsa_problem_t* p, const int32_t* ctx_lens,
                                          const void* q, const void* qs, const void* Kcache,
                                          const void* Vcache, const void* Kslc, void* O,
                                          int32_t* idx, float* score, float* w, void* ws,
                                          size_t ws_bytes, hsa_stream_t stream) {
  TRY(need_small(ctx_lens, "ctx_lens"));
  return decode_impl(p, q, qs, Kcache, Vcache, Kslc, O, idx, score, w, ws, ws_bytes, stream,
                     false, ctx_lens);
}

HSA_EXPORT hsa_status_t hsa_pool_chunks(const hsa_problem_t* p, const void* K, void* Kslc,
                                        const int32_t* chunk_ids, int n_ids,
                                        hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_SELECT, p, &d));
  TRY(need_tensor(K, "K"));
  if (d.nC > 0) TRY(need_tensor(Kslc, "Kslc"));
  TRY(need_small(chunk_ids, "chunk_ids"));
  if (n_ids < 1 || n_ids > (d.nC > 1 ? d.nC : 1))
    return fail(HSA_ERR_INVALID_ARG, "n_ids=%d is outside [1, max(nC, 1)]", n_ids);
  TRY(check_pending());
  return launched(hsa::launch_pool_chunks(d, K, Kslc, chunk_ids, n_ids, (hipStream_t)stream),
                  "pool_chunks");
}

HSA_EXPORT hsa_status_t hsa_fwd_layers(const hsa_problem_t* p, int n_layers, const void* Q,
                                       const void* K, const void* V, const int32_t* idx,
                                       const float* w, void* O, void* ws, size_t ws_bytes,
                                       hsa_stream_t stream) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_FWD, p, &d));
  if (n_layers < 1) return fail(HSA_ERR_INVALID_ARG, "n_layers=%d must be positive", n_layers);
  TRY(need_tensor(Q, "Q"));
  TRY(need_tensor(K, "K"));
  TRY(need_tensor(V, "V"));
  TRY(need_small(idx, "idx"));
  TRY(need_small(w, "w"));
  TRY(need_tensor(O, "O"));
  TRY(check_ws(HSA_OP_FWD, d, ws, ws_bytes));
  TRY(check_pending());
  forget_state(ws);
  hipStream_t s = (hipStream_t)stream;
  const size_t el = d.dtype == HSA_BF16 ? 2 : 4;
  const size_t q_ls = (size_t)d.B * d.L * d.Hq * d.D * el;
  const size_t kv_ls = (size_t)d.B * d.L * d.Hkv * d.D * el;
  const bool mfma = hsa::fwd_mfma_supported(d);
  for (int l = 0; l < n_layers; ++l) {
    const char* Ql = (const char*)Q + l * q_ls;
    const char* Kl = (const char*)K + l * kv_ls;
    const char* Vl = (const char*)V + l * kv_ls;
    char* Ol = (char*)O + l * q_ls;
    // the layers share the selection: its index is built for the first layer only
    const hipError_t e =
        mfma ? hsa::launch_fwd_mfma(d, Ql, Kl, Vl, idx, w, Ol, (char*)ws, s, l > 0)
             : hsa::launch_fwd_generic(d, Ql, Kl, Vl, idx, w, Ol, nullptr, s);
    if (e != hipSuccess) return launched(e, "fwd_layers");
    if (mfma && l == n_layers - 1) record_state(ws, p, Ql, Kl, idx, w);
  }
  return ok();
}

namespace {

hsa_status_t decode_shared_impl(const hsa_problem_t* p, int n_layers, const void* q,
                                const void* Kcache, const void* Vcache, const int32_t* idx,
                                const float* w, void* O, hsa_stream_t stream, bool host_kv) {
  hsa::Dims d;
  TRY(check_problem(HSA_OP_DECODE, p, &d));
  if (n_layers < 1 || n_layers > 65535)
    return fail(HSA_ERR_INVALID_ARG, "n_layers=%d is outside [1, 65535]", n_layers);
  TRY(need_tensor(q, "q"));
  TRY(need_tensor(Kcache, "Kcache"));
  TRY(need_tensor(Vcache, "Vcache"));
  TRY(need_small(idx, "idx"));
  TRY(need_small(w, "w"));
  TRY(need_tensor(O, "O"));
  if (host_kv) {
    const void *kd = nullptr, *vd = nullptr;
    TRY(host_view(Kcache, "Kcache", &kd));
    TRY(host_view(Vcache, "Vcache", &vd));
    if (!aligned(kd, 16) || !aligned(vd, 16))
      return fail(HSA_ERR_INVALID_ARG, "the device view of the caches is not 16-byte aligned");
    Kcache = kd;
    Vcache = vd;
  }
  TRY(check_pending());
  return launched(hsa::launch_decode_shared(d, n_layers, q, Kcache, Vcache, idx, w, O, host_kv,
                                            (hipStream_t)stream),
                  "decode_shared");
}

}  // namespace

HSA_EXPORT hsa_status_t hsa_decode_shared(const hsa_problem_t* p, int n_layers, const void* q,
                                          const void* Kcache, const void* Vcache,
                                          const int32_t* idx, const float* w, void* O,
                                          hsa_stream_t stream) {
  return decode_shared_impl(p, n_layers, q, Kcache, Vcache, idx, w, O, stream, false);
}

HSA_EXPORT hsa_status_t hsa_decode_shared_host_kv(const hsa_problem_t* p, int n_layers,
                                                  const void* q, const void* Kcache,
                                                  const void* Vcache, const int32_t* idx,
                                                  const float* w, void* O,
                                                  hsa_stream_t stream) {
  return decode_shared_impl(p, n_layers, q, Kcache, Vcache, idx, w, O, stream, true);
}
