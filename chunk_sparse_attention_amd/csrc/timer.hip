// timer.hip -- optional HIP-event timing of the library's kernel launches.
//
// When enabled, every launch of a timed kernel class is bracketed by a pair of HIP events
// recorded on the launch's own stream, so the elapsed time between them is that kernel's
// duration on the device.  Disabled (the default) the launch sites pay one relaxed atomic
// load.  Used by measurement tools; never needed for correct results.
#include <atomic>
#include <mutex>
#include <vector>

#include "hsa.h"
#include "hsa_launch.h"

namespace hsa {
namespace {

constexpr int kMaxRecords = 4096;  // per kernel class; later launches are not recorded

struct ClassRecords {
  std::vector<hipEvent_t> start, stop;  // created on demand, reused after a reset
  int used = 0;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
ClassRecords g_rec[HSA_KERNEL_COUNT];

}  // namespace

Timed::Timed(int kc, hipStream_t s) : kc_(kc), slot_(-1), s_(s) {
  if (!g_enabled.load(std::memory_order_relaxed) || kc < 0 || kc >= HSA_KERNEL_COUNT) return;
  std::lock_guard<std::mutex> lk(g_mu);
  ClassRecords& r = g_rec[kc];
  if (r.used >= kMaxRecords) return;
  if (r.used == (int)r.start.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return;
    }
    r.start.push_back(a);
    r.stop.push_back(b);
  }
  if (hipEventRecord(r.start[r.used], s) != hipSuccess) return;
  slot_ = r.used++;
}

Timed::~Timed() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  (void)hipEventRecord(g_rec[kc_].stop[slot_], s_);
}

}  // namespace hsa

#define HSA_EXPORT extern "C" __attribute__((visibility("default")))

HSA_EXPORT hsa_status_t hsa_timer_enable(int enable) {
  std::lock_guard<std::mutex> lk(hsa::g_mu);
  if (enable)
    for (auto& r : hsa::g_rec) r.used = 0;
  hsa::g_enabled.store(enable != 0);
  return HSA_OK;
}

HSA_EXPORT hsa_status_t hsa_timer_read(int kernel, int* launches, double* total_ms) {
  if (kernel < 0 || kernel >= HSA_KERNEL_COUNT || !launches || !total_ms)
    return HSA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(hsa::g_mu);
  const auto& r = hsa::g_rec[kernel];
  double sum = 0.0;
  for (int i = 0; i < r.used; ++i) {
    if (hipEventSynchronize(r.stop[i]) != hipSuccess) return HSA_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.start[i], r.stop[i]) != hipSuccess) return HSA_ERR_HIP;
    sum += ms;
  }
  *launches = r.used;
  *total_ms = sum;
  return HSA_OK;
}
