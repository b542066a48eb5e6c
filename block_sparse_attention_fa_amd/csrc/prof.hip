// Per-kernel timing: every launch made while profiling is on records a start
// and a stop hipEvent on its stream; backlite_profile_read() waits for the
// recorded events and accumulates the elapsed times per kernel.
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/backlite.h"
#include "prof.h"

namespace backlite {
namespace {

const char* kNames[PK_COUNT] = {"fwd", "mask_select", "mask_transpose", "delta", "kmean", "dkdv", "dq", "gs_slots", "dk_plan", "dk_reduce"};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<ProfRec> g_pending;
std::vector<hipEvent_t> g_pool;
double g_ms[PK_COUNT];
long long g_count[PK_COUNT];

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Called with g_mu held: wait for every pending record and fold it in.
hipError_t drain() {
  hipError_t err = hipSuccess;
  for (ProfRec& r : g_pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e == hipSuccess) {
      g_ms[r.kernel] += ms;
      g_count[r.kernel] += 1;
    } else if (err == hipSuccess) {
      err = e;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_pending.clear();
  return err;
}

}  // namespace

ProfRec prof_begin(ProfKernel k, hipStream_t st) {
  ProfRec r{-1, nullptr, nullptr};
  if (!g_on.load(std::memory_order_relaxed)) return r;
  std::lock_guard<std::mutex> lk(g_mu);
  r.start = get_event();
  r.stop = get_event();
  if (r.start && r.stop && hipEventRecord(r.start, st) == hipSuccess) {
    r.kernel = (int)k;
  } else {
    if (r.start) g_pool.push_back(r.start);
    if (r.stop) g_pool.push_back(r.stop);
    r.start = r.stop = nullptr;
  }
  return r;
}

void prof_end(const ProfRec& r, hipStream_t st) {
  if (r.kernel < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(r.stop, st) == hipSuccess) {
    g_pending.push_back(r);
  } else {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
}

}  // namespace backlite

using namespace backlite;

extern "C" {

int backlite_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!on) (void)drain();
  g_on.store(on ? 1 : 0);
  return BACKLITE_OK;
}

int backlite_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  (void)drain();
  std::memset(g_ms, 0, sizeof(g_ms));
  std::memset(g_count, 0, sizeof(g_count));
  return BACKLITE_OK;
}

int backlite_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return BACKLITE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  if (drain() != hipSuccess) return BACKLITE_ERR_HIP;
  for (int i = 0; i < PK_COUNT; ++i)
    if (std::strcmp(kNames[i], kernel) == 0) {
      *total_ms = g_ms[i];
      *launches = g_count[i];
      return BACKLITE_OK;
    }
  return BACKLITE_ERR_INVALID_ARG;
}

}  // extern "C"
