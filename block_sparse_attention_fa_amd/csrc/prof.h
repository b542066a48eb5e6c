// Opt-in per-kernel timing with HIP events recorded on the launch stream
// (backlite_profile_* in include/backlite.h).  When disabled, the hooks cost
// one relaxed atomic load.
#pragma once
#include <hip/hip_runtime.h>

namespace backlite {

enum ProfKernel {
  PK_FWD = 0,
  PK_MASK_SELECT,
  PK_MASK_TRANSPOSE,
  PK_DELTA,
  PK_KMEAN,
  PK_DKDV,
  PK_DQ,
  PK_GS_SLOTS,
  PK_DK_PLAN,
  PK_DK_REDUCE,
  PK_COUNT
};

struct ProfRec {
  int kernel;  // -1: profiling off, nothing recorded
  hipEvent_t start, stop;
};

// Records the start event when profiling is on.
ProfRec prof_begin(ProfKernel k, hipStream_t st);
// Records the stop event and queues the pair for backlite_profile_read.
void prof_end(const ProfRec& r, hipStream_t st);

struct ProfScope {
  ProfRec rec;
  hipStream_t st;
  ProfScope(ProfKernel k, hipStream_t s) : rec(prof_begin(k, s)), st(s) {}
  ~ProfScope() { prof_end(rec, st); }
};

}  // namespace backlite
