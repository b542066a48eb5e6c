// Argument block shared by the backward kernels (bwd.hip: D, key means,
// G_K/G_V; bwd_dq.hip: G_Q).
#pragma once
#include "bl_device.h"

namespace backlite {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* olo;  // optional bf16 residual of O (O_fp32 ~ O + olo)
  const uint16_t* dout;
  const float* lse;
  const int32_t* qcnt;
  const uint16_t* qidx;
  const int32_t* kcnt;
  const uint16_t* kidx;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dbuf;  // D, [B, H, n]
  float* kbar;  // per key tile mean of K over its valid keys, [B, Hk, T, d]
  int B, n, H, Hk, T;
  float scale;
  float scale_log2;
};

}  // namespace backlite
