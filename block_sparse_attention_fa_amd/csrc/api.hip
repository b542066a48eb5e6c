// C ABI of the BackLite hot path: argument validation, sizes, error strings,
// and dispatch to the HIP kernels.  Declarations and the contract of every
// entry point are in include/backlite.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/backlite.h"

namespace backlite {
hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int n, int H,
                      int Hk, int d, float scale, int causal, int window, uint16_t* o, uint16_t* olo,
                      float* lse, float* tlse, double* tw, hipStream_t st);
hipError_t launch_mask(const float* tlse, const double* tw, const float* lse, int B, int H, int n, int causal,
                       int window, int q_tile, double negl, uint8_t* keep, int32_t* qcnt, uint16_t* qidx,
                       int32_t* kcnt, uint16_t* kidx, int64_t* stats, hipStream_t st);
hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* olo, const uint16_t* dout, const float* lse, const int32_t* qcnt,
                      const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n,
                      int H, int Hk, int d, float scale, int causal, int window, int q_tile, uint16_t* dq,
                      uint16_t* dk, uint16_t* dv, float* dbuf, float* lse2, float* kbar, int32_t* gsinfo, uint32_t* qbase,
                      uint32_t* kslot, uint16_t* gs, float* gsl, long long gs_cap, int32_t* dkplan,
                      float* dkpart, int dk_chmin, int dk_pcap, float* dqacc, hipStream_t st);
size_t similarity_elems();
hipError_t launch_similarity(const uint16_t* a, const uint16_t* b, long m, double* out, hipStream_t st);
}  // namespace backlite

namespace {

constexpr int kTile = 128;
constexpr int kMaxN = 131072;  // 1024 tiles: the mask kernel's LDS sort capacity

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BACKLITE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ntiles(int n) { return (n + kTile - 1) / kTile; }
int ntiles(int n, int tile) { return (n + tile - 1) / tile; }

// Rows per backward query tile: 128 (the forward's tiles) or 64 (half-height
// backward tiles, a finer mask; the README forms the mask "for each backward
// tile pair", and a backward's tiles need not match the forward's).
int check_q_tile(int q_tile) {
  if (q_tile != 64 && q_tile != 128)
    return fail(BACKLITE_ERR_UNSUPPORTED, "q_tile must be 64 or 128 (got %d)", q_tile);
  return BACKLITE_OK;
}

// Shape checks shared by fwd and bwd.  Sizes must keep every element index of
// the largest tensor below 2^62 and the grid below 2^31 workgroups.
int check_shape(int B, int n, int H, int Hk, int d) {
  if (B < 1 || n < 1 || H < 1 || Hk < 1)
    return fail(BACKLITE_ERR_INVALID_ARG, "B, n, H, H_k must be >= 1 (got B=%d n=%d H=%d H_k=%d)", B, n,
                H, Hk);
  if (H % Hk != 0) return fail(BACKLITE_ERR_INVALID_ARG, "H (%d) must be a multiple of H_k (%d)", H, Hk);
  if (n > kMaxN) return fail(BACKLITE_ERR_UNSUPPORTED, "n = %d exceeds the supported maximum %d", n, kMaxN);
  if (d != 64 && d != 128) return fail(BACKLITE_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d);
  if ((long long)B * H * ntiles(n) > 0x7fffffffLL)
    return fail(BACKLITE_ERR_INVALID_ARG, "B*H*ceil(n/128) exceeds 2^31");
  return BACKLITE_OK;
}

int check_ptr(const void* p, const char* name, bool allow_null = false) {
  if (p == nullptr) {
    if (allow_null) return BACKLITE_OK;
    return fail(BACKLITE_ERR_INVALID_ARG, "%s is NULL", name);
  }
  if (!aligned16(p)) return fail(BACKLITE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return BACKLITE_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(BACKLITE_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  return BACKLITE_OK;
}

// Sliding window: 0 = none; w > 0 lets query i see keys i - w < j <= i, so it
// needs causal attention.
int check_window(int causal, int window) {
  if (window < 0) return fail(BACKLITE_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
  if (window > 0 && !causal) return fail(BACKLITE_ERR_INVALID_ARG, "a sliding window (%d) requires causal", window);
  return BACKLITE_OK;
}

bool env_on(const char* name) {
  const char* env = std::getenv(name);
  return env && env[0] && env[0] != '0';
}
bool verbose() { return env_on("BACKLITE_VERBOSE"); }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BACKLITE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define TRY(x)                        \
  do {                                \
    int _r = (x);                     \
    if (_r != BACKLITE_OK) return _r; \
  } while (0)

}  // namespace

extern "C" {

size_t backlite_tile_lse_elems(int B, int H, int n, int causal) {
  if (B < 1 || H < 1 || n < 1) return 0;
  const size_t T = (size_t)ntiles(n);
  const size_t pairs = causal ? T * (T + 1) / 2 : T * T;
  return (size_t)B * H * pairs * kTile;
}

size_t backlite_mask_elems(int B, int H, int n, int q_tile) {
  if (B < 1 || H < 1 || n < 1 || (q_tile != 64 && q_tile != 128)) return 0;
  return (size_t)B * H * ntiles(n, q_tile) * ntiles(n);
}

size_t backlite_count_elems(int B, int H, int n, int tile) {
  if (B < 1 || H < 1 || n < 1 || (tile != 64 && tile != 128)) return 0;
  return (size_t)B * H * ntiles(n, tile);
}

namespace {
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t delta_bytes(int B, int H, int n) { return round256((size_t)B * H * n * sizeof(float)); }
}  // namespace

namespace {
// chunked G_K/G_V work: plan (header, chunk table, per-key-tile counts) and
// the fp32 partial slots of split key tiles
size_t dkplan_bytes(int B, int H_k, int n) {
  const size_t NK = (size_t)B * H_k * ntiles(n);
  return round256((4 + 11 * NK) * sizeof(int32_t));
}
size_t dkpart_bytes(int B, int H_k, int n, int d) {
  const size_t NK = (size_t)B * H_k * ntiles(n);
  return round256(NK * 2 * 128 * (size_t)d * sizeof(float));
}
}  // namespace

size_t backlite_bwd_workspace_bytes(int B, int H, int H_k, int n, int d) {
  if (B < 1 || H < 1 || H_k < 1 || n < 1 || d < 1) return 0;
  return 2 * delta_bytes(B, H, n) + round256((size_t)B * H_k * ntiles(n) * d * sizeof(float)) +
         dkplan_bytes(B, H_k, n) + dkpart_bytes(B, H_k, n, d);
}

namespace {
// one stored tile: bf16 G_S of q_tile x 128 + fp32 residual sums [4][q_tile]
size_t slot_bytes(int q_tile) { return (size_t)q_tile * 128 * 2 + 4 * (size_t)q_tile * 4; }
constexpr size_t kStateBytes = 256;                          // gsinfo words
// stored-path index arrays after the base workspace: state, qbase [B,H,Tq], kslot [B,H,T,Tq]
size_t gs_index_bytes(int B, int H, int n, int q_tile) {
  const size_t T = (size_t)ntiles(n), Tq = (size_t)ntiles(n, q_tile);
  return kStateBytes + round256((size_t)B * H * Tq * 4) + round256((size_t)B * H * T * Tq * 4);
}
}  // namespace

size_t backlite_bwd_workspace_bytes_stored(int B, int H, int H_k, int n, int d, int q_tile, int64_t max_tiles) {
  const size_t base = backlite_bwd_workspace_bytes(B, H, H_k, n, d);
  if (base == 0 || max_tiles < 1) return base;
  if (q_tile != 64 && q_tile != 128) return 0;
  return base + gs_index_bytes(B, H, n, q_tile) + (size_t)max_tiles * slot_bytes(q_tile);
}

size_t backlite_bwd_state_offset(int B, int H, int H_k, int n, int d) {
  return backlite_bwd_workspace_bytes(B, H, H_k, n, d);
}

int backlite_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B, int n, int H,
                 int H_k, int d, float scale, int causal, int window, uint16_t* O, uint16_t* O_lo,
                 float* lse_row, float* tile_lse, double* tile_w, void* stream) {
  TRY(check_shape(B, n, H, H_k, d));
  TRY(check_scale(scale));
  TRY(check_window(causal, window));
  TRY(check_ptr(Q, "Q"));
  TRY(check_ptr(K, "K"));
  TRY(check_ptr(V, "V"));
  TRY(check_ptr(O, "O"));
  TRY(check_ptr(O_lo, "O_lo", true));
  TRY(check_ptr(lse_row, "lse_row"));
  TRY(check_ptr(tile_lse, "tile_lse", true));
  TRY(check_ptr(tile_w, "tile_w", true));
  if (tile_w != nullptr && tile_lse == nullptr)
    return fail(BACKLITE_ERR_INVALID_ARG, "tile_w needs tile_lse (the per-row statistics it is reduced from)");
  return hip_status(backlite::launch_fwd(Q, K, V, B, n, H, H_k, d, scale, causal ? 1 : 0, window, O, O_lo,
                                         lse_row, tile_lse, tile_w, (hipStream_t)stream),
                    "backlite_fwd launch");
}

}  // extern "C"

namespace {
// Shared by backlite_mask (per-row statistics) and backlite_mask_compact
// (tile_w); exactly one of tile_lse / tile_w is used, or neither with negl 0.
int mask_impl(bool compact, const float* tile_lse, const double* tile_w, const float* lse_row, int B, int H,
              int n, int causal, int window, int q_tile, float negl_prob, uint8_t* keep, int32_t* qcnt,
              uint16_t* qidx, int32_t* kcnt, uint16_t* kidx, int64_t* stats, void* stream) {
  if (B < 1 || n < 1 || H < 1)
    return fail(BACKLITE_ERR_INVALID_ARG, "B, n, H must be >= 1 (got B=%d n=%d H=%d)", B, n, H);
  if (n > kMaxN) return fail(BACKLITE_ERR_UNSUPPORTED, "n = %d exceeds the supported maximum %d", n, kMaxN);
  if ((long long)B * H * ntiles(n) > 0x7fffffffLL)
    return fail(BACKLITE_ERR_INVALID_ARG, "B*H*ceil(n/128) exceeds 2^31");
  TRY(check_window(causal, window));
  TRY(check_q_tile(q_tile));
  if (!std::isfinite(negl_prob) || negl_prob < 0.f || negl_prob >= 1.f)
    return fail(BACKLITE_ERR_INVALID_ARG, "negl_prob must be finite and in [0, 1) (got %g)",
                (double)negl_prob);
  if (tile_lse == nullptr && tile_w == nullptr && negl_prob != 0.f)
    return fail(BACKLITE_ERR_INVALID_ARG, "the statistics may be NULL only with negl_prob == 0");
  TRY(check_ptr(tile_lse, "tile_lse", true));
  TRY(check_ptr(tile_w, "tile_w", true));
  if (!compact) TRY(check_ptr(lse_row, "lse_row"));
  TRY(check_ptr(keep, "keep"));
  TRY(check_ptr(qcnt, "qcnt"));
  TRY(check_ptr(qidx, "qidx"));
  TRY(check_ptr(kcnt, "kcnt"));
  TRY(check_ptr(kidx, "kidx"));
  TRY(check_ptr(stats, "stats", true));
  hipError_t e = backlite::launch_mask(tile_w ? nullptr : tile_lse, tile_w, lse_row, B, H, n, causal ? 1 : 0, window,
                                       q_tile, (double)negl_prob, keep, qcnt, qidx, kcnt, kidx, stats,
                                       (hipStream_t)stream);
  int r = hip_status(e, "backlite_mask launch");
  if (r == BACKLITE_OK && verbose()) {
    // synchronous readback of the counts: a debugging aid, off by default
    const size_t nq = (size_t)B * H * ntiles(n, q_tile), nk = (size_t)B * H * ntiles(n);
    std::vector<int32_t> qc(nq), kc(nk);
    long long hs[2] = {0, 0};
    e = hipMemcpyAsync(qc.data(), qcnt, nq * 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpyAsync(kc.data(), kcnt, nk * 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess && stats) e = hipMemcpyAsync(hs, stats, sizeof(hs), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "BACKLITE_VERBOSE readback");
    long long kept = 0, cand = 0;
    int qmin = 1 << 30, qmax = 0, kmin = 1 << 30, kmax = 0;
    for (size_t i = 0; i < nq; ++i) {
      kept += qc[i];
      qmin = std::min(qmin, (int)qc[i]);
      qmax = std::max(qmax, (int)qc[i]);
    }
    for (size_t i = 0; i < nk; ++i) {
      kmin = std::min(kmin, (int)kc[i]);
      kmax = std::max(kmax, (int)kc[i]);
    }
    const int T = ntiles(n), Tq = ntiles(n, q_tile), w = (window > 0 && window < n) ? window : 0;
    for (int qt = 0; qt < Tq; ++qt) {  // candidate key tiles per query tile
      const int first = qt * q_tile, last = std::min(n, first + q_tile) - 1;
      int lo = 0, hi = T - 1;
      if (causal) hi = last / kTile;
      if (w && first - w + 1 > 0) lo = (first - w + 1) / kTile;
      cand += hi - lo + 1;
    }
    cand *= (long long)B * H;
    std::fprintf(stderr,
                 "[backlite] mask B=%d H=%d n=%d causal=%d window=%d q_tile=%d negl_prob=%g: kept %lld of %lld "
                 "candidate tiles (density %.4f, sparsity %.4f); q-list length min %d mean %.1f max %d; k-list "
                 "length min %d mean %.1f max %d",
                 B, H, n, causal ? 1 : 0, w, q_tile, (double)negl_prob, kept, cand, cand ? (double)kept / cand : 0.0,
                 cand ? 1.0 - (double)kept / cand : 0.0, qmin, (double)kept / nq, qmax, kmin, (double)kept / nk,
                 kmax);
    if (stats) std::fprintf(stderr, "; stats buffer (accumulated) %lld / %lld", hs[1], hs[0]);
    std::fprintf(stderr, "\n");
  }
  return r;
}
}  // namespace

extern "C" {

int backlite_mask(const float* tile_lse, const float* lse_row, int B, int H, int n, int causal,
                  int window, int q_tile, float negl_prob, uint8_t* keep, int32_t* qcnt, uint16_t* qidx,
                  int32_t* kcnt, uint16_t* kidx, int64_t* stats, void* stream) {
  return mask_impl(false, tile_lse, nullptr, lse_row, B, H, n, causal, window, q_tile, negl_prob, keep, qcnt, qidx,
                   kcnt, kidx, stats, stream);
}

int backlite_mask_compact(const double* tile_w, int B, int H, int n, int causal, int window, int q_tile,
                          float negl_prob, uint8_t* keep, int32_t* qcnt, uint16_t* qidx, int32_t* kcnt,
                          uint16_t* kidx, int64_t* stats, void* stream) {
  return mask_impl(true, nullptr, tile_w, nullptr, B, H, n, causal, window, q_tile, negl_prob, keep, qcnt, qidx,
                   kcnt, kidx, stats, stream);
}

}  // extern "C"

namespace {

int check_bwd_args(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const uint16_t* O,
                   const uint16_t* O_lo, const uint16_t* dO, const float* lse_row, const int32_t* qcnt,
                   const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n, int H, int H_k,
                   int d, float scale, int causal, int window, int q_tile, uint16_t* dQ, uint16_t* dK, uint16_t* dV) {
  TRY(check_shape(B, n, H, H_k, d));
  TRY(check_scale(scale));
  TRY(check_window(causal, window));
  TRY(check_q_tile(q_tile));
  TRY(check_ptr(Q, "Q"));
  TRY(check_ptr(K, "K"));
  TRY(check_ptr(V, "V"));
  TRY(check_ptr(O, "O"));
  TRY(check_ptr(O_lo, "O_lo", true));
  TRY(check_ptr(dO, "dO"));
  TRY(check_ptr(lse_row, "lse_row"));
  TRY(check_ptr(qcnt, "qcnt"));
  TRY(check_ptr(qidx, "qidx"));
  TRY(check_ptr(kcnt, "kcnt"));
  TRY(check_ptr(kidx, "kidx"));
  TRY(check_ptr(dQ, "dQ"));
  TRY(check_ptr(dK, "dK"));
  TRY(check_ptr(dV, "dV"));
  return BACKLITE_OK;
}

int min_chunk() {
  int chmin = 16;  // smallest chunk of a split G_K/G_V list (BACKLITE_DKDV_MIN_CHUNK overrides)
  if (const char* env = std::getenv("BACKLITE_DKDV_MIN_CHUNK")) {
    const int v = std::atoi(env);
    if (v >= 1) chmin = v;
  }
  return chmin;
}

// Launch the backward with its base workspace at ws (D, LSE*log2 e, key means,
// chunk plan, then pcap fp32 partial slots) and the stored-G_S part (NULL
// gsinfo: none).
int run_bwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const uint16_t* O, const uint16_t* O_lo,
            const uint16_t* dO, const float* lse_row, const int32_t* qcnt, const uint16_t* qidx,
            const int32_t* kcnt, const uint16_t* kidx, int B, int n, int H, int H_k, int d, float scale, int causal,
            int window, int q_tile, uint16_t* dQ, uint16_t* dK, uint16_t* dV, char* ws, int pcap, int32_t* gsinfo,
            uint32_t* qbase, uint32_t* kslot, uint16_t* gs, float* gsl, long long cap, void* stream,
            const char* what, float* dqacc = nullptr) {
  const size_t kbar_off = 2 * delta_bytes(B, H, n);
  const size_t plan_off = kbar_off + round256((size_t)B * H_k * ntiles(n) * d * sizeof(float));
  const size_t part_off = plan_off + dkplan_bytes(B, H_k, n);
  return hip_status(backlite::launch_bwd(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d,
                                         scale, causal ? 1 : 0, window, q_tile, dQ, dK, dV, (float*)ws,
                                         (float*)(ws + delta_bytes(B, H, n)), (float*)(ws + kbar_off), gsinfo, qbase,
                                         kslot, gs, gsl, cap, (int32_t*)(ws + plan_off), (float*)(ws + part_off),
                                         min_chunk(), pcap, dqacc, (hipStream_t)stream),
                    what);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free backward: one copy per GPU the library runs
// on, held until the process ends.  Host code never uses the array's name as
// an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)256 << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_for_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BACKLITE_ERR_UNSUPPORTED, "device index %d beyond the %d the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(BACKLITE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = (char*)g_scratch[dev];
  return BACKLITE_OK;
}

// partial slots a scratch of kScratchBytes leaves after the fixed parts; <= 0: too small
long long noalloc_partial_slots(int B, int H, int H_k, int n, int d) {
  const size_t fixed = 2 * delta_bytes(B, H, n) + round256((size_t)B * H_k * ntiles(n) * d * sizeof(float)) +
                       dkplan_bytes(B, H_k, n);
  if (fixed >= kScratchBytes) return 0;
  const long long NK = (long long)B * H_k * ntiles(n);
  const long long slots = (long long)((kScratchBytes - fixed) / ((size_t)2 * 128 * d * sizeof(float)));
  return slots < NK ? slots : NK;
}

}  // namespace

extern "C" {

int backlite_bwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const uint16_t* O,
                 const uint16_t* O_lo, const uint16_t* dO, const float* lse_row, const int32_t* qcnt, const uint16_t* qidx,
                 const int32_t* kcnt, const uint16_t* kidx, int B, int n, int H, int H_k, int d,
                 float scale, int causal, int window, int q_tile, uint16_t* dQ, uint16_t* dK, uint16_t* dV,
                 void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_bwd_args(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d, scale, causal, window,
                     q_tile, dQ, dK, dV));
  if (env_on("BACKLITE_CHECK")) {
    // validate copies of the lists on the host before anything is launched
    const size_t T = (size_t)ntiles(n), Tq = (size_t)ntiles(n, q_tile);
    const size_t nq = (size_t)B * H * Tq, nk = (size_t)B * H * T;
    std::vector<int32_t> qc(nq), kc(nk);
    std::vector<uint16_t> qi(nq * T), ki(nk * Tq);
    hipError_t e = hipMemcpyAsync(qc.data(), qcnt, nq * 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpyAsync(kc.data(), kcnt, nk * 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpyAsync(qi.data(), qidx, nq * T * 2, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpyAsync(ki.data(), kidx, nk * Tq * 2, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "BACKLITE_CHECK list readback");
    char msg[400];
    if (backlite_check_lists(qc.data(), qi.data(), kc.data(), ki.data(), B, H, n, causal, window, q_tile, msg,
                             sizeof(msg)) != BACKLITE_OK)
      return fail(BACKLITE_ERR_INVALID_ARG, "BACKLITE_CHECK: %s", msg);
  }
  const size_t need = backlite_bwd_workspace_bytes(B, H, H_k, n, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(BACKLITE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  TRY(check_ptr(workspace, "workspace"));
  char* ws = (char*)workspace;
  // stored-G_S slots when the workspace holds the index arrays and at least one slot
  int32_t* gsinfo = nullptr;
  uint32_t *qbase = nullptr, *kslot = nullptr;
  uint16_t* gs = nullptr;
  float* gsl = nullptr;
  long long cap = 0;
  const size_t idx = gs_index_bytes(B, H, n, q_tile), sb = slot_bytes(q_tile);
  if (workspace_bytes >= need + idx + sb) {
    const size_t Tq = (size_t)ntiles(n, q_tile);
    cap = (long long)((workspace_bytes - need - idx) / sb);
    if (cap > 0xffffffffLL) cap = 0xffffffffLL;  // slot indices are 32-bit
    gsinfo = (int32_t*)(ws + need);
    qbase = (uint32_t*)(ws + need + kStateBytes);
    kslot = (uint32_t*)(ws + need + kStateBytes + round256((size_t)B * H * Tq * 4));
    gs = (uint16_t*)(ws + need + idx);
    gsl = (float*)(ws + need + idx + (size_t)cap * q_tile * 128 * 2);
  }
  const int NK = B * H_k * ntiles(n);
  const int r = run_bwd(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d, scale, causal,
                        window, q_tile, dQ, dK, dV, ws, NK, gsinfo, qbase, kslot, gs, gsl, cap, stream,
                        "backlite_bwd launch");
  if (r == BACKLITE_OK && verbose()) {
    // which G_Q path served the kept tiles (a synchronous readback, debugging only)
    int32_t st[3] = {0, 0, 0};
    if (gsinfo) {
      hipError_t e = hipMemcpyAsync(st, gsinfo, sizeof(st), hipMemcpyDeviceToHost, (hipStream_t)stream);
      if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
      if (e != hipSuccess) return hip_status(e, "BACKLITE_VERBOSE readback");
      std::fprintf(stderr,
                   "[backlite] bwd B=%d H=%d H_k=%d n=%d d=%d: %lld G_S slots; %d kept tiles, %d with a slot; G_Q "
                   "from stored G_S for %s query tiles, recomputed for the rest\n",
                   B, H, H_k, n, d, cap, st[1], st[2], st[0] ? "all" : "a prefix of the");
    } else {
      std::fprintf(stderr, "[backlite] bwd B=%d H=%d H_k=%d n=%d d=%d: no G_S slots, G_Q recomputed\n", B, H, H_k,
                   n, d);
    }
  }
  return r;
}

size_t backlite_bwd_atomic_workspace_bytes(int B, int H, int H_k, int n, int d) {
  const size_t base = backlite_bwd_workspace_bytes(B, H, H_k, n, d);
  if (base == 0) return 0;
  return base + round256((size_t)B * H * ntiles(n) * kTile * d * sizeof(float));
}

int backlite_bwd_atomic(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const uint16_t* O,
                        const uint16_t* O_lo, const uint16_t* dO, const float* lse_row, const int32_t* qcnt,
                        const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n, int H,
                        int H_k, int d, float scale, int causal, int window, uint16_t* dQ, uint16_t* dK,
                        uint16_t* dV, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_bwd_args(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d, scale, causal, window,
                     kTile, dQ, dK, dV));
  const size_t need = backlite_bwd_atomic_workspace_bytes(B, H, H_k, n, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(BACKLITE_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  TRY(check_ptr(workspace, "workspace"));
  char* ws = (char*)workspace;
  const size_t base = backlite_bwd_workspace_bytes(B, H, H_k, n, d);
  return run_bwd(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d, scale, causal, window,
                 kTile, dQ, dK, dV, ws, B * H_k * ntiles(n), nullptr, nullptr, nullptr, nullptr, nullptr, 0, stream,
                 "backlite_bwd_atomic launch", (float*)(ws + base));
}

size_t backlite_bwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

int backlite_bwd_noalloc(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const uint16_t* O,
                         const uint16_t* O_lo, const uint16_t* dO, const float* lse_row, const int32_t* qcnt,
                         const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n, int H,
                         int H_k, int d, float scale, int causal, int window, int q_tile, uint16_t* dQ,
                         uint16_t* dK, uint16_t* dV, void* stream) {
  TRY(check_bwd_args(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d, scale, causal, window,
                     q_tile, dQ, dK, dV));
  const long long pcap = noalloc_partial_slots(B, H, H_k, n, d);
  if (pcap < 1)
    return fail(BACKLITE_ERR_WORKSPACE,
                "B=%d H=%d H_k=%d n=%d d=%d needs more than the %zu bytes of the allocation-free scratch "
                "(use backlite_bwd with a workspace)",
                B, H, H_k, n, d, kScratchBytes);
  char* ws = nullptr;
  TRY(scratch_for_current_device(&ws));
  return run_bwd(Q, K, V, O, O_lo, dO, lse_row, qcnt, qidx, kcnt, kidx, B, n, H, H_k, d, scale, causal, window,
                 q_tile, dQ, dK, dV, ws, (int)pcap, nullptr, nullptr, nullptr, nullptr, nullptr, 0, stream,
                 "backlite_bwd_noalloc launch");
}

size_t backlite_similarity_elems(void) { return backlite::similarity_elems(); }

int backlite_similarity_sums(const uint16_t* a, const uint16_t* b, int64_t m, double* out, void* stream) {
  if (m < 0) return fail(BACKLITE_ERR_INVALID_ARG, "element count must be >= 0 (got %lld)", (long long)m);
  TRY(check_ptr(a, "a"));
  TRY(check_ptr(b, "b"));
  TRY(check_ptr(out, "out"));
  return hip_status(backlite::launch_similarity(a, b, (long)m, out, (hipStream_t)stream), "backlite_similarity_sums");
}

const char* backlite_status_string(int status) {
  switch (status) {
    case BACKLITE_OK: return "ok";
    case BACKLITE_ERR_INVALID_ARG: return "invalid argument";
    case BACKLITE_ERR_UNSUPPORTED: return "unsupported configuration";
    case BACKLITE_ERR_WORKSPACE: return "workspace too small";
    case BACKLITE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* backlite_last_error(void) { return g_err; }

}  // extern "C"
