/*
 * backlite.h — C ABI of the BackLite attention hot path for AMD MI355X (gfx950).
 *
 * BackLite ("Introducing BackLite: Attention Backpropagation Acceleration Using
 * Dynamic Sparsity", section "Using Sparsity"; BackLite README, "How It Works /
 * Sparse Backward Masking") runs an exact attention forward that also records
 * softmax statistics per tile, turns those statistics into a block-sparse tile
 * mask, and runs the attention backward over the kept tiles only.  This library
 * exposes the three stages as separate calls:
 *
 *   backlite_fwd   Q,K,V            -> O, LSE_row, tile_LSE
 *   backlite_mask  tile_LSE,LSE_row -> keep bitmap + per-tile work lists
 *   backlite_bwd   Q,K,V,O,G_O,LSE_row, lists -> G_Q, G_K, G_V
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates device memory and holds no state between calls; every
 *    call is re-entrant.  Inputs are never written.
 *  - bf16 tensors are passed as uint16_t bit patterns.  Q, O, G_O, G_Q are
 *    [B, n, H, d] and K, V, G_K, G_V are [B, n, H_k, d], contiguous, d
 *    fastest (the README's (batch, seq_len, heads, head_dim) layout).
 *  - Query head h reads key/value head h / (H / H_k) (grouped-query attention,
 *    README "Usage": key/value carry heads_k <= heads).
 *  - The forward's tiles are 128 query rows x 128 keys; T = ceil(n / 128).
 *    The backward's query tiles have q_tile rows, 128 or 64 (the README forms
 *    the mask "for each backward tile pair", "How It Works / Sparse Backward
 *    Masking", and a backward's tiles need not match the forward's; half-height
 *    query tiles give a finer mask); Tq = ceil(n / q_tile).  Key tiles stay 128.
 *  - All launches are asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  Argument validation is synchronous: a call that fails
 *    validation returns an error code and launches nothing.
 *  - Pointers must be non-NULL (except where stated) and 16-byte aligned.
 *  - Return value: BACKLITE_OK or a negative backlite_status.  The detail of
 *    the last failure on the calling thread is in backlite_last_error().
 *  - NaN/Inf inside tensors are not checked; they propagate.
 */
#ifndef BACKLITE_H
#define BACKLITE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BACKLITE_OK = 0,
  BACKLITE_ERR_INVALID_ARG = -1, /* a size, pointer, scale or probability is out of range */
  BACKLITE_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim not 64 or 128) */
  BACKLITE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than backlite_bwd_workspace_bytes */
  BACKLITE_ERR_HIP = -4          /* a HIP launch failed; hipError string in backlite_last_error() */
} backlite_status;

/* Number of float elements of the tile-LSE buffer backlite_fwd writes.
 * Layout: for each (b, h), one block of 128 floats per candidate tile pair
 * (qt, kt); float r of a block is the log-sum-exp of row 128*qt + r over the
 * keys of tile kt.  Non-causal: pair index qt*T + kt (T*T pairs).  Causal:
 * only pairs kt <= qt exist, pair index qt*(qt+1)/2 + kt (T*(T+1)/2 pairs).
 * Returns 0 for invalid sizes. */
size_t backlite_tile_lse_elems(int B, int H, int n, int causal);

/* Number of elements of each mask array: keep and qidx are [B, H, Tq, T],
 * kidx is [B, H, T, Tq] (Tq query tiles of q_tile rows).  0 for invalid sizes
 * or a q_tile other than 64 or 128. */
size_t backlite_mask_elems(int B, int H, int n, int q_tile);

/* Number of int32 elements of a count array over tiles of `tile` rows (64 or
 * 128): qcnt is [B, H, Tq] (tile = q_tile), kcnt is [B, H, T] (tile = 128). */
size_t backlite_count_elems(int B, int H, int n, int tile);

/* Bytes of device workspace backlite_bwd needs: the per-row D = rowsum(G_O*O)
 * values in fp32 [B, H, n], the row LSE times log2(e) in fp32 [B, H, n], the
 * per-key-tile mean of K in fp32 [B, H_k, T, d], the plan of the G_K/G_V
 * chunks (int32, 4 + 11 NK with NK = B*H_k*T), and fp32 partial sums for key
 * tiles whose lists are split over several workgroups (NK x 2 x 128 x d),
 * each part rounded up to 256 bytes.  0 for invalid sizes. */
size_t backlite_bwd_workspace_bytes(int B, int H, int H_k, int n, int d);

/* Bytes of a backward workspace that also holds slots for up to max_tiles
 * kept tile pairs, enabling the stored-G_S path of backlite_bwd (the G_K/G_V
 * pass keeps each kept tile's G_S = P * (G_P - D) in bf16, and G_Q = scale *
 * G_S K is then formed from the stored tiles instead of a second
 * recomputation of S, P and G_P; "Introducing BackLite", backward equations).
 * Layout after the base workspace: 256 bytes of state words, slot starts per
 * query tile uint32 [B, H, Tq], slots per k-list entry uint32 [B, H, T, Tq],
 * then the slots (each q_tile x 128 bf16 G_S, 32 or 16 KB, plus 4 x q_tile
 * fp32 sums of its rounding residual).  The workspace serves backward calls
 * with that q_tile.  Any workspace of at least the base size plus the state
 * and index arrays plus one slot enables the path.  Slots are dealt to the
 * kept tiles in query-tile order (b, h, qt, then q-list order); every query
 * tile whose kept tiles all received a slot takes its G_Q from the stored
 * tiles, and the remaining query tiles are recomputed.  So a slot budget
 * smaller than the kept tiles still serves a prefix of the query tiles, and
 * the choice is made on the device: the host reads nothing back.
 * max_tiles < 1 returns the base size. */
size_t backlite_bwd_workspace_bytes_stored(int B, int H, int H_k, int n, int d, int q_tile, int64_t max_tiles);

/* Byte offset, within a workspace enabling the stored path, of its state
 * words (int32): [0] = 1 if every kept tile of the last backlite_bwd on it had
 * a slot (G_Q came from stored G_S for every query tile), [1] = the kept tile
 * pairs it counted, [2] = how many of them had a slot.  Valid once that call
 * has completed on its stream. */
size_t backlite_bwd_state_offset(int B, int H, int H_k, int n, int d);

/* Forward: exact attention plus per-(row, key tile) statistics.
 *
 * ("Introducing BackLite", "Backpropagation for attention": S = scale*Q K^T,
 * P = row softmax(S), O = P V; README phase 1: the forward records the
 * log-sum-exp of every (query tile, key tile) alongside O and the full-row
 * LSE.)  Causal: key j is visible to query i iff j <= i.
 *
 *   Q [B,n,H,d], K, V [B,n,H_k,d] bf16 in; scale > 0 and finite (the usual
 *   choice is 1/sqrt(d)); causal 0/1.
 *   window >= 0: 0 = none; w > 0 (causal only, else BACKLITE_ERR_INVALID_ARG)
 *     is a sliding window, key j visible to query i iff i - w < j <= i (the
 *     blog's Nanochat runs, "Training Nanochat", mix such window layers with
 *     full causal ones).  tile_lse keeps the causal layout; entries of tile
 *     pairs wholly outside the window are left unwritten, and rows of a
 *     candidate tile that see none of its keys get -inf.  backlite_mask and
 *     backlite_bwd must be given the same window.  w >= n equals causal.
 *   O [B,n,H,d] bf16 out.
 *   O_lo [B,n,H,d] bf16 out, optional (may be NULL): the rounding residual
 *     bf16(O_fp32 - O) of the output, so that O + O_lo carries about 16
 *     significant bits.  backlite_bwd uses it for D = rowsum(G_O * O): an error
 *     in D shifts a whole row of G_S (whose row sum should vanish) and G_Q then
 *     picks up that shift times the keys' mean vector, which bf16 O alone makes
 *     visible (about 1% relative on keys with a large shared component).
 *   lse_row [B,H,n] fp32 out: natural-log LSE of each row of scale*Q K^T.
 *   tile_lse: fp32 out, backlite_tile_lse_elems() floats (layout above), the
 *     natural-log LSE of each row over one key tile.  Rows >= n of the last
 *     query tile are written as -inf.  May be NULL: then no statistics are
 *     written (the negl_prob = 0 dense mode).
 *   tile_w: fp64 out, optional (may be NULL; needs tile_lse): the compact
 *     statistics, backlite_tile_lse_elems() / 64 doubles: two per tile pair,
 *     in the pair layout of tile_lse, for the two 64-row halves of the query
 *     tile.  Entry (qt, kt, j) is the mask's log-weight of half j:
 *     max over its valid rows i of (tile_lse[i, kt] - lse_row[i]), formed in
 *     fp64 from the fp32 values the call writes, exactly as backlite_mask forms
 *     it (-inf for a half with no valid row); a 128-row query tile's weight is
 *     the larger of its two.  So backlite_mask_compact on tile_w selects the
 *     same tiles as backlite_mask on (tile_lse, lse_row), for either q_tile.
 *     tile_lse is then only staging: it may be reused once the call has run,
 *     and tile_w (64 rows reduced to one value, 32x fewer bytes) is what is
 *     kept until the backward.  Written for candidate pairs only.
 * Requires B, n, H, H_k >= 1, H % H_k == 0, d in {64, 128}. */
int backlite_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                 int B, int n, int H, int H_k, int d, float scale, int causal, int window,
                 uint16_t* O, uint16_t* O_lo, float* lse_row, float* tile_lse, double* tile_w,
                 void* stream);

/* Mask from statistics (README phase 2; "Using Sparsity").
 *
 * For every (b, h, query tile qt of q_tile rows: 128, or 64 for half-height
 * backward tiles) and candidate key tile kt (all kt; when causal, the key
 * tiles whose first key is at or before the query tile's last row; with a
 * sliding window w also kt >= the tile holding key (first row) - w + 1, i.e.
 * the tiles with a key inside some row's window):
 *   a(qt,kt) = max over valid rows i of tile qt of (tile_lse[i,kt] - lse_row[i]),
 *              computed in fp64 from the fp32 inputs; the tile weight is
 *              w = exp(a) = the largest p_tile = exp(LSE_tile - LSE_row) of the
 *              tile's rows;
 *   candidates are ordered by (a ascending, kt ascending); w is summed in fp64
 *   in that order, left to right; every tile whose running sum is still
 *   < negl_prob is skipped, every other candidate is kept.
 * Outputs (all written in full for every (b, h, tile)):
 *   keep [B,H,Tq,T] uint8: 1 = tile (qt, kt) is computed by the backward.
 *   qcnt [B,H,Tq] int32, qidx [B,H,Tq,T] uint16: for query tile qt, its kept
 *     key tiles in ascending order in qidx[..., qt, 0:qcnt]; the rest of the
 *     row is left unspecified.
 *   kcnt [B,H,T], kidx [B,H,T,Tq]: the same per key tile kt (kept query tiles,
 *     ascending).
 *   backlite_bwd must be given the same q_tile.
 *   stats: optional (may be NULL) int64[2], ACCUMULATED into (not cleared):
 *     [0] += candidate tile pairs, [1] += kept tile pairs.
 *   With the environment variable BACKLITE_VERBOSE=1 the call synchronises and
 *   prints the kept and candidate tile counts, the density, and the minimum,
 *   mean and maximum q-list and k-list lengths to stderr.
 * tile_lse may be NULL only with negl_prob == 0 (every candidate is kept).
 * negl_prob must be finite and in [0, 1); with negl_prob <= 1 every query tile
 * keeps at least one key tile. */
int backlite_mask(const float* tile_lse, const float* lse_row,
                  int B, int H, int n, int causal, int window, int q_tile, float negl_prob,
                  uint8_t* keep, int32_t* qcnt, uint16_t* qidx,
                  int32_t* kcnt, uint16_t* kidx, int64_t* stats, void* stream);

/* Block-sparse backward ("Introducing BackLite", backward equations and
 * "Using Sparsity"; README "How It Works": skipped tiles cost no loads and no
 * FLOPs):
 *   D = rowsum(G_O * O) over the full row, with O + O_lo when O_lo (the
 *     forward's optional residual output) is given, else O alone;
 *   for every kept tile pair: P = exp(scale*Q K^T - LSE_row) (causal-masked),
 *   G_V += P^T G_O, G_P = G_O V^T, G_S = P * (G_P - D),
 *   G_Q += scale * G_S K, G_K += scale * G_S^T Q.
 * Tiles absent from the lists contribute nothing.  G_K / G_V of a key/value
 * head sum over its query heads.  Every element of dQ, dK, dV is written (key
 * rows no list reaches get zeros).
 *   qcnt/qidx drive G_Q (per query tile); kcnt/kidx drive G_K, G_V (per key
 *   tile); both must describe the same tile set (as backlite_mask writes them
 *   with the same q_tile, 64 or 128: the query tiles' rows; with 64 the
 *   G_K/G_V pass takes two list items per 128-row step and the G_Q passes work
 *   on 64-row tiles).
 *   workspace: device buffer of at least backlite_bwd_workspace_bytes(); its
 *   contents on entry are ignored.  A larger one (see
 *   backlite_bwd_workspace_bytes_stored) enables the stored-G_S path, chosen
 *   on the device when every kept tile has a slot; both paths compute the
 *   same gradients (G_S rounded to bf16 for the G_Q product either way).
 * The G_K/G_V work of a key tile whose list is much longer than the average
 * (e.g. an attention-sink key tile kept by every query tile) is split over
 * several workgroups whose fp32 partial sums are added in a fixed order; the
 * environment variable BACKLITE_DKDV_MIN_CHUNK (default 16) sets the smallest
 * chunk length in tiles.
 * The result is deterministic (no atomics): repeated calls give identical bits.
 * Lists: the kernels read counts clamped to [0, T] and treat entries >= T as
 * empty tiles, so malformed lists cannot address memory outside the tensors;
 * they can still give wrong gradients.  With the environment variable
 * BACKLITE_CHECK=1 the call first copies the four lists to the host (a
 * synchronous readback) and validates them with backlite_check_lists, returning
 * BACKLITE_ERR_INVALID_ARG with the reason before launching anything.  With
 * BACKLITE_VERBOSE=1 it reports, after a synchronising readback, how many kept
 * tiles had a G_S slot. */
int backlite_bwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                 const uint16_t* O, const uint16_t* O_lo, const uint16_t* dO, const float* lse_row,
                 const int32_t* qcnt, const uint16_t* qidx,
                 const int32_t* kcnt, const uint16_t* kidx,
                 int B, int n, int H, int H_k, int d, float scale, int causal, int window, int q_tile,
                 uint16_t* dQ, uint16_t* dK, uint16_t* dV,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Fused single-pass variant of backlite_bwd with an fp32-atomic G_Q (the
 * FlashAttention-style alternative to a second pass over each query tile's
 * key tiles, "Flash Attention Backward Pass" of the tutorial computes dQ per
 * query block instead): the G_K/G_V pass also multiplies each kept tile's
 * G_S (bf16 hi + lo parts) by its K rows and adds the result to an fp32
 * accumulator with global atomics; a conversion pass writes G_Q = scale * acc
 * in bf16.  128-row query tiles only.  The atomics' order varies, so G_Q is
 * not bit-reproducible (G_K, G_V are, and equal backlite_bwd's).  workspace:
 * at least backlite_bwd_atomic_workspace_bytes() = the base workspace plus an
 * fp32 [B, H, 128 ceil(n/128), d] accumulator.  Other arguments, layouts and
 * errors as backlite_bwd.  Measured slower than backlite_bwd on the workloads
 * here (the accumulator's atomic traffic); kept as the measured alternative. */
size_t backlite_bwd_atomic_workspace_bytes(int B, int H, int H_k, int n, int d);
int backlite_bwd_atomic(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                        const uint16_t* O, const uint16_t* O_lo, const uint16_t* dO, const float* lse_row,
                        const int32_t* qcnt, const uint16_t* qidx,
                        const int32_t* kcnt, const uint16_t* kidx,
                        int B, int n, int H, int H_k, int d, float scale, int causal, int window,
                        uint16_t* dQ, uint16_t* dK, uint16_t* dV,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation as backlite_bwd with a workspace of the base
 * size (G_Q recomputed, no stored-G_S slots), but its workspace is a device
 * array inside the library, backlite_bwd_noalloc_scratch_bytes() = 256 MiB per
 * GPU, reserved when the library's code is loaded on that GPU and held until
 * the process ends.  The caller passes inputs and outputs only; the call makes
 * no hipMalloc / hipFree and no other device allocation.  The scratch belongs
 * to the calling thread's current device, which must be the stream's device.
 * Every call on a GPU shares that GPU's scratch and leaves its contents behind
 * (nothing in it needs to start at zero): calls that overlap on one GPU, on
 * different streams or from different threads, race and must be serialised by
 * the caller.  To fit the fixed scratch, split G_K/G_V lists are cut into
 * longer chunks when their fp32 partial sums would not fit (the results then
 * differ from backlite_bwd's by fp32 summation order; with no list split, or
 * where the partial slots fit, they are identical bit for bit).  Shapes whose
 * D, key-mean and plan arrays alone exceed the scratch return
 * BACKLITE_ERR_WORKSPACE before anything is launched.  BACKLITE_CHECK and
 * BACKLITE_VERBOSE are not consulted (their readbacks allocate host memory). */
size_t backlite_bwd_noalloc_scratch_bytes(void);
int backlite_bwd_noalloc(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                         const uint16_t* O, const uint16_t* O_lo, const uint16_t* dO, const float* lse_row,
                         const int32_t* qcnt, const uint16_t* qidx,
                         const int32_t* kcnt, const uint16_t* kidx,
                         int B, int n, int H, int H_k, int d, float scale, int causal, int window, int q_tile,
                         uint16_t* dQ, uint16_t* dK, uint16_t* dV, void* stream);

/* Mask from compact statistics: the tile_w output of backlite_fwd in place of
 * (tile_lse, lse_row); everything else as backlite_mask (q_tile 64 or 128),
 * and the same keep bitmap and lists for the same forward.  tile_w may be NULL only with
 * negl_prob == 0.  The pages speak of statistics per (query tile, key tile)
 * ("Using Sparsity") and report the method's small extra peak memory
 * ("Training Nanochat"); tile_w is that per-pair form, reduced inside the
 * forward from the per-row values. */
int backlite_mask_compact(const double* tile_w, int B, int H, int n, int causal, int window, int q_tile,
                          float negl_prob, uint8_t* keep, int32_t* qcnt, uint16_t* qidx,
                          int32_t* kcnt, uint16_t* kidx, int64_t* stats, void* stream);

/* Per-kernel timing (opt-in).  While enabled, every kernel the library
 * launches is bracketed by two hipEvents recorded on its launch stream.
 * backlite_profile_read waits for the outstanding events and returns, for the
 * named kernel, the accumulated elapsed time and the number of launches since
 * the last reset.  Kernel names: "fwd", "mask_select", "mask_transpose",
 * "delta", "kmean", "dkdv", "dq", "dk_plan" (the G_K/G_V chunk plan),
 * "dk_reduce" (sums of split chunks), "gs_slots" (slot assignment of the stored
 * path; "dkdv" and "dq" then also count the launch of the pass variant that
 * returns at once).  Process-wide state, thread-safe; enabling
 * adds two event records per launch.  read returns BACKLITE_ERR_INVALID_ARG
 * for an unknown name or NULL outputs, BACKLITE_ERR_HIP if an event failed. */
int backlite_profile_enable(int on);
int backlite_profile_reset(void);
int backlite_profile_read(const char* kernel, double* total_ms, int64_t* launches);

/* Validation of work lists held in HOST memory (plain C++, no GPU needed):
 * the form backlite_mask writes and backlite_bwd expects.  qcnt [B, H, Tq],
 * qidx [B, H, Tq, Tk], kcnt [B, H, Tk], kidx [B, H, Tk, Tq], with Tq =
 * ceil(n / q_tile) query tiles of q_tile rows (64 or 128) and Tk = ceil(n / 128)
 * key tiles.  Checks: counts within [0, Tq] / [0, Tk]; lists strictly
 * ascending with entries below Tk / Tq; every q-list pair a candidate (causal:
 * the key tile's first key <= the query tile's last row; window w > 0: its
 * last key > the query tile's first row - w, as in "Introducing BackLite",
 * "Training Nanochat", sliding-window layers); the k-lists holding exactly the
 * q-lists' pairs.  Returns BACKLITE_OK, or BACKLITE_ERR_INVALID_ARG with the
 * first violation described in msg (msg_len bytes, may be NULL / 0). */
int backlite_check_lists(const int32_t* qcnt, const uint16_t* qidx, const int32_t* kcnt,
                         const uint16_t* kidx, int B, int H, int n, int causal, int window,
                         int q_tile, char* msg, size_t msg_len);

/* Sums behind the gradient-similarity metrics of negl_prob calibration
 * ("Introducing BackLite", "Experiments": BackLite's gradients are compared
 * with exact attention's by cosine similarity and relative L2): for bf16
 * device tensors a, b of m elements, out[0..3] = sum a*b, sum a*a, sum b*b,
 * sum (a-b)^2, in fp64 (each product in fp32).  out is a device fp64 buffer of
 * backlite_similarity_elems() doubles; past out[3] it is scratch.  Deterministic
 * (fixed partial sums, added in order); asynchronous on stream. */
size_t backlite_similarity_elems(void);
int backlite_similarity_sums(const uint16_t* a, const uint16_t* b, int64_t m, double* out, void* stream);

/* Static text for a status code. */
const char* backlite_status_string(int status);

/* Detail of the last failing call on the calling thread ("" if none). */
const char* backlite_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BACKLITE_H */
