// Host-side validation of the backward's work lists (plain C++, no HIP).
//
// The backward trusts its q-lists and k-lists: every entry names a tile whose
// rows it loads.  backlite_check_lists verifies, on host copies, what
// backlite_mask guarantees by construction (BackLite README, "How It Works /
// Sparse Backward Masking": the mask selects, per query tile, a subset of the
// key tiles the attention pattern allows):
//   - every count lies in [0, number of tiles of the other side];
//   - every list is strictly ascending and names existing tiles;
//   - every q-list entry is a candidate pair: with causal attention the key
//     tile's first key is at or before the query tile's last row, and with a
//     sliding window w its last key is after the query tile's first row - w;
//   - the k-lists hold exactly the pairs of the q-lists.
// It is compiled into libbacklite.so (backlite_bwd runs it on copies of the
// lists when BACKLITE_CHECK=1) and, on its own, into the sanitizer test build.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <vector>

#include "backlite.h"

namespace {

constexpr int kKeyTile = 128;

int report(char* msg, size_t len, const char* fmt, ...) {
  if (msg != nullptr && len > 0) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(msg, len, fmt, ap);
    va_end(ap);
  }
  return BACKLITE_ERR_INVALID_ARG;
}

}  // namespace

extern "C" int backlite_check_lists(const int32_t* qcnt, const uint16_t* qidx, const int32_t* kcnt,
                                    const uint16_t* kidx, int B, int H, int n, int causal, int window,
                                    int q_tile, char* msg, size_t msg_len) {
  if (msg != nullptr && msg_len > 0) msg[0] = '\0';
  if (qcnt == nullptr || qidx == nullptr || kcnt == nullptr || kidx == nullptr)
    return report(msg, msg_len, "a list pointer is NULL");
  if (B < 1 || H < 1 || n < 1) return report(msg, msg_len, "B, H, n must be >= 1");
  if (q_tile != 64 && q_tile != 128) return report(msg, msg_len, "q_tile must be 64 or 128 (got %d)", q_tile);
  if (window < 0 || (window > 0 && !causal)) return report(msg, msg_len, "invalid window %d", window);
  const long Tq = (n + q_tile - 1) / q_tile;
  const long Tk = (n + kKeyTile - 1) / kKeyTile;
  const long w = (window > 0 && window < n) ? window : 0;
  std::vector<uint8_t> pair((size_t)(Tq * Tk));
  for (long bh = 0; bh < (long)B * H; ++bh) {
    const long b = bh / H, h = bh % H;
    std::fill(pair.begin(), pair.end(), 0);
    long total = 0;
    for (long qt = 0; qt < Tq; ++qt) {
      const long c = qcnt[bh * Tq + qt];
      if (c < 0 || c > Tk)
        return report(msg, msg_len, "qcnt[b=%ld, h=%ld, qt=%ld] = %ld is outside [0, %ld]", b, h, qt, c, Tk);
      const uint16_t* row = qidx + (bh * Tq + qt) * Tk;
      const long first_row = qt * q_tile;
      const long last_row = (qt + 1) * q_tile - 1 < n - 1 ? (qt + 1) * q_tile - 1 : n - 1;
      for (long i = 0; i < c; ++i) {
        const long kt = row[i];
        if (kt >= Tk)
          return report(msg, msg_len, "q-list (b=%ld, h=%ld, qt=%ld) entry %ld = %ld is not a key tile (< %ld)",
                        b, h, qt, i, kt, Tk);
        if (i > 0 && kt <= (long)row[i - 1])
          return report(msg, msg_len, "q-list (b=%ld, h=%ld, qt=%ld) is not strictly ascending at entry %ld",
                        b, h, qt, i);
        const long first_key = kt * kKeyTile;
        const long last_key = (kt + 1) * kKeyTile - 1 < n - 1 ? (kt + 1) * kKeyTile - 1 : n - 1;
        if (causal && first_key > last_row)
          return report(msg, msg_len, "pair (qt=%ld, kt=%ld) of (b=%ld, h=%ld) lies above the causal diagonal",
                        qt, kt, b, h);
        if (w && last_key <= first_row - w)
          return report(msg, msg_len, "pair (qt=%ld, kt=%ld) of (b=%ld, h=%ld) lies outside the window %ld", qt,
                        kt, b, h, w);
        pair[(size_t)(qt * Tk + kt)] = 1;
      }
      total += c;
    }
    long ktotal = 0;
    for (long kt = 0; kt < Tk; ++kt) {
      const long c = kcnt[bh * Tk + kt];
      if (c < 0 || c > Tq)
        return report(msg, msg_len, "kcnt[b=%ld, h=%ld, kt=%ld] = %ld is outside [0, %ld]", b, h, kt, c, Tq);
      const uint16_t* col = kidx + (bh * Tk + kt) * Tq;
      for (long i = 0; i < c; ++i) {
        const long qt = col[i];
        if (qt >= Tq)
          return report(msg, msg_len, "k-list (b=%ld, h=%ld, kt=%ld) entry %ld = %ld is not a query tile (< %ld)",
                        b, h, kt, i, qt, Tq);
        if (i > 0 && qt <= (long)col[i - 1])
          return report(msg, msg_len, "k-list (b=%ld, h=%ld, kt=%ld) is not strictly ascending at entry %ld",
                        b, h, kt, i);
        if (!pair[(size_t)(qt * Tk + kt)])
          return report(msg, msg_len, "k-list (b=%ld, h=%ld, kt=%ld) holds qt=%ld, which that q-list lacks", b,
                        h, kt, qt);
      }
      ktotal += c;
    }
    if (ktotal != total)
      return report(msg, msg_len, "(b=%ld, h=%ld): the q-lists hold %ld pairs, the k-lists %ld", b, h, total,
                    ktotal);
  }
  return BACKLITE_OK;
}
