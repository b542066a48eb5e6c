// Test driver for backlite_check_lists under the address and undefined-
// behaviour sanitizers (host code only).  Each argument is a case file:
// int32 header {B, H, n, causal, window, expect_ok}, then qcnt int32 [B,H,T],
// qidx uint16 [B,H,T,T], kcnt int32 [B,H,T], kidx uint16 [B,H,T,T] (T = key
// tiles of 128 = query tiles of 128).  Prints "ok <file>" when the verdict is
// the expected one, and exits non-zero otherwise.
#include <cstdio>
#include <vector>

#include "backlite.h"

int main(int argc, char** argv) {
  int bad = 0;
  for (int a = 1; a < argc; ++a) {
    FILE* f = std::fopen(argv[a], "rb");
    if (!f) {
      std::printf("cannot open %s\n", argv[a]);
      return 2;
    }
    int hdr[6];
    if (std::fread(hdr, sizeof(int), 6, f) != 6) return 2;
    const int B = hdr[0], H = hdr[1], n = hdr[2], causal = hdr[3], window = hdr[4], expect_ok = hdr[5];
    const size_t T = (size_t)(n + 127) / 128, nc = (size_t)B * H * T;
    std::vector<int32_t> qc(nc), kc(nc);
    std::vector<uint16_t> qi(nc * T), ki(nc * T);
    bool rd = std::fread(qc.data(), 4, nc, f) == nc && std::fread(qi.data(), 2, nc * T, f) == nc * T &&
              std::fread(kc.data(), 4, nc, f) == nc && std::fread(ki.data(), 2, nc * T, f) == nc * T;
    std::fclose(f);
    if (!rd) return 2;
    char msg[256];
    const int rc = backlite_check_lists(qc.data(), qi.data(), kc.data(), ki.data(), B, H, n, causal, window, 128,
                                        msg, sizeof(msg));
    if ((rc == BACKLITE_OK) == (expect_ok != 0)) {
      std::printf("ok %s\n", argv[a]);
    } else {
      std::printf("MISMATCH %s: rc %d (%s)\n", argv[a], rc, msg);
      bad = 1;
    }
  }
  return bad;
}
