// Host-only driver for the sanitizer build of the library's host code (the
// chunk planner, argument validation, pool sizing, head-chunk picking and
// every entry point's error paths). It never reaches a kernel launch: every
// call either is host-only or fails validation first. Exits non-zero on a
// wrong status; AddressSanitizer / UndefinedBehaviorSanitizer abort on
// their own findings.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/upipe_attn.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main() {
  void* fake = reinterpret_cast<void*>(0x10000);
  // pool sizes over a grid of shapes, valid and not
  const int64_t Ss[] = {-1, 0, 1, 63, 64, 65, 1000, 131072, 5242880, (1ll << 24) - 1, 1ll << 24, 1ll << 40};
  const int hs[] = {-1, 0, 1, 2, 3, 4, 6, 8, 64};
  for (int64_t S : Ss)
    for (int Hq : hs)
      for (int Hkv : hs)
        for (int hc : hs)
          for (int d : {32, 64, 96, 128})
            for (int dt : {-1, 0, 1, 2}) {
              const size_t f = upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, hc, dt);
              const size_t b = upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, hc, dt);
              const size_t w = upipe_attn_workspace_bytes(S, Hq, Hkv, d, hc, dt);
              EXPECT(w == (f > b ? f : b));
              if (!f) EXPECT(std::strlen(upipe_last_error()) > 0);
              (void)upipe_attn_block_fwd_workspace_bytes(S, Hq * 64, Hq, Hkv, d, hc);
            }
  // the chunk plan
  int32_t q0[64], kv0[64], nkv[64], fl[64];
  for (int Hq : hs)
    for (int Hkv : hs)
      for (int hc : hs) {
        const int n = upipe_attn_plan(Hq, Hkv, hc, 64, q0, kv0, nkv, fl);
        if (n > 0) {
          EXPECT(n == Hq / hc);
          for (int c = 0; c < n; ++c) EXPECT(q0[c] == c * hc && kv0[c] >= 0 && kv0[c] < Hkv);
        }
        EXPECT(upipe_attn_plan(Hq, Hkv, hc, 0, nullptr, nullptr, nullptr, nullptr) <= 0 || Hq / hc == 0);
      }
  // head-chunk picking
  EXPECT(upipe_attn_pick_head_chunk(5242880, 8, 1, 128, 0, (size_t)1 << 50) == 8);
  EXPECT(upipe_attn_pick_head_chunk(5242880, 8, 1, 128, 0, 1) == UPIPE_EWORKSPACE);
  EXPECT(upipe_attn_pick_head_chunk(0, 8, 1, 128, 0, 1) == UPIPE_EINVAL);
  // error paths of every entry point (nothing reaches the device)
  EXPECT(upipe_attn_fwd(fake, fake, fake, fake, nullptr, (float*)fake, 0, 4, 1, 128, 1, 1, 0, fake, 1 << 30, nullptr) ==
         UPIPE_EINVAL);
  EXPECT(upipe_attn_fwd(fake, fake, fake, fake, nullptr, (float*)fake, 256, 4, 1, 128, 1, 1, 0, fake, 16, nullptr) ==
         UPIPE_EWORKSPACE);
  EXPECT(upipe_attn_bwd(fake, fake, fake, fake, nullptr, fake, (float*)fake, nullptr, fake, fake, 256, 4, 1, 128, 1,
                        1, 0, fake, (size_t)1 << 40, nullptr) == UPIPE_EINVAL);
  EXPECT(upipe_attn_fwd_docs(fake, fake, fake, fake, nullptr, (float*)fake, 256, 4, 1, 128, 1, 1, nullptr, 0, 0, fake,
                             (size_t)1 << 40, nullptr) == UPIPE_EINVAL);
  EXPECT(upipe_attn_bwd_docs(fake, fake, fake, fake, nullptr, fake, (float*)fake, fake, fake, fake, 256, 4, 1, 128, 1,
                             1, (const int32_t*)fake, -3, 0, fake, (size_t)1 << 40, nullptr) == UPIPE_EINVAL);
  EXPECT(upipe_attn_fwd_noalloc(fake, fake, fake, fake, nullptr, (float*)fake, 1 << 20, 4, 1, 128, 1, 1, 0, nullptr) ==
         UPIPE_EWORKSPACE);
  EXPECT(upipe_attn_block_fwd(fake, fake, fake, fake, fake, (float*)fake, nullptr, (float*)fake, 256, 100, 4, 1, 128, 1,
                              1, fake, (size_t)1 << 40, nullptr) == UPIPE_EUNSUPPORTED);
  EXPECT(upipe_gemm_bf16(fake, 64, 0, 0, 1, fake, 64, 0, 0, 1, fake, 64, 0, 0, 1, 0, 64, 64, 100, nullptr) ==
         UPIPE_EUNSUPPORTED);
  EXPECT(upipe_ce_loss_tiled(fake, fake, (const int32_t*)fake, (float*)fake, nullptr, nullptr, 1000, 128, 1001, 128,
                             1.f, fake, (size_t)1 << 40, nullptr) == UPIPE_EUNSUPPORTED);
  EXPECT(upipe_ce_loss_workspace_bytes(1000, 128, 1000, 100, 1) == 0);
  // timing bookkeeping with nothing recorded
  EXPECT(upipe_profile_enable(0) == UPIPE_OK);
  int total = -1;
  EXPECT(upipe_profile_completed(&total) == 0 && total == 0);
  EXPECT(upipe_profile_read(0, nullptr, nullptr, nullptr) == 0);
  upipe_profile_reset();
  std::printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
