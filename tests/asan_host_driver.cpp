// Host-side exercise of the C ABI for an AddressSanitizer build of the library's host code
// (tests/test_asan_host.py builds it with the sanitizer on the host pass only and runs it with no
// GPU visible). Every call either is host arithmetic (the size queries, moe_saved_views,
// moe_status_str, moe_abi_version) or is rejected by the argument checks before any HIP call:
// shapes outside the limits, NULL or misaligned pointers, unknown dtypes and flags, a backward
// without saved activations. The pointers are placeholders that are never dereferenced.
// Exit status: the number of failed expectations (AddressSanitizer aborts on a memory error).
#include <stdint.h>
#include <stdio.h>

#include "moe_routed.h"

static int fails = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__);           \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

static void* const A = (void*)(uintptr_t)0x100000;  // 16-byte aligned placeholder
static void* const U = (void*)(uintptr_t)0x100001;  // misaligned placeholder

static moe_shape shape(int64_t T, int64_t D, int64_t F, int64_t E, int64_t K, int32_t dt,
                       int32_t flags) {
  moe_shape s;
  s.T = T; s.D = D; s.F = F; s.E = E; s.K = K; s.ids_dtype = dt; s.flags = flags;
  return s;
}

int main() {
  EXPECT(moe_abi_version() == MOE_ABI_VERSION);
  for (int st = -40; st <= 40; ++st) EXPECT(moe_status_str(st) != NULL);

  // size queries over a sweep of edge values: a rejected shape gives 0 for all three, an
  // accepted one a plan and a workspace
  const int64_t Ts[] = {-1, 0, 1, 2, 255, 256, 257, 4096, 1 << 20, (1LL << 25) - 1024, 1LL << 30};
  const int64_t Ws[] = {-64, 0, 32, 64, 100, 128, 7168, 32768, 1 << 22, (1 << 22) + 64};
  const int64_t Es[] = {-1, 0, 1, 8, 1024, 1025};
  const int64_t Ks[] = {-1, 0, 1, 2, 8, 64, 65};
  const int32_t dts[] = {MOE_IDS_I32, MOE_IDS_I64, 7};
  const int32_t fls[] = {0, MOE_SAVE_FOR_BACKWARD, MOE_SAVE_FOR_BACKWARD | MOE_RECOMPUTE,
                         MOE_KEEP_XG | MOE_WGRAD_F32 | MOE_WGRAD_ACCUMULATE, 1 << 12};
  long accepted = 0, total = 0;
  for (int64_t T : Ts)
    for (int64_t D : Ws)
      for (int64_t F : Ws)
        for (int64_t E : Es)
          for (int64_t K : Ks)
            for (int32_t dt : dts)
              for (int32_t fl : fls) {
                const moe_shape s = shape(T, D, F, E, K, dt, fl);
                const size_t pb = moe_plan_bytes(&s), sb = moe_saved_bytes(&s),
                             wb = moe_workspace_bytes(&s);
                ++total;
                if (pb == 0) {
                  EXPECT(sb == 0 && wb == 0);
                  // a rejected shape is rejected by every call, before its pointers matter
                  EXPECT(moe_plan(&s, A, A, 0, NULL) != MOE_OK);
                  EXPECT(moe_forward(&s, A, (const uint16_t*)A, (const float*)A,
                                     (const uint16_t*)A, (const uint16_t*)A, (uint16_t*)A, A, A,
                                     0, NULL) != MOE_OK);
                } else {
                  ++accepted;
                  EXPECT(wb > 0);
                  EXPECT((sb > 0) == ((fl & MOE_SAVE_FOR_BACKWARD) != 0));
                  // NULL plan and misaligned pointers are rejected for an accepted shape
                  EXPECT(moe_plan(&s, A, NULL, 0, NULL) == MOE_E_NULL);
                  EXPECT(moe_plan(&s, A, U, 0, NULL) == MOE_E_ALIGN);
                  EXPECT(moe_forward(&s, A, NULL, (const float*)A, (const uint16_t*)A,
                                     (const uint16_t*)A, (uint16_t*)A, A, A, 0, NULL) ==
                         MOE_E_NULL);
                  if (fl & MOE_SAVE_FOR_BACKWARD) {
                    uint16_t *xg = NULL, *h13 = NULL, *a = NULL, *y = NULL;
                    EXPECT(moe_saved_views(&s, A, &xg, &h13, &a, &y) == MOE_OK);
                    const uintptr_t lo = (uintptr_t)A, hi = lo + sb;
                    EXPECT((uintptr_t)y >= lo && (uintptr_t)y < hi);
                    if (xg) EXPECT((uintptr_t)xg >= lo && (uintptr_t)xg < hi);
                  } else {
                    EXPECT(moe_backward(&s, A, A, (const uint16_t*)A, (const uint16_t*)A,
                                        (const float*)A, (const uint16_t*)A, (const uint16_t*)A,
                                        (uint16_t*)A, A, A, (float*)A, A, 0, NULL) ==
                           MOE_E_STATE);
                  }
                }
              }
  printf("%ld shapes, %ld accepted, %d failed expectations\n", total, accepted, fails);
  EXPECT(accepted > 0 && accepted < total);
  return fails;
}
