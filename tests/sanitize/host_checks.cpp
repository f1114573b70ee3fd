// Host-side checks of the C ABI built with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; no GPU is touched).
//
// Every call here returns before any HIP call: argument validation with
// null, negative, oversized and unsupported arguments; workspace sizing over
// the whole parameter space (the sequential carving of the layouts runs with
// a null base); the timing hook's argument checks; return-code texts.  A
// sanitizer report or a failed expectation exits non-zero.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "shampoo.h"

static int g_fail = 0;

#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
                   __LINE__, #cond);                                     \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

int main() {
  void* fake = reinterpret_cast<void*>(0x10000);  // never dereferenced on these paths
  float* ff = static_cast<float*>(fake);
  const shampoo_block* fb = static_cast<const shampoo_block*>(fake);
  shampoo_scale* fs = static_cast<shampoo_scale*>(fake);
  int32_t* fi = static_cast<int32_t*>(fake);
  const size_t big = size_t(1) << 40;

  // Workspace sizing: every op, precision and variant over a grid of B and counts.
  const int Bs[] = {0, 32, 63, 64, 100, 128, 192, 256, 640, 1024, 2048, 8192, 16384, 16448, -64};
  const int64_t counts[] = {-1, 0, 1, 7, 576, int64_t(1) << 20};
  for (int op = 0; op <= 7; ++op)
    for (int B : Bs)
      for (int64_t n : counts)
        for (int v = -1; v <= 300; v += 13)
          for (int prec = -1; prec <= 2; ++prec) {
            const size_t w = shampoo_workspace_bytes(op, n, B, v, prec);
            if (n < 0 || B < 64 || B > 16384 || B % 64 != 0) EXPECT(w == 0);
            (void)w;
          }
  const size_t s_ndb = shampoo_workspace_bytes(SHAMPOO_OP_NEWTON, 32, 256, SHAMPOO_NDB, SHAMPOO_F32);
  EXPECT(s_ndb >= size_t(5) * 32 * 256 * 256 * 4);
  EXPECT(shampoo_workspace_bytes(SHAMPOO_OP_NEWTON, 32, 256, SHAMPOO_NDB | SHAMPOO_SYM_COUPLING, SHAMPOO_F32) ==
         s_ndb);

  // Argument validation of every entry point.
  EXPECT(shampoo_accumulate(fb, -1, 64, ff, 0.9f, 0.1f, SHAMPOO_F32, nullptr, 0, nullptr) == SHAMPOO_EINVAL);
  EXPECT(shampoo_accumulate(fb, 2, 100, ff, 0.9f, 0.1f, SHAMPOO_F32, nullptr, 0, nullptr) == SHAMPOO_EUNSUPPORTED);
  EXPECT(shampoo_accumulate(fb, 2, 128, ff, 0.9f, 0.1f, SHAMPOO_BF16_IN, nullptr, 0, nullptr) ==
         SHAMPOO_EWORKSPACE);
  EXPECT(shampoo_accumulate(nullptr, 2, 64, ff, 0.9f, 0.1f, SHAMPOO_F32, nullptr, 0, nullptr) == SHAMPOO_EINVAL);
  EXPECT(shampoo_accumulate(nullptr, 0, 64, nullptr, 0.9f, 0.1f, SHAMPOO_F32, nullptr, 0, nullptr) == SHAMPOO_OK);
  EXPECT(shampoo_scale_power(ff, 4, 64, 0.f, SHAMPOO_SCALE_POWER, ff, 33, 20, 2.f, fs, fi, fake, big, nullptr) ==
         SHAMPOO_EINVAL);
  EXPECT(shampoo_scale_power(ff, 4, 64, -1.f, SHAMPOO_SCALE_FROBENIUS, nullptr, 0, 0, 0.f, fs, fi, fake, big,
                             nullptr) == SHAMPOO_EINVAL);
  EXPECT(shampoo_scale_power(ff, 4, 64, 0.f, SHAMPOO_SCALE_POWER, ff, 8, 20, 2.f, fs, fi, fake, 16, nullptr) ==
         SHAMPOO_EWORKSPACE);
  for (int variant = -2; variant <= 0x400; variant += 0x55)
    for (int p = -1; p <= 9; ++p)
      for (int iters : {-1, 0, 1, 100, 101}) {
        const int rc = shampoo_invroot_newton(ff, fs, 4, 64, p, variant, iters, ff, nullptr, fi, fake, 16, nullptr);
        EXPECT(rc != SHAMPOO_OK);  // a 16-byte workspace is never enough
      }
  EXPECT(shampoo_invroot_newton(ff, fs, 4, 64, 4, SHAMPOO_NDB, 5, ff, nullptr, fi, nullptr, big, nullptr) ==
         SHAMPOO_EWORKSPACE);
  EXPECT(shampoo_invroot_newton(nullptr, nullptr, 0, 64, 4, SHAMPOO_NDB, 5, nullptr, nullptr, nullptr, nullptr, 0,
                                nullptr) == SHAMPOO_OK);
  for (int degree : {-1, 0, 1, 256, 257})
    for (int prec : {int(SHAMPOO_F32), int(SHAMPOO_BF16_IN), 2, int(SHAMPOO_F32 | SHAMPOO_FULL_PRODUCTS)}) {
      const int rc = shampoo_invroot_cheby(ff, fs, 4, 192, 4, degree, 1e-12, prec, ff, fi, fake, 16, nullptr);
      EXPECT(rc != SHAMPOO_OK);
    }
  EXPECT(shampoo_invroot_cheby(ff, fs, 4, 64, 4, 8, -1.0, SHAMPOO_F32, ff, fi, fake, big, nullptr) == SHAMPOO_EINVAL);
  EXPECT(shampoo_precondition(ff, fb, 2, 64, fb, SHAMPOO_F32, fake, 16, nullptr) == SHAMPOO_EWORKSPACE);
  EXPECT(shampoo_precondition(ff, nullptr, 2, 64, fb, SHAMPOO_F32, fake, big, nullptr) == SHAMPOO_EINVAL);
  EXPECT(shampoo_graft_update(fb, fb, fb, fb, fb, 3, 128, 1e-3f, 0.9f, 0.999f, 1e-8f, 0, nullptr, fake, big,
                              nullptr) == SHAMPOO_EINVAL);
  EXPECT(shampoo_graft_update(fb, fb, fb, fb, fb, 3, 128, 1e-3f, 0.9f, 0.999f, 1e-8f, 1, nullptr, fake, 0,
                              nullptr) == SHAMPOO_EWORKSPACE);
  EXPECT(shampoo_graft_update_noalloc(fb, fb, fb, fb, fb, 8193, 1024, 1e-3f, 0.9f, 0.95f, 1e-8f, 1, nullptr,
                                      nullptr) == SHAMPOO_ESCRATCH);
  EXPECT(shampoo_graft_update_noalloc(fb, fb, fb, fb, fb, int64_t(1) << 40, 16384, 1e-3f, 0.9f, 0.95f, 1e-8f, 1,
                                      nullptr, nullptr) == SHAMPOO_EUNSUPPORTED);

  // Timing hook arguments and return-code texts.
  EXPECT(shampoo_timing_hook(SHAMPOO_TIME_ALL + 1, nullptr, nullptr, 4) == SHAMPOO_EINVAL);
  EXPECT(shampoo_timing_hook(SHAMPOO_TIME_NDB_P, nullptr, nullptr, 4) == SHAMPOO_EINVAL);
  EXPECT(shampoo_timing_hook(SHAMPOO_TIME_OFF, nullptr, nullptr, 0) == SHAMPOO_OK);
  EXPECT(shampoo_timing_count() == 0);
  for (int code = -8; code <= 2; ++code) EXPECT(std::strlen(shampoo_strerror(code)) > 0);
  EXPECT(shampoo_abi_version() == SHAMPOO_ABI_VERSION);

  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
