// Host-side checks of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer (built with the sanitizers on the host code only; no GPU needed):
// the chunk planner over ordinary and extreme shapes, and the argument checks
// of every entry point, which must return before any GPU work.  Prints "ok"
// and exits 0, or names the first failed check and exits 1.
#include <stdint.h>
#include <stdio.h>

#include "ckl.h"

static int g_fail = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      g_fail = 1;                                                    \
    }                                                                \
  } while (0)

int main() {
  // planner: every plan fits its budget, chunks are within N
  const int64_t Ns[] = {0, 1, 2, 255, 256, 257, 4096, 32768, 131072, 262144, (int64_t)1 << 31};
  const int64_t ds[] = {8, 256, 2880, 3072, (int64_t)1 << 20};
  const int64_t Vs[] = {1, 127, 128, 129, 32000, 201088, (int64_t)1 << 26};
  const int64_t Ks[] = {1, 100, 2048};
  const uint64_t budgets[] = {0, 1ull << 20, 6ull << 30, ~0ull >> 8};
  const int64_t chunks[] = {0, 1, 256, 8192, (int64_t)1 << 31};
  int planned = 0;
  for (int64_t N : Ns)
    for (int64_t d : ds)
      for (int64_t V : Vs)
        for (int64_t K : Ks)
          for (uint64_t b : budgets)
            for (int pass = 0; pass < 3; ++pass)
              for (int dt = 0; dt < 2; ++dt)
                for (int64_t c : chunks) {
                  int64_t C = -1;
                  uint64_t bytes = 0;
                  const int st = ckl_plan_pass(pass, N, d, V, K, dt, c, b, &C, &bytes);
                  if (K > V) CHECK(st == CKL_EINVAL);
                  if (st == CKL_OK && N == 0) {
                    CHECK(C == 0 && bytes == 0);  // an empty batch: no chunk, no workspace
                  } else if (st == CKL_OK) {
                    ++planned;
                    CHECK(C >= 1 && C <= N);
                    if (c > 0) CHECK(C == (c < N ? c : N));
                    CHECK(C <= ((int64_t)1 << 20));
                    if (b != 0) CHECK(bytes <= b);
                  } else {
                    CHECK(st == CKL_EINVAL || st == CKL_EBUDGET || st == CKL_EUNSUPPORTED);
                  }
                  if (pass == 0 && c == 0) {
                    int64_t C2 = -1;
                    uint64_t bytes2 = 0;
                    CHECK(ckl_plan(N, d, V, K, dt, b, &C2, &bytes2) == st);
                    if (st == CKL_OK) CHECK(C2 == C && bytes2 == bytes);
                  }
                }
  CHECK(planned > 1000);
  CHECK(ckl_plan(64, 8, 10, 2, 7, 0, nullptr, nullptr) == CKL_EINVAL);
  CHECK(ckl_plan_pass(3, 64, 8, 10, 2, 0, 0, 0, nullptr, nullptr) == CKL_EINVAL);
  CHECK(ckl_plan(-5, 8, 10, 2, 0, 0, nullptr, nullptr) == CKL_EINVAL);
  CHECK(ckl_plan(64, 12, 10, 2, 0, 0, nullptr, nullptr) == CKL_EUNSUPPORTED);
  CHECK(ckl_plan(64, 8, ((int64_t)1 << 26) + 1, 2, 0, 0, nullptr, nullptr) == CKL_EUNSUPPORTED);

  // argument checks: fake, never dereferenced pointers; each call must return
  // its error before touching the GPU
  void* g = (void*)(uintptr_t)(1 << 20);
  void* mis = (void*)(uintptr_t)((1 << 20) + 2);
  const int32_t* ids = (const int32_t*)g;
  const float* tl = (const float*)g;
  float* fo = (float*)g;
  CHECK(ckl_fwd_bwd(nullptr, g, ids, tl, nullptr, 4, 8, 10, 2, 0, fo, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd_bwd(g, mis, ids, tl, nullptr, 4, 8, 10, 2, 0, fo, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd_bwd(g, g, ids, tl, nullptr, 4, 8, 10, 11, 0, fo, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd_bwd(g, g, ids, tl, nullptr, 4, 8, 10, 2, -1, fo, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd_bwd(g, g, ids, tl, nullptr, 4, 8, 10, 2, 0, nullptr, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd_bwd_f32(fo, fo, ids, tl, nullptr, 4, 12, 10, 2, 0, fo, fo, fo, nullptr) == CKL_EUNSUPPORTED);
  CHECK(ckl_fwd_bwd_f32(fo, fo, ids, tl, nullptr, 4, 8, 10, 4000, 0, fo, fo, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd_bwd_ex(2, g, g, ids, tl, nullptr, 4, 8, 10, 2, 0, fo, g, fo, nullptr, nullptr, nullptr) ==
        CKL_EINVAL);
  CHECK(ckl_fwd_bwd_ex(0, g, g, ids, tl, nullptr, 4, 8, 10, 2, 0, fo, g, fo, (float*)mis, nullptr, nullptr) ==
        CKL_EINVAL);
  CHECK(ckl_fwd_bwd_noalloc(0, g, g, ids, tl, nullptr, 256, 2880, 201088, 100, 0, fo, g, fo, nullptr, nullptr,
                            nullptr) == CKL_EBUDGET);
  CHECK(ckl_fwd(0, g, g, ids, tl, nullptr, 4, 8, 10, 2, 0, fo, nullptr, nullptr, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd(1, g, g, ids, tl, nullptr, (int64_t)1 << 40, 8, 10, 2, 0, fo, fo, nullptr, nullptr) ==
        CKL_EUNSUPPORTED);
  CHECK(ckl_bwd(0, g, g, ids, tl, nullptr, nullptr, nullptr, 4, 8, 10, 2, 0, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_bwd(0, g, g, ids, tl, nullptr, fo, (const float*)mis, 4, 8, 10, 2, 0, g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_topk(0, nullptr, 4, 10, 2, (int32_t*)g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_topk(0, nullptr, 0, 10, 2, nullptr, nullptr, nullptr) == CKL_OK);  // no rows: nothing to do
  CHECK(ckl_topk(0, g, -1, 10, 2, (int32_t*)g, fo, nullptr) == CKL_EINVAL);
  // an empty batch still needs W and the outputs it writes
  CHECK(ckl_fwd_bwd(nullptr, g, nullptr, nullptr, nullptr, 0, 8, 10, 2, 0, fo, nullptr, nullptr, nullptr) ==
        CKL_EINVAL);
  CHECK(ckl_fwd_bwd(nullptr, g, nullptr, nullptr, nullptr, 0, 8, 10, 11, 0, fo, nullptr, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_fwd(0, nullptr, g, nullptr, nullptr, nullptr, 0, 8, 10, 2, 0, nullptr, nullptr, nullptr, nullptr) ==
        CKL_EINVAL);
  CHECK(ckl_bwd(0, nullptr, g, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 8, 10, 2, 0, nullptr, nullptr,
                nullptr) == CKL_EINVAL);
  CHECK(ckl_topk(0, g, 4, 5000, 3000, (int32_t*)g, fo, nullptr) == CKL_EUNSUPPORTED);
  CHECK(ckl_topk(0, g, 4, 10, 11, (int32_t*)g, fo, nullptr) == CKL_EINVAL);
  CHECK(ckl_debug_rows(nullptr, ids, tl, nullptr, 4, 10, 2, 1.f, 1, fo, (int32_t*)g, g, fo, fo, nullptr) ==
        CKL_EINVAL);
  CHECK(ckl_debug_rows(fo, ids, tl, nullptr, 4, ((int64_t)1 << 26) + 1, 2, 1.f, 1, fo, (int32_t*)g, g, fo, fo,
                       nullptr) == CKL_EUNSUPPORTED);
  double t = 0;
  int64_t n = 0;
  CHECK(ckl_timing_query(99, &t, &n) == CKL_EINVAL);
  CHECK(ckl_timing_query(0, nullptr, &n) == CKL_EINVAL);
  for (int s = -6; s <= 1; ++s) CHECK(ckl_strerror(s) != nullptr);
  CHECK(ckl_workspace_bytes_held() == 0);
  ckl_release_workspace();
  if (g_fail) return 1;
  printf("ok (%d plans)\n", planned);
  return 0;
}
