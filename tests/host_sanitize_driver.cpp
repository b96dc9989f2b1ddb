// Host-only driver for the AddressSanitizer / UndefinedBehaviorSanitizer
// build of the library's host code (tests/test_host_sanitizers.py builds it
// with g++ together with csrc/bbsa_plan.cpp and csrc/bbsa_host.cpp).
//
// It exercises, without any GPU: the planner and the plan checker over a
// grid of shapes and seeds (plus planted violations); the argument
// validation and launch sizing of bbsa_forward (setup_forward) on valid,
// invalid and extreme arguments; and the work-map query, which runs the
// kernels' item mapping and key-list construction on the host.  Any
// sanitizer report aborts the process with a non-zero status; the driver
// itself prints "ok" and returns 0 when every check holds.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "bbsa.h"
#include "bbsa_schedule.h"

using namespace bbsa_sched;

static int g_fail = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static void planner() {
  for (int H : {1, 3, 12})
    for (int nb : {6, 9, 16, 64, 257})
      for (int r : {1, 2, 3, 5, 20})
        for (uint64_t seed : {0ull, 1ull, 0xffffffffffffffffull}) {
          if (nb < 5 + r) {
            std::vector<int32_t> ra(1);
            CHECK(bbsa_plan_rand_attn(ra.data(), H, nb, r, seed) == BBSA_ERR_SHAPE);
            continue;
          }
          std::vector<int32_t> ra((size_t)H * (nb - 2) * r, -7);
          CHECK(bbsa_plan_rand_attn(ra.data(), H, nb, r, seed) == BBSA_OK);
          CHECK(bbsa_check_rand_attn(ra.data(), H, nb, r) == BBSA_OK);
          ra[ra.size() / 2] = nb - 1;   // a global block is never a random pick
          CHECK(bbsa_check_rand_attn(ra.data(), H, nb, r) == BBSA_ERR_PLAN);
        }
  int32_t one = 0;
  CHECK(bbsa_plan_rand_attn(nullptr, 1, 8, 1, 0) == BBSA_ERR_ARG);
  CHECK(bbsa_plan_rand_attn(&one, 0, 8, 1, 0) == BBSA_ERR_ARG);
  CHECK(bbsa_plan_rand_attn(&one, 1, 8, 0, 0) == BBSA_ERR_ARG);
  CHECK(bbsa_plan_rand_attn(&one, 1, INT_MIN, 1, 0) == BBSA_ERR_ARG);
  CHECK(bbsa_check_rand_attn(nullptr, 1, 8, 1) == BBSA_ERR_ARG);
  CHECK(bbsa_check_rand_attn(&one, 1, 4, 1) == BBSA_ERR_SHAPE);
}

static void validation() {
  void *const P = (void *)(uintptr_t)4096;
  const int32_t *ra = (const int32_t *)(uintptr_t)4096;
  Launch ln;
  struct Case {
    int B, H, L, d, block, r, dtype, want;
  };
  const Case cases[] = {
      {4, 12, 4096, 64, 64, 3, BBSA_BF16, BBSA_OK},
      {1, 16, 32768, 64, 128, 2, BBSA_BF16, BBSA_OK},
      {1, 2, 1024, 64, 64, 3, BBSA_F32, BBSA_OK},
      {1, 2, 704, 64, 64, 3, BBSA_BF16, BBSA_OK_FULL_FALLBACK},
      {1, 1, 64, 64, 64, 1, BBSA_F32, BBSA_OK_FULL_FALLBACK},
      {0, 1, 1024, 64, 64, 3, BBSA_BF16, BBSA_ERR_ARG},
      {1, 1, 1024, 64, 64, 0, BBSA_BF16, BBSA_ERR_ARG},
      {1, 1, 1000, 64, 64, 3, BBSA_BF16, BBSA_ERR_SHAPE},
      {1, 1, 1024, 128, 64, 3, BBSA_BF16, BBSA_ERR_UNSUPPORTED},
      {1, 1, 1024, 64, 32, 3, BBSA_BF16, BBSA_ERR_UNSUPPORTED},
      {1, 1, 1024, 64, 64, 3, 7, BBSA_ERR_UNSUPPORTED},
      {1, 1, 8192, 64, 64, 60, BBSA_BF16, BBSA_ERR_UNSUPPORTED},
      {INT_MAX, INT_MAX, INT_MAX - 1, 64, 64, 3, BBSA_BF16, BBSA_ERR_SHAPE},
      {INT_MAX, INT_MAX, INT_MAX - 63, 64, 64, 3, BBSA_BF16, BBSA_ERR_UNSUPPORTED},
      {INT_MAX, INT_MAX, 1 << 20, 64, 64, 3, BBSA_BF16, BBSA_ERR_UNSUPPORTED},
      {1, 1, (1 << 24) + 64, 64, 64, 3, BBSA_BF16, BBSA_ERR_UNSUPPORTED},
      {1, 1, 1 << 24, 64, 64, 3, BBSA_BF16, BBSA_OK},   // 4096-key chunks: chunks * nb = 2^30
      {1, 1, 11 << 20, 64, 64, 3, BBSA_BF16, BBSA_OK},
      {1, 1, 1 << 23, 64, 64, 3, BBSA_F32, BBSA_ERR_UNSUPPORTED},   // 256-key chunks: chunks * nb = 2^32
      {1, 1, 5 << 20, 64, 64, 3, BBSA_F32, BBSA_OK},
      {1, 1, INT_MAX, 64, 64, INT_MAX, BBSA_BF16, BBSA_ERR_SHAPE},
      {1, 1, 1 << 20, 64, 128, INT_MAX / 128, BBSA_BF16, BBSA_OK_FULL_FALLBACK},
  };
  for (const Case &c : cases) {
    const int st = setup_forward(P, P, P, nullptr, ra, c.B, c.H, c.L, c.d, c.block, c.r, P, c.dtype, &ln);
    if (st != c.want)
      std::fprintf(stderr, "setup B%d H%d L%d d%d block%d r%d dtype%d: got %d want %d\n", c.B, c.H, c.L, c.d,
                   c.block, c.r, c.dtype, st, c.want);
    CHECK(st == c.want);
  }
  // bbsa_forward_ex: flags, ragged lengths, lse alignment.
  float *const lse = (float *)(uintptr_t)4096;
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, 1000, 64, 64, 3, P, lse, 0, 0u, &ln) == BBSA_ERR_SHAPE);
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, 1000, 64, 64, 3, P, lse, 0, 1u, &ln) == BBSA_OK);
  CHECK(ln.p.nb == 16 && ln.p.L == 1000 && (ln.p.mode & kModeRagged));
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, 1000, 64, 64, 3, P, lse, 0, 8u, &ln) == BBSA_ERR_ARG);
  CHECK(setup_forward_ex(P, P, P, (const float *)P, ra, 1, 1, 1024, 64, 64, 3, P, lse, 0, 2u, &ln) == BBSA_OK);
  CHECK(ln.p.mode == (kModeMask | kModeQK));
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, 1024, 64, 64, 3, P, lse, 0, 2u, &ln) == BBSA_OK);
  CHECK(ln.p.mode == 0);   // query x key masking without a mask: nothing to do
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, 1024, 64, 64, 3, P, (float *)(uintptr_t)4098, 0, 0u, &ln) ==
        BBSA_ERR_ARG);
  CHECK(setup_forward_ex(P, P, P, nullptr, nullptr, 1, 1, 700, 64, 64, 3, P, nullptr, 0, 1u, &ln) ==
        BBSA_OK_FULL_FALLBACK);
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, (1 << 23) - 1, 64, 64, 3, P, nullptr, BBSA_F32, 1u, &ln) ==
        BBSA_ERR_UNSUPPORTED);   // chunks * nb >= 2^31
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, (1 << 24) - 1, 64, 64, 3, P, nullptr, 0, 1u, &ln) == BBSA_OK);
  CHECK(ln.p.chunks * ln.p.nb == (1 << 30));
  CHECK(setup_forward_ex(P, P, P, nullptr, ra, 1, 1, (1 << 24) + 1, 64, 64, 3, P, nullptr, 0, 1u, &ln) ==
        BBSA_ERR_UNSUPPORTED);   // L > 2^24
  // Null and misaligned pointers.
  void *const M = (void *)(uintptr_t)4104;
  CHECK(setup_forward(nullptr, P, P, nullptr, ra, 1, 1, 1024, 64, 64, 3, P, 0, &ln) == BBSA_ERR_ARG);
  CHECK(setup_forward(P, P, P, nullptr, ra, 1, 1, 1024, 64, 64, 3, nullptr, 0, &ln) == BBSA_ERR_ARG);
  CHECK(setup_forward(M, P, P, nullptr, ra, 1, 1, 1024, 64, 64, 3, P, 0, &ln) == BBSA_ERR_ARG);
  CHECK(setup_forward(P, P, P, (const float *)M, ra, 1, 1, 1024, 64, 64, 3, P, 0, &ln) == BBSA_ERR_ARG);
  CHECK(setup_forward(P, P, P, nullptr, nullptr, 1, 1, 1024, 64, 64, 3, P, 0, &ln) == BBSA_ERR_ARG);
  CHECK(setup_forward(P, P, P, nullptr, nullptr, 1, 1, 704, 64, 64, 3, P, 0, &ln) == BBSA_OK_FULL_FALLBACK);
  CHECK(setup_forward(P, P, P, nullptr, ra, 1, 1, 1024, 64, 64, 3, P, 0, nullptr) == BBSA_ERR_ARG);
  // The largest accepted bf16 shape: the last chunk of a full row still has
  // in-range block bounds, computed with the kernels' arithmetic.
  CHECK(setup_forward(P, P, P, nullptr, ra, 1, 1, 11 << 20, 64, 64, 3, P, 0, &ln) == BBSA_OK);
  {
    const Params &p = ln.p;
    Item it{0, p.nb - 1, 0, 1, p.chunks - 1};
    for (int lane = 0; lane < 64; ++lane) {
      int rnd = 0, rslot = -1;
      KeyWalk w = make_walk_base(p, it, lane, rnd, rslot);
      CHECK(w.blk >= 0 && w.blk < p.nb);
      CHECK(w.n_steps > 0);
    }
  }
}

static void work_maps() {
  struct Shape {
    int B, H, L, block, r, dtype;
  };
  const Shape shapes[] = {{4, 12, 4096, 64, 3, BBSA_BF16}, {1, 16, 32768, 128, 2, BBSA_BF16},
                          {2, 12, 16384, 64, 3, BBSA_BF16}, {1, 2, 1024, 64, 3, BBSA_F32},
                          {3, 3, 1024, 64, 2, BBSA_BF16},   {1, 2, 128, 64, 1, BBSA_BF16},
                          {1, 1, 2880, 64, 20, BBSA_BF16}};
  for (const Shape &s : shapes) {
    const int nb = s.L / s.block;
    std::vector<int32_t> plan((size_t)s.H * (nb > 2 ? nb - 2 : 1) * s.r, 1);
    const bool full = s.L <= (5 + 2 * s.r) * s.block;
    if (!full) CHECK(bbsa_plan_rand_attn(plan.data(), s.H, nb, s.r, 11) == BBSA_OK);
    int64_t count = 0, grid = 0;
    int st = bbsa_work_map(s.B, s.H, s.L, 64, s.block, s.r, (bbsa_dtype)s.dtype, 0u, full ? nullptr : plan.data(),
                           nullptr, 0, &count, &grid);
    CHECK(st >= 0 && count > 0 && grid > 0);
    std::vector<int32_t> rec((size_t)count * BBSA_WORK_RECORD_INTS);
    // A buffer one record short: the query must not write past it.
    int64_t count2 = 0, grid2 = 0;
    st = bbsa_work_map(s.B, s.H, s.L, 64, s.block, s.r, (bbsa_dtype)s.dtype, 0u, full ? nullptr : plan.data(),
                       rec.data(), count - 1, &count2, &grid2);
    CHECK(st >= 0 && count2 == count && grid2 == grid);
    st = bbsa_work_map(s.B, s.H, s.L, 64, s.block, s.r, (bbsa_dtype)s.dtype, 0u, full ? nullptr : plan.data(),
                       rec.data(), count, &count2, &grid2);
    CHECK(st >= 0);
    for (int64_t i = 0; i < count; ++i) {
      const int32_t *r = rec.data() + i * BBSA_WORK_RECORD_INTS;
      CHECK(r[3] >= 0 && r[3] < s.B * s.H);
      for (int t = r[8]; t < r[9]; ++t) CHECK(r[16 + t] >= 0 && r[16 + t] < nb);
    }
  }
  int64_t c = 0, g = 0;
  CHECK(bbsa_work_map(1, 1, 1024, 64, 64, 3, BBSA_BF16, 0u, nullptr, nullptr, 0, nullptr, &g) == BBSA_ERR_ARG);
  CHECK(bbsa_work_map(1, 1, 1024, 64, 64, 3, BBSA_BF16, 0u, nullptr, nullptr, 0, &c, &g) == BBSA_ERR_ARG);
}

int main() {
  planner();
  validation();
  work_maps();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
