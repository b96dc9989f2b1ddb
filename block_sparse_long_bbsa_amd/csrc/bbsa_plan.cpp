// Host planner for the BigBird random-block adjacency (rand_attn).
//
// The pages ("models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
// section "随机块掩码是如何生成的") fix what the plan must satisfy: each middle
// query block row gets num_rand_blocks key blocks drawn from the middle block
// indices with the row's own 3-block window removed, fixed per head when the
// layer is built, seeded by the layer index.  They draw with numpy's
// permutation; this planner uses a fully specified stream instead so the plan
// is reproducible bit for bit:
//   * SplitMix64 (Steele, Lea & Flood, OOPSLA 2014), one stream per seed,
//     consumed head by head, row by row, pick by pick;
//   * exactly uniform bounded draws by rejection of outputs below 2^64 mod m;
//   * a partial Fisher-Yates shuffle of the row's ascending candidate list.
#include <cstdint>
#include <vector>

#include "bbsa.h"

namespace {

struct SplitMix64 {
  uint64_t state;
  explicit SplitMix64(uint64_t seed) : state(seed) {}
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  // Uniform in [0, m), m >= 1.  (0 - m) % m == 2^64 mod m in unsigned arithmetic.
  uint64_t below(uint64_t m) {
    const uint64_t reject_below = (0 - m) % m;
    for (;;) {
      const uint64_t x = next();
      if (x >= reject_below) return x % m;
    }
  }
};

}  // namespace

extern "C" int bbsa_plan_rand_attn(int32_t *rand_attn, int H, int nb, int r, uint64_t seed) {
  if (!rand_attn || H < 1 || nb < 1 || r < 1) return BBSA_ERR_ARG;
  if (nb < 5 + r) return BBSA_ERR_SHAPE;
  SplitMix64 rng(seed);
  std::vector<int32_t> cand;
  cand.reserve(nb);
  for (int h = 0; h < H; ++h) {
    for (int i = 1; i <= nb - 2; ++i) {
      cand.clear();
      for (int c = 1; c <= nb - 2; ++c)
        if (c < i - 1 || c > i + 1) cand.push_back(c);
      const uint64_t n = cand.size();
      int32_t *row = rand_attn + ((int64_t)h * (nb - 2) + (i - 1)) * r;
      for (int t = 0; t < r; ++t) {
        const uint64_t j = (uint64_t)t + rng.below(n - (uint64_t)t);
        const int32_t tmp = cand[t];
        cand[t] = cand[j];
        cand[j] = tmp;
        row[t] = cand[t];
      }
    }
  }
  return BBSA_OK;
}

extern "C" int bbsa_check_rand_attn(const int32_t *rand_attn, int H, int nb, int r) {
  if (!rand_attn || H < 1 || nb < 1 || r < 1) return BBSA_ERR_ARG;
  if (nb < 5 + r) return BBSA_ERR_SHAPE;
  for (int h = 0; h < H; ++h) {
    for (int i = 1; i <= nb - 2; ++i) {
      const int32_t *row = rand_attn + ((int64_t)h * (nb - 2) + (i - 1)) * r;
      for (int t = 0; t < r; ++t) {
        const int32_t c = row[t];
        if (c < 1 || c > nb - 2) return BBSA_ERR_PLAN;
        if (c >= i - 1 && c <= i + 1) return BBSA_ERR_PLAN;
        for (int u = 0; u < t; ++u)
          if (row[u] == c) return BBSA_ERR_PLAN;
      }
    }
  }
  return BBSA_OK;
}
