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
//   * a partial Fisher-Yates shuffle of the row's ascending candidate list;
//   * optionally, the page's last_idx limit: only blocks wholly inside the
//     first last_idx tokens are candidates (same stream, same shuffle), and a
//     plan built for a longer sequence serves a shorter one through its first
//     nb - 2 rows (bbsa_truncate_rand_attn).
#include <algorithm>
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

// Largest block a random pick may take: nb - 2 without a cap; with
// last_idx > 0 (tokens) only blocks wholly inside the first last_idx tokens,
// min(nb - 2, last_idx / block - 1).  Returns -1 for a cap without a block size.
int64_t cap_block(int nb, int block, int last_idx) {
  if (last_idx <= 0) return (int64_t)nb - 2;
  if (block < 1) return -1;
  return std::min<int64_t>((int64_t)nb - 2, (int64_t)(last_idx / block) - 1);
}

// Candidates of middle row i: ascending blocks 1..top outside {i-1, i, i+1}.
void candidates(int i, int64_t top, std::vector<int32_t> &cand) {
  cand.clear();
  for (int64_t c = 1; c <= top; ++c)
    if (c < i - 1 || c > i + 1) cand.push_back((int32_t)c);
}

int plan_impl(int32_t *rand_attn, int H, int nb, int r, uint64_t seed, int64_t top) {
  if (!rand_attn || H < 1 || nb < 1 || r < 1) return BBSA_ERR_ARG;
  if (nb < 5 + r) return BBSA_ERR_SHAPE;
  if (top < 0) return BBSA_ERR_ARG;
  std::vector<int32_t> cand;
  cand.reserve(nb);
  // Every middle row needs r candidates (a low cap can leave fewer).
  for (int i = 1; i <= nb - 2; ++i) {
    candidates(i, top, cand);
    if ((int64_t)cand.size() < r) return BBSA_ERR_SHAPE;
  }
  SplitMix64 rng(seed);
  for (int h = 0; h < H; ++h) {
    for (int i = 1; i <= nb - 2; ++i) {
      candidates(i, top, cand);
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

int check_impl(const int32_t *rand_attn, int H, int nb, int r, int64_t top) {
  if (!rand_attn || H < 1 || nb < 1 || r < 1) return BBSA_ERR_ARG;
  if (nb < 5 + r) return BBSA_ERR_SHAPE;
  if (top < 0) return BBSA_ERR_ARG;
  for (int h = 0; h < H; ++h) {
    for (int i = 1; i <= nb - 2; ++i) {
      const int32_t *row = rand_attn + ((int64_t)h * (nb - 2) + (i - 1)) * r;
      for (int t = 0; t < r; ++t) {
        const int32_t c = row[t];
        if (c < 1 || c > nb - 2 || c > top) return BBSA_ERR_PLAN;
        if (c >= i - 1 && c <= i + 1) return BBSA_ERR_PLAN;
        for (int u = 0; u < t; ++u)
          if (row[u] == c) return BBSA_ERR_PLAN;
      }
    }
  }
  return BBSA_OK;
}

}  // namespace

extern "C" int bbsa_plan_rand_attn(int32_t *rand_attn, int H, int nb, int r, uint64_t seed) {
  return plan_impl(rand_attn, H, nb, r, seed, (int64_t)nb - 2);
}

extern "C" int bbsa_plan_rand_attn_capped(int32_t *rand_attn, int H, int nb, int r, uint64_t seed,
                                          int block, int last_idx) {
  return plan_impl(rand_attn, H, nb, r, seed, cap_block(nb, block, last_idx));
}

extern "C" int bbsa_check_rand_attn(const int32_t *rand_attn, int H, int nb, int r) {
  return check_impl(rand_attn, H, nb, r, (int64_t)nb - 2);
}

extern "C" int bbsa_check_rand_attn_capped(const int32_t *rand_attn, int H, int nb, int r, int block,
                                           int last_idx) {
  return check_impl(rand_attn, H, nb, r, cap_block(nb, block, last_idx));
}

extern "C" int bbsa_truncate_rand_attn(const int32_t *src, int H, int nb_src, int r, int32_t *dst, int nb) {
  if (!src || !dst || H < 1 || r < 1 || nb < 3 || nb_src < nb) return BBSA_ERR_ARG;
  for (int h = 0; h < H; ++h)
    for (int i = 0; i < nb - 2; ++i)
      for (int t = 0; t < r; ++t)
        dst[((int64_t)h * (nb - 2) + i) * r + t] = src[((int64_t)h * (nb_src - 2) + i) * r + t];
  return check_impl(dst, H, nb, r, (int64_t)nb - 2);
}
