// The attention probabilities of the BigBird block-sparse pattern as a dense
// [B, H, L, L] fp32 matrix: exact zeros outside the pattern, the row softmax
// of the attended keys inside it.
//
// What is produced ("BigBirdPegasus 长序列条件生成模型详解…", section
// "三类注意力组合全局 局部 随机": the sparse attention weights are scattered back
// into a full (bsz, n_heads, seq_len, seq_len) matrix when the caller asks
// for the attention outputs; section "使用限制与注意事项": most of that matrix
// is zero).  The scores, padding bias, options (query x key masking, a length
// padded to the block) and pattern are those of bbsa_forward_ex.
//
// An inspection path: one workgroup of 256 threads per 64-row query tile,
// fp32 arithmetic on the vector units with the key block staged in LDS.  Four
// threads share a query row, each taking every fourth group of four keys.
// Per row, three passes over the attended key blocks: the largest padding
// bias (the "level", so that a row whose keys all share one mask value keeps
// full fp32 precision instead of rounding s - 10000), the running max and
// sum of exp(s + bias - level), then the probabilities.  Blocks outside the
// pattern are written as zeros in the last pass.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bbsa.h"
#include "bbsa_schedule.h"

namespace {

using namespace bbsa_sched;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 64;            // query rows per workgroup
constexpr int kKPad = kD + 1;        // LDS row pitch of the key block (no bank conflicts)
constexpr float kPadBias = -10000.0f;
constexpr float kLog2e = 1.4426950408889634f;

struct ProbParams {
  const void *q, *k;
  const float *mask;        // [B, L] or null
  const int32_t *rand_attn; // [H, nb-2, r] (null on the fallback)
  float *probs;             // [B, H, L, L]
  int B, H, L, nb, block, r;
  int full;                 // every key block attended
  int qk;                   // query x key masking
  int bf16;                 // element type of q and k
};

__device__ inline float load_elem(const void *base, int64_t i, bool bf16) {
  if (bf16) return (float)((const __bf16 *)base)[i];
  return ((const float *)base)[i];
}

// Does query block i attend key block j?  ("models 仓库中的 BigBird…", section
// "BigBird：从二次方注意力到线性稀疏注意力": global rows and columns, the
// 3-block window, the row's plan entries.)
__device__ inline bool attends(const ProbParams &p, const int32_t *plan_row, int i, int j) {
  if (p.full || i == 0 || i == p.nb - 1 || j == 0 || j == p.nb - 1 || (j >= i - 1 && j <= i + 1)) return true;
  for (int t = 0; t < p.r; ++t)
    if (min(max(plan_row[t], 0), p.nb - 1) == j) return true;
  return false;
}

__global__ __launch_bounds__(kThreads) void bbsa_probs_kernel(ProbParams p) {
  __shared__ float ks[128 * kKPad];          // one key block (up to 128 keys), fp32
  const int qtiles = p.block / kRows;
  const int wg = (int)blockIdx.x;
  const int qt = wg % qtiles;
  const int i = (wg / qtiles) % p.nb;        // query block
  const int bh = wg / (qtiles * p.nb);
  const int b = bh / p.H, h = bh % p.H;
  const int tid = (int)threadIdx.x;
  const int row = tid >> 2, sub = tid & 3;
  const int t = i * p.block + qt * kRows + row;           // query token
  const bool row_live = t < p.L;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = p.mask ? p.mask + (int64_t)b * p.L : nullptr;
  const int32_t *plan_row = (!p.full && i >= 1 && i <= p.nb - 2)
                                ? p.rand_attn + ((int64_t)h * (p.nb - 2) + (i - 1)) * p.r
                                : nullptr;

  // The query row in registers (row L - 1 stands in for rows past L).
  float qv[kD];
  {
    const int tr = row_live ? t : p.L - 1;
#pragma unroll
    for (int e = 0; e < kD; ++e) qv[e] = load_elem(p.q, bh * seq + (int64_t)tr * kD + e, p.bf16);
  }
  // Query side of the bias: with query x key masking the key bias is scaled
  // by the query's mask value (the rest is a per-row constant).
  const float fq = p.qk ? (row_live && mrow ? mrow[t] : 0.0f) : 1.0f;
  // Key bias (relative to nothing yet) of key u; positions past L are padding.
  auto key_bias = [&](int u) -> float {
    const float m = u < p.L ? (mrow ? mrow[u] : 1.0f) : 0.0f;
    return fq * (kPadBias * (1.0f - m));
  };
  const int kpb = p.block / 16;              // key groups of 4 per thread per block: keys 16 g + 4 sub + e

  // Stage key block j in LDS as fp32 (rows past L as zeros).
  auto stage = [&](int j) {
    __syncthreads();
    for (int x = tid; x < p.block * kD; x += kThreads) {
      const int kr = x / kD, e = x % kD;
      const int u = j * p.block + kr;
      ks[kr * kKPad + e] = u < p.L ? load_elem(p.k, bh * seq + (int64_t)u * kD + e, p.bf16) : 0.0f;
    }
    __syncthreads();
  };
  auto score = [&](int kr) -> float {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < kD; ++e) acc = __builtin_fmaf(qv[e], ks[kr * kKPad + e], acc);
    return acc;
  };
  // Combine a value across the four threads of a row.
  auto row_max = [&](float x) {
    x = fmaxf(x, __shfl_xor(x, 1));
    return fmaxf(x, __shfl_xor(x, 2));
  };
  auto row_sum = [&](float x) {
    x += __shfl_xor(x, 1);
    return x + __shfl_xor(x, 2);
  };

  // Pass 0: the row's bias level (largest bias among its attended keys).
  float level = -3.0e38f;
  for (int j = 0; j < p.nb; ++j) {
    if (!attends(p, plan_row, i, j)) continue;
    for (int g = 0; g < kpb; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) level = fmaxf(level, key_bias(j * p.block + 16 * g + 4 * sub + e));
  }
  level = row_max(level);

  // Pass 1: running max and sum of exp(s + bias - level).
  float m = -3.0e38f, l = 0.0f;
  for (int j = 0; j < p.nb; ++j) {
    if (!attends(p, plan_row, i, j)) continue;
    stage(j);
    for (int g = 0; g < kpb; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kr = 16 * g + 4 * sub + e;
        const float s = score(kr) + (key_bias(j * p.block + kr) - level);
        if (s > m) {
          l *= exp2f((m - s) * kLog2e);
          m = s;
        }
        l += exp2f((s - m) * kLog2e);
      }
  }
  const float M = row_max(m);
  l *= exp2f((m - M) * kLog2e);
  const float inv = 1.0f / row_sum(l);

  // Pass 2: the probabilities of attended blocks, zeros elsewhere.
  float *prow = p.probs + ((int64_t)bh * p.L + (row_live ? t : 0)) * p.L;
  const bool vec = (p.L % 4) == 0;           // whole 16-byte stores when rows stay aligned
  for (int j = 0; j < p.nb; ++j) {
    const bool att = attends(p, plan_row, i, j);
    if (att) stage(j);
    for (int g = 0; g < kpb; ++g) {
      const int kr0 = 16 * g + 4 * sub;
      const int u0 = j * p.block + kr0;
      f32x4 pv = {0.f, 0.f, 0.f, 0.f};
      if (att) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = score(kr0 + e) + (key_bias(u0 + e) - level);
          pv[e] = exp2f((s - M) * kLog2e) * inv;
        }
      }
      if (!row_live) continue;
      if (vec && u0 + 3 < p.L) {
        *(f32x4 *)(prow + u0) = pv;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (u0 + e < p.L) prow[u0 + e] = pv[e];
      }
    }
  }
}

}  // namespace

extern "C" int bbsa_attention_probs(const void *q, const void *k, const float *mask, const int32_t *rand_attn,
                                    int B, int H, int L, int d, int block, int r, float *probs,
                                    hipStream_t stream, bbsa_dtype dtype, unsigned flags) {
  // Same validation as the forward (q and k stand in for v and out).
  Launch ln;
  const int st = setup_forward_ex(q, k, q, mask, rand_attn, B, H, L, d, block, r, (void *)q, nullptr, (int)dtype,
                                  flags, &ln);
  if (st < 0) return st;
  if (!probs || ((uintptr_t)probs & 3)) return BBSA_ERR_ARG;
  const Params &fp = ln.p;
  const int64_t grid = (int64_t)B * H * fp.nb * fp.qtiles;
  if (grid > 0x7fffffff) return BBSA_ERR_UNSUPPORTED;
  ProbParams p;
  p.q = q; p.k = k; p.mask = mask; p.rand_attn = ln.full ? nullptr : rand_attn; p.probs = probs;
  p.B = B; p.H = H; p.L = L; p.nb = fp.nb; p.block = block; p.r = r;
  p.full = ln.full ? 1 : 0;
  p.qk = (fp.mode & kModeQK) ? 1 : 0;
  p.bf16 = dtype == BBSA_BF16 ? 1 : 0;
  hipLaunchKernelGGL(bbsa_probs_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  return st;
}
