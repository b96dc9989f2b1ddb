// Backward pass of the BigBird block-sparse attention for fp32 inputs: dQ,
// dK, dV in fp32.
//
// What is computed is the bf16 backward's ("models 仓库中的 BigBird…", section
// "梯度检查点的实现方式": the operator is trained through and its forward is
// recomputed; "BigBirdPegasus…", section "使用限制与注意事项": the sparse
// probability matrix carries no gradient of its own): with P the masked row
// softmax of the scores plus bias over the forward's pattern, out = P V and
// dO the gradient of out,
//   D = rowsum(dO * out),  dV = P^T dO,  dS = P * (dO V^T - D),
//   dQ = dS K,  dK = dS^T Q.
//
// A parity path on the vector units, in fp32 throughout: one thread per
// query row (dq) or per key row (dk, dv), 64 rows per workgroup, the other
// side's rows staged in LDS and read as broadcasts.  Each query row's
// normaliser is recomputed here relative to its padding-bias level (the
// largest bias among its attended keys, as the fp32 forward does), so a row
// whose keys all share one mask value keeps full fp32 precision; the
// forward's lse is not read.
//
// Kernels:
//   * bbsa_bwd_f32_rows: per query row, three passes over the row's key list
//     (the forward's): the bias level, the running max and sum (the log2
//     normaliser), then dq = sum_u P_tu (dP_tu - D_t) k_u.  It also stores
//     D_t and (level_t, normaliser_t) for the column kernels;
//   * bbsa_bwd_f32_cols<DK>: per key row u of block j, every query block i
//     whose key list holds j (with its multiplicity in that list), all its
//     rows t: dv_u += P_tu dO_t, or dk_u += P_tu (dP_tu - D_t) q_t.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bbsa.h"
#include "bbsa_schedule.h"

namespace {

using namespace bbsa_sched;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kR = 64;                 // rows per workgroup, one thread each
constexpr int kPitch = kD + 4;         // LDS row pitch in floats (16-byte aligned rows)
constexpr float kPadBias = -10000.0f;
constexpr float kLog2e = 1.4426950408889634f;

struct F32Params {
  const float *q, *k, *v, *o, *dout;
  const float *mask;         // [B, L] or null
  const int32_t *rand_attn;  // [H, nb-2, r] or null (fallback)
  float *dq, *dk, *dv, *delta;
  float *rowterm;            // [B, H, L][2]: bias level, log2 normaliser relative to it
  int B, H, L, nb, block, r;
  int full;                  // every block attends every block
  int qk;                    // query x key masking
};

__device__ inline float mask_at(const F32Params &p, const float *mrow, int pos) {
  return pos < p.L ? (mrow ? mrow[pos] : 1.0f) : 0.0f;
}

// Length of query block i's key list, and its entry t (the forward's blocks:
// every block for a global row or on the fallback; else the two global
// blocks, the window without them in ascending order, the plan's blocks,
// clamped).
__device__ inline int list_len(const F32Params &p, int i) {
  if (p.full || i == 0 || i == p.nb - 1) return p.nb;
  return 2 + ((i == 1 || i == p.nb - 2) ? 2 : 3) + p.r;
}
__device__ inline int list_entry(const F32Params &p, const int32_t *plan_row, int i, int t) {
  if (p.full || i == 0 || i == p.nb - 1) return t;
  if (t == 0) return 0;
  if (t == 1) return p.nb - 1;
  const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
  const int w0 = (i == 1) ? 1 : i - 1;
  if (t < 2 + nw) return w0 + (t - 2);
  return min(max(plan_row[t - 2 - nw], 0), p.nb - 1);
}
__device__ inline const int32_t *plan_row_of(const F32Params &p, int h, int i) {
  if (p.full || i == 0 || i == p.nb - 1) return nullptr;
  return p.rand_attn + ((int64_t)h * (p.nb - 2) + (i - 1)) * p.r;
}

// 64 rows of a [L, 64] fp32 matrix into LDS (rows at or past L as zeros).
__device__ inline void stage_rows(float *dst, const float *src, int L, int row0, int tid) {
  for (int x = tid; x < kR * (kD / 4); x += kR) {
    const int rr = x / (kD / 4), c4 = x % (kD / 4);
    const int row = row0 + rr;
    f32x4 val = {0.f, 0.f, 0.f, 0.f};
    if (row < L) val = *(const f32x4 *)(src + (int64_t)row * kD + 4 * c4);
    *(f32x4 *)(dst + rr * kPitch + 4 * c4) = val;
  }
}
__device__ inline float dot_lds(const float (&x)[kD], const float *row) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < kD; e += 4) {
    const f32x4 y = *(const f32x4 *)(row + e);
    acc = __builtin_fmaf(x[e], y[0], acc);
    acc = __builtin_fmaf(x[e + 1], y[1], acc);
    acc = __builtin_fmaf(x[e + 2], y[2], acc);
    acc = __builtin_fmaf(x[e + 3], y[3], acc);
  }
  return acc;
}
__device__ inline void axpy_lds(float (&acc)[kD], float a, const float *row) {
#pragma unroll
  for (int e = 0; e < kD; e += 4) {
    const f32x4 y = *(const f32x4 *)(row + e);
    acc[e] = __builtin_fmaf(a, y[0], acc[e]);
    acc[e + 1] = __builtin_fmaf(a, y[1], acc[e + 1]);
    acc[e + 2] = __builtin_fmaf(a, y[2], acc[e + 2]);
    acc[e + 3] = __builtin_fmaf(a, y[3], acc[e + 3]);
  }
}
__device__ inline void load_row(float (&x)[kD], const float *src, int L, int row) {
#pragma unroll
  for (int e = 0; e < kD; e += 4) {
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (row < L) y = *(const f32x4 *)(src + (int64_t)row * kD + e);
    x[e] = y[0]; x[e + 1] = y[1]; x[e + 2] = y[2]; x[e + 3] = y[3];
  }
}
__device__ inline void store_row(float *dst, int L, int row, const float (&x)[kD]) {
  if (row >= L) return;
#pragma unroll
  for (int e = 0; e < kD; e += 4) *(f32x4 *)(dst + (int64_t)row * kD + e) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};
}

// Workgroup w: query tile (64 rows) w % tiles of query block (w / tiles) % nb
// of pair w / (tiles * nb).
__global__ __launch_bounds__(kR) void bbsa_bwd_f32_rows(F32Params p) {
  __shared__ __attribute__((aligned(16))) float ks[kR * kPitch];
  __shared__ __attribute__((aligned(16))) float vs[kR * kPitch];
  __shared__ float kbias[kR];   // 1 - mask of the staged keys
  const int tiles = p.block / kR;
  const int wg = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int i = (wg / tiles) % p.nb;
  const int bh = wg / (tiles * p.nb);
  const int b = bh / p.H, h = bh % p.H;
  const int t = i * p.block + (wg % tiles) * kR + tid;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = p.mask ? p.mask + (int64_t)b * p.L : nullptr;
  const int32_t *plan_row = plan_row_of(p, h, i);
  const int n = list_len(p, i);

  float q[kD], dO[kD];
  load_row(q, p.q + bh * seq, p.L, t);
  load_row(dO, p.dout + bh * seq, p.L, t);
  float D;
  {
    float o[kD];
    load_row(o, p.o + bh * seq, p.L, t);
    D = 0.0f;
#pragma unroll
    for (int e = 0; e < kD; ++e) D = __builtin_fmaf(dO[e], o[e], D);
  }
  // Bias of key u for this row: mq * kPadBias * (1 - m_u).
  const float mq = p.qk ? mask_at(p, mrow, t) : 1.0f;
  const float cb = mq * kPadBias;

  // Pass 0: the bias level (the largest bias among the attended keys).
  float level = -3.0e38f;
  for (int x = 0; x < n; ++x) {
    const int j = list_entry(p, plan_row, i, x);
    for (int kr = 0; kr < p.block; ++kr) level = fmaxf(level, cb * (1.0f - mask_at(p, mrow, j * p.block + kr)));
  }
  // Passes 1 and 2 walk the keys 64 at a time through LDS.
  auto stage = [&](int key0) {
    __syncthreads();
    stage_rows(ks, p.k + bh * seq, p.L, key0, tid);
    stage_rows(vs, p.v + bh * seq, p.L, key0, tid);
    kbias[tid] = 1.0f - mask_at(p, mrow, key0 + tid);
    __syncthreads();
  };
  // Pass 1: running max and sum of 2^z, z = (s + bias - level) log2e.
  float M = -3.0e38f, S = 0.0f;
  for (int x = 0; x < n; ++x) {
    const int j = list_entry(p, plan_row, i, x);
    for (int half = 0; half < p.block; half += kR) {
      stage(j * p.block + half);
      for (int kr = 0; kr < kR; ++kr) {
        const float z = (dot_lds(q, ks + kr * kPitch) + (__builtin_fmaf(cb, kbias[kr], -level))) * kLog2e;
        if (z > M) {
          S *= exp2f(M - z);
          M = z;
        }
        S += exp2f(z - M);
      }
    }
  }
  const float norm = M + log2f(S);
  // Pass 2: dq.
  float dq[kD];
#pragma unroll
  for (int e = 0; e < kD; ++e) dq[e] = 0.0f;
  for (int x = 0; x < n; ++x) {
    const int j = list_entry(p, plan_row, i, x);
    for (int half = 0; half < p.block; half += kR) {
      stage(j * p.block + half);
      for (int kr = 0; kr < kR; ++kr) {
        const float z = (dot_lds(q, ks + kr * kPitch) + (__builtin_fmaf(cb, kbias[kr], -level))) * kLog2e;
        const float pr = exp2f(z - norm);
        const float ds = pr * (dot_lds(dO, vs + kr * kPitch) - D);
        axpy_lds(dq, ds, ks + kr * kPitch);
      }
    }
  }
  store_row(p.dq + bh * seq, p.L, t, dq);
  if (t < p.L) {
    const int64_t row = (int64_t)bh * p.L + t;
    p.delta[row] = D;
    p.rowterm[2 * row] = level;
    p.rowterm[2 * row + 1] = norm;
  }
}

// How many times key block j appears in query block i's key list.
__device__ inline int multiplicity(const F32Params &p, const int32_t *plan_row, int i, int j) {
  if (p.full || i == 0 || i == p.nb - 1) return 1;
  int m = 0;
  const int n = list_len(p, i);
  for (int x = 0; x < n; ++x) m += list_entry(p, plan_row, i, x) == j ? 1 : 0;
  return m;
}

// Workgroup w: key tile w % tiles of key block (w / tiles) % nb of pair
// w / (tiles * nb).  DK: dk = sum_t P_tu (dP_tu - D_t) q_t; else dv =
// sum_t P_tu dO_t.
template <bool DK>
__global__ __launch_bounds__(kR) void bbsa_bwd_f32_cols(F32Params p) {
  __shared__ __attribute__((aligned(16))) float qs[kR * kPitch];
  __shared__ __attribute__((aligned(16))) float gs[kR * kPitch];
  __shared__ float lv[kR], nm[kR], dd[kR], mqs[kR];
  const int tiles = p.block / kR;
  const int wg = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int j = (wg / tiles) % p.nb;
  const int bh = wg / (tiles * p.nb);
  const int b = bh / p.H, h = bh % p.H;
  const int u = j * p.block + (wg % tiles) * kR + tid;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = p.mask ? p.mask + (int64_t)b * p.L : nullptr;

  float kk[kD], vv[kD], acc[kD];
  load_row(kk, p.k + bh * seq, p.L, u);
  if (DK) load_row(vv, p.v + bh * seq, p.L, u);
#pragma unroll
  for (int e = 0; e < kD; ++e) acc[e] = 0.0f;
  const float kb = kPadBias * (1.0f - mask_at(p, mrow, u));   // the key's bias before the query factor

  for (int i = 0; i < p.nb; ++i) {
    const int mult = multiplicity(p, plan_row_of(p, h, i), i, j);
    if (mult == 0) continue;
    for (int half = 0; half < p.block; half += kR) {
      const int t0 = i * p.block + half;
      if (t0 >= p.L) break;
      __syncthreads();
      stage_rows(qs, p.q + bh * seq, p.L, t0, tid);
      stage_rows(gs, p.dout + bh * seq, p.L, t0, tid);
      {
        const int t = t0 + tid;
        const int64_t row = (int64_t)bh * p.L + t;
        const bool live = t < p.L;
        lv[tid] = live ? p.rowterm[2 * row] : 0.0f;
        nm[tid] = live ? p.rowterm[2 * row + 1] : 0.0f;
        dd[tid] = live ? p.delta[row] : 0.0f;
        mqs[tid] = p.qk ? mask_at(p, mrow, t) : 1.0f;
      }
      __syncthreads();
      const int rows = min(kR, p.L - t0);
      for (int tr = 0; tr < rows; ++tr) {
        const float z = (dot_lds(kk, qs + tr * kPitch) + (__builtin_fmaf(mqs[tr], kb, -lv[tr]))) * kLog2e;
        const float pr = (float)mult * exp2f(z - nm[tr]);
        if (DK) {
          const float ds = pr * (dot_lds(vv, gs + tr * kPitch) - dd[tr]);
          axpy_lds(acc, ds, qs + tr * kPitch);
        } else {
          axpy_lds(acc, pr, gs + tr * kPitch);
        }
      }
    }
  }
  store_row((DK ? p.dk : p.dv) + bh * seq, p.L, u, acc);
}

}  // namespace

int bbsa_sched::launch_backward_f32(const void *q, const void *k, const void *v, const void *out,
                                    const void *dout, const float *mask, const int32_t *rand_attn, int B,
                                    int H, int L, int nb, int block, int r, bool full, bool qk, void *dq,
                                    void *dk, void *dv, float *delta, hipStream_t stream) {
  F32Params p;
  p.q = (const float *)q; p.k = (const float *)k; p.v = (const float *)v; p.o = (const float *)out;
  p.dout = (const float *)dout; p.mask = mask; p.rand_attn = full ? nullptr : rand_attn;
  p.dq = (float *)dq; p.dk = (float *)dk; p.dv = (float *)dv; p.delta = delta;
  p.B = B; p.H = H; p.L = L; p.nb = nb; p.block = block; p.r = r;
  p.full = full ? 1 : 0;
  p.qk = qk ? 1 : 0;
  const int64_t grid = (int64_t)B * H * nb * (block / kR);
  if (grid > 0x7fffffff) return BBSA_ERR_UNSUPPORTED;
  float *ws = nullptr;
  const int rc = library_workspace((size_t)B * H * L * 2 * sizeof(float), stream, &ws);
  if (rc != BBSA_OK) return rc;
  p.rowterm = ws;
  hipLaunchKernelGGL(bbsa_bwd_f32_rows, dim3((unsigned)grid), dim3(kR), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  hipLaunchKernelGGL(bbsa_bwd_f32_cols<false>, dim3((unsigned)grid), dim3(kR), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  hipLaunchKernelGGL(bbsa_bwd_f32_cols<true>, dim3((unsigned)grid), dim3(kR), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  return BBSA_OK;
}
