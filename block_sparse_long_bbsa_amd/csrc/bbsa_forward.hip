// BigBird block-sparse attention forward for MI355X (gfx950).
//
// What is computed ("models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的
// 完整实践", section "BigBird：从二次方注意力到线性稀疏注意力"; "BigBirdPegasus
// 长序列条件生成模型详解…", section "三类注意力组合全局 局部 随机"): for every
// (batch, head), query block 0 and query block nb-1 attend to every key block;
// middle query block i attends to key blocks {0, nb-1}, its window
// {i-1, i, i+1} and the r blocks rand_attn[h][i-1]; padded keys get an
// additive -10000; each query row takes a softmax over the keys it attends.
//
// How it is computed here (the pages' five-segment einsum layout is not used):
//   * one wavefront owns 64 query rows (a "query tile") of one query block and
//     walks a list of key blocks in steps of 32 keys;
//   * scores are computed transposed, S^T = K Q^T, on MFMA 16x16x32 bf16, so
//     that each lane holds all of its queries' scores for 8 keys and the row
//     max needs only two cross-lane swaps (v_permlane32/16_swap);
//   * K goes from HBM straight into MFMA operand registers (16-byte loads);
//     V goes through LDS in an XOR-swizzled row-major tile and is read back
//     transposed with ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T;
//   * P is rounded to bf16 in registers and used directly as the B operand
//     (the lane layout of the S^T accumulator matches it after a fixed
//     permutation of the key order inside each 32-key step);
//   * online softmax in base 2 with a lazy rescale (the running reference max
//     moves only when a new max exceeds it by more than 2^8 in probability);
//   * the two global query blocks are split along the keys into chunks whose
//     partial (O, max, sum) go to a workspace and are merged by a second
//     kernel with the log-sum-exp rule;
//   * work items are mapped onto the 8 XCDs so that all items of one
//     (batch, head) run on one XCD and share its L2.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "bbsa.h"

namespace {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 64;        // head dimension
constexpr int kQT = 64;       // query rows per wavefront
constexpr int kStep = 32;     // keys per softmax step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPadBias = -10000.0f;
// Lazy rescale threshold (raw score units): unnormalised probabilities stay <= 2^8.
constexpr float kTau = 8.0f / 1.4426950408889634f;
constexpr float kInitMax = -1.0e30f;
// One split-K partial: O[64][64] fp32, then the 64 reference maxima, then the 64 sums.
constexpr int kPartialFloats = kQT * kD + 2 * kQT;

struct Params {
  const void *q, *k, *v;
  const float *mask;         // [B, L] or null
  const int32_t *rand_attn;  // [H, nb-2, r]
  void *out;
  float *ws;                 // split-K partials
  int64_t seq_stride;        // L * d elements per (batch, head)
  int B, H, L, nb, block, r;
  int qtiles;                // block / 64
  int n_rows_global;         // query blocks handled as full rows: 2, or nb on the fallback
  int chunks;                // key chunks per full row
  int chunk_blocks;          // key blocks per chunk
  int n_global_items;        // per (batch, head): n_rows_global * qtiles * chunks
  int items_per_bh;          // n_global_items + middle items
  int bh_total;              // B * H
  int xcd_remap;             // 1: map workgroups so one (batch, head) stays on one XCD
};

struct Item {
  int bh;
  int qblock;     // query block index
  int qt;         // query tile inside the block
  int grow;       // full-row index (partials), -1 for a middle row
  int chunk;      // key chunk of a full row
};

__device__ inline Item decode_item(const Params &p, int wg) {
  int bh, local;
  if (p.xcd_remap) {
    // Workgroups are dispatched round-robin over the 8 XCDs: wg % 8 is the XCD.
    const int xcd = wg & 7, slot = wg >> 3;
    bh = xcd + 8 * (slot / p.items_per_bh);
    local = slot % p.items_per_bh;
  } else {
    bh = wg / p.items_per_bh;
    local = wg % p.items_per_bh;
  }
  const bool global_row = local < p.n_global_items;
  const int per_row = p.qtiles * p.chunks;
  const int m = local - p.n_global_items;
  const int grow = global_row ? local / per_row : -1;
  const int rem = global_row ? local % per_row : 0;
  Item it;
  it.bh = bh;   // >= bh_total marks an idle workgroup
  it.grow = grow;
  it.qt = global_row ? rem / p.chunks : m % p.qtiles;
  it.chunk = global_row ? rem % p.chunks : 0;
  it.qblock = global_row ? ((p.n_rows_global == 2) ? (grow == 0 ? 0 : p.nb - 1) : grow)
                         : 1 + m / p.qtiles;
  return it;
}

// Key blocks of a middle query block i, in processing order:
// the two global blocks, the window without them, then the random blocks.
__device__ inline int middle_count(const Params &p, int i) {
  const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
  return 2 + nw + p.r;
}
__device__ inline int middle_block(const Params &p, const int32_t *ra_row, int i, int t) {
  if (t == 0) return 0;
  if (t == 1) return p.nb - 1;
  const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
  const int w0 = (i == 1) ? 1 : i - 1;
  if (t < 2 + nw) return w0 + (t - 2);
  const int j = ra_row[t - 2 - nw];
  return min(max(j, 0), p.nb - 1);   // never read outside the sequence
}

__device__ inline float group4_max(float x) {
  // Lanes l, l^16, l^32, l^48 hold the same query column.
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Online-softmax state of the 4 query columns a lane holds (one per 16-query tile nt).
struct SoftmaxState {
  float m[4];   // reference max (raw score units), identical across the 4 lane groups
  float l[4];   // per-lane partial row sum of exp2 values
};

// Row max + lazy rescale for one 32-key step.  s[mt][nt][i] holds the score of
// key 16*mt + 4*g + i for query 16*nt + c.  o[dt][nt] is the O^T accumulator.
__device__ inline void softmax_rescale(f32x4 (&s)[2][4], SoftmaxState &st, f32x4 (&o)[4][4]) {
  float mloc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float a = __builtin_fmaxf(__builtin_fmaxf(s[0][nt][0], s[0][nt][1]), s[0][nt][2]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[0][nt][3]), s[1][nt][0]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[1][nt][1]), s[1][nt][2]);
    mloc[nt] = group4_max(__builtin_fmaxf(a, s[1][nt][3]));
  }
  bool need = false;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) need |= mloc[nt] > st.m[nt] + kTau;
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bool up = mloc[nt] > st.m[nt] + kTau;
      const float alpha = up ? __builtin_amdgcn_exp2f((st.m[nt] - mloc[nt]) * kLog2e) : 1.0f;
      st.m[nt] = up ? mloc[nt] : st.m[nt];
      st.l[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][nt] *= alpha;
    }
  }
}

// p = exp2((s - m) * log2 e) in place; accumulate the lane's partial row sums.
__device__ inline void softmax_exp(f32x4 (&s)[2][4], SoftmaxState &st) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float nm = -st.m[nt] * kLog2e;
    float acc = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][i], kLog2e, nm));
        s[mt][nt][i] = e;
        acc += e;
      }
    }
    st.l[nt] += acc;
  }
}

// Add the key-side padding bias to every score when any key of this step is padded.
__device__ inline void apply_mask(f32x4 (&s)[2][4], const f32x4 (&mk)[2]) {
  float bias[2][4];
  bool any = false;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bias[mt][i] = kPadBias * (1.0f - mk[mt][i]);
      any |= bias[mt][i] != 0.0f;
    }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[mt][nt][i] += bias[mt][i];
  }
}

// Key offset (in keys) of step `step` of an item.
struct KeyWalk {
  int n_steps;
  int steps_per_block;
  int first_block;     // full-row chunk: first key block
  int qblock;          // middle row: query block index
  const int32_t *ra_row;
  bool middle;
  __device__ inline int key0(const Params &p, int step) const {
    const int t = step / steps_per_block, sb = step - t * steps_per_block;
    const int blk = middle ? middle_block(p, ra_row, qblock, t) : first_block + t;
    return blk * p.block + sb * kStep;
  }
};

__device__ inline KeyWalk make_walk(const Params &p, const Item &it) {
  KeyWalk w;
  w.steps_per_block = p.block / kStep;
  w.qblock = it.qblock;
  w.middle = it.grow < 0;
  if (w.middle) {
    const int h = it.bh % p.H;
    w.ra_row = p.rand_attn + ((int64_t)h * (p.nb - 2) + (it.qblock - 1)) * p.r;
    w.first_block = 0;
    w.n_steps = middle_count(p, it.qblock) * w.steps_per_block;
  } else {
    w.ra_row = nullptr;
    w.first_block = it.chunk * p.chunk_blocks;
    const int nblk = min(p.chunk_blocks, p.nb - w.first_block);
    w.n_steps = nblk * w.steps_per_block;
  }
  return w;
}

// Finish an item: either normalise and store the output rows, or store a
// split-K partial (unnormalised O, reference max, row sum).
template <typename OutT>
__device__ inline void finish_item(const Params &p, const Item &it, int q0, SoftmaxState &st,
                                   f32x4 (&o)[4][4]) {
  const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  float lsum[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) lsum[nt] = group4_sum(st.l[nt]);
  if (it.grow >= 0 && p.chunks > 1) {
    const int64_t pidx = (((int64_t)it.bh * p.n_rows_global + it.grow) * p.qtiles + it.qt) * p.chunks + it.chunk;
    float *part = p.ws + pidx * kPartialFloats;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *(f32x4 *)(part + (16 * nt + c) * kD + 16 * dt + 4 * g) = o[dt][nt];
    if (g == 0) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        part[kQT * kD + 16 * nt + c] = st.m[nt];
        part[kQT * kD + kQT + 16 * nt + c] = lsum[nt];
      }
    }
    return;
  }
  OutT *out = (OutT *)p.out + (int64_t)it.bh * p.seq_stride;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float inv = 1.0f / lsum[nt];
    OutT *row = out + (int64_t)(q0 + 16 * nt + c) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const f32x4 y = o[dt][nt] * inv;
      if constexpr (sizeof(OutT) == 2) {
        *(bf16x4 *)(row + 16 * dt + 4 * g) = __builtin_convertvector(y, bf16x4);
      } else {
        *(f32x4 *)(row + 16 * dt + 4 * g) = y;
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 path
//
// V tile in LDS: 32 keys x 64 d bf16, row-major, 128 B per key.  The 16-byte
// chunk j of key row k is stored at chunk position j ^ swz(k) with
// swz(k) = ((k >> 1) & 3) << 1, which makes both the 16-byte writes and the
// 8-byte transposed reads free of bank conflicts.
__device__ inline int v_swz(int row) { return ((row >> 1) & 3) << 1; }

template <bool HAS_MASK>
__global__ __launch_bounds__(64) void bbsa_attn_bf16(Params p) {
  const Item it = decode_item(p, blockIdx.x);
  if (it.bh >= p.bh_total) return;
  __shared__ __attribute__((aligned(16))) unsigned char vlds[kStep * kD * 2];

  const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  const int b = it.bh / p.H;
  const bf16_t *Q = (const bf16_t *)p.q + (int64_t)it.bh * p.seq_stride;
  const bf16_t *K = (const bf16_t *)p.k + (int64_t)it.bh * p.seq_stride;
  const bf16_t *V = (const bf16_t *)p.v + (int64_t)it.bh * p.seq_stride;
  const float *mrow = HAS_MASK ? p.mask + (int64_t)b * p.L : nullptr;
  const int q0 = it.qblock * p.block + it.qt * kQT;

  // Q^T operand: lane (c, g) holds Q[q0 + 16nt + c][32s + 8g .. +7].
  bf16x8 qf[4][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qf[nt][s] = *(const bf16x8 *)(Q + (int64_t)(q0 + 16 * nt + c) * kD + 32 * s + 8 * g);

  // LDS addresses.  Writes: 4 x 1 KB, lane -> key row (lane >> 3) + 8u, chunk lane & 7.
  const int wrow = lane >> 3, wchunk = lane & 7;
  const int woff = wrow * 128 + 16 * (wchunk ^ v_swz(wrow));
  // Transposed reads: lane (c, g) with j = c >> 2, qq = c & 3 reads key row
  // 16mt + 4g + j, d = 16dt + 4qq .. +3.
  int roff[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = 16 * mt + 4 * g + (c >> 2), qq = c & 3;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int chunk = 2 * dt + (qq >> 1);
      roff[mt][dt] = row * 128 + 16 * (chunk ^ v_swz(row)) + 8 * (qq & 1);
    }
  }

  const KeyWalk walk = make_walk(p, it);
  SoftmaxState st;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) { st.m[nt] = kInitMax; st.l[nt] = 0.0f; }
  f32x4 o[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prefetch registers for the next step.
  bf16x8 kf[2][2];
  i32x4 vst[4];
  f32x4 mk[2];
  auto load_step = [&](int key0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        kf[mt][s] = *(const bf16x8 *)(K + (int64_t)(key0 + 16 * mt + c) * kD + 32 * s + 8 * g);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vst[u] = *(const i32x4 *)(V + (int64_t)(key0 + 8 * u + wrow) * kD + 8 * wchunk);
    if (HAS_MASK) {
      mk[0] = *(const f32x4 *)(mrow + key0 + 4 * g);
      mk[1] = *(const f32x4 *)(mrow + key0 + 16 + 4 * g);
    }
  };
  load_step(walk.key0(p, 0));

  for (int step = 0; step < walk.n_steps; ++step) {
    // Stage this step's V tile; copy its K and mask out of the prefetch registers.
#pragma unroll
    for (int u = 0; u < 4; ++u) *(i32x4 *)(vlds + woff + 1024 * u) = vst[u];
    bf16x8 kc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s) kc[mt][s] = kf[mt][s];
    f32x4 mc[2];
    if (HAS_MASK) { mc[0] = mk[0]; mc[1] = mk[1]; }
    if (step + 1 < walk.n_steps) load_step(walk.key0(p, step + 1));

    // S^T = K Q^T for 32 keys x 64 queries.
    f32x4 s[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[mt][0], qf[nt][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[mt][1], qf[nt][1], acc, 0, 0, 0);
        s[mt][nt] = acc;
      }
    if (HAS_MASK) apply_mask(s, mc);
    softmax_rescale(s, st, o);
    softmax_exp(s, st);

    // P^T operand: key order (mt, i) matches the V^T operand's k slots.
    bf16x8 pf[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bf16x4 lo = __builtin_convertvector(s[0][nt], bf16x4);
      const bf16x4 hi = __builtin_convertvector(s[1][nt], bf16x4);
      pf[nt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // V^T operand via transposed LDS reads.
    bf16x8 vt[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vlds + roff[0][dt]));
      const s16x4 bb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vlds + roff[1][dt]));
      vt[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[dt], pf[nt], o[dt][nt], 0, 0, 0);
  }
  finish_item<bf16_t>(p, it, q0, st, o);
}

// ---------------------------------------------------------------- fp32 path
//
// Same walk and softmax on MFMA 16x16x4 f32.  The d contraction uses the
// order d = 16g + s (s = MFMA step) on both operands; the PV contraction
// steps over (mt, i) with key 16mt + 4g + i, read straight from memory.
template <bool HAS_MASK>
__global__ __launch_bounds__(64) void bbsa_attn_f32(Params p) {
  const Item it = decode_item(p, blockIdx.x);
  if (it.bh >= p.bh_total) return;
  const int lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  const int b = it.bh / p.H;
  const float *Q = (const float *)p.q + (int64_t)it.bh * p.seq_stride;
  const float *K = (const float *)p.k + (int64_t)it.bh * p.seq_stride;
  const float *V = (const float *)p.v + (int64_t)it.bh * p.seq_stride;
  const float *mrow = HAS_MASK ? p.mask + (int64_t)b * p.L : nullptr;
  const int q0 = it.qblock * p.block + it.qt * kQT;

  float qf[4][16];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f32x4 x = *(const f32x4 *)(Q + (int64_t)(q0 + 16 * nt + c) * kD + 16 * g + 4 * s4);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[nt][4 * s4 + e] = x[e];
    }

  const KeyWalk walk = make_walk(p, it);
  SoftmaxState st;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) { st.m[nt] = kInitMax; st.l[nt] = 0.0f; }
  f32x4 o[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int step = 0; step < walk.n_steps; ++step) {
    const int key0 = walk.key0(p, step);
    f32x4 s[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float kf[16];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4 x = *(const f32x4 *)(K + (int64_t)(key0 + 16 * mt + c) * kD + 16 * g + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) kf[4 * s4 + e] = x[e];
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[ks], qf[nt][ks], acc, 0, 0, 0);
        s[mt][nt] = acc;
      }
    }
    if (HAS_MASK) {
      f32x4 mc[2];
      mc[0] = *(const f32x4 *)(mrow + key0 + 4 * g);
      mc[1] = *(const f32x4 *)(mrow + key0 + 16 + 4 * g);
      apply_mask(s, mc);
    }
    softmax_rescale(s, st, o);
    softmax_exp(s, st);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float *vrow = V + (int64_t)(key0 + 16 * mt + 4 * g + i) * kD + c;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const float va = vrow[16 * dt];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, s[mt][nt][i], o[dt][nt], 0, 0, 0);
        }
      }
  }
  finish_item<float>(p, it, q0, st, o);
}

// ---------------------------------------------------------------- split-K merge
//
// One workgroup per (batch, head, full row, query tile); thread t handles query
// t >> 2 and 16 consecutive d.  out = sum_c w_c O_c / sum_c w_c l_c with
// w_c = 2^((m_c - M) log2 e), M = max_c m_c.
template <typename OutT>
__global__ __launch_bounds__(256) void bbsa_combine(Params p) {
  const int idx = blockIdx.x;
  const int qt = idx % p.qtiles;
  const int t2 = idx / p.qtiles;
  const int grow = t2 % p.n_rows_global;
  const int bh = t2 / p.n_rows_global;
  const float *base = p.ws + (int64_t)idx * p.chunks * kPartialFloats;
  const int q = threadIdx.x >> 2, dq = threadIdx.x & 3;
  float M = kInitMax;
  for (int ch = 0; ch < p.chunks; ++ch) M = __builtin_fmaxf(M, base[(int64_t)ch * kPartialFloats + kQT * kD + q]);
  float den = 0.0f;
  f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int ch = 0; ch < p.chunks; ++ch) {
    const float *part = base + (int64_t)ch * kPartialFloats;
    const float w = __builtin_amdgcn_exp2f((part[kQT * kD + q] - M) * kLog2e);
    den += w * part[kQT * kD + kQT + q];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += w * *(const f32x4 *)(part + q * kD + 16 * dq + 4 * e);
  }
  const float inv = 1.0f / den;
  const int qblock = (p.n_rows_global == 2) ? (grow == 0 ? 0 : p.nb - 1) : grow;
  OutT *row = (OutT *)p.out + (int64_t)bh * p.seq_stride + (int64_t)(qblock * p.block + qt * kQT + q) * kD + 16 * dq;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4 y = acc[e] * inv;
    if constexpr (sizeof(OutT) == 2) {
      *(bf16x4 *)(row + 4 * e) = __builtin_convertvector(y, bf16x4);
    } else {
      *(f32x4 *)(row + 4 * e) = y;
    }
  }
}

// ---------------------------------------------------------------- host side

struct DeviceWorkspace {
  void *ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_mutex;
std::vector<DeviceWorkspace> g_ws;

constexpr int kMaxTimed = 4096;
struct Timing {
  bool enabled = false;
  bool created = false;
  int n = 0;
  hipEvent_t ev[kMaxTimed][4];
  bool has_combine[kMaxTimed];
};
Timing g_timing;

int ensure_workspace(size_t bytes, float **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BBSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DeviceWorkspace &w = g_ws[dev];
  if (w.bytes < bytes) {
    if (w.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return BBSA_ERR_HIP;
      if (hipFree(w.ptr) != hipSuccess) return BBSA_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, bytes) != hipSuccess) { w.ptr = nullptr; return BBSA_ERR_HIP; }
    w.bytes = bytes;
  }
  *out = (float *)w.ptr;
  return BBSA_OK;
}

}  // namespace

extern "C" int bbsa_forward(const void *q, const void *k, const void *v, const float *mask,
                            const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                            void *out, hipStream_t stream, int dtype) {
  if (!q || !k || !v || !out) return BBSA_ERR_ARG;
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || block <= 0 || r < 1) return BBSA_ERR_ARG;
  if (dtype != BBSA_BF16 && dtype != BBSA_F32) return BBSA_ERR_UNSUPPORTED;
  if (d != kD || (block != 64 && block != 128)) return BBSA_ERR_UNSUPPORTED;
  if (L % block != 0) return BBSA_ERR_SHAPE;
  const int nb = L / block;
  const bool full = (int64_t)L <= (int64_t)(5 + 2 * (int64_t)r) * block;
  if (!full) {
    if (!rand_attn) return BBSA_ERR_ARG;
    if (nb < 5 + r) return BBSA_ERR_SHAPE;
  }

  Params p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.mask = mask; p.rand_attn = rand_attn; p.out = out;
  p.seq_stride = (int64_t)L * kD;
  p.B = B; p.H = H; p.L = L; p.nb = nb; p.block = block; p.r = r;
  p.qtiles = block / kQT;
  p.n_rows_global = full ? nb : 2;
  // Full rows are cut into chunks of about 2048 keys so they do not form the tail.
  p.chunk_blocks = 2048 / block;
  if (p.chunk_blocks > nb) p.chunk_blocks = nb;
  p.chunks = (nb + p.chunk_blocks - 1) / p.chunk_blocks;
  p.n_global_items = p.n_rows_global * p.qtiles * p.chunks;
  const int n_middle = full ? 0 : (nb - 2) * p.qtiles;
  const int64_t bh = (int64_t)B * H;
  const int64_t items_per_bh = (int64_t)p.n_global_items + n_middle;
  p.xcd_remap = bh >= 8 ? 1 : 0;
  const int64_t grid = p.xcd_remap ? 8 * ((bh + 7) / 8) * items_per_bh : bh * items_per_bh;
  const int64_t n_partials = (p.chunks > 1) ? bh * p.n_rows_global * p.qtiles * p.chunks : 0;
  if (grid > 0x7fffffff || bh > 0x7fffffff || (int64_t)B * H * L * kD > ((int64_t)1 << 40) ||
      bh * p.n_rows_global * p.qtiles > 0x7fffffff)
    return BBSA_ERR_UNSUPPORTED;
  p.items_per_bh = (int)items_per_bh;
  p.bh_total = (int)bh;

  if (n_partials > 0) {
    const int rc = ensure_workspace((size_t)n_partials * kPartialFloats * sizeof(float), &p.ws);
    if (rc != BBSA_OK) return rc;
  }

  const bool timed = g_timing.enabled && g_timing.n < kMaxTimed;
  const int tslot = g_timing.n;
  if (timed && hipEventRecord(g_timing.ev[tslot][0], stream) != hipSuccess) return BBSA_ERR_HIP;
  const dim3 g1((unsigned)grid), b1(64);
  if (dtype == BBSA_BF16) {
    if (mask) hipLaunchKernelGGL(bbsa_attn_bf16<true>, g1, b1, 0, stream, p);
    else hipLaunchKernelGGL(bbsa_attn_bf16<false>, g1, b1, 0, stream, p);
  } else {
    if (mask) hipLaunchKernelGGL(bbsa_attn_f32<true>, g1, b1, 0, stream, p);
    else hipLaunchKernelGGL(bbsa_attn_f32<false>, g1, b1, 0, stream, p);
  }
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  if (timed && hipEventRecord(g_timing.ev[tslot][1], stream) != hipSuccess) return BBSA_ERR_HIP;
  if (n_partials > 0) {
    if (timed && hipEventRecord(g_timing.ev[tslot][2], stream) != hipSuccess) return BBSA_ERR_HIP;
    const dim3 g2((unsigned)(bh * p.n_rows_global * p.qtiles)), b2(256);
    if (dtype == BBSA_BF16) hipLaunchKernelGGL(bbsa_combine<bf16_t>, g2, b2, 0, stream, p);
    else hipLaunchKernelGGL(bbsa_combine<float>, g2, b2, 0, stream, p);
    if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
    if (timed && hipEventRecord(g_timing.ev[tslot][3], stream) != hipSuccess) return BBSA_ERR_HIP;
  }
  if (timed) {
    g_timing.has_combine[tslot] = n_partials > 0;
    g_timing.n++;
  }
  return full ? BBSA_OK_FULL_FALLBACK : BBSA_OK;
}

extern "C" const char *bbsa_status_string(int status) {
  switch (status) {
    case BBSA_OK: return "ok";
    case BBSA_OK_FULL_FALLBACK: return "ok: sequence too short for the sparse pattern, computed full attention";
    case BBSA_ERR_ARG: return "invalid argument (null pointer, non-positive size or r < 1)";
    case BBSA_ERR_SHAPE: return "invalid shape (length not a multiple of the block, or nb < 5 + r)";
    case BBSA_ERR_UNSUPPORTED: return "unsupported configuration (d != 64, block not 64/128, dtype, or size)";
    case BBSA_ERR_HIP: return "HIP runtime error";
    case BBSA_ERR_PLAN: return "rand_attn violates the plan invariants";
    default: return "unknown status";
  }
}

extern "C" void bbsa_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  for (size_t dev = 0; dev < g_ws.size(); ++dev) {
    if (!g_ws[dev].ptr) continue;
    if (hipSetDevice((int)dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(g_ws[dev].ptr);
    }
    g_ws[dev].ptr = nullptr;
    g_ws[dev].bytes = 0;
  }
  (void)hipSetDevice(cur);
}

extern "C" int bbsa_version(void) { return 100; }

extern "C" int bbsa_timing_enable(int enable) {
  if (enable && !g_timing.created) {
    for (int i = 0; i < kMaxTimed; ++i)
      for (int j = 0; j < 4; ++j)
        if (hipEventCreate(&g_timing.ev[i][j]) != hipSuccess) return BBSA_ERR_HIP;
    g_timing.created = true;
  }
  g_timing.enabled = enable != 0;
  g_timing.n = 0;
  return BBSA_OK;
}

extern "C" int bbsa_timing_read(double *main_ms, double *combine_ms, int *calls) {
  if (!main_ms || !combine_ms || !calls) return BBSA_ERR_ARG;
  double a = 0.0, c = 0.0;
  for (int i = 0; i < g_timing.n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timing.ev[i][1]) != hipSuccess) return BBSA_ERR_HIP;
    if (hipEventElapsedTime(&ms, g_timing.ev[i][0], g_timing.ev[i][1]) != hipSuccess) return BBSA_ERR_HIP;
    a += ms;
    if (g_timing.has_combine[i]) {
      if (hipEventSynchronize(g_timing.ev[i][3]) != hipSuccess) return BBSA_ERR_HIP;
      if (hipEventElapsedTime(&ms, g_timing.ev[i][2], g_timing.ev[i][3]) != hipSuccess) return BBSA_ERR_HIP;
      c += ms;
    }
  }
  *main_ms = a;
  *combine_ms = c;
  *calls = g_timing.n;
  g_timing.n = 0;
  return BBSA_OK;
}
