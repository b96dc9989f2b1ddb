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
//   * the bf16 kernel is persistent: each wavefront pulls work items from the
//     queue of its own XCD (items of the (batch, head) pairs assigned to that
//     XCD, so they share its L2) and streams through them without draining
//     its pipeline: the next item's Q and first K/V tiles are fetched while
//     the current item's last step computes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>
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
  int *ctrl;                 // work-queue counters (see the control block layout below)
  int n_waves;               // persistent wavefronts launched
};

// Control block (int32): queue counter of XCD class x at ctrl[32 * x]
// (x = 0..7, one 128-byte line each), finished-wavefront counter at
// ctrl[kDoneSlot].  All zero between calls: the last wavefront to finish
// resets them.
constexpr int kQueueStride = 32;
constexpr int kDoneSlot = 8 * kQueueStride;
constexpr int kCtrlInts = kDoneSlot + kQueueStride;

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

// Items of XCD class x: the (batch, head) pairs bh = x, x + 8, ... in order,
// each contributing items_per_bh items (full-row chunks first).
__device__ inline int class_items(const Params &p, int x) {
  const int nbh = (p.bh_total > x) ? (p.bh_total - x + 7) / 8 : 0;
  return nbh * p.items_per_bh;
}

__device__ inline Item item_from_ticket(const Params &p, int ticket) {
  const int x = ticket & 7, k = ticket >> 3;
  const int bh = x + 8 * (k / p.items_per_bh);
  const int local = k % p.items_per_bh;
  const bool global_row = local < p.n_global_items;
  const int per_row = p.qtiles * p.chunks;
  const int m = local - p.n_global_items;
  const int grow = global_row ? local / per_row : -1;
  const int rem = global_row ? local % per_row : 0;
  Item it;
  it.bh = bh;
  it.grow = grow;
  it.qt = global_row ? rem / p.chunks : m % p.qtiles;
  it.chunk = global_row ? rem % p.chunks : 0;
  it.qblock = global_row ? ((p.n_rows_global == 2) ? (grow == 0 ? 0 : p.nb - 1) : grow)
                         : 1 + m / p.qtiles;
  return it;
}

// Claim the next item: first from the home XCD's queue, then from the others.
// Returns a ticket (k * 8 + class) or -1 when every queue is drained.  Only
// lane 0 touches the counters; the result is broadcast.
__device__ inline int claim_item(const Params &p, int home, int first_try) {
  int ticket = -1;
  if (__builtin_amdgcn_workitem_id_x() == 0) {
    int k = first_try;
    if (k >= 0 && k < class_items(p, home)) {
      ticket = k * 8 + home;
    } else {
      for (int d = 1; d < 8; ++d) {
        const int x = (home + d) & 7;
        const int n = class_items(p, x);
        int *q = p.ctrl + kQueueStride * x;
        if (n == 0 || __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
        k = __hip_atomic_fetch_add(q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (k < n) { ticket = k * 8 + x; break; }
      }
    }
  }
  return __builtin_amdgcn_readfirstlane(ticket);
}

// Start a claim on the home queue: returns the raw counter value (lane 0; other
// lanes -1).  Resolved later by claim_item.
__device__ inline int claim_issue(const Params &p, int home) {
  int k = -1;
  if (__builtin_amdgcn_workitem_id_x() == 0)
    k = __hip_atomic_fetch_add(p.ctrl + kQueueStride * home, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return k;
}

// The last wavefront to finish puts the control block back to zero for the next call.
__device__ inline void wave_exit(const Params &p) {
  if (__builtin_amdgcn_workitem_id_x() == 0) {
    const int old = __hip_atomic_fetch_add(p.ctrl + kDoneSlot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == p.n_waves - 1) {
      for (int x = 0; x < 8; ++x)
        __hip_atomic_store(p.ctrl + kQueueStride * x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctrl + kDoneSlot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
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

// Lazy rescale for one 32-key step.  s[mt][nt][i] holds the score of key
// 16*mt + 4*g + i for query 16*nt + c; o[dt][nt] is the O^T accumulator.
// Fast path: every lane compares its own 8 scores per query with the
// reference max + tau; only if some score exceeds it anywhere in the
// wavefront is the full row max formed across the 4 lane groups and the
// reference moved (for the queries that need it).
__device__ inline void softmax_rescale(f32x4 (&s)[2][4], SoftmaxState &st, f32x4 (&o)[4][4]) {
  float mloc[4];
  bool need = false;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float a = __builtin_fmaxf(__builtin_fmaxf(s[0][nt][0], s[0][nt][1]), s[0][nt][2]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[0][nt][3]), s[1][nt][0]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[1][nt][1]), s[1][nt][2]);
    mloc[nt] = __builtin_fmaxf(a, s[1][nt][3]);
    need |= mloc[nt] > st.m[nt] + kTau;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float mrow = group4_max(mloc[nt]);
      const bool up = mrow > st.m[nt] + kTau;
      const float alpha = up ? __builtin_amdgcn_exp2f((st.m[nt] - mrow) * kLog2e) : 1.0f;
      st.m[nt] = up ? mrow : st.m[nt];
      st.l[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][nt] *= alpha;
    }
  }
}

// p = exp2((s - m) * log2 e) in place (unnormalised probabilities).
__device__ inline void softmax_exp(f32x4 (&s)[2][4], const SoftmaxState &st) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float nm = -st.m[nt] * kLog2e;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[mt][nt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][i], kLog2e, nm));
  }
}

// Lane-partial row sums of fp32 probabilities.
__device__ inline void row_sum_f32(const f32x4 (&s)[2][4], SoftmaxState &st) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float acc = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += s[mt][nt][i];
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

// The key blocks an item walks, one 32-key step at a time.  At item start,
// lane t of `blk` holds the t-th key block of the item (at most 64 blocks);
// steps read it back with v_readlane, so advancing touches no memory.
struct KeyWalk {
  int n_steps;
  int steps_per_block;
  int blk;             // per lane: key block at list position `lane`
};

struct WalkCursor {
  int t, sb, key0;
  __device__ inline void start(const Params &p, const KeyWalk &w) {
    t = 0;
    sb = 0;
    key0 = __builtin_amdgcn_readfirstlane(w.blk) * p.block;
  }
  __device__ inline void advance(const Params &p, const KeyWalk &w) {
    if (++sb == w.steps_per_block) {
      sb = 0;
      ++t;
      key0 = __builtin_amdgcn_readlane(w.blk, t) * p.block;
    } else {
      key0 += kStep;
    }
  }
};

__device__ inline KeyWalk make_walk(const Params &p, const Item &it) {
  const int lane = (int)__builtin_amdgcn_workitem_id_x();
  KeyWalk w;
  w.steps_per_block = p.block / kStep;
  if (it.grow < 0) {
    // Middle query block i: the two global blocks, the window without them,
    // then the random blocks (clamped so a bad plan never reads outside).
    const int i = it.qblock;
    const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
    const int w0 = (i == 1) ? 1 : i - 1;
    const int h = it.bh % p.H;
    const int32_t *ra_row = p.rand_attn + ((int64_t)h * (p.nb - 2) + (i - 1)) * p.r;
    int blk = 0;
    if (lane == 1) blk = p.nb - 1;
    else if (lane >= 2 && lane < 2 + nw) blk = w0 + (lane - 2);
    else if (lane >= 2 + nw && lane < 2 + nw + p.r) blk = min(max(ra_row[lane - 2 - nw], 0), p.nb - 1);
    w.blk = blk;
    w.n_steps = (2 + nw + p.r) * w.steps_per_block;
  } else {
    const int first = it.chunk * p.chunk_blocks;
    const int nblk = min(p.chunk_blocks, p.nb - first);
    w.blk = first + min(lane, nblk - 1);
    w.n_steps = nblk * w.steps_per_block;
  }
  return w;
}

// Finish an item: either normalise and store the output rows, or store a
// split-K partial (unnormalised O, reference max, row sum).
template <typename OutT>
__device__ inline void finish_item(const Params &p, const Item &it, int q0, SoftmaxState &st,
                                   f32x4 (&o)[4][4]) {
  const int lane = (int)__builtin_amdgcn_workitem_id_x(), c = lane & 15, g = lane >> 4;
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
// Per wavefront, LDS holds two K tiles and two V tiles of 32 keys x 64 d bf16,
// row-major, 128 B per key row.  Tiles are filled straight from HBM with
// global_load_lds_dwordx4 (lane l of an instruction writes the 16 bytes at
// tile + 1024u + 16l, i.e. key row 8u + l/8, chunk position l%8) and stored
// XOR-swizzled: the 16-byte chunk j of row k sits at position j ^ f(k).
//   K: f(k) = (k & 7) ^ ((k >> 3) & 1) -- the 16-byte A-operand reads of 16
//      consecutive rows hit distinct banks.
//   V: f(k) = ((k >> 1) & 3) << 1     -- the 8-byte transposed reads
//      (ds_read_b64_tr_b16) of 16 consecutive rows spread evenly over banks.
//
// Software pipeline of one item (steps j = 0 .. n-1 of 32 keys):
//   iteration j: softmax of step j (vector ALUs) runs interleaved with
//   S(j+1) = K(j+1) Q^T and O^T += V(j-1)^T P(j-1) (matrix cores).
// K tiles are fetched two steps ahead, V tiles one step ahead.
constexpr int kTileBytes = kStep * kD * 2;          // 4 KB
__device__ inline int k_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ inline int v_swz(int row) { return ((row >> 1) & 3) << 1; }

typedef __attribute__((address_space(1))) const void gptr_t;
typedef __attribute__((address_space(3))) void lptr_t;

__device__ inline void dma16(const void *src, unsigned char *lds_dst) {
  __builtin_amdgcn_global_load_lds((gptr_t *)src, (lptr_t *)lds_dst, 16, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Row sums of the bf16-rounded probabilities (the values the PV product uses):
// one v_dot2 against (1, 1) per pair.
__device__ inline void row_sum_bf16(const bf16x8 (&pf)[4], SoftmaxState &st) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float acc = st.l[nt];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[nt], pf[nt], 0, 1), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[nt], pf[nt], 2, 3), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[nt], pf[nt], 4, 5), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[nt], pf[nt], 6, 7), ones, acc, false);
    st.l[nt] = acc;
  }
}

// Rescale decision for one step (before its exponentials): moves the
// reference max of the queries that need it and rescales their row sums;
// returns whether the O accumulator must be rescaled by `alpha` once the
// PV product still in flight has been added.
__device__ inline bool rescale_decide(const f32x4 (&s)[2][4], SoftmaxState &st, float (&alpha)[4]) {
  float mloc[4];
  bool need = false;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float a = __builtin_fmaxf(__builtin_fmaxf(s[0][nt][0], s[0][nt][1]), s[0][nt][2]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[0][nt][3]), s[1][nt][0]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[1][nt][1]), s[1][nt][2]);
    mloc[nt] = __builtin_fmaxf(a, s[1][nt][3]);
    need |= mloc[nt] > st.m[nt] + kTau;
  }
  if (!__builtin_amdgcn_ballot_w64(need)) return false;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float mrow = group4_max(mloc[nt]);
    const bool up = mrow > st.m[nt] + kTau;
    alpha[nt] = up ? __builtin_amdgcn_exp2f((st.m[nt] - mrow) * kLog2e) : 1.0f;
    st.m[nt] = up ? mrow : st.m[nt];
    st.l[nt] *= alpha[nt];
  }
  return true;
}

__device__ inline void copy_scores(const f32x4 (&from)[2][4], f32x4 (&to)[2][4]) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) to[mt][nt] = from[mt][nt];
}

// Scheduling hints: interleave `nmfma` MFMAs with `per` VALU instructions each.
#define BBSA_INTERLEAVE(nmfma, per)                              \
  do {                                                           \
    _Pragma("unroll") for (int _i = 0; _i < (nmfma); ++_i) {     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
      __builtin_amdgcn_sched_group_barrier(0x002, (per), 0);     \
    }                                                            \
  } while (0)

template <bool HAS_MASK>
__global__ __launch_bounds__(64, 2) void bbsa_attn_bf16(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * kTileBytes];
  unsigned char *const kbuf = lds;                    // K tiles: kbuf + (i & 1) * kTileBytes
  unsigned char *const vbuf = lds + 2 * kTileBytes;   // V tiles
  const int lane = (int)__builtin_amdgcn_workitem_id_x(), c = lane & 15, g = lane >> 4;
  const int home = (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7);  // HW_REG_XCC_ID

  // Static assignment: wavefront w serves XCD class w % 8 (the XCD it runs
  // on) and takes that class's items w/8, w/8 + W, w/8 + 2W, ... with W the
  // number of wavefronts of the class.
  const int wg = (int)__builtin_amdgcn_workgroup_id_x();
  const int cls = wg & 7;
  const int stride = (p.n_waves - cls + 7) / 8;
  const int n_cls = class_items(p, cls);
  int kidx = wg >> 3;
  if (kidx >= n_cls) return;
  (void)home;

  // DMA sources (element offsets inside a 32-key step).  Row of instruction u
  // is 8u + lane/8; K's swizzle flips with the parity of u, V's does not.
  const int drow = lane >> 3;
  const int kcol_even = 8 * ((lane & 7) ^ drow);
  const int kcol_odd = 8 * ((lane & 7) ^ drow ^ 1);
  const int vcol = 8 * ((lane & 7) ^ v_swz(drow));
  // LDS read offsets.  K A-operand: row 16mt + c, chunk 4s + g.
  int koff[2];
#pragma unroll
  for (int ss = 0; ss < 2; ++ss) koff[ss] = c * 128 + 16 * ((4 * ss + g) ^ k_swz(c));
  // V^T transposed reads: key row 16mt + 4g + c/4, d = 16dt + 4(c%4) .. +3.
  int voff[4];
  {
    const int row = 4 * g + (c >> 2), qq = c & 3;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      voff[dt] = row * 128 + 16 * ((2 * dt + (qq >> 1)) ^ v_swz(row)) + 8 * (qq & 1);
  }

  auto dma_k = [&](int bh, int key0, int slot) {
    const bf16_t *kb = (const bf16_t *)p.k + (int64_t)bh * p.seq_stride + (int64_t)(key0 + drow) * kD;
    unsigned char *dst = kbuf + slot * kTileBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(kb + u * 8 * kD + ((u & 1) ? kcol_odd : kcol_even), dst + 1024 * u);
  };
  auto dma_v = [&](int bh, int key0, int slot) {
    const bf16_t *vb = (const bf16_t *)p.v + (int64_t)bh * p.seq_stride + (int64_t)(key0 + drow) * kD;
    unsigned char *dst = vbuf + slot * kTileBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(vb + u * 8 * kD + vcol, dst + 1024 * u);
  };
  auto load_mask = [&](int bh, int key0, f32x4 (&mk)[2]) {
    const float *mrow = p.mask + (int64_t)(bh / p.H) * p.L + key0;
    mk[0] = *(const f32x4 *)(mrow + 4 * g);
    mk[1] = *(const f32x4 *)(mrow + 16 + 4 * g);
  };
  auto read_k = [&](int slot, bf16x8 (&kc)[2][2]) {
    const unsigned char *src = kbuf + slot * kTileBytes;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) kc[mt][ss] = *(const bf16x8 *)(src + koff[ss] + 2048 * mt);
  };
  auto read_vt = [&](int slot, bf16x8 (&vt)[4]) {
    const unsigned char *src = vbuf + slot * kTileBytes;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + voff[dt]));
      const s16x4 bb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + voff[dt] + 2048));
      vt[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  bf16x8 qf[4][2];
  // Q^T operand: lane (c, g) holds Q[q0 + 16nt + c][32s + 8g .. +7].
  auto load_q = [&](const Item &it) {
    const bf16_t *Q = (const bf16_t *)p.q + (int64_t)it.bh * p.seq_stride +
                      (int64_t)(it.qblock * p.block + it.qt * kQT) * kD;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
        qf[nt][ss] = *(const bf16x8 *)(Q + (int64_t)(16 * nt + c) * kD + 32 * ss + 8 * g);
  };
  auto scores = [&](const bf16x8 (&kc)[2][2], f32x4 (&sc)[2][4]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[mt][0], qf[nt][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[mt][1], qf[nt][1], acc, 0, 0, 0);
        sc[mt][nt] = acc;
      }
  };

  SoftmaxState st;
  f32x4 o[4][4];
  Item it = item_from_ticket(p, kidx * 8 + cls);

  for (;;) {
    const KeyWalk walk = make_walk(p, it);
    const int n = walk.n_steps;           // >= 2
    WalkCursor ck, cv;                    // K runs two steps ahead of V
    ck.start(p, walk);
    cv.start(p, walk);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) { st.m[nt] = kInitMax; st.l[nt] = 0.0f; }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Prologue: K(0), K(1), Q; S(0).
    f32x4 mk[2];
    if (HAS_MASK) load_mask(it.bh, ck.key0, mk);
    dma_k(it.bh, ck.key0, 0);
    load_q(it);
    ck.advance(p, walk);
    dma_k(it.bh, ck.key0, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x4 sA[2][4], sB[2][4];
    {
      bf16x8 kc[2][2];
      read_k(0, kc);
      scores(kc, sA);
      if (HAS_MASK) apply_mask(sA, mk);
    }

    bf16x8 pf[4];       // P of the previous step
    // One pipeline iteration j.  HAS_S: S(j+1) exists; HAS_PV: step j-1 exists.
    // s_cur holds S(j) (softmaxed here); S(j+1) is written to s_next.
    auto iteration = [&](int j, auto has_s_t, auto has_pv_t, f32x4 (&s_cur)[2][4], f32x4 (&s_next)[2][4]) {
      constexpr bool HAS_S = decltype(has_s_t)::value;
      constexpr bool HAS_PV = decltype(has_pv_t)::value;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // K(j+1), V(j-1), mask(j+1)
      bf16x8 kc[2][2], vt[4];
      if (HAS_S) read_k((j + 1) & 1, kc);
      if (HAS_PV) read_vt((j - 1) & 1, vt);
      f32x4 mk_next[2];
      if (HAS_S && HAS_MASK) load_mask(it.bh, ck.key0, mk_next);
      if (j + 2 < n) {
        ck.advance(p, walk);
        dma_k(it.bh, ck.key0, j & 1);
      }
      dma_v(it.bh, cv.key0, j & 1);
      cv.advance(p, walk);

      float alpha[4];
      const bool resc = rescale_decide(s_cur, st, alpha);

      if (HAS_S) scores(kc, s_next);
      if (HAS_PV) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[dt], pf[nt], o[dt][nt], 0, 0, 0);
      }
      softmax_exp(s_cur, st);
      // P^T operand: key order (mt, i) matches the V^T operand's k slots.
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x4 lo = __builtin_convertvector(s_cur[0][nt], bf16x4);
        const bf16x4 hi = __builtin_convertvector(s_cur[1][nt], bf16x4);
        pf[nt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      row_sum_bf16(pf, st);
      if (HAS_S && HAS_PV) BBSA_INTERLEAVE(32, 3);
      else BBSA_INTERLEAVE(16, 6);
      if (resc) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[dt][nt] *= alpha[nt];
      }
      if (HAS_S && HAS_MASK) apply_mask(s_next, mk_next);
    };

    using T = std::true_type;
    using F = std::false_type;
    iteration(0, T{}, F{}, sA, sB);
    copy_scores(sB, sA);
    for (int j = 1; j < n - 1; ++j) {
      iteration(j, T{}, T{}, sA, sB);
      copy_scores(sB, sA);
    }
    iteration(n - 1, F{}, T{}, sA, sB);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // V(n-1)
    {
      bf16x8 vt[4];
      read_vt((n - 1) & 1, vt);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[dt], pf[nt], o[dt][nt], 0, 0, 0);
    }
    finish_item<bf16_t>(p, it, it.qblock * p.block + it.qt * kQT, st, o);
    kidx += stride;
    if (kidx >= n_cls) break;
    it = item_from_ticket(p, kidx * 8 + cls);
  }
}

// ---------------------------------------------------------------- fp32 path
//
// Same walk and softmax on MFMA 16x16x4 f32.  The d contraction uses the
// order d = 16g + s (s = MFMA step) on both operands; the PV contraction
// steps over (mt, i) with key 16mt + 4g + i, read straight from memory.
template <bool HAS_MASK>
__global__ __launch_bounds__(64) void bbsa_attn_f32(Params p) {
  const Item it = decode_item(p, (int)__builtin_amdgcn_workgroup_id_x());
  if (it.bh >= p.bh_total) return;
  const int lane = (int)__builtin_amdgcn_workitem_id_x(), c = lane & 15, g = lane >> 4;
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

  WalkCursor cur;
  cur.start(p, walk);
  for (int step = 0; step < walk.n_steps; ++step) {
    if (step > 0) cur.advance(p, walk);
    const int key0 = cur.key0;
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
    row_sum_f32(s, st);
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
// One 64-thread workgroup per (batch, head, full row, query tile, 16-query
// slice); thread t handles query 16 * slice + t / 4 and 16 consecutive d.
// out = sum_c w_c O_c / sum_c w_c l_c with w_c = 2^((m_c - M) log2 e),
// M = max_c m_c.
template <typename OutT>
__global__ __launch_bounds__(64) void bbsa_combine(Params p) {
  const int wg = (int)__builtin_amdgcn_workgroup_id_x();
  const int slice = wg & 3, idx = wg >> 2;
  const int qt = idx % p.qtiles;
  const int t2 = idx / p.qtiles;
  const int grow = t2 % p.n_rows_global;
  const int bh = t2 / p.n_rows_global;
  const float *base = p.ws + (int64_t)idx * p.chunks * kPartialFloats;
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int q = 16 * slice + (tid >> 2), dq = tid & 3;
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
  void *ptr = nullptr;       // split-K partials
  size_t bytes = 0;
  int *ctrl = nullptr;       // work-queue control block, zero between calls
  int waves[2] = {0, 0};     // persistent wavefronts of bbsa_attn_bf16<false/true>
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

// Per-device state for one call: the control block and the persistent grid
// size of the bf16 kernel (created on first use), and the partials buffer.
int device_state(size_t bytes, bool masked, float **ws, int **ctrl, int *waves) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BBSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DeviceWorkspace &w = g_ws[dev];
  if (!w.ctrl) {
    int cus = 0, occ0 = 0, occ1 = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return BBSA_ERR_HIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ0, (const void *)bbsa_attn_bf16<false>, 64, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ1, (const void *)bbsa_attn_bf16<true>, 64, 0) != hipSuccess)
      return BBSA_ERR_HIP;
    int *c = nullptr;
    if (hipMalloc(&c, kCtrlInts * sizeof(int)) != hipSuccess) return BBSA_ERR_HIP;
    if (hipMemset(c, 0, kCtrlInts * sizeof(int)) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      (void)hipFree(c);
      return BBSA_ERR_HIP;
    }
    w.ctrl = c;
    w.waves[0] = (occ0 > 0 ? occ0 : 1) * cus;
    w.waves[1] = (occ1 > 0 ? occ1 : 1) * cus;
  }
  *ctrl = w.ctrl;
  *waves = w.waves[masked ? 1 : 0];
  if (bytes > 0 && w.bytes < bytes) {
    if (w.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return BBSA_ERR_HIP;
      if (hipFree(w.ptr) != hipSuccess) return BBSA_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, bytes) != hipSuccess) { w.ptr = nullptr; return BBSA_ERR_HIP; }
    w.bytes = bytes;
  }
  *ws = (float *)w.ptr;
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
    if (5 + r > 64) return BBSA_ERR_UNSUPPORTED;   // a middle row lists at most 64 key blocks
  }

  Params p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v; p.mask = mask; p.rand_attn = rand_attn; p.out = out;
  p.seq_stride = (int64_t)L * kD;
  p.B = B; p.H = H; p.L = L; p.nb = nb; p.block = block; p.r = r;
  p.qtiles = block / kQT;
  p.n_rows_global = full ? nb : 2;
  // Full rows are cut into chunks of 1024 keys so they do not form the tail.
  p.chunk_blocks = 1024 / block;
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

  int waves = 0;
  {
    const int rc = device_state((size_t)n_partials * kPartialFloats * sizeof(float), mask != nullptr,
                                &p.ws, &p.ctrl, &waves);
    if (rc != BBSA_OK) return rc;
  }
  const int64_t total_items = bh * items_per_bh;
  p.n_waves = (int)(total_items < waves ? total_items : waves);
  if (p.n_waves < 8) p.n_waves = 8;   // every XCD class gets a wavefront

  const bool timed = g_timing.enabled && g_timing.n < kMaxTimed;
  const int tslot = g_timing.n;
  if (timed && hipEventRecord(g_timing.ev[tslot][0], stream) != hipSuccess) return BBSA_ERR_HIP;
  const dim3 b1(64);
  if (dtype == BBSA_BF16) {
    const dim3 g1((unsigned)p.n_waves);
    if (mask) hipLaunchKernelGGL(bbsa_attn_bf16<true>, g1, b1, 0, stream, p);
    else hipLaunchKernelGGL(bbsa_attn_bf16<false>, g1, b1, 0, stream, p);
  } else {
    const dim3 g1((unsigned)grid);
    if (mask) hipLaunchKernelGGL(bbsa_attn_f32<true>, g1, b1, 0, stream, p);
    else hipLaunchKernelGGL(bbsa_attn_f32<false>, g1, b1, 0, stream, p);
  }
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  if (timed && hipEventRecord(g_timing.ev[tslot][1], stream) != hipSuccess) return BBSA_ERR_HIP;
  if (n_partials > 0) {
    if (timed && hipEventRecord(g_timing.ev[tslot][2], stream) != hipSuccess) return BBSA_ERR_HIP;
    const dim3 g2((unsigned)(4 * bh * p.n_rows_global * p.qtiles)), b2(64);
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
    DeviceWorkspace &w = g_ws[dev];
    if (!w.ptr && !w.ctrl) continue;
    if (hipSetDevice((int)dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      if (w.ptr) (void)hipFree(w.ptr);
      if (w.ctrl) (void)hipFree(w.ctrl);
    }
    w = DeviceWorkspace();
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
