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
//   * a work item is 64 query rows of one query block against the key blocks
//     of a middle row or one key chunk of a global row, walked in steps of
//     32 keys; on the bf16 path one wavefront runs one item and a 256-thread
//     workgroup runs four consecutive items, on the fp32 path the four
//     wavefronts of a workgroup split one item's query rows;
//   * bf16 path: scores are computed transposed, S^T = K Q^T, on MFMA
//     32x32x16 bf16, so each lane holds 16 keys of one query column and the
//     row max needs a single cross-lane swap; a probability costs one FMA
//     (score * log2(e) - reference max) and one v_exp_f32;
//   * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ...
//     lds, XOR-swizzled rows); K is read back as the MFMA A operand, V is read back
//     transposed with ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T;
//     P is rounded to bf16 in registers and used directly as the B operand;
//   * software pipeline: the softmax of step j runs between the MFMAs of
//     S(j+1) and of the PV product of step j-1; K tiles are fetched two steps
//     ahead, V tiles one step ahead;
//   * online softmax in base 2 with a lazy rescale (the reference max moves
//     only when a score exceeds it by more than 8, i.e. p > 2^8);
//   * the two global query blocks are split along the keys into chunks; on
//     the bf16 path the four chunks of a workgroup merge their partials
//     (O, max, sum) in LDS with the log-sum-exp rule, and longer rows (and
//     the fp32 path) leave partials in a workspace for a second kernel;
//   * workgroups are mapped onto the 8 XCDs so that all items of one
//     (batch, head) run on one XCD and share its L2;
//   * bf16 path with a mask: an item whose key list holds a key of mask 1
//     drops the listed blocks whose keys all have mask 0 (their
//     probabilities are exactly zero), after one probe of the mask per
//     listed block in its prologue.
// The work decomposition itself (launch sizing, item mapping, key-block
// lists) is in bbsa_schedule.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "bbsa.h"
#include "bbsa_schedule.h"


namespace {

using namespace bbsa_sched;

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPadBias = -10000.0f;
// Lazy rescale threshold (raw score units): unnormalised probabilities stay <= 2^8.
constexpr float kTau = 8.0f / 1.4426950408889634f;
constexpr float kTauLog2 = 8.0f;
constexpr float kInitMax = -1.0e30f;
constexpr float kLn2 = 0.6931471805599453f;

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

// fp32 path: each wavefront owns kNT 16-query tiles of its item.
constexpr int kNT = 1;
static_assert(kF32Waves * kNT == 4, "the fp32 workgroup's wavefronts split an item's four 16-row tiles");

// Online-softmax state of the kNT query columns a lane holds (one per 16-query tile nt).
// The scores are taken relative to a padding-bias level: key k contributes
// s_k + (bias_k - level), where level is the largest bias among the keys seen
// so far (uniform over the wavefront).  A row whose keys all share one mask
// value therefore sees its scores unchanged, instead of s_k - 10000 rounded
// to fp32's spacing of about 1e-3 at that magnitude; keys below the level
// carry the (exact, for 0/1 masks) difference.
struct SoftmaxState {
  float m[kNT];   // reference max (raw score units, relative to the level), identical across the 4 lane groups
  float l[kNT];   // per-lane partial row sum of exp2 values
  float level;    // padding-bias level (uniform)
};

// Lazy rescale for one 32-key step.  s[mt][nt][i] holds the score of key
// 16*mt + 4*g + i for query 16*nt + c; o[dt][nt] is the O^T accumulator.
// Fast path: every lane compares its own 8 scores per query with the
// reference max + tau; only if some score exceeds it anywhere in the
// wavefront is the full row max formed across the 4 lane groups and the
// reference moved (for the queries that need it).
__device__ inline void softmax_rescale(f32x4 (&s)[2][kNT], SoftmaxState &st, f32x4 (&o)[4][kNT]) {
  float mloc[kNT];
  bool need = false;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    float a = __builtin_fmaxf(__builtin_fmaxf(s[0][nt][0], s[0][nt][1]), s[0][nt][2]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[0][nt][3]), s[1][nt][0]);
    a = __builtin_fmaxf(__builtin_fmaxf(a, s[1][nt][1]), s[1][nt][2]);
    mloc[nt] = __builtin_fmaxf(a, s[1][nt][3]);
    need |= mloc[nt] > st.m[nt] + kTau;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
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
__device__ inline void softmax_exp(f32x4 (&s)[2][kNT], const SoftmaxState &st) {
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const float nm = -st.m[nt] * kLog2e;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[mt][nt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][i], kLog2e, nm));
  }
}

// Lane-partial row sums of fp32 probabilities.
__device__ inline void row_sum_f32(const f32x4 (&s)[2][kNT], SoftmaxState &st) {
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    float acc = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += s[mt][nt][i];
    st.l[nt] += acc;
  }
}

// Add the key-side padding bias, relative to the state's level, to every
// score.  A step whose largest bias exceeds the level raises the level first;
// the reference max moves down by the same amount, so it stays the same
// absolute value (what was accumulated against the old level is rescaled, or
// vanishes, through the ordinary rescale that follows).
// With query x key masking each query row scales the key bias (and so the
// level) by its own mask value mq (the rest of -10000 (1 - m_q m_k) is a
// per-row constant that cancels in the softmax).
template <bool QK>
__device__ inline void apply_mask(f32x4 (&s)[2][kNT], const f32x4 (&mk)[2], SoftmaxState &st,
                                  const float (&mq)[kNT]) {
  float bias[2][4];
  float bmax = kInitMax;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bias[mt][i] = kPadBias * (1.0f - mk[mt][i]);
      bmax = __builtin_fmaxf(bmax, bias[mt][i]);
    }
  // Lanes l, l^16, l^32, l^48 hold the step's four groups of 8 keys.
  bmax = group4_max(bmax);
  if (bmax > st.level) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) st.m[nt] += (QK ? mq[nt] : 1.0f) * (st.level - bmax);
    st.level = bmax;
  }
  bool any = false;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bias[mt][i] -= st.level;
      any |= bias[mt][i] != 0.0f;
    }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[mt][nt][i] += QK ? mq[nt] * bias[mt][i] : bias[mt][i];
  }
}

struct WalkCursor {
  int t, sb, key0;
  __device__ inline void start(const Params &p, const KeyWalk &w) {
    t = 0;
    sb = 0;
    key0 = __builtin_amdgcn_readfirstlane(w.first_blk * p.block);   // uniform; no plan entry needed
  }
  // Start at position t0 of the block list (plan entries already merged).
  __device__ inline void start_at(const Params &p, const KeyWalk &w, int t0) {
    t = t0;
    sb = 0;
    key0 = __builtin_amdgcn_readlane(w.blk, t0) * p.block;
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

__device__ inline int lane_id() { return (int)__builtin_amdgcn_workitem_id_x() & 63; }

__device__ inline KeyWalk make_walk(const Params &p, const Item &it) {
  int rnd, rslot;
  KeyWalk w = make_walk_base(p, it, lane_id(), rnd, rslot);
  merge_plan(p, w, rnd, rslot);
  w.n_steps = __builtin_amdgcn_readfirstlane(w.n_steps);
  return w;
}

// The fp32 O^T accumulator o[dt][nt] holds, in lane (c, g) and register i,
// d = 16g + 4i + dt of query 16 nt + c: the four d-tiles together give four
// consecutive d.
__device__ inline f32x4 d_run(const f32x4 (&o)[4][kNT], int nt, int i) {
  return f32x4{o[0][nt][i], o[1][nt][i], o[2][nt][i], o[3][nt][i]};
}

// Finish an item of the fp32 path: either normalise and store the output rows, or store a
// split-K partial (unnormalised O, reference max, row sum).
template <typename OutT, bool RAGGED, bool QK>
__device__ inline void finish_item(const Params &p, const Item &it, int q0, int nt0, SoftmaxState &st,
                                   f32x4 (&o)[4][kNT], const float (&mq)[kNT]) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  float lsum[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) lsum[nt] = group4_sum(st.l[nt]);
  const bool full_part = it.grow >= 0 && p.nparts > 1, mid_part = it.grow < 0 && p.mparts > 1;
  if (full_part || mid_part) {
    const int64_t pidx =
        full_part ? (((int64_t)it.bh * p.n_rows_global + it.grow) * p.qtiles + it.qt) * p.nparts + it.chunk
                  : p.mid_part_base + (((int64_t)it.bh * (p.nb - 2) + (it.qblock - 1)) * p.qtiles + it.qt) * p.mparts + it.chunk;
    float *part = p.ws + pidx * kPartialFloats;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4 *)(part + (16 * (nt0 + nt) + c) * kD + 16 * g + 4 * i) = d_run(o, nt, i);
    if (g == 0) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        part[kQT * kD + 16 * (nt0 + nt) + c] = st.m[nt] * kLog2e;   // log2 units, relative to the level
        part[kQT * kD + kQT + 16 * (nt0 + nt) + c] = lsum[nt];
      }
    }
    // Every wavefront of the item holds the same level; the first one stores it.
    if (lane == 0 && nt0 == 0) part[kQT * kD + 2 * kQT] = st.level;
    return;
  }
  OutT *out = (OutT *)p.out + (int64_t)it.bh * p.seq_stride;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int qrow = q0 + 16 * (nt0 + nt) + c;
    if (RAGGED && qrow >= p.L) continue;
    if (p.lse && g == 0) {
      // Natural log-sum-exp: the reference (relative to the scaled level),
      // the level, the log of the row sum, the query x key constant.
      const float f = QK ? mq[nt] : 1.0f;
      p.lse[(int64_t)it.bh * p.L + qrow] =
          st.m[nt] + f * st.level + logf(lsum[nt]) + (QK ? kPadBias * (1.0f - mq[nt]) : 0.0f);
    }
    const float inv = 1.0f / lsum[nt];
    OutT *row = out + (int64_t)qrow * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 y = d_run(o, nt, i) * inv;
      if constexpr (sizeof(OutT) == 2) {
        *(bf16x4 *)(row + 16 * g + 4 * i) = __builtin_convertvector(y, bf16x4);
      } else {
        *(f32x4 *)(row + 16 * g + 4 * i) = y;
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 path
//
// LDS per wavefront: two K tiles and two V tiles of 32 keys x 64 d bf16,
// row-major (128 B per key row).  Tiles are filled straight from HBM with
// buffer_load_dwordx4 ... lds: lane l of instruction u writes the 16 bytes at
// tile + 1024u + 16l (key row 8u + l/8, chunk position l%8).  The 16-byte
// chunk j of key row k is stored at position j ^ f(k):
//   K: f(k) = ((k >> 1) & 7) ^ ((k & 1) << 2) -- the 16-byte A-operand reads
//      (row c, chunk 2k + h) of 8 or 16 consecutive rows hit distinct banks;
//   V: f(k) = ((k >> 1) & 1) << 2             -- the 8-byte transposed reads
//      (rows 16s + 8r + 0..7, 64 contiguous bytes each) spread evenly.
constexpr int kTileBytes = kStep * kD * 2;          // 4 KB
__device__ inline int k_swz(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ inline int v_swz(int row) { return ((row >> 1) & 1) << 2; }

typedef __attribute__((address_space(3))) void lptr_t;
// Word 3 of a raw buffer resource: 32-bit data format, no swizzle, no stride.
constexpr int kBufferWord3 = 0x00020000;

// Scheduling hints: interleave `nmfma` MFMAs with `per` VALU instructions each.
#define BBSA_INTERLEAVE(nmfma, per)                              \
  do {                                                           \
    _Pragma("unroll") for (int _i = 0; _i < (nmfma); ++_i) {     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
      __builtin_amdgcn_sched_group_barrier(0x002, (per), 0);     \
    }                                                            \
  } while (0)

__device__ inline float tree_max16(const f32x16 &v) {
  const float a0 = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
  const float a1 = __builtin_fmaxf(__builtin_fmaxf(v[3], v[4]), v[5]);
  const float a2 = __builtin_fmaxf(__builtin_fmaxf(v[6], v[7]), v[8]);
  const float a3 = __builtin_fmaxf(__builtin_fmaxf(v[9], v[10]), v[11]);
  const float a4 = __builtin_fmaxf(__builtin_fmaxf(v[12], v[13]), v[14]);
  const float b0 = __builtin_fmaxf(__builtin_fmaxf(a0, a1), a2);
  const float b1 = __builtin_fmaxf(__builtin_fmaxf(a3, a4), v[15]);
  return __builtin_fmaxf(b0, b1);
}

// Value of the other half of the wavefront (lane l ^ 32).
__device__ inline float swap_halves(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const int lane = lane_id();
  return __uint_as_float(lane < 32 ? a[1] : a[0]);
}

constexpr int kWaveLds = 4 * kTileBytes;          // 16 KB per wavefront: K and V double buffers

// One wavefront per item, kGroup items per workgroup.  The wavefronts of a
// workgroup run independent items, except that a group of full-row items is
// the kGroup key chunks of one row tile: those merge their partial results
// through LDS at the end (one barrier), so a row of up to kGroup chunks
// needs no separate merge kernel.
template <int MODE>
__global__ __launch_bounds__(kGroup * 64, 2) void bbsa_attn_bf16(Params p) {
  // MASKING: scores get a padding bias (a mask, or positions past L);
  // RAGGED: L is not a multiple of the block; QK: query x key masking.
  constexpr bool MASKING = (MODE & (kModeMask | kModeRagged)) != 0;
  constexpr bool RAGGED = (MODE & kModeRagged) != 0;
  constexpr bool QK = (MODE & kModeQK) != 0;
  const int wv = __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_workitem_id_x() >> 6);
  const Item it = decode_item(p, (int)__builtin_amdgcn_workgroup_id_x(), wv);
  // Idle items only occur as whole groups of full-row items or among middle
  // rows, so no wavefront that leaves here is awaited at the merge barrier.
  if (it.bh >= p.bh_total) return;
  // kGroup wavefront regions first (the LDS transfers address the first
  // 64 KB), then the full-row merge's per-row maxima and sums.
  __shared__ __attribute__((aligned(1024))) unsigned char lds_all[kGroup * kWaveLds + kGroup * 2 * kQT * 4];
  unsigned char *const lds = lds_all + wv * kWaveLds;
  unsigned char *const kbuf = lds;                    // K tile i at kbuf + (i & 1) * kTileBytes
  unsigned char *const vbuf = lds + 2 * kTileBytes;   // V tiles
  float *const merge_ml = (float *)(lds_all + kGroup * kWaveLds);   // [wavefront][64 maxima, 64 sums]

  const int lane = lane_id();
  const int c = lane & 31, h = lane >> 5;             // MFMA 32x32 lane coordinates
  const int G = lane >> 4, cc = lane & 15;            // 16-lane groups of the transposed reads
  const int b = fdiv(it.bh, p.div_heads);
  const bf16_t *Kbh = (const bf16_t *)p.k + (int64_t)it.bh * p.seq_stride;
  const bf16_t *Vbh = (const bf16_t *)p.v + (int64_t)it.bh * p.seq_stride;
  const float *mrow = (MASKING && p.mask) ? p.mask + (int64_t)b * p.L : nullptr;
  const int q0 = it.qblock * p.block + it.qt * kQT;

  // DMA sources inside a 32-key step (elements): instruction u loads key row
  // 8u + lane/8, chunk (lane % 8) ^ f(row).
  const int drow = lane >> 3;
  int kdma[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kdma[u] = (8 * u + drow) * kD + 8 * ((lane & 7) ^ k_swz(8 * u + drow));
  const int vdma = drow * kD + 8 * ((lane & 7) ^ v_swz(drow));   // v_swz(8u + drow) == v_swz(drow)
  // K A-operand reads, k-step k: row c, chunk 2k + h.
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = c * 128 + 16 * ((2 * kk + h) ^ k_swz(c));
  // V^T transposed reads for d-tile dt, key step s, run r: the lane reads key row
  // 16s + 8r + 4(G/2) + cc/4, d = 32dt + 16(G%2) + 4(cc%4) .. +3.
  int voff[2];
  {
    const int row = 4 * (G >> 1) + (cc >> 2);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int chunk = 4 * dt + 2 * (G & 1) + ((cc & 3) >> 1);
      voff[dt] = row * 128 + 16 * (chunk ^ v_swz(row)) + 8 * (cc & 1);
    }
  }

  // Q^T operand: lane (c, h) holds Q[q0 + 32nt + c][16k + 8h .. +7] (rows
  // past L, which exist only with a ragged length, read row L - 1 and are
  // never stored).
  bf16x8 qf[2][4];
  {
    const bf16_t *Q = (const bf16_t *)p.q + (int64_t)it.bh * p.seq_stride;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = RAGGED ? min(q0 + 32 * nt + c, p.L - 1) : q0 + 32 * nt + c;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qf[nt][kk] = *(const bf16x8 *)(Q + (int64_t)row * kD + 16 * kk + 8 * h);
    }
  }
  // Query-side mask value of the lane's two query columns (query x key
  // masking scales the key bias by it; the rest of -10000 (1 - m_q m_k) is a
  // per-row constant that cancels in the softmax).
  float mq[2] = {1.0f, 1.0f};
  if (QK) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = q0 + 32 * nt + c;
      mq[nt] = (RAGGED && row >= p.L) ? 0.0f : mrow[row];
    }
  }

  // The plan entries are merged into the walk after the prologue's wait: the
  // first two K tiles lie in the first block and do not need them.
  int rnd, rslot;
  KeyWalk walk = make_walk_base(p, it, lane, rnd, rslot);
  int n = __builtin_amdgcn_readfirstlane(walk.n_steps);   // >= 2, or 0 for an empty chunk
  // First key of step i: block i / steps_per_block of the list (a lane of
  // walk.blk), then 32 keys per step inside it.  Branch-free; uniform.
  const int lg_spb = walk.steps_per_block >> 1;      // steps_per_block is 2 or 4
  auto key_of = [&](int i) -> int {
    return __builtin_amdgcn_readlane(walk.blk, i >> lg_spb) * p.block + (i & (walk.steps_per_block - 1)) * kStep;
  };

  // Key blocks whose keys all have mask 0 hold scores 10000 below those of a
  // key with mask 1.  Once the tile's list holds such a key, their
  // probabilities are exactly zero in fp32 (and in exact arithmetic to far
  // below fp64's range: e^-9890 and less), and they leave the reference max
  // alone, so the tile drops them from its list and the result is the same.
  // List position 0 stays (its transfers are issued before the list is
  // final).  With query x key masking a query row of mask 0 sees no key
  // bias at all, so only tiles whose rows all have mask 1 drop blocks.
  // The probe reads two mask values per lane and 64 keys of each listed
  // block (block 64: lanes 32-63 repeat lanes 0-31) after the prologue's
  // wait, when the plan entries are in the list.
  const bool wide = p.block > 64;
  const int nblk0 = n >> lg_spb;
  struct MaskProbe {
    float m[8][2];
  };
  const int probe_voff = (wide ? 2 * lane : 2 * (lane & 31)) * 4;
  const __amdgpu_buffer_rsrc_t mrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)mrow, (short)0, MASKING ? p.L * 4 : 0, kBufferWord3);
  // Mask values of list positions [t0, t1) (at most 8; the rest repeat t1 - 1).
  auto probe_load = [&](int t0, int t1, MaskProbe &pr) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int blk = __builtin_amdgcn_readlane(walk.blk, min(t0 + u, t1 - 1));
      const auto mv = __builtin_amdgcn_raw_buffer_load_b64(mrs, probe_voff, blk * p.block * 4, 0);
      pr.m[u][0] = __uint_as_float(mv[0]);
      pr.m[u][1] = __uint_as_float(mv[1]);
    }
  };
  // Bit t of padded: every key of position t has mask 0 (either sign); valid:
  // the largest mask value probed is 1 (a key of mask 1 exists; values above
  // 1 only make the test fail, which leaves every block in).
  auto probe_bits = [&](int t0, int t1, const MaskProbe &pr, uint64_t &padded, bool &valid) {
    float mx = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t bit = (t0 + u < t1) ? (1ull << (t0 + u)) : 0ull;
      const uint32_t nz = (__float_as_uint(pr.m[u][0]) | __float_as_uint(pr.m[u][1])) << 1;
      if (!__builtin_amdgcn_ballot_w64(nz != 0u)) padded |= bit;
      mx = __builtin_fmaxf(mx, __builtin_fmaxf(pr.m[u][0], pr.m[u][1]));
    }
    valid |= __builtin_amdgcn_ballot_w64(mx == 1.0f) != 0;
  };
  // Drop the padded positions (stable compaction: kept position t moves to
  // the number of kept positions below it, dropped ones follow in order, a
  // permutation of the 64 lanes that leaves lanes past the list in place).
  // Returns the new step count.
  auto drop_padded = [&](int n_in, uint64_t padded, bool valid) -> int {
    if (!valid || (QK && __builtin_amdgcn_ballot_w64(mq[0] != 1.0f || mq[1] != 1.0f))) return n_in;
    const int nblk = n_in >> lg_spb;
    const uint64_t all = nblk >= 64 ? ~0ull : (1ull << nblk) - 1;
    const uint64_t keep = (all & ~padded) | 1ull;
    if (keep == all) return n_in;
    const int nkeep = __builtin_popcountll(keep);
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0u));
    const int dst = ((keep >> lane) & 1) ? rank : nkeep + (lane - rank);
    walk.blk = __builtin_amdgcn_ds_permute(dst * 4, walk.blk);
    return nkeep * walk.steps_per_block;
  };

  // K and V of this (batch, head) as buffer resources (L x d rows): the DMA
  // source of a lane is a 32-bit per-lane offset plus a scalar offset for the
  // step.
  // The record count is an unsigned 32-bit byte count: L * 128 reaches 2^31
  // at the longest supported L, so it is formed in 64 bits and passed as its
  // low 32 bits.
  const int kv_bytes = (int)(uint32_t)(p.seq_stride * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)Kbh, (short)0, kv_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)Vbh, (short)0, kv_bytes, kBufferWord3);
  // The instruction offset 1024u moves both the LDS destination and the
  // source by 1024u bytes: one M0 value per tile.
  int kdma_b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kdma_b[u] = 2 * kdma[u] - 1024 * u;
  const int vdma_b = 2 * vdma;
  // The hardware range check covers the per-lane offset and the instruction
  // offset, not the scalar offset.  Every key of an aligned length lies
  // inside the pair's rows, so the step's row offset rides in the scalar
  // offset; with a ragged length the last block reaches past L, so there the
  // row offset joins the per-lane offset and the rows past L read as zeros.
  auto dma_k = [&](int key0, int slot) {
    unsigned char *dst = kbuf + slot * kTileBytes;
    const int so = RAGGED ? 0 : key0 * (kD * 2);
    const int vo = RAGGED ? key0 * (kD * 2) : 0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lptr_t *)dst, 16, kdma_b[0] + vo, so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lptr_t *)dst, 16, kdma_b[1] + vo, so, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lptr_t *)dst, 16, kdma_b[2] + vo, so, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lptr_t *)dst, 16, kdma_b[3] + vo, so, 3072, 0);
  };
  auto dma_v = [&](int key0, int slot) {
    unsigned char *dst = vbuf + slot * kTileBytes;
    const int so = RAGGED ? 0 : key0 * (kD * 2);
    const int vo = RAGGED ? vdma_b + key0 * (kD * 2) : vdma_b;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lptr_t *)dst, 16, vo, so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lptr_t *)dst, 16, vo, so, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lptr_t *)dst, 16, vo, so, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lptr_t *)dst, 16, vo, so, 3072, 0);
  };
  // Mask value of key key0 + lane % 32 (one float per lane, lanes l and l + 32
  // equal); positions past L are padding.
  auto load_mask = [&](int key0) -> float {
    if constexpr (!MASKING) {
      return 1.0f;
    } else if constexpr (RAGGED) {
      const int key = key0 + c;
      return key < p.L ? (mrow ? mrow[key] : 1.0f) : 0.0f;
    } else {
      return mrow[key0 + c];
    }
  };
  auto read_k = [&](int slot, bf16x8 (&kc)[4]) {
    const unsigned char *src = kbuf + slot * kTileBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kc[kk] = *(const bf16x8 *)(src + koff[kk]);
  };
  auto read_vt = [&](int slot, bf16x8 (&vt)[2][2]) {
    const unsigned char *src = vbuf + slot * kTileBytes;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + voff[dt] + 2048 * s));
        const s16x4 bb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + voff[dt] + 2048 * s + 1024));
        vt[dt][s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };

  // Online softmax state (log2 units).  mref: reference max of each of the
  // lane's two query columns (equal in lanes c and c + 32); l: lane-partial
  // row sums, two running chains per column that the dot2 instructions
  // accumulate into directly (no per-step temporaries).
  float mref[2] = {0.0f, 0.0f}, l[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  f32x16 o[2][2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][nt][e] = 0.0f;

  // S(j) for query half nt: 32 keys x 32 queries.
  auto score_half = [&](const bf16x8 (&kc)[4], int nt) -> f32x16 {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[kk], qf[nt][kk], acc, 0, 0, 0);
    return acc;
  };
  // Padding bias for the step whose lane value is mval: nothing when every key
  // is valid, one scalar when all 32 keys share a mask value, per key otherwise.
  auto apply_mask = [&](f32x16 (&sc)[2], float mval) {
    if (!MASKING) return;
    const unsigned long long pad = __builtin_amdgcn_ballot_w64(mval != 1.0f);
    if (!pad) return;
    const float m0 = __builtin_amdgcn_readfirstlane(mval);
    const float bl = kPadBias;
    if (!__builtin_amdgcn_ballot_w64(mval != m0)) {
      const float bias = bl * (1.0f - m0);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sc[nt] += QK ? bias * mq[nt] : bias;
      return;
    }
    // Per key: register 4j + i holds key 8j + 4h + i, whose mask sits in lane 8j + 4h + i.
    f32x16 bias;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 8 * (e >> 2) + 4 * h + (e & 3);
      bias[e] = bl * (1.0f - __uint_as_float(__builtin_amdgcn_ds_bpermute(key * 4, __float_as_uint(mval))));
    }
    if constexpr (QK) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[nt][e] = __builtin_fmaf(bias[e], mq[nt], sc[nt][e]);
    } else {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) sc[nt] += bias;
    }
  };
  // p = 2^(s - mref) for query half nt, rounded to bf16 for the PV product; the
  // row sums add the rounded values (the ones the product uses).
  auto softmax_half = [&](f32x16 &sc, int nt, bf16x8 (&pfo)[2]) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const float nm = mref[nt];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      sc[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], kLog2e, -nm));
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 lo = {sc[8 * s + 0], sc[8 * s + 1], sc[8 * s + 2], sc[8 * s + 3]};
      const f32x4 hi = {sc[8 * s + 4], sc[8 * s + 5], sc[8 * s + 6], sc[8 * s + 7]};
      pfo[s] = __builtin_shufflevector(__builtin_convertvector(lo, bf16x4), __builtin_convertvector(hi, bf16x4),
                                       0, 1, 2, 3, 4, 5, 6, 7);
      l[nt][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pfo[s], pfo[s], 0, 1), ones, l[nt][0], false);
      l[nt][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pfo[s], pfo[s], 2, 3), ones, l[nt][1], false);
      l[nt][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pfo[s], pfo[s], 4, 5), ones, l[nt][0], false);
      l[nt][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pfo[s], pfo[s], 6, 7), ones, l[nt][1], false);
    }
  };

  if (n == 0) {
    // An empty key chunk (a row shorter than kGroup blocks): a neutral partial.
    mref[0] = mref[1] = kInitMax;
  } else {
    // Prologue: K(0), K(1) and their mask values; S(0).  Each step's padding
    // bias is added at the top of the iteration that takes its softmax.
    const int key_0 = key_of(0), key_1 = key_of(1);
    float mk_cur = load_mask(key_0);            // mask of step j (j = 0)
    dma_k(key_0, 0);
    float mk_next = load_mask(key_1);           // mask of step j + 1
    dma_k(key_1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    merge_plan(p, walk, rnd, rslot);
    constexpr bool kProbe = MASKING && !RAGGED;
    const bool probe = kProbe && p.skip_padded;
    MaskProbe pr_a, pr_b;
    if (kProbe && probe) {
      probe_load(0, min(nblk0, 8), pr_a);
      if (nblk0 > 8) probe_load(8, min(nblk0, 16), pr_b);
    }
    if (kProbe && probe) {
      uint64_t padded = 0;
      bool valid = false;
      probe_bits(0, min(nblk0, 8), pr_a, padded, valid);
      if (nblk0 > 8) probe_bits(8, min(nblk0, 16), pr_b, padded, valid);
      // Lists longer than 16 blocks (more than 11 random blocks): the rest, 8 at a time.
      for (int t0 = 16; t0 < nblk0; t0 += 8) {
        probe_load(t0, min(nblk0, t0 + 8), pr_a);
        probe_bits(t0, min(nblk0, t0 + 8), pr_a, padded, valid);
      }
      n = __builtin_amdgcn_readfirstlane(drop_padded(n, padded, valid));
    }
    f32x16 sc[2];
    {
      bf16x8 kc[4];
      read_k(0, kc);
      sc[0] = score_half(kc, 0);
      sc[1] = score_half(kc, 1);
    }

    bf16x8 pf[2][2];    // P of the previous step: [nt][key step s]
    bool resc_pending = false;
    float alpha_pending[2] = {1.0f, 1.0f};
    // One pipeline iteration j: the PV product of step j-1, the softmax of step
    // j (in sc) and S(j+1), computed half by half into the registers the
    // softmax of that half has just consumed.
    auto iteration = [&](int j, auto has_s_t, auto has_pv_t, auto first_t, auto steady_t) {
      constexpr bool HAS_S = decltype(has_s_t)::value;
      constexpr bool HAS_PV = decltype(has_pv_t)::value;
      constexpr bool FIRST = decltype(first_t)::value;
      constexpr bool STEADY = decltype(steady_t)::value;   // j + 2 < n
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // K(j+1), V(j-1), mask(j+2) from iteration j-1
      bf16x8 kc[4], vt[2][2];
      if (HAS_S) read_k((j + 1) & 1, kc);
      if (HAS_PV) read_vt((j - 1) & 1, vt);
      apply_mask(sc, mk_cur);
      float mk_n2 = 1.0f;
      if (STEADY || j + 2 < n) {
        const int kk0 = key_of(j + 2);
        mk_n2 = load_mask(kk0);
        dma_k(kk0, j & 1);
      }
      dma_v(key_of(j), j & 1);

      // A rescale decided in the previous iteration applies to O now: after the
      // PV product of step j-2 and before that of step j-1 (whose probabilities
      // already use the new reference).
      if (resc_pending) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) o[dt][nt] *= alpha_pending[nt];
        resc_pending = false;
      }
      // Rescale decision for step j (before its exponentials).
      {
        float ml[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          ml[nt] = tree_max16(sc[nt]) * kLog2e - mref[nt];
        const bool need = FIRST || ml[0] > kTauLog2 || ml[1] > kTauLog2;
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const float mrow = __builtin_fmaxf(ml[nt], swap_halves(ml[nt]));
            const float sh = (FIRST || mrow > kTauLog2) ? mrow : 0.0f;
            mref[nt] += sh;
            alpha_pending[nt] = __builtin_amdgcn_exp2f(-sh);
            if (!FIRST) {
              l[nt][0] *= alpha_pending[nt];
              l[nt][1] *= alpha_pending[nt];
            }
          }
          // The first step has no O to rescale.
          resc_pending = !FIRST;
        }
      }

      if (HAS_PV) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
              o[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt[dt][s], pf[nt][s], o[dt][nt], 0, 0, 0);
      }
      softmax_half(sc[0], 0, pf[0]);
      if (HAS_S) sc[0] = score_half(kc, 0);
      softmax_half(sc[1], 1, pf[1]);
      if (HAS_S) sc[1] = score_half(kc, 1);
      if (HAS_PV) {
        BBSA_INTERLEAVE(8, 5);
      }
      if (HAS_S) {
        BBSA_INTERLEAVE(4, 10);
        BBSA_INTERLEAVE(4, 2);
      }
      mk_cur = mk_next;
      mk_next = mk_n2;
    };

    using T = std::true_type;
    using F = std::false_type;
    iteration(0, T{}, F{}, T{}, F{});
    int j = 1;
    for (; j + 2 < n; ++j) iteration(j, T{}, T{}, F{}, T{});
    for (; j < n - 1; ++j) iteration(j, T{}, T{}, F{}, F{});
    iteration(n - 1, F{}, T{}, F{}, F{});
    // Drain: PV of the last step.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (resc_pending) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[dt][nt] *= alpha_pending[nt];
    }
    {
      bf16x8 vt[2][2];
      read_vt((n - 1) & 1, vt);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            o[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt[dt][s], pf[nt][s], o[dt][nt], 0, 0, 0);
    }
  }

  // Finish: full row sums, then normalised bf16 output or a split-K partial.
  float lsum[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lp = l[nt][0] + l[nt][1];
    lsum[nt] = lp + swap_halves(lp);
  }
  if (it.grow >= 0) {
    // Full-row chunk: each wavefront leaves its unnormalised 64 x 64 fp32
    // tile in its own region (16-byte chunk k of row q at chunk k ^ (q & 15)
    // of the 256-byte LDS row) and its row maxima and sums in merge_ml.
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 y = {o[dt][nt][4 * jj], o[dt][nt][4 * jj + 1], o[dt][nt][4 * jj + 2], o[dt][nt][4 * jj + 3]};
          const int q = 32 * nt + c, k = 8 * dt + 2 * jj + h;
          *(f32x4 *)(lds + q * 256 + 16 * (k ^ (q & 15))) = y;
        }
    if (h == 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        merge_ml[wv * 2 * kQT + 32 * nt + c] = mref[nt];
        merge_ml[wv * 2 * kQT + kQT + 32 * nt + c] = lsum[nt];
      }
    }
    __syncthreads();   // the kGroup wavefronts are the kGroup chunks of this row tile
    // Wavefront wv merges rows 16 wv .. 16 wv + 15; lane: row r, d = 16 qd .. 16 qd + 15.
    const int r = 16 * wv + (lane >> 2), qd = lane & 3;
    float mi[kGroup], M = kInitMax;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      mi[i] = merge_ml[i * 2 * kQT + r];
      M = __builtin_fmaxf(M, mi[i]);
    }
    float den = 0.0f;
    f32x4 acc[4] = {};
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float w = __builtin_amdgcn_exp2f(mi[i] - M);
      den += w * merge_ml[i * 2 * kQT + kQT + r];
      const unsigned char *trow = lds_all + i * kWaveLds + r * 256;
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] += w * *(const f32x4 *)(trow + 16 * ((4 * qd + t) ^ (r & 15)));
    }
    if (p.nparts == 1) {
      if (!RAGGED || q0 + r < p.L) {
        const float inv = 1.0f / den;
        bf16_t *orow = (bf16_t *)p.out + (int64_t)it.bh * p.seq_stride + (int64_t)(q0 + r) * kD + 16 * qd;
        const bf16x8 v0 = __builtin_shufflevector(__builtin_convertvector(acc[0] * inv, bf16x4),
                                                  __builtin_convertvector(acc[1] * inv, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 v1 = __builtin_shufflevector(__builtin_convertvector(acc[2] * inv, bf16x4),
                                                  __builtin_convertvector(acc[3] * inv, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
        __builtin_nontemporal_store(v0, (bf16x8 *)orow);
        __builtin_nontemporal_store(v1, (bf16x8 *)(orow + 8));
        if (p.lse && qd == 0) {
          // Natural log-sum-exp of the row: (M + log2 den) / log2(e), plus the
          // query x key constant -10000 (1 - m_q).
          const float cq = QK ? kPadBias * (1.0f - mrow[q0 + r]) : 0.0f;
          p.lse[(int64_t)it.bh * p.L + q0 + r] = (M + log2f(den)) * kLn2 + cq;
        }
      }
    } else {
      // A partial over this group of chunks for the merge kernel (bias
      // level 0: the bf16 scores carry the whole padding bias).
      const int64_t pidx = (((int64_t)it.bh * p.n_rows_global + it.grow) * p.qtiles + it.qt) * p.nparts + it.chunk / kGroup;
      float *part = p.ws + pidx * kPartialFloats;
#pragma unroll
      for (int t = 0; t < 4; ++t) *(f32x4 *)(part + r * kD + 16 * qd + 4 * t) = acc[t];
      if (qd == 0) {
        part[kQT * kD + r] = M;
        part[kQT * kD + kQT + r] = den;
      }
      if (wv == 0 && lane == 0) part[kQT * kD + 2 * kQT] = 0.0f;
    }
    return;
  }
  // The normalised 64 x 64 bf16 tile goes through LDS (the free K buffers)
  // so that the global stores are whole 128-byte rows: 16-byte chunk k of
  // row q sits at chunk k ^ (q & 7) of the LDS row.
  {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float inv = 1.0f / lsum[nt];
      const int q = 32 * nt + c;
      unsigned char *lrow = kbuf + q * 128;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 y = {o[dt][nt][4 * jj], o[dt][nt][4 * jj + 1], o[dt][nt][4 * jj + 2], o[dt][nt][4 * jj + 3]};
          *(bf16x4 *)(lrow + 16 * ((4 * dt + jj) ^ (q & 7)) + 8 * h) = __builtin_convertvector(y * inv, bf16x4);
        }
    }
  }
  if (p.lse && h == 0) {
    // Natural log-sum-exp of each row: (mref + log2 l) / log2(e), plus the
    // query x key constant -10000 (1 - m_q).
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = q0 + 32 * nt + c;
      if (!RAGGED || row < p.L)
        p.lse[(int64_t)it.bh * p.L + row] = (mref[nt] + log2f(lsum[nt])) * kLn2 +
                                            (QK ? kPadBias * (1.0f - mq[nt]) : 0.0f);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the tile is in this wavefront's own LDS region
  {
    bf16_t *out = (bf16_t *)p.out + (int64_t)it.bh * p.seq_stride + (int64_t)q0 * kD;
    const int ch = lane & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = 8 * i + (lane >> 3);
      const bf16x8 v = *(const bf16x8 *)(kbuf + q * 128 + 16 * (ch ^ (q & 7)));
      if (!RAGGED || q0 + q < p.L)
        __builtin_nontemporal_store(v, (bf16x8 *)(out + (int64_t)q * kD + 8 * ch));   // never re-read here
    }
  }
}

// ---------------------------------------------------------------- fp32 path
//
// Same walk and softmax on MFMA 16x16x4 f32, one item per workgroup of
// kF32Waves wavefronts that split its query rows (all read the same K and V
// rows, which the later wavefronts find in the caches).  The d contraction
// uses the order d = 16g + s (s = MFMA step) on both operands; the PV
// contraction steps over (mt, i) with key 16mt + 4g + i, read straight from
// memory.
template <int MODE>
__global__ __launch_bounds__(64 * kF32Waves) void bbsa_attn_f32(Params p) {
  constexpr bool MASKING = (MODE & (kModeMask | kModeRagged)) != 0;
  constexpr bool RAGGED = (MODE & kModeRagged) != 0;
  constexpr bool QK = (MODE & kModeQK) != 0;
  const Item it = decode_item(p, (int)__builtin_amdgcn_workgroup_id_x(), 0);
  if (it.bh >= p.bh_total) return;
  // The kF32Waves wavefronts of a workgroup split the item's 64 query rows:
  // wavefront wv owns the 16-query tiles nt0 .. nt0 + kNT - 1.
  const int nt0 = kNT * __builtin_amdgcn_readfirstlane((int)__builtin_amdgcn_workitem_id_x() >> 6);
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  const int b = fdiv(it.bh, p.div_heads);
  const float *Q = (const float *)p.q + (int64_t)it.bh * p.seq_stride;
  const float *K = (const float *)p.k + (int64_t)it.bh * p.seq_stride;
  const float *V = (const float *)p.v + (int64_t)it.bh * p.seq_stride;
  const float *mrow = (MASKING && p.mask) ? p.mask + (int64_t)b * p.L : nullptr;
  const int q0 = it.qblock * p.block + it.qt * kQT;

  // Query rows past L (a ragged length) read row L - 1 and are never stored.
  float qf[kNT][16];
  float mq[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int row = q0 + 16 * (nt0 + nt) + c;
    const int lrow = RAGGED ? min(row, p.L - 1) : row;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f32x4 x = *(const f32x4 *)(Q + (int64_t)lrow * kD + 16 * g + 4 * s4);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[nt][4 * s4 + e] = x[e];
    }
    mq[nt] = QK ? ((RAGGED && row >= p.L) ? 0.0f : mrow[row]) : 1.0f;
  }

  const KeyWalk walk = make_walk(p, it);
  SoftmaxState st;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) { st.m[nt] = kInitMax; st.l[nt] = 0.0f; }
  st.level = MASKING ? kInitMax : 0.0f;
  f32x4 o[4][kNT];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operands of one step: K rows 16mt + c (d = 16g .. 16g+15) and the V
  // values of keys 16mt + 4g + i at d = 4c + dt (one 16-byte load per key:
  // the PV product's d-tile dt holds the d = dt mod 4 columns).  The next
  // step's are loaded while the current one is computed.
  struct StepOperands {
    float kf[2][16];
    float va[2][4][4];
    f32x4 mc[2];
  };
  // With a ragged length, key rows past L read as zeros (and count as padding).
  auto load_step = [&](int key0, StepOperands &x) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int kr = key0 + 16 * mt + c;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        f32x4 v4 = *(const f32x4 *)(K + (int64_t)(RAGGED ? min(kr, p.L - 1) : kr) * kD + 16 * g + 4 * s4);
        if (RAGGED && kr >= p.L) v4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) x.kf[mt][4 * s4 + e] = v4[e];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vr = key0 + 16 * mt + 4 * g + i;
        f32x4 v4 = *(const f32x4 *)(V + (int64_t)(RAGGED ? min(vr, p.L - 1) : vr) * kD + 4 * c);
        if (RAGGED && vr >= p.L) v4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) x.va[mt][i][dt] = v4[dt];
      }
    }
    if constexpr (RAGGED) {
      // Element loads: the mask row of a ragged length is not 16-byte aligned.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + 16 * mt + 4 * g + e;
          x.mc[mt][e] = key < p.L ? (mrow ? mrow[key] : 1.0f) : 0.0f;
        }
    } else if constexpr (MASKING) {
      x.mc[0] = *(const f32x4 *)(mrow + key0 + 4 * g);
      x.mc[1] = *(const f32x4 *)(mrow + key0 + 16 + 4 * g);
    }
  };

  // A middle row split into key parts walks list positions [pos0, pos1).
  int pos0 = 0, n_steps = walk.n_steps;
  if (it.grow < 0 && p.mparts > 1) {
    const int nblk = walk.n_steps / walk.steps_per_block;
    pos0 = it.chunk * nblk / p.mparts;
    n_steps = ((it.chunk + 1) * nblk / p.mparts - pos0) * walk.steps_per_block;
  }
  WalkCursor cur;
  cur.start_at(p, walk, pos0);
  StepOperands nxt;
  load_step(cur.key0, nxt);
  for (int step = 0; step < n_steps; ++step) {
    const StepOperands x = nxt;
    if (step + 1 < n_steps) {
      cur.advance(p, walk);
      load_step(cur.key0, nxt);
    }
    f32x4 s[2][kNT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.kf[mt][ks], qf[nt][ks], acc, 0, 0, 0);
        s[mt][nt] = acc;
      }
    if (MASKING) {
      f32x4 mc[2] = {x.mc[0], x.mc[1]};
      apply_mask<QK>(s, mc, st, mq);
    }
    softmax_rescale(s, st, o);
    softmax_exp(s, st);
    row_sum_f32(s, st);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.va[mt][i][dt], s[mt][nt][i], o[dt][nt], 0, 0, 0);
  }
  finish_item<float, RAGGED, QK>(p, it, q0, nt0, st, o, mq);
}

// ---------------------------------------------------------------- split-K merge
//
// One 64-thread workgroup per (batch, head, full row, query tile, 4-query
// slice); 16 threads per query, each owning 4 consecutive d:
// out = sum_c w_c O_c / sum_c w_c l_c with w_c = 2^(m_c - M), M the largest
// reference maximum (log2 units), accumulated in one pass.
constexpr int kMergeBatch = 8;   // chunks whose loads are in flight together
template <typename OutT>
__global__ __launch_bounds__(64) void bbsa_combine(Params p) {
  const int wg = (int)__builtin_amdgcn_workgroup_id_x();
  const int slice = wg % kMergeSlices, idx = wg / kMergeSlices;
  const int qt = idx % p.qtiles;
  const int t2 = idx / p.qtiles;
  const int rows = p.comb_rows_global + p.comb_rows_mid;
  const int row = t2 % rows;
  const int bh = t2 / rows;
  // Full rows first (their chunk partials), then the middle rows' key parts.
  const bool full_row = row < p.comb_rows_global;
  const int i_mid = row - p.comb_rows_global;
  const int np = full_row ? p.nparts : p.mparts;
  const int64_t first = full_row ? (((int64_t)bh * p.n_rows_global + row) * p.qtiles + qt) * p.nparts
                                 : p.mid_part_base + (((int64_t)bh * (p.nb - 2) + i_mid) * p.qtiles + qt) * p.mparts;
  const float *base = p.ws + first * kPartialFloats;
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int q = 4 * slice + (tid >> 4), dq = tid & 15;
  const int qblock = full_row ? ((p.n_rows_global == 2) ? (row == 0 ? 0 : p.nb - 1) : row) : 1 + i_mid;
  const int qrow = qblock * p.block + qt * kQT + q;
  if ((p.mode & kModeRagged) && qrow >= p.L) return;   // a row past a ragged length: nothing to write
  // Query x key masking scales each row's bias, and so its levels, by the
  // row's mask value.
  const bool qk = (p.mode & kModeQK) != 0;
  const float mq = qk ? p.mask[(int64_t)fdiv(bh, p.div_heads) * p.L + qrow] : 1.0f;
  // Each partial's maxima are relative to its padding-bias level: partial c
  // enters with exponent m_c + mq (level_c - top level) * log2(e), where the
  // level difference is exact for 0/1 masks (and 0 on the bf16 path).
  // bf16 partials all have level 0 (their scores carry the whole bias), so
  // their merge needs no first pass over the level words.
  constexpr bool kLevels = sizeof(OutT) != 2;
  float top = 0.0f;
  if constexpr (kLevels) {
    top = kInitMax;
    for (int ch = 0; ch < np; ++ch) top = __builtin_fmaxf(top, base[(int64_t)ch * kPartialFloats + kQT * kD + 2 * kQT]);
  }
  // One pass, kMergeBatch chunks at a time: all loads of a batch are issued
  // before any of them is used; the running (M, den, acc) is rescaled when a
  // batch raises the maximum.
  float M = kInitMax, den = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < np; c0 += kMergeBatch) {
    float mc[kMergeBatch], lc[kMergeBatch];
    f32x4 oc[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int ch = min(c0 + u, np - 1);   // repeats stay unused
      const float *part = base + (int64_t)ch * kPartialFloats;
      mc[u] = kLevels ? part[kQT * kD + q] + mq * (part[kQT * kD + 2 * kQT] - top) * kLog2e : part[kQT * kD + q];
      lc[u] = part[kQT * kD + kQT + q];
      oc[u] = *(const f32x4 *)(part + q * kD + 4 * dq);
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (c0 + u < np) Mb = __builtin_fmaxf(Mb, mc[u]);
    const float r = __builtin_amdgcn_exp2f(M - Mb);
    den *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w = (c0 + u < np) ? __builtin_amdgcn_exp2f(mc[u] - Mb) : 0.0f;
      den += w * lc[u];
      acc += w * oc[u];
    }
    M = Mb;
  }
  const f32x4 y = acc * (1.0f / den);
  if (p.lse && dq == 0)
    p.lse[(int64_t)bh * p.L + qrow] =
        (M + log2f(den)) * kLn2 + mq * top + (qk ? kPadBias * (1.0f - mq) : 0.0f);
  OutT *dst = (OutT *)p.out + (int64_t)bh * p.seq_stride + (int64_t)qrow * kD + 4 * dq;
  if constexpr (sizeof(OutT) == 2) {
    *(bf16x4 *)dst = __builtin_convertvector(y, bf16x4);
  } else {
    *(f32x4 *)dst = y;
  }
}

// ---------------------------------------------------------------- host side

// Library-owned split-K workspaces, one per (device, stream): calls on one
// stream are ordered by the stream, calls on different streams never share
// a buffer.  A workspace grows in powers of two; the buffer it outgrows is
// kept (not freed) until bbsa_release_workspace, because kernels already
// enqueued, or a HIP graph captured earlier, may still use it.
struct DeviceWorkspace {
  void *ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_mutex;                                          // guards g_ws, g_retired
std::map<std::pair<int, hipStream_t>, DeviceWorkspace> g_ws;
std::vector<std::pair<int, void *>> g_retired;               // (device, buffer)

constexpr int kMaxTimed = 4096;
struct Timing {
  std::mutex mu;                                             // guards everything below
  bool enabled = false;
  bool created = false;
  int n = 0;
  hipEvent_t ev[kMaxTimed][4];
  bool has_combine[kMaxTimed];
};
Timing g_timing;

int ensure_workspace(size_t bytes, hipStream_t stream, float **ws) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BBSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceWorkspace &w = g_ws[std::make_pair(dev, stream)];
  if (w.bytes < bytes) {
    // Allocating is not allowed while the stream is being captured into a
    // graph: the caller runs one eager call of the shape first.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return BBSA_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return BBSA_ERR_CAPTURE;
    size_t grow = (size_t)1 << 20;
    while (grow < bytes) grow <<= 1;
    void *ptr = nullptr;
    if (hipMalloc(&ptr, grow) != hipSuccess) return BBSA_ERR_HIP;
    if (w.ptr) g_retired.emplace_back(dev, w.ptr);
    w.ptr = ptr;
    w.bytes = grow;
  }
  *ws = (float *)w.ptr;
  return BBSA_OK;
}

}  // namespace

// The library's per-(device, stream) workspace for other kernels of the
// library (the backward's split partials), with the same growth rules.
int bbsa_sched::library_workspace(size_t bytes, hipStream_t stream, float **ws) {
  return ensure_workspace(bytes, stream, ws);
}

namespace {

// Enqueue the kernels of a validated call (its workspace pointer set).
int launch_forward(const Launch &ln, hipStream_t stream, bbsa_dtype dtype, int status) {
  const Params &p = ln.p;
  std::unique_lock<std::mutex> tlock(g_timing.mu);
  const bool timed = g_timing.enabled && g_timing.n < kMaxTimed;
  const int tslot = g_timing.n;
  if (timed) {
    g_timing.n++;
    g_timing.has_combine[tslot] = ln.comb_grid > 0;
  } else {
    tlock.unlock();
  }
  if (timed && hipEventRecord(g_timing.ev[tslot][0], stream) != hipSuccess) return BBSA_ERR_HIP;
  const dim3 g1((unsigned)ln.grid), b1((unsigned)ln.block_threads);
  switch (p.mode | (dtype == BBSA_BF16 ? 0 : 8)) {
    case 0: hipLaunchKernelGGL(bbsa_attn_bf16<0>, g1, b1, 0, stream, p); break;
    case kModeMask: hipLaunchKernelGGL(bbsa_attn_bf16<kModeMask>, g1, b1, 0, stream, p); break;
    case kModeRagged: hipLaunchKernelGGL(bbsa_attn_bf16<kModeRagged>, g1, b1, 0, stream, p); break;
    case kModeMask | kModeRagged:
      hipLaunchKernelGGL(bbsa_attn_bf16<kModeMask | kModeRagged>, g1, b1, 0, stream, p);
      break;
    case kModeMask | kModeQK: hipLaunchKernelGGL(bbsa_attn_bf16<kModeMask | kModeQK>, g1, b1, 0, stream, p); break;
    case kModeMask | kModeRagged | kModeQK:
      hipLaunchKernelGGL(bbsa_attn_bf16<kModeMask | kModeRagged | kModeQK>, g1, b1, 0, stream, p);
      break;
    case 8: hipLaunchKernelGGL(bbsa_attn_f32<0>, g1, b1, 0, stream, p); break;
    case 8 | kModeMask: hipLaunchKernelGGL(bbsa_attn_f32<kModeMask>, g1, b1, 0, stream, p); break;
    case 8 | kModeRagged: hipLaunchKernelGGL(bbsa_attn_f32<kModeRagged>, g1, b1, 0, stream, p); break;
    case 8 | kModeMask | kModeRagged:
      hipLaunchKernelGGL(bbsa_attn_f32<kModeMask | kModeRagged>, g1, b1, 0, stream, p);
      break;
    case 8 | kModeMask | kModeQK: hipLaunchKernelGGL(bbsa_attn_f32<kModeMask | kModeQK>, g1, b1, 0, stream, p); break;
    case 8 | kModeMask | kModeRagged | kModeQK:
      hipLaunchKernelGGL(bbsa_attn_f32<kModeMask | kModeRagged | kModeQK>, g1, b1, 0, stream, p);
      break;
    default: return BBSA_ERR_ARG;
  }
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  if (timed && hipEventRecord(g_timing.ev[tslot][1], stream) != hipSuccess) return BBSA_ERR_HIP;
  if (ln.comb_grid > 0) {
    if (timed && hipEventRecord(g_timing.ev[tslot][2], stream) != hipSuccess) return BBSA_ERR_HIP;
    const dim3 g2((unsigned)ln.comb_grid), b2(64);
    if (dtype == BBSA_BF16) hipLaunchKernelGGL(bbsa_combine<bf16_t>, g2, b2, 0, stream, p);
    else hipLaunchKernelGGL(bbsa_combine<float>, g2, b2, 0, stream, p);
    if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
    if (timed && hipEventRecord(g_timing.ev[tslot][3], stream) != hipSuccess) return BBSA_ERR_HIP;
  }
  return status;
}

// Fixed split-K scratch of bbsa_forward_noalloc: one array per device, held
// until the process ends.  Host code never uses the array's name as an
// address (on the host it only stands in for the symbol): the device address
// is looked up once per device with hipGetSymbolAddress and kept here.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;                 // guards g_scratch_ptr
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

// Device address of the current device's scratch array (looked up on the
// first call on that device, with that device current).
int scratch_address(float **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BBSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BBSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return BBSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = (float *)g_scratch_ptr[dev];
  return BBSA_OK;
}

}  // namespace

extern "C" int bbsa_forward(const void *q, const void *k, const void *v, const float *mask,
                            const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                            void *out, hipStream_t stream, bbsa_dtype dtype) {
  Launch ln;
  const int st = setup_forward(q, k, v, mask, rand_attn, B, H, L, d, block, r, out, (int)dtype, &ln);
  if (st < 0) return st;
  if (ln.n_partials > 0) {
    const int rc = ensure_workspace((size_t)ln.n_partials * kPartialFloats * sizeof(float), stream, &ln.p.ws);
    if (rc != BBSA_OK) return rc;
  }
  return launch_forward(ln, stream, dtype, st);
}

extern "C" int bbsa_forward_ex(const void *q, const void *k, const void *v, const float *mask,
                               const int32_t *rand_attn, int B, int H, int L, int d, int block, int r, void *out,
                               float *lse, hipStream_t stream, bbsa_dtype dtype, unsigned flags) {
  Launch ln;
  const int st =
      setup_forward_ex(q, k, v, mask, rand_attn, B, H, L, d, block, r, out, lse, (int)dtype, flags, &ln);
  if (st < 0) return st;
  if (ln.n_partials > 0) {
    const int rc = ensure_workspace((size_t)ln.n_partials * kPartialFloats * sizeof(float), stream, &ln.p.ws);
    if (rc != BBSA_OK) return rc;
  }
  return launch_forward(ln, stream, dtype, st);
}

extern "C" int bbsa_forward_noalloc(const void *q, const void *k, const void *v, const float *mask,
                                    const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                                    void *out, hipStream_t stream, bbsa_dtype dtype) {
  Launch ln;
  const int st = setup_forward(q, k, v, mask, rand_attn, B, H, L, d, block, r, out, (int)dtype, &ln);
  if (st < 0) return st;
  if (ln.n_partials > 0) {
    if ((size_t)ln.n_partials * kPartialFloats * sizeof(float) > kScratchBytes) return BBSA_ERR_SCRATCH;
    const int rc = scratch_address(&ln.p.ws);
    if (rc != BBSA_OK) return rc;
  }
  return launch_forward(ln, stream, dtype, st);
}

extern "C" const char *bbsa_status_string(int status) {
  switch (status) {
    case BBSA_OK: return "ok";
    case BBSA_OK_FULL_FALLBACK: return "ok: sequence too short for the sparse pattern, computed full attention";
    case BBSA_ERR_ARG: return "invalid argument (null or misaligned pointer, non-positive size or r < 1)";
    case BBSA_ERR_SHAPE: return "invalid shape (length not a multiple of the block, or nb < 5 + r)";
    case BBSA_ERR_UNSUPPORTED: return "unsupported configuration (d != 64, block not 64/128, dtype, or size)";
    case BBSA_ERR_HIP: return "HIP runtime error";
    case BBSA_ERR_PLAN: return "rand_attn violates the plan invariants";
    case BBSA_ERR_CAPTURE: return "the workspace must grow while the stream is being captured (run one eager call of this shape first)";
    case BBSA_ERR_SCRATCH: return "the call needs more split-K scratch than bbsa_forward_noalloc's fixed 16 MiB";
    default: return "unknown status";
  }
}

extern "C" void bbsa_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  std::vector<std::pair<int, void *>> all = g_retired;
  for (auto &kv : g_ws)
    if (kv.second.ptr) all.emplace_back(kv.first.first, kv.second.ptr);
  int synced = -1;
  for (auto &dv : all) {
    if (hipSetDevice(dv.first) != hipSuccess) continue;
    if (synced != dv.first) {
      (void)hipDeviceSynchronize();
      synced = dv.first;
    }
    (void)hipFree(dv.second);
  }
  g_ws.clear();
  g_retired.clear();
  (void)hipSetDevice(cur);
}

extern "C" int bbsa_version(void) { return 200; }

extern "C" int bbsa_timing_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
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
  std::lock_guard<std::mutex> lock(g_timing.mu);
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
