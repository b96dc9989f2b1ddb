// Backward pass of the BigBird block-sparse attention (bf16): dQ, dK, dV.
//
// What is computed ("models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的
// 完整实践", section "梯度检查点的实现方式": the operator is trained through
// and the encoder can recompute its forward; "BigBirdPegasus 长序列条件生成模型
// 详解…", section "使用限制与注意事项": the sparse probability matrix carries no
// gradient of its own): with P the masked row softmax of the scores plus
// bias, out = P V and dO the gradient of out,
//   D = rowsum(dO * out),  dV = P^T dO,  dS = P * (dO V^T - D),
//   dQ = dS K,  dK = dS^T Q,
// over the pattern of the forward (the same options: padding mask, query x
// key masking, a length padded to the block).  P is recomputed from the
// forward's row log-sum-exp, so nothing of size L x L is stored.
//
// Kernels:
//   * bbsa_bwd_dq: one wavefront per 32-query tile, walking the tile's key
//     blocks (the forward's blocks; a chunk of every block for a global row)
//     32 keys at a time: S^T = K Q^T and dP^T = V dO^T on MFMA 32x32x16
//     bf16 (Q and dO in registers, K and V rows from LDS), dS^T = P^T (dP^T
//     - D) in registers, then dQ^T += K^T dS^T (K read transposed from
//     LDS).  It also forms D for its rows and stores D and the rows' log2
//     exponent term for the next kernel;
//   * bbsa_bwd_dkdv: one wavefront per 32-key tile, walking the query blocks
//     that attend its key block (global rows, the window, and the rows whose
//     plan picked it, found by scanning the plan; a chunk of every block for
//     a global column) 32 queries at a time: S = Q K^T and dP = dO V^T (K
//     and V in registers, Q and dO rows from LDS), dV^T += dO^T P and
//     dK^T += Q^T dS (Q and dO read transposed);
//   * bbsa_bwd_merge: sums the fp32 partials of the split global rows and
//     columns into their bf16 gradients.
// Every tile goes from memory to LDS with buffer_load ... lds; the row offset
// rides in the range-checked per-lane offset, so rows past L read as zeros.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "bbsa.h"
#include "bbsa_schedule.h"

namespace {

using namespace bbsa_sched;

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lptr_t;

constexpr int kT = 32;                          // rows of a work tile and of a step
constexpr int kTile = kT * kD * 2;              // 4 KB: 32 rows x 64 bf16
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPadBias = -10000.0f;
constexpr int kBufferWord3 = 0x00020000;        // raw buffer: 32-bit format, no swizzle, no stride

// LDS row swizzles (16-byte chunk j of row k sits at chunk j ^ f(k)), with
// 128-byte rows over 64 four-byte banks.  R, for tiles read only by rows
// (MFMA A operands): the 16 rows that one row read serves at a time land on
// 16 distinct chunk positions.  B, for tiles read both by rows and
// transposed (ds_read_b64_tr_b16): the same property for row reads, and the
// four rows that each 32-lane half of a transposed read covers sit on eight
// distinct chunk positions.  B(k + 8) = B(k) ^ 2 and B(k + 16) = B(k).
__device__ inline int swz_r(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ inline int swz_b(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

__device__ inline int lane_id() { return (int)__builtin_amdgcn_workitem_id_x() & 63; }

// A global row or column is walked in chunks of about kChunkBlocks blocks,
// and in at least two: fewer, longer chunks leave fewer partials to merge,
// and two halves keep the global items from forming the tail (at nb = 64 two
// chunks beat one, four and eight; at nb = 256 four beat eight and 32).
constexpr int kChunkBlocks = 64;
constexpr int kMaskBytes = 256;                 // per-step array of 64 floats (lanes 32..63 repeat 0..31)

struct BwdParams {
  const bf16_t *q, *k, *v, *o, *dout;
  const float *lse;          // [B, H, L]
  const float *mask;         // [B, L] or null
  const int32_t *rand_attn;  // [H, nb-2, r] or null (fallback)
  float *delta;              // [B, H, L]: D = rowsum(dO * out), written by the dq kernel
  float *rterm;              // [B, H, L]: -(log2e lse - (1 - mq) log2e kPadBias), written by the dq kernel
  int *live;                 // [B, H, nb * tiles]: 1 if some row of the query tile may weigh a padded key (dq kernel)
  bf16_t *dq, *dk, *dv;
  float *ws;                 // split partials of the global rows (dq) and columns (dk, dv)
  int B, H, L, nb, block, r;
  int full;                  // every block attends every block
  int qk;                    // query x key masking
  int tiles;                 // 32-row tiles per block
  int chunks;                // chunks of a global row or column (1: no partials)
  int n_grows;               // global rows (and columns) per pair: 2, or nb on the fallback
  int lanes;                 // XCD lanes: 8 when there are at least 8 pairs, else 1
  int glob_items;            // per pair: n_grows * tiles * chunks
  int mid_items;             // per pair: (nb - 2) * tiles (0 on the fallback)
  int n_glob_lane;           // global items before the first middle item, per XCD lane
  int64_t n_part;            // partials per gradient
  int skip;                  // 1: steps whose keys are all padded are skipped for rows that attend a real key
};

// A query row whose log-sum-exp exceeds -5000 (natural units) attends keys
// far above the padding bias: a key of mask 0 then has a probability
// exp(s - 10000 - lse) below exp(s - 5000), exactly zero in fp32 for any
// score s below about 4900, so a step whose keys all have mask 0 adds
// exactly nothing to such rows' dQ, or to its keys' dK and dV (the forward
// leaves the same blocks out).  In log2 units: lse2 > -kLiveLog2.
constexpr float kLiveLog2 = 5000.0f * 1.4426950408889634f;

// Work item: a 32-row tile of block blk (a query block for dq, a key block
// for dk/dv) of pair bh; a global row or column is split into `chunks`
// ranges of blocks.  Workgroup w runs on XCD w % 8 and, with the XCD lanes,
// serves only the pairs x, x + 8, ... (x = w % 8), so the tiles a pair
// re-reads stay in one L2; the global items of a lane come first.
struct BwdItem {
  int bh, blk, tile, chunk, g;
  bool glob;
};
__device__ inline BwdItem decode(const BwdParams &p, int wg) {
  const int x = wg % p.lanes, slot = wg / p.lanes;
  BwdItem it;
  it.chunk = 0;
  it.g = 0;
  if (slot < p.n_glob_lane) {
    const int j = slot / p.glob_items, loc = slot % p.glob_items;
    it.bh = x + j * p.lanes;
    it.glob = true;
    it.g = loc / (p.tiles * p.chunks);
    const int rem = loc % (p.tiles * p.chunks);
    it.tile = rem / p.chunks;
    it.chunk = rem % p.chunks;
    it.blk = p.full ? it.g : (it.g == 0 ? 0 : p.nb - 1);
  } else if (p.mid_items > 0) {
    const int s2 = slot - p.n_glob_lane;
    const int j = s2 / p.mid_items, loc = s2 % p.mid_items;
    it.bh = x + j * p.lanes;
    it.glob = false;
    it.blk = 1 + loc / p.tiles;
    it.tile = loc % p.tiles;
  } else {
    it.bh = 0x7fffffff;   // idle
    it.glob = false;
    it.blk = it.tile = 0;
  }
  // Uniform by construction; stated so that addresses built from them stay
  // in scalar registers.
  it.bh = __builtin_amdgcn_readfirstlane(it.bh);
  it.blk = __builtin_amdgcn_readfirstlane(it.blk);
  it.tile = __builtin_amdgcn_readfirstlane(it.tile);
  it.chunk = __builtin_amdgcn_readfirstlane(it.chunk);
  it.g = __builtin_amdgcn_readfirstlane(it.g);
  it.glob = __builtin_amdgcn_readfirstlane((int)it.glob) != 0;
  return it;
}

// Per-lane DMA state of one 32 x 64 tile: lane l of instruction u loads row
// 8u + l/8 of the tile into LDS position tile + 1024u + 16l.
struct TileDma {
  int off_r[4];              // source byte offsets within the tile, R swizzle
  int off_b;                 // B swizzle, instructions 0 and 2 (1 and 3: off_b ^ 32)
  __device__ void init(int lane) {
    const int drow = lane >> 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) off_r[u] = 2 * ((8 * u + drow) * kD + 8 * ((lane & 7) ^ swz_r(8 * u + drow))) - 1024 * u;
    off_b = 2 * (drow * kD + 8 * ((lane & 7) ^ swz_b(drow)));
  }
};

// A row index past every supported length (L <= 2^24): its transfers are
// out of the buffer's range, so they write zeros and read no memory.
constexpr int kNoRow = 1 << 24;

// Rows row0 .. row0+31 of a [L, 64] bf16 matrix (buffer resource rs) into
// LDS; rows at or past L read as zeros (the offset is range-checked).  The
// offsets are 32-bit unsigned: row0 * 128 reaches 2^31 for kNoRow.
__device__ inline void dma_rows(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, const TileDma &t, int row0, bool bsw) {
  const int base = (int)((unsigned)row0 * (kD * 2));
  if (bsw) {
    const int b0 = t.off_b + base, b1 = (t.off_b ^ 32) + base;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, b0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, b1, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, b0, 0, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, b1, 0, 3072, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[0] + base, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[1] + base, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[2] + base, 0, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[3] + base, 0, 3072, 0);
  }
}
// Floats pos0 + (lane % 32) of a float buffer resource into LDS (64 floats,
// the upper 32 repeating the lower); positions past the range read as 0.
__device__ inline void dma_floats(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, int pos0, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 4, (int)(4u * (unsigned)(pos0 + (lane & 31))), 0, 0, 0);
}

// A operands of the rows of a tile: row c, d = 16kk + 8h .. +7.
template <bool BSW>
__device__ inline void read_rows(const unsigned char *src, int c, int h, bf16x8 (&a)[4]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    a[kk] = *(const bf16x8 *)(src + c * 128 + 16 * ((2 * kk + h) ^ (BSW ? swz_b(c) : swz_r(c))));
}

// A operands of the transposed B-swizzled tile X (rows r, columns d): for
// d-tile dt and row step s, lane (c, h) gets X^T[32dt + c][the row slots
// 8h .. 8h+7 of step s], in the slot order that the B operands packed by
// pack_b use (slot 8h + e is row 16s + 4h + (e & 3) + 8 (e >> 2)).
// toff[dt] addresses rows 0-7 (and 16-23 at +2048); rows 8-15 and 24-31
// sit at (toff[dt] ^ 32) + 1024 and + 3072, as B(k + 8) = B(k) ^ 2.
__device__ inline void read_tr(const unsigned char *src, const int (&toff)[2], bf16x8 (&a)[2][2]) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + toff[dt] + 2048 * s));
      const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + (toff[dt] ^ 32) + 2048 * s + 1024));
      a[dt][s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}
__device__ inline void tr_offsets(int lane, int (&toff)[2]) {
  const int G = lane >> 4, cc = lane & 15;
  const int row = 4 * (G >> 1) + (cc >> 2);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int chunk = 4 * dt + 2 * (G & 1) + ((cc & 3) >> 1);
    toff[dt] = row * 128 + 16 * (chunk ^ swz_b(row)) + 8 * (cc & 1);
  }
}

// B operands from a 32x32 MFMA result x (lane (c, h), register 4j + i =
// row 8j + 4h + i of column c): for row step s, the lane's rows of that step
// as bf16, in the slot order read_tr matches.
__device__ inline void pack_b(const f32x16 &x, bf16x8 (&b)[2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const f32x4 lo = {x[8 * s + 0], x[8 * s + 1], x[8 * s + 2], x[8 * s + 3]};
    const f32x4 hi = {x[8 * s + 4], x[8 * s + 5], x[8 * s + 6], x[8 * s + 7]};
    b[s] = __builtin_shufflevector(__builtin_convertvector(lo, bf16x4), __builtin_convertvector(hi, bf16x4), 0, 1, 2,
                                   3, 4, 5, 6, 7);
  }
}

__device__ inline f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Flip the sign of every bf16 element (the sign bit of each half).
__device__ inline void negate(bf16x8 (&x)[4]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    x[kk] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x[kk]) ^ 0x80008000u);
  }
}
__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.0f;
  return z;
}

// Register operands of 32 rows of a [L, 64] bf16 matrix in the B layout:
// lane (c, h) holds row row0 + c, d = 16kk + 8h .. +7 (zeros at or past L).
__device__ inline void load_b_rows(const bf16_t *base, int L, int row0, int c, int h, bf16x8 (&b)[4]) {
  const int row = row0 + c;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8 x = *(const bf16x8 *)(base + (int64_t)min(row, L - 1) * kD + 16 * kk + 8 * h);
    if (row >= L) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (__bf16)0.0f;
    }
    b[kk] = x;
  }
}

// Store a 32x32 MFMA result holding X^T (rows d = 32dt + 8j + 4h + i, column
// = row c of X): as bf16 rows row0 + c of a [L, 64] matrix, or as the fp32
// [32][64] partial `part`.
__device__ inline void store_t(bf16_t *base, int L, int row0, int c, int h, const f32x16 (&x)[2]) {
  const int row = row0 + c;
  if (row >= L) return;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 y = {x[dt][4 * j], x[dt][4 * j + 1], x[dt][4 * j + 2], x[dt][4 * j + 3]};
      *(bf16x4 *)(base + (int64_t)row * kD + 32 * dt + 8 * j + 4 * h) = __builtin_convertvector(y, bf16x4);
    }
}
__device__ inline void store_partial(float *part, int c, int h, const f32x16 (&x)[2]) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 y = {x[dt][4 * j], x[dt][4 * j + 1], x[dt][4 * j + 2], x[dt][4 * j + 3]};
      *(f32x4 *)(part + c * kD + 32 * dt + 8 * j + 4 * h) = y;
    }
}

__device__ inline float mask_at(const BwdParams &p, const float *mrow, int pos) {
  return pos < p.L ? (mrow ? mrow[pos] : 1.0f) : 0.0f;
}

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, kBufferWord3);
}

// LDS slots of the step pipelines: the transfers of step st + kSlots - 1
// go out while step st computes.
constexpr int kSlots = 2;

// Wait until at most KEEP vector-memory operations are outstanding: the
// transfers of the steps after this one already issued (issued for every
// step, past the end too, as out-of-range transfers of kNoRow), so that
// this step's have landed.  Memory loads complete in issue order.
template <int KEEP>
__device__ inline void wait_step() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KEEP) : "memory");
}
__device__ inline void wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Key block of list position t of middle query block i (the forward's blocks:
// the two global blocks, the window without them in ascending order, the
// plan's blocks).
__device__ inline int list_block(const BwdParams &p, const int32_t *plan_row, int i, int t) {
  if (t == 0) return 0;
  if (t == 1) return p.nb - 1;
  const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
  const int w0 = (i == 1) ? 1 : i - 1;
  if (t < 2 + nw) return w0 + (t - 2);
  return min(max(plan_row[t - 2 - nw], 0), p.nb - 1);
}

template <int S>
using SlotId = std::integral_constant<int, S>;

// Runs step(SlotId<st % kSlots>, st) for st = 0 .. n-1 with the slot as a
// compile-time constant, so that every LDS access names one of the slots'
// separate arrays and the compiler's own waits for the transfers into LDS
// wait for the right slot only.
template <class Step>
__device__ inline void run_steps(int n, Step &&step) {
  int st = 0;
  if constexpr (kSlots == 3) {
    for (; st + 3 <= n; st += 3) {
      step(SlotId<0>{}, st);
      step(SlotId<1>{}, st + 1);
      step(SlotId<2>{}, st + 2);
    }
    if (st < n) step(SlotId<0>{}, st);
    if (st + 1 < n) step(SlotId<1>{}, st + 1);
  } else {
    static_assert(kSlots == 2, "two or three slots");
    for (; st + 2 <= n; st += 2) {
      step(SlotId<0>{}, st);
      step(SlotId<1>{}, st + 1);
    }
    if (st < n) step(SlotId<0>{}, st);
  }
}
// Slot of the transfers issued during a step in slot S.
template <int S>
using IssueSlot = SlotId<(S + kSlots - 1) % kSlots>;

// dQ: one wavefront per 32-query tile; workgroups of one wavefront.  LDS
// slots, each K (B swizzle) and V (R swizzle) of one step and the key mask.
template <bool MASKED>
__global__ __launch_bounds__(64) void bbsa_bwd_dq(BwdParams p) {
  const BwdItem it = decode(p, (int)blockIdx.x);
  if (it.bh >= p.B * p.H) return;
  __shared__ __attribute__((aligned(1024))) unsigned char kv0[2 * kTile], kv1[2 * kTile], kv2[2 * kTile];
  __shared__ __attribute__((aligned(256))) unsigned char mk0[kMaskBytes], mk1[kMaskBytes], mk2[kMaskBytes];
  auto kv = [&](auto S) -> unsigned char * {
    if constexpr (decltype(S)::value == 0) return kv0;
    else if constexpr (decltype(S)::value == 1) return kv1;
    else return kv2;
  };
  auto mk = [&](auto S) -> unsigned char * {
    if constexpr (decltype(S)::value == 0) return mk0;
    else if constexpr (decltype(S)::value == 1) return mk1;
    else return mk2;
  };
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int bh = it.bh, i = it.blk;
  const int b = bh / p.H, hh = bh % p.H;
  const int q0 = i * p.block + it.tile * kT;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = MASKED ? p.mask + (int64_t)b * p.L : nullptr;
  const int32_t *plan_row = it.glob ? nullptr : p.rand_attn + ((int64_t)hh * (p.nb - 2) + (i - 1)) * p.r;
  const int spb = p.block / kT, lg_spb = spb >> 1;   // 2 or 4 steps per block
  // List positions walked: a chunk of the blocks for a global row, the
  // forward's list for a middle row.
  int pos0 = 0, pos1;
  if (it.glob) {
    pos0 = it.chunk * p.nb / p.chunks;
    pos1 = (it.chunk + 1) * p.nb / p.chunks;
  } else {
    pos1 = 2 + ((i == 1 || i == p.nb - 2) ? 2 : 3) + p.r;
  }
  int n_steps = __builtin_amdgcn_readfirstlane((pos1 - pos0) * spb);
  // The middle row's key blocks, lane t holding list position t (at most 64).
  int blocks = it.glob ? 0 : list_block(p, plan_row, i, min(lane, pos1 - 1));
  auto key_of = [&](int st) {
    const int pos = pos0 + (st >> lg_spb);
    const int row =
        (it.glob ? pos : __builtin_amdgcn_readlane(blocks, min(pos, 63))) * p.block + (st & (spb - 1)) * kT;
    return __builtin_amdgcn_readfirstlane(st < n_steps ? row : kNoRow);
  };

  TileDma dma;
  dma.init(lane);
  int toff[2];
  tr_offsets(lane, toff);
  const auto krs = rsrc(p.k + bh * seq, seq * 2);
  const auto vrs = rsrc(p.v + bh * seq, seq * 2);
  const auto mrs = rsrc(mrow, (int64_t)p.L * 4);

  // Q and dO of the tile (B operands), and the query column's lse (log2
  // units, the query x key constant taken out), D and mask factor.
  bf16x8 qf[4], df[4];
  load_b_rows(p.q + bh * seq, p.L, q0, c, h, qf);
  load_b_rows(p.dout + bh * seq, p.L, q0, c, h, df);
  const int qrow = q0 + c;
  const bool qlive = qrow < p.L;
  const float mq = p.qk ? (qlive ? mask_at(p, mrow, qrow) : 0.0f) : 1.0f;
  const float lse2 =
      qlive ? (p.lse[(int64_t)bh * p.L + qrow] - (p.qk ? kPadBias * (1.0f - mq) : 0.0f)) * kLog2e : 0.0f;
  // D of the query row: dO (in registers) against the row of out, lane
  // (c, h) taking half of row c's columns.  The tile's item (the first
  // chunk's, for a global row) stores D and -lse2 for the dk/dv kernel.
  float dlt;
  {
    bf16x8 of[4];
    load_b_rows(p.o + bh * seq, p.L, q0, c, h, of);
    float acc = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)df[kk][e], (float)of[kk][e], acc);
    dlt = acc + __shfl_xor(acc, 32);
    if (qlive && h == 0 && (!it.glob || it.chunk == 0)) {
      p.delta[(int64_t)bh * p.L + qrow] = dlt;
      p.rterm[(int64_t)bh * p.L + qrow] = -lse2;
    }
  }
  // The dP^T product runs on -dO from an accumulator holding D, so that it
  // yields D - dP^T and dS^T = -P^T (D - dP^T) needs no subtraction.
  negate(df);
  f32x16 dinit;
#pragma unroll
  for (int e = 0; e < 16; ++e) dinit[e] = dlt;
  // The exponent of P in log2 units is s log2e + (1 - m) cpad - lse2 for a
  // key of mask value m: the bias term is exactly 0 for m = 1.
  const float cpad = mq * kPadBias * kLog2e;
  // Steps whose 32 keys all have mask 0 add nothing when every row of the
  // tile attends a real key (and, under query x key masking, has mask 1;
  // rows past L have zero Q and dO).
  const bool tile_live = __builtin_amdgcn_ballot_w64(qlive && ((p.qk && mq != 1.0f) || lse2 <= -kLiveLog2)) != 0;
  const bool drop_dead = MASKED && p.skip && !tile_live;
  if (MASKED && p.skip && lane == 0 && (!it.glob || it.chunk == 0))
    p.live[((int64_t)bh * p.nb + i) * p.tiles + it.tile] = tile_live ? 1 : 0;

  auto issue = [&](auto S, int st) {
    const int key0 = key_of(st);
    dma_rows(krs, kv(S), dma, key0, true);
    dma_rows(vrs, kv(S) + kTile, dma, key0, false);
    if (MASKED) dma_floats(mrs, mk(S), key0, lane);
  };
  constexpr int kPerStep = MASKED ? 9 : 8;

  // A middle row whose rows all attend a real key leaves out the listed
  // blocks whose keys all have mask 0 (list position 0, in flight first,
  // stays): one 8-byte mask probe per lane and listed block, issued before
  // the first step's transfers, then a stable compaction of the list.
  const bool compact = MASKED && drop_dead && !it.glob && p.L % p.block == 0;
  const int npos = pos1 - pos0;
  float pm[8][2];
  auto probe_load = [&](int t0) {
    const int off = (p.block > 64 ? 2 * lane : 2 * (lane & 31)) * 4;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int blk = __builtin_amdgcn_readlane(blocks, min(t0 + u, npos - 1));
      const auto mv = __builtin_amdgcn_raw_buffer_load_b64(mrs, off, blk * p.block * 4, 0);
      pm[u][0] = __uint_as_float(mv[0]);
      pm[u][1] = __uint_as_float(mv[1]);
    }
  };
  uint64_t padded = 0;
  auto probe_bits = [&](int t0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t nz = (__float_as_uint(pm[u][0]) | __float_as_uint(pm[u][1])) << 1;   // 0: both are +-0
      if (t0 + u < npos && !__builtin_amdgcn_ballot_w64(nz != 0u)) padded |= 1ull << (t0 + u);
    }
  };
  if (compact) probe_load(0);

  // Transfers go out for every step below n_steps + 2, so the compiler's
  // own wait before each slot's reads also counts only that slot's.
  f32x16 dq[2] = {zero16(), zero16()};
  issue(SlotId<0>{}, 0);
  if (compact) {
    probe_bits(0);
    for (int t0 = 8; t0 < npos; t0 += 8) {
      probe_load(t0);
      probe_bits(t0);
    }
    const uint64_t all = npos >= 64 ? ~0ull : (1ull << npos) - 1;
    const uint64_t keep = (all & ~padded) | 1ull;
    if (keep != all) {
      const int nkeep = __builtin_popcountll(keep);
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0u));
      const int dst = ((keep >> lane) & 1) ? rank : nkeep + (lane - rank);
      blocks = __builtin_amdgcn_ds_permute(dst * 4, blocks);
      n_steps = __builtin_amdgcn_readfirstlane(nkeep * spb);
    }
  }
  if constexpr (kSlots == 3) issue(SlotId<1>{}, 1);
  run_steps(n_steps, [&](auto S, int st) {
    wait_step<(kSlots - 2) * kPerStep>();
    const unsigned char *s = kv(S);
    const int key0 = key_of(st);
    bf16x8 kr[4], vr[4], kt[2][2];
    read_rows<true>(s, c, h, kr);
    read_rows<false>(s + kTile, c, h, vr);
    read_tr(s, toff, kt);
    // x = (1 - m) cpad - lse2 per key; without a mask only keys past L
    // (the last block of a ragged length) carry the bias.
    // A step whose 32 keys are all real and unmasked (the common case)
    // takes x = -lse2 throughout.
    bool plain, dead = false;
    if (MASKED) {
      const float mkey = *(const float *)(mk(S) + 4 * c);
      plain = __builtin_amdgcn_ballot_w64(mkey != 1.0f) == 0;
      if (drop_dead) dead = __builtin_amdgcn_ballot_w64(mkey != 0.0f) == 0;
    } else {
      plain = key0 + kT <= p.L;
    }
    // The transfers of step st + kSlots - 1 go into the slot step st - 1 read.
    issue(IssueSlot<decltype(S)::value>{}, st + kSlots - 1);
    if (dead) return;
    f32x16 sc = mfma(kr[0], qf[0], zero16());   // S^T[key][query c]
    f32x16 dp = mfma(vr[0], df[0], dinit);      // D - dP^T[key][query c]
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) {
      sc = mfma(kr[kk], qf[kk], sc);
      dp = mfma(vr[kk], df[kk], dp);
    }
    // P^T and dS^T; register 4jj + ii is key key0 + 8jj + 4h + ii.
    if (plain) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = -__builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], kLog2e, -lse2)) * dp[e];
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 xb;
        if (MASKED) {
          const f32x4 m = *(const f32x4 *)(mk(S) + 4 * (8 * jj + 4 * h));
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) xb[ii] = __builtin_fmaf(1.0f - m[ii], cpad, -lse2);
        } else {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) xb[ii] = key0 + 8 * jj + 4 * h + ii < p.L ? -lse2 : cpad - lse2;
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int e = 4 * jj + ii;
          sc[e] = -__builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], kLog2e, xb[ii])) * dp[e];
        }
      }
    }
    bf16x8 dsb[2];
    pack_b(sc, dsb);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) dq[dt] = mfma(kt[dt][ss], dsb[ss], dq[dt]);   // dQ^T[d][query c]
  });
  wait_all();   // the transfers past the end
  if (it.glob && p.chunks > 1) {
    const int64_t idx = (((int64_t)bh * p.n_grows + it.g) * p.tiles + it.tile) * p.chunks + it.chunk;
    store_partial(p.ws + idx * (kT * kD), c, h, dq);
  } else {
    store_t(p.dq + bh * seq, p.L, q0, c, h, dq);
  }
}

// dK, dV: one wavefront per 32-key tile.  The query blocks that attend key
// block j: a chunk of every block for a global key block (or on the
// fallback); else the two global blocks, the window {j-1, j, j+1} (without
// repeating a global one) and the middle blocks whose plan row picked j,
// gathered in an LDS list and walked at least 64 blocks at a time.  LDS
// slots, each Q and dO (B swizzle) of one step with the step's lse, D and
// query mask values.
template <bool QK>
__global__ __launch_bounds__(64) void bbsa_bwd_dkdv(BwdParams p) {
  const BwdItem it = decode(p, (int)blockIdx.x);
  if (it.bh >= p.B * p.H) return;
  constexpr int kVec = 3 * kMaskBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char qd0[2 * kTile], qd1[2 * kTile], qd2[2 * kTile];
  __shared__ __attribute__((aligned(256))) unsigned char vc0[kVec], vc1[kVec], vc2[kVec];
  __shared__ int blist[128];
  auto qd = [&](auto S) -> unsigned char * {
    if constexpr (decltype(S)::value == 0) return qd0;
    else if constexpr (decltype(S)::value == 1) return qd1;
    else return qd2;
  };
  auto vc = [&](auto S) -> unsigned char * {
    if constexpr (decltype(S)::value == 0) return vc0;
    else if constexpr (decltype(S)::value == 1) return vc1;
    else return vc2;
  };
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int bh = it.bh, j = it.blk;
  const int b = bh / p.H, hh = bh % p.H;
  const int k0 = j * p.block + it.tile * kT;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = p.mask ? p.mask + (int64_t)b * p.L : nullptr;
  const int spb = p.block / kT, lg_spb = spb >> 1;   // 2 or 4 steps per block

  TileDma dma;
  dma.init(lane);
  int toff[2];
  tr_offsets(lane, toff);
  const auto qrs = rsrc(p.q + bh * seq, seq * 2);
  const auto drs = rsrc(p.dout + bh * seq, seq * 2);
  const auto lrs = rsrc(p.rterm + (int64_t)bh * p.L, (int64_t)p.L * 4);
  const auto ers = rsrc(p.delta + (int64_t)bh * p.L, (int64_t)p.L * 4);
  const auto mrs = rsrc(mrow, (int64_t)p.L * 4);

  // K and V of the tile (B operands: lane (c, h) = key k0 + c); the key
  // column's padding bias.
  bf16x8 kf[4], vf[4];
  load_b_rows(p.k + bh * seq, p.L, k0, c, h, kf);
  load_b_rows(p.v + bh * seq, p.L, k0, c, h, vf);
  // The key column's padding bias in log2 units (exactly 0 for a real,
  // unmasked key).  The exponent of P is s log2e + rt + x, with rt the
  // query row's term -(log2e lse - (1 - mq) log2e kPadBias) from the dq
  // kernel (the lse of a query of mask value mq holds the constant
  // (1 - mq) kPadBias under query x key masking; mq = 1 otherwise) and
  // x = kb2 (key-side masking) or mq kb2 (query x key).  A tile whose 32
  // keys all have kb2 = 0 takes x = 0.
  const float kb2 = kPadBias * (1.0f - mask_at(p, mrow, k0 + c)) * kLog2e;
  const bool plain = __builtin_amdgcn_ballot_w64(kb2 != 0.0f) == 0;
  // A tile whose keys all have mask 0 (or lie past L) gets nothing from the
  // query rows that attend a real key (and have mask 1 under query x key
  // masking): such steps are skipped.
  const bool dead_keys = p.skip && __builtin_amdgcn_ballot_w64(mask_at(p, mrow, k0 + c) != 0.0f) == 0;
  // The dP product runs on -V from an accumulator holding D (the step's D
  // values, read from LDS): it yields D - dP, and dS = -P (D - dP).
  negate(vf);

  f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};
  constexpr int kPerStep = QK ? 11 : 10;
  // Walk the query blocks of list positions [0, n) (block of position t:
  // from the LDS list, or first + t for a range), 32 queries a step.
  auto walk = [&](int n, bool from_list, int first) {
    // A tile whose keys all have mask 0 walks only the query blocks with a
    // tile whose rows may weigh a padded key (the dq kernel's flags): the
    // others add exactly nothing.  Lane t holds list position t (lists of
    // up to 64 blocks; longer ones are walked whole).
    bool compacted = false;
    int plist = 0;
    if (dead_keys && n <= 64) {
      const int blk = from_list ? blist[min(lane, 127)] : first + lane;
      const int blk_c = min(max(blk, 0), p.nb - 1);   // lanes past the list read a valid flag, unused
      bool live = false;
      for (int s2 = 0; s2 < p.tiles; ++s2) live |= p.live[((int64_t)bh * p.nb + blk_c) * p.tiles + s2] != 0;
      live = live && lane < n;
      const uint64_t keep = __builtin_amdgcn_ballot_w64(live);
      const int nkeep = __builtin_popcountll(keep);
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0u));
      const int dst = ((keep >> lane) & 1) ? rank : nkeep + (lane - rank);
      plist = __builtin_amdgcn_ds_permute(dst * 4, blk);
      n = nkeep;
      compacted = true;
    }
    const int n_steps = __builtin_amdgcn_readfirstlane(n * spb);
    auto row_of = [&](int st) {
      const int t = min(st >> lg_spb, 127);
      const int blk = compacted ? __builtin_amdgcn_readlane(plist, min(t, 63)) : (from_list ? blist[t] : first + t);
      const int row = blk * p.block + (st & (spb - 1)) * kT;
      return __builtin_amdgcn_readfirstlane(st < n_steps ? row : kNoRow);
    };
    auto issue = [&](auto S, int st) {
      const int row0 = row_of(st);
      dma_rows(qrs, qd(S), dma, row0, true);
      dma_rows(drs, qd(S) + kTile, dma, row0, true);
      dma_floats(lrs, vc(S), row0, lane);
      dma_floats(ers, vc(S) + kMaskBytes, row0, lane);
      if (QK) dma_floats(mrs, vc(S) + 2 * kMaskBytes, row0, lane);
    };
    issue(SlotId<0>{}, 0);
    if constexpr (kSlots == 3) issue(SlotId<1>{}, 1);
    run_steps(n_steps, [&](auto S, int st) {
      wait_step<(kSlots - 2) * kPerStep>();
      const unsigned char *s = qd(S);
      const unsigned char *v = vc(S);
      bf16x8 qr[4], dr[4], qt[2][2], dt2[2][2];
      read_rows<true>(s, c, h, qr);
      read_rows<true>(s + kTile, c, h, dr);
      read_tr(s, toff, qt);
      read_tr(s + kTile, toff, dt2);
      // Register 4jj + ii is query row0 + 8jj + 4h + ii; its row term, D and
      // mask value (rows past L read as 0: their Q and dO are zeros, so they
      // add nothing).
      f32x4 rt[4], dl[4], mqv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        rt[jj] = *(const f32x4 *)(v + 4 * (8 * jj + 4 * h));
        dl[jj] = *(const f32x4 *)(v + kMaskBytes + 4 * (8 * jj + 4 * h));
        if (QK) mqv[jj] = *(const f32x4 *)(v + 2 * kMaskBytes + 4 * (8 * jj + 4 * h));
        else mqv[jj] = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
      }
      issue(IssueSlot<decltype(S)::value>{}, st + kSlots - 1);
      if (dead_keys) {
        bool live = false;   // some row whose padded keys may carry weight
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) live |= rt[jj][ii] >= kLiveLog2 || (QK && mqv[jj][ii] != 1.0f);
        if (!__builtin_amdgcn_ballot_w64(live)) return;
      }
      f32x16 dinit;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) dinit[4 * jj + ii] = dl[jj][ii];
      f32x16 sc = mfma(qr[0], kf[0], zero16());   // S[query][key c]
      f32x16 dp = mfma(dr[0], vf[0], dinit);      // D - dP[query][key c]
#pragma unroll
      for (int kk = 1; kk < 4; ++kk) {
        sc = mfma(qr[kk], kf[kk], sc);
        dp = mfma(dr[kk], vf[kk], dp);
      }
      if (plain) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int e = 4 * jj + ii;
            sc[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], kLog2e, rt[jj][ii]));
            dp[e] = -sc[e] * dp[e];
          }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int e = 4 * jj + ii;
            const float y = QK ? __builtin_fmaf(mqv[jj][ii], kb2, rt[jj][ii]) : rt[jj][ii] + kb2;
            sc[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], kLog2e, y));
            dp[e] = -sc[e] * dp[e];
          }
      }
      bf16x8 pb[2], db[2];
      pack_b(sc, pb);
      pack_b(dp, db);
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          dv[d2] = mfma(dt2[d2][ss], pb[ss], dv[d2]);   // dV^T[d][key c]
          dk[d2] = mfma(qt[d2][ss], db[ss], dk[d2]);    // dK^T[d][key c]
        }
    });
    wait_all();   // the transfers past the end
  };

  if (it.glob) {
    const int first = it.chunk * p.nb / p.chunks;
    walk((it.chunk + 1) * p.nb / p.chunks - first, false, first);
  } else {
    // The fixed blocks, then the plan rows that picked j, 64 entries of the
    // plan per pass; the list is walked once it holds 64 blocks or the plan
    // is done.  Rows of the plan are middle blocks outside j's window, so
    // none repeats a fixed block (a clamped bad plan's repeats are skipped).
    int n_fixed = 0;
    int fixed[5];
    fixed[n_fixed++] = 0;
    fixed[n_fixed++] = p.nb - 1;
    for (int x = j - 1; x <= j + 1; ++x)
      if (x > 0 && x < p.nb - 1) fixed[n_fixed++] = x;
    if (lane == 0)
      for (int x = 0; x < n_fixed; ++x) blist[x] = fixed[x];
    int n = n_fixed;
    const int32_t *plan_h = p.rand_attn + (int64_t)hh * (p.nb - 2) * p.r;
    const int n_entries = (p.nb - 2) * p.r;
    // The plan is read kScan passes of 64 entries at a time: the loads of
    // a batch are issued together, then its passes run one after another.
    constexpr int kScan = 4;
    int pv[kScan];
    for (int e0 = 0;; e0 += 64) {
      const int pass = (e0 >> 6) & (kScan - 1);
      if (pass == 0) {
#pragma unroll
        for (int u = 0; u < kScan; ++u) pv[u] = plan_h[min(e0 + 64 * u + lane, n_entries - 1)];
      }
      const int pe = pass == 0 ? pv[0] : pass == 1 ? pv[1] : pass == 2 ? pv[2] : pv[3];
      if (e0 < n_entries) {
        const int e = e0 + lane;
        const bool hit = e < n_entries && min(max(pe, 0), p.nb - 1) == j;
        unsigned long long bits = __builtin_amdgcn_ballot_w64(hit);
        while (bits) {
          const int l = __builtin_ctzll(bits);
          bits &= bits - 1;
          const int row = 1 + (e0 + l) / p.r;
          bool dup = false;
          for (int x = 0; x < n_fixed; ++x) dup |= fixed[x] == row;
          if (dup) continue;
          if (lane == 0) blist[n] = row;
          ++n;
        }
      }
      const bool last = e0 + 64 >= n_entries;
      if (n >= 64 || last) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        walk(n, true, 0);
        n = 0;
      }
      if (last) break;
    }
  }
  if (it.glob && p.chunks > 1) {
    const int64_t idx = (((int64_t)bh * p.n_grows + it.g) * p.tiles + it.tile) * p.chunks + it.chunk;
    store_partial(p.ws + (p.n_part + idx) * (kT * kD), c, h, dk);
    store_partial(p.ws + (2 * p.n_part + idx) * (kT * kD), c, h, dv);
  } else {
    store_t(p.dk + bh * seq, p.L, k0, c, h, dk);
    store_t(p.dv + bh * seq, p.L, k0, c, h, dv);
  }
}

// Sum the chunk partials of each global tile (dq, dk, dv) into its bf16
// rows: one 256-thread workgroup per tile, eight floats per thread.
__global__ __launch_bounds__(256) void bbsa_bwd_merge(BwdParams p) {
  const int64_t tiles_per = p.n_part / p.chunks;   // global tiles per gradient
  const int64_t w = blockIdx.x;
  const int which = (int)(w / tiles_per);
  const int64_t t = w % tiles_per;
  const int tile = (int)(t % p.tiles);
  const int g = (int)((t / p.tiles) % p.n_grows);
  const int bh = (int)(t / ((int64_t)p.tiles * p.n_grows));
  const int blk = p.full ? g : (g == 0 ? 0 : p.nb - 1);
  const int r = threadIdx.x >> 3, d0 = 8 * (threadIdx.x & 7);
  const int row = blk * p.block + tile * kT + r;
  if (row >= p.L) return;
  const float *base = p.ws + ((int64_t)which * p.n_part + t * p.chunks) * (kT * kD) + r * kD + d0;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int ch = 0; ch < p.chunks; ++ch) {
    a0 += *(const f32x4 *)(base + (int64_t)ch * (kT * kD));
    a1 += *(const f32x4 *)(base + (int64_t)ch * (kT * kD) + 4);
  }
  bf16_t *out = (which == 0 ? p.dq : which == 1 ? p.dk : p.dv) + (int64_t)bh * p.L * kD + (int64_t)row * kD + d0;
  *(bf16x4 *)out = __builtin_convertvector(a0, bf16x4);
  *(bf16x4 *)(out + 4) = __builtin_convertvector(a1, bf16x4);
}

}  // namespace

extern "C" int bbsa_backward(const void *q, const void *k, const void *v, const void *out, const void *dout,
                             const float *lse, const float *mask, const int32_t *rand_attn, int B, int H, int L,
                             int d, int block, int r, void *dq, void *dk, void *dv, float *delta,
                             hipStream_t stream, bbsa_dtype dtype, unsigned flags) {
  Launch ln;
  const int st = setup_forward_ex(q, k, v, mask, rand_attn, B, H, L, d, block, r, (void *)out, (float *)lse,
                                  (int)dtype, flags, &ln);
  if (st < 0) return st;
  if (!dout || !lse || !dq || !dk || !dv || !delta) return BBSA_ERR_ARG;
  auto misaligned = [](const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) != 0; };
  if (misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) || misaligned(delta, 4))
    return BBSA_ERR_ARG;
  if (dtype == BBSA_F32) {
    const int rc = launch_backward_f32(q, k, v, out, dout, mask, ln.full ? nullptr : rand_attn, B, H, L, ln.p.nb,
                                       block, r, ln.full, (ln.p.mode & kModeQK) != 0, dq, dk, dv, delta, stream);
    return rc < 0 ? rc : st;
  }
  BwdParams p;
  p.q = (const bf16_t *)q; p.k = (const bf16_t *)k; p.v = (const bf16_t *)v; p.o = (const bf16_t *)out;
  p.dout = (const bf16_t *)dout; p.lse = lse; p.mask = mask; p.rand_attn = ln.full ? nullptr : rand_attn;
  p.delta = delta; p.dq = (bf16_t *)dq; p.dk = (bf16_t *)dk; p.dv = (bf16_t *)dv; p.ws = nullptr;
  p.B = B; p.H = H; p.L = L; p.nb = ln.p.nb; p.block = block; p.r = r;
  p.full = ln.full ? 1 : 0;
  p.qk = (ln.p.mode & kModeQK) ? 1 : 0;
  p.skip = (mask && !(flags & BBSA_FLAG_KEEP_PADDED_BLOCKS)) ? 1 : 0;
  p.tiles = block / kT;
  p.chunks = std::max(std::min(p.nb, 2), (p.nb + kChunkBlocks - 1) / kChunkBlocks);
  p.n_grows = ln.full ? p.nb : 2;
  const int64_t bh = (int64_t)B * H;
  p.lanes = bh >= 8 ? 8 : 1;
  p.glob_items = p.n_grows * p.tiles * p.chunks;
  p.mid_items = ln.full ? 0 : (p.nb - 2) * p.tiles;
  const int64_t pairs_per_lane = (bh + p.lanes - 1) / p.lanes;
  const int64_t n_glob_lane = pairs_per_lane * p.glob_items;
  const int64_t grid = p.lanes * (n_glob_lane + pairs_per_lane * p.mid_items);
  const int64_t rows = bh * L;
  p.n_part = bh * p.n_grows * p.tiles * p.chunks;
  if (grid > 0x7fffffff || n_glob_lane > 0x7fffffff || (rows + 31) / 32 > 0x7fffffff ||
      (int64_t)p.glob_items * pairs_per_lane > 0x7fffffff)
    return BBSA_ERR_UNSUPPORTED;
  p.n_glob_lane = (int)n_glob_lane;
  // Workspace: the row terms, the query tiles' flags, then (with split rows)
  // the partials.
  {
    const size_t rt_floats = ((size_t)rows + 63) / 64 * 64;
    const size_t live_ints = ((size_t)bh * p.nb * p.tiles + 63) / 64 * 64;
    const size_t part_floats = p.chunks > 1 ? (size_t)(3 * p.n_part) * kT * kD : 0;
    float *ws = nullptr;
    const int rc = library_workspace((rt_floats + live_ints + part_floats) * sizeof(float), stream, &ws);
    if (rc != BBSA_OK) return rc;
    p.rterm = ws;
    p.live = (int *)(ws + rt_floats);
    p.ws = ws + rt_floats + live_ints;
  }
  if (mask) hipLaunchKernelGGL(bbsa_bwd_dq<true>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  else hipLaunchKernelGGL(bbsa_bwd_dq<false>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  if (p.qk) hipLaunchKernelGGL(bbsa_bwd_dkdv<true>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  else hipLaunchKernelGGL(bbsa_bwd_dkdv<false>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  if (p.chunks > 1) {
    hipLaunchKernelGGL(bbsa_bwd_merge, dim3((unsigned)(3 * (p.n_part / p.chunks))), dim3(256), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  }
  return st;
}
