// Work decomposition of the BigBird block-sparse attention forward: the
// launch parameters, the mapping from (workgroup, wavefront) to a work item,
// and the key-block list each item walks.  Everything here compiles for the
// host as well as for gfx950, so that the host can validate a call, size its
// launch and reproduce the kernels' item mapping (for the work-map query and
// the CPU tests) with the very code the kernels run.
//
// What is covered ("models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的
// 完整实践", section "BigBird：从二次方注意力到线性稀疏注意力"; "BigBirdPegasus
// 长序列条件生成模型详解…", sections "三类注意力组合全局 局部 随机" and
// "序列过短时的自动回退"): per (batch, head), query blocks 0 and nb-1 attend
// every key block; a middle query block i attends {0, nb-1}, {i-1, i, i+1}
// and the r blocks of its plan row; a sequence of at most (5 + 2r) blocks is
// computed as full attention (every query block a full row).
//
// Host compilers that are not hipcc see this file with __host__ and
// __device__ defined empty on their command line.
#ifndef BBSA_SCHEDULE_H
#define BBSA_SCHEDULE_H

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "bbsa.h"

namespace bbsa_sched {

constexpr int kD = 64;        // head dimension
constexpr int kQT = 64;       // query rows per work unit (one wavefront's tile)
constexpr int kStep = 32;     // keys per softmax step
constexpr int kGroup = 4;     // items per bf16 workgroup (one per wavefront)
constexpr int kF32Waves = 4;  // wavefronts per fp32 workgroup (they split one item's rows)
// Below this many wavefronts of work the fp32 path cuts its items finer:
// full-row chunks of kF32SmallChunkKeys keys, middle rows in kF32SmallParts
// key parts (about two wavefronts per SIMD are needed to fill the chip).
constexpr int64_t kF32SplitBelowWaves = 2048;
constexpr int kF32SmallChunkKeys = 128;
constexpr int kF32SmallParts = 4;
// One split-K partial: O[64][64] fp32, then the 64 reference maxima (log2
// units), then the 64 row sums, then the partial's padding-bias level (the
// maxima are relative to it; see the fp32 kernel) and three unused floats
// that keep every partial 16-byte aligned.
constexpr int kPartialFloats = kQT * kD + 2 * kQT + 4;
constexpr int kMergeSlices = kQT / 4;   // merge-kernel workgroups per row tile
constexpr int kMaxL = 1 << 24;          // longest supported sequence (tokens)
// Wavefront slots of the bf16 attention kernel on MI355X: 256 CUs, two
// four-wavefront workgroups each.
constexpr int64_t kBf16Slots = 2048;

// Division of 31-bit non-negative integers by a divisor fixed at launch:
// q = (mulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.s = 0;
  while ((1ull << f.s) < d) ++f.s;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << f.s) - d)) / d + 1);
  return f;
}
__host__ __device__ inline int fdiv(int n, const FastDiv &f) {
  const uint32_t hi = (uint32_t)(((uint64_t)(uint32_t)n * f.m) >> 32);
  return (int)((hi + (uint32_t)n) >> f.s);
}

// Kernel variants (template argument of the attention kernels).
constexpr int kModeMask = 1;     // a padding mask is given
constexpr int kModeRagged = 2;   // L is not a multiple of the block: positions L .. nb * block - 1 are padding
constexpr int kModeQK = 4;       // query x key masking: bias -10000 (1 - m[query] m[key])

struct Params {
  const void *q, *k, *v;
  const float *mask;         // [B, L] or null
  const int32_t *rand_attn;  // [H, nb-2, r]
  void *out;
  float *lse;                // [B, H, L] row log-sum-exp, or null
  float *ws;                 // split-K partials
  int64_t seq_stride;        // L * d elements per (batch, head)
  int B, H, L, nb, block, r; // L: the real length; nb = ceil(L / block)
  int mode;                  // kMode* bits of the launched kernels
  int qtiles;                // block / 64: 64-row query tiles per query block
  int n_rows_global;         // query blocks handled as full rows: 2, or nb on the fallback
  int chunks;                // key chunks per full row (block range [c nb / chunks, (c + 1) nb / chunks))
  int group;                 // items per workgroup: 4 on the bf16 path (a full row's chunks in fours), else 1
  int nparts;                // split-K partials per full row left for the merge kernel: chunks / group
  int mparts;                // key parts per middle row (fp32 path with few items: 4; else 1)
  int comb_rows_global;      // per (batch, head): full rows the merge kernel combines (0 or n_rows_global)
  int comb_rows_mid;         // per (batch, head): middle rows the merge kernel combines (0 or nb - 2)
  int64_t mid_part_base;     // index of the first middle-row partial in the workspace
  int n_global_items;        // per (batch, head): n_rows_global * qtiles * chunks
  int items_per_bh;          // n_global_items + middle items
  int bh_total;              // B * H
  int xcd_remap;             // 1: map workgroups so one (batch, head) stays on one XCD
  int skip_padded;           // 1: bf16 tiles leave out key blocks whose keys are all padded
  int n_glob;                // full-row items before the first middle item (per XCD lane)
  FastDiv div_global;        // n_global_items
  FastDiv div_mid;           // middle items per (batch, head), at least 1
  FastDiv div_row;           // qtiles * chunks
  FastDiv div_chunks;        // chunks
  FastDiv div_qtiles;        // qtiles
  FastDiv div_mparts;        // mparts
  FastDiv div_heads;         // H
};

// A work item: one 64-row query tile (qt) of query block qblock of one
// (batch, head), against either the key blocks of a middle row (or one key
// part of them) or one key chunk of a full row.
struct Item {
  int bh;
  int qblock;
  int qt;
  int grow;       // full-row index (partials), -1 for a middle row
  int chunk;      // key chunk of a full row, or key part of a middle row
};

// Workgroup -> item.  Workgroups are dispatched in index order, so the
// longest items (full-row chunks) of every (batch, head) come first and the
// middle rows fill in behind them; this keeps long items out of the tail.
// With the XCD remap, workgroup w runs on XCD x = w % 8 and serves only the
// (batch, head) pairs x, x + 8, x + 16, ..., so all items of one pair share
// one L2.  With p.group items per workgroup, wavefront wv of workgroup wg
// takes item wv of the workgroup's run of p.group consecutive items; the
// full-row items of a pair come as whole groups (their count is a multiple of
// p.group), so a group of full-row items is the p.group chunks of one row
// tile.  All divisions use the launch's precomputed FastDiv constants.
__host__ __device__ inline Item decode_item(const Params &p, int wg, int wv) {
  const int lg_lanes = p.xcd_remap ? 3 : 0;
  const int x = wg & ((1 << lg_lanes) - 1), slot = (wg >> lg_lanes) * p.group + wv;
  const bool g = slot < p.n_glob;
  const int sg = g ? slot : 0, sm = g ? 0 : slot - p.n_glob;
  const int jg = fdiv(sg, p.div_global), jm = fdiv(sm, p.div_mid);
  const int j = g ? jg : jm;
  const int local = g ? sg - jg * p.n_global_items : p.n_global_items + (sm - jm * (int)p.div_mid.d);
  const int bh = x + (j << lg_lanes);
  const bool global_row = local < p.n_global_items;
  const int lr = global_row ? local : 0;
  const int m = global_row ? 0 : local - p.n_global_items;
  const int grow = fdiv(lr, p.div_row);
  const int rem = lr - grow * (int)p.div_row.d;
  const int qt_g = fdiv(rem, p.div_chunks);
  // Middle item m = key part + mparts * (query tile + qtiles * (row - 1)).
  const int mp = fdiv(m, p.div_mparts);
  const int mq = fdiv(mp, p.div_qtiles);
  Item it;
  it.bh = bh;   // >= bh_total marks an idle wavefront
  it.grow = global_row ? grow : -1;
  it.qt = global_row ? qt_g : mp - mq * p.qtiles;
  it.chunk = global_row ? rem - qt_g * p.chunks : m - mp * p.mparts;
  it.qblock = global_row ? ((p.n_rows_global == 2) ? (grow == 0 ? 0 : p.nb - 1) : grow) : 1 + mq;
  return it;
}

// The key blocks an item walks, one 32-key step at a time.  Lane t of `blk`
// holds the t-th key block of the item (at most 64 blocks); the kernels read
// it back with v_readlane, so advancing touches no memory.
struct KeyWalk {
  int n_steps;         // uniform
  int steps_per_block; // uniform
  int blk;             // per lane: key block at list position `lane`
  int first_blk;       // uniform: the block at position 0
};

// The key block list of an item, seen from lane `lane`, in two parts so that
// the plan entries can be loaded early and used late: make_walk_base fills
// everything but the random blocks and reads the lane's plan entry (rnd;
// rslot is the lane's slot in the plan row, -1 if none); merge_plan puts the
// random blocks in, clamped to [0, nb) so that a bad plan never reads outside
// the sequence.  A middle row lists the two global blocks, its window without
// them, then its random blocks; a full-row chunk lists every p.group-th block
// of its group's range (below).  A three-block window is listed by block
// index mod 3: the four consecutive query blocks of a workgroup have
// overlapping windows, and this order puts a block they share at the same
// list position, so their wavefronts fetch it at the same step and the later
// fetches find it in the caches.
__host__ __device__ inline KeyWalk make_walk_base(const Params &p, const Item &it, int lane, int &rnd,
                                                  int &rslot) {
  KeyWalk w;
  w.steps_per_block = p.block / kStep;
  const bool middle = it.grow < 0;
  const int i = it.qblock;
  const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
  // A full-row chunk: the p.group chunks of a workgroup (a power of two)
  // share their group's block range [g0, g1), and chunk u of the group takes
  // every p.group-th block of it from g0 + u, so that blocks whose keys are
  // all padded (a padded tail) spread evenly over the chunks that merge
  // together.  May be empty if the range has fewer than p.group blocks.
  const int u = it.chunk & (p.group - 1), lgg = 31 - __builtin_clz((unsigned)p.group);
  const int g0 = fdiv((it.chunk - u) * p.nb, p.div_chunks);
  const int g1 = fdiv((it.chunk - u + p.group) * p.nb, p.div_chunks);
  const int first = g0 + u;
  const int nblk = middle ? 2 + nw + p.r : std::max(0, (g1 - first + p.group - 1) >> lgg);
  w.n_steps = nblk * w.steps_per_block;
  w.first_blk = middle ? 0 : first;
  int blk;
  rslot = -1;
  rnd = 0;
  if (middle) {
    const int w0 = (i == 1) ? 1 : i - 1;
    const int h = it.bh - fdiv(it.bh, p.div_heads) * p.H;
    const int32_t *ra_row = p.rand_attn + ((int64_t)h * (p.nb - 2) + (i - 1)) * p.r;
    const int t = lane - 2 - nw;
    rnd = ra_row[std::min(std::max(t, 0), p.r - 1)];
    rslot = (t >= 0 && t < p.r) ? t : -1;
    blk = 0;
    if (lane == 1) blk = p.nb - 1;
    else if (lane >= 2 && lane < 2 + nw) blk = (nw == 3) ? (i - 1) + ((lane - 2) - (i - 1) % 3 + 3) % 3 : w0 + (lane - 2);
  } else {
    blk = first + (std::max(std::min(lane, nblk - 1), 0) << lgg);
  }
  w.blk = blk;
  return w;
}
__host__ __device__ inline void merge_plan(const Params &p, KeyWalk &w, int rnd, int rslot) {
  if (rslot >= 0) w.blk = std::min(std::max(rnd, 0), p.nb - 1);
}

// Launch geometry of one call.
struct Launch {
  Params p;
  int64_t grid;         // attention-kernel workgroups
  int block_threads;    // threads per attention-kernel workgroup
  int64_t comb_grid;    // merge-kernel workgroups (0: no merge kernel)
  int64_t n_partials;   // split-K partials in the workspace
  bool full;            // short-sequence fallback: full attention
};

// Validate a forward call and size its launch.  flags: BBSA_FLAG_* (a
// length that is not a multiple of the block needs BBSA_FLAG_PAD_TO_BLOCK);
// lse: optional row log-sum-exp output.  Returns BBSA_OK,
// BBSA_OK_FULL_FALLBACK or a negative status; no HIP call is made.
inline int setup_forward_ex(const void *q, const void *k, const void *v, const float *mask,
                            const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                            void *out, float *lse, int dtype, unsigned flags, Launch *launch) {
  if (!q || !k || !v || !out || !launch) return BBSA_ERR_ARG;
  if (flags & ~(unsigned)(BBSA_FLAG_PAD_TO_BLOCK | BBSA_FLAG_QUERY_KEY_MASK | BBSA_FLAG_KEEP_PADDED_BLOCKS))
    return BBSA_ERR_ARG;
  // The kernels move q, k, v, out and the mask in 16-byte pieces.
  auto misaligned = [](const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) != 0; };
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
      (mask && misaligned(mask, 16)) || (rand_attn && misaligned(rand_attn, 4)) || (lse && misaligned(lse, 4)))
    return BBSA_ERR_ARG;
  if (B <= 0 || H <= 0 || L <= 0 || d <= 0 || block <= 0 || r < 1) return BBSA_ERR_ARG;
  if (dtype != BBSA_BF16 && dtype != BBSA_F32) return BBSA_ERR_UNSUPPORTED;
  if (d != kD || (block != 64 && block != 128)) return BBSA_ERR_UNSUPPORTED;
  const bool ragged = L % block != 0;
  if (ragged && !(flags & BBSA_FLAG_PAD_TO_BLOCK)) return BBSA_ERR_SHAPE;
  if (L > kMaxL) return BBSA_ERR_UNSUPPORTED;
  const int nb = L / block + (ragged ? 1 : 0);
  // The fallback test on the padded length: (5 + 2r) * block is a multiple
  // of the block, so it is the same test on L.
  const bool full = (int64_t)L <= (int64_t)(5 + 2 * (int64_t)r) * block;
  if (!full) {
    if (!rand_attn) return BBSA_ERR_ARG;
    if (nb < 5 + r) return BBSA_ERR_SHAPE;
    if (5 + r > 64) return BBSA_ERR_UNSUPPORTED;   // a middle row lists at most 64 key blocks
  }
  // Sizes the 32-bit item arithmetic and the 2^40-element addressing cover;
  // one (batch, head)'s K or V rows must fit a 32-bit byte range (the bf16
  // kernel addresses them through a buffer resource): L <= 2^24.
  const int64_t bh = (int64_t)B * H;
  if (bh > 0x7fffffff || (int64_t)B * H * nb * block * kD > ((int64_t)1 << 40)) return BBSA_ERR_UNSUPPORTED;

  Params p{};
  p.q = q; p.k = k; p.v = v; p.mask = mask; p.rand_attn = rand_attn; p.out = out; p.lse = lse;
  p.seq_stride = (int64_t)L * kD;
  p.B = B; p.H = H; p.L = L; p.nb = nb; p.block = block; p.r = r;
  p.mode = (mask ? kModeMask : 0) | (ragged ? kModeRagged : 0) |
           ((mask && (flags & BBSA_FLAG_QUERY_KEY_MASK)) ? kModeQK : 0);
  p.skip_padded = (mask && !ragged && dtype == BBSA_BF16 && !(flags & BBSA_FLAG_KEEP_PADDED_BLOCKS)) ? 1 : 0;
  p.qtiles = block / kQT;
  p.n_rows_global = full ? nb : 2;
  // Full rows are cut into chunks so they do not form the tail: 256 keys on
  // the slower fp32 path; on the bf16 path 1024, 2048 or 4096 keys, the
  // longest whose 32-key steps stay within one wavefront slot's share of
  // the launch's steps (kBf16Slots slots), since longer chunks leave fewer
  // partials to merge.  On the bf16 path the chunk count is a multiple of
  // kGroup: each workgroup runs kGroup chunks of one row tile and merges
  // them in LDS, and the merge kernel combines the chunks / kGroup group
  // results (none for rows of up to 4 chunks).
  int per_chunk = 256 / block;   // blocks
  if (dtype == BBSA_BF16) {
    const int64_t spb = block / kStep;
    const int64_t steps = bh * p.qtiles * spb *
                          ((int64_t)p.n_rows_global * nb + (full ? 0 : (int64_t)(nb - 2) * (5 + r)));
    int keys = 1024;
    while (keys < 4096 && 2 * keys / kStep <= steps / kBf16Slots) keys *= 2;
    per_chunk = keys / block;
  }
  bool f32_small = false;
  if (dtype == BBSA_F32 && !full) {
    const int64_t items = bh * p.qtiles * (2 * (int64_t)((nb + per_chunk - 1) / per_chunk) + (nb - 2));
    if (items * kF32Waves < kF32SplitBelowWaves) {
      f32_small = true;
      per_chunk = std::max(1, kF32SmallChunkKeys / block);
    }
  }
  if (dtype == BBSA_BF16) {
    p.group = kGroup;
    p.chunks = kGroup * ((nb + kGroup * per_chunk - 1) / (kGroup * per_chunk));
  } else {
    p.group = 1;
    p.chunks = (nb + per_chunk - 1) / per_chunk;
  }
  p.nparts = p.chunks / p.group;
  p.n_global_items = p.n_rows_global * p.qtiles * p.chunks;
  p.mparts = f32_small ? kF32SmallParts : 1;
  const int64_t n_middle = full ? 0 : (int64_t)(nb - 2) * p.qtiles * p.mparts;
  const int64_t items_per_bh = (int64_t)p.n_global_items + n_middle;
  p.xcd_remap = bh >= 8 ? 1 : 0;
  const int64_t items_per_lane = (p.xcd_remap ? (bh + 7) / 8 : bh) * items_per_bh;
  const int64_t grid = (p.xcd_remap ? 8 : 1) * ((items_per_lane + p.group - 1) / p.group);
  const int64_t n_part_full = (p.nparts > 1) ? bh * p.n_rows_global * p.qtiles * p.nparts : 0;
  const int64_t n_part_mid = (p.mparts > 1) ? bh * (nb - 2) * p.qtiles * p.mparts : 0;
  p.mid_part_base = n_part_full;
  p.comb_rows_global = (p.nparts > 1) ? p.n_rows_global : 0;
  p.comb_rows_mid = (p.mparts > 1) ? nb - 2 : 0;
  const int64_t comb_grid = (int64_t)kMergeSlices * bh * (p.comb_rows_global + p.comb_rows_mid) * p.qtiles;
  // The chunk bounds c * nb / chunks are formed in 32-bit arithmetic.
  if (items_per_lane > 0x7fffffff || grid > 0x7fffffff || comb_grid > 0x7fffffff ||
      (int64_t)p.chunks * nb > 0x7fffffff)
    return BBSA_ERR_UNSUPPORTED;
  p.items_per_bh = (int)items_per_bh;
  p.bh_total = (int)bh;
  p.n_glob = (int)((p.xcd_remap ? (bh + 7) / 8 : bh) * p.n_global_items);
  p.div_global = make_fastdiv((uint32_t)p.n_global_items);
  p.div_mid = make_fastdiv((uint32_t)std::max<int64_t>(n_middle, 1));
  p.div_row = make_fastdiv((uint32_t)(p.qtiles * p.chunks));
  p.div_chunks = make_fastdiv((uint32_t)p.chunks);
  p.div_qtiles = make_fastdiv((uint32_t)p.qtiles);
  p.div_mparts = make_fastdiv((uint32_t)p.mparts);
  p.div_heads = make_fastdiv((uint32_t)H);

  launch->p = p;
  launch->grid = grid;
  launch->block_threads = (dtype == BBSA_BF16) ? 64 * p.group : 64 * kF32Waves;
  launch->comb_grid = (n_part_full + n_part_mid > 0) ? comb_grid : 0;
  launch->n_partials = n_part_full + n_part_mid;
  launch->full = full;
  return full ? BBSA_OK_FULL_FALLBACK : BBSA_OK;
}

// The library-owned workspace of the current device and `stream` (see
// bbsa_forward in bbsa.h), at least `bytes` long.
int library_workspace(size_t bytes, hipStream_t stream, float **ws);

// The fp32 backward's kernels (csrc/bbsa_backward_f32.hip), launched by
// bbsa_backward after its argument checks; nb is the padded block count.
int launch_backward_f32(const void *q, const void *k, const void *v, const void *out, const void *dout,
                        const float *mask, const int32_t *rand_attn, int B, int H, int L, int nb, int block,
                        int r, bool full, bool qk, void *dq, void *dk, void *dv, float *delta,
                        hipStream_t stream);

inline int setup_forward(const void *q, const void *k, const void *v, const float *mask,
                         const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                         void *out, int dtype, Launch *launch) {
  return setup_forward_ex(q, k, v, mask, rand_attn, B, H, L, d, block, r, out, nullptr, dtype, 0u, launch);
}

}  // namespace bbsa_sched

#endif  // BBSA_SCHEDULE_H
