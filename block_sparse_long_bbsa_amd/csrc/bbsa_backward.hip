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
//   * bbsa_bwd_delta: D per query row (fp32);
//   * bbsa_bwd_dq: one wavefront per 32-query tile, walking the tile's key
//     blocks (the forward's list) 32 keys at a time: S^T = K Q^T and
//     dP^T = V dO^T on MFMA 32x32x16 bf16 (Q and dO in registers, K and V
//     rows from LDS), dS^T = P^T (dP^T - D) in registers, then
//     dQ^T += K^T dS^T (K read transposed from LDS);
//   * bbsa_bwd_dkdv: one wavefront per 32-key tile, walking the query blocks
//     that attend its key block (global rows, the window, and the rows whose
//     plan picked it, found by scanning the plan) 32 queries at a time:
//     S = Q K^T and dP = dO V^T (K and V in registers, Q and dO rows from
//     LDS), dV^T += dO^T P and dK^T += Q^T dS (Q and dO read transposed).
// Every tile goes from memory to LDS with buffer_load ... lds; the row offset
// rides in the range-checked per-lane offset, so rows past L read as zeros.
#include <hip/hip_runtime.h>

#include <cstdint>

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

// LDS row swizzles (16-byte chunk j of row k sits at chunk j ^ f(k)): R for
// tiles read by rows (MFMA A operand), T for tiles read transposed.
__device__ inline int swz_r(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ inline int swz_t(int row) { return ((row >> 1) & 1) << 2; }

__device__ inline int lane_id() { return (int)__builtin_amdgcn_workitem_id_x() & 63; }

struct BwdParams {
  const bf16_t *q, *k, *v, *o, *dout;
  const float *lse;          // [B, H, L]
  const float *mask;         // [B, L] or null
  const int32_t *rand_attn;  // [H, nb-2, r] or null (fallback)
  float *delta;              // [B, H, L]
  bf16_t *dq, *dk, *dv;
  int B, H, L, nb, block, r;
  int full;                  // every block attends every block
  int qk;                    // query x key masking
  int tiles;                 // 32-row tiles per block
};

// Per-lane DMA state of one 32 x 64 tile: lane l of instruction u loads row
// 8u + l/8 of the tile into LDS position tile + 1024u + 16l.
struct TileDma {
  int off_r[4];              // source byte offsets within the tile, R swizzle
  int off_t;                 // T swizzle (the same for the four instructions)
  __device__ void init(int lane) {
    const int drow = lane >> 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) off_r[u] = 2 * ((8 * u + drow) * kD + 8 * ((lane & 7) ^ swz_r(8 * u + drow))) - 1024 * u;
    off_t = 2 * (drow * kD + 8 * ((lane & 7) ^ swz_t(drow)));
  }
};

// Rows row0 .. row0+31 of a [L, 64] bf16 matrix (buffer resource rs) into
// LDS; rows at or past L read as zeros.
__device__ inline void dma_rows(__amdgpu_buffer_rsrc_t rs, unsigned char *dst, const TileDma &t, int row0, bool tsw) {
  const int base = row0 * (kD * 2);
  if (tsw) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_t + base, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_t + base, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_t + base, 0, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_t + base, 0, 3072, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[0] + base, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[1] + base, 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[2] + base, 0, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t *)dst, 16, t.off_r[3] + base, 0, 3072, 0);
  }
}

// A operands of the rows of an R-swizzled tile: row c, d = 16kk + 8h .. +7.
__device__ inline void read_rows(const unsigned char *src, int c, int h, bf16x8 (&a)[4]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a[kk] = *(const bf16x8 *)(src + c * 128 + 16 * ((2 * kk + h) ^ swz_r(c)));
}

// A operands of the transposed T-swizzled tile X (rows r, columns d): for
// d-tile dt and row step s, lane (c, h) gets X^T[32dt + c][the row slots
// 8h .. 8h+7 of step s], in the slot order that the B operands packed by
// pack_b use (slot 8h + e is row 16s + 4h + (e & 3) + 8 (e >> 2)).
__device__ inline void read_tr(const unsigned char *src, const int (&toff)[2], bf16x8 (&a)[2][2]) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + toff[dt] + 2048 * s));
      const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + toff[dt] + 2048 * s + 1024));
      a[dt][s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}
__device__ inline void tr_offsets(int lane, int (&toff)[2]) {
  const int G = lane >> 4, cc = lane & 15;
  const int row = 4 * (G >> 1) + (cc >> 2);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int chunk = 4 * dt + 2 * (G & 1) + ((cc & 3) >> 1);
    toff[dt] = row * 128 + 16 * (chunk ^ swz_t(row)) + 8 * (cc & 1);
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
// = row c of X) as bf16 rows row0 + c of a [L, 64] matrix.
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

__device__ inline float mask_at(const BwdParams &p, const float *mrow, int pos) {
  return pos < p.L ? (mrow ? mrow[pos] : 1.0f) : 0.0f;
}

// D[t] = sum_e dO[t, e] out[t, e] (one thread per row).
__global__ __launch_bounds__(256) void bbsa_bwd_delta(BwdParams p) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= (int64_t)p.B * p.H * p.L) return;
  const bf16x8 *a = (const bf16x8 *)(p.dout + row * kD);
  const bf16x8 *b = (const bf16x8 *)(p.o + row * kD);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kD / 8; ++i) {
    const bf16x8 x = a[i], y = b[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
  }
  p.delta[row] = acc;
}

// Key block of list position t of middle query block i (the forward's list:
// the two global blocks, the window without them, the plan's blocks), or the
// block itself for a full row.
__device__ inline int list_block(const BwdParams &p, const int32_t *plan_row, int i, int t, bool full_row) {
  if (full_row) return t;
  if (t == 0) return 0;
  if (t == 1) return p.nb - 1;
  const int nw = (i == 1 || i == p.nb - 2) ? 2 : 3;
  const int w0 = (i == 1) ? 1 : i - 1;
  if (t < 2 + nw) return w0 + (t - 2);
  return min(max(plan_row[t - 2 - nw], 0), p.nb - 1);
}

// dQ: one wavefront per 32-query tile; workgroups of one wavefront.  The
// tiles of the full rows (blocks 0 and nb-1, or every block on the fallback)
// come first in the grid.
__global__ __launch_bounds__(64) void bbsa_bwd_dq(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * 3 * kTile];   // per slot: K rows, K transposed, V rows
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int n_full_rows = p.full ? p.nb : 2;
  const int per_bh_full = n_full_rows * p.tiles;
  const int per_bh = p.nb * p.tiles;
  int w = (int)blockIdx.x;
  int bh, i, tile;
  if (w < p.B * p.H * per_bh_full) {
    bh = w / per_bh_full;
    const int x = w % per_bh_full;
    const int g = x / p.tiles;
    tile = x % p.tiles;
    i = p.full ? g : (g == 0 ? 0 : p.nb - 1);
  } else {
    w -= p.B * p.H * per_bh_full;
    const int per_bh_mid = per_bh - per_bh_full;
    bh = w / per_bh_mid;
    const int x = w % per_bh_mid;
    i = 1 + x / p.tiles;
    tile = x % p.tiles;
  }
  const int b = bh / p.H, hh = bh % p.H;
  const bool full_row = p.full || i == 0 || i == p.nb - 1;
  const int q0 = i * p.block + tile * kT;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = p.mask ? p.mask + (int64_t)b * p.L : nullptr;
  const int32_t *plan_row = full_row ? nullptr : p.rand_attn + ((int64_t)hh * (p.nb - 2) + (i - 1)) * p.r;
  const int n_blocks = full_row ? p.nb : (2 + ((i == 1 || i == p.nb - 2) ? 2 : 3) + p.r);
  const int steps_per_block = p.block / kT;
  const int n_steps = n_blocks * steps_per_block;

  TileDma dma;
  dma.init(lane);
  int toff[2];
  tr_offsets(lane, toff);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p.k + bh * seq), (short)0, p.L * kD * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p.v + bh * seq), (short)0, p.L * kD * 2, kBufferWord3);

  // Q and dO of the tile (B operands), and the query column's lse (log2
  // units, with the query x key constant taken out), D and mask factor.
  bf16x8 qf[4], df[4];
  load_b_rows(p.q + bh * seq, p.L, q0, c, h, qf);
  load_b_rows(p.dout + bh * seq, p.L, q0, c, h, df);
  const int qrow = q0 + c;
  const bool qlive = qrow < p.L;
  const float mq = p.qk ? (qlive ? mask_at(p, mrow, qrow) : 0.0f) : 1.0f;
  const float lse2 = qlive ? (p.lse[(int64_t)bh * p.L + qrow] - (p.qk ? kPadBias * (1.0f - mq) : 0.0f)) * kLog2e : 0.0f;
  const float dlt = qlive ? p.delta[(int64_t)bh * p.L + qrow] : 0.0f;

  auto key_of = [&](int st) {
    return list_block(p, plan_row, i, st / steps_per_block, full_row) * p.block + (st % steps_per_block) * kT;
  };
  auto issue = [&](int st) {
    unsigned char *s = lds + (st & 1) * 3 * kTile;
    const int key0 = key_of(st);
    dma_rows(krs, s, dma, key0, false);
    dma_rows(krs, s + kTile, dma, key0, true);
    dma_rows(vrs, s + 2 * kTile, dma, key0, false);
  };

  f32x16 dq[2] = {zero16(), zero16()};
  issue(0);
  for (int st = 0; st < n_steps; ++st) {
    // The transfer of step st has landed; the LDS reads of step st-1 (the
    // slot the next transfer overwrites) were consumed by its products.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (st + 1 < n_steps) issue(st + 1);
    const unsigned char *s = lds + (st & 1) * 3 * kTile;
    const int key0 = key_of(st);
    bf16x8 kr[4], vr[4], kt[2][2];
    read_rows(s, c, h, kr);
    read_rows(s + 2 * kTile, c, h, vr);
    read_tr(s + kTile, toff, kt);
    f32x16 sc = zero16(), dp = zero16();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      sc = mfma(kr[kk], qf[kk], sc);   // S^T[key][query c]
      dp = mfma(vr[kk], df[kk], dp);   // dP^T[key][query c]
    }
    // P^T and dS^T; register 4j + i is key key0 + 8j + 4h + i.
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + 8 * (e >> 2) + 4 * h + (e & 3);
      const float bias = mq * (kPadBias * (1.0f - mask_at(p, mrow, key)));
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e] + bias, kLog2e, -lse2));
      sc[e] = pr * (dp[e] - dlt);
    }
    bf16x8 dsb[2];
    pack_b(sc, dsb);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) dq[dt] = mfma(kt[dt][ss], dsb[ss], dq[dt]);   // dQ^T[d][query c]
  }
  store_t(p.dq + bh * seq, p.L, q0, c, h, dq);
}

// dK, dV: one wavefront per 32-key tile.  The query blocks that attend key
// block j: every block for a global key block (or on the fallback); else the
// two global blocks, the window {j-1, j, j+1} (without repeating a global
// one) and the middle blocks whose plan row picked j.
__global__ __launch_bounds__(64) void bbsa_bwd_dkdv(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * 4 * kTile];   // per slot: Q rows, Q tr, dO rows, dO tr
  const int lane = lane_id(), c = lane & 31, h = lane >> 5;
  const int n_full_cols = p.full ? p.nb : 2;
  const int per_bh_full = n_full_cols * p.tiles;
  const int per_bh = p.nb * p.tiles;
  int w = (int)blockIdx.x;
  int bh, j, tile;
  if (w < p.B * p.H * per_bh_full) {
    bh = w / per_bh_full;
    const int x = w % per_bh_full;
    const int g = x / p.tiles;
    tile = x % p.tiles;
    j = p.full ? g : (g == 0 ? 0 : p.nb - 1);
  } else {
    w -= p.B * p.H * per_bh_full;
    const int per_bh_mid = per_bh - per_bh_full;
    bh = w / per_bh_mid;
    const int x = w % per_bh_mid;
    j = 1 + x / p.tiles;
    tile = x % p.tiles;
  }
  const int b = bh / p.H, hh = bh % p.H;
  const bool full_col = p.full || j == 0 || j == p.nb - 1;
  const int k0 = j * p.block + tile * kT;
  const int64_t seq = (int64_t)p.L * kD;
  const float *mrow = p.mask ? p.mask + (int64_t)b * p.L : nullptr;
  const int steps_per_block = p.block / kT;

  TileDma dma;
  dma.init(lane);
  int toff[2];
  tr_offsets(lane, toff);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p.q + bh * seq), (short)0, p.L * kD * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p.dout + bh * seq), (short)0, p.L * kD * 2, kBufferWord3);

  // K and V of the tile (B operands: lane (c, h) = key k0 + c); the key
  // column's padding bias.
  bf16x8 kf[4], vf[4];
  load_b_rows(p.k + bh * seq, p.L, k0, c, h, kf);
  load_b_rows(p.v + bh * seq, p.L, k0, c, h, vf);
  const float kbias = kPadBias * (1.0f - mask_at(p, mrow, k0 + c));

  // The query blocks, in three groups: the fixed ones (globals and the
  // window, or all blocks), then plan rows found 64 entries at a time.
  int fixed[5];
  int n_fixed = 0;
  if (!full_col) {
    fixed[n_fixed++] = 0;
    fixed[n_fixed++] = p.nb - 1;
    for (int x = j - 1; x <= j + 1; ++x)
      if (x > 0 && x < p.nb - 1) fixed[n_fixed++] = x;
  }

  f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};
  // One query block: its query steps through LDS, accumulating dK and dV.
  auto run_block = [&](int i) {
    const int nst = steps_per_block;
    auto issue = [&](int st) {
      unsigned char *s = lds + (st & 1) * 4 * kTile;
      const int row0 = i * p.block + st * kT;
      dma_rows(qrs, s, dma, row0, false);
      dma_rows(qrs, s + kTile, dma, row0, true);
      dma_rows(drs, s + 2 * kTile, dma, row0, false);
      dma_rows(drs, s + 3 * kTile, dma, row0, true);
    };
    issue(0);
    for (int st = 0; st < nst; ++st) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (st + 1 < nst) issue(st + 1);
      const unsigned char *s = lds + (st & 1) * 4 * kTile;
      const int row0 = i * p.block + st * kT;
      bf16x8 qr[4], dr[4], qt[2][2], dt2[2][2];
      read_rows(s, c, h, qr);
      read_rows(s + 2 * kTile, c, h, dr);
      read_tr(s + kTile, toff, qt);
      read_tr(s + 3 * kTile, toff, dt2);
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc = mfma(qr[kk], kf[kk], sc);   // S[query][key c]
        dp = mfma(dr[kk], vf[kk], dp);   // dP[query][key c]
      }
      // Register 4jj + ii is query row0 + 8jj + 4h + ii.
      f32x16 pm, dsv;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qrow = row0 + 8 * (e >> 2) + 4 * h + (e & 3);
        float pr = 0.0f, ds = 0.0f;
        if (qrow < p.L) {
          const float mq = p.qk ? mask_at(p, mrow, qrow) : 1.0f;
          const float lse2 =
              (p.lse[(int64_t)bh * p.L + qrow] - (p.qk ? kPadBias * (1.0f - mq) : 0.0f)) * kLog2e;
          pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e] + mq * kbias, kLog2e, -lse2));
          ds = pr * (dp[e] - p.delta[(int64_t)bh * p.L + qrow]);
        }
        pm[e] = pr;
        dsv[e] = ds;
      }
      bf16x8 pb[2], db[2];
      pack_b(pm, pb);
      pack_b(dsv, db);
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          dv[d2] = mfma(dt2[d2][ss], pb[ss], dv[d2]);   // dV^T[d][key c]
          dk[d2] = mfma(qt[d2][ss], db[ss], dk[d2]);    // dK^T[d][key c]
        }
    }
  };

  if (full_col) {
    for (int i = 0; i < p.nb; ++i) run_block(i);
  } else {
    for (int x = 0; x < n_fixed; ++x) run_block(fixed[x]);
    // Plan rows that picked j (rows are middle blocks outside j's window,
    // so none repeats a fixed block); a bad plan's entries are clamped as in
    // the forward.
    const int32_t *plan_h = p.rand_attn + (int64_t)hh * (p.nb - 2) * p.r;
    const int n_entries = (p.nb - 2) * p.r;
    for (int e0 = 0; e0 < n_entries; e0 += 64) {
      const int e = e0 + lane;
      const bool hit = e < n_entries && min(max(plan_h[min(e, n_entries - 1)], 0), p.nb - 1) == j;
      unsigned long long bits = __builtin_amdgcn_ballot_w64(hit);
      while (bits) {
        const int l = __builtin_ctzll(bits);
        bits &= bits - 1;
        const int row = 1 + (e0 + l) / p.r;   // middle query block of that plan entry
        // A clamped bad plan could pick a fixed block; it is counted once.
        bool dup = false;
        for (int x = 0; x < n_fixed; ++x) dup |= fixed[x] == row;
        if (!dup) run_block(row);
      }
    }
  }
  store_t(p.dk + bh * seq, p.L, k0, c, h, dk);
  store_t(p.dv + bh * seq, p.L, k0, c, h, dv);
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
  if (dtype != BBSA_BF16) return BBSA_ERR_UNSUPPORTED;
  BwdParams p;
  p.q = (const bf16_t *)q; p.k = (const bf16_t *)k; p.v = (const bf16_t *)v; p.o = (const bf16_t *)out;
  p.dout = (const bf16_t *)dout; p.lse = lse; p.mask = mask; p.rand_attn = ln.full ? nullptr : rand_attn;
  p.delta = delta; p.dq = (bf16_t *)dq; p.dk = (bf16_t *)dk; p.dv = (bf16_t *)dv;
  p.B = B; p.H = H; p.L = L; p.nb = ln.p.nb; p.block = block; p.r = r;
  p.full = ln.full ? 1 : 0;
  p.qk = (ln.p.mode & kModeQK) ? 1 : 0;
  p.tiles = block / kT;
  const int64_t rows = (int64_t)B * H * L;
  const int64_t grid = (int64_t)B * H * p.nb * p.tiles;
  if (grid > 0x7fffffff || (rows + 255) / 256 > 0x7fffffff) return BBSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(bbsa_bwd_delta, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  hipLaunchKernelGGL(bbsa_bwd_dq, dim3((unsigned)grid), dim3(64), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  hipLaunchKernelGGL(bbsa_bwd_dkdv, dim3((unsigned)grid), dim3(64), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return BBSA_ERR_HIP;
  return st;
}
