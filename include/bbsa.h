/*
 * bbsa.h -- C ABI of the BigBird block-sparse attention forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *
 *   "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
 *   section "BigBird：从二次方注意力到线性稀疏注意力": Q, K and V are split
 *   into blocks of `block` tokens; the first and the last query block attend
 *   to the whole sequence; every middle query block attends to the first and
 *   the last key block, to a 3-block window around itself and to
 *   `num_rand_blocks` (here `r`) random key blocks; masked positions get an
 *   additive -10000 before the row softmax.
 *
 *   Same page, section "随机块掩码是如何生成的": the random blocks of each
 *   middle row come from a per-head adjacency (`rand_attn`) that never
 *   overlaps the row's window; the plan is fixed per head when the layer is
 *   built, with the layer index as the seed.
 *
 *   "BigBirdPegasus 长序列条件生成模型详解从稀疏注意力原理到 Transformers 实战",
 *   sections "序列长度的块对齐要求" (length must be a multiple of the block:
 *   error otherwise), "序列过短时的自动回退" (full attention when the length
 *   does not exceed (5 + 2r) * block), "使用限制与注意事项" (r = 0 is not
 *   supported).
 *
 * Readings taken where the pages are silent: no internal softmax scale (fold
 * 1/sqrt(d) into Q); the padding mask is applied on the key side only, as
 * bias -10000 * (1 - mask[b, key]); rows 1 and nb-2 attend 4 + r distinct
 * blocks; the random plan is drawn with SplitMix64 (see bbsa_plan_rand_attn).
 *
 * Layouts: q, k, v, out are [B, H, L, d] row-major (d contiguous) in device
 * memory; mask is float32 [B, L]; rand_attn is int32 [H, nb-2, r] where
 * nb = L / block and row i-1 lists the random key blocks of middle query
 * block i.  Supported: d = 64, block in {64, 128}, bf16 or fp32 elements.
 *
 * Ownership: the caller owns every buffer it passes; the library never frees
 * caller memory.  The library owns one split-K workspace per device (grown on
 * demand with hipMalloc, released by bbsa_release_workspace); it is used only
 * when a row needs more than one partial: bf16 rows longer than 4096 keys,
 * fp32 rows longer than 256 keys, and, in fp32 calls with fewer than 2048
 * wavefronts of work, full rows longer than 128 keys and every middle row.
 *
 * Errors: every function returns a status code (below); no C++ exception
 * crosses this interface.  Argument checks run on the host before any HIP
 * call, so an invalid call leaves the device untouched.
 */
#ifndef BBSA_H
#define BBSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out. */
typedef enum { BBSA_BF16 = 0, BBSA_F32 = 1 } bbsa_dtype;

/* Status codes. */
enum {
  BBSA_OK = 0,               /* success */
  BBSA_OK_FULL_FALLBACK = 1, /* success; L <= (5+2r)*block, computed as full attention */
  BBSA_ERR_ARG = -1,         /* null or misaligned pointer, or B/H/L/d/block <= 0, or r < 1 */
  BBSA_ERR_SHAPE = -2,       /* L % block != 0, or nb < 5 + r where a plan is required */
  BBSA_ERR_UNSUPPORTED = -3, /* d != 64, block not in {64, 128}, unknown dtype, too large */
  BBSA_ERR_HIP = -4,         /* a HIP call or kernel launch failed */
  BBSA_ERR_PLAN = -5         /* rand_attn violates an invariant (bbsa_check_rand_attn) */
};

/*
 * Build the random-block adjacency on the host.
 *
 * rand_attn: host buffer of H * (nb-2) * r int32, caller-owned, written as
 *            [H][nb-2][r].
 * For each head h (in order), each middle row i = 1..nb-2 (in order), pick t
 * = 0..r-1: the candidates are the middle blocks 1..nb-2 at distance > 1 from
 * i (ascending); pick t swaps candidate t with candidate t + U(n - t) (partial
 * Fisher-Yates) and stores it.  U(m) is an exactly uniform draw from one
 * SplitMix64 stream seeded with `seed` (rejection of outputs below
 * 2^64 mod m, then mod m).
 *
 * Returns BBSA_OK; BBSA_ERR_ARG for a null buffer, H < 1, nb < 1 or r < 1;
 * BBSA_ERR_SHAPE when nb < 5 + r (a middle row would have fewer than r
 * candidates).
 */
int bbsa_plan_rand_attn(int32_t *rand_attn, int H, int nb, int r, uint64_t seed);

/*
 * Check a host plan [H][nb-2][r]: every entry a middle block (1..nb-2), the r
 * entries of a row distinct, none within distance 1 of the row's block.
 * Returns BBSA_OK, BBSA_ERR_PLAN on a violation, BBSA_ERR_ARG / _SHAPE on bad
 * arguments.
 */
int bbsa_check_rand_attn(const int32_t *rand_attn, int H, int nb, int r);

/*
 * Block-sparse attention forward on `stream`.
 *
 * q, k, v:   device, [B, H, L, d] of `dtype`, 16-byte aligned (as are out
 *            and mask; rand_attn 4-byte aligned), else BBSA_ERR_ARG.
 * mask:      device float32 [B, L], 1 = valid key, 0 = padding (fractional
 *            values act through the bias -10000 * (1 - mask)); NULL = all
 *            keys valid.
 * rand_attn: device int32 [H, nb-2, r] from bbsa_plan_rand_attn; ignored
 *            (may be NULL) when the call falls back to full attention.  A
 *            plan that breaks the invariants never causes an out-of-bounds
 *            read (indices are clamped), but the result is then unspecified.
 * out:       device, [B, H, L, d] of `dtype`, fully overwritten.
 * stream:    HIP stream; kernels are enqueued on it, no host synchronisation.
 * dtype:     BBSA_BF16 (fp32 accumulation, bf16 output) or BBSA_F32.
 *
 * Limits (BBSA_ERR_UNSUPPORTED beyond them): d = 64; block 64 or 128;
 * on the sparse path 5 + r <= 64 (a middle row attends at most 64 key
 * blocks); B * H * L * d <= 2^40 elements; at most 2^31 - 1 workgroups.
 *
 * Returns BBSA_OK, or BBSA_OK_FULL_FALLBACK when L <= (5 + 2r) * block (every
 * query block then attends every key block), or a negative error code.  All
 * argument checks happen before any HIP call.  The library-owned workspace
 * (used only when a full row needs more than one partial, see above) is
 * allocated or grown on first use for a shape, which synchronises the
 * device; such calls that overlap on one device through different streams
 * must not race on it (the library serialises its own bookkeeping with a
 * mutex, not the kernels).  Calls that need no workspace (bf16 with
 * L <= 4096) share nothing.
 *
 * Graph capture: a call enqueues kernel launches only (no memset, no copy,
 * no host synchronisation), so it can be recorded into a HIP graph once the
 * workspace is large enough, e.g. after one eager call of the same shape;
 * replays then reuse the captured pointers.  Kernel timing must be off
 * during capture.
 */
int bbsa_forward(const void *q, const void *k, const void *v, const float *mask,
                 const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                 void *out, hipStream_t stream, int dtype);

/* Static string describing a status code. */
const char *bbsa_status_string(int status);

/* Free the library-owned workspace on every device. */
void bbsa_release_workspace(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int bbsa_version(void);

/*
 * Kernel timing for benchmarks.  When enabled, bbsa_forward records a pair of
 * HIP events on `stream` around its main attention kernel and around its
 * split-K combine kernel when one runs (combine_ms counts 0 otherwise).
 * bbsa_timing_read synchronises on the recorded
 * events, returns the summed durations in milliseconds and the number of
 * timed calls, then clears the record.  At most 4096 calls are recorded
 * between reads; later calls are not timed.
 */
int bbsa_timing_enable(int enable);
int bbsa_timing_read(double *main_ms, double *combine_ms, int *calls);

#ifdef __cplusplus
}
#endif

#endif /* BBSA_H */
