/*
 * bbsa.h -- C ABI of the BigBird block-sparse attention forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The pages this library implements are cited by title and section:
 *   [BB] "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践"
 *   [BP] "BigBirdPegasus 长序列条件生成模型详解从稀疏注意力原理到 Transformers 实战"
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
 * caller memory.  The library owns split-K workspaces (see bbsa_forward).
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

/* Options of bbsa_forward_ex (bit flags). */
enum {
  BBSA_FLAG_PAD_TO_BLOCK = 1,   /* L need not be a multiple of the block */
  BBSA_FLAG_QUERY_KEY_MASK = 2, /* bias -10000 (1 - mask[query] mask[key]) */
  BBSA_FLAG_KEEP_PADDED_BLOCKS = 4 /* also compute key blocks whose keys are all padded */
};

/* Status codes. */
enum {
  BBSA_OK = 0,               /* success */
  BBSA_OK_FULL_FALLBACK = 1, /* success; L <= (5+2r)*block, computed as full attention */
  BBSA_ERR_ARG = -1,         /* null or misaligned pointer, or B/H/L/d/block <= 0, or r < 1 */
  BBSA_ERR_SHAPE = -2,       /* L % block != 0, or nb < 5 + r where a plan is required */
  BBSA_ERR_UNSUPPORTED = -3, /* d != 64, block not in {64, 128}, unknown dtype, too large */
  BBSA_ERR_HIP = -4,         /* a HIP call or kernel launch failed */
  BBSA_ERR_PLAN = -5,        /* rand_attn violates an invariant (bbsa_check_rand_attn) */
  BBSA_ERR_CAPTURE = -6,     /* the workspace would have to grow during stream capture */
  BBSA_ERR_SCRATCH = -7      /* bbsa_forward_noalloc: more split-K scratch than its fixed maximum */
};

/*
 * Build the random-block adjacency on the host.
 *
 * Implements [BB] section "随机块掩码是如何生成的": every middle query block
 * (all blocks but the first and the last) gets r random key blocks drawn from
 * the middle blocks with its own 3-block window removed, fixed per head when
 * the layer is built and seeded by the layer index; [BP] section
 * "三类注意力组合全局 局部 随机" (num_random_blocks per query block).  The
 * pages draw with numpy's permutation; this planner draws from a specified
 * stream so that every implementation can reproduce the plan bit for bit.
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
 * Check a host plan [H][nb-2][r] against the invariants [BB] section
 * "随机块掩码是如何生成的" fixes: every entry a middle block (1..nb-2), the r
 * entries of a row distinct, none within distance 1 of the row's block (the
 * random blocks never overlap the window).
 *
 * rand_attn: host buffer, read only.  Returns BBSA_OK, BBSA_ERR_PLAN on a
 * violation, BBSA_ERR_ARG for a null buffer or H, nb, r < 1, BBSA_ERR_SHAPE
 * when nb < 5 + r.
 */
int bbsa_check_rand_attn(const int32_t *rand_attn, int H, int nb, int r);

/*
 * The plan with the random range capped, and its checker.
 *
 * Implements the limit [BB] section "随机块掩码是如何生成的" describes: the
 * layer draws its random blocks only from the first last_idx = 1024 tokens,
 * builds the plan once for its maximum length and uses its first
 * from_seq_length / block - 2 rows for a shorter sequence.  With
 * last_idx > 0, the candidates of every row are the blocks of
 * bbsa_plan_rand_attn's list that lie wholly inside the first last_idx tokens
 * (block c with (c + 1) * block <= last_idx); the stream, the shuffle and the
 * layout are those of bbsa_plan_rand_attn, so a cap at or beyond block nb - 2
 * gives exactly the uncapped plan.  last_idx <= 0 means no cap.
 *
 * rand_attn: host buffer [H][nb-2][r], caller-owned (written by the planner,
 * read by the checker).  Returns BBSA_OK; BBSA_ERR_ARG for a null buffer,
 * H, nb or r < 1, or last_idx > 0 with block < 1; BBSA_ERR_SHAPE when
 * nb < 5 + r or the cap leaves some row fewer than r candidates;
 * BBSA_ERR_PLAN (checker) when an entry breaks an invariant or the cap.
 */
int bbsa_plan_rand_attn_capped(int32_t *rand_attn, int H, int nb, int r, uint64_t seed,
                               int block, int last_idx);
int bbsa_check_rand_attn_capped(const int32_t *rand_attn, int H, int nb, int r, int block,
                                int last_idx);

/*
 * Keep the first nb-2 rows of a plan built for nb_src >= nb blocks (the
 * shorter-sequence use [BB] section "随机块掩码是如何生成的" describes).
 * src: host [H][nb_src-2][r]; dst: host [H][nb-2][r], caller-owned.  Returns
 * BBSA_OK when dst is a valid plan for nb blocks, BBSA_ERR_PLAN when a kept
 * pick is not a middle block of the shorter sequence (or breaks another
 * invariant), BBSA_ERR_ARG for null buffers, H or r < 1, nb < 3 or
 * nb_src < nb.
 */
int bbsa_truncate_rand_attn(const int32_t *src, int H, int nb_src, int r, int32_t *dst, int nb);

/*
 * Block-sparse attention forward on `stream`.
 *
 * Implements [BB] section "BigBird：从二次方注意力到线性稀疏注意力": Q, K, V
 * are cut into blocks of `block` tokens; query blocks 0 and nb-1 attend every
 * key block; every middle query block i attends key blocks 0 and nb-1, the
 * window {i-1, i, i+1} and the r blocks rand_attn[h][i-1]; padded keys get an
 * additive -10000 before the row softmax; out = softmax(scores) V per row.
 * [BP] sections "三类注意力组合全局 局部 随机" (the same three parts, rows 1
 * and nb-2 included), "序列长度的块对齐要求" (L must be a multiple of the
 * block: BBSA_ERR_SHAPE), "序列过短时的自动回退" (full attention when
 * L <= (5 + 2r) * block) and "使用限制与注意事项" (r >= 1).
 *
 * q, k, v:   device, [B, H, L, d] of `dtype`, 16-byte aligned (as are out
 *            and mask; rand_attn 4-byte aligned), else BBSA_ERR_ARG.
 * mask:      device float32 [B, L], 1 = valid key, 0 = padding (fractional
 *            values act through the bias -10000 * (1 - mask)); NULL = all
 *            keys valid.  On the bf16 path with a mask (L a multiple of the
 *            block), a 64-row query tile whose key list holds a key of mask 1
 *            leaves out the listed key blocks whose mask values are all 0
 *            (except the first block of its list): their probabilities are
 *            exactly zero in fp32, so the output and the log-sum-exp are
 *            those of computing them, as long as no padded key's score
 *            exceeds a valid key's score of the same tile by about 9890 (the
 *            -10000 bias would not mask it either).  bbsa_forward_ex's
 *            BBSA_FLAG_KEEP_PADDED_BLOCKS computes every block.
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
 * blocks); L <= 2^24; B * H * L * d <= 2^40 elements; at most 2^31 - 1
 * workgroups; (key chunks per full row) * nb < 2^31, which binds only the
 * fp32 path (256-key chunks: about L <= 5.9 million tokens with block 64).
 *
 * Returns BBSA_OK, or BBSA_OK_FULL_FALLBACK when L <= (5 + 2r) * block (every
 * query block then attends every key block), or a negative error code.  All
 * argument checks happen before any HIP call.
 *
 * Workspace: rows that leave more than one split-K partial (bf16 rows of
 * more than four key chunks of 1024 to 4096 keys, so only some rows longer
 * than 4096 keys; fp32 rows longer than 256 keys, and in fp32 calls with
 * fewer than 2048 wavefronts of work full rows longer than 128 keys and
 * every middle row) use a library-owned workspace, one per (device, stream).
 * Calls on one stream are ordered by the stream; calls on different streams
 * use different workspaces and may overlap.  A workspace is allocated or
 * grown (powers of two, at least 1 MiB) with hipMalloc on the first call
 * that needs more; the outgrown buffer stays allocated until
 * bbsa_release_workspace.  Growth while `stream` is being captured into a
 * graph returns BBSA_ERR_CAPTURE: make one eager call of the shape first.
 *
 * Graph capture: a call enqueues kernel launches only (no memset, no copy,
 * no host synchronisation), so once its workspace is large enough it can be
 * recorded into a HIP graph; replays use the captured buffers, which stay
 * valid until bbsa_release_workspace (that call invalidates such graphs).
 * Kernel timing must be off during capture.
 */
int bbsa_forward(const void *q, const void *k, const void *v, const float *mask,
                 const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                 void *out, hipStream_t stream, bbsa_dtype dtype);

/*
 * bbsa_forward with options, and the row log-sum-exp.
 *
 * flags (bit OR of):
 *   BBSA_FLAG_PAD_TO_BLOCK: L need not be a multiple of `block`.  [BP]
 *     section "序列长度的块对齐要求": the encoder pads its input to a
 *     multiple of the block size and cuts the padding off its output.  The
 *     call behaves as if q, k, v were extended with zero rows and the mask
 *     with zeros up to nb = ceil(L / block) blocks, then trimmed: positions
 *     L .. nb*block-1 are never read or written (the kernels treat them as
 *     padded keys with zero K and V), rand_attn is the plan of nb blocks
 *     ([H, nb-2, r]) and the fallback test is L <= (5 + 2r) * block.  The
 *     tensors keep their [B, H, L, d] / [B, L] layout with the real L.
 *   BBSA_FLAG_QUERY_KEY_MASK: the bias of query t and key u is
 *     -10000 * (1 - mask[b, t] * mask[b, u]), the outer product of the query
 *     and key masks that [BB] section "随机块掩码是如何生成的" builds the band
 *     mask from (BigBirdMasks' einsum), instead of the key-side
 *     -10000 * (1 - mask[b, u]).  Rows of valid queries are unchanged; a
 *     padded query row gets the same bias on every key, i.e. a softmax of
 *     its raw scores.  No effect without a mask.  (Padded key blocks are
 *     then left out only by tiles whose query rows all have mask 1.)
 *   BBSA_FLAG_KEEP_PADDED_BLOCKS: compute every key block of the pattern,
 *     also those whose keys all have mask 0 (see `mask` under bbsa_forward).
 * lse: device float32 [B, H, L], 4-byte aligned, caller-owned, or NULL: the
 *     natural log-sum-exp of each query row's scores (bias included) over
 *     the keys it attends, the quantity a recompute-based backward needs.
 *     On the bf16 path the row sums add the bf16-rounded probabilities, so
 *     lse carries a relative error of up to 2^-9 in the sum (about 2e-3 in
 *     lse); on the fp32 path it is exact to fp32 rounding of its terms.
 *
 * Other arguments, limits, workspace use and errors as bbsa_forward; an
 * unknown flag bit is BBSA_ERR_ARG, a length that is not a multiple of the
 * block without BBSA_FLAG_PAD_TO_BLOCK is BBSA_ERR_SHAPE.  With flags 0 and
 * lse NULL the call is exactly bbsa_forward.
 */
int bbsa_forward_ex(const void *q, const void *k, const void *v, const float *mask,
                    const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                    void *out, float *lse, hipStream_t stream, bbsa_dtype dtype, unsigned flags);

/*
 * The attention probabilities as a dense matrix (output_attentions).
 *
 * [BP] section "三类注意力组合全局 局部 随机": the block-sparse weights are
 * scattered back into a full (batch, heads, L, L) attention matrix for
 * callers that ask for the attention outputs; section "使用限制与注意事项":
 * most of that matrix is zero and carries no gradient.  probs[b, h, t, u] is
 * the softmax weight of key u in query row t (the scores, padding bias,
 * options and pattern of bbsa_forward_ex with the same arguments and flags),
 * exactly 0 for every key block outside the row's pattern.  Computed in fp32
 * from q and k alone (each row's max and sum are formed in fp32 over the
 * attended keys, relative to the row's largest padding bias, so rows whose
 * keys all share one mask value keep fp32 precision); v is not needed.
 *
 * probs: device float32 [B, H, L, L], 4-byte aligned, caller-owned, fully
 * overwritten (B * H * L * L * 4 bytes: an inspection path for moderate L).
 * Other arguments, validation and status codes as bbsa_forward_ex.
 */
int bbsa_attention_probs(const void *q, const void *k, const float *mask, const int32_t *rand_attn,
                         int B, int H, int L, int d, int block, int r, float *probs,
                         hipStream_t stream, bbsa_dtype dtype, unsigned flags);

/*
 * Backward pass: the gradients of bbsa_forward_ex's output with respect to
 * q, k and v.
 *
 * [BB] section "梯度检查点的实现方式": the encoder is trained through this
 * operator and may recompute its forward instead of storing activations;
 * [BP] section "使用限制与注意事项": the sparse attention matrix carries no
 * gradient of its own.  With P the pattern's row softmax (bias included),
 * out = P V and dout the gradient of out:
 *   dv = P^T dout,  ds = P * (dout v^T - rowsum(dout * out)),
 *   dq = ds k,  dk = ds^T q.
 * P is recomputed from q, k and the forward's row log-sum-exp, so the
 * forward must have been run with the same arguments and flags and its
 * `out` and `lse` passed here.
 *
 * q, k, v, out, dout: device [B, H, L, d] of `dtype`, 16-byte aligned.
 * lse:   device float32 [B, H, L] from bbsa_forward_ex.
 * dq, dk, dv: device [B, H, L, d] of `dtype`, caller-owned, fully
 *        overwritten.
 * delta: device float32 [B, H, L], caller-owned, overwritten with
 *        rowsum(dout * out).
 * mask, rand_attn, shapes, flags: as for bbsa_forward_ex.
 *
 * BBSA_BF16: MFMA kernels; three kernels on `stream` (two when nb = 1),
 * using the library's workspace for `stream` (B * H * L floats of row
 * terms, B * H * nb * block / 32 ints of query-tile flags, plus fp32
 * partials of the split global rows and columns:
 * 3 * B * H * 2 * block * 64 * c floats with nb = ceil(L / block) and
 * c = max(min(nb, 2), ceil(nb / 64)) chunks per row, or nb in place of 2 on
 * the full-attention fallback).
 * With a mask (bf16), steps whose keys all have mask 0 are left out for the
 * query rows whose lse exceeds -5000 (and whose mask is 1 under query x key
 * masking): their probabilities are exactly zero in fp32 for scores below
 * about 4900, so the gradients equal those of computing them;
 * BBSA_FLAG_KEEP_PADDED_BLOCKS computes every step.
 * BBSA_F32: an fp32 path on the vector units (three kernels; workspace
 * 2 * B * H * L floats), which recomputes each row's normaliser relative to
 * its padding-bias level as the fp32 forward does, so rows whose keys all
 * share one mask value keep fp32 precision; `lse` is checked but not read.
 * Errors as bbsa_forward_ex.  The workspace grows as bbsa_forward's does,
 * and BBSA_ERR_CAPTURE is returned if it would have to grow while `stream`
 * is being captured.
 */
int bbsa_backward(const void *q, const void *k, const void *v, const void *out, const void *dout,
                  const float *lse, const float *mask, const int32_t *rand_attn, int B, int H, int L,
                  int d, int block, int r, void *dq, void *dk, void *dv, float *delta,
                  hipStream_t stream, bbsa_dtype dtype, unsigned flags);

/*
 * bbsa_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, computation, results and errors as bbsa_forward; the
 * split-K partials (the only device memory beyond inputs and outputs) go to a
 * fixed 16 MiB array that the library holds on each device it runs on until
 * the process ends, so the call itself allocates nothing.  That fits 1007
 * partials of 16.3 KiB: every bf16 call with L <= 4096 (none needed), and
 * in general B * H * 2 * (block / 64) * ceil(L / (4 c)) <= 1007, where c is
 * the full-row chunk length: 1024, 2048 or 4096 keys, longer for launches
 * with more work (4096 at B 8, H 16, L 32768).  A call
 * needing more returns BBSA_ERR_SCRATCH before any HIP call.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or different host threads) race and must be ordered by the
 * caller; each call writes every partial it reads, so nothing needs clearing
 * between calls.
 */
int bbsa_forward_noalloc(const void *q, const void *k, const void *v, const float *mask,
                         const int32_t *rand_attn, int B, int H, int L, int d, int block, int r,
                         void *out, hipStream_t stream, bbsa_dtype dtype);

/* Static string describing a status code. */
const char *bbsa_status_string(int status);

/*
 * Free every library-owned workspace (current and outgrown) on every device,
 * after synchronising each device that has one.  Graphs captured with calls
 * that used a workspace must not be replayed afterwards.
 */
void bbsa_release_workspace(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int bbsa_version(void);

/*
 * Kernel timing for benchmarks.  When enabled, bbsa_forward records a pair of
 * HIP events on `stream` around its main attention kernel and around its
 * split-K combine kernel when one runs (combine_ms counts 0 otherwise).
 * bbsa_timing_read synchronises on the recorded events, returns the summed
 * durations in milliseconds and the number of timed calls, then clears the
 * record.  At most 4096 calls are recorded between reads; later calls are
 * not timed.  The record is guarded by a lock: calls from several threads
 * are counted correctly (they are serialised while timing is on).
 */
int bbsa_timing_enable(int enable);
int bbsa_timing_read(double *main_ms, double *combine_ms, int *calls);

/*
 * Work decomposition of a forward call (a query for tests and tools; no HIP
 * call).  For the shape, dtype and flags of a bbsa_forward_ex call (flags 0:
 * a bbsa_forward call) with host plan
 * `rand_attn` (may be NULL on the fallback), runs on the host the same item
 * mapping and key-list construction the kernels run (the lists as built,
 * before a masked bf16 call leaves out its fully padded key blocks, which
 * depends on the mask's values), and writes one record
 * of BBSA_WORK_RECORD_INTS int32 per work item (a 64-row query tile against
 * a key list) of the attention kernel:
 *   [0] workgroup  [1] wavefront  [2] 0 (reserved)
 *   [3] batch*H+head  [4] query block  [5] query tile  [6] full-row index
 *   (-1 for a middle row)  [7] key chunk (full row) or key part (middle row)
 *   [8], [9] first and one-past-last key-list position the unit walks
 *   [10] 32-key steps per block  [11] chunks per full row  [12] partials per
 *   full row left for the merge kernel  [13] key parts per middle row
 *   [14], [15] unused (-1)  [16 + t] key block at list position t for
 *   t in [rec[8], rec[9]), else -1.
 * records: host buffer of capacity * BBSA_WORK_RECORD_INTS int32, or NULL to
 * count only; at most `capacity` records are written.  *count receives the
 * number of items, *grid the attention kernel's workgroup count.  Returns
 * what bbsa_forward would return for the shape (pointer arguments aside).
 */
#define BBSA_WORK_RECORD_INTS 80
int bbsa_work_map(int B, int H, int L, int d, int block, int r, bbsa_dtype dtype, unsigned flags,
                  const int32_t *rand_attn, int32_t *records, int64_t capacity,
                  int64_t *count, int64_t *grid);

#ifdef __cplusplus
}
#endif

#endif /* BBSA_H */
