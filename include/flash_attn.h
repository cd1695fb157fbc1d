/*
 * flash_attn.h -- C ABI of the MI355X (gfx950) tiled attention forward pass.
 *
 * The operation. For every (batch b, head h) and query row i:
 *
 *     O[b,h,i,:] = sum_j P[i,j] V[b,h,j,:],   P[i,:] = softmax_j( scale * Q[b,h,i,:].K[b,h,j,:] )
 *     LSE[b,h,i] = log sum_j exp( scale * Q[b,h,i,:].K[b,h,j,:] )      (natural log)
 *
 * with the sums over the keys j the mask keeps. This is ordinary scaled
 * dot-product attention ("Flash Attention" overview page, "The Problem with
 * Standard Attention"), computed the way the pages' tiled methods do: a query
 * row-block streams over key/value blocks, carrying a running max, a running
 * sum and an output accumulator under the online-softmax rescale (Lab 3 page
 * "Tiled attention with online softmax"; Lesson 91 deck, slide 11 "Online
 * softmax: tiled update equations"), and writes O and the logsumexp once,
 * never forming the S x S score matrix ("Flash Attention" page, "IO-Aware
 * Algorithm": write the output once at the end).
 *
 * Mask (keep(i, j)):
 *   causal == 0 : every key (window must be 0);
 *   causal == 1 : j <= i (diagonal kept: the Lab 3 page's lower-triangular
 *                 mask), and if window > 0 also  (i - j < window  OR  j < n_sink).
 *   window = width counted in keys including the query itself; window == 0
 *   means no window; n_sink = number of leading key positions that every
 *   query may see (the Lab 3 page's exercise on "sink" tokens plus a sliding
 *   window); n_sink is ignored when window == 0.
 *
 * Callers include no HIP header; every pointer is a plain address.
 */
#ifndef IO_AWARE_TILED_FLASH_AMD_FLASH_ATTN_H
#define IO_AWARE_TILED_FLASH_AMD_FLASH_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. lse is always fp32. */
enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 };

/* Return codes. */
enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,     /* an argument breaks a precondition; nothing was launched or written */
  FA_ERR_UNSUPPORTED = -2, /* valid request this build does not implement (head dim, sizes) */
  FA_ERR_HIP = -3          /* the HIP runtime reported an error while launching */
};

/*
 * flash_attn_fwd -- enqueue the attention forward pass on `stream`.
 *
 * q, k, v : device pointers, [B, H, S, D] dense row-major (D fastest), element
 *           type `dtype`, 16-byte aligned. Read only; they may alias each other.
 * o       : device pointer, [B, H, S, D], `dtype`, 16-byte aligned. Must not
 *           overlap q, k or v. Every element is written.
 * lse     : device pointer, [B, H, S] fp32, 4-byte aligned. Must not overlap
 *           q, k, v or o. Every element is written: the natural-log
 *           logsumexp of the scaled, masked score row.
 * B, H, S : >= 1.   D : head dimension, one of 16, 32, 64, 128.
 * causal  : 0 or 1.  window >= 0 (window > 0 needs causal == 1).  n_sink >= 0.
 * scale   : finite fp32 multiplier of Q.K (used as given: 0 and negative values
 *           are valid; there is no "default" substitution).
 * stream  : a hipStream_t, or NULL for the default stream.
 * dtype   : FA_F32, FA_F16 or FA_BF16.
 *
 * Precision: products of the stored inputs, fp32 accumulation; for f16/bf16 the
 * softmax weights are rounded to the input type (nearest-even) before the
 * second contraction; O is rounded to `dtype` once, at the end.
 *
 * Ownership and timing: the caller owns every buffer. The call validates its
 * arguments on the host, enqueues one kernel and returns without waiting;
 * o and lse are valid once `stream` has been synchronised. The library
 * allocates no device memory and keeps no per-call state; concurrent calls
 * from several threads are safe.
 *
 * Errors: FA_ERR_INVALID (NULL pointer, B/H/S < 1, causal not 0/1, window < 0,
 * window > 0 with causal == 0, n_sink < 0, non-finite scale, unknown dtype,
 * misaligned pointer, o overlapping q/k/v, lse overlapping q/k/v/o, byte sizes
 * overflowing int64),
 * FA_ERR_UNSUPPORTED (D not in {16,32,64,128}; S, B*H or the grid beyond the
 * 32-bit index range), FA_ERR_HIP (launch failure). On any error nothing is
 * enqueued and flash_attn_last_error() describes it.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t S, int64_t D,
                   int causal, int64_t window, int64_t n_sink, float scale,
                   void* stream, int dtype);

/*
 * flash_attn_fwd_ext -- flash_attn_fwd with grouped key/value heads and an
 * optional ALiBi bias.
 *
 * Grouped heads ("Lesson 91" deck, slide 32 "MQA: one shared K, V for all
 * query heads", and its note on grouped-query attention): q and o hold H
 * query heads, k and v hold H_kv key/value heads, and query head h reads
 * key/value head h / (H / H_kv) -- consecutive query heads form the groups.
 * H_kv = 1 is multi-query attention, H_kv = H ordinary attention.
 *
 * ALiBi (same deck, slides 20-25 and 28): if alibi_slopes is non-NULL, the
 * logit of (i, j) in query head h is scale * Q_i.K_j - alibi_slopes[h] * |i - j|,
 * the bias added before the softmax (and so inside the logsumexp). The deck's
 * slopes are 2^(-8 h'/H) for h' = h + 1; any finite slopes are accepted.
 *
 * q, o    : device pointers, [B, H, S, D], `dtype`, 16-byte aligned.
 * k, v    : device pointers, [B, H_kv, S, D], `dtype`, 16-byte aligned.
 * lse     : device pointer, [B, H, S] fp32, 4-byte aligned.
 * H_kv    : >= 1 and a divisor of H.
 * alibi_slopes : device pointer to H fp32 slopes (4-byte aligned), or NULL for
 *           no bias. Read only; must not overlap o or lse.
 * Everything else, the precision, ownership, timing and errors are those of
 * flash_attn_fwd, plus FA_ERR_INVALID for H_kv < 1, H_kv not dividing H, a
 * misaligned or overlapping alibi_slopes.
 */
int flash_attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D,
                       int causal, int64_t window, int64_t n_sink, float scale,
                       const float* alibi_slopes, void* stream, int dtype);

/*
 * flash_attn_fwd_split -- flash_attn_fwd_ext with the keys of every query
 * block split into n_split ranges computed by separate work-groups, then
 * merged. More work-groups in flight for short sequences or few heads.
 *
 * Each range yields a partial result (O_s normalised within the range, LSE_s;
 * (0, -inf) for a row that sees no key of the range), and the partials merge
 * into O and LSE by LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s
 * (the online-softmax rescale of the Lesson 91 deck, slide 11, applied once
 * per range; the NumPy tiled-block guide ends on reducing partial outputs
 * across workers). The result equals flash_attn_fwd_ext's up to rounding
 * order; O is rounded to `dtype` once, after the merge.
 *
 * n_split   : 1..256. 1 computes exactly flash_attn_fwd_ext (no workspace
 *             needed). n_split > 1 needs dtype FA_BF16 / FA_F16 and D 64 or
 *             128 (else FA_ERR_UNSUPPORTED).
 * workspace : device memory the caller owns, >= flash_attn_split_workspace_bytes(
 *             B, H, S, D, n_split) bytes, 16-byte aligned, overlapping no
 *             tensor. Scratch only: its contents on entry do not matter and
 *             are undefined afterwards. Calls that share a workspace must not
 *             overlap in time.
 * Everything else as flash_attn_fwd_ext, plus FA_ERR_INVALID for n_split out
 * of range or a missing / small / misaligned / overlapping workspace. Two
 * kernels are enqueued on `stream` (partials, then the merge).
 */
int flash_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D,
                         int causal, int64_t window, int64_t n_sink, float scale,
                         const float* alibi_slopes, int64_t n_split, void* workspace,
                         int64_t workspace_bytes, void* stream, int dtype);

/*
 * flash_attn_split_workspace_bytes -- host-only: the workspace bytes
 * flash_attn_fwd_split needs for this shape (0 for n_split == 1), or -1 with
 * flash_attn_last_error() set for invalid sizes.
 */
int64_t flash_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D,
                                         int64_t n_split);

/*
 * flash_attn_merge -- merge n_parts partial attention results row by row, as
 * flash_attn_fwd_split does internally (and as a sequence-sharded pass would
 * after computing partials on key shards).
 *
 * o_parts   : device, fp32 [n_parts, rows, D], 16-byte aligned (each partial
 *             normalised within its key range).
 * lse_parts : device, fp32 [n_parts, rows], 4-byte aligned (-inf: the part
 *             saw no key for that row and weighs zero).
 * o         : device, [rows, D] in `dtype`, 16-byte aligned; lse: device fp32
 *             [rows], 4-byte aligned. A row with no finite partial becomes
 *             (0, -inf). Outputs must not overlap the inputs or each other.
 * n_parts in [1, 4096], rows >= 1, D in {16, 32, 64, 128} (else
 * FA_ERR_UNSUPPORTED). Asynchronous on `stream`, like flash_attn_fwd.
 */
int flash_attn_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, int64_t rows,
                     int64_t D, void* o, float* lse, void* stream, int dtype);

/*
 * flash_attn_bwd -- gradients of the forward pass, by recomputation from its
 * logsumexp (the Lesson 91 deck: the tile loop keeps only m, l and O; the
 * backward recomputes the score tiles rather than storing them). With P the
 * softmax weights of the forward call and dP = dout V^T:
 *     dv = P^T dout,   dS = P * (dP - rowsum(dout * o)),
 *     dq = scale dS K,   dk = scale dS^T Q,
 * where a key/value head's dk, dv sum over the query heads that read it.
 *
 * q, o, dout, dq : device, [B, H, S, D], `dtype`, 16-byte aligned.
 * k, v, dk, dv   : device, [B, H_kv, S, D], `dtype`, 16-byte aligned.
 * lse            : device fp32 [B, H, S]: the lse flash_attn_fwd(_ext) wrote
 *                  for the same inputs and arguments (o likewise).
 * B, H, H_kv, S, D, causal, window, n_sink, scale, alibi_slopes, stream,
 *                  dtype: as in flash_attn_fwd_ext, with dtype FA_BF16 /
 *                  FA_F16 and D 64 or 128 (else FA_ERR_UNSUPPORTED).
 * workspace      : device scratch of >= flash_attn_bwd_workspace_bytes(B, H, S)
 *                  bytes (two per-row fp32 arrays: rowsum(dout * o) and
 *                  lse * log2(e), S padded to a multiple of 128 rows per head),
 *                  16-byte aligned; contents on entry do not matter. Calls
 *                  sharing it must not overlap.
 * Precision: fp32 accumulation; P and dS rounded to `dtype` before their
 * products (like P in the forward); outputs rounded once.
 * Outputs must not overlap any input, each other or the workspace. Two
 * kernels are enqueued on `stream`; errors as flash_attn_fwd.
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t H_kv, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
                   float scale, const float* alibi_slopes, void* workspace,
                   int64_t workspace_bytes, void* stream, int dtype);

/*
 * flash_attn_bwd_noalloc -- flash_attn_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * The two per-row arrays flash_attn_bwd keeps in its workspace live instead in
 * a static device array of the library, 32 MiB per GPU, held from the
 * library's first use on that GPU until the process ends. The call allocates
 * nothing and calls no allocating routine. Its limit: the workspace
 * flash_attn_bwd would need, flash_attn_bwd_workspace_bytes(B, H, S), must be
 * at most 32 MiB (8 bytes per row of B*H*S, S rounded up to a multiple of 128:
 * about 4.19 million rows); larger shapes return FA_ERR_UNSUPPORTED.
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (from several streams or threads) race and must not be issued.
 * Calls in sequence on a stream are safe; nothing of an earlier call's
 * contents is read.
 *
 * Arguments, results, precision and the other errors are those of
 * flash_attn_bwd; FA_ERR_HIP also reports a failure to look up the array.
 */
int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal,
                           int64_t window, int64_t n_sink, float scale,
                           const float* alibi_slopes, void* stream, int dtype);

/* flash_attn_bwd_workspace_bytes -- host-only: bytes of flash_attn_bwd's
 * workspace for this shape, or -1 (flash_attn_last_error set) if invalid. */
int64_t flash_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S);

/*
 * flash_attn_fwd_counted -- flash_attn_fwd plus an instrumentation counter.
 *
 * block_pairs : device pointer to one uint64 (8-byte aligned), or NULL. When
 *               non-NULL, each work-group atomically adds the number of key/value
 *               blocks it computed, so after the call the counter has grown by
 *               the number of (query-block, key-block) tile pairs processed. Blocks
 *               the mask hides completely are skipped and not counted (the causal
 *               saving the Lab 3 page's block-pair exercise asks about).
 * Same arguments, results, errors and timing as flash_attn_fwd otherwise.
 */
int flash_attn_fwd_counted(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t S, int64_t D,
                           int causal, int64_t window, int64_t n_sink, float scale,
                           void* stream, int dtype, uint64_t* block_pairs);

/*
 * flash_attn_tile_shape -- host-only query of the tile flash_attn_fwd uses for
 * a problem of this shape: *block_q query rows per work-group and *block_k keys
 * per streamed key/value block (the kernel and its work-group size are chosen
 * from B*H, S, D, dtype and the window: window is the call's sliding window,
 * 0 for none). With ALiBi slopes or a key split the bf16/f16
 * D=64/128 kernel never takes the small-grid schedule, whose 64-row blocks
 * (four key parts at D = 64) this query may report. Returns FA_OK,
 * FA_ERR_INVALID (NULL output, B/H/S < 1, window < 0, unknown dtype) or
 * FA_ERR_UNSUPPORTED (D not implemented). Touches no GPU. Tuning aids, read
 * per call when set: FLASH_ATTN_WAVES=4|8 fixes the work-group size of the
 * bf16/f16 D=64/128 kernel, FLASH_ATTN_PARTS=0|2|4 the key parts of its
 * small-grid schedule (0 = off).
 */
int flash_attn_tile_shape(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int64_t window,
                          int* block_q, int* block_k);

/*
 * flash_attn_fwd_kernel -- host-only query of the kernel a forward call would
 * launch for this problem: writes a NUL-terminated description (kernel
 * template, dtype, head dim, work-group shape, tile) into the caller's host
 * buffer buf of buf_bytes bytes, truncated to fit (128 bytes always suffice).
 * alibi: nonzero when slopes are passed (flash_attn_fwd_ext); n_split: 1, or
 * the key split of flash_attn_fwd_split; window: the call's sliding window, 0
 * for none. Returns FA_OK, FA_ERR_INVALID (NULL or empty buffer, B/H/S < 1,
 * window < 0, unknown dtype, n_split outside [1, 256]; buf
 * then holds "") or FA_ERR_UNSUPPORTED (head dim, or a split the fast kernel
 * cannot take). Touches no GPU; honours FLASH_ATTN_WAVES and
 * FLASH_ATTN_PARTS like the calls.
 */
int flash_attn_fwd_kernel(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int alibi,
                          int64_t n_split, int64_t window, char* buf, int64_t buf_bytes);

/*
 * flash_attn_bwd_kernel -- host-only query of the two kernels flash_attn_bwd
 * (and flash_attn_bwd_noalloc) would launch: the dQ kernel, then one of two
 * dK/dV kernels, chosen from the grid, the causal mask and the window; alibi
 * (nonzero when slopes are passed) selects the ALiBi instances of both.
 * Writes a NUL-terminated description into buf (buf_bytes bytes, truncated
 * to fit; 256 bytes always suffice). Returns FA_OK, FA_ERR_INVALID (NULL or
 * empty buffer, B/H/S < 1, H_kv not dividing H, unknown dtype, window < 0;
 * buf then holds "") or FA_ERR_UNSUPPORTED (not bf16 / f16 with D 64 or
 * 128). Touches no GPU; honours FLASH_ATTN_DKV=1|2 like the call.
 */
int flash_attn_bwd_kernel(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int dtype,
                          int causal, int64_t window, int alibi, char* buf, int64_t buf_bytes);

/*
 * flash_attn_last_error -- text of the last error raised on the calling
 * thread (empty string if none). The pointer stays valid until the thread's
 * next call into this library.
 */
const char* flash_attn_last_error(void);

/* flash_attn_version -- static version string of the library. */
const char* flash_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_TILED_FLASH_AMD_FLASH_ATTN_H */
