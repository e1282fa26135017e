/*
 * dspk.h -- C ABI of the MI355X (gfx950) verify pass of lossless speculative
 * decoding.
 *
 * A verify round ("mlx-dspark" wiki summary, section "Architecture", first
 * bullet): the target model evaluates the anchor token and the m drafted
 * tokens together in one pass; each draft is then checked against the token
 * distribution the target itself produced at that position, and the drafts up
 * to the first failed check are kept.  With greedy checks the output is what
 * plain one-token decoding would give; with temperature > 0 the
 * Leviathan/Chen min(1, p/q) test keeps the output an exact sample of the
 * target.
 *
 * The library computes the data-parallel part of that round:
 *   dspk_qgemm_verify   - every projection of the target over the M = m + 1
 *                         rows, through affine group-quantised weights;
 *   dspk_qgemm_prefill  - the same projection for many rows (a prompt);
 *   dspk_lmhead_argmax  - the vocabulary projection fused with the row argmax;
 *   dspk_accept_greedy  - longest matching prefix plus the target's token;
 *   dspk_lmhead_argmax_accept_greedy - the two calls above in one launch;
 *   dspk_accept_sample  - min(1, p/q) acceptance with residual resampling.
 *   dspk_accept_sample_ex - the same over penalised, top-k/top-p truncated distributions.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is DEVICE memory (hipMalloc / torch) owned by the
 *   caller, except that the acceptance results (accept_len, committed) may
 *   also be pinned host memory mapped for the device (hipHostMalloc, torch
 *   pin_memory): the kernels only write them, so a round's result can land on
 *   the host with no copy launch.  The library never allocates, frees or
 *   synchronises; every call only enqueues kernels on `stream` (a
 *   hipStream_t, NULL = default stream) and returns.  Results are valid once
 *   the stream reaches that point.
 * - Return value: DSPK_OK (0) on success, a negative DSPK_E* code otherwise;
 *   dspk_last_error() then holds a message (thread-local).  Nothing is
 *   enqueued when a call fails its argument checks.  There is no fallback
 *   path and no clamping of bad arguments.
 * - Faults that depend on data values (non-finite logits, bad uniforms, draft
 *   ids out of range) cannot be seen on the host without a sync; the
 *   acceptance kernels report them on the device (accept_len = -1).
 * - Calls that share a workspace must be ordered on one stream.
 */
#ifndef DSPK_H
#define DSPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPK_OK            0
#define DSPK_EINVAL      (-1) /* null / misaligned pointer, bad size or stride  */
#define DSPK_EUNSUPPORTED (-2) /* valid request outside what the kernels handle */
#define DSPK_EDEVICE     (-3) /* HIP launch error                              */

#define DSPK_F32  0           /* y / logits element type: float32              */
#define DSPK_BF16 1           /* y element type: bfloat16 (round to nearest even) */

#define DSPK_GROUP     64     /* quantisation group width along K              */
#define DSPK_MAX_ROWS  32     /* largest M (anchor + drafts, or B requests x rows) */
#define DSPK_MAX_GROUPED 4    /* most weights in one grouped call              */

/*
 * One weight matrix W[n][k] (out features x in features) in its interchange
 * layout, the input of dspk_qweight_pack.
 *
 * bits 2, 3, 4 or 8 -- affine group quantisation, w[r][c] = s[r][c/64] *
 *   q[r][c] + b[r][c/64], the plain reading of the pages' "quantised" target
 *   weights with per-group parameters ("mlx-dspark" wiki summary, "Key
 *   techniques", custom kernels bullet; the lower-bit rows are the pages'
 *   ternary and 3-bit targets, "mlx-dspark 0.7.0"):
 *     codes  : uint32[n][k*bits/32]: each row one LSB-first bit stream, code
 *              c at stream bits bits*c .. bits*c + bits-1, bit i of the
 *              stream in bit i%32 of word i/32 (so 32/bits codes per word
 *              for 2, 4 and 8 bits; 3-bit codes may straddle two words);
 *              unsigned 0 .. 2^bits-1;
 *     scales : IEEE binary16 [n][k/64], row-major;
 *     biases : IEEE binary16 [n][k/64], row-major.
 * bits 16 -- unquantised bfloat16 control: codes = bf16[n][k], scales and
 *   biases must be NULL.
 * group must be 64; k must be a multiple of 64; codes must be 16-byte
 * aligned; scales/biases 2-byte aligned.  The struct itself is host memory.
 */
typedef struct dspk_qweight {
    int32_t n;
    int32_t k;
    int32_t bits;
    int32_t group;
    const void *codes;
    const uint16_t *scales;
    const uint16_t *biases;
} dspk_qweight;

/*
 * The same weight in the library's tiled layout, which the projection and
 * vocabulary-head calls stream.  `tiles` is device memory of
 * dspk_tiled_bytes(n, k, bits) bytes, 256-byte aligned, written by
 * dspk_qweight_pack.
 *
 * Layout: 64-column blocks in column order, each cut along K into units of
 * KU = 128 (8-bit), 256 (4-bit) or 64 (bf16) elements; unit u of block b
 * starts at byte (b * ceil(k / KU) + u) * UNIT, UNIT = 8192 + 4 * KU bytes
 * for 4/8-bit and 8192 for bf16.  A unit holds its codes as eight 1 KiB slots
 * of 64 x 16 bytes, each 16-byte piece the codes one lane of a wave feeds to
 * the matrix cores, then (4/8-bit) one dword (scale | bias << 16) per column
 * and group.  The exact byte order is documented in the packing source; it
 * is a layout of this library, not an interchange format.  Columns past n
 * and K past k are zero.  About 6% larger than codes alone at 8-bit, like
 * the interchange layout with its scales and biases.
 */
typedef struct dspk_tiled_weight {
    int32_t n;
    int32_t k;
    int32_t bits;
    int32_t group;           /* must be 64 */
    const void *tiles;
} dspk_tiled_weight;

/* Library version: major*10000 + minor*100 + patch. */
int dspk_version(void);

/* Message for the last non-zero return on this thread ("" if none). */
const char *dspk_last_error(void);

/* Bytes of a weight in the tiled layout (0 if the shape or bits are invalid). */
size_t dspk_tiled_bytes(int32_t n, int32_t k, int32_t bits);

/*
 * Convert `w` (interchange layout, device memory) into the tiled layout at
 * `tiles` (device memory, >= dspk_tiled_bytes(w->n, w->k, w->bits) bytes,
 * 256-byte aligned, not overlapping w).  A one-time, load-time step: one
 * kernel on `stream`, a pure permutation of the bytes.  Errors: DSPK_EINVAL
 * (NULL, misaligned, bad shape, tiles too small), DSPK_EUNSUPPORTED (bits,
 * group), DSPK_EDEVICE.
 */
int dspk_qweight_pack(const dspk_qweight *w, void *tiles, size_t tiles_bytes, void *stream);

/*
 * Activation rows (x, h) are row-major bf16 [m][ld]: element (row i, column r)
 * at index i * ld + r, ld >= k and ld % 8 == 0, base 16-byte aligned.  So a
 * projection's bf16 output (y_dtype = DSPK_BF16, ldy % 8 == 0) is directly the
 * next call's input.
 */

/*
 * Workspaces of the projection and head calls (dspk_qgemm_verify,
 * dspk_qgemm_verify_grouped, dspk_lmhead_argmax,
 * dspk_lmhead_argmax_accept_greedy).  They hold arrival counters, the head's
 * row keys and the partial sums of column blocks whose K range is split
 * between workgroups, at offsets that depend only on the device (not on the
 * call's shape, width or format).  Contract:
 *  - zero-fill a workspace once, before its first use;
 *  - every completed call returns the counters and keys to zero (partial sums
 *    are always written before they are read), so ONE workspace of at least
 *    the size each call needs serves any sequence of these calls, of any
 *    shapes, widths and formats;
 *  - calls that share a workspace must be ordered on one stream: overlapping
 *    calls on one workspace race and give wrong results;
 *  - a sampling workspace (dspk_sample_workspace_bytes) is a different kind:
 *    it keeps per-call statistics, so do not pass it to these calls, nor
 *    theirs to the sampling calls, without zero-filling it again.
 * dspk_qgemm_workspace_bytes(n, k, m) is the size for a weight of n columns
 * (about 12.6 MB of partial-sum space on a 256-CU device, plus 16 bytes per
 * 64 columns); it is never 0 for valid arguments, and a buffer of that size
 * serves every width 1..DSPK_MAX_ROWS and format.
 */
size_t dspk_qgemm_workspace_bytes(int32_t n, int32_t k, int32_t m);

/*
 * Verify-pass projection: y[i][c] = sum_r x[i][r] * w[c][r] for the M rows
 * i < m (anchor plus drafts), fp32 accumulation.  Each weight group is read
 * from HBM and dequantised once per call and reused for all M rows -- the
 * pages' point that verifying m extra rows must not re-read the weights per
 * row ("mlx-dspark" wiki summary, "Key techniques", custom kernels bullet;
 * the 1-bit counter-example in "mlx-dspark 0.7.0", "PrismML Bonsai 27B").
 *
 *   w         : tiled weight (see dspk_tiled_weight, dspk_qweight_pack).
 *   x         : bf16 activations, row-major [m][ldx] (see above): ldx >= k,
 *               ldx % 8 == 0, 16-byte aligned, m * ldx * 2 < 2^31.
 *   m         : rows, 1 .. DSPK_MAX_ROWS.
 *   y         : output [m][ldy], element type y_dtype (DSPK_F32 | DSPK_BF16),
 *               ldy >= n; 4-byte aligned.
 *   workspace : >= dspk_qgemm_workspace_bytes(n, k, m) bytes, 256-byte
 *               aligned, zero-filled before first use (see the contract above).
 * Results are deterministic: the same call on the same inputs gives the same
 * bits (the K split is fixed by the shapes, not by scheduling).
 * Errors: DSPK_EINVAL (null or misaligned pointer, n < 1, k % 64, ldx/ldy,
 * m out of 1..32, workspace too small), DSPK_EUNSUPPORTED (bits not in
 * {2, 3, 4, 8, 16}, group != 64, activation rows of 2 GiB or more),
 * DSPK_EDEVICE.
 */
int dspk_qgemm_verify(const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx, int32_t m,
                      void *y, int32_t y_dtype, int64_t ldy,
                      void *workspace, size_t ws_bytes, void *stream);

/*
 * How projection launches are decomposed, process-wide (measurement and
 * tests; results are within the same error bound either way, and each
 * decomposition is deterministic):
 *   DSPK_VARIANT_AUTO    (default) the slab kernel -- one workgroup per
 *                        16-column tile over the whole K range, no
 *                        cross-workgroup traffic -- for 8-bit and bf16 calls
 *                        of at most 16 rows whose tiles are short enough
 *                        (the weights one CU streams stay under a limit that
 *                        depends on the rows), else stream-K;
 *   DSPK_VARIANT_STREAMK persistent workgroups over contiguous K ranges, split
 *                        column blocks completed by the last workgroup to arrive;
 *   DSPK_VARIANT_SLAB    the slab kernel for every projection;
 *   DSPK_VARIANT_DOT     the slab decomposition with the K reduction on the
 *                        vector ALUs (bf16 dot2 instructions) instead of the
 *                        matrix cores -- 8-bit weights and m <= 4 only, other
 *                        calls as DSPK_VARIANT_AUTO.
 * The vocabulary-head calls are always stream-K.  The initial setting comes
 * from the environment variable DSPK_VARIANT (auto | streamk | slab | dot).
 * Returns the previous setting, or DSPK_EINVAL for an unknown value.  Not
 * synchronised with calls in flight on other threads.
 */
#define DSPK_VARIANT_AUTO    0
#define DSPK_VARIANT_STREAMK 1
#define DSPK_VARIANT_SLAB    2
#define DSPK_VARIANT_DOT     3
int dspk_set_projection_variant(int32_t variant);

/*
 * Grouped form for weights that read the same rows (q/k/v, gate/up): one
 * launch for `count` (1 .. DSPK_MAX_GROUPED) weights with equal k and bits.
 * y[g] is the output of w[g] with leading dimension ldy[g].  The workspace is
 * the sum of dspk_qgemm_workspace_bytes over the weights.  The launch splits
 * K over the workgroups differently from separate calls, so its results
 * agree with theirs to fp32 rounding (both within the error bound of the
 * single call), and are themselves deterministic.
 */
int dspk_qgemm_verify_grouped(int32_t count, const dspk_tiled_weight *w,
                              const uint16_t *x, int64_t ldx, int32_t m,
                              void *const *y, int32_t y_dtype, const int64_t *ldy,
                              void *workspace, size_t ws_bytes, void *stream);

/*
 * dspk_qgemm_verify_grouped without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It allocates nothing (no
 * hipMalloc, no allocating library call); its workspace is a file-scope
 * device array of the library, one per GPU, which each GPU holds until the
 * process ends (about 12.7 MB).  Results are those of
 * dspk_qgemm_verify_grouped on the same arguments, bit for bit.
 *  - The array's device address is fetched once per device, on the device
 *    that is current at the first call; the first call on a device also
 *    enqueues one small clearing kernel on `stream` ahead of the projection.
 *    `stream` must belong to the current device.
 *  - Every call on a GPU shares that GPU's array: calls that overlap on one
 *    GPU (different streams, or host threads without ordering) race and give
 *    wrong results.  Calls ordered on one stream are safe; each completed
 *    call leaves the array ready for the next.
 *  - Limit: the call's counters must fit the array -- at most 4096 64-column
 *    blocks (262144 columns over all `count` weights) on a device of up to
 *    256 CUs; larger calls return DSPK_EUNSUPPORTED and enqueue nothing.
 * Other arguments, checks and errors are those of dspk_qgemm_verify_grouped;
 * DSPK_EDEVICE also reports a failed scratch set-up.
 */
int dspk_qgemm_verify_grouped_noalloc(int32_t count, const dspk_tiled_weight *w,
                                      const uint16_t *x, int64_t ldx, int32_t m,
                                      void *const *y, int32_t y_dtype, const int64_t *ldy,
                                      void *stream);

/*
 * Prefill projection: the same y = x . deq(W)^T for many rows at once -- a
 * prompt's tokens, the wide-row form of the pass ("mlx-dspark" wiki summary,
 * "Key techniques": a weight group dequantised once and reused for all rows).
 * Tiled for the matrix cores (128 x 128 or 64 x 128 output blocks); exact
 * like the verify projection (codes contracted exactly, fp32 accumulation,
 * one scale/bias update per group).  For a prompt's last row only, call
 * dspk_lmhead_argmax with m = 1 on that row.
 *
 *   w         : tiled weight (any format).
 *   x         : bf16 activations, ROW-major [m][ldx]: ldx >= k, ldx % 8 == 0,
 *               16-byte aligned.
 *   m         : rows, >= 1.
 *   y         : output [m][ldy], y_dtype (DSPK_F32 | DSPK_BF16), ldy >= n.
 *   workspace : NULL, or >= dspk_prefill_workspace_bytes(n, k, m, bits)
 *               bytes, 256-byte aligned, zero-filled before its first use;
 *               every call leaves its counters zero again, so one buffer
 *               serves any sequence of prefill calls ordered on one stream
 *               (calls that overlap must not share it).  With a workspace,
 *               launches with fewer output blocks than the CUs hold at once
 *               split K over several workgroups; the last of a block's
 *               workgroups adds their partial sums in a fixed order.
 * Deterministic for a given call shape and workspace choice (a K split
 * changes the summation order, so results with and without a workspace
 * may differ by rounding).  Errors: DSPK_EINVAL (pointers, alignment,
 * ldx/ldy, m < 1, a workspace that is too small), DSPK_EUNSUPPORTED (bits,
 * group), DSPK_EDEVICE.
 */
int dspk_qgemm_prefill(const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx, int32_t m,
                       void *y, int32_t y_dtype, int64_t ldy, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Workspace for dspk_qgemm_prefill over an n x k weight of `bits` and m
 * rows: 0 when no launch of that shape splits K (a NULL workspace then
 * serves), else the bytes the split needs.  It depends on the device's CU
 * count and on dspk_set_prefill_block_rows. */
size_t dspk_prefill_workspace_bytes(int32_t n, int32_t k, int32_t m, int32_t bits);

/*
 * Row block of dspk_qgemm_prefill: 0 (initial) chooses per call between
 * 128-row and 64-row output blocks from the rows, the columns and the
 * device's CU count (64 where 128-row blocks would leave CUs idle or unevenly
 * loaded); 64 or 128 forces one.  Both blocks produce bit-identical results;
 * this setting is for measurement and tests.  Returns the previous setting,
 * or DSPK_EINVAL for another value.  Not synchronised with calls in flight
 * on other threads.
 */
int dspk_set_prefill_block_rows(int32_t rows);

/* Workspace for dspk_lmhead_argmax (and the fused greedy head) over a
 * vocabulary of v entries: any hidden size, width 1..DSPK_MAX_ROWS and
 * format; the same contract as dspk_qgemm_workspace_bytes, and one buffer may
 * serve both kinds of call. */
size_t dspk_lmhead_workspace_bytes(int32_t v, int32_t m);

/*
 * Target logits and greedy tokens: z[i][c] = sum_r h[i][r] * w_lm[c][r] over
 * the vocabulary c < v = w->n, and argmax[i] = the smallest c with z[i][c]
 * equal to the row maximum (a NaN counts as the maximum).  These are the
 * target's own tokens that the drafts are compared with ("mlx-dspark" wiki
 * summary, "Architecture").  The tie rule is the reading taken where the
 * project page leaves ties to floating-point rounding.
 *
 *   w         : vocabulary head, tiled like dspk_qgemm_verify's weights.
 *   h         : bf16 final hidden rows, row-major [m][ldh], ldh >= k,
 *               ldh % 8 == 0, 16-byte aligned.
 *   argmax    : int32 [m] output.
 *   logits    : float32 [m][ldl] output, or NULL to skip writing logits.
 *   workspace : >= dspk_lmhead_workspace_bytes(v, m), 256-byte aligned,
 *               zero-filled before first use (contract above).
 * The result is deterministic (independent of workgroup order).
 */
int dspk_lmhead_argmax(const dspk_tiled_weight *w, const uint16_t *h, int64_t ldh, int32_t m,
                       int32_t *argmax, float *logits, int64_t ldl,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * A greedy round's head and acceptance in one launch: exactly the results of
 * dspk_lmhead_argmax over m = b * m_rows rows followed by dspk_accept_greedy
 * on its ids (same argmax, accept_len and committed), with the acceptance run
 * by the head's last workgroup, so a greedy round needs no separate accept
 * launch ("mlx-dspark" wiki summary, "Architecture": each draft is checked
 * against the target's own prediction and the drafts before the first
 * mismatch are kept).
 *
 *   b, m_rows  : requests and rows per request, b * m_rows <= DSPK_MAX_ROWS;
 *                request r owns rows r * m_rows .. r * m_rows + m_rows - 1
 *   draft_ids  : int32 [b][m_rows - 1] (may be NULL when m_rows == 1)
 *   accept_len : int32 [b] output;  committed : int32 [b][m_rows] output
 * Other arguments are as in dspk_lmhead_argmax (argmax [b * m_rows] is still
 * written).  Errors: as dspk_lmhead_argmax, and DSPK_EINVAL for the rows or
 * the acceptance pointers.
 */
int dspk_lmhead_argmax_accept_greedy(const dspk_tiled_weight *w, const uint16_t *h, int64_t ldh, int32_t b,
                                     int32_t m_rows, int32_t *argmax, float *logits, int64_t ldl,
                                     const int32_t *draft_ids, int32_t *accept_len, int32_t *committed,
                                     void *workspace, size_t ws_bytes, void *stream);

/*
 * Greedy acceptance for b requests of m_rows rows each ("mlx-dspark" wiki
 * summary, "Architecture": keep the drafts up to the first mismatch; "Key
 * techniques": a round commits 1 + sum p^i tokens, i.e. always the target's
 * own token after the accepted drafts).
 *
 *   target_ids : int32 [b][m_rows]   row j's greedy token (from dspk_lmhead_argmax)
 *   draft_ids  : int32 [b][m_rows-1] draft j is compared with row j
 *   accept_len : int32 [b] output, committed tokens per request (1 .. m_rows)
 *   committed  : int32 [b][m_rows] output: accepted drafts, then the target's
 *                token of the first mismatching row (or the last row), then -1.
 * b >= 1, 1 <= m_rows <= DSPK_MAX_ROWS.
 */
int dspk_accept_greedy(const int32_t *target_ids, const int32_t *draft_ids,
                       int32_t b, int32_t m_rows,
                       int32_t *accept_len, int32_t *committed, void *stream);

/* Workspace for dspk_accept_sample and dspk_accept_sample_ex: zero-filled
 * before first use; the calls leave their arrival counter at zero, so one
 * buffer of the largest (v, m_rows) serves any sequence of sampling calls
 * ordered on one stream.  Not to be shared with projection or head calls
 * (see the workspace contract above). */
size_t dspk_sample_workspace_bytes(int32_t v, int32_t m_rows);

/*
 * Stochastic acceptance (Leviathan/Chen; "mlx-dspark" wiki summary,
 * "Architecture"; "mlx-dspark 0.7.0", "How it works": an exact sample of the
 * target at temperature T).  p_j = softmax(z_j / T).  For j = 0 .. m_rows-2
 * draft j is accepted iff u_j * q_j(d_j) < p_j(d_j); at the first reject the
 * token is drawn from norm(max(0, p_j - q_j)) (from p_j if that has no mass)
 * with u_{m_rows-1}; if all drafts pass, the bonus token is drawn from
 * p_{m_rows-1} with u_{m_rows-1}.  Draws are index-order inverse CDFs: the
 * first c whose inclusive prefix sum exceeds u * total.
 *
 *   logits   : float32 [m_rows][ldz] target logits (v columns used)
 *   q        : float32 [m_rows-1][ldq] draft distributions (used as given)
 *   draft_ids: int32 [m_rows-1]
 *   uniforms : float32 [m_rows]: u_j for draft j, the last one for the final draw
 *   temperature > 0 and finite.
 *   accept_len : int32 [1] output (committed count, 1 .. m_rows; -1 on a data
 *                fault: non-finite logit, non-finite or negative q, uniform
 *                outside [0, 1), draft id outside [0, v));
 *   committed  : int32 [m_rows] output, padded with -1 (all -1 on a fault).
 *   workspace  : >= dspk_sample_workspace_bytes(v, m_rows), 256-byte aligned,
 *                zero-filled before first use.
 * 2 <= m_rows <= DSPK_MAX_ROWS, v >= 1.
 */
int dspk_accept_sample(const float *logits, int64_t ldz,
                       const float *q, int64_t ldq, const int32_t *draft_ids,
                       const float *uniforms, int32_t m_rows, int32_t v, float temperature,
                       int32_t *accept_len, int32_t *committed,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * Sampling options of dspk_accept_sample_ex.
 *
 *   temperature       : > 0 and finite;
 *   top_k             : keep the k most probable entries (0: off; >= v: off);
 *   top_p             : in (0, 1]; keep the smallest leading set whose mass
 *                       reaches top_p of the top-k mass (1: off);
 *   presence_penalty,
 *   frequency_penalty : finite; OpenAI penalties on the target logits.
 */
typedef struct dspk_sample_params {
    float temperature;
    int32_t top_k;
    float top_p;
    float presence_penalty;
    float frequency_penalty;
} dspk_sample_params;

/*
 * Stochastic acceptance over the penalised, truncated target
 * ("mlx-dspark releases", v0.1.0 notes: one top-k / top-p filter applied to
 * the draft and to the target keeps speculative sampling an exact sample of
 * the filtered target; v0.2.0 notes: presence/frequency penalties act on the
 * target logits, and the committed tokens are those one-token decoding of
 * the penalised target would give).
 *
 * Row j's penalised logits: z'_j(c) = z_j(c) - presence * [n_j(c) > 0]
 * - frequency * n_j(c), where n_j(c) = counts[c] + #{i < j : draft_i = c}
 * (row j is reached only after drafts 0 .. j-1 were accepted).
 * p_j = softmax(z'_j / T).  Truncation orders a row's entries by value
 * (larger first, ties by the smaller column), keeps the first top_k, then
 * keeps an entry iff the kept mass before it is below top_p times the top-k
 * mass.  p~_j is p_j truncated and renormalised; q~_j is q_j truncated the
 * same way and renormalised (all zero if nothing with mass is kept).
 * Without truncation (top_k = 0 or >= v, and top_p = 1) q is used as given.
 * Then the rule of dspk_accept_sample with p~ and q~: accept draft j iff
 * u_j * q~_j(d_j) < p~_j(d_j); at the first reject draw from
 * norm(max(0, p~_j - q~_j)) (from p~_j if that has no mass), else the bonus
 * from p~_{m_rows-1}, with u_{m_rows-1}, index-order inverse CDF.
 *
 *   params : host pointer (read during the call only);
 *   counts : int32 [v] device, the history's token counts, or NULL (none);
 *            a negative count is a data fault.
 * Other arguments, faults and the workspace are as in dspk_accept_sample.
 * Returns DSPK_EINVAL for a bad parameter (temperature <= 0 or not finite,
 * top_k < 0, top_p outside (0, 1], a non-finite penalty).
 * Truncation bounds are found by exact radix selection over unique order keys;
 * masses for top-p are counted in fixed point with unit (largest entry of the
 * row) / 2^37, so an entry whose preceding mass is within v * 2^-37 of the
 * top-p threshold may fall on either side.
 */
int dspk_accept_sample_ex(const float *logits, int64_t ldz,
                          const float *q, int64_t ldq, const int32_t *draft_ids,
                          const float *uniforms, int32_t m_rows, int32_t v,
                          const dspk_sample_params *params, const int32_t *counts,
                          int32_t *accept_len, int32_t *committed,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * Draft-cap policy (host code; no GPU, no workspace).
 *
 * The cap -- how many drafts a round verifies -- does not change what is
 * committed, only how fast ("mlx-dspark 0.7.0", "Tuning": the cap is
 * measured per machine and format, not hard-coded).  A round that drafts c
 * tokens commits 1 + sum_{i=1..c} alpha^i tokens in expectation, alpha the
 * per-position acceptance ("mlx-dspark" wiki summary, "Key techniques",
 * auto-calibration bullet), and costs one verify pass at width c + 1 plus the
 * drafter's work ("mlx-dspark 0.7.0", "The Apple-Silicon speedup ceiling").
 *
 *   verify_us : host double [n], verify round time (us) at width 1 .. n,
 *               as measured on this device (e.g. the benchmark's curve);
 *   draft_us  : host double [n] or NULL, drafter time per round at cap
 *               0 .. n-1 (entry 0 is ignored: a parked round drafts nothing).
 *
 * dspk_choose_cap returns the cap c in 0 .. n-1 with the most expected
 * tokens per microsecond (ties: the smaller cap; 0 = speculation parked)
 * and stores that rate in *tokens_per_us if not NULL; it returns DSPK_EINVAL
 * for n outside 1 .. DSPK_MAX_ROWS, non-positive or non-finite times, or
 * alpha outside [0, 1] (these calls set no message).
 */
int32_t dspk_choose_cap(const double *verify_us, const double *draft_us, int32_t n, double alpha,
                        double *tokens_per_us);

/*
 * A cap controller: the curves above plus a live acceptance estimate (an
 * exponentially weighted count of accepted / tested draft positions; a
 * round that accepts a of d drafts tested a positions plus the first
 * reject).  While the best cap is 0 (parked), every probe_every-th round
 * drafts probe_cap tokens so that the estimate can recover ("mlx-dspark
 * 0.7.0", "Tuning": park with periodic probe rounds).  Plain host struct,
 * owned by the caller; one controller per request stream.
 */
typedef struct dspk_cap_controller {
    double verify_us[DSPK_MAX_ROWS];
    double draft_us[DSPK_MAX_ROWS];
    int32_t n;
    double decay;          /* weight of the past per observed round, (0, 1] */
    double hits, trials;   /* weighted accepted and tested positions */
    int32_t probe_every;
    int32_t probe_cap;
    int32_t parked_rounds;
} dspk_cap_controller;

/* prior_alpha counts as one tested position; probe_cap in 1 .. n-1. */
int dspk_cap_init(dspk_cap_controller *ctl, const double *verify_us, const double *draft_us, int32_t n,
                  double decay, double prior_alpha, int32_t probe_every, int32_t probe_cap);
/* Cap for the next round (0 = a plain step), or DSPK_EINVAL. */
int32_t dspk_cap_next(dspk_cap_controller *ctl);
/* Record a round's outcome: drafted tokens, accepted drafts (0 .. drafted). */
int dspk_cap_observe(dspk_cap_controller *ctl, int32_t drafted, int32_t accepted);
/* The current acceptance estimate. */
double dspk_cap_alpha(const dspk_cap_controller *ctl);

#ifdef __cplusplus
}
#endif

#endif /* DSPK_H */
