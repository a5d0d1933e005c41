/*
 * lce.h -- C ABI of liblce.so: fused linear cross-entropy on AMD MI355X (gfx950).
 *
 * Computes, for hidden states H [n_tok][d_model] and an output projection
 * W [vocab][d_model] (row-major, as the lossk function table of
 * "Loss functions and resident-context kernels" specifies), the cross-entropy
 * of softmax(H W^T) against integer targets WITHOUT materializing the
 * [n_tok][vocab] logit tensor, its analytic gradients, a z-loss term
 * (the square of each token's log-sum-exp), and logit distillation against a
 * full teacher distribution ("Fuse distillation + z-loss in the triton
 * monolithic path", Fast-LLM pull request 566, section "What it does").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Status: every function that can refuse returns an int32 status from the
 *   lossk range 580-599 ("Status codes" section of the lossk page); 589 and
 *   590 are this library's extensions inside that range.  Nothing throws or
 *   aborts.  On any refusal no output is modified.
 * Ownership: the caller owns every buffer, including the workspace.  The
 *   library allocates no device memory and keeps no pointer after returning.
 *   Its only state between calls: the backward's launch plan, memoized per
 *   shape (the first call on a new shape spends a few milliseconds of host
 *   time choosing it), and the static scratch of
 *   lce_distill_fwd_bwd_noalloc.  Neither changes a result; calls are
 *   reentrant given distinct workspaces.  Calls that share one workspace must
 *   be ordered (same stream).
 * Streams: device work is enqueued on the caller's stream (a hipStream_t
 *   passed as void*; NULL = the null stream).  Calls that hand back device
 *   scalars (lce_forward, lce_forward_backward, lce_shard_merge,
 *   lce_distill_fwd_bwd and lce_ce_logits_fwd_bwd with a non-NULL out, and
 *   lce_distill_fwd_bwd_noalloc) synchronize that stream once before
 *   returning.  lce_backward, lce_shard_forward, lce_shard_backward, and the
 *   five calls above with out == NULL never wait: they return once their
 *   kernels are enqueued (no allocation, no memset, so they can be captured
 *   in a HIP graph), and the scalars and the verdict of the target guard
 *   reach the host through lce_loss_fetch.
 * Validation order: dimensions -> chunk -> scalars -> dtypes -> buffer
 *   lengths and workspace size -> objective id -> device-side target guard
 *   -> compute.  The target guard runs on the device; when it fails, every
 *   compute kernel of that call exits before writing, and 586 is returned by
 *   the call (synchronous calls) or by the next lce_loss_fetch.
 * Precision: bf16 and fp16 inputs are multiplied on the matrix cores with
 *   fp32 accumulation; every softmax statistic is fp32 and every token sum
 *   fp64.  fp64 inputs run end to end in fp64.  16-bit gradients (d_hidden,
 *   logit gradients) are rounded to the input type; with fp16, grad_out is
 *   where a loss scale goes (fp16's exponent range is narrow).
 */
#ifndef LCE_H
#define LCE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (lossk "Status codes" section) ---------------------- */
#define LCE_OK 580                           /* checks passed / work ran            */
#define LCE_EMPTY_DIMENSION 581              /* a required dimension < 1            */
#define LCE_LENGTH_MISMATCH 582              /* a buffer shorter than its shape     */
#define LCE_DIMENSION_TOO_LARGE 583          /* a dimension above its ceiling       */
#define LCE_WORK_BUDGET_EXCEEDED 584         /* n_tok*d_model*vocab > 2^46          */
#define LCE_NON_FINITE_SCALAR 585            /* NaN/Inf scalar, or temperature <= 0 */
#define LCE_TARGET_OUT_OF_RANGE 586          /* a target id < 0 or >= vocab         */
#define LCE_CHUNK_EXCEEDS_LOGIT_BUDGET 587   /* chunk*vocab > 2^27                  */
#define LCE_UNKNOWN_OBJECTIVE 588            /* distillation objective id not 0..2  */
#define LCE_DEVICE_ERROR 589                 /* extension: a HIP call failed        */
#define LCE_DTYPE_MISMATCH 590               /* extension: unsupported dtype combo  */

/* Budgets of the lossk table: total work 2^46 cells, peak logits 2^27 cells.
 * Per-dimension ceilings (the page states only that each dimension has one):
 * n_tok <= 2^24, d_model <= 2^16, vocab <= 2^24; equality passes. */
#define LCE_MAX_WORK_CELLS (((int64_t)1) << 46)
#define LCE_MAX_LOGIT_CELLS (((int64_t)1) << 27)
#define LCE_MAX_N_TOK (((int64_t)1) << 24)
#define LCE_MAX_D_MODEL (((int64_t)1) << 16)
#define LCE_MAX_VOCAB (((int64_t)1) << 24)

/* ---- dtypes ------------------------------------------------------------ */
#define LCE_BF16 1
#define LCE_F32 2
#define LCE_F64 3
#define LCE_I64 4
#define LCE_F16 5
#define LCE_U8 6

/* A flat buffer: data points to numel contiguous elements of dtype.
 * Device buffers hold device pointers (hipMalloc / torch CUDA tensors). */
typedef struct lce_tensor {
  void *data;
  int64_t numel;
  int32_t dtype;
} lce_tensor;

/* Result of lce_peak_cells (the lossk reporter of chunked against
 * materialized logit cells). */
typedef struct lce_peak {
  double chunked_cells;       /* min(chunk, n_tok) * vocab                 */
  double materialized_cells;  /* n_tok * vocab                             */
  double ratio;               /* materialized / chunked                    */
  int64_t n_chunks;           /* ceil(n_tok / chunk)                       */
  int32_t status;             /* lce_chunk_check(chunk, vocab), or 581     */
} lce_peak;

/* Scalars of a forward or distillation call (host memory). */
typedef struct lce_loss {
  double loss_sum;   /* sum over counted tokens of the per-token loss        */
  double loss_mean;  /* loss_sum / n_counted (0 when nothing is counted)     */
  double z_sum;      /* sum over counted tokens of lse^2 (unscaled z-loss)   */
  double z_mean;     /* z_sum / n_counted                                    */
  int64_t n_counted; /* number of counted (unmasked) tokens                  */
} lce_loss;

/* ---- host-only contract (no device needed) ----------------------------- */

/* Name of a status code; any code not listed above gives "unknown_status"
 * (lossk table, loss_status_name).  Returns a static string. */
const char *lce_status_name(int32_t code);

/* Shape check (lossk table, loss_dims_check): 581 if any dimension < 1,
 * 583 if any is above its ceiling, 584 if n_tok*d_model*vocab > 2^46
 * (decided by dividing the budget down, never by an overflowing product),
 * else 580. */
int32_t lce_dims_check(int64_t n_tok, int64_t d_model, int64_t vocab);

/* Peak-memory check (lossk table, loss_chunk_check): 581 if chunk or vocab
 * < 1, 587 if chunk*vocab > 2^27 (refused, never clamped), else 580. */
int32_t lce_chunk_check(int64_t chunk, int64_t vocab);

/* chunk*vocab as a double; -1.0 when chunk or vocab < 1
 * (lossk table, loss_logit_cells). */
double lce_logit_cells(int64_t chunk, int64_t vocab);

/* 1 when n*d*v <= ceiling, by successive division (lossk table,
 * loss_work_fits); 0 otherwise or when any argument is < 1. */
int32_t lce_work_fits(int64_t n, int64_t d, int64_t v, int64_t ceiling);

/* Chunked against materialized logit cells (lossk table,
 * ce_peak_logit_cells, and the page's opening example).  Fills *out and
 * returns out->status: 581 (all numbers -1, n_chunks 0) when any argument
 * is < 1, else lce_chunk_check(chunk, vocab) with the numbers filled in.
 * A chunk larger than the batch holds only n_tok rows. */
int32_t lce_peak_cells(int64_t n_tok, int64_t vocab, int64_t chunk, lce_peak *out);

/* Bytes of device workspace lce_forward and lce_backward need for this
 * shape and compute dtype (LCE_BF16, LCE_F16 or LCE_F64).  Negative = -status when
 * the shape, chunk or dtype is refused.  Each logit-derived buffer of the
 * workspace stays within chunk*vocab cells, with two floors where the budget
 * is smaller than the unit of work: one token's forward partials
 * (2*ceil(vocab/128) cells, 2*ceil(vocab/64) for fp64) and one vocabulary row
 * for every token, rounded up to 64, in the backward. */
int64_t lce_workspace_bytes(int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                            int32_t dtype);

/* Bytes of device workspace lce_forward_backward needs (-status if refused):
 * lce_workspace_bytes, or more when the call keeps the whole batch's logits
 * (16-bit inputs and a chunk of at least the batch; still at most
 * chunk*vocab logit cells). */
int64_t lce_forward_backward_workspace_bytes(int64_t n_tok, int64_t d_model, int64_t vocab,
                                             int64_t chunk, int32_t dtype);

/* Which algorithm lce_forward_backward runs for a shape (host only): 1 when
 * it keeps the logits, 0 when it runs the two-call algorithm, -status when
 * the shape, chunk or dtype is refused.  1 needs all of: 16-bit inputs
 * (LCE_BF16 or LCE_F16); d_model a multiple of 64; a chunk that holds the
 * whole batch (chunk >= max(n_tok rounded up to 4, n_tok rounded up to 64
 * divided by 2)); and a launch-cost model of both algorithms that puts the
 * kept path at least 1% ahead (it saves the recompute but writes every kept
 * logit in fp32 from the forward GEMM, then reads it back and writes the
 * 16-bit gradient in a streaming pass; measured on 512 x 151936 heads the
 * kept path runs 1.03-1.05x the two calls at d_model 1024 and 1.21-1.26x at
 * 4096).  The call additionally needs hidden, weight and d_weight 16-byte
 * aligned, which only the pointers can tell. */
int32_t lce_forward_backward_keeps_logits(int64_t n_tok, int64_t d_model, int64_t vocab,
                                          int64_t chunk, int32_t dtype);

/* Bytes of device workspace lce_distill_fwd_bwd needs (-status if refused). */
int64_t lce_distill_workspace_bytes(int64_t n_tok, int64_t vocab);

/* ---- device entry points ------------------------------------------------ */

/* Fused projection + chunked cross-entropy, forward (lossk table,
 * fused_linear_ce_flat; "lossk: the loss is where the memory goes"), with
 * z-loss and a loss mask (Fast-LLM 566, "What it does").
 *   hidden    [n_tok*d_model] LCE_BF16, LCE_F16 or LCE_F64, row-major [n_tok][d_model]
 *   weight    [vocab*d_model] same dtype, row-major [vocab][d_model]
 *   targets   [n_tok] LCE_I64, each must satisfy 0 <= y < vocab (586)
 *   loss_mask [n_tok] LCE_U8 (1 = counted) or data == NULL (all counted)
 *   chunk     tokens whose logits may exist at once: each logit-derived
 *             buffer of the call holds at most chunk*vocab cells (587 above
 *             2^27; floors as for lce_workspace_bytes)
 *   z_coef    z-loss coefficient; only validated here (z_sum is unscaled)
 *   lse_out   [n_tok] per-token log-sum-exp, LCE_F32 for 16-bit inputs,
 *             LCE_F64 for fp64 inputs; lce_backward takes it back
 *   workspace LCE_U8, numel >= lce_workspace_bytes(...)
 *   out       host pointer; receives the scalars after the call synchronizes
 *             the stream.  NULL: asynchronous; nothing waits on the device,
 *             the scalars stay in the workspace for lce_loss_fetch and a bad
 *             target (586) shows there or in the next lce_backward.
 * Per-token losses are summed in token order with a fixed reduction tree,
 * so the result is bit-identical for every chunk size (lossk page,
 * "Chunk invariance is checked to the last bit"). */
int32_t lce_forward(const lce_tensor *hidden, const lce_tensor *weight,
                    const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n_tok,
                    int64_t d_model, int64_t vocab, int64_t chunk, double z_coef,
                    lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out, void *stream);

/* The scalars of the last lce_forward, lce_forward_backward,
 * lce_shard_merge, lce_distill_fwd_bwd or lce_ce_logits_fwd_bwd on this
 * workspace (lce_backward on the same workspace keeps them): synchronizes
 * `stream`, fills *out.  Returns 586 when that call, or any lce_backward,
 * lce_shard_forward or lce_shard_backward enqueued on this workspace since,
 * met a target out of range (the scalars are then not filled in), 582 for a
 * NULL out or a workspace shorter than its control block, 590 for a
 * workspace that is not LCE_U8.  The scalars are meaningful only after one
 * of the five calls above on this workspace; on a shard call's workspace
 * only the status is. */
int32_t lce_loss_fetch(const lce_tensor *workspace, lce_loss *out, void *stream);

/* Analytic backward of loss_mean + z_coef*z_mean scaled by grad_out
 * (lossk table, fused_linear_ce_bwd_flat; Fast-LLM 566, "What it does"):
 *   d[t][v] = (g + 2 g_z lse_t) softmax_t[v] - g [v == y_t],
 *   g = grad_out/C, g_z = z_coef*grad_out/C, C = counted tokens, masked -> 0;
 *   d_hidden = d W,  d_weight (+)= d^T H.
 *   lse        [n_tok] from lce_forward on the same inputs (F32 / F64)
 *   d_hidden   [n_tok*d_model] in hidden's dtype (overwritten)
 *   d_weight   [vocab*d_model] LCE_F32 for 16-bit inputs, LCE_F64 for fp64;
 *              overwritten, or added to when accumulate_d_weight != 0
 * Logits are recomputed from H and W; the logit-gradient buffer holds at
 * most chunk*vocab cells at once.
 * Asynchronous: returns 580 once the kernels are enqueued on `stream` (or a
 * host-side refusal, or 589 when a launch fails) without waiting for the
 * device.  A target out of range makes every kernel of the call exit before
 * writing (d_hidden and d_weight keep their contents); lce_loss_fetch on the
 * same workspace then returns 586. */
int32_t lce_backward(const lce_tensor *hidden, const lce_tensor *weight,
                     const lce_tensor *targets, const lce_tensor *loss_mask,
                     const lce_tensor *lse, int64_t n_tok, int64_t d_model, int64_t vocab,
                     int64_t chunk, double z_coef, double grad_out, lce_tensor *d_hidden,
                     lce_tensor *d_weight, int32_t accumulate_d_weight,
                     lce_tensor *workspace, void *stream);

/* Forward and backward in one call (lossk table: the flat forward and
 * backward pair; Fast-LLM 566 fuses a label loss's forward and backward the
 * same way): the loss scalars (out), lse_out and the gradients of
 * grad_out * (loss_mean + z_coef * z_mean), with the arguments of
 * lce_forward and lce_backward and one stream synchronization at the end.
 *   workspace  numel >= lce_forward_backward_workspace_bytes(...)
 *   out        host pointer: the call synchronizes the stream and fills it.
 *              NULL: asynchronous, as lce_forward with a NULL out; the
 *              scalars and the target guard's verdict (586) stay in the
 *              workspace for lce_loss_fetch
 * The logits are computed once -- kept in fp32 ([vocab][ld] cells, at most
 * chunk*vocab), reduced to lse, turned in place into the logit gradient and
 * fed to the d_hidden and d_weight products (6 n d_model vocab flops
 * instead of 8) -- exactly when lce_forward_backward_keeps_logits(...) is 1
 * for the shape AND hidden, weight and d_weight are 16-byte aligned.  The
 * logit gradient then has the same values as lce_backward's, so lse, the
 * loss scalars and d_weight equal the two-call results bit for bit and
 * d_hidden agrees to fp32 summation order.  Otherwise the call runs
 * lce_forward's and lce_backward's algorithm.  Status codes as lce_forward
 * and lce_backward. */
int32_t lce_forward_backward(const lce_tensor *hidden, const lce_tensor *weight,
                             const lce_tensor *targets, const lce_tensor *loss_mask,
                             int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                             double z_coef, double grad_out, lce_tensor *lse_out,
                             lce_tensor *d_hidden, lce_tensor *d_weight,
                             int32_t accumulate_d_weight, lce_tensor *workspace, lce_loss *out,
                             void *stream);

/* Distillation against a teacher distribution, fused forward + backward,
 * with z-loss over the same student softmax (Fast-LLM 566, "What it does"
 * and "Changes": returns loss, z-loss and the logit gradient).
 *   student, teacher [n_tok*vocab] logits, LCE_BF16, LCE_F16, LCE_F32 or LCE_F64
 *                    (same dtype), row-major [n_tok][vocab]
 *   loss_mask        [n_tok] LCE_U8 or data == NULL
 *   objective        0 soft-target cross-entropy -sum q log p,
 *                    1 forward KL(q||p), 2 reverse KL(p||q)   (else 588)
 *   temperature      > 0 and finite (else 585); x = s/T, y = u/T
 *   grad_logits      [n_tok*vocab] in the student's dtype:
 *                    (grad_out/C) (dL/dx + 2 z_coef lse(x) p) / T, masked rows 0
 *   workspace        LCE_U8, numel >= lce_distill_workspace_bytes(...)
 *   out              host; loss_sum/loss_mean = distillation loss,
 *                    z_sum/z_mean = unscaled z-loss, n_counted = C; the call
 *                    synchronizes the stream to fill it.  NULL: the call
 *                    returns once its kernels are enqueued and
 *                    lce_loss_fetch(workspace) returns the scalars later. */
int32_t lce_distill_fwd_bwd(const lce_tensor *student, const lce_tensor *teacher,
                            const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                            int32_t objective, double temperature, double z_coef,
                            double grad_out, lce_tensor *grad_logits, lce_tensor *workspace,
                            lce_loss *out, void *stream);

/* lce_distill_fwd_bwd for callers that cannot allocate device memory (tight
 * serving loops, harnesses that forbid hipMalloc): the same computation,
 * arguments and statuses without the workspace argument.  Like
 * lce_distill_fwd_bwd it synchronizes the stream once to return the scalars,
 * so it is not meant for a stream under graph capture.  Its scratch (control block and per-row results) is a
 * static device array of this library, 256 + 16 * 65536 bytes per GPU, held
 * by every GPU the library runs on until the process ends; the call itself
 * allocates nothing.
 *   n_tok     at most 65536 (else 582: the static scratch is too short)
 * The call clears what must start at zero.  Every call on one GPU shares
 * that GPU's scratch, so calls that overlap on one GPU (different streams or
 * host threads) race; order them.  Returns 589 if the scratch's device
 * address cannot be obtained. */
int32_t lce_distill_fwd_bwd_noalloc(const lce_tensor *student, const lce_tensor *teacher,
                                    const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                                    int32_t objective, double temperature, double z_coef,
                                    double grad_out, lce_tensor *grad_logits, lce_loss *out,
                                    void *stream);

/* ---- vocabulary shards: one GPU's rows of a vocabulary-parallel head ---- */

/* The lossk reduction (per token lse and target logit, "Loss functions and
 * resident-context kernels", lossk table) split over row ranges of the head:
 * each shard reports per-token {m, s, z} and an exchange folds them, in the
 * form the Fast-LLM 566 tensor-parallel tests exercise ("Changes",
 * "Validation").  Shards must partition [0, vocab_total).
 *   weight_shard rows [vocab_offset, vocab_offset + vocab_shard) of the head,
 *                [vocab_shard*d_model], dtype as hidden
 *   targets      global ids, each 0 <= y < vocab_total (else 586)
 *   vocab_total  rows of the whole head; vocab_offset >= 0 and
 *                vocab_offset + vocab_shard <= vocab_total (else 582;
 *                vocab_total > LCE_MAX_VOCAB: 583)
 *   chunk        bounds the shard's logit buffers: chunk * vocab_shard cells
 *   workspace    numel >= lce_workspace_bytes(n_tok, d_model, vocab_shard,
 *                chunk, dtype)
 * lce_shard_forward writes stats[3*n_tok] in the accumulator dtype (LCE_F32
 * for 16-bit inputs, LCE_F64 for fp64): stats[t] = m_t, the shard's largest
 * logit of token t; stats[n_tok + t] = s_t = sum over the shard's rows of
 * exp(z - m_t); stats[2*n_tok + t] = z[t][y_t] when the shard holds row y_t,
 * else 0.  It returns once its kernels are enqueued (no host wait, so the
 * records can go straight into the exchange): a target out of range makes
 * its kernels exit before writing the records and is reported as 586 by
 * lce_loss_fetch(workspace), as for lce_backward; check it before trusting
 * the records (the scalars lce_loss_fetch returns are meaningless for a
 * shard's workspace). */
int32_t lce_shard_forward(const lce_tensor *hidden, const lce_tensor *weight_shard,
                          const lce_tensor *targets, int64_t n_tok, int64_t d_model,
                          int64_t vocab_shard, int64_t vocab_offset, int64_t vocab_total,
                          int64_t chunk, lce_tensor *stats, lce_tensor *workspace, void *stream);

/* The exchange: stats holds n_shards records of 3*n_tok values each (shard q
 * at stats[q*3*n_tok], any order of shards gives the same rows; they are
 * folded in index order): lse_t = M + log sum_q s_q exp(m_q - M) with M the
 * largest m_q, z_y = sum_q z_q; loss and z-loss over counted tokens as
 * lce_forward.
 *   stats     LCE_F32 or LCE_F64, numel >= n_shards*3*n_tok
 *   loss_mask [n_tok] LCE_U8 or data == NULL
 *   lse_out   [n_tok], stats' dtype (the backward's lse)
 *   workspace LCE_U8, numel >= lce_distill_workspace_bytes(n_tok, 1)
 *   out       host loss scalars; synchronizes the stream.  NULL: the call
 *             returns once its kernels are enqueued and
 *             lce_loss_fetch(workspace) returns the scalars later. */
int32_t lce_shard_merge(const lce_tensor *stats, int32_t n_shards, const lce_tensor *loss_mask,
                        int64_t n_tok, lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out,
                        void *stream);

/* A shard's backward with the merged lse: d_weight_shard [vocab_shard *
 * d_model] (LCE_F32 | LCE_F64; overwritten, or added to when
 * accumulate_d_weight != 0) and the shard's d_hidden partial
 * sum over its rows of dlogit * W, [n_tok*d_model] in the accumulator dtype
 * (overwritten); the sum of the partials over all shards is d_hidden.
 * Other arguments and statuses as lce_backward. */
int32_t lce_shard_backward(const lce_tensor *hidden, const lce_tensor *weight_shard,
                           const lce_tensor *targets, const lce_tensor *loss_mask,
                           const lce_tensor *lse, int64_t n_tok, int64_t d_model,
                           int64_t vocab_shard, int64_t vocab_offset, int64_t vocab_total,
                           int64_t chunk, double z_coef, double grad_out,
                           lce_tensor *d_hidden_partial, lce_tensor *d_weight_shard,
                           int32_t accumulate_d_weight, lce_tensor *workspace, void *stream);

/* Label cross-entropy with z-loss from materialized logits, fused forward +
 * backward: the lossk page's ce_from_logits reference function ("Loss
 * functions and resident-context kernels", lossk table) on the device, with
 * the loss mask and z term of Fast-LLM 566 ("What it does", "Changes").
 *   logits       [n_tok*vocab] LCE_BF16, LCE_F16, LCE_F32 or LCE_F64, row-major
 *                [n_tok][vocab]
 *   targets      [n_tok] LCE_I64, each 0 <= y < vocab (else 586, with
 *                grad_logits untouched)
 *   loss_mask    [n_tok] LCE_U8 or data == NULL (all rows counted)
 *   grad_logits  [n_tok*vocab] in the logits' dtype, overwritten with
 *                (grad_out/C)((1 + 2 z_coef lse) softmax - onehot(y)), masked
 *                rows 0; NULL or data == NULL computes the loss only (the
 *                logits are then read once)
 *   workspace    LCE_U8, numel >= lce_distill_workspace_bytes(n_tok, vocab)
 *   out          host; loss_sum/loss_mean = sum/mean over counted rows of
 *                lse - z[y], z_sum/z_mean = unscaled lse^2, n_counted = C;
 *                the call returns after the scalars reach the host.  NULL:
 *                it returns once its kernels are enqueued; lce_loss_fetch
 *                (workspace) then returns the scalars, or 586 for a target
 *                out of range (grad_logits untouched, as in the synchronous
 *                call).
 * Statuses as lce_distill_fwd_bwd (no objective or temperature). */
int32_t lce_ce_logits_fwd_bwd(const lce_tensor *logits, const lce_tensor *targets,
                              const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                              double z_coef, double grad_out, lce_tensor *grad_logits,
                              lce_tensor *workspace, lce_loss *out, void *stream);

/* ---- optional kernel timing (for benchmarks and profilers) ------------- */

/* Kernel kinds a timed call can bracket with events. */
#define LCE_K_GUARD 0        /* target guard and counted-token count            */
#define LCE_K_FWD_GEMM 1     /* forward logit GEMM with the online-LSE epilogue */
#define LCE_K_FWD_MERGE 2    /* per-token merge of (max, sum) pairs             */
#define LCE_K_REDUCE 3       /* fixed-order token sums                          */
#define LCE_K_DLOGIT_GEMM 4  /* backward logit recompute -> logit gradient      */
#define LCE_K_DW_GEMM 5      /* d_weight rows of a slab                         */
#define LCE_K_DH_GEMM 6      /* split-K d_hidden accumulation                   */
#define LCE_K_DH_FINAL 7     /* fold of the d_hidden splits                     */
#define LCE_K_DISTILL 8      /* distillation row kernel                         */
#define LCE_K_BWD_GEMM 9     /* one launch of the slab-pipelined 16-bit backward:*/
                             /* d_hidden and d_weight of slab k with the logit  */
                             /* gradient of slab k+1                            */
#define LCE_K_LABEL_CE 10    /* label cross-entropy row kernel (logits in)      */
#define LCE_K_DLOGIT_ROWS 11 /* single call: kept logits -> logit gradient      */
#define LCE_NUM_KERNELS 12

/* One slot per kernel kind.  start/stop hold `capacity` caller-created
 * hipEvent_t handles (as void*); a timed call records start[i]/stop[i] on
 * its stream around the i-th launch of that kind (i counted from `used`,
 * which the call advances; launches beyond capacity are not recorded).
 * Slots with capacity 0 are ignored.  The caller owns the events. */
typedef struct lce_timer_slot {
  void **start;
  void **stop;
  int32_t capacity;
  int32_t used;
} lce_timer_slot;

typedef struct lce_timers {
  lce_timer_slot slot[LCE_NUM_KERNELS];
} lce_timers;

/* Same as lce_forward / lce_backward / lce_forward_backward /
 * lce_distill_fwd_bwd, recording
 * events into *timers (NULL = no timing, identical to the plain call). */
int32_t lce_forward_timed(const lce_tensor *hidden, const lce_tensor *weight,
                          const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n_tok,
                          int64_t d_model, int64_t vocab, int64_t chunk, double z_coef,
                          lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out,
                          void *stream, lce_timers *timers);
int32_t lce_backward_timed(const lce_tensor *hidden, const lce_tensor *weight,
                           const lce_tensor *targets, const lce_tensor *loss_mask,
                           const lce_tensor *lse, int64_t n_tok, int64_t d_model, int64_t vocab,
                           int64_t chunk, double z_coef, double grad_out, lce_tensor *d_hidden,
                           lce_tensor *d_weight, int32_t accumulate_d_weight,
                           lce_tensor *workspace, void *stream, lce_timers *timers);
int32_t lce_forward_backward_timed(const lce_tensor *hidden, const lce_tensor *weight,
                                   const lce_tensor *targets, const lce_tensor *loss_mask,
                                   int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                                   double z_coef, double grad_out, lce_tensor *lse_out,
                                   lce_tensor *d_hidden, lce_tensor *d_weight,
                                   int32_t accumulate_d_weight, lce_tensor *workspace,
                                   lce_loss *out, void *stream, lce_timers *timers);
int32_t lce_distill_fwd_bwd_timed(const lce_tensor *student, const lce_tensor *teacher,
                                  const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                                  int32_t objective, double temperature, double z_coef,
                                  double grad_out, lce_tensor *grad_logits,
                                  lce_tensor *workspace, lce_loss *out, void *stream,
                                  lce_timers *timers);
int32_t lce_ce_logits_fwd_bwd_timed(const lce_tensor *logits, const lce_tensor *targets,
                                    const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                                    double z_coef, double grad_out, lce_tensor *grad_logits,
                                    lce_tensor *workspace, lce_loss *out, void *stream,
                                    lce_timers *timers);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */
