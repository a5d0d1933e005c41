/*
 * lce_oracle.c -- plain, slow, CPU fp64 oracle for fused linear cross-entropy.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with the
 * GPU library in lm_head_linear_amd/.
 *
 * Sources (cited by page title and section):
 *   [P1] "Loss functions and resident-context kernels" (algenta docs):
 *        the lossk function table, "Status codes", "A worked example: uniform
 *        logits give exactly log(vocab)", "The two budgets are genuinely
 *        different questions", "Chunk invariance is checked to the last bit",
 *        "The backward's gradient check is a cancellation identity".
 *   [P3] "Fuse distillation + z-loss in the triton monolithic path"
 *        (Fast-LLM pull request 566), sections "What it does" and "Changes".
 *
 * Conventions:
 *   - IEEE fp64, round to nearest even, built with -O2 -ffp-contract=off and
 *     no fast-math, so a*b+c is always a rounded product then a rounded sum.
 *   - Every sum is taken in ascending index order with one accumulator.
 *   - Work is split over threads by token (forward, d_hidden, distillation)
 *     or by vocabulary row (d_weight).  Each output is produced by one
 *     thread in a fixed order, so results are bit-identical for any thread
 *     count.
 *   - exp/log are the C library's.
 *
 * Readings taken where the pages are silent:
 *   per-dimension ceilings n_tok <= 2^24, d_model <= 2^16, vocab <= 2^24;
 *   equality with a ceiling passes; mask value 1 = token counted, NULL mask =
 *   all counted; mean over counted tokens; all tokens masked -> zeros and ok;
 *   z-loss reported unscaled (the objective adds z_coef times it); distillation
 *   divides both logit sets by the temperature with no T^2 factor; forward-KL
 *   is KL(teacher||student), reverse-KL is KL(student||teacher); the
 *   distillation "cross-entropy" is the soft-target -sum q log p.
 *
 * Parity pins: every function here is pinned by a -m "not gpu" test in
 * tests/test_oracle.py (printed values, closed forms, library routines,
 * finite differences, identities).  The temperature placement and the z-loss
 * under temperature have no pin beyond their identities: parity unpinned for
 * those two readings.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status vocabulary of lossk, [P1] "Status codes"; 589 and 590 are
 * extensions inside lossk's 580-599 range. */
enum {
  ORC_OK = 580,
  ORC_EMPTY_DIMENSION = 581,
  ORC_LENGTH_MISMATCH = 582,
  ORC_DIMENSION_TOO_LARGE = 583,
  ORC_WORK_BUDGET_EXCEEDED = 584,
  ORC_NON_FINITE_SCALAR = 585,
  ORC_TARGET_OUT_OF_RANGE = 586,
  ORC_CHUNK_EXCEEDS_LOGIT_BUDGET = 587,
  ORC_UNKNOWN_OBJECTIVE = 588,
  ORC_DEVICE_ERROR = 589,
  ORC_DTYPE_MISMATCH = 590
};

/* [P1] lossk table: total-work ceiling 2^46 cells, peak-logit ceiling 2^27
 * cells.  The per-dimension ceilings are a reading (the page says
 * only that each dimension is "under its ceiling"). */
#define ORC_MAX_WORK_CELLS (((int64_t)1) << 46)
#define ORC_MAX_LOGIT_CELLS (((int64_t)1) << 27)
#define ORC_MAX_N_TOK (((int64_t)1) << 24)
#define ORC_MAX_D_MODEL (((int64_t)1) << 16)
#define ORC_MAX_VOCAB (((int64_t)1) << 24)

/* ------------------------------------------------------------------------ */
/* Contract: pure integer arithmetic, [P1] lossk function table.            */
/* ------------------------------------------------------------------------ */

const char *orc_status_name(int code) {
  switch (code) {
  case 580: return "ok";
  case 581: return "empty_dimension";
  case 582: return "length_mismatch";
  case 583: return "dimension_too_large";
  case 584: return "work_budget_exceeded";
  case 585: return "non_finite_scalar";
  case 586: return "target_id_out_of_range";
  case 587: return "chunk_exceeds_logit_budget";
  case 588: return "unknown_objective";
  case 589: return "device_error";
  case 590: return "dtype_mismatch";
  default: return "unknown_status";
  }
}

/* n*d*v <= ceiling, decided by dividing the ceiling down instead of
 * multiplying up, so nothing overflows.  For positive integers,
 * floor(floor(c/v)/d) = floor(c/(v*d)), and n*d*v <= c iff n <= that. */
int orc_work_fits(int64_t n, int64_t d, int64_t v, int64_t ceiling) {
  if (n < 1 || d < 1 || v < 1 || ceiling < 0) return 0;
  int64_t q = ceiling / v;
  q = q / d;
  return n <= q;
}

int orc_dims_check(int64_t n_tok, int64_t d_model, int64_t vocab) {
  if (n_tok < 1 || d_model < 1 || vocab < 1) return ORC_EMPTY_DIMENSION;
  if (n_tok > ORC_MAX_N_TOK || d_model > ORC_MAX_D_MODEL || vocab > ORC_MAX_VOCAB)
    return ORC_DIMENSION_TOO_LARGE;
  if (!orc_work_fits(n_tok, d_model, vocab, ORC_MAX_WORK_CELLS))
    return ORC_WORK_BUDGET_EXCEEDED;
  return ORC_OK;
}

/* chunk*vocab > 2^27 iff chunk > floor(2^27 / vocab) for positive integers. */
int orc_chunk_check(int64_t chunk, int64_t vocab) {
  if (chunk < 1 || vocab < 1) return ORC_EMPTY_DIMENSION;
  if (chunk > ORC_MAX_LOGIT_CELLS / vocab) return ORC_CHUNK_EXCEEDS_LOGIT_BUDGET;
  return ORC_OK;
}

/* chunk*vocab as a double; -1.0 when the request is malformed. */
double orc_logit_cells(int64_t chunk, int64_t vocab) {
  if (chunk < 1 || vocab < 1) return -1.0;
  return (double)chunk * (double)vocab;
}

/* What a chunked call holds against the materialized form.
 * out3 = {chunked_cells, materialized_cells, ratio}; *n_chunks = ceil(n/c).
 * A chunk larger than the batch holds only n_tok rows. */
int orc_peak_cells(int64_t n_tok, int64_t vocab, int64_t chunk, double *out3,
                   int64_t *n_chunks) {
  if (n_tok < 1 || vocab < 1 || chunk < 1) {
    out3[0] = -1.0; out3[1] = -1.0; out3[2] = -1.0; *n_chunks = 0;
    return ORC_EMPTY_DIMENSION;
  }
  int64_t held = chunk < n_tok ? chunk : n_tok;
  out3[0] = orc_logit_cells(held, vocab);
  out3[1] = orc_logit_cells(n_tok, vocab);
  out3[2] = out3[1] / out3[0];
  *n_chunks = n_tok / chunk + (n_tok % chunk != 0);
  return orc_chunk_check(chunk, vocab);
}

/* Every one of the first n_tok targets lies in [0, vocab); a negative id is
 * an error, never a mask. */
int orc_targets_in_range(const int64_t *targets, int64_t n_tok, int64_t vocab) {
  for (int64_t t = 0; t < n_tok; ++t)
    if (targets[t] < 0 || targets[t] >= vocab) return 0;
  return 1;
}

static int is_fin(double x) { return isfinite(x) != 0; }

/* ------------------------------------------------------------------------ */
/* A tiny static parallel-for: thread k runs items k, k+T, k+2T, ...         */
/* ------------------------------------------------------------------------ */

typedef void (*orc_item_fn)(void *ctx, int64_t item);
typedef struct { orc_item_fn fn; void *ctx; int64_t n_items; int tid, nthr; } orc_job;

static void *orc_worker(void *p) {
  orc_job *j = (orc_job *)p;
  for (int64_t i = j->tid; i < j->n_items; i += j->nthr) j->fn(j->ctx, i);
  return NULL;
}

static void orc_parallel_for(int nthreads, int64_t n_items, orc_item_fn fn, void *ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads == 1 || n_items <= 1) {
    for (int64_t i = 0; i < n_items; ++i) fn(ctx, i);
    return;
  }
  pthread_t th[256];
  orc_job jobs[256];
  for (int k = 0; k < nthreads; ++k) {
    jobs[k].fn = fn; jobs[k].ctx = ctx; jobs[k].n_items = n_items;
    jobs[k].tid = k; jobs[k].nthr = nthreads;
    pthread_create(&th[k], NULL, orc_worker, &jobs[k]);
  }
  for (int k = 0; k < nthreads; ++k) pthread_join(th[k], NULL);
}

/* ------------------------------------------------------------------------ */
/* Log-sum-exp of one row, two passes, ascending index ([P1] names a frozen  */
/* logsumexp reduction; the plain max-shifted form is used here).           */
/* ------------------------------------------------------------------------ */

static double row_lse(const double *x, int64_t n) {
  double m = x[0];
  for (int64_t i = 1; i < n; ++i)
    if (x[i] > m) m = x[i];
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s = s + exp(x[i] - m);
  return m + log(s);
}

/* Cross-entropy from materialized logits [n_tok][vocab] ([P1] lossk table and
 * the uniform-logits worked example).  loss_t = lse_t - L[t][y_t];
 * mean = (sum over t ascending of loss_t) / n_tok. */
int orc_ce_from_logits(const double *logits, const int64_t *targets, int64_t n_tok,
                       int64_t vocab, double *loss_tok, double *mean_loss) {
  if (n_tok < 1 || vocab < 1) return ORC_EMPTY_DIMENSION;
  if (!orc_targets_in_range(targets, n_tok, vocab)) return ORC_TARGET_OUT_OF_RANGE;
  double sum = 0.0;
  for (int64_t t = 0; t < n_tok; ++t) {
    const double *row = logits + t * vocab;
    double lse = row_lse(row, vocab);
    double l = lse - row[targets[t]];
    if (loss_tok) loss_tok[t] = l;
    sum = sum + l;
  }
  *mean_loss = sum / (double)n_tok;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Logits: z[t][v] = sum over d ascending of W[v][d]*H[t][d]                 */
/* ([P1] lossk table: weight is [vocab][d_model] row-major, hidden is        */
/* [n_tok][d_model]).                                                       */
/* ------------------------------------------------------------------------ */

static double dot_asc(const double *a, const double *b, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc = acc + a[i] * b[i];
  return acc;
}

/* Logit rows of up to four tokens.  The four tokens share one read of each
 * W row purely for speed; each logit keeps its own accumulator and its own
 * ascending-d order, so every value equals dot_asc(W[v], H[t]) bit for bit. */
static void logit_rows4(const double *W, int64_t D, int64_t V, const double *const *h,
                        int cnt, double *const *out) {
  if (cnt != 4) {
    for (int k = 0; k < cnt; ++k)
      for (int64_t v = 0; v < V; ++v) out[k][v] = dot_asc(W + v * D, h[k], D);
    return;
  }
  const double *h0 = h[0], *h1 = h[1], *h2 = h[2], *h3 = h[3];
  for (int64_t v = 0; v < V; ++v) {
    const double *w = W + v * D;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      double wd = w[d];
      a0 = a0 + wd * h0[d];
      a1 = a1 + wd * h1[d];
      a2 = a2 + wd * h2[d];
      a3 = a3 + wd * h3[d];
    }
    out[0][v] = a0; out[1][v] = a1; out[2][v] = a2; out[3][v] = a3;
  }
}

/* ------------------------------------------------------------------------ */
/* Fused projection + chunked cross-entropy ([P1] lossk table: the fused     */
/* function; "lossk: the loss is where the memory goes"), with z-loss        */
/* ([P3] "What it does": forward scalar lse^2) and the shared loss mask and  */
/* divisor ([P3] "What it does").                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *H, *W;
  const int64_t *targets;
  int64_t D, V, k0, rows;      /* this chunk: tokens k0 .. k0+rows-1 */
  double *buf;                 /* chunk buffer, rows x V */
  double *lse_out, *loss_tok;
} fwd_ctx;

/* One item = a group of up to four tokens of the current chunk. */
static void fwd_item(void *p, int64_t g) {
  fwd_ctx *c = (fwd_ctx *)p;
  int64_t r0 = g * 4;
  int cnt = (int)((c->rows - r0) < 4 ? (c->rows - r0) : 4);
  const double *h[4];
  double *out[4];
  for (int k = 0; k < cnt; ++k) {
    h[k] = c->H + (c->k0 + r0 + k) * c->D;
    out[k] = c->buf + (r0 + k) * c->V;
  }
  logit_rows4(c->W, c->D, c->V, h, cnt, out);
  for (int k = 0; k < cnt; ++k) {
    int64_t t = c->k0 + r0 + k;
    double lse = row_lse(out[k], c->V);
    c->lse_out[t] = lse;
    c->loss_tok[t] = lse - out[k][c->targets[t]];
  }
}

/* out5 = {loss_sum, loss_mean, z_sum, z_mean, n_counted}.  lse_out and
 * loss_tok receive every token's value (masked tokens included); the sums
 * take counted tokens only, in token order. */
int orc_fused_forward(const double *H, const double *W, const int64_t *targets,
                      const uint8_t *mask, int64_t n_tok, int64_t d_model, int64_t vocab,
                      int64_t chunk, double z_coef, int nthreads, double *lse_out,
                      double *loss_tok, double *out5) {
  int st = orc_dims_check(n_tok, d_model, vocab);
  if (st != ORC_OK) return st;
  st = orc_chunk_check(chunk, vocab);
  if (st != ORC_OK) return st;
  if (!is_fin(z_coef)) return ORC_NON_FINITE_SCALAR;
  if (!orc_targets_in_range(targets, n_tok, vocab)) return ORC_TARGET_OUT_OF_RANGE;

  int64_t held = chunk < n_tok ? chunk : n_tok;
  double *buf = (double *)malloc(sizeof(double) * (size_t)held * (size_t)vocab);
  if (!buf) return ORC_DEVICE_ERROR;
  for (int64_t k0 = 0; k0 < n_tok; k0 += chunk) {
    fwd_ctx c;
    c.H = H; c.W = W; c.targets = targets; c.D = d_model; c.V = vocab;
    c.k0 = k0; c.rows = (n_tok - k0) < chunk ? (n_tok - k0) : chunk;
    c.buf = buf; c.lse_out = lse_out; c.loss_tok = loss_tok;
    orc_parallel_for(nthreads, (c.rows + 3) / 4, fwd_item, &c);
  }
  free(buf);

  double loss_sum = 0.0, z_sum = 0.0;
  int64_t counted = 0;
  for (int64_t t = 0; t < n_tok; ++t) {
    if (mask && !mask[t]) continue;
    loss_sum = loss_sum + loss_tok[t];
    z_sum = z_sum + lse_out[t] * lse_out[t];
    counted += 1;
  }
  out5[0] = loss_sum;
  out5[1] = counted ? loss_sum / (double)counted : 0.0;
  out5[2] = z_sum;
  out5[3] = counted ? z_sum / (double)counted : 0.0;
  out5[4] = (double)counted;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Analytic backward ([P1] lossk table: gradients w.r.t. hidden and weight;  */
/* [P3] "What it does": a label loss superposes softmax and a one-hot, and   */
/* z-loss adds 2*grad_z*lse*p).  With g = grad_out/C and                     */
/* g_z = z_coef*grad_out/C, the logit gradient of counted token t is         */
/*   d[t][v] = (g + 2*g_z*lse_t) * exp(z[t][v] - lse_t) - g*[v == y_t]      */
/* and 0 for a masked token.  dH[t][j] = sum_v ascending d[t][v]*W[v][j];    */
/* dW[v][j] = (accumulate ? dW_in[v][j] : 0) + sum_t ascending d[t][v]*H[t][j]. */
/* lse must be the one orc_fused_forward returned.                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *H, *W, *lse;
  const int64_t *targets;
  const uint8_t *mask;
  int64_t n, D, V;
  double g, gz;
  const int64_t *rows;  /* which tokens (dH) or vocabulary rows (dW) */
  double *out;          /* one output row of D values per listed row */
  int accumulate;
} bwd_ctx;

static double dlogit(const bwd_ctx *c, int64_t t, int64_t v, double z) {
  double lse = c->lse[t];
  double p = exp(z - lse);
  double coef = c->g + 2.0 * c->gz * lse;
  double d = coef * p;
  if (v == c->targets[t]) d = d - c->g;
  return d;
}

static void dh_item(void *p, int64_t i) {
  bwd_ctx *c = (bwd_ctx *)p;
  int64_t t = c->rows[i];
  double *o = c->out + i * c->D;
  for (int64_t j = 0; j < c->D; ++j) o[j] = 0.0;
  if (c->mask && !c->mask[t]) return;
  const double *h = c->H + t * c->D;
  for (int64_t v = 0; v < c->V; ++v) {
    const double *w = c->W + v * c->D;
    double d = dlogit(c, t, v, dot_asc(w, h, c->D));
    for (int64_t j = 0; j < c->D; ++j) o[j] = o[j] + d * w[j];
  }
}

static void dw_item(void *p, int64_t i) {
  bwd_ctx *c = (bwd_ctx *)p;
  int64_t v = c->rows[i];
  double *o = c->out + i * c->D;
  const double *w = c->W + v * c->D;
  double *acc = (double *)calloc((size_t)c->D, sizeof(double));
  for (int64_t t = 0; t < c->n; ++t) {
    if (c->mask && !c->mask[t]) continue;
    const double *h = c->H + t * c->D;
    double d = dlogit(c, t, v, dot_asc(w, h, c->D));
    for (int64_t j = 0; j < c->D; ++j) acc[j] = acc[j] + d * h[j];
  }
  for (int64_t j = 0; j < c->D; ++j) o[j] = c->accumulate ? o[j] + acc[j] : acc[j];
  free(acc);
}

static int bwd_setup(bwd_ctx *c, const double *H, const double *W, const int64_t *targets,
                     const uint8_t *mask, const double *lse, int64_t n_tok, int64_t d_model,
                     int64_t vocab, double z_coef, double grad_out) {
  int st = orc_dims_check(n_tok, d_model, vocab);
  if (st != ORC_OK) return st;
  if (!is_fin(z_coef) || !is_fin(grad_out)) return ORC_NON_FINITE_SCALAR;
  if (!orc_targets_in_range(targets, n_tok, vocab)) return ORC_TARGET_OUT_OF_RANGE;
  int64_t counted = 0;
  for (int64_t t = 0; t < n_tok; ++t) counted += (!mask || mask[t]) ? 1 : 0;
  c->H = H; c->W = W; c->lse = lse; c->targets = targets; c->mask = mask;
  c->n = n_tok; c->D = d_model; c->V = vocab;
  c->g = counted ? grad_out / (double)counted : 0.0;
  c->gz = counted ? z_coef * grad_out / (double)counted : 0.0;
  return ORC_OK;
}

/* d_hidden rows for the listed tokens: out is [n_rows][d_model]. */
int orc_backward_dh_rows(const double *H, const double *W, const int64_t *targets,
                         const uint8_t *mask, const double *lse, int64_t n_tok,
                         int64_t d_model, int64_t vocab, double z_coef, double grad_out,
                         const int64_t *rows, int64_t n_rows, int nthreads, double *out) {
  bwd_ctx c;
  int st = bwd_setup(&c, H, W, targets, mask, lse, n_tok, d_model, vocab, z_coef, grad_out);
  if (st != ORC_OK) return st;
  c.rows = rows; c.out = out; c.accumulate = 0;
  orc_parallel_for(nthreads, n_rows, dh_item, &c);
  return ORC_OK;
}

/* d_weight rows for the listed vocabulary rows: out is [n_rows][d_model] and
 * holds dW_in on entry when accumulate is set. */
int orc_backward_dw_rows(const double *H, const double *W, const int64_t *targets,
                         const uint8_t *mask, const double *lse, int64_t n_tok,
                         int64_t d_model, int64_t vocab, double z_coef, double grad_out,
                         const int64_t *rows, int64_t n_rows, int accumulate, int nthreads,
                         double *out) {
  bwd_ctx c;
  int st = bwd_setup(&c, H, W, targets, mask, lse, n_tok, d_model, vocab, z_coef, grad_out);
  if (st != ORC_OK) return st;
  c.rows = rows; c.out = out; c.accumulate = accumulate;
  orc_parallel_for(nthreads, n_rows, dw_item, &c);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Distillation against a full teacher distribution, with z-loss over the    */
/* same student softmax ([P3] "What it does" and "Changes").  For a counted  */
/* row t, with temperature T:                                                */
/*   x = s/T, y = u/T, ls = x - lse(x), lq = y - lse(y), p = e^ls, q = e^lq  */
/*   objective 0, cross-entropy: L = -sum q*ls,         dL/dx = p - q        */
/*   objective 1, forward KL(q||p): L = sum q*(lq-ls),  dL/dx = p - q        */
/*   objective 2, reverse KL(p||q): L = sum p*(ls-lq),  dL/dx = p*(ls-lq-L)  */
/*   grad[t][v] = (grad_out/C) * (dL/dx_v + 2*z_coef*lse(x)*p_v) / T         */
/* loss = sum L_t / C, z_loss = sum lse(x)^2 / C; masked rows get zeros.     */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *S, *U;
  const uint8_t *mask;
  int64_t V;
  int objective;
  double T, z_coef, scale;  /* scale = grad_out / C */
  const int64_t *rows;
  double *grad;             /* [n_rows][V] or NULL */
  double *row_loss, *row_lse;
} dis_ctx;

static void dis_item(void *p, int64_t i) {
  dis_ctx *c = (dis_ctx *)p;
  int64_t t = c->rows[i];
  int64_t V = c->V;
  double *g = c->grad ? c->grad + i * V : NULL;
  if (c->mask && !c->mask[t]) {
    if (g) for (int64_t v = 0; v < V; ++v) g[v] = 0.0;
    c->row_loss[i] = 0.0;
    c->row_lse[i] = 0.0;
    return;
  }
  double *x = (double *)malloc(sizeof(double) * (size_t)V * 4);
  double *y = x + V, *ls = y + V, *lq = ls + V;
  for (int64_t v = 0; v < V; ++v) {
    x[v] = c->S[t * V + v] / c->T;
    y[v] = c->U[t * V + v] / c->T;
  }
  double lse_x = row_lse(x, V), lse_y = row_lse(y, V);
  for (int64_t v = 0; v < V; ++v) {
    ls[v] = x[v] - lse_x;
    lq[v] = y[v] - lse_y;
  }
  double L = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    if (c->objective == 0) L = L - exp(lq[v]) * ls[v];
    else if (c->objective == 1) L = L + exp(lq[v]) * (lq[v] - ls[v]);
    else L = L + exp(ls[v]) * (ls[v] - lq[v]);
  }
  if (g) {
    for (int64_t v = 0; v < V; ++v) {
      double pv = exp(ls[v]);
      double dldx;
      if (c->objective == 2) dldx = pv * (ls[v] - lq[v] - L);
      else dldx = pv - exp(lq[v]);
      g[v] = c->scale * (dldx + 2.0 * c->z_coef * lse_x * pv) / c->T;
    }
  }
  c->row_loss[i] = L;
  c->row_lse[i] = lse_x;
  free(x);
}

/* Full call: grad is [n_tok][vocab] (may be NULL to skip gradients);
 * out5 = {loss, z_loss, n_counted, loss_sum, z_sum}. */
int orc_distill(const double *S, const double *U, const uint8_t *mask, int64_t n_tok,
                int64_t vocab, int objective, double temperature, double z_coef,
                double grad_out, int nthreads, double *grad, double *out5) {
  if (n_tok < 1 || vocab < 1) return ORC_EMPTY_DIMENSION;
  if (n_tok > ORC_MAX_N_TOK || vocab > ORC_MAX_VOCAB) return ORC_DIMENSION_TOO_LARGE;
  if (!is_fin(z_coef) || !is_fin(grad_out) || !is_fin(temperature) || !(temperature > 0.0))
    return ORC_NON_FINITE_SCALAR;
  if (objective < 0 || objective > 2) return ORC_UNKNOWN_OBJECTIVE;
  int64_t counted = 0;
  for (int64_t t = 0; t < n_tok; ++t) counted += (!mask || mask[t]) ? 1 : 0;
  int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_tok);
  double *rl = (double *)malloc(sizeof(double) * (size_t)n_tok * 2);
  for (int64_t t = 0; t < n_tok; ++t) rows[t] = t;
  dis_ctx c;
  c.S = S; c.U = U; c.mask = mask; c.V = vocab; c.objective = objective;
  c.T = temperature; c.z_coef = z_coef;
  c.scale = counted ? grad_out / (double)counted : 0.0;
  c.rows = rows; c.grad = grad; c.row_loss = rl; c.row_lse = rl + n_tok;
  orc_parallel_for(nthreads, n_tok, dis_item, &c);
  double loss_sum = 0.0, z_sum = 0.0;
  for (int64_t t = 0; t < n_tok; ++t) {
    if (mask && !mask[t]) continue;
    loss_sum = loss_sum + c.row_loss[t];
    z_sum = z_sum + c.row_lse[t] * c.row_lse[t];
  }
  out5[0] = counted ? loss_sum / (double)counted : 0.0;
  out5[1] = counted ? z_sum / (double)counted : 0.0;
  out5[2] = (double)counted;
  out5[3] = loss_sum;
  out5[4] = z_sum;
  free(rows);
  free(rl);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Label cross-entropy with z-loss from materialized logits: the lossk       */
/* reference (ce_from_logits_flat, [P1] lossk table) with the loss mask and  */
/* the z term of [P3] ("What it does", "Changes"), forward and backward.     */
/*   lse_t = log sum_v exp(z[t][v]),  L_t = lse_t - z[t][y_t]                */
/*   dL_t/dz_v = p_v - [v == y_t],  d(lse_t^2)/dz_v = 2 lse_t p_v,           */
/*   p_v = exp(z[t][v] - lse_t)                                              */
/*   grad[t][v] = (grad_out/C) (dL_t/dz_v + z_coef d(lse_t^2)/dz_v)          */
/* loss = sum L_t / C, z_loss = sum lse_t^2 / C over counted rows; masked    */
/* rows get zeros.                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *Z;
  const int64_t *targets;
  const uint8_t *mask;
  int64_t V;
  double z_coef, scale;     /* scale = grad_out / C */
  const int64_t *rows;
  double *grad;             /* [n_rows][V] or NULL */
  double *row_loss, *row_lse;
} lbl_ctx;

static void lbl_item(void *p, int64_t i) {
  lbl_ctx *c = (lbl_ctx *)p;
  int64_t t = c->rows[i];
  int64_t V = c->V;
  double *g = c->grad ? c->grad + i * V : NULL;
  if (c->mask && !c->mask[t]) {
    if (g) for (int64_t v = 0; v < V; ++v) g[v] = 0.0;
    c->row_loss[i] = 0.0;
    c->row_lse[i] = 0.0;
    return;
  }
  const double *z = c->Z + t * V;
  int64_t y = c->targets[t];
  double lse = row_lse(z, V);
  if (g) {
    for (int64_t v = 0; v < V; ++v) {
      double pv = exp(z[v] - lse);
      double dce = pv - (v == y ? 1.0 : 0.0);
      double dz = 2.0 * lse * pv;
      g[v] = c->scale * (dce + c->z_coef * dz);
    }
  }
  c->row_loss[i] = lse - z[y];
  c->row_lse[i] = lse;
}

/* Full call: grad is [n_tok][vocab] (may be NULL to skip gradients);
 * out5 = {loss, z_loss, n_counted, loss_sum, z_sum}. */
int orc_ce_logits(const double *Z, const int64_t *targets, const uint8_t *mask, int64_t n_tok,
                  int64_t vocab, double z_coef, double grad_out, int nthreads, double *grad,
                  double *out5) {
  if (n_tok < 1 || vocab < 1) return ORC_EMPTY_DIMENSION;
  if (n_tok > ORC_MAX_N_TOK || vocab > ORC_MAX_VOCAB) return ORC_DIMENSION_TOO_LARGE;
  if (!is_fin(z_coef) || !is_fin(grad_out)) return ORC_NON_FINITE_SCALAR;
  if (!orc_targets_in_range(targets, n_tok, vocab)) return ORC_TARGET_OUT_OF_RANGE;
  int64_t counted = 0;
  for (int64_t t = 0; t < n_tok; ++t) counted += (!mask || mask[t]) ? 1 : 0;
  int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_tok);
  double *rl = (double *)malloc(sizeof(double) * (size_t)n_tok * 2);
  for (int64_t t = 0; t < n_tok; ++t) rows[t] = t;
  lbl_ctx c;
  c.Z = Z; c.targets = targets; c.mask = mask; c.V = vocab; c.z_coef = z_coef;
  c.scale = counted ? grad_out / (double)counted : 0.0;
  c.rows = rows; c.grad = grad; c.row_loss = rl; c.row_lse = rl + n_tok;
  orc_parallel_for(nthreads, n_tok, lbl_item, &c);
  double loss_sum = 0.0, z_sum = 0.0;
  for (int64_t t = 0; t < n_tok; ++t) {
    if (mask && !mask[t]) continue;
    loss_sum = loss_sum + c.row_loss[t];
    z_sum = z_sum + c.row_lse[t] * c.row_lse[t];
  }
  out5[0] = counted ? loss_sum / (double)counted : 0.0;
  out5[1] = counted ? z_sum / (double)counted : 0.0;
  out5[2] = (double)counted;
  out5[3] = loss_sum;
  out5[4] = z_sum;
  free(rows);
  free(rl);
  return ORC_OK;
}

/* Selected rows of a larger batch: Z_rows, targets_rows and mask_rows hold
 * only the listed rows; n_counted is the divisor C of the whole batch. */
int orc_ce_logits_rows(const double *Z_rows, const int64_t *targets_rows,
                       const uint8_t *mask_rows, int64_t n_rows, int64_t vocab, double z_coef,
                       double grad_out, int64_t n_counted, int nthreads, double *grad_rows,
                       double *row_loss, double *row_lse) {
  if (n_rows < 1 || vocab < 1) return ORC_EMPTY_DIMENSION;
  if (!is_fin(z_coef) || !is_fin(grad_out)) return ORC_NON_FINITE_SCALAR;
  if (!orc_targets_in_range(targets_rows, n_rows, vocab)) return ORC_TARGET_OUT_OF_RANGE;
  int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_rows);
  for (int64_t t = 0; t < n_rows; ++t) rows[t] = t;
  lbl_ctx c;
  c.Z = Z_rows; c.targets = targets_rows; c.mask = mask_rows; c.V = vocab; c.z_coef = z_coef;
  c.scale = n_counted ? grad_out / (double)n_counted : 0.0;
  c.rows = rows; c.grad = grad_rows; c.row_loss = row_loss; c.row_lse = row_lse;
  orc_parallel_for(nthreads, n_rows, lbl_item, &c);
  free(rows);
  return ORC_OK;
}

/* Selected rows only (for large shapes): grad_rows is [n_rows][vocab];
 * row_loss and row_lse receive L_t and lse(x_t) for each listed row.
 * n_counted is the divisor C of the whole batch. */
int orc_distill_rows(const double *S, const double *U, const uint8_t *mask, int64_t vocab,
                     int objective, double temperature, double z_coef, double grad_out,
                     int64_t n_counted, const int64_t *rows, int64_t n_rows, int nthreads,
                     double *grad_rows, double *row_loss, double *row_lse) {
  if (vocab < 1) return ORC_EMPTY_DIMENSION;
  if (!is_fin(z_coef) || !is_fin(grad_out) || !is_fin(temperature) || !(temperature > 0.0))
    return ORC_NON_FINITE_SCALAR;
  if (objective < 0 || objective > 2) return ORC_UNKNOWN_OBJECTIVE;
  dis_ctx c;
  c.S = S; c.U = U; c.mask = mask; c.V = vocab; c.objective = objective;
  c.T = temperature; c.z_coef = z_coef;
  c.scale = n_counted ? grad_out / (double)n_counted : 0.0;
  c.rows = rows; c.grad = grad_rows; c.row_loss = row_loss; c.row_lse = row_lse;
  orc_parallel_for(nthreads, n_rows, dis_item, &c);
  return ORC_OK;
}
