/*
 * oracle.c -- plain, slow, single-threaded float64 CPU reference for the
 * batched speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU path; both sides only see the same seeded
 * inputs.
 *
 * Pages cited (by title and section):
 *   [A] "推测解码与连续批处理深度实战：突破自回归生成的双重瓶颈"
 *       (ybb.press llm-inference), section 1.2 (数学原理) and 1.3.
 *   [B] the blog.hotdry.top post on speculative decoding and dynamic
 *       batching, part "推测解码：算法层的并行验证艺术", item 流程编排.
 *   [C] "LLM推理服务的推测解码与PagedAttention内存管理", the flow under
 *       推测解码（Speculative Decoding）原理.
 *   [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
 *       vLLM生产级实现", sections 2.1 and 2.2.
 *
 * What is computed, for every sequence b with gamma = gamma_b drafts, in the
 * pages' order:
 *   1. The target scores all gamma+1 positions at once ([A] 1.2 step 2,
 *      [C] step 2): for every target row i in [0, gamma] and draft row i in
 *      [0, gamma) the distribution softmax(l / T):
 *        z_k = l_k / T,  M = max_k z_k,  s = sum_k exp(z_k - M),
 *        p_k = exp(z_k - M) / s.
 *      The pages never define T (only an API field temperature=0.7 appears in
 *      [D] 4.2); the reading taken is the usual one, the same scalar T > 0
 *      divides the target and the draft logits.
 *   2. Accept test, positions in order ([A] 1.2 step 3, [C] step 3, [D] 2.2):
 *      draft token x_i is accepted with probability min(1, p_i(x)/q_i(x)).
 *      With the pre-drawn uniform u_i in [0, 1): accept iff u_i < r_i where
 *      r_i = p_i(x_i) / q_i(x_i) (strict, so r_i >= 1 always accepts).
 *   3. Stop at the first rejection and drop every later draft ([D] 2.1,
 *      [B] 流程编排).  n_b = the index j of the first rejection, or gamma.
 *   4. Final draw with the last uniform of the sequence:
 *        j < gamma : from norm(max(0, p_j - q_j)) ([A] 1.2 step 3 writes it
 *                    clip(p_i - q_i, 0); [D] 2.2 writes norm(max(0, p - q)));
 *        j = gamma : the bonus token, from p_gamma, the target's (gamma+1)-th
 *                    distribution (implied by the gamma+1 scored positions of
 *                    [A] 1.2 step 2 and the gamma+1 exponent of [A] 1.3 /
 *                    [C]'s expected-speed-up formula).
 *      Inverse CDF over ascending token id: w_k the weights, C_k their
 *      running sum in ascending k, S = C_{V-1}, t = u * S, and the token is
 *      the smallest k with C_k > t (never a zero-weight token).  If rounding
 *      leaves t >= C_{V-1}, the last k with w_k > 0.  In exact arithmetic a
 *      rejection has S >= q_j(x) - p_j(x) > 0; the computed S is 0 only when
 *      that difference is below the rounding of the normalisers (every other
 *      p_k then rounds to q_k).  The draw then falls back to p_j, and the
 *      sequence is flagged with an unbounded E.
 *   5. Output: out[i] = x_i for i < n_b, out[n_b] = the drawn token, and
 *      out[i] = -1 for n_b < i <= gamma, at the sequence's target-row slots.
 *
 * Arithmetic: every sum (the normalisers s, the running sum C_k) is a
 * compensated sum (Neumaier's running correction), so its rounding error is
 * a few units of the last place of the total whatever the number of terms;
 * the pages define these sums exactly, and the compensation only brings the
 * double result closer to that definition.
 *
 * Diagnostics: the distance |u_i - r_i| of every evaluated test, and for the
 * final draw min(t - C_{k-1}, C_k - t) / S.  Each computed threshold carries
 * a bound on its own rounding error (first-order propagation of the
 * per-operation bounds through z = l / T, exp(z - M), the sums, the
 * divisions and p - q): E_r for r_i, and E for every C_k / S.  A decision is
 * a tie when the uniform lies within `tie_tol` (the caller passes 1e-6) of a
 * threshold known to within that bound, i.e. when the distance is below
 * tie_tol + E; the reported distances are the guaranteed ones, the raw
 * distance minus the bound (never below 0).  A sequence is flagged when any
 * of its decisions is a tie; flag bit 3 marks a final draw whose bound E
 * exceeds a tenth of the tie window (a residual of two distributions that
 * agree to about the double rounding of their normalisers).
 *
 * Layout: packed ragged rows, cu[b] = sum of gamma_{b'} for b' < b; target
 * row of (b, i) is cu[b] + b + i, draft row is cu[b] + i; one uniform per
 * target row (gamma_b tests, then the final draw).  Logits are f32 (dtype 0)
 * or bf16 bit patterns (dtype 1); both are widened exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

/* Exact widening of one stored logit to double. */
static double load_logit(const void *base, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

#define U64 0x1p-53   /* unit roundoff of double */

/* Neumaier's compensated sum: a running total and a running correction that
 * collects what each addition rounded away. */
typedef struct {
  double hi, lo;
} csum;

static void csum_add(csum *a, double x) {
  const double t = a->hi + x;
  if (fabs(a->hi) >= fabs(x)) a->lo += (a->hi - t) + x;
  else a->lo += (x - t) + a->hi;
  a->hi = t;
}

static double csum_value(const csum *a) { return a->hi + a->lo; }

/* Bound on the relative error of one computed term exp(z - M) against the
 * exact exp((l - l_max) / T): z = l / T and M each carry one rounding, z - M
 * one more, exp less than one ulp.  The maximum's own term is exp(0) = 1
 * with no error, and a -inf logit gives exactly 0. */
static double term_err(double z, double M) {
  if (z == M || z == -INFINITY) return 0.0;
  return U64 * (fabs(z) + fabs(M) + fabs(z - M)) + 2.0 * U64;
}

/* Step 1 for one row: M = max_k l_k / T and s = sum_k exp(l_k / T - M);
 * *s_err receives a bound on the relative error of s (its terms' errors
 * plus the compensated sum's own). */
static void row_normaliser(const void *base, int dtype, int64_t row,
                           int64_t ld, int64_t vocab, double T,
                           double *M_out, double *s_out, double *s_err) {
  const int64_t off = row * ld;
  double M = -INFINITY;
  for (int64_t k = 0; k < vocab; ++k) {
    double z = load_logit(base, dtype, off + k) / T;
    if (z > M) M = z;
  }
  csum s = {0.0, 0.0};
  double err = 0.0;
  for (int64_t k = 0; k < vocab; ++k) {
    double z = load_logit(base, dtype, off + k) / T;
    const double e = exp(z - M);
    csum_add(&s, e);
    err += e * term_err(z, M);
  }
  *M_out = M;
  *s_out = csum_value(&s);
  if (s_err) *s_err = err / *s_out + 2.0 * U64 + (double)vocab * U64 * U64;
}

/* p_k of one row, given its normaliser; *rel (may be NULL) receives a bound
 * on its relative error, given the normaliser's bound s_err. */
static double prob(const void *base, int dtype, int64_t row, int64_t ld,
                   int64_t k, double T, double M, double s, double s_err,
                   double *rel) {
  const double z = load_logit(base, dtype, row * ld + k) / T;
  if (rel) *rel = term_err(z, M) + s_err + U64;
  return exp(z - M) / s;
}

/* softmax(l / T) of one row into p[0..vocab). */
int oracle_row_softmax(const void *logits, int dtype, int64_t vocab,
                       float temperature, double *p) {
  if (!logits || !p || vocab <= 0 || !(temperature > 0.0f)) return ORACLE_EINVAL;
  double M, s;
  const double T = (double)temperature;
  row_normaliser(logits, dtype, 0, vocab, vocab, T, &M, &s, NULL);
  for (int64_t k = 0; k < vocab; ++k) p[k] = prob(logits, dtype, 0, vocab, k, T, M, s, 0.0, NULL);
  return ORACLE_OK;
}

/* sum_k min(p_k, q_k) for one target row and one draft row: the probability
 * that a draft token drawn from q passes the accept test. */
double oracle_overlap_mass(const void *target_row, const void *draft_row,
                           int dtype, int64_t vocab, float temperature) {
  double Mp, sp, Mq, sq;
  const double T = (double)temperature;
  row_normaliser(target_row, dtype, 0, vocab, vocab, T, &Mp, &sp, NULL);
  row_normaliser(draft_row, dtype, 0, vocab, vocab, T, &Mq, &sq, NULL);
  csum a = {0.0, 0.0};
  for (int64_t k = 0; k < vocab; ++k) {
    double p = prob(target_row, dtype, 0, vocab, k, T, Mp, sp, 0.0, NULL);
    double q = prob(draft_row, dtype, 0, vocab, k, T, Mq, sq, 0.0, NULL);
    csum_add(&a, p < q ? p : q);
  }
  return csum_value(&a);
}

/* The inverse-CDF draw of step 4 over weights w[0..vocab) whose absolute
 * errors add up to at most w_err: C_k the compensated running sum in
 * ascending k, S = C_{V-1}, t = u * S, the token the smallest k with
 * C_k > t, else (t at or past the rounded total) the last k with w_k > 0.
 * *S_out receives S, *df_out the distance min(t - C_{k-1}, C_k - t) / S of
 * u * S to the nearest boundary of the token's interval, and *E_out a bound
 * on the error of every C_k / S (the weights' errors, twice for C_k and for
 * S, the sums' own few ulps, the rounding of t); unbounded when S = 0.
 * Returns the token, or -1 when every weight is 0. */
static int64_t inverse_cdf(const double *w, double *C, int64_t vocab, double w_err,
                           double u, double *S_out, double *df_out, double *E_out) {
  csum run = {0.0, 0.0};
  for (int64_t k = 0; k < vocab; ++k) {
    csum_add(&run, w[k]);
    C[k] = csum_value(&run);
  }
  const double S = C[vocab - 1];
  const double t = u * S;
  int64_t tok = -1;
  for (int64_t k = 0; k < vocab; ++k)
    if (C[k] > t) { tok = k; break; }
  if (tok < 0)
    for (int64_t k = vocab - 1; k >= 0; --k)
      if (w[k] > 0.0) { tok = k; break; }
  double df = 0.0;
  if (tok >= 0 && S > 0.0) {
    const double lo = tok > 0 ? C[tok - 1] : 0.0;
    df = fmin(t - lo, C[tok] - t) / S;
    if (df < 0.0) df = 0.0;
  }
  *S_out = S;
  *df_out = df;
  *E_out = S > 0.0 ? 2.0 * (w_err + (2.0 * U64 + (double)vocab * U64 * U64) * S) / S + 4.0 * U64
                   : INFINITY;
  return tok;
}

/*
 * The whole verify step.  Outputs (all caller-owned, host memory):
 *   out_tokens[R_t]          int32, n_b + 1 tokens per sequence then -1
 *   out_num_accepted[B]      int32, n_b in [0, gamma_b]
 *   out_p_draft, out_q_draft [R_d] double p_i(x_i), q_i(x_i) (may be NULL)
 *   out_residual_sum[B]      double S of norm(max(0, p - q)), 0 on the bonus
 *                            path (may be NULL)
 *   tie_accept[R_d]          double |u_i - r_i| less the bound on r_i's error
 *                            (>= 0), NaN for tests not evaluated (may be NULL)
 *   tie_final[B]             double final-draw boundary distance less the
 *                            bound E (>= 0) (may be NULL)
 *   final_err[B]             double E, the bound on the error of every C_k / S
 *                            of the final draw (may be NULL)
 *   flagged[B]               int32 bit0: an accept test within tie_tol of r_i,
 *                            bit1: the final draw within tie_tol of a
 *                            boundary, bit2: empty residual fallback, bit3:
 *                            E above tie_tol / 10 (may be NULL)
 * Returns 0, or a negative code for invalid arguments / allocation failure.
 */
int oracle_verify(int32_t num_seqs, const int32_t *cu_draft,
                  const void *target_logits, const void *draft_logits,
                  int64_t ld, int64_t vocab, int dtype,
                  const int32_t *draft_tokens, const float *uniforms,
                  float temperature, double tie_tol,
                  int32_t *out_tokens, int32_t *out_num_accepted,
                  double *out_p_draft, double *out_q_draft,
                  double *out_residual_sum, double *tie_accept,
                  double *tie_final, double *final_err, int32_t *flagged) {
  if (num_seqs < 0 || vocab <= 0 || ld < vocab || (dtype != 0 && dtype != 1) ||
      !(temperature > 0.0f) || !isfinite(temperature))
    return ORACLE_EINVAL;
  if (num_seqs == 0) return ORACLE_OK;
  if (!cu_draft || !target_logits || !uniforms || !out_tokens || !out_num_accepted)
    return ORACLE_EINVAL;
  const double T = (double)temperature;

  int64_t max_gamma = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    int64_t g = (int64_t)cu_draft[b + 1] - cu_draft[b];
    if (g < 0) return ORACLE_EINVAL;
    if (g > max_gamma) max_gamma = g;
  }
  if (max_gamma > 0 && (!draft_logits || !draft_tokens)) return ORACLE_EINVAL;

  const size_t rows = (size_t)(max_gamma + 1);
  double *Mp = malloc(sizeof(double) * rows), *sp = malloc(sizeof(double) * rows);
  double *Mq = malloc(sizeof(double) * rows), *sq = malloc(sizeof(double) * rows);
  double *ep_s = malloc(sizeof(double) * rows), *eq_s = malloc(sizeof(double) * rows);
  double *w = malloc(sizeof(double) * (size_t)vocab);
  double *C = malloc(sizeof(double) * (size_t)vocab);
  int rc = ORACLE_OK;
  if (!Mp || !sp || !Mq || !sq || !ep_s || !eq_s || !w || !C) {
    rc = ORACLE_ENOMEM;
    goto done;
  }

  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t gamma = (int64_t)cu_draft[b + 1] - cu_draft[b];
    const int64_t trow0 = (int64_t)cu_draft[b] + b; /* target row of (b, 0) */
    const int64_t drow0 = (int64_t)cu_draft[b];     /* draft row of (b, 0) */
    int32_t flag = 0;

    /* 1. normalisers of all gamma+1 target rows and gamma draft rows. */
    for (int64_t i = 0; i <= gamma; ++i)
      row_normaliser(target_logits, dtype, trow0 + i, ld, vocab, T, &Mp[i], &sp[i], &ep_s[i]);
    for (int64_t i = 0; i < gamma; ++i)
      row_normaliser(draft_logits, dtype, drow0 + i, ld, vocab, T, &Mq[i], &sq[i], &eq_s[i]);

    /* p_i(x_i), q_i(x_i) for every draft position (reported for all i). */
    for (int64_t i = 0; i < gamma; ++i) {
      const int64_t x = draft_tokens[drow0 + i];
      double p = 0.0, q = 0.0;
      if (x >= 0 && x < vocab) {
        p = prob(target_logits, dtype, trow0 + i, ld, x, T, Mp[i], sp[i], 0.0, NULL);
        q = prob(draft_logits, dtype, drow0 + i, ld, x, T, Mq[i], sq[i], 0.0, NULL);
      }
      if (out_p_draft) out_p_draft[drow0 + i] = p;
      if (out_q_draft) out_q_draft[drow0 + i] = q;
      if (tie_accept) tie_accept[drow0 + i] = NAN;
    }

    /* 2-3. accept tests in position order, stop at the first rejection. */
    int64_t j = gamma;
    for (int64_t i = 0; i < gamma; ++i) {
      const int64_t x = draft_tokens[drow0 + i];
      if (x < 0 || x >= vocab) { rc = ORACLE_EINVAL; goto done; }
      double ep, eq;
      const double p = prob(target_logits, dtype, trow0 + i, ld, x, T, Mp[i], sp[i], ep_s[i], &ep);
      const double q = prob(draft_logits, dtype, drow0 + i, ld, x, T, Mq[i], sq[i], eq_s[i], &eq);
      const double r = p / q;
      const double r_err = r * (ep + eq + U64);
      const double u = (double)uniforms[trow0 + i];
      const double d = fabs(u - r);
      if (tie_accept) tie_accept[drow0 + i] = fmax(d - r_err, 0.0);
      if (d < tie_tol + r_err) flag |= 1;
      if (!(u < r)) { j = i; break; }
    }

    /* 4. final draw weights: residual at j, or the bonus distribution, and
     *    the sum of their error bounds. */
    const int64_t tj = trow0 + j;
    double w_err = 0.0;
    for (int64_t k = 0; k < vocab; ++k) {
      double ep, eq;
      const double p = prob(target_logits, dtype, tj, ld, k, T, Mp[j], sp[j], ep_s[j], &ep);
      if (j < gamma) {
        const double q = prob(draft_logits, dtype, drow0 + j, ld, k, T, Mq[j], sq[j], eq_s[j], &eq);
        w[k] = p - q > 0.0 ? p - q : 0.0;
        w_err += p * ep + q * eq + U64 * fabs(p - q);
      } else {
        w[k] = p;
        w_err += p * ep;
      }
    }
    const double u = (double)uniforms[trow0 + gamma];
    double S, df, E;
    int64_t tok = inverse_cdf(w, C, vocab, w_err, u, &S, &df, &E);
    const double S_reported = (j < gamma) ? S : 0.0;
    if (!(S > 0.0)) { /* empty residual (rounding only): draw from p_j instead */
      flag |= 4;
      w_err = 0.0;
      for (int64_t k = 0; k < vocab; ++k) {
        double ep;
        w[k] = prob(target_logits, dtype, tj, ld, k, T, Mp[j], sp[j], ep_s[j], &ep);
        w_err += w[k] * ep;
      }
      double E_p;
      tok = inverse_cdf(w, C, vocab, w_err, u, &S, &df, &E_p);
      E = INFINITY;   /* the residual itself is below the oracle's resolution */
    }
    if (df < tie_tol + E) flag |= 2;
    if (E > 0.1 * tie_tol) flag |= 8;

    /* 5. outputs at the sequence's target-row slots. */
    for (int64_t i = 0; i <= gamma; ++i) {
      int32_t v;
      if (i < j) v = draft_tokens[drow0 + i];
      else if (i == j) v = (int32_t)tok;
      else v = -1;
      out_tokens[trow0 + i] = v;
    }
    out_num_accepted[b] = (int32_t)j;
    if (out_residual_sum) out_residual_sum[b] = S_reported;
    if (tie_final) tie_final[b] = fmax(df - E, 0.0);
    if (final_err) final_err[b] = E;
    if (flagged) flagged[b] = flag;
  }
done:
  free(Mp); free(sp); free(Mq); free(sq); free(ep_s); free(eq_s); free(w); free(C);
  return rc;
}

/*
 * Greedy verification ([B] 流程编排: candidates are compared with the
 * target's choice in order; at the first mismatch the matching prefix is
 * kept and decoding restarts there).  With T -> 0 the target's choice at a
 * position is the argmax of its logits; ties go to the lowest token id.
 * The token emitted at the first mismatch is the target's argmax there; when
 * every draft matches, the bonus is the argmax of the (gamma+1)-th row.
 * out_argmax (optional, [R_t]) receives each target row's argmax.
 */
static int64_t row_argmax(const void *base, int dtype, int64_t row, int64_t ld,
                          int64_t vocab) {
  const int64_t off = row * ld;
  int64_t best = 0;
  double bv = load_logit(base, dtype, off);
  for (int64_t k = 1; k < vocab; ++k) {
    const double v = load_logit(base, dtype, off + k);
    if (v > bv) { bv = v; best = k; }
  }
  return best;
}

int oracle_verify_greedy(int32_t num_seqs, const int32_t *cu_draft,
                         const void *target_logits, int64_t ld, int64_t vocab,
                         int dtype, const int32_t *draft_tokens,
                         int32_t *out_tokens, int32_t *out_num_accepted,
                         int32_t *out_argmax) {
  if (num_seqs < 0 || vocab <= 0 || ld < vocab || (dtype != 0 && dtype != 1))
    return ORACLE_EINVAL;
  if (num_seqs == 0) return ORACLE_OK;
  if (!cu_draft || !target_logits || !out_tokens || !out_num_accepted)
    return ORACLE_EINVAL;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t gamma = (int64_t)cu_draft[b + 1] - cu_draft[b];
    const int64_t trow0 = (int64_t)cu_draft[b] + b;
    const int64_t drow0 = (int64_t)cu_draft[b];
    if (gamma < 0 || (gamma > 0 && !draft_tokens)) return ORACLE_EINVAL;
    int64_t j = gamma;
    for (int64_t i = 0; i <= gamma; ++i) {
      const int64_t a = row_argmax(target_logits, dtype, trow0 + i, ld, vocab);
      if (out_argmax) out_argmax[trow0 + i] = (int32_t)a;
    }
    for (int64_t i = 0; i < gamma; ++i) {
      const int64_t x = draft_tokens[drow0 + i];
      if (x < 0 || x >= vocab) return ORACLE_EINVAL;
      if (x != row_argmax(target_logits, dtype, trow0 + i, ld, vocab)) { j = i; break; }
    }
    for (int64_t i = 0; i <= gamma; ++i) {
      int32_t v;
      if (i < j) v = draft_tokens[drow0 + i];
      else if (i == j) v = (int32_t)row_argmax(target_logits, dtype, trow0 + j, ld, vocab);
      else v = -1;
      out_tokens[trow0 + i] = v;
    }
    out_num_accepted[b] = (int32_t)j;
  }
  return ORACLE_OK;
}

/*
 * Verification of a deterministic draft (the draft proposes tokens without a
 * distribution, as n-gram / prompt-lookup drafting does: [A] 1.4 and 3.3,
 * [D] 4.1).
 * The draft distribution is then the point mass q = delta_x, so the general
 * rule specialises to: accept x with probability min(1, p(x) / 1) = p(x), and
 * on rejection resample from norm(max(0, p - delta_x)) = p with x removed and
 * renormalised.  Same layout, uniforms, draw convention and diagnostics as
 * oracle_verify; there are no draft logits.  out_q_draft is 1.
 */
int oracle_verify_onehot(int32_t num_seqs, const int32_t *cu_draft,
                         const void *target_logits, int64_t ld, int64_t vocab,
                         int dtype, const int32_t *draft_tokens,
                         const float *uniforms, float temperature, double tie_tol,
                         int32_t *out_tokens, int32_t *out_num_accepted,
                         double *out_p_draft, double *out_residual_sum,
                         double *tie_accept, double *tie_final, double *final_err,
                         int32_t *flagged) {
  if (num_seqs < 0 || vocab <= 0 || ld < vocab || (dtype != 0 && dtype != 1) ||
      !(temperature > 0.0f) || !isfinite(temperature))
    return ORACLE_EINVAL;
  if (num_seqs == 0) return ORACLE_OK;
  if (!cu_draft || !target_logits || !uniforms || !out_tokens || !out_num_accepted)
    return ORACLE_EINVAL;
  const double T = (double)temperature;
  int64_t max_gamma = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t g = (int64_t)cu_draft[b + 1] - cu_draft[b];
    if (g < 0) return ORACLE_EINVAL;
    if (g > max_gamma) max_gamma = g;
  }
  if (max_gamma > 0 && !draft_tokens) return ORACLE_EINVAL;
  const size_t rows = (size_t)(max_gamma + 1);
  double *Mp = malloc(sizeof(double) * rows), *sp = malloc(sizeof(double) * rows);
  double *ep_s = malloc(sizeof(double) * rows);
  double *w = malloc(sizeof(double) * (size_t)vocab);
  double *C = malloc(sizeof(double) * (size_t)vocab);
  int rc = ORACLE_OK;
  if (!Mp || !sp || !ep_s || !w || !C) {
    rc = ORACLE_ENOMEM;
    goto done;
  }
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t gamma = (int64_t)cu_draft[b + 1] - cu_draft[b];
    const int64_t trow0 = (int64_t)cu_draft[b] + b;
    const int64_t drow0 = (int64_t)cu_draft[b];
    int32_t flag = 0;
    for (int64_t i = 0; i <= gamma; ++i)
      row_normaliser(target_logits, dtype, trow0 + i, ld, vocab, T, &Mp[i], &sp[i], &ep_s[i]);
    for (int64_t i = 0; i < gamma; ++i) {
      const int64_t x = draft_tokens[drow0 + i];
      if (x < 0 || x >= vocab) { rc = ORACLE_EINVAL; goto done; }
      if (out_p_draft)
        out_p_draft[drow0 + i] = prob(target_logits, dtype, trow0 + i, ld, x, T, Mp[i], sp[i], 0.0, NULL);
      if (tie_accept) tie_accept[drow0 + i] = NAN;
    }
    /* accept with probability p(x): u < p(x) / q(x) with q(x) = 1 */
    int64_t j = gamma;
    for (int64_t i = 0; i < gamma; ++i) {
      const int64_t x = draft_tokens[drow0 + i];
      double ep;
      const double px = prob(target_logits, dtype, trow0 + i, ld, x, T, Mp[i], sp[i], ep_s[i], &ep) / 1.0;
      const double px_err = px * ep;
      const double u = (double)uniforms[trow0 + i];
      const double d = fabs(u - px);
      if (tie_accept) tie_accept[drow0 + i] = fmax(d - px_err, 0.0);
      if (d < tie_tol + px_err) flag |= 1;
      if (!(u < px)) { j = i; break; }
    }
    /* residual max(0, p - delta_x): p with x removed; or the bonus row p */
    const int64_t tj = trow0 + j;
    double w_err = 0.0;
    for (int64_t k = 0; k < vocab; ++k) {
      double ep;
      const double p = prob(target_logits, dtype, tj, ld, k, T, Mp[j], sp[j], ep_s[j], &ep);
      if (j < gamma) {
        const double q = (k == draft_tokens[drow0 + j]) ? 1.0 : 0.0;
        w[k] = p - q > 0.0 ? p - q : 0.0;
        w_err += p * ep + U64 * fabs(p - q);
      } else {
        w[k] = p;
        w_err += p * ep;
      }
    }
    const double u = (double)uniforms[trow0 + gamma];
    double S, df, E;
    int64_t tok = inverse_cdf(w, C, vocab, w_err, u, &S, &df, &E);
    const double S_reported = (j < gamma) ? S : 0.0;
    if (!(S > 0.0)) {   /* p(x) = 1: draw from p_j instead */
      flag |= 4;
      w_err = 0.0;
      for (int64_t k = 0; k < vocab; ++k) {
        double ep;
        w[k] = prob(target_logits, dtype, tj, ld, k, T, Mp[j], sp[j], ep_s[j], &ep);
        w_err += w[k] * ep;
      }
      double E_p;
      tok = inverse_cdf(w, C, vocab, w_err, u, &S, &df, &E_p);
      E = INFINITY;
    }
    if (df < tie_tol + E) flag |= 2;
    if (E > 0.1 * tie_tol) flag |= 8;
    for (int64_t i = 0; i <= gamma; ++i) {
      int32_t v;
      if (i < j) v = draft_tokens[drow0 + i];
      else if (i == j) v = (int32_t)tok;
      else v = -1;
      out_tokens[trow0 + i] = v;
    }
    out_num_accepted[b] = (int32_t)j;
    if (out_residual_sum) out_residual_sum[b] = S_reported;
    if (tie_final) tie_final[b] = fmax(df - E, 0.0);
    if (final_err) final_err[b] = E;
    if (flagged) flagged[b] = flag;
  }
done:
  free(Mp); free(sp); free(ep_s); free(w); free(C);
  return rc;
}

/*
 * Tree verification.  "大模型推理加速新范式" section 3.2 (Tree Attention): the
 * draft proposes several candidates per position, forming a tree, and the
 * target scores every node of the tree in one pass, so that at least one
 * path is more likely to be accepted.  The page gives no acceptance rule for
 * a tree; the readings taken here are the plainest ones the rest of the
 * pages support:
 *   greedy (T -> 0):   from the root, move to the lowest-index child whose
 *                      token is the argmax of the current node's row ([B]
 *                      流程编排: compare with the target's choice); stop when
 *                      no child matches and emit that argmax.
 *   point candidates:  candidates carry no distribution (top-k proposals),
 *                      so each is a point mass.  The children of the current
 *                      node are tried in index order; child c is accepted
 *                      with probability p'(x_c), where p' is the current
 *                      node's p with the tokens of already rejected siblings
 *                      removed and renormalised (the residual of the point
 *                      rule, applied after each rejection); a token already
 *                      rejected has p' = 0.  After every child is rejected,
 *                      or at a node without children, the final token is
 *                      drawn from p' (p itself when nothing was rejected).
 *                      Each token then has exactly probability p_k of being
 *                      emitted at each depth.
 * Layout, per sequence b with N_b >= 1 nodes at global rows
 * g = cu_nodes[b] + n, n in [0, N_b): node 0 is the root (the last
 * committed token); parent[g] is the local index of node n's parent
 * (0 <= parent < n for n >= 1); tokens[g] its token (ignored for the root);
 * target row g is the target's distribution of the token after node n;
 * uniforms[g] is node n's accept test (n >= 1) and the root's slot holds the
 * final draw.  Outputs at the sequence's N_b slots: out_tokens = the accepted
 * nodes' tokens, then the final token, then -1; out_path = the accepted
 * nodes' local indices, then -1; out_num_accepted = the accepted depth.
 */
static int tree_geometry_ok(int32_t num_seqs, const int32_t *cu, const int32_t *parent,
                            const int32_t *tokens, int64_t vocab, int need_tokens) {
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t g0 = cu[b], N = (int64_t)cu[b + 1] - cu[b];
    if (N < 1) return 0;
    for (int64_t n = 1; n < N; ++n) {
      const int32_t pn = parent[g0 + n];
      if (pn < 0 || pn >= n) return 0;
      if (need_tokens && (tokens[g0 + n] < 0 || tokens[g0 + n] >= vocab)) return 0;
    }
  }
  return 1;
}

int oracle_verify_tree_greedy(int32_t num_seqs, const int32_t *cu_nodes, const int32_t *parent,
                              const int32_t *tokens, const void *target_logits, int64_t ld,
                              int64_t vocab, int dtype, int32_t *out_tokens, int32_t *out_path,
                              int32_t *out_num_accepted) {
  if (num_seqs < 0 || vocab <= 0 || ld < vocab || (dtype != 0 && dtype != 1))
    return ORACLE_EINVAL;
  if (num_seqs == 0) return ORACLE_OK;
  if (!cu_nodes || !parent || !tokens || !target_logits || !out_tokens || !out_path ||
      !out_num_accepted)
    return ORACLE_EINVAL;
  if (!tree_geometry_ok(num_seqs, cu_nodes, parent, tokens, vocab, 1)) return ORACLE_EINVAL;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t g0 = cu_nodes[b], N = (int64_t)cu_nodes[b + 1] - cu_nodes[b];
    for (int64_t n = 0; n < N; ++n) {
      out_tokens[g0 + n] = -1;
      out_path[g0 + n] = -1;
    }
    int64_t cur = 0, depth = 0;
    for (;;) {
      const int64_t a = row_argmax(target_logits, dtype, g0 + cur, ld, vocab);
      int64_t next = -1;
      for (int64_t n = cur + 1; n < N; ++n)
        if (parent[g0 + n] == cur && tokens[g0 + n] == a) { next = n; break; }
      out_tokens[g0 + depth] = (int32_t)a;
      if (next < 0) break;
      out_path[g0 + depth] = (int32_t)next;
      ++depth;
      cur = next;
    }
    out_num_accepted[b] = (int32_t)depth;
  }
  return ORACLE_OK;
}

int oracle_verify_tree_point(int32_t num_seqs, const int32_t *cu_nodes, const int32_t *parent,
                             const int32_t *tokens, const void *target_logits, int64_t ld,
                             int64_t vocab, int dtype, const float *uniforms, float temperature,
                             double tie_tol, int32_t *out_tokens, int32_t *out_path,
                             int32_t *out_num_accepted, double *out_tie, int32_t *flagged) {
  if (num_seqs < 0 || vocab <= 0 || ld < vocab || (dtype != 0 && dtype != 1) ||
      !(temperature > 0.0f) || !isfinite(temperature))
    return ORACLE_EINVAL;
  if (num_seqs == 0) return ORACLE_OK;
  if (!cu_nodes || !parent || !tokens || !target_logits || !uniforms || !out_tokens ||
      !out_path || !out_num_accepted)
    return ORACLE_EINVAL;
  if (!tree_geometry_ok(num_seqs, cu_nodes, parent, tokens, vocab, 1)) return ORACLE_EINVAL;
  const double T = (double)temperature;
  double *p = malloc(sizeof(double) * (size_t)vocab);
  double *w = malloc(sizeof(double) * (size_t)vocab);
  double *C = malloc(sizeof(double) * (size_t)vocab);
  unsigned char *removed = calloc((size_t)vocab, 1);
  if (!p || !w || !C || !removed) { free(p); free(w); free(C); free(removed); return ORACLE_ENOMEM; }
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t g0 = cu_nodes[b], N = (int64_t)cu_nodes[b + 1] - cu_nodes[b];
    for (int64_t n = 0; n < N; ++n) {
      out_tokens[g0 + n] = -1;
      out_path[g0 + n] = -1;
    }
    int32_t flag = 0;
    double tie = INFINITY;
    int64_t cur = 0, depth = 0;
    for (;;) {
      /* the current node's p */
      double M, s, s_err;
      row_normaliser(target_logits, dtype, g0 + cur, ld, vocab, T, &M, &s, &s_err);
      for (int64_t k = 0; k < vocab; ++k)
        p[k] = prob(target_logits, dtype, g0 + cur, ld, k, T, M, s, 0.0, NULL);
      /* its children in index order, each a point-mass candidate */
      int any_removed = 0;
      int64_t next = -1;
      for (int64_t n = cur + 1; n < N && next < 0; ++n) {
        if (parent[g0 + n] != cur) continue;
        const int64_t x = tokens[g0 + n];
        double r;
        if (removed[x]) {
          r = 0.0;                     /* already rejected: p'(x) = 0 */
        } else if (!any_removed) {
          r = p[x];                    /* nothing removed yet: p' = p */
        } else {
          csum rest = {0.0, 0.0};      /* mass of the tokens not removed */
          for (int64_t k = 0; k < vocab; ++k)
            if (!removed[k]) csum_add(&rest, p[k]);
          r = p[x] / csum_value(&rest);
        }
        const double u = (double)uniforms[g0 + n];
        const double d = fabs(u - r);
        if (d < tie) tie = d;
        if (d < tie_tol) flag |= 1;
        if (u < r) {
          next = n;
        } else {
          removed[x] = 1;
          any_removed = 1;
        }
      }
      if (next >= 0) {
        for (int64_t n = cur + 1; n < N; ++n)    /* the next level starts afresh */
          if (parent[g0 + n] == cur) removed[tokens[g0 + n]] = 0;
        out_tokens[g0 + depth] = tokens[g0 + next];
        out_path[g0 + depth] = (int32_t)next;
        ++depth;
        cur = next;
        continue;
      }
      /* final draw from p without the rejected tokens (each weight p_k
       * carries the relative error bound of its row) */
      double w_err = 0.0;
      for (int64_t k = 0; k < vocab; ++k) {
        double ek;
        prob(target_logits, dtype, g0 + cur, ld, k, T, M, s, s_err, &ek);
        w[k] = removed[k] ? 0.0 : p[k];
        w_err += w[k] * ek;
      }
      const double u = (double)uniforms[g0];
      double S, df, E;
      int64_t tok = inverse_cdf(w, C, vocab, w_err, u, &S, &df, &E);
      if (!(S > 0.0)) {
        flag |= 4;
        tok = inverse_cdf(p, C, vocab, 0.0, u, &S, &df, &E);
      }
      if (tok >= 0) {
        if (df < tie) tie = df;
        if (df < tie_tol + E) flag |= 2;
      }
      out_tokens[g0 + depth] = (int32_t)tok;
      for (int64_t n = 1; n < N; ++n) removed[tokens[g0 + n]] = 0;
      break;
    }
    out_num_accepted[b] = (int32_t)depth;
    if (out_tie) out_tie[b] = tie;
    if (flagged) flagged[b] = flag;
  }
  free(p); free(w); free(C); free(removed);
  return ORACLE_OK;
}
