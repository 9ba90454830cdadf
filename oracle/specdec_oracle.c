/*
 * specdec_oracle.c -- CPU reference for the speculative-decoding verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the GPU library, and it never calls into it.
 *
 * Plain, single-threaded and slow on purpose: every function is a direct
 * transcription of the definition it cites, with no blocking, fusion or
 * reordering, so that it can be checked against the pages by eye.
 *
 * Sources (cited by title and section; the pages are four web articles):
 *   [LLMI]  "LLM Inference & Speculative Decoding: From Roofline Physics to
 *            Lossless Acceleration" (arman1o1.github.io)
 *   [MATH]  "Speculative Decoding: Mathematical Foundations, Distribution
 *            Preservation Proofs, Tree-Structured Verification, and
 *            Memory-Bandwidth Amortization" (llms.blog)
 *   [LESS]  "Speculative decoding." lesson (gtadkapally.com, learn-cs)
 *   [PREP]  "Speculative Decoding: Draft, Verify, Accept" (vanos001.github.io)
 *
 * Precision.  fp64 throughout, except where the pages fix fp32: for T > 0 the
 * target and draft probabilities p and q, the residual (p - q)+ and the ratio
 * p/q are fp32 values ([LLMI] section 4, failure mode 1: compute p, q and
 * (p - q)+ in FP32).  Here they are computed in fp64 and rounded once to fp32.
 * Normalisers (max, sum of exponentials) and every cumulative sum are fp64.
 *
 * Planted mistakes.  Compiling with -DORACLE_PLANT=<n> (n > 0) builds a
 * deliberately wrong variant; the negative-control tests use these to show
 * that the pins catch each kind of mistake.  The default build has none.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif
/* Planted-mistake catalogue (test builds only). */
#define PLANT_RESAMPLE_FROM_P 1   /* on reject, draw from p instead of (p-q)+  */
#define PLANT_RESIDUAL_SIGN 2     /* residual (q-p)+ instead of (p-q)+         */
#define PLANT_NO_BONUS 3          /* all accepted: no bonus token             */
#define PLANT_TEMP_MULTIPLY 4     /* logits * T instead of logits / T         */
#define PLANT_LINEAR_TRANSPOSE 5  /* W read as [d, V] instead of [V, d]       */
#define PLANT_UNIFORM_SLOTS 6     /* accept/sample uniform slots swapped      */
#define PLANT_DRAW_LE 7           /* inverse CDF with <= instead of <         */
#define PLANT_ARGMAX_LAST_TIE 8   /* ties resolved to the highest index       */
#define PLANT_GREEDY_KEEP_DRAFT 9 /* greedy mismatch emits the draft token    */
#define PLANT_RATIO_INVERTED 10   /* accept with q/p instead of p/q           */
#define PLANT_NO_MAX_SHIFT 11     /* softmax without subtracting the max      */
#define PLANT_ROW_OFFSET 12       /* draft row i+1 paired with target row i   */
#define PLANT_DROP_LAST_TERM 13   /* dot product drops the last k term        */
#define PLANT_ACCEPT_LE 14        /* accept when u <= ratio (boundary)        */
#define PLANT_TREE_DEPTH 15       /* tree depth counts the root as depth 1    */
#define PLANT_TREE_SELF_ARGMAX 16 /* tree node checked against its own row    */
#define PLANT_KV_FREE_ORDER 17    /* rollback frees blocks front to back      */
#define PLANT_KV_OFFSET 18        /* in-block offset taken as t / block_size  */
#define PLANT_TOPK_TIE_HIGH 19    /* top-k ties broken towards higher indices */
#define PLANT_TOPP_STRICT 20      /* top-p stops only when the mass exceeds p */

/* The draft is given either as logits (softmax at temperature T) or as
 * probabilities used as given. */
#define ORACLE_Q_LOGITS 0
#define ORACLE_Q_PROBS 1
/* The draft is the one-hot distribution at the drafted token: a greedy draft,
 * or prompt lookup ([LESS] "Where drafts come from": a lookup draft's q is
 * one-hot; "Why the output is exactly p": so is a greedy draft's). */
#define ORACLE_Q_ONEHOT 2

/* q is clamped below at this value before dividing ([LLMI] section 2 listing). */
static const float Q_FLOOR = 1e-12f;

/* bf16 holds the upper 16 bits of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Scoring: the linear layer Y = X W of [LLMI] section 0 (roofline of a linear
 * layer over N tokens) and [MATH] "Prefill vs. Verification Arithmetic
 * Intensity": one pass scores all gamma+1 positions.  X is [N, d] row-major,
 * W is stored [V, d] row-major (one output row per vocabulary entry), so
 * Y[n][v] = sum_k X[n][k] * W[v][k].  Products of two bf16 values are exact
 * in fp64; the sum runs over k in order in fp64. */
static double dot_row(const uint16_t* x, const uint16_t* W, int64_t v, int64_t d, int64_t V) {
  double s = 0.0;
  int64_t kend = d;
#if ORACLE_PLANT == PLANT_DROP_LAST_TERM
  kend = d - 1;
#endif
  for (int64_t k = 0; k < kend; ++k) {
#if ORACLE_PLANT == PLANT_LINEAR_TRANSPOSE
    double w = bf16_value(W[k * V + v]);
#else
    (void)V;
    double w = bf16_value(W[v * d + k]);
#endif
    s += bf16_value(x[k]) * w;
  }
  return s;
}

void oracle_linear(const uint16_t* X, const uint16_t* W, int64_t N, int64_t d, int64_t V, double* Y) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t v = 0; v < V; ++v) Y[n * V + v] = dot_row(X + n * d, W, v, d, V);
}

/* Individual entries Y[n_idx[i]][v_idx[i]], for sampled checks at full size. */
void oracle_linear_entries(const uint16_t* X, const uint16_t* W, int64_t d, int64_t V, const int64_t* n_idx,
                           const int64_t* v_idx, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = dot_row(X + n_idx[i] * d, W, v_idx[i], d, V);
}

/* ------------------------------------------------------------------------ */
/* Temperature softmax ([LESS] "First: what an output distribution is": the
 * logits are divided by T, exponentiated and divided by their total).  The
 * maximum is subtracted first, which leaves the result unchanged in exact
 * arithmetic and keeps exp() finite.  Output p[v] is fp32 (see header);
 * *m_out and *Z_out receive the fp64 max and normaliser. */
void oracle_softmax(const float* z, int64_t V, double T, float* p, double* m_out, double* Z_out) {
  double m = -INFINITY;
  for (int64_t v = 0; v < V; ++v) {
#if ORACLE_PLANT == PLANT_TEMP_MULTIPLY
    double a = (double)z[v] * T;
#else
    double a = (double)z[v] / T;
#endif
    if (a > m) m = a;
  }
#if ORACLE_PLANT == PLANT_NO_MAX_SHIFT
  m = 0.0;
#endif
  double Z = 0.0;
  for (int64_t v = 0; v < V; ++v) {
#if ORACLE_PLANT == PLANT_TEMP_MULTIPLY
    double a = (double)z[v] * T;
#else
    double a = (double)z[v] / T;
#endif
    Z += exp(a - m);
  }
  for (int64_t v = 0; v < V; ++v) {
#if ORACLE_PLANT == PLANT_TEMP_MULTIPLY
    double a = (double)z[v] * T;
#else
    double a = (double)z[v] / T;
#endif
    p[v] = (float)(exp(a - m) / Z);
  }
  if (m_out) *m_out = m;
  if (Z_out) *Z_out = Z;
}

/* Greedy pick ([LESS] "First: what an output distribution is": greedy takes the
 * largest entry).  Ties go to the lowest index.  *gap_out receives the
 * distance between the largest value and the largest value at any other
 * index (0 on a tie), which measures how close the decision was. */
int64_t oracle_argmax(const float* z, int64_t V, double* gap_out) {
  int64_t best = 0;
  for (int64_t v = 1; v < V; ++v) {
#if ORACLE_PLANT == PLANT_ARGMAX_LAST_TIE
    if (z[v] >= z[best]) best = v;
#else
    if (z[v] > z[best]) best = v;
#endif
  }
  if (gap_out) {
    double second = -INFINITY;
    for (int64_t v = 0; v < V; ++v)
      if (v != best && (double)z[v] > second) second = (double)z[v];
    *gap_out = (V > 1) ? (double)z[best] - second : INFINITY;
  }
  return best;
}

/* ------------------------------------------------------------------------ */
/* The acceptance rule ([LLMI] section 2, "Speculative Acceptance Rule";
 * [MATH] "The Modified Rejection Sampling Algorithm"; [PREP] "The
 * rejection-sampling correctness argument"): keep the drafted token x with
 * probability min(1, p(x)/q(x)).  With a uniform u in [0, 1) this is the
 * event u < min(1, p(x)/q(x)) (strict, as in the [LLMI] listing and the
 * [PREP] demo).  q(x) is floored at 1e-12 before dividing.  The ratio is an
 * fp32 value.  *margin receives |u - ratio|, the distance of the decision
 * from its threshold. */
int oracle_accept(float p_x, float q_x, float u, double* margin) {
#if ORACLE_PLANT == PLANT_RATIO_INVERTED
  float pp = p_x > Q_FLOOR ? p_x : Q_FLOOR;
  float ratio = q_x / pp;
#else
  float qq = q_x > Q_FLOOR ? q_x : Q_FLOOR;
  float ratio = p_x / qq;
#endif
  if (margin) *margin = fabs((double)u - (double)ratio);
  float thr = ratio < 1.0f ? ratio : 1.0f;
#if ORACLE_PLANT == PLANT_ACCEPT_LE
  return u <= thr;
#else
  return u < thr;
#endif
}

/* Residual distribution ([LLMI] section 2; [MATH] "The Modified Rejection
 * Sampling Algorithm"; [LESS] "The acceptance rule"): r(v) = max(0, p(v) -
 * q(v)), to be normalised by its total.  r[v] is an fp32 value; the return
 * value is the fp64 total S = sum_v r[v], which equals 1 - alpha in exact
 * arithmetic. */
double oracle_residual(const float* p, const float* q, int64_t V, float* r) {
  double S = 0.0;
  for (int64_t v = 0; v < V; ++v) {
#if ORACLE_PLANT == PLANT_RESIDUAL_SIGN
    float d = q[v] - p[v];
#else
    float d = p[v] - q[v];
#endif
    r[v] = d > 0.0f ? d : 0.0f;
    S += (double)r[v];
  }
  return S;
}

/* Categorical draw by inverse CDF ([LESS] "First: what an output distribution
 * is": lay the probabilities end to end, draw a uniform, take the slice it
 * lands in; [PREP] demo `sample`).  The weights w need not be normalised: with
 * S = sum_v w[v] and C_v = sum_{j <= v} w[j] (fp64, in vocabulary order), the
 * result is the smallest v with u*S < C_v.  A zero-weight entry is therefore
 * never chosen.  If rounding leaves no such v, the largest v with w[v] > 0 is
 * taken.  Returns -1 when S == 0.  *margin receives min(t - C_{v-1}, C_v - t)/S
 * with t = u*S: the normalised distance of the draw from the nearest slice
 * edge; *mass receives S. */
int64_t oracle_draw(const float* w, int64_t V, float u, double* margin, double* mass) {
  double S = 0.0;
  for (int64_t v = 0; v < V; ++v) S += (double)w[v];
  if (mass) *mass = S;
  if (!(S > 0.0)) {
    if (margin) *margin = INFINITY;
    return -1;
  }
  double t = (double)u * S;
  double C = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    double prev = C;
    C += (double)w[v];
#if ORACLE_PLANT == PLANT_DRAW_LE
    int hit = t <= C;
#else
    int hit = t < C;
#endif
    if (hit) {
      if (margin) {
        double a = t - prev, b = C - t;
        *margin = (a < b ? a : b) / S;
      }
      return v;
    }
  }
  int64_t last = V - 1;
  while (last > 0 && !(w[last] > 0.0f)) --last;
  if (margin) *margin = 0.0;
  return last;
}

/* ------------------------------------------------------------------------ */
/* One verification step for one sequence, given probability rows.
 *   p:      [gamma+1, V] target probabilities (row i scores the position after
 *           the i-th draft token; row gamma is the bonus row)
 *   q:      [gamma, V] draft probabilities
 *   x:      [gamma] drafted token ids
 *   u:      [gamma+1, 2] uniforms: u[i][0] decides the accept test at row i,
 *           u[i][1] drives the draw if row i is the row where the step ends
 *   tokens: [gamma+1] output, -1 beyond the emitted count
 * Returns the number of emitted tokens (1 .. gamma+1).
 * The test runs left to right and stops at the first rejection ([LLMI]
 * section 2 listing; [MATH] "The Modified Rejection Sampling Algorithm";
 * [LESS] "Draft, then verify").  A rejection at row i emits a draw from the
 * residual (falling back to p when the residual has no mass, as the [PREP]
 * demo does); if all gamma are kept, a bonus token is drawn from row gamma.
 * accept_margin[i] (rows that were tested; others untouched) and *draw_margin
 * record how close each decision was. */
static int verify_one_probs(const float* p, const float* q, const int32_t* x, const float* u, int64_t gamma,
                            int64_t V, float* scratch, int32_t* tokens, double* accept_margin,
                            double* draw_margin, double* draw_mass) {
  int64_t slot_acc = 0, slot_smp = 1;
#if ORACLE_PLANT == PLANT_UNIFORM_SLOTS
  slot_acc = 1;
  slot_smp = 0;
#endif
  for (int64_t i = 0; i <= gamma; ++i) tokens[i] = -1;
  for (int64_t i = 0; i < gamma; ++i) {
    const float* pi = p + i * V;
#if ORACLE_PLANT == PLANT_ROW_OFFSET
    const float* qi = q + ((i + 1 < gamma) ? i + 1 : i) * V;
#else
    const float* qi = q + i * V;
#endif
    int64_t xi = x[i];
    double am = 0.0;
    int keep = oracle_accept(pi[xi], qi[xi], u[i * 2 + slot_acc], &am);
    if (accept_margin) accept_margin[i] = am;
    if (keep) {
      tokens[i] = (int32_t)xi;
      continue;
    }
    double S;
#if ORACLE_PLANT == PLANT_RESAMPLE_FROM_P
    memcpy(scratch, pi, (size_t)V * sizeof(float));
    S = 1.0;
#else
    S = oracle_residual(pi, qi, V, scratch);
#endif
    const float* w = (S > 0.0) ? scratch : pi;
    double dm = 0.0;
    double dS = 0.0;
    tokens[i] = (int32_t)oracle_draw(w, V, u[i * 2 + slot_smp], &dm, &dS);
    if (draw_margin) *draw_margin = dm;
    if (draw_mass) *draw_mass = dS;
    return (int)(i + 1);
  }
#if ORACLE_PLANT == PLANT_NO_BONUS
  if (draw_margin) *draw_margin = INFINITY;
  if (draw_mass) *draw_mass = 0.0;
  return (int)gamma;
#else
  double dm = 0.0, dS = 0.0;
  tokens[gamma] = (int32_t)oracle_draw(p + gamma * V, V, u[gamma * 2 + slot_smp], &dm, &dS);
  if (draw_margin) *draw_margin = dm;
  if (draw_mass) *draw_mass = dS;
  return (int)(gamma + 1);
#endif
}

/* Batched step on probability rows: p [B, gamma+1, V], q [B, gamma, V],
 * x [B, gamma], u [B, gamma+1, 2]; outputs tokens [B, gamma+1] (-1 padded),
 * num_emitted [B], optional accept_margin [B, gamma] (NaN where untested),
 * draw_margin [B] and draw_mass [B] (total weight S of the distribution the
 * last token was drawn from).  scratch must hold V floats.  Returns 0, or -1
 * on a draft token outside [0, V). */
int oracle_verify_probs(const float* p, const float* q, const int32_t* x, const float* u, int64_t B, int64_t gamma,
                        int64_t V, float* scratch, int32_t* tokens, int32_t* num_emitted, double* accept_margin,
                        double* draw_margin, double* draw_mass) {
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < gamma; ++i)
      if (x[b * gamma + i] < 0 || x[b * gamma + i] >= V) return -1;
  for (int64_t b = 0; b < B; ++b) {
    if (accept_margin)
      for (int64_t i = 0; i < gamma; ++i) accept_margin[b * gamma + i] = NAN;
    num_emitted[b] = verify_one_probs(p + b * (gamma + 1) * V, q + b * gamma * V, x + b * gamma,
                                      u + b * (gamma + 1) * 2, gamma, V, scratch, tokens + b * (gamma + 1),
                                      accept_margin ? accept_margin + b * gamma : 0,
                                      draw_margin ? draw_margin + b : 0, draw_mass ? draw_mass + b : 0);
  }
  return 0;
}

/* Greedy step (T = 0) for one sequence ([LLMI] section 4, failure mode 1;
 * [MATH] "Greedy Decoding Equivalence"; [LESS] "The acceptance rule", greedy
 * case): g_i = argmax of target row i; drafted x_i is kept iff x_i == g_i; the
 * first mismatch emits g_i and ends the step; if all match, the bonus is
 * g_gamma.  accept_margin[i] and *draw_margin hold the top-2 logit gap of the
 * rows that decided. */
static int verify_one_greedy(const float* z, const int32_t* x, int64_t gamma, int64_t V, int32_t* tokens,
                             double* accept_margin, double* draw_margin) {
  for (int64_t i = 0; i <= gamma; ++i) tokens[i] = -1;
  for (int64_t i = 0; i < gamma; ++i) {
    double gap = 0.0;
    int64_t g = oracle_argmax(z + i * V, V, &gap);
    if (accept_margin) accept_margin[i] = gap;
    if (x[i] == g) {
      tokens[i] = x[i];
      continue;
    }
#if ORACLE_PLANT == PLANT_GREEDY_KEEP_DRAFT
    tokens[i] = x[i];
#else
    tokens[i] = (int32_t)g;
#endif
    if (draw_margin) *draw_margin = gap;
    return (int)(i + 1);
  }
  double gap = 0.0;
  tokens[gamma] = (int32_t)oracle_argmax(z + gamma * V, V, &gap);
  if (draw_margin) *draw_margin = gap;
  return (int)(gamma + 1);
}

/* The full step from logits.
 *   target: [B, gamma+1, V] fp32 target logits
 *   draft:  [B, gamma, V] fp32 draft logits (draft_kind 0) or probabilities
 *           (draft_kind 1, used as given); not read for draft_kind 2 (q is
 *           one-hot at the drafted token) or at T == 0
 *   x:      [B, gamma] drafted token ids
 *   T:      temperature; T == 0 selects the greedy rule, T > 0 sampling
 *   u:      [B, gamma+1, 2] uniforms in [0, 1); ignored at T == 0
 * Outputs as in oracle_verify_probs.  For T > 0 the probability rows of each
 * sequence are formed with oracle_softmax (row by row, as they are needed)
 * and the step runs on them.  scratch must hold 2*(gamma+1)*V floats.
 * Returns 0, -1 on a token outside [0, V), -2 on T < 0 or NaN. */
int oracle_verify(const float* target, const float* draft, int draft_kind, const int32_t* x, double T, const float* u,
                  int64_t B, int64_t gamma, int64_t V, float* scratch, int32_t* tokens, int32_t* num_emitted,
                  double* accept_margin, double* draw_margin, double* draw_mass) {
  if (!(T >= 0.0)) return -2;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < gamma; ++i)
      if (x[b * gamma + i] < 0 || x[b * gamma + i] >= V) return -1;
  float* prow = scratch;                    /* [gamma+1, V] */
  float* qrow = scratch + (gamma + 1) * V;  /* [gamma, V]   */
  float* work = qrow + gamma * V;           /* [V]          */
  for (int64_t b = 0; b < B; ++b) {
    const float* zt = target + b * (gamma + 1) * V;
    const int32_t* xb = x + b * gamma;
    int32_t* tb = tokens + b * (gamma + 1);
    double* amb = accept_margin ? accept_margin + b * gamma : 0;
    double* dmb = draw_margin ? draw_margin + b : 0;
    double* dsb = draw_mass ? draw_mass + b : 0;
    if (dsb) *dsb = 0.0;
    if (amb)
      for (int64_t i = 0; i < gamma; ++i) amb[i] = NAN;
    if (T == 0.0) {
      num_emitted[b] = verify_one_greedy(zt, xb, gamma, V, tb, amb, dmb);
      continue;
    }
    for (int64_t i = 0; i <= gamma; ++i) oracle_softmax(zt + i * V, V, T, prow + i * V, 0, 0);
    for (int64_t i = 0; i < gamma; ++i) {
      const float* dq = draft_kind == ORACLE_Q_ONEHOT ? 0 : draft + (b * gamma + i) * V;
      if (draft_kind == ORACLE_Q_ONEHOT) {
        for (int64_t v = 0; v < V; ++v) qrow[i * V + v] = 0.0f;
        qrow[i * V + xb[i]] = 1.0f;
      } else if (draft_kind == ORACLE_Q_PROBS) {
        memcpy(qrow + i * V, dq, (size_t)V * sizeof(float));
      } else {
        oracle_softmax(dq, V, T, qrow + i * V, 0, 0);
      }
    }
    num_emitted[b] = verify_one_probs(prow, qrow, xb, u + b * (gamma + 1) * 2, gamma, V, work, tb, amb, dmb, dsb);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Warping of a distribution by top-k and top-p before the rule ([LESS] "Why
 * the output is exactly p": temperature, top-k and top-p are applied to p
 * before the rule, and to q before drafting; [PREP] "Correctness": the rule
 * reproduces whatever p it is given).  The pages fix no details; the reading
 * taken here: temperature first, then top-k, then top-p; entries are ranked
 * by logit (larger first), ties by index (lower first); top-k keeps the first
 * k of that ranking (k <= 0 or k >= V: all); top-p keeps the shortest prefix
 * of the top-k survivors whose probabilities (fp32, the softmax over the
 * survivors) sum (fp64) to at least top_p, and at least one entry (top_p >= 1:
 * all); the kept entries are renormalised. */

static const float* g_rank_z; /* ranking key for qsort (the oracle is single-threaded) */

static int rank_cmp(const void* pa, const void* pb) {
  const int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  const float za = g_rank_z[a], zb = g_rank_z[b];
  if (za > zb) return -1;
  if (za < zb) return 1;
#if ORACLE_PLANT == PLANT_TOPK_TIE_HIGH
  return a < b ? 1 : (a > b ? -1 : 0);
#else
  return a < b ? -1 : (a > b ? 1 : 0);
#endif
}

/* Warped probabilities p [V] (fp32, 0 outside the kept set) of logits z at
 * temperature T > 0.  order: V ints of scratch.  margin (optional): the
 * distance of top_p from the cumulative sums just before and at the top-p cut
 * (infinite without top-p), for counting near ties.  Returns the number kept. */
int64_t oracle_warp(const float* z, int64_t V, double T, int64_t top_k, double top_p, float* p, int32_t* order,
                    double* margin) {
  for (int64_t v = 0; v < V; ++v) order[v] = (int32_t)v;
  g_rank_z = z;
  qsort(order, (size_t)V, sizeof(int32_t), rank_cmp);
  const int64_t n1 = (top_k > 0 && top_k < V) ? top_k : V;
  const double m = (double)z[order[0]] / T;
  double Z1 = 0.0;
  for (int64_t j = 0; j < n1; ++j) Z1 += exp((double)z[order[j]] / T - m);
  int64_t n2 = n1;
  if (margin) *margin = INFINITY;
  if (top_p < 1.0) {
    double cum = 0.0;
    for (int64_t j = 0; j < n1; ++j) {
      const double before = cum;
      cum += (double)(float)(exp((double)z[order[j]] / T - m) / Z1);
#if ORACLE_PLANT == PLANT_TOPP_STRICT
      if (cum > top_p) {
#else
      if (cum >= top_p) {
#endif
        n2 = j + 1;
        if (margin) *margin = fmin(cum - top_p, fabs(top_p - before));
        break;
      }
    }
  }
  double Z2 = 0.0;
  for (int64_t j = 0; j < n2; ++j) Z2 += exp((double)z[order[j]] / T - m);
  for (int64_t v = 0; v < V; ++v) p[v] = 0.0f;
  for (int64_t j = 0; j < n2; ++j) p[order[j]] = (float)(exp((double)z[order[j]] / T - m) / Z2);
  return n2;
}

/* The step with warping (T > 0): the target rows, and the draft rows given as
 * logits, are warped with the same top_k and top_p before the rule; draft
 * probabilities and one-hot drafts are used as given.  At T == 0 the greedy
 * rule ignores the warping (it keeps the argmax).  warp_margin [B]: the
 * smallest top-p margin over the rows of the sequence.  scratch: 2*(gamma+1)*V
 * floats; order: V ints.  Returns as oracle_verify. */
int oracle_verify_warped(const float* target, const float* draft, int draft_kind, const int32_t* x, double T,
                         const float* u, int64_t B, int64_t gamma, int64_t V, int64_t top_k, double top_p,
                         float* scratch, int32_t* order, int32_t* tokens, int32_t* num_emitted, double* accept_margin,
                         double* draw_margin, double* draw_mass, double* warp_margin) {
  if (!(T >= 0.0)) return -2;
  if (T == 0.0) {
    for (int64_t b = 0; b < B && warp_margin; ++b) warp_margin[b] = INFINITY;
    return oracle_verify(target, draft, draft_kind, x, T, u, B, gamma, V, scratch, tokens, num_emitted, accept_margin,
                         draw_margin, draw_mass);
  }
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < gamma; ++i)
      if (x[b * gamma + i] < 0 || x[b * gamma + i] >= V) return -1;
  float* prow = scratch;
  float* qrow = scratch + (gamma + 1) * V;
  float* work = qrow + gamma * V;
  for (int64_t b = 0; b < B; ++b) {
    double wm = INFINITY, mg;
    for (int64_t i = 0; i <= gamma; ++i) {
      oracle_warp(target + (b * (gamma + 1) + i) * V, V, T, top_k, top_p, prow + i * V, order, &mg);
      wm = fmin(wm, mg);
    }
    for (int64_t i = 0; i < gamma; ++i) {
      const int32_t xi = x[b * gamma + i];
      if (draft_kind == ORACLE_Q_ONEHOT) {
        for (int64_t v = 0; v < V; ++v) qrow[i * V + v] = 0.0f;
        qrow[i * V + xi] = 1.0f;
      } else if (draft_kind == ORACLE_Q_PROBS) {
        memcpy(qrow + i * V, draft + (b * gamma + i) * V, (size_t)V * sizeof(float));
      } else {
        oracle_warp(draft + (b * gamma + i) * V, V, T, top_k, top_p, qrow + i * V, order, &mg);
        wm = fmin(wm, mg);
      }
    }
    if (accept_margin)
      for (int64_t i = 0; i < gamma; ++i) accept_margin[b * gamma + i] = NAN;
    if (draw_mass) draw_mass[b] = 0.0;
    num_emitted[b] = verify_one_probs(prow, qrow, x + b * gamma, u + b * (gamma + 1) * 2, gamma, V, work,
                                      tokens + b * (gamma + 1), accept_margin ? accept_margin + b * gamma : 0,
                                      draw_margin ? draw_margin + b : 0, draw_mass ? draw_mass + b : 0);
    if (warp_margin) warp_margin[b] = wm;
  }
  return 0;
}

/* Draws one token per row from softmax(z/T) with the given uniforms, by the
 * same inverse-CDF rule.  Used by the tests to make drafted tokens that follow
 * q, as the pages require of a draft ([LESS] "Why the output is exactly p":
 * q must be the distribution actually drawn from).  scratch holds V floats. */
void oracle_sample_rows(const float* z, int64_t rows, int64_t V, double T, const float* u, float* scratch,
                        int32_t* out) {
  for (int64_t r = 0; r < rows; ++r) {
    oracle_softmax(z + r * V, V, T, scratch, 0, 0);
    out[r] = (int32_t)oracle_draw(scratch, V, u[r], 0, 0);
  }
}

/* ------------------------------------------------------------------------ */
/* Acceptance rate alpha = sum_v min(p(v), q(v)) ([LLMI] section 2, overall
 * acceptance probability; [MATH] proof, total acceptance rate). */
double oracle_acceptance_rate(const float* p, const float* q, int64_t V) {
  double a = 0.0;
  for (int64_t v = 0; v < V; ++v) a += (double)(p[v] < q[v] ? p[v] : q[v]);
  return a;
}

/* Expected emitted tokens per verification pass with i.i.d. acceptance alpha
 * over gamma drafts: (1 - alpha^(gamma+1)) / (1 - alpha), gamma+1 at alpha = 1
 * ([LLMI] section 2; [MATH] "Expected Accepted Tokens per Speculative Round";
 * [LESS] "How many tokens per pass"; [PREP] "Throughput math"). */
double oracle_expected_tokens(double alpha, int64_t gamma) {
  if (fabs(1.0 - alpha) < 1e-12) return (double)(gamma + 1);
  return (1.0 - pow(alpha, (double)(gamma + 1))) / (1.0 - alpha);
}

/* The same expectation when row i has its own acceptance probability
 * alpha[i]: the step emits more than k tokens iff the first k drafts are all
 * kept, so E = sum_{k=0}^{gamma} prod_{i<k} alpha[i]. */
double oracle_expected_tokens_rows(const double* alpha, int64_t gamma) {
  double e = 0.0, run = 1.0;
  for (int64_t k = 0; k <= gamma; ++k) {
    e += run;
    if (k < gamma) run *= alpha[k];
  }
  return e;
}

/* ------------------------------------------------------------------------ */
/* Tree verification ([LLMI] section 3, the tree attention mask and depth
 * offsets; [MATH] "SpecInfer and Tree-Based Verification").  A tree of M
 * nodes is flattened in an order where every parent comes before its
 * children: parents[0] = -1 (node 0, the root, is the last token already in
 * the text) and parents[i] is in [0, i) for i >= 1.  A node whose parent index
 * is outside that range is taken as detached: it is its own only ancestor,
 * has depth 0 and is never accepted. */

/* Parent of node i if the link is well formed, else -1. */
static int64_t tree_parent(const int32_t* parents, int64_t i) {
  if (i == 0) return -1;
  const int64_t p = parents[i];
  return (p >= 0 && p < i) ? p : -1;
}

/* Depth of every node (edges from the root) and its ancestor set as a bit mask
 * (bit j set iff node j is an ancestor of i or i itself; M <= 64), found by
 * walking the parent links up from each node.  Optionally the additive mask
 * the pages use, [M, M] with 0 where attention is allowed and -inf elsewhere. */
void oracle_tree_mask(const int32_t* parents, int64_t M, uint64_t* mask, int32_t* depth, float* additive) {
  for (int64_t i = 0; i < M; ++i) {
    uint64_t bits = 0;
    int32_t dpt = 0;
    for (int64_t cur = i; cur != -1; cur = tree_parent(parents, cur)) {
      bits |= (uint64_t)1 << cur;
      if (tree_parent(parents, cur) != -1) ++dpt;
    }
#if ORACLE_PLANT == PLANT_TREE_DEPTH
    dpt += 1;
#endif
    if (mask) mask[i] = bits;
    if (depth) depth[i] = dpt;
    if (additive)
      for (int64_t j = 0; j < M; ++j) additive[i * M + j] = ((bits >> j) & 1) ? 0.0f : -INFINITY;
  }
}

/* Greedy verification of one tree (T == 0).  z: [M, V] target logits, row i
 * scoring the position after node i along its path.  Node i >= 1 is accepted
 * iff its parent is accepted and its token equals the argmax of the parent's
 * row (lowest index on ties); the root always is.  The accepted nodes form
 * paths from the root; the deepest accepted node a (lowest index among equals)
 * ends the path that is kept.  Emits the tokens of the path after the root,
 * then the argmax of row a.  nodes receives the path root .. a (the positions
 * whose keys and values survive).  Returns the number of emitted tokens,
 * depth(a) + 1.  scratch: 3*M ints. */
int oracle_tree_greedy(const float* z, const int32_t* parents, const int32_t* node_tokens, int64_t M, int64_t V,
                       int32_t* scratch, int32_t* tokens, int32_t* nodes) {
  int32_t* best = scratch;          /* argmax of each row */
  int32_t* accepted = scratch + M;
  int32_t* depth = scratch + 2 * M;
  oracle_tree_mask(parents, M, 0, depth, 0);
  for (int64_t i = 0; i < M; ++i) best[i] = (int32_t)oracle_argmax(z + i * V, V, 0);
  int64_t a = 0;
  for (int64_t i = 0; i < M; ++i) {
    const int64_t p = tree_parent(parents, i);
    if (i == 0) {
      accepted[i] = 1;
    } else {
#if ORACLE_PLANT == PLANT_TREE_SELF_ARGMAX
      accepted[i] = p >= 0 && accepted[p] && node_tokens[i] == best[i];
#else
      accepted[i] = p >= 0 && accepted[p] && node_tokens[i] == best[p];
#endif
    }
    if (accepted[i] && depth[i] > depth[a]) a = i;
  }
  /* the path root .. a, root first */
  const int64_t n = depth[a] + 1;
  int64_t cur = a;
  for (int64_t j = n - 1; j >= 0; --j) {
    nodes[j] = (int32_t)cur;
    cur = cur >= 0 ? tree_parent(parents, cur) : -1;
  }
  for (int64_t j = n; j < M; ++j) nodes[j] = -1;
  for (int64_t j = 1; j < n; ++j) tokens[j - 1] = nodes[j] >= 0 ? node_tokens[nodes[j]] : -1;
  tokens[n - 1] = best[a];
  for (int64_t j = n; j < M; ++j) tokens[j] = -1;
  return (int)n;
}

/* ------------------------------------------------------------------------ */
/* Paged KV cache ([LLMI] section 1, paged block allocation and instant
 * speculative rollback).  Keys and values live in a pool of fixed-size
 * physical blocks, [num_blocks][heads][block_size][head_dim] elements of
 * elem bytes.  Request r keeps a block table (its logical blocks in order)
 * and a length; token position t lives in logical block t / block_size at
 * offset t % block_size.  Free blocks form a stack: it starts as
 * num_blocks-1, ..., 1, 0 (so the first block handed out is 0), allocation
 * takes from its top, and rollback pushes a request's trailing blocks back,
 * the last logical block first.  A batch is served request by request in
 * index order.  tables: [R][max_blocks]; stack: [num_blocks]; *top: number
 * of free blocks. */

void oracle_kv_init(int32_t* stack, int32_t* top, int32_t* seq_lens, int64_t R, int64_t num_blocks) {
  for (int64_t i = 0; i < num_blocks; ++i) stack[i] = (int32_t)(num_blocks - 1 - i);
  *top = (int32_t)num_blocks;
  for (int64_t r = 0; r < R; ++r) seq_lens[r] = 0;
}

static int64_t blocks_for_len(int64_t len, int64_t block_size) { return (len + block_size - 1) / block_size; }

/* Appends n_new tokens to every request: new keys/values [R][heads][n_new][head_dim].
 * Returns 0, or 1 (changing nothing) when the free blocks do not cover the
 * batch, or 2 (changing nothing) when a request would need more than
 * max_blocks blocks. */
int oracle_kv_append(uint8_t* kpool, uint8_t* vpool, int32_t* tables, int32_t* seq_lens, int32_t* stack, int32_t* top,
                     const uint8_t* knew, const uint8_t* vnew, int64_t R, int64_t n_new, int64_t heads,
                     int64_t block_size, int64_t head_dim, int64_t elem, int64_t max_blocks) {
  int64_t need = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t nb = blocks_for_len(seq_lens[r] + n_new, block_size);
    if (nb > max_blocks) return 2;
    need += nb - blocks_for_len(seq_lens[r], block_size);
  }
  if (need > *top) return 1;
  const int64_t row = head_dim * elem;  /* bytes of one token of one head */
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t i = 0; i < n_new; ++i) {
      const int64_t pos = seq_lens[r] + i;
      const int64_t logical = pos / block_size;
#if ORACLE_PLANT == PLANT_KV_OFFSET
      const int64_t off = (pos / block_size) % block_size;
#else
      const int64_t off = pos % block_size;
#endif
      if (pos % block_size == 0) tables[r * max_blocks + logical] = stack[--*top]; /* a new logical block */
      const int64_t phys = tables[r * max_blocks + logical];
      for (int64_t h = 0; h < heads; ++h) {
        const int64_t dst = ((phys * heads + h) * block_size + off) * row;
        const int64_t src = ((r * heads + h) * n_new + i) * row;
        memcpy(kpool + dst, knew + src, (size_t)row);
        memcpy(vpool + dst, vnew + src, (size_t)row);
      }
    }
    seq_lens[r] += (int32_t)n_new;
  }
  return 0;
}

/* Rolls request r back to keep_lens[r] tokens, freeing the blocks it no
 * longer needs (the last logical block first).  No key or value moves.  A
 * request asked to grow is left as it is; returns the number of such. */
int oracle_kv_rollback(int32_t* tables, int32_t* seq_lens, int32_t* stack, int32_t* top, const int32_t* keep_lens,
                       int64_t R, int64_t block_size, int64_t max_blocks) {
  int bad = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t keep = keep_lens[r];
    if (keep < 0 || keep > seq_lens[r]) {
      ++bad;
      continue;
    }
    const int64_t have = blocks_for_len(seq_lens[r], block_size), needed = blocks_for_len(keep, block_size);
#if ORACLE_PLANT == PLANT_KV_FREE_ORDER
    for (int64_t j = needed; j < have; ++j) stack[(*top)++] = tables[r * max_blocks + j];
#else
    for (int64_t j = have - 1; j >= needed; --j) stack[(*top)++] = tables[r * max_blocks + j];
#endif
    seq_lens[r] = (int32_t)keep;
  }
  return bad;
}

/* Contiguous keys and values of request r, [heads][seq_len][head_dim]. */
void oracle_kv_gather(const uint8_t* kpool, const uint8_t* vpool, const int32_t* tables, const int32_t* seq_lens,
                      int64_t r, int64_t heads, int64_t block_size, int64_t head_dim, int64_t elem, int64_t max_blocks,
                      uint8_t* kout, uint8_t* vout) {
  const int64_t len = seq_lens[r], row = head_dim * elem;
  for (int64_t h = 0; h < heads; ++h)
    for (int64_t t = 0; t < len; ++t) {
      const int64_t phys = tables[r * max_blocks + t / block_size];
      const int64_t src = ((phys * heads + h) * block_size + t % block_size) * row;
      memcpy(kout + (h * len + t) * row, kpool + src, (size_t)row);
      memcpy(vout + (h * len + t) * row, vpool + src, (size_t)row);
    }
}

/* Which mistake (if any) this compiled copy of the oracle carries (ORACLE_PLANT); 0 for the real oracle. */
int oracle_planted(void) { return ORACLE_PLANT; }
