/*
 * oracle.c - plain double-precision CPU oracle (test infrastructure only;
 * see oracle.h for the page legend and the readings R1..R18).
 *
 * Parity status of each function (what pins it, in tests/test_oracle_pins.py):
 *   oracle_summaries      pinned: numpy min/max per block, hand fixture
 *   oracle_score          pinned: hand fixture, upper-bound property, equality
 *                         at S=1, second closed form of the bound
 *   oracle_candidates /
 *   oracle_num_selected   pinned: hand fixtures of D, C and k
 *   oracle_select         pinned: brute force over all k-subsets, exact token
 *                         top-k at S=1, scale invariance
 *   oracle_attend_tokens /
 *   oracle_attend         pinned: budget 100% equals the independent dense
 *                         softmax, single token, hand fixture, LSE partition
 *                         identity
 *   oracle_fuse           pinned: LSE identity over random partitions
 *   oracle_maw_update     pinned: closed forms of the decay-0.95 average
 *   oracle_dense_mass     pinned: numpy softmax over the dense set per head,
 *                         summed per block and averaged over unequal heads;
 *                         mass conservation over D
 *   oracle_maw_step       pinned: hand fixture (blocks with a token outside D
 *                         keep MAW, blocks inside D take the average)
 *   oracle_maw_flag       pinned: hand fixture at S = 32 and a selection hand
 *                         case at S = 2 on either side of beta*S/|D|
 *   oracle_select_heads   pinned: brute force over all k-subsets per head at
 *                         G = 3, independence of the heads, equal rows give
 *                         the group selection
 *   oracle_lfps_candidates pinned: hand fixture (thresholds, growth by the
 *                         offsets, the mean filter, slash offsets, candidates)
 *   oracle_lfps_select    pinned: brute force over all k-subsets of C; equals
 *                         oracle_select when C holds that selection
 *   oracle_attend_mass    pinned: numpy softmax over T summed per block;
 *                         mass conservation
 *   oracle_lfps_update /
 *   oracle_lfps_init      pinned: closed forms of the decay, slash offsets of
 *                         an impulse, init of one and two prefill positions
 *                         against numpy softmax masses
 *   oracle_attend_heads   pinned: each head over its own token list by
 *                         oracle_attend_tokens; full budget equals the
 *                         independent dense softmax for every head
 *   The readings themselves - group max (R1), per-block MAW (R8), the
 *   beta/|D| flag scale (R9) and the lexicographic flag-then-score order
 *   (R11) - are not fixed by the pages; the pins above fix the oracle to
 *   those readings, not the readings to the pages.
 * A committed mutation sweep (tests/test_oracle_mutants.py) plants one
 * plausible mistake at a time in a copy of this file and checks that some
 * pin fails for each.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double, exact (bf16 is the top half of an IEEE
 * binary32). */
static double widen(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int64_t oracle_num_blocks(int64_t N, int32_t S) {
  return N <= 0 ? 0 : (N + S - 1) / S;
}

/* Dense set: the first n_s tokens (attention sinks, [FLX] Figure 3(c) and
 * Figure 4) and the W most recent tokens (the GPU-resident recent window,
 * [HGCA] "What carries the argument"). */
int32_t oracle_in_dense(int64_t j, int64_t N, int32_t n_s, int32_t W) {
  if (j < 0 || j >= N) return 0;
  if (j < (int64_t)n_s) return 1;
  if (j >= N - (int64_t)W) return 1;
  return 0;
}

int64_t oracle_dense_count(int64_t N, int32_t n_s, int32_t W) {
  int64_t c = 0;
  for (int64_t j = 0; j < N; ++j) c += oracle_in_dense(j, N, n_s, W);
  return c;
}

/* Candidate blocks: those with at least one token the dense set does not
 * already cover (R4: only such blocks can add tokens to the attended set). */
int64_t oracle_candidates(int64_t N, int32_t S, int32_t n_s, int32_t W,
                          int8_t *cand) {
  int64_t n_blk = oracle_num_blocks(N, S), n = 0;
  for (int64_t i = 0; i < n_blk; ++i) {
    int8_t any = 0;
    for (int64_t j = i * S; j < (i + 1) * S && j < N; ++j)
      if (!oracle_in_dense(j, N, n_s, W)) any = 1;
    if (cand) cand[i] = any;
    n += any;
  }
  return n;
}

/* Budget as a token fraction of N ([FLX] Figure 2 "budget=5%", Figure 7 text
 * "(32, 0.02)", Figure 8 "(blk, bgt)"), converted to whole blocks (R3). */
int64_t oracle_num_selected(int64_t N, int32_t S, int64_t budget_ppm,
                            int64_t n_cand) {
  int64_t den = (int64_t)1000000 * (int64_t)S;
  int64_t k = (budget_ppm * N + den - 1) / den;
  if (k > n_cand) k = n_cand;
  if (k < 0) k = 0;
  return k;
}

/* Per-block min/max key summaries (the block metadata that Quest-style
 * scoring reads; Quest is named in [LFPS] "Extended reading notes" as the
 * block-based baseline and in [IDX] "Builds on"). */
void oracle_summaries(const uint16_t *K, int64_t ldk, int64_t N, int32_t d,
                      int32_t S, uint16_t *mn, uint16_t *mx) {
  int64_t n_blk = oracle_num_blocks(N, S);
  for (int64_t i = 0; i < n_blk; ++i) {
    for (int32_t c = 0; c < d; ++c) {
      int64_t j0 = i * S;
      uint16_t lo = K[j0 * ldk + c], hi = K[j0 * ldk + c];
      for (int64_t j = j0 + 1; j < (i + 1) * S && j < N; ++j) {
        uint16_t x = K[j * ldk + c];
        if (widen(x) < widen(lo)) lo = x;
        if (widen(x) > widen(hi)) hi = x;
      }
      mn[i * d + c] = lo;
      mx[i * d + c] = hi;
    }
  }
}

/* R2: U_h(i) = sum_c max(q_hc * m_ic, q_hc * M_ic), an upper bound of
 * q_h . k_j for every key j of block i.  R1: U(i) = max over the group. */
void oracle_score(const uint16_t *q, int32_t G, int32_t d, const uint16_t *mn,
                  const uint16_t *mx, int64_t n_blk, double *Uh, double *U,
                  float *u) {
  for (int64_t i = 0; i < n_blk; ++i) {
    double best = -INFINITY;
    for (int32_t h = 0; h < G; ++h) {
      double s = 0.0;
      for (int32_t c = 0; c < d; ++c) {
        double qc = widen(q[h * d + c]);
        double a = qc * widen(mn[i * d + c]);
        double b = qc * widen(mx[i * d + c]);
        s += (a > b) ? a : b;
      }
      if (Uh) Uh[(int64_t)h * n_blk + i] = s;
      if (s > best) best = s;
    }
    U[i] = best;
    u[i] = (float)best;
  }
}

/* R9: HGCA keeps an entry whose moving-average attention weight exceeds beta
 * divided by the number of GPU-resident (dense) entries ([HGCA] "What carries
 * the argument"); per block this compares the mean per-token mass MAW/S with
 * beta/|D|. */
int32_t oracle_maw_flag(double maw, int64_t n_dense, double beta, int32_t S) {
  if (!(beta > 0.0)) return 0;
  return maw * (double)n_dense > beta * (double)S;
}

/* Ordering context for qsort, one per thread (the oracle's functions may be
 * called from several threads at once, one unit each). */
typedef struct {
  const float *u;
  const int8_t *flag;
} order_ctx;
static _Thread_local order_ctx g_order;

/* R5/R11: (flag desc, score desc, index asc) - a total order. */
static int cmp_blocks(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  if (g_order.flag[a] != g_order.flag[b])
    return g_order.flag[a] > g_order.flag[b] ? -1 : 1;
  if (g_order.u[a] != g_order.u[b]) return g_order.u[a] > g_order.u[b] ? -1 : 1;
  return a < b ? -1 : (a > b ? 1 : 0);
}

static int cmp_int32(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return a < b ? -1 : (a > b ? 1 : 0);
}

/* Top-k block selection under a token budget ([FLX] "Core claim", Figure 2(d):
 * per-head top-k over blocks; [HGCA] MAW threshold; R1-R5, R9, R11). */
int64_t oracle_select(const uint16_t *q, int32_t G, int32_t d,
                      const uint16_t *mn, const uint16_t *mx, int64_t N,
                      int32_t S, int32_t n_s, int32_t W, int64_t budget_ppm,
                      const double *maw, double beta, int32_t *sel, double *U,
                      float *u, int8_t *flag) {
  int64_t n_blk = oracle_num_blocks(N, S);
  if (n_blk == 0) return 0;
  double *U_ = (double *)malloc(sizeof(double) * n_blk);
  float *u_ = (float *)malloc(sizeof(float) * n_blk);
  int8_t *f_ = (int8_t *)calloc(n_blk, 1);
  int8_t *cand = (int8_t *)malloc(n_blk);
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * n_blk);

  oracle_score(q, G, d, mn, mx, n_blk, NULL, U_, u_);
  /* The sign of zero carries no order: -0 and +0 are the same score. */
  for (int64_t i = 0; i < n_blk; ++i)
    if (u_[i] == 0.0f) u_[i] = 0.0f;
  int64_t n_dense = oracle_dense_count(N, n_s, W);
  if (maw)
    for (int64_t i = 0; i < n_blk; ++i)
      f_[i] = (int8_t)oracle_maw_flag(maw[i], n_dense, beta, S);

  int64_t n_cand = oracle_candidates(N, S, n_s, W, cand);
  int64_t k = oracle_num_selected(N, S, budget_ppm, n_cand);

  int64_t m = 0;
  for (int64_t i = 0; i < n_blk; ++i)
    if (cand[i]) order[m++] = (int32_t)i;
  g_order.u = u_;
  g_order.flag = f_;
  qsort(order, (size_t)m, sizeof(int32_t), cmp_blocks);
  for (int64_t t = 0; t < k; ++t) sel[t] = order[t];
  qsort(sel, (size_t)k, sizeof(int32_t), cmp_int32);

  if (U) memcpy(U, U_, sizeof(double) * n_blk);
  if (u) memcpy(u, u_, sizeof(float) * n_blk);
  if (flag) memcpy(flag, f_, (size_t)n_blk);
  free(U_);
  free(u_);
  free(f_);
  free(cand);
  free(order);
  return k;
}

/* Per-query-head selection, the literal per-head reading: the pages count
 * and budget attention heads one query head at a time ([FLX] Figure 4: the
 * output deviation of each of Llama-3.1-8B's 32 heads; Figure 5: a minimum
 * budget per head for the 32 heads of a layer; [HGCA] What carries the
 * argument: the sparse set is chosen per head).  Under grouped-query
 * attention the G query heads of a KV head read the same blocks, so each
 * head's set is oracle_select over a group of that one head: its own bound,
 * the KV head's k, MAW flags and order. */
int64_t oracle_select_heads(const uint16_t *q, int32_t G, int32_t d,
                            const uint16_t *mn, const uint16_t *mx, int64_t N,
                            int32_t S, int32_t n_s, int32_t W,
                            int64_t budget_ppm, const double *maw, double beta,
                            int32_t *sel, int64_t ld_sel) {
  int64_t k = 0;
  for (int32_t h = 0; h < G; ++h)
    k = oracle_select(q + (int64_t)h * d, 1, d, mn, mx, N, S, n_s, W, budget_ppm, maw, beta,
                      sel + (int64_t)h * ld_sel, NULL, NULL, NULL);
  return k;
}

/* Softmax attention of each query head over a token list, in the max-shifted
 * form ([HGCA] referee minor comment on section 3.3: subtract the maximum
 * before exponentiating).  R18: natural-log lse of scaled logits. */
void oracle_attend_tokens(const uint16_t *q, int32_t G, int32_t d,
                          const uint16_t *K, int64_t ldk, const uint16_t *V,
                          int64_t ldv, const int64_t *tok, int64_t n_tok,
                          double scale, double *O, double *lse, double *p) {
  double *s = (double *)malloc(sizeof(double) * (n_tok > 0 ? n_tok : 1));
  for (int32_t h = 0; h < G; ++h) {
    for (int32_t c = 0; c < d; ++c) O[h * d + c] = 0.0;
    if (n_tok == 0) {
      lse[h] = -INFINITY;
      continue;
    }
    double mx = -INFINITY;
    for (int64_t t = 0; t < n_tok; ++t) {
      const uint16_t *kr = K + tok[t] * ldk;
      double acc = 0.0;
      for (int32_t c = 0; c < d; ++c) acc += widen(q[h * d + c]) * widen(kr[c]);
      s[t] = scale * acc;
      if (s[t] > mx) mx = s[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < n_tok; ++t) z += exp(s[t] - mx);
    lse[h] = mx + log(z);
    for (int64_t t = 0; t < n_tok; ++t) {
      double w = exp(s[t] - lse[h]);
      if (p) p[(int64_t)h * n_tok + t] = w;
      const uint16_t *vr = V + tok[t] * ldv;
      for (int32_t c = 0; c < d; ++c) O[h * d + c] += w * widen(vr[c]);
    }
  }
  free(s);
}

/* Attention over T = D U tokens(Sel) (R4), the split-K partial that the pages
 * merge ([HGCA] "What carries the argument": dense recent window plus sparse
 * selected entries). */
int64_t oracle_attend(const uint16_t *q, int32_t G, int32_t d,
                      const uint16_t *K, int64_t ldk, const uint16_t *V,
                      int64_t ldv, int64_t N, int32_t S, int32_t n_s,
                      int32_t W, const int32_t *sel, int64_t k, double scale,
                      double *O, double *lse) {
  int8_t *inT = (int8_t *)calloc(N > 0 ? N : 1, 1);
  for (int64_t j = 0; j < N; ++j) inT[j] = (int8_t)oracle_in_dense(j, N, n_s, W);
  for (int64_t t = 0; t < k; ++t)
    for (int64_t j = (int64_t)sel[t] * S; j < ((int64_t)sel[t] + 1) * S && j < N; ++j)
      inT[j] = 1;
  int64_t n_tok = 0;
  for (int64_t j = 0; j < N; ++j) n_tok += inT[j];
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (n_tok > 0 ? n_tok : 1));
  int64_t t = 0;
  for (int64_t j = 0; j < N; ++j)
    if (inT[j]) tok[t++] = j;
  oracle_attend_tokens(q, G, d, K, ldk, V, ldv, tok, n_tok, scale, O, lse, NULL);
  free(tok);
  free(inT);
  return n_tok;
}

/* Per-query-head attention: head h attends T_h = D U tokens(sel_h), its own
 * selection (a group of one head in oracle_attend). */
void oracle_attend_heads(const uint16_t *q, int32_t G, int32_t d,
                         const uint16_t *K, int64_t ldk, const uint16_t *V,
                         int64_t ldv, int64_t N, int32_t S, int32_t n_s,
                         int32_t W, const int32_t *sel, int64_t ld_sel,
                         const int64_t *k, double scale, double *O,
                         double *lse) {
  for (int32_t h = 0; h < G; ++h)
    oracle_attend(q + (int64_t)h * d, 1, d, K, ldk, V, ldv, N, S, n_s, W,
                  sel + (int64_t)h * ld_sel, k[h], scale, O + (int64_t)h * d, lse + h);
}

/* Learn from the past ([LFPS] What carries the argument: a vertical table per
 * absolute position and a slash table per relative position, decayed by r =
 * 0.95 after every step; Figure 4: thresholds and means of the two tables,
 * initial candidates above the thresholds, grown by the offsets {-1, 0, 1, 2},
 * keeping the grown indices whose scores exceed the means; Assumptions & free
 * parameters: a = 0.2 sets the threshold).  Readings: positions are blocks of
 * S tokens and the slash offset is counted from the newest token's block; the
 * threshold's kurtosis estimator is not given, so tau interpolates between the
 * table's mean and maximum by a; a kept block must also hold a token outside
 * D (the dense tokens are attended anyway). */
static void lfps_stats(const double *phi, int64_t n, double *mu, double *mx) {
  double sum = 0.0, m = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    sum += phi[i];
    if (phi[i] > m) m = phi[i];
  }
  *mu = n > 0 ? sum / (double)n : 0.0;
  *mx = n > 0 ? m : 0.0;
}

int64_t oracle_lfps_candidates(const double *phi_v, const double *phi_s, int64_t N,
                               int32_t S, int32_t n_s, int32_t W, double a,
                               int8_t *inC) {
  int64_t n_blk = oracle_num_blocks(N, S);
  if (n_blk == 0) return 0;
  int64_t b = n_blk - 1;
  double mu_v, mx_v, mu_s, mx_s;
  lfps_stats(phi_v, b + 1, &mu_v, &mx_v);
  lfps_stats(phi_s, b + 1, &mu_s, &mx_s);
  double tau_v = mu_v + a * (mx_v - mu_v), tau_s = mu_s + a * (mx_s - mu_s);
  int8_t *c0 = (int8_t *)calloc(n_blk, 1);
  int8_t *cand = (int8_t *)malloc(n_blk);
  for (int64_t i = 0; i <= b; ++i) c0[i] = (int8_t)(phi_v[i] > tau_v || phi_s[b - i] > tau_s);
  oracle_candidates(N, S, n_s, W, cand);
  int64_t n = 0;
  for (int64_t i = 0; i < n_blk; ++i) {
    int grown = 0;
    for (int e = -1; e <= 2; ++e) {  /* i = c + e for some c in C0 */
      int64_t c = i - e;
      if (c >= 0 && c <= b && c0[c]) grown = 1;
    }
    int above = phi_v[i] > mu_v || phi_s[b - i] > mu_s;
    inC[i] = (int8_t)(grown && above && cand[i]);
    n += inC[i];
  }
  free(c0);
  free(cand);
  return n;
}

int64_t oracle_lfps_select(const uint16_t *q, int32_t G, int32_t d,
                           const uint16_t *mn, const uint16_t *mx, int64_t N,
                           int32_t S, int32_t n_s, int32_t W, int64_t budget_ppm,
                           const double *phi_v, const double *phi_s, double a,
                           int32_t *sel, double *U, float *u) {
  int64_t n_blk = oracle_num_blocks(N, S);
  if (n_blk == 0) return 0;
  double *U_ = (double *)malloc(sizeof(double) * n_blk);
  float *u_ = (float *)malloc(sizeof(float) * n_blk);
  int8_t *f_ = (int8_t *)calloc(n_blk, 1);
  int8_t *inC = (int8_t *)malloc(n_blk);
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * n_blk);
  oracle_score(q, G, d, mn, mx, n_blk, NULL, U_, u_);
  for (int64_t i = 0; i < n_blk; ++i)
    if (u_[i] == 0.0f) u_[i] = 0.0f;
  int64_t nC = oracle_lfps_candidates(phi_v, phi_s, N, S, n_s, W, a, inC);
  int64_t k = oracle_num_selected(N, S, budget_ppm, nC);
  int64_t m = 0;
  for (int64_t i = 0; i < n_blk; ++i)
    if (inC[i]) order[m++] = (int32_t)i;
  g_order.u = u_;
  g_order.flag = f_;
  qsort(order, (size_t)m, sizeof(int32_t), cmp_blocks);
  for (int64_t t = 0; t < k; ++t) sel[t] = order[t];
  qsort(sel, (size_t)k, sizeof(int32_t), cmp_int32);
  if (U) memcpy(U, U_, sizeof(double) * n_blk);
  if (u) memcpy(u, u_, sizeof(float) * n_blk);
  free(U_);
  free(u_);
  free(f_);
  free(inC);
  free(order);
  return k;
}

/* The mass each block receives under the softmax over the attended set
 * ([LFPS] the tables aggregate the step's attention weights; reading of their
 * "half-normalised" weights: normalised over the tokens the step attends,
 * averaged over the group's query heads). */
void oracle_attend_mass(const uint16_t *q, int32_t G, int32_t d, const uint16_t *K,
                        int64_t ldk, int64_t N, int32_t S, int32_t n_s, int32_t W,
                        const int32_t *sel, int64_t k, double scale, double *a_blk) {
  int64_t n_blk = oracle_num_blocks(N, S);
  for (int64_t i = 0; i < n_blk; ++i) a_blk[i] = 0.0;
  int8_t *inT = (int8_t *)calloc(N > 0 ? N : 1, 1);
  for (int64_t j = 0; j < N; ++j) inT[j] = (int8_t)oracle_in_dense(j, N, n_s, W);
  for (int64_t t = 0; t < k; ++t)
    for (int64_t j = (int64_t)sel[t] * S; j < ((int64_t)sel[t] + 1) * S && j < N; ++j)
      inT[j] = 1;
  int64_t nT = 0;
  for (int64_t j = 0; j < N; ++j) nT += inT[j];
  if (nT > 0) {
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * nT);
    int64_t t = 0;
    for (int64_t j = 0; j < N; ++j)
      if (inT[j]) tok[t++] = j;
    double *O = (double *)malloc(sizeof(double) * G * d);
    double *lse = (double *)malloc(sizeof(double) * G);
    double *p = (double *)malloc(sizeof(double) * G * nT);
    oracle_attend_tokens(q, G, d, K, ldk, K, ldk, tok, nT, scale, O, lse, p);
    for (int32_t h = 0; h < G; ++h)
      for (int64_t tt = 0; tt < nT; ++tt) a_blk[tok[tt] / S] += p[(int64_t)h * nT + tt] / (double)G;
    free(p);
    free(lse);
    free(O);
    free(tok);
  }
  free(inT);
}

/* [LFPS] What carries the argument: both tables decay by r after every step
 * and take the step's weights (Eq. (10) read as the convex update, as MAW). */
void oracle_lfps_update(double *phi_v, double *phi_s, const double *a_blk,
                        int64_t n_blk, double r) {
  int64_t b = n_blk - 1;
  for (int64_t i = 0; i <= b; ++i) phi_v[i] = r * phi_v[i] + (1.0 - r) * a_blk[i];
  for (int64_t o = 0; o <= b; ++o) phi_s[o] = r * phi_s[o] + (1.0 - r) * a_blk[b - o];
}

/* [LFPS] Assumptions & free parameters: the tables start from the last s = 32
 * prefill steps (Eq. (4)); each such step attends causally to every earlier
 * token (the prefill is dense). */
void oracle_lfps_init(const uint16_t *q, int32_t s, int32_t G, int32_t d,
                      const uint16_t *K, int64_t ldk, int64_t N, int32_t S,
                      double scale, double r, double *phi_v, double *phi_s) {
  int64_t n_blk = oracle_num_blocks(N, S);
  for (int64_t i = 0; i < n_blk; ++i) phi_v[i] = phi_s[i] = 0.0;
  double *a = (double *)malloc(sizeof(double) * (n_blk > 0 ? n_blk : 1));
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
  double *O = (double *)malloc(sizeof(double) * G * d);
  double *lse = (double *)malloc(sizeof(double) * G);
  double *p = (double *)malloc(sizeof(double) * G * (N > 0 ? N : 1));
  for (int32_t u = 0; u < s; ++u) {
    int64_t pos = N - s + u;
    if (pos < 0) continue;
    int64_t nb = pos / S + 1;
    for (int64_t j = 0; j <= pos; ++j) tok[j] = j;
    oracle_attend_tokens(q + (int64_t)u * G * d, G, d, K, ldk, K, ldk, tok, pos + 1, scale, O,
                         lse, p);
    for (int64_t i = 0; i < nb; ++i) a[i] = 0.0;
    for (int32_t h = 0; h < G; ++h)
      for (int64_t j = 0; j <= pos; ++j) a[j / S] += p[(int64_t)h * (pos + 1) + j] / (double)G;
    oracle_lfps_update(phi_v, phi_s, a, nb, r);
  }
  free(p);
  free(lse);
  free(O);
  free(tok);
  free(a);
}

/* The MAW input of one step (R8, and R10 as read from HGCA): HGCA's moving
 * average is fed only by the attention weights of the GPU-side partial, the
 * dense recent window, normalised over that window alone ([HGCA] "What
 * carries the argument": the threshold is beta over the number of GPU-side
 * entries; referee report on section 3.2.2 / Algorithm 1: the average is
 * updated from the window's weights only).  Here the GPU-side entries are D:
 * per query head h the softmax over D, p_hj = e^{s_hj - lse_D,h}; per block
 * a_i = (1/G) sum_h sum_{j in D, j in block i} p_hj.  a_i = 0 for blocks
 * with no token in D; sum_i a_i = 1 when D is not empty. */
void oracle_dense_mass(const uint16_t *q, int32_t G, int32_t d,
                       const uint16_t *K, int64_t ldk, int64_t N, int32_t S,
                       int32_t n_s, int32_t W, double scale, double *a_blk) {
  int64_t n_blk = oracle_num_blocks(N, S);
  for (int64_t i = 0; i < n_blk; ++i) a_blk[i] = 0.0;
  int64_t nD = oracle_dense_count(N, n_s, W);
  if (nD == 0) return;
  int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * nD);
  int64_t t = 0;
  for (int64_t j = 0; j < N; ++j)
    if (oracle_in_dense(j, N, n_s, W)) tok[t++] = j;
  double *O = (double *)malloc(sizeof(double) * (size_t)G * d);
  double *lse = (double *)malloc(sizeof(double) * (size_t)G);
  double *p = (double *)malloc(sizeof(double) * (size_t)G * nD);
  /* attend_tokens reads V only to form O, which is not used here */
  oracle_attend_tokens(q, G, d, K, ldk, K, ldk, tok, nD, scale, O, lse, p);
  for (int32_t h = 0; h < G; ++h)
    for (int64_t tt = 0; tt < nD; ++tt)
      a_blk[tok[tt] / S] += p[(int64_t)h * nD + tt] / (double)G;
  free(p);
  free(lse);
  free(O);
  free(tok);
}

/* Independent textbook softmax over every token: weights e^{s_j - max}
 * normalised by their sum; no shared helper with oracle_attend_tokens. */
void oracle_dense(const uint16_t *q, int32_t G, int32_t d, const uint16_t *K,
                  int64_t ldk, const uint16_t *V, int64_t ldv, int64_t N,
                  double scale, double *O, double *lse) {
  double *w = (double *)malloc(sizeof(double) * (N > 0 ? N : 1));
  for (int32_t h = 0; h < G; ++h) {
    double big = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
      double dot = 0.0;
      for (int32_t c = 0; c < d; ++c)
        dot += widen(K[j * ldk + c]) * widen(q[h * d + c]);
      w[j] = dot * scale;
      if (w[j] > big) big = w[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      w[j] = exp(w[j] - big);
      sum += w[j];
    }
    for (int32_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < N; ++j) acc += w[j] * widen(V[j * ldv + c]);
      O[h * d + c] = N > 0 ? acc / sum : 0.0;
    }
    lse[h] = N > 0 ? big + log(sum) : -INFINITY;
  }
  free(w);
}

/* LSE fusion identity ([HGCA] "What carries the argument": for a partition
 * of keys into I and J the full output is
 * (e^{lse_I} O_I + e^{lse_J} O_J) / (e^{lse_I} + e^{lse_J})), applied to any
 * number of parts in the max-subtracted form (referee minor comment on
 * section 3.3). */
void oracle_fuse(int64_t P, int32_t d, const double *O_parts,
                 const double *lse_parts, double *O, double *lse) {
  double m = -INFINITY;
  for (int64_t i = 0; i < P; ++i)
    if (lse_parts[i] > m) m = lse_parts[i];
  for (int32_t c = 0; c < d; ++c) O[c] = 0.0;
  if (m == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double z = 0.0;
  for (int64_t i = 0; i < P; ++i)
    if (lse_parts[i] != -INFINITY) z += exp(lse_parts[i] - m);
  *lse = m + log(z);
  for (int64_t i = 0; i < P; ++i) {
    if (lse_parts[i] == -INFINITY) continue;
    double w = exp(lse_parts[i] - *lse);
    for (int32_t c = 0; c < d; ++c) O[c] += w * O_parts[i * d + c];
  }
}

/* Moving average with decay r ([LFPS] "What carries the argument" and
 * "Assumptions & free parameters": decay factor r = 0.95; [HGCA] MAW, whose
 * own factor is not reported): MAW <- r MAW + (1 - r) a for every entry
 * given. */
void oracle_maw_update(double *maw, const double *a, int64_t n_blk, double r) {
  for (int64_t i = 0; i < n_blk; ++i) maw[i] = r * maw[i] + (1.0 - r) * a[i];
}

/* One MAW step of a unit (R10): a block all of whose tokens lie in D takes
 * the average of its dense-partial mass a (oracle_dense_mass); every other
 * block keeps its value.  [HGCA] keeps the newest KV blocks in a GPU-side
 * circular buffer and evicts old blocks whole ("What carries the argument"),
 * and the average of an entry that has left the GPU side is frozen (referee
 * report on section 3.2.2 / Algorithm 1): a block leaves the GPU side when
 * its oldest token leaves D. */
void oracle_maw_step(double *maw, const double *a, int64_t N, int32_t S,
                     int32_t n_s, int32_t W, double r) {
  int64_t n_blk = oracle_num_blocks(N, S);
  for (int64_t i = 0; i < n_blk; ++i) {
    int inside = 1;
    for (int64_t j = i * S; j < (i + 1) * S && j < N; ++j)
      if (!oracle_in_dense(j, N, n_s, W)) inside = 0;
    if (inside) maw[i] = r * maw[i] + (1.0 - r) * a[i];
  }
}
