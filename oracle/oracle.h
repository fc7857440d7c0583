/*
 * oracle.h - plain, slow, double-precision CPU oracle for decode-step
 * block-sparse top-score attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP path and must never be used to
 * produce a result of the product path.
 *
 * Every function works on ONE (sequence, KV head) unit, on the logical token
 * order (token j is row j), with bf16 inputs given as their raw 16-bit
 * patterns and widened exactly to double.  Plain loops, no blocking, no
 * reordering beyond what the definitions state.
 *
 * Pages cited (title; the section, figure or equation named at each use):
 *   [FLX]  "An Efficient Hybrid Sparse Attention with CPU-GPU Parallelism for
 *          Long-Context Inference" (Fluxion, pith.science 2605.07719)
 *   [SPIN] "Unifying Sparse Attention with Hierarchical Memory for Scalable
 *          Long-Context LLM Serving" (pith.science 2604.26837)
 *   [HGCA] "HGCA: Hybrid GPU-CPU Attention for Long Context LLM Inference"
 *          (pith.science 2507.03153)
 *   [LFPS] "Learn from the Past: Fast Sparse Indexing for Large Language Model
 *          Decoding" (pith.science OT6KG5FY, arXiv 2506.15704)
 *   [IDX]  mlsanity index page of the Fluxion paper ("Builds on" list).
 *
 * Readings taken where the pages leave a step open (each is listed with its
 * reason in the design notes of the repository):
 *   R1  selection is per KV head; the group score is the max over the G
 *       query heads that share the KV head.
 *   R2  the block score is the channel-wise upper bound
 *       U_h = sum_c max(q_c * m_c, q_c * M_c)   (Quest is only named).
 *   R3  budget is a fraction (parts per million) of the current token count
 *       N; k = min(|C|, ceil(budget_ppm * N / (1e6 * S))); sinks and the
 *       recent window are extra.
 *   R4  the attended set is the union of the dense set and the selected
 *       blocks (a token is counted once).
 *   R5  selection order is (flag desc, fp32 score desc, block index asc).
 *   R8-R10  the moving average of attention weight (MAW) is kept per block.
 *       Its input a is the group-mean softmax mass of the block's dense
 *       tokens under the dense partial alone (softmax over D, HGCA's
 *       GPU-side window); blocks whose tokens all lie in D take
 *       MAW <- r*MAW + (1-r)*a, the others keep their value (frozen from the
 *       step their oldest token leaves D); a block is flagged when
 *       MAW * |D| > beta * S.
 *   R18 scale 1/sqrt(d) unless given; lse is a natural log of scaled logits.
 */
#ifndef BSTS_ORACLE_H
#define BSTS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of blocks of size S covering N tokens (the last may be partial). */
int64_t oracle_num_blocks(int64_t N, int32_t S);

/* Dense set D = [0, min(n_s, N)) U [max(0, N - W), N): its size |D|. */
int64_t oracle_dense_count(int64_t N, int32_t n_s, int32_t W);

/* 1 if token j lies in D. */
int32_t oracle_in_dense(int64_t j, int64_t N, int32_t n_s, int32_t W);

/* Candidate flags: cand[i] = 1 if block i holds at least one token outside D.
 * Returns |C|. */
int64_t oracle_candidates(int64_t N, int32_t S, int32_t n_s, int32_t W,
                          int8_t *cand /* [n_blk] */);

/* k = min(n_cand, ceil(budget_ppm * N / (1e6 * S))) in 64-bit integers. */
int64_t oracle_num_selected(int64_t N, int32_t S, int64_t budget_ppm,
                            int64_t n_cand);

/* Per-block key summaries: for block i, over tokens [iS, min(N,(i+1)S)),
 * mn[i][c] = min_j K[j][c], mx[i][c] = max_j K[j][c] (by value).
 * K row j starts at K + j*ldk (bf16 bits).  mn, mx: [n_blk][d] bf16 bits. */
void oracle_summaries(const uint16_t *K, int64_t ldk, int64_t N, int32_t d,
                      int32_t S, uint16_t *mn, uint16_t *mx);

/* Block scores.  q: [G][d] bf16 bits (query heads of one KV group).
 * Uh[h*n_blk + i] (optional) = sum_c max(q_hc*mn_ic, q_hc*mx_ic) in double;
 * U[i] = max_h Uh; u[i] = (float)U[i] (round to nearest even). */
void oracle_score(const uint16_t *q, int32_t G, int32_t d, const uint16_t *mn,
                  const uint16_t *mx, int64_t n_blk, double *Uh /* or NULL */,
                  double *U, float *u);

/* MAW threshold flag of block i: MAW[i] * |D| > beta * S (beta <= 0: none). */
int32_t oracle_maw_flag(double maw, int64_t n_dense, double beta, int32_t S);

/* Top-k block selection for one unit.  maw may be NULL (no flag).  Writes the
 * k selected block indices in ascending order to sel and returns k.
 * Optional outputs (NULL to skip): U, u as oracle_score; flag[n_blk]. */
int64_t oracle_select(const uint16_t *q, int32_t G, int32_t d,
                      const uint16_t *mn, const uint16_t *mx, int64_t N,
                      int32_t S, int32_t n_s, int32_t W, int64_t budget_ppm,
                      const double *maw, double beta, int32_t *sel,
                      double *U, float *u, int8_t *flag);

/* Per-query-head selection: each of the G query heads of a KV head ranks the
 * candidate blocks by its own bound U_h alone, with the k, MAW flags and
 * order of oracle_select (a group of one head).  sel: [G][ld_sel], row h
 * holds head h's k entries ascending (ld_sel >= n_blk).  Returns k. */
int64_t oracle_select_heads(const uint16_t *q, int32_t G, int32_t d,
                            const uint16_t *mn, const uint16_t *mx, int64_t N,
                            int32_t S, int32_t n_s, int32_t W,
                            int64_t budget_ppm, const double *maw, double beta,
                            int32_t *sel, int64_t ld_sel);

/* Softmax attention of G heads over an explicit list of distinct tokens.
 * s_j = scale * q_h . k_j;  lse_h = log sum_j e^{s_j};
 * O_h = sum_j e^{s_j - lse_h} v_j.  An empty list gives lse = -inf, O = 0.
 * p (optional) [G][n_tok]: the softmax weights e^{s_j - lse_h}. */
void oracle_attend_tokens(const uint16_t *q, int32_t G, int32_t d,
                          const uint16_t *K, int64_t ldk, const uint16_t *V,
                          int64_t ldv, const int64_t *tok, int64_t n_tok,
                          double scale, double *O /* [G][d] */,
                          double *lse /* [G] */, double *p /* or NULL */);

/* Attention over T = D U tokens(sel) (a set).  Returns |T|. */
int64_t oracle_attend(const uint16_t *q, int32_t G, int32_t d,
                      const uint16_t *K, int64_t ldk, const uint16_t *V,
                      int64_t ldv, int64_t N, int32_t S, int32_t n_s,
                      int32_t W, const int32_t *sel, int64_t k, double scale,
                      double *O, double *lse);

/* Per-query-head attention: head h attends T_h = D U tokens(its own
 * selection), row h of sel [G][ld_sel] with k[h] entries.  O: [G][d],
 * lse: [G]. */
void oracle_attend_heads(const uint16_t *q, int32_t G, int32_t d,
                         const uint16_t *K, int64_t ldk, const uint16_t *V,
                         int64_t ldv, int64_t N, int32_t S, int32_t n_s,
                         int32_t W, const int32_t *sel, int64_t ld_sel,
                         const int64_t *k, double scale, double *O,
                         double *lse);

/* Learn-from-the-past tables at block granularity: phi_v[i] for block i
 * (vertical: a fixed absolute position), phi_s[o] for block offset o from the
 * block of the newest token, b = floor((N-1)/S) (slash: a fixed relative
 * position); both [n_blk] and 0 at the start.
 * Candidates: over the entries [0, b] of each table, mean mu and maximum M,
 * threshold tau = mu + a (M - mu); C0 = blocks i <= b with phi_v[i] > tau_v
 * or phi_s[b - i] > tau_s; C0 grows by the offsets {-1, 0, 1, 2}; a grown
 * block is kept when one of its two scores exceeds that table's mean and it
 * holds a token outside D.  inC: [n_blk].  Returns |C|. */
int64_t oracle_lfps_candidates(const double *phi_v, const double *phi_s, int64_t N,
                               int32_t S, int32_t n_s, int32_t W, double a,
                               int8_t *inC);

/* Selection among the table candidates C: the k = min(|C|, ceil(budget*N/S))
 * best of C by (u desc, index asc), u as oracle_score; written ascending to
 * sel.  Returns k.  U, u optional as oracle_select. */
int64_t oracle_lfps_select(const uint16_t *q, int32_t G, int32_t d,
                           const uint16_t *mn, const uint16_t *mx, int64_t N,
                           int32_t S, int32_t n_s, int32_t W, int64_t budget_ppm,
                           const double *phi_v, const double *phi_s, double a,
                           int32_t *sel, double *U, float *u);

/* Attention mass per block under the softmax over the attended set T = D U
 * tokens(sel): a_blk[i] = (1/G) sum_h sum_{j in T, j in block i} p_hj. */
void oracle_attend_mass(const uint16_t *q, int32_t G, int32_t d, const uint16_t *K,
                        int64_t ldk, int64_t N, int32_t S, int32_t n_s, int32_t W,
                        const int32_t *sel, int64_t k, double scale, double *a_blk);

/* Table update after a step with n_blk blocks (b = n_blk - 1):
 * phi_v[i] <- r phi_v[i] + (1-r) a[i] and phi_s[o] <- r phi_s[o] + (1-r) a[b-o]
 * for i, o in [0, b]. */
void oracle_lfps_update(double *phi_v, double *phi_s, const double *a_blk,
                        int64_t n_blk, double r);

/* Tables from the last s prefill positions: zeroed on [0, n_blk(N)), then for
 * u = 0 .. s-1 in order, the query of position p = N - s + u (q: [s][G][d])
 * attends to [0, p] (causal, dense) and its block masses update the tables
 * with n_blk = floor(p/S) + 1. */
void oracle_lfps_init(const uint16_t *q, int32_t s, int32_t G, int32_t d,
                      const uint16_t *K, int64_t ldk, int64_t N, int32_t S,
                      double scale, double r, double *phi_v, double *phi_s);

/* MAW input: a_blk[i] = (1/G) sum_h sum_{j in D, j in block i} p_hj with p_h
 * the softmax of head h over the dense set D alone (0 for blocks with no
 * token in D).  a_blk: [n_blk]. */
void oracle_dense_mass(const uint16_t *q, int32_t G, int32_t d,
                       const uint16_t *K, int64_t ldk, int64_t N, int32_t S,
                       int32_t n_s, int32_t W, double scale, double *a_blk);

/* Independent naive dense softmax attention over all tokens [0, N). */
void oracle_dense(const uint16_t *q, int32_t G, int32_t d, const uint16_t *K,
                  int64_t ldk, const uint16_t *V, int64_t ldv, int64_t N,
                  double scale, double *O, double *lse);

/* LSE fusion of P partial results (O_i normalised over its own part, lse_i
 * natural log): lse = m + log sum_i e^{lse_i - m}, m = max_i lse_i;
 * O = sum_i e^{lse_i - lse} O_i.  Parts with lse = -inf drop out; if all are
 * -inf the result is lse = -inf, O = 0. */
void oracle_fuse(int64_t P, int32_t d, const double *O_parts /* [P][d] */,
                 const double *lse_parts /* [P] */, double *O, double *lse);

/* MAW update for every entry: maw[i] <- r * maw[i] + (1 - r) * a[i]. */
void oracle_maw_update(double *maw, const double *a, int64_t n_blk, double r);

/* One MAW step of a unit of N tokens: blocks whose tokens all lie in D take
 * maw[i] <- r * maw[i] + (1 - r) * a[i]; the others keep maw[i]. */
void oracle_maw_step(double *maw, const double *a, int64_t N, int32_t S,
                     int32_t n_s, int32_t W, double r);

#ifdef __cplusplus
}
#endif

#endif /* BSTS_ORACLE_H */
