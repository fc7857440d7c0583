/*
 * sparse_decode.h - C ABI of libsparse_decode.so: decode-step block-sparse
 * top-score attention over a paged KV cache on one MI355X (gfx950).
 *
 * One decode step of one layer is four stream-ordered calls:
 *
 *   append_kv    the step's new token(s) join the paged store; per-block key
 *                summaries are kept exact.
 *   select_topk  every KV block is scored against the query and a top-k block
 *                set is chosen per KV head under a token budget.
 *   sparse_attend  split-K attention over the dense sinks + recent window and
 *                the selected blocks, emitting normalised (O_i, lse_i)
 *                partials.
 *   fuse_lse     the partials are merged with the exact log-sum-exp identity
 *                and the per-block moving average of attention weight (MAW)
 *                is updated on the device.
 *
 * Pages whose method this follows (title; section or figure):
 *   [FLX]  "An Efficient Hybrid Sparse Attention with CPU-GPU Parallelism for
 *          Long-Context Inference" - block-sparse attention parameterised by
 *          (block size, budget) with per-head top-k (Core claim; Figure 2(d);
 *          Figure 8 "(blk, bgt)"), dense attention sinks (Figure 3(c)).
 *   [SPIN] "Unifying Sparse Attention with Hierarchical Memory for Scalable
 *          Long-Context LLM Serving" - sparsity granularities mapped onto a
 *          shared page-based KV substrate (What carries the argument); Select
 *          then Retrieve, decode only (Figure 3).
 *   [HGCA] "HGCA: Hybrid GPU-CPU Attention for Long Context LLM Inference" -
 *          dense recent window + sparse selected entries merged by the exact
 *          LSE identity; MAW threshold beta / #dense entries (What carries the
 *          argument); append vs decode processes (Figure 2).
 *   [LFPS] "Learn from the Past: Fast Sparse Indexing for Large Language Model
 *          Decoding" - decay r = 0.95 of the running score tables (What carries
 *          the argument); block-based Quest baseline (Extended reading notes).
 *
 * Conventions for every call:
 *   - Pointers marked "dev" are device pointers the caller owns (allocated on
 *     the context's device); "host" pointers are read before the call returns.
 *     Nothing is freed on the caller's behalf.
 *   - bf16 tensors are raw 16-bit patterns (IEEE binary32 upper halves).
 *   - Every argument is validated on the host before anything is enqueued; a
 *     negative status means nothing was enqueued and sd_last_error() says why.
 *   - Work is asynchronous on the configured stream.  Device faults surface as
 *     SD_EHIP at the next sd_sync()/sparse_decode_destroy().
 *   - A context is bound to one device and one stream and is not thread-safe.
 *   - No C++ exception crosses this boundary.
 */
#ifndef SPARSE_DECODE_H
#define SPARSE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sd_ctx sd_ctx;
typedef int32_t sd_status;

#define SD_OK 0
#define SD_EINVAL (-1)       /* bad argument or configuration               */
#define SD_ENOMEM (-2)       /* page pool exhausted or device alloc failed  */
#define SD_EHIP (-3)         /* a HIP runtime call failed                   */
#define SD_EUNSUPPORTED (-4) /* valid request outside the built kernels     */
#define SD_ESTATE (-5)       /* call out of order (e.g. fuse without attend) */

/* Library limits. */
#define SD_PAGE_SIZE 16         /* tokens per KV page                       */
#define SD_MAX_GROUP 8          /* query heads per KV head                  */
#define SD_MAX_KV_HEADS 64
#define SD_MAX_BLOCK 64         /* largest block size in tokens             */

typedef struct {
  int32_t max_seqs;       /* sequence slots; seq ids are 0..max_seqs-1       */
  int32_t num_layers;     /* independent layers (each owns its own pool)     */
  int32_t num_q_heads;    /* Hq                                              */
  int32_t num_kv_heads;   /* Hkv; Hq % Hkv == 0, Hq/Hkv <= SD_MAX_GROUP      */
  int32_t head_dim;       /* d in {64, 128}                                  */
  int32_t page_size;      /* must be SD_PAGE_SIZE                            */
  int32_t num_pages;      /* pages per layer in the pool                     */
  int32_t max_seq_len;    /* tokens per sequence                             */
  int32_t sink_tokens;    /* n_s: first tokens always attended ([FLX] sinks) */
  int32_t recent_window;  /* W: last tokens always attended ([HGCA] window)  */
  const int32_t *block_size; /* host [Hkv]: block size per KV head, a multiple
                                of 16 and <= 64 ([FLX] head-specific
                                granularity)                                 */
  const int32_t *budget_ppm; /* host [Hkv]: budget per KV head as parts per
                                million of the current token count N; k =
                                min(|candidates|, ceil(ppm*N/(1e6*S)))       */
  float softmax_scale;    /* 0 -> 1/sqrt(head_dim)                           */
  float maw_decay;        /* r in [0,1); 0 -> 0.95 ([LFPS] r = 0.95)         */
  float maw_beta;         /* beta of the MAW flag; <= 0 turns the flag off   */
  uint64_t page_shuffle_seed; /* 0: pages handed out in order; else a seeded
                                 random permutation of the free list         */
  void *stream;           /* hipStream_t; NULL = the default stream          */
  int32_t select_per_query_head; /* 0: one block set per KV head, ranked by
                                    the group's largest bound; 1: one set per
                                    query head, ranked by its own bound
                                    ([FLX] Figures 4 and 5: heads counted and
                                    budgeted one query head at a time).  With
                                    1, select_topk writes and sparse_attend
                                    reads blk_idx [n][Hq][k_cap] and blk_cnt
                                    [n][Hq]; the pages of the union of a KV
                                    head's sets are read once, each query head
                                    attends D and its own blocks; the
                                    one-launch step returns SD_EUNSUPPORTED */
  int32_t lfps_select;    /* 1: select among the candidates of the
                             learn-from-the-past tables ([LFPS] What carries
                             the argument, Figure 4) at block granularity: a
                             vertical table per block and a slash table per
                             block offset from the newest block; candidates
                             above tau = mean + a (max - mean) of either table,
                             grown by the offsets {-1,0,1,2} and kept when above
                             a table's mean and outside D; only they are scored
                             (exact group bound), the k = min(|C|, budget)
                             best taken.  fuse_lse then updates the tables with
                             decay maw_decay by each block's mass under the
                             softmax over the attended set.  Needs maw_beta <= 0
                             and select_per_query_head = 0; the one-launch step
                             returns SD_EUNSUPPORTED.  Tables start at 0
                             (sd_lfps_init fills them from the prefill)       */
  float lfps_a;           /* the threshold parameter a in [0, 1] ([LFPS]
                             Assumptions & free parameters: 0.2)             */
} sd_config;

/* Host-only check of a configuration (no device is touched).  err may be NULL;
 * otherwise up to err_len bytes of explanation are written on failure. */
sd_status sd_validate_config(const sd_config *cfg, char *err, size_t err_len);

/* Create a context on the current HIP device: allocates the per-layer KV
 * pools [num_pages][Hkv][16][d] bf16 (K and V), page tables, block summaries,
 * MAW tables and scratch.  All sequences start empty.  SD_EUNSUPPORTED if a
 * unit could need more than 256 partial slots per query head (budget x
 * max_seq_len too large for the block size) or if the sinks and the recent
 * window span more than 2048 pages. */
sd_status sparse_decode_init(const sd_config *cfg, sd_ctx **out);

/* Synchronise the stream and free every device buffer of the context. */
sd_status sparse_decode_destroy(sd_ctx *ctx);

/* Sizes callers must allocate: k_cap = largest block count select_topk may
 * write per (sequence, KV head); p_cap = largest number of split-K partials
 * sparse_attend may write per query head. */
sd_status sd_caps(const sd_ctx *ctx, int32_t *k_cap, int32_t *p_cap);

/* Append n_new[i] tokens to sequence seq_ids[i] of one layer ([HGCA] append
 * process, Figure 2; [SPIN] page substrate).  k_bf16, v_bf16: dev
 * [sum_i n_new[i]][Hkv][d] bf16, rows of sequence i after those of i-1.
 * Pages come from the layer's free list; if the pool cannot hold every new
 * token the call fails with SD_ENOMEM and changes nothing.  The per-block
 * min/max key summaries of every touched block are updated exactly (blocks of
 * each KV head's own size).  New blocks start with MAW 0.
 * seq_ids, n_new: host [n_seqs]; ids must be distinct. */
sd_status append_kv(sd_ctx *ctx, int32_t layer, int32_t n_seqs,
                    const int32_t *seq_ids, const int32_t *n_new,
                    const void *k_bf16, const void *v_bf16);

/* Score every block of each (sequence, KV head) and select its top-k blocks
 * ([FLX] Core claim and Figure 2(d); Quest-style bound).  For block i,
 * U_h(i) = sum_c max(q_hc*min_ic, q_hc*max_ic) is accumulated in double in
 * channel order and the group score is the max over the KV head's query heads,
 * rounded once to fp32.  Candidates are blocks with a token outside the dense
 * set D = [0, n_s) U [N-W, N).  With maw_beta > 0 a block whose
 * MAW*|D| > beta*S is ranked before all others ([HGCA] threshold).  Order:
 * (flag desc, score desc, index asc); the first k are written ascending.
 * q_bf16: dev [n_seqs][Hq][d].  blk_idx: dev [n_seqs][Hkv][k_cap] int32
 * (entries past the count are left untouched).  blk_cnt: dev [n_seqs][Hkv].
 * With select_per_query_head each query head h ranks by its own U_h (the
 * same k, flags and order) and blk_idx / blk_cnt are [n_seqs][Hq][k_cap] /
 * [n_seqs][Hq]. */
sd_status select_topk(sd_ctx *ctx, int32_t layer, int32_t n_seqs,
                      const int32_t *seq_ids, const void *q_bf16,
                      int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap);

/* Split-K attention over T = D U tokens(selected blocks), a set ([HGCA] dense
 * window + sparse entries; flash-decoding split).  The attended tokens of a
 * (sequence, KV head) are cut into 16-token pages that P parts share (P <=
 * p_cap, about 40 pages per part); part p of query head h writes
 * o_part[n][h][p][:] (fp32, normalised within the part) and
 * lse_part[n][h][p] (natural log of the part's sum of exp(scaled logits));
 * slots [P, p_cap) get lse = -inf and O = 0.  blk_idx / blk_cnt are as written by
 * select_topk (ascending, distinct; a repeated entry would count its tokens
 * twice); entries outside [0, n_blk) attend nothing.  The log softmax mass of
 * each dense page, which fuse_lse needs for MAW, is kept inside the context
 * for this layer.
 * With select_per_query_head, blk_idx / blk_cnt are per query head (as
 * select_topk writes them): query head h attends D U tokens(its own
 * entries); the union of a KV head's sets is formed first (entries outside
 * the blocks that can hold a candidate are dropped, repeats count once) and
 * its pages are read once for the whole group. */
sd_status sparse_attend(sd_ctx *ctx, int32_t layer, int32_t n_seqs,
                        const int32_t *seq_ids, const void *q_bf16,
                        const int32_t *blk_idx, const int32_t *blk_cnt,
                        int32_t k_cap, float *o_part, float *lse_part,
                        int32_t p_cap);

/* Exact LSE fusion of the partials ([HGCA] What carries the argument, in the
 * max-subtracted form): lse = m + log sum_p e^{lse_p - m}, O = sum_p
 * e^{lse_p - lse} O_p; parts with lse = -inf drop out.  o: dev [n_seqs][Hq][d]
 * fp32, lse: dev [n_seqs][Hq] fp32.
 * layer >= 0: must follow sparse_attend of the same layer and sequences
 * (SD_ESTATE otherwise); MAW of each (sequence, KV head) is then updated
 * from the dense partial alone ([HGCA] What carries the argument and the
 * referee report on section 3.2.2 / Algorithm 1: the moving average is fed by
 * the GPU-side window's weights, normalised over that window, and frozen once
 * an entry has left it; [LFPS] decay r): every block whose tokens all lie in
 * D takes MAW <- r*MAW + (1-r)*a, a = the group-mean mass of the block under
 * the softmax over D alone; every other block keeps its MAW.
 * layer == -1: pure fusion of n_seqs*Hq heads over all p_cap slots, no MAW
 * (seq_ids may be NULL); p_cap <= 256 (SD_EUNSUPPORTED otherwise).
 * o_part must be 16-byte aligned (SD_EINVAL otherwise). */
sd_status fuse_lse(sd_ctx *ctx, int32_t layer, int32_t n_seqs,
                   const int32_t *seq_ids, const float *o_part,
                   const float *lse_part, int32_t p_cap, float *o, float *lse);

/* Fused decode step of one layer ([HGCA] Figure 2: the append process, then
 * the decode process; [SPIN] Figure 3: select, then attend; [HGCA] What
 * carries the argument: partials merged by the exact LSE identity): the
 * optional append of one token per sequence (k_new, v_new: dev
 * [n_seqs][Hkv][d] bf16, both NULL to skip), then select_topk +
 * sparse_attend + fuse_lse, in one launch per 64 sequences (after the
 * append's): block scoring with the top-k of each (sequence, KV head) done by
 * its last scoring workgroup, the attention parts, and the LSE fusion and MAW
 * update done by the last part of each (sequence, KV head).  The selection
 * and MAW equal the separate calls' bit for bit; O and lse equal them to fp32
 * rounding (the step visits the selected pages in key order, the separate
 * attend call in ascending order).
 * blk_idx/blk_cnt/o_part/lse_part are written as by the separate calls, except
 * that partial slots a unit does not use are left unspecified.  o_part must be
 * 16-byte aligned (SD_EINVAL otherwise).  A selection wait that runs out of
 * time (it cannot in a correct launch) makes the next sd_sync return
 * SD_EHIP. */
sd_status sparse_decode_step(sd_ctx *ctx, int32_t layer, int32_t n_seqs,
                             const int32_t *seq_ids, const void *k_new,
                             const void *v_new, const void *q_bf16,
                             int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap,
                             float *o_part, float *lse_part, int32_t p_cap,
                             float *o, float *lse);

/* sparse_decode_step for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, results and errors as sparse_decode_step, but the step's
 * scratch (per-block keys, score-tile candidate lists, top-k spill arrays,
 * selection hand-off tags, arrival counters, page log-masses) lives in one
 * library-wide static device array of SD_STATIC_SCRATCH_BYTES per GPU (held
 * from the library's first context on that GPU until the process ends)
 * instead of the context's own buffers.  The call allocates nothing: no
 * hipMalloc/hipFree and no host allocation.  It first clears, with a fill
 * kernel on the context's stream, the part of the array that must start at
 * zero.  SD_EUNSUPPORTED if the context's scratch (about max_seqs * Hkv *
 * (28 * ceil(max_seq_len / (256 * min block size)) * 256 + 16 + 8 * k_cap)
 * bytes, plus the page log-masses) exceeds the array; SD_EHIP if the array's
 * device address could not be resolved.  Every call on one GPU, from any
 * context or stream, shares the array: calls that overlap in time race and
 * give wrong results, so callers must order them (one stream, or events). */
#define SD_STATIC_SCRATCH_BYTES (32u << 20)
sd_status sparse_decode_step_noalloc(sd_ctx *ctx, int32_t layer, int32_t n_seqs,
                                     const int32_t *seq_ids, const void *k_new,
                                     const void *v_new, const void *q_bf16,
                                     int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap,
                                     float *o_part, float *lse_part, int32_t p_cap,
                                     float *o, float *lse);

/* Return a sequence slot to empty in every layer: its pages go back to the
 * free lists, its length becomes 0 and its MAW table is cleared.  Waits for
 * the stream first. */
sd_status sd_release_seq(sd_ctx *ctx, int32_t seq_id);

/* Current token count of a sequence in a layer (host-side bookkeeping). */
sd_status sd_seq_len(const sd_ctx *ctx, int32_t layer, int32_t seq_id,
                     int32_t *len);

/* Wait for all work on the context's stream; reports deferred HIP errors. */
sd_status sd_sync(sd_ctx *ctx);

/* Learn-from-the-past tables of one layer from the prefill ([LFPS]
 * Assumptions & free parameters: the last s = 32 prefill steps initialise the
 * tables, Eq. (4)): for each sequence the queries of its last s_steps
 * positions p = N - s_steps + u, u = 0 .. s_steps-1 (q_prefill: dev
 * [n_seqs][s_steps][Hq][d] bf16), each attending causally and densely to
 * [0, p]; the tables are zeroed, then take the s_steps block-mass updates in
 * order.  Needs lfps_select; SD_EINVAL for s_steps < 1 or more than N of a
 * sequence.  Allocates and frees a scratch of n_seqs * Hkv * s_steps *
 * max_blocks floats (not for use inside graph capture). */
sd_status sd_lfps_init(sd_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                       const void *q_prefill, int32_t s_steps);

/* Text of the last error on this context (never NULL). */
const char *sd_last_error(const sd_ctx *ctx);


/* Debug/parity export of one sequence of one layer to host memory (waits for
 * the stream).  Layouts:
 *   SD_DEBUG_PAGE_TABLE  int32 [ceil(max_seq_len/16)] page ids (in use: the
 *                        first ceil(len/16))
 *   SD_DEBUG_SUMMARY     for each KV head h in order: bf16 pairs
 *                        [ceil(len/S_h)][d][2] = (min, max)
 *   SD_DEBUG_MAW         for each KV head h in order: fp32 [ceil(len/S_h)]
 *   SD_DEBUG_K / _V      bf16 [len][Hkv][d], gathered through the page table
 *   SD_DEBUG_LFPS        for each KV head h in order: fp32 [2][ceil(len/S_h)],
 *                        the vertical table by block, then the slash table by
 *                        block offset (SD_EUNSUPPORTED without lfps_select)
 *   SD_DEBUG_LFPS_CAND   int32 [Hkv]: the number of table candidates |C| of
 *                        each KV head's last select_topk (lfps_select only)
 *   SD_DEBUG_SCORES      for each KV head h in order: fp32 [1 + ceil(len/S_h)]:
 *                        element 0 the error bound eps the head's last
 *                        selection used, then per block the approximate group
 *                        score that selection ranked (the fp32 value of its
 *                        order key); NaN for blocks that were not scored as
 *                        candidates, and everywhere on a head that selects
 *                        nothing (SD_EUNSUPPORTED with one selection per
 *                        query head).  Every scored block's exact score lies
 *                        within eps of its approximate one ([LFPS] Core claim:
 *                        the selection is the exact top-k; blocks within the
 *                        band of the k-th are re-scored exactly).  Valid right
 *                        after select_topk or sparse_decode_step of this layer
 *                        and sequence (the scratch it reads is shared by every
 *                        layer; the allocation-free step keeps its own).
 * bytes must equal the size reported by sd_debug_bytes. */
#define SD_DEBUG_PAGE_TABLE 0
#define SD_DEBUG_SUMMARY 1
#define SD_DEBUG_MAW 2
#define SD_DEBUG_K 3
#define SD_DEBUG_V 4
#define SD_DEBUG_SCORES 5
#define SD_DEBUG_LFPS 6
#define SD_DEBUG_LFPS_CAND 7
sd_status sd_debug_bytes(const sd_ctx *ctx, int32_t what, int32_t layer,
                         int32_t seq_id, size_t *bytes);
sd_status sd_debug_copy(sd_ctx *ctx, int32_t what, int32_t layer,
                        int32_t seq_id, void *host_dst, size_t bytes);

/* Overwrite the MAW table of one (layer, sequence) from host fp32 values laid
 * out as SD_DEBUG_MAW (test hook for threshold cases; waits for the stream). */
sd_status sd_debug_set_maw(sd_ctx *ctx, int32_t layer, int32_t seq_id,
                           const float *host_src, size_t bytes);

/* Overwrite the learn-from-the-past tables of one (layer, sequence) from host
 * fp32 values laid out as SD_DEBUG_LFPS (test hook; waits for the stream). */
sd_status sd_debug_set_lfps(sd_ctx *ctx, int32_t layer, int32_t seq_id,
                            const float *host_src, size_t bytes);

/* Streaming-read probe, for measurement only (no part of the decode path):
 * the HBM read rate a plain kernel reaches on this GPU, against which the
 * decode step's own rate can be read.  Reads `bytes` bytes at `src` once
 * (device memory, 16-byte aligned, bytes > 0 and a multiple of 16) with
 * `sink_words` workgroups of 256 threads, each thread reading 16-byte words
 * grid-stride, eight in flight; writes the XOR of each workgroup's words to
 * sink[0 .. sink_words) (device, caller-owned).  Needs no context;
 * stream-ordered and asynchronous on `stream` (hipStream_t, NULL = the null
 * stream).  Returns SD_EINVAL (nothing launched) for a NULL pointer, a
 * misaligned src, a bad size or sink_words < 1; SD_EHIP if the launch fails. */
sd_status sd_read_probe(const void *src, size_t bytes, uint32_t *sink, int32_t sink_words,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_DECODE_H */
