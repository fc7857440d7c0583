// sd_internal.h - types shared by the host runtime and the gfx950 kernels of
// libsparse_decode.so.  Not part of the public ABI (include/sparse_decode.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "sparse_decode.h"

namespace sd {

constexpr int kPage = SD_PAGE_SIZE;  // tokens per KV page
constexpr int kLaunchSeqs = 64;      // sequences per kernel launch
constexpr int kPartPages = 40;       // attended pages per attention workgroup (target)
constexpr int kScoreTile = 256;      // blocks scored by one workgroup
constexpr int kTileAhead = 2;        // 16-block summary groups a score wave keeps in flight
constexpr int kTopkRegRows = 20;     // top-k rows of 64 block words kept in registers
constexpr int kTopkUnc = 512;        // uncertain blocks the top-k lists in LDS
constexpr int kFastTiles = 8;        // score tiles per unit of the fast top-k, at most
constexpr int kPtLds = 4096;         // page-table entries a selected chunk copies to LDS, at most
constexpr int kFuseSlots = 256;      // partial slots per query head, at most
constexpr int kFuseDenseLds = 2048;  // dense pages (sinks + window) per unit, at most
constexpr int kWideM = 40;           // blocks per thread of the four-wave top-k: units up to 10240 blocks

// Units the four-wave top-k ranks (more blocks than the one-wave top-k keeps
// in registers).
__host__ __device__ inline bool wide_unit(int n_blk) {
  return n_blk > kTopkRegRows * 64 && n_blk <= 256 * kWideM;
}
// Slot of block blk's key in its unit's key array: the block index, except
// in units the four-wave top-k ranks, where thread t's blocks sit at t,
// t + 256, ..., so that its loads are coalesced.
__host__ __device__ inline int key_slot(int blk, int n_blk) {
  if (!wide_unit(n_blk)) return blk;
  const int m = (n_blk + 255) / 256, t = blk / m;
  return (blk - t * m) * 256 + t;
}

// Per-KV-head constants, resident in device memory for the context's life
// (read with uniform addresses, so they come through the scalar cache).
struct HeadInfo {
  int32_t S;             // block size in tokens
  int32_t ppm;           // budget, parts per million of N
  int32_t nbmax;         // ceil(max_seq_len / S): blocks per sequence
  int32_t kcap;          // most blocks ever selected on this head
  int64_t summ_off;      // uint16 offset of this head's summary region
  int64_t maw_off;       // float offset of this head's MAW region
};

// Sequences of one launch: slot id and current token count; max_scored =
// the most blocks any of its units scores (blocks that can hold a candidate).
struct SeqBatch {
  int32_t n;
  int32_t seq[kLaunchSeqs];
  int32_t len[kLaunchSeqs];
  int32_t max_scored;
};

// Per-launch append plan (host-computed).
struct AppendBatch {
  int32_t n;
  int32_t seq[kLaunchSeqs];
  int32_t old_len[kLaunchSeqs];
  int32_t n_new[kLaunchSeqs];
  int32_t src_row[kLaunchSeqs];  // first row of this sequence in k_new/v_new
};

// Device state of one layer.
struct LayerDev {
  uint16_t *k;     // [num_pages][Hkv][d/8][16][8] bf16: per page and head, each group of
                   // 8 channels holds the 16 tokens' values contiguously (256 B)
  uint16_t *v;     // [num_pages][Hkv][d][16] bf16: V pages stored transposed
  int32_t *pt;     // [max_seqs][pages_per_seq]
  uint16_t *summ;  // per head h: [max_seqs][d/4][nbmax_h][8] bf16
  float *maw;      // per head h: [max_seqs][nbmax_h]
  float *phi;      // learn-from-the-past tables, per head h: [max_seqs][2][nbmax_h]
                   // (vertical by block, then slash by block offset); NULL unless on
};

// Problem constants common to every kernel of a context.
struct Dims {
  int32_t Hq, Hkv, G, d;
  int32_t pages_per_seq;
  int32_t n_sink, window;
  float scale_log2;    // softmax scale * log2(e)
  float maw_decay;
  float maw_beta;
  int32_t key_stride;  // uint32 keys per (seq, kv head) in scratch
  int32_t lm_sel0;     // log-mass slots of dense pages; selected pages follow
  int32_t lm_cap;      // log-mass slots per (seq, query head)
  int32_t kcap;        // selected block slots per (seq, kv head)
  int32_t pqh;         // 1: one selection per query head (unit arrays of the
                       // selection are per query head), 0: per KV head
  int32_t ucap;        // entries of a KV head's union of its query heads' sets
  int32_t lfps;        // 1: selection among the learn-from-the-past table candidates
  float lfps_a;        // its threshold parameter a
};

// Scratch owned by the context.  Per-unit arrays have key_stride entries, a
// multiple of 64.
struct Scratch {
  // (per-query-head selection: [max_seqs][Hq] in place of [max_seqs][Hkv]
  // in keyflag, keys, ulist, ukeys and unit_acc)
  unsigned long long *keyflag;  // [max_seqs][Hkv][key_stride] key | MAW flag << 32
  uint32_t *keys;    // [max_seqs][Hkv][key_stride] top-k words past LDS (long units)
  int32_t *ulist;    // [max_seqs][Hkv][key_stride] uncertain blocks past LDS
  uint32_t *ukeys;   // [max_seqs][Hkv][key_stride] their exact keys
  uint32_t *unit_acc;  // [max_seqs][Hkv][4] error bound (float bits, max) and
                       // flagged candidates (count) of the score tiles, 0 between
                       // steps; the bound the unit's last selection used; the
                       // table candidates of its last learn-from-the-past selection
  float *lm_pg;      // [max_seqs][Hq][lm_cap] log softmax mass of each attended page
  uint32_t *arrive;  // [max_seqs][Hkv][4] last-arriver counters (kept at 0): score
                     // tiles, attention parts, dense pages done (+ the top-k), spare
  unsigned long long *cand;  // [max_seqs][Hkv][key_stride] per-tile lists of the 64
                             // largest keys (key << 32 | ~block), tile t's at [64 t, 64 t + 64)
  unsigned long long *rtag;    // [max_seqs][Hkv] step << 32 | selected count, published
                               // after the selection
  unsigned long long *seltag;  // [max_seqs][Hkv][kcap] step << 32 | block of the selection
  uint32_t *err;     // [1] nonzero once a step kernel's wait ran out of time
  int32_t *uni;      // per-query-head selection: [max_seqs][Hkv][ucap] the union of
                     // the group's sets, ascending, block | head mask << 24
  int32_t *ucnt;     //   and its size, [max_seqs][Hkv]
};

// Everything a kernel needs about the context (passed by value).
struct Ctx {
  LayerDev L;
  const HeadInfo *heads;
  Dims dm;
  Scratch sc;
};

// ---- launchers (sd_kernels.hip) -------------------------------------------
// Each returns hipSuccess or the launch error; none synchronises.

hipError_t launch_append(const Ctx &c, const AppendBatch &b, int max_new,
                         int max_touch_blocks, const uint16_t *k_new,
                         const uint16_t *v_new, hipStream_t st);

// Score + top-k (last arriver per unit).
hipError_t launch_select(const Ctx &c, const SeqBatch &b, int max_blocks, const uint16_t *q,
                         int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, hipStream_t st);

// Selection among the learn-from-the-past table candidates (one workgroup
// per (sequence, KV head)); max_blocks: the most blocks of a unit.
hipError_t launch_lfps_select(const Ctx &c, const SeqBatch &b, int max_blocks, const uint16_t *q,
                              int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, hipStream_t st);

// The tables from the last s_steps prefill positions (q_prefill:
// [n][s_steps][Hq][d] bf16); A: scratch [n][Hkv][s_steps][key_stride] floats
// for the block masses.
hipError_t launch_lfps_init(const Ctx &c, const SeqBatch &b, int max_blocks, const uint16_t *q_prefill,
                            int s_steps, float *A, hipStream_t st);

// Per-query-head selection: the union of each KV head's query-head sets
// (blk_idx [n][Hq][k_cap], blk_cnt [n][Hq]) into the context's scratch, for
// the attention.
hipError_t launch_union(const Ctx &c, const SeqBatch &b, const int32_t *blk_idx,
                        const int32_t *blk_cnt, int32_t k_cap, hipStream_t st);

// Attention: P workgroups per unit, one partial slot each (slots [P, p_cap)
// emptied); keeps the dense pages' log-masses for the fusion call.
hipError_t launch_attend(const Ctx &c, const SeqBatch &b, int P, const uint16_t *q,
                         const int32_t *blk_idx, const int32_t *blk_cnt, int32_t k_cap,
                         float *o_part, float *lse_part, int32_t p_cap, hipStream_t st);

// The whole step in one launch: scoring, top-k, P attention parts per unit,
// fusion and MAW (epoch: a nonzero number that differs between launches;
// ptl_cap: page-table entries a part may copy to LDS, 0 for none).  k_new,
// v_new ([n][Hkv][d], or null): the token each sequence has just been given
// (its page and length already set on the host); the attention reads it
// from these rows and the fusion writes it into the pool and the summaries.
// Only for a token whose block lies wholly in the recent window.
hipError_t launch_step(const Ctx &c, const SeqBatch &b, int max_blocks, int P, const uint16_t *q,
                       int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, float *o_part,
                       float *lse_part, int32_t p_cap, float *o, float *lse, uint32_t epoch,
                       int ptl_cap, const uint16_t *k_new, const uint16_t *v_new,
                       hipStream_t st);

// Workgroups of the one-launch step that can be resident on the device at
// once (0 if unknown).
int step_capacity(const Ctx &c, int max_blocks, int ptl_cap);

// Fusion of the partials: with_maw = the P slots of the attend call and MAW
// (layer call); otherwise every slot of p_cap <= kFuseSlots is fused (layer -1).
// (with the learn-from-the-past tables on, sel_idx / sel_cnt / k_cap are the
// selection the attention call took, and max_blocks the most blocks of a unit)
hipError_t launch_fuse(const Ctx &c, const SeqBatch &b, bool with_maw, int P,
                       const float *o_part, const float *lse_part, int32_t p_cap,
                       float *o, float *lse, const int32_t *sel_idx, const int32_t *sel_cnt,
                       int32_t k_cap, int max_blocks, hipStream_t st);

hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t st);
hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t st);

}  // namespace sd
