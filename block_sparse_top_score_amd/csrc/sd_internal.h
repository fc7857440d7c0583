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
constexpr int kChunkTokens = 256;    // token slots of one split-K chunk

// Per-KV-head constants, resident in device memory for the context's life
// (read with uniform addresses, so they come through the scalar cache).
struct HeadInfo {
  int32_t S;             // block size in tokens
  int32_t ppm;           // budget, parts per million of N
  int32_t nbmax;         // ceil(max_seq_len / S): blocks per sequence
  int32_t chunk_blocks;  // kChunkTokens / S
  int64_t summ_off;      // uint16 offset of this head's summary region
  int64_t maw_off;       // float offset of this head's MAW region
};

// Sequences of one launch: slot id and current token count.
struct SeqBatch {
  int32_t n;
  int32_t seq[kLaunchSeqs];
  int32_t len[kLaunchSeqs];
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
  uint16_t *k;     // [num_pages][Hkv][16][d] bf16
  uint16_t *v;     // [num_pages][Hkv][16][d] bf16
  int32_t *pt;     // [max_seqs][pages_per_seq]
  uint16_t *summ;  // per head h: [max_seqs][d/4][nbmax_h][8] bf16
  float *maw;      // per head h: [max_seqs][nbmax_h]
};

// Problem constants common to every kernel of a context.
struct Dims {
  int32_t Hq, Hkv, G, d;
  int32_t pages_per_seq;
  int32_t n_sink, window;
  float scale_log2;  // softmax scale * log2(e)
  float maw_decay;
  float maw_beta;
  int32_t key_stride;  // uint32 keys per (seq, kv head) in scratch
  int32_t u_cap;       // attended-block slots per (seq, kv head)
};

// Scratch owned by the context.
struct Scratch {
  double2 *qpm;   // [kLaunchSeqs][Hq][d] (min(q,0), max(q,0)) in double
  uint32_t *keys; // [max_seqs][Hkv][key_stride] order-preserving fp32 keys
  uint8_t *flags; // [max_seqs][Hkv][key_stride] MAW threshold flags
  float *lmass;   // [max_seqs][Hq][u_cap] per attended block log-mass
  int32_t *ublk;  // [max_seqs][Hkv][u_cap] block id of attended slot u
  int32_t *ucnt;  // [max_seqs][Hkv] number of attended blocks
};

// ---- launchers (sd_kernels.hip) -------------------------------------------
// Each returns hipSuccess or the launch error; none synchronises.

hipError_t launch_append(const LayerDev &L, const HeadInfo *d_heads,
                         const Dims &dm, const AppendBatch &b, int max_new,
                         int max_touch_blocks, const uint16_t *k_new,
                         const uint16_t *v_new, hipStream_t st);

hipError_t launch_select(const LayerDev &L, const HeadInfo *d_heads,
                         const Dims &dm, const Scratch &sc, const SeqBatch &b,
                         int max_blocks, const uint16_t *q, int32_t *blk_idx,
                         int32_t *blk_cnt, int32_t k_cap, hipStream_t st);

hipError_t launch_attend(const LayerDev &L, const HeadInfo *d_heads,
                         const Dims &dm, const Scratch &sc, const SeqBatch &b,
                         const uint16_t *q, const int32_t *blk_idx,
                         const int32_t *blk_cnt, int32_t k_cap, float *o_part,
                         float *lse_part, int32_t p_cap, hipStream_t st);

// with_maw: update MAW from the attend scratch; L may be null otherwise.
hipError_t launch_fuse(const LayerDev *L, const HeadInfo *d_heads,
                       const Dims &dm, const Scratch &sc, const SeqBatch &b,
                       bool with_maw, const float *o_part,
                       const float *lse_part, int32_t p_cap, float *o,
                       float *lse, hipStream_t st);

hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t st);

}  // namespace sd
