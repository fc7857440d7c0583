// sd_kernels.hip - gfx950 kernels of the decode-step block-sparse top-score
// attention path (wave64, hand-written HIP, no library kernels).
//
// Pages cited (title; section or figure):
//   [FLX]  "An Efficient Hybrid Sparse Attention with CPU-GPU Parallelism for
//          Long-Context Inference": per-head top-k block selection under a
//          (block size, budget) configuration (Core claim, Figure 2(d),
//          Figure 8); attention sinks (Figure 3(c)).
//   [SPIN] "Unifying Sparse Attention with Hierarchical Memory for Scalable
//          Long-Context LLM Serving": block granularities over shared pages
//          (What carries the argument); Select then attend (Figure 3).
//   [HGCA] "HGCA: Hybrid GPU-CPU Attention for Long Context LLM Inference":
//          dense recent window + selected entries, exact LSE fusion, MAW and
//          its beta threshold (What carries the argument); max subtraction
//          (referee minor comment on section 3.3).
//   [LFPS] "Learn from the Past: Fast Sparse Indexing for Large Language
//          Model Decoding": decay r = 0.95 of running score tables (What
//          carries the argument); block-based Quest (Extended reading notes).
#include <cfloat>
#include <cmath>

#include "sd_internal.h"

namespace sd {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// DPP lane exchange inside a 16-lane row (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within 16

// Sum over groups of L consecutive lanes (L = 8 or 16); every lane of the
// group receives the group sum.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if constexpr (L == 16) x += dpp<kRowMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Geometry of one (sequence, KV head): dense set D = [0, ns) U [wlo, N)
// ([FLX] sinks, [HGCA] recent window); head blocks [0, hb) touch the sinks,
// tail blocks [tb, n_blk) touch the window.
struct Geom {
  int N, S, n_blk, ns, wlo, hb, tb;
};
__device__ __forceinline__ Geom geom(int N, int S, int n_s, int W) {
  Geom g;
  g.N = N;
  g.S = S;
  g.n_blk = (N + S - 1) / S;
  g.ns = min(n_s, N);
  g.wlo = max(0, N - W);
  g.hb = (g.ns + S - 1) / S;
  g.tb = (W > 0 && N > 0) ? g.wlo / S : g.n_blk;
  if (g.hb >= g.tb) {  // every block touches D
    g.hb = g.n_blk;
    g.tb = g.n_blk;
  }
  return g;
}

// Block i is a candidate iff it holds a token outside D.
__device__ __forceinline__ bool is_candidate(const Geom &g, int i) {
  if (g.ns >= g.wlo) return false;
  int lo = i * g.S, hi = min(lo + g.S, g.N);
  return !(hi <= g.ns || lo >= g.wlo);
}

__device__ __forceinline__ int dense_count(const Geom &g) {
  return g.ns + (g.N - g.wlo) - max(0, g.ns - g.wlo);
}

// k = min(n_cand, ceil(ppm * N / (1e6 * S))) in 64-bit integers.
__device__ __forceinline__ int budget_blocks(int ppm, int N, int S) {
  long long den = 1000000LL * S;
  return (int)(((long long)ppm * N + den - 1) / den);
}

__device__ __forceinline__ int lower_bound(const int32_t *a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ uint32_t order_key(float u) {
  if (u == 0.0f) u = 0.0f;  // -0 and +0 are the same score
  uint32_t b = __float_as_uint(u);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// append: scatter new K/V rows into their pages ([SPIN] page substrate;
// [HGCA] append process, Figure 2).
template <int D>
__global__ __launch_bounds__(256) void k_append_kv(
    uint16_t *__restrict__ kpool, uint16_t *__restrict__ vpool,
    const int32_t *__restrict__ pt, AppendBatch b, int Hkv, int pps,
    int tok_per_wg, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new) {
  const int i = blockIdx.y;
  const int n_new = b.n_new[i];
  const int t0 = blockIdx.x * tok_per_wg;
  if (t0 >= n_new) return;
  const int seq = b.seq[i];
  const int nt = min(tok_per_wg, n_new - t0);
  constexpr int V8 = D / 8;  // uint4 per row
  const int per_tok = Hkv * V8;
  const uint4 *ks = reinterpret_cast<const uint4 *>(k_new) +
                    (size_t)(b.src_row[i] + t0) * per_tok;
  const uint4 *vs = reinterpret_cast<const uint4 *>(v_new) +
                    (size_t)(b.src_row[i] + t0) * per_tok;
  for (int idx = threadIdx.x; idx < nt * per_tok; idx += blockDim.x) {
    int t = idx / per_tok, r = idx - t * per_tok;
    int h = r / V8, c8 = r - h * V8;
    int pos = b.old_len[i] + t0 + t;
    int page = pt[(size_t)seq * pps + pos / kPage];
    size_t dst = (((size_t)page * Hkv + h) * kPage + (pos % kPage)) * V8 + c8;
    reinterpret_cast<uint4 *>(kpool)[dst] = ks[idx];
    reinterpret_cast<uint4 *>(vpool)[dst] = vs[idx];
  }
}

// append: exact per-block min/max key summaries of every touched block.
// Thread = (touched block, channel quad); tokens of the block are folded in
// logical order, starting from the stored summary if the block already held
// tokens.  Layout per (seq, head): [d/4][nbmax][4 x (min, max)] bf16.
template <int D>
__global__ __launch_bounds__(256) void k_append_summ(
    uint16_t *__restrict__ summ, const HeadInfo *__restrict__ heads,
    AppendBatch b, int Hkv, const uint16_t *__restrict__ k_new) {
  const int h = blockIdx.y, i = blockIdx.z;
  const int n_new = b.n_new[i];
  if (n_new <= 0) return;
  const HeadInfo hi = heads[h];
  const int S = hi.S;
  const int old_len = b.old_len[i], new_len = old_len + n_new;
  const int first = old_len / S, last = (new_len - 1) / S;
  const int n_touch = last - first + 1;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int C4 = D / 4;
  if (idx >= n_touch * C4) return;
  const int tb = idx / C4, c4 = idx - tb * C4;
  const int blk = first + tb;
  const int seq = b.seq[i];
  uint16_t *sp = summ + hi.summ_off + (size_t)seq * C4 * hi.nbmax * 8 +
                 ((size_t)c4 * hi.nbmax + blk) * 8;
  const int t_lo = max(blk * S, old_len), t_hi = min(blk * S + S, new_len);
  float mn[4], mx[4];
  uint16_t bmn[4], bmx[4];
  const uint16_t *src0 = k_new + ((size_t)(b.src_row[i] + t_lo - old_len) * Hkv + h) * D + 4 * c4;
  int t = t_lo;
  if (blk * S < old_len) {
    uint4 w = *reinterpret_cast<const uint4 *>(sp);
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bmn[j] = (uint16_t)(ws[j] & 0xffffu);
      bmx[j] = (uint16_t)(ws[j] >> 16);
    }
  } else {
    uint2 w = *reinterpret_cast<const uint2 *>(src0);
    uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint16_t x = (uint16_t)((ws[j >> 1] >> (16 * (j & 1))) & 0xffffu);
      bmn[j] = x;
      bmx[j] = x;
    }
    ++t;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mn[j] = __uint_as_float((uint32_t)bmn[j] << 16);
    mx[j] = __uint_as_float((uint32_t)bmx[j] << 16);
  }
  for (; t < t_hi; ++t) {
    const uint16_t *src = k_new + ((size_t)(b.src_row[i] + t - old_len) * Hkv + h) * D + 4 * c4;
    uint2 w = *reinterpret_cast<const uint2 *>(src);
    uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint16_t x = (uint16_t)((ws[j >> 1] >> (16 * (j & 1))) & 0xffffu);
      float f = __uint_as_float((uint32_t)x << 16);
      if (f < mn[j]) { mn[j] = f; bmn[j] = x; }
      if (f > mx[j]) { mx[j] = f; bmx[j] = x; }
    }
  }
  uint4 out;
  out.x = (uint32_t)bmn[0] | ((uint32_t)bmx[0] << 16);
  out.y = (uint32_t)bmn[1] | ((uint32_t)bmx[1] << 16);
  out.z = (uint32_t)bmn[2] | ((uint32_t)bmx[2] << 16);
  out.w = (uint32_t)bmn[3] | ((uint32_t)bmx[3] << 16);
  *reinterpret_cast<uint4 *>(sp) = out;
}

// ---------------------------------------------------------------------------
// select, step 1: split each query value into (min(q,0), max(q,0)) in double,
// so that max(q*m, q*M) = q- * m + q+ * M with one of the two terms zero.
__global__ __launch_bounds__(256) void k_qprep(const uint16_t *__restrict__ q,
                                               double2 *__restrict__ qpm,
                                               int n) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) {
    double x = (double)__uint_as_float((uint32_t)q[idx] << 16);
    qpm[idx] = make_double2(fmin(x, 0.0), fmax(x, 0.0));
  }
}

// select, step 2: block score ([LFPS] block-based Quest, Extended reading
// notes): U_h(i) = sum_c max(q_hc m_ic, q_hc M_ic), accumulated in double in
// channel order (the products of bf16 values are exact, so every partial sum
// equals the plain sequential double sum); group score = max over the KV
// head's query heads, rounded once to fp32 and mapped to an order-preserving
// uint32 key (0 = not a candidate).  One lane per block; the query terms are
// wave-uniform and come through the scalar cache.
template <int D, int G>
__global__ __launch_bounds__(64) void k_score(
    const uint16_t *__restrict__ summ, const float *__restrict__ maw,
    const HeadInfo *__restrict__ heads, SeqBatch b, Dims dm,
    const double2 *__restrict__ qpm, uint32_t *__restrict__ keys,
    uint8_t *__restrict__ flags) {
  const int h = blockIdx.y, i = blockIdx.z;
  const HeadInfo hi = heads[h];
  const int N = b.len[i], seq = b.seq[i];
  const Geom g = geom(N, hi.S, dm.n_sink, dm.window);
  if ((int)blockIdx.x * 64 >= g.n_blk) return;
  const int blk = blockIdx.x * 64 + threadIdx.x;
  const bool live = blk < g.n_blk;
  const int blk_c = live ? blk : g.n_blk - 1;
  constexpr int C4 = D / 4;
  const uint4 *sp = reinterpret_cast<const uint4 *>(
                        summ + hi.summ_off + (size_t)seq * C4 * hi.nbmax * 8) + blk_c;
  const double2 *qp = qpm + ((size_t)i * dm.Hq + (size_t)h * G) * D;
  double acc[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) acc[gg] = 0.0;
#pragma unroll
  for (int c4 = 0; c4 < C4; ++c4) {
    const uint4 w = sp[(size_t)c4 * hi.nbmax];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double m = (double)bf16_lo(ws[j]);
      const double M = (double)bf16_hi(ws[j]);
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const double2 qq = qp[gg * D + 4 * c4 + j];
        acc[gg] = fma(qq.x, m, acc[gg]);
        acc[gg] = fma(qq.y, M, acc[gg]);
      }
    }
  }
  double U = acc[0];
#pragma unroll
  for (int gg = 1; gg < G; ++gg) U = fmax(U, acc[gg]);
  if (!live) return;
  const size_t ko = ((size_t)seq * dm.Hkv + h) * dm.key_stride + blk;
  keys[ko] = is_candidate(g, blk) ? order_key((float)U) : 0u;
  if (dm.maw_beta > 0.0f) {
    const float mw = maw[hi.maw_off + (size_t)seq * hi.nbmax + blk];
    flags[ko] = ((double)mw * (double)dense_count(g) > (double)dm.maw_beta * (double)hi.S) ? 1 : 0;
  }
}

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_excl_scan(int v, int *sh, int *total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int x = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  int incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

// select, step 3: per (seq, KV head) top-k of the keys, ordered by
// (flag desc, score desc, index asc) ([FLX] per-head top-k; [HGCA] MAW
// threshold first).  Radix select over 8-bit digits finds the k-th key T; the
// output is compacted in ascending block order, taking keys > T and the
// lowest-index keys == T.
__global__ __launch_bounds__(256) void k_topk(const HeadInfo *__restrict__ heads,
                                              SeqBatch b, Dims dm,
                                              const uint32_t *__restrict__ keys_all,
                                              const uint8_t *__restrict__ flags_all,
                                              int32_t *__restrict__ blk_idx,
                                              int32_t *__restrict__ blk_cnt,
                                              int k_cap) {
  __shared__ int hist[256];
  __shared__ int scan_sh[256];
  __shared__ int sh_vals[4];
  const int h = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const HeadInfo hi = heads[h];
  const int N = b.len[i], seq = b.seq[i];
  const Geom g = geom(N, hi.S, dm.n_sink, dm.window);
  const int n = g.n_blk;
  const uint32_t *keys = keys_all + ((size_t)seq * dm.Hkv + h) * dm.key_stride;
  const uint8_t *flags = flags_all + ((size_t)seq * dm.Hkv + h) * dm.key_stride;
  const bool use_flag = dm.maw_beta > 0.0f;

  if (tid < 4) sh_vals[tid] = 0;
  __syncthreads();
  int lc = 0, lf = 0;
  for (int j = tid; j < n; j += 256) {
    uint32_t key = keys[j];
    if (key) {
      ++lc;
      if (use_flag && flags[j]) ++lf;
    }
  }
  lc = wave_sum_i(lc);
  lf = wave_sum_i(lf);
  if ((tid & 63) == 0) {
    atomicAdd(&sh_vals[0], lc);
    atomicAdd(&sh_vals[1], lf);
  }
  __syncthreads();
  const int C = sh_vals[0], F = sh_vals[1];
  const int kk = min(C, budget_blocks(hi.ppm, N, hi.S));
  // subset for the radix step: flagged candidates when they alone fill k,
  // otherwise the unflagged candidates (all flagged ones are taken).
  const bool take_flagged = F < kk;
  const int want_flag = take_flagged ? 0 : 1;
  int kr = take_flagged ? kk - F : kk;
  uint32_t prefix = 0, mask = 0;
  const bool radix = kr > 0;
  if (radix) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += 256) {
        uint32_t key = keys[j];
        int fl = use_flag ? flags[j] : 0;
        if (key && fl == want_flag && (key & mask) == prefix)
          atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 4l..4l+3; find digit d with
        // count(> d) < kr <= count(>= d), scanning from the top.
        int c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2],
            c3 = hist[4 * tid + 3];
        int s = c0 + c1 + c2 + c3;
        // suffix sum over lanes > tid
        int suf = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          int x = __shfl_down(suf, o, 64);
          if (tid + o < 64) suf += x;
        }
        int above = suf - s;  // digits >= 4(tid+1)
        int cs[4] = {c0, c1, c2, c3};
        int acc = above;
        for (int q = 3; q >= 0; --q) {
          if (acc < kr && acc + cs[q] >= kr) {
            sh_vals[2] = 4 * tid + q;
            sh_vals[3] = acc;
          }
          acc += cs[q];
        }
      }
      __syncthreads();
      const int digit = sh_vals[2];
      kr -= sh_vals[3];
      prefix |= (uint32_t)digit << shift;
      mask |= 0xffu << shift;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;
  // ordered compaction
  const int per = (n + 255) / 256;
  const int j0 = min(n, tid * per), j1 = min(n, j0 + per);
  int leq = 0;
  if (radix)
    for (int j = j0; j < j1; ++j) {
      uint32_t key = keys[j];
      int fl = use_flag ? flags[j] : 0;
      if (key && fl == want_flag && key == T) ++leq;
    }
  int tot;
  const int eq_base = block_excl_scan(leq, scan_sh, &tot);
  int eq_rank = eq_base;
  int lsel = 0;
  for (int j = j0; j < j1; ++j) {
    uint32_t key = keys[j];
    if (!key) continue;
    int fl = use_flag ? flags[j] : 0;
    bool s = false;
    if (take_flagged && fl) s = true;
    else if (radix && fl == want_flag) {
      if (key > T) s = true;
      else if (key == T) { s = eq_rank < kr; ++eq_rank; }
    }
    lsel += s;
  }
  int out = block_excl_scan(lsel, scan_sh, &tot);
  // second pass writes (recomputing the same decisions)
  eq_rank = eq_base;
  int32_t *dst = blk_idx + ((size_t)i * dm.Hkv + h) * k_cap;
  for (int j = j0; j < j1; ++j) {
    uint32_t key = keys[j];
    if (!key) continue;
    int fl = use_flag ? flags[j] : 0;
    bool s = false;
    if (take_flagged && fl) s = true;
    else if (radix && fl == want_flag) {
      if (key > T) s = true;
      else if (key == T) { s = eq_rank < kr; ++eq_rank; }
    }
    if (s && out < k_cap) dst[out++] = j;
  }
  if (tid == 0) blk_cnt[(size_t)i * dm.Hkv + h] = kk;
}

// ---------------------------------------------------------------------------
// attend: split-K softmax attention of the G query heads of one KV head over
// one chunk of its attended blocks (dense sinks + window + selected blocks,
// each token once; [HGCA] What carries the argument).  Writes the chunk's
// normalised O and lse per head, and the log of each block's softmax mass
// (for the MAW update).  Lanes of a 16 (d=128) or 8 (d=64) lane group share
// one K/V row, 16 bytes each.
template <int D, int G>
__global__ __launch_bounds__(256) void k_attend(
    LayerDev L, const HeadInfo *__restrict__ heads, SeqBatch b, Dims dm,
    Scratch sc, const uint16_t *__restrict__ q,
    const int32_t *__restrict__ blk_idx, const int32_t *__restrict__ blk_cnt,
    int k_cap, float *__restrict__ o_part, float *__restrict__ lse_part,
    int p_cap) {
  constexpr int LPR = D / 8;           // lanes per row
  constexpr int RPW = 64 / LPR;        // rows per wave per step
  constexpr int RPS = 4 * RPW;         // rows per workgroup step
  constexpr int GP = G <= 4 ? 4 : 8;   // padded head count in LDS
  constexpr int MAXCB = kChunkTokens / kPage;
  __shared__ float p_sh[kChunkTokens][GP];
  __shared__ float red_sh[4][G][D];
  __shared__ float stat_sh[2][4][G];
  __shared__ float bsum_sh[MAXCB][G];
  __shared__ int blk_sh[MAXCB];
  __shared__ unsigned long long mask_sh[MAXCB];
  __shared__ int geo_sh[2];

  const int chunk = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const HeadInfo hi = heads[h];
  const int N = b.len[i], seq = b.seq[i], S = hi.S, CB = hi.chunk_blocks;
  const Geom g = geom(N, S, dm.n_sink, dm.window);
  const int32_t *sel = blk_idx + ((size_t)i * dm.Hkv + h) * k_cap;
  const int qh0 = h * G;

  if (tid == 0) {
    int k = min(max(blk_cnt[(size_t)i * dm.Hkv + h], 0), k_cap);
    int a = lower_bound(sel, k, g.hb), bb = lower_bound(sel, k, g.tb);
    if (bb < a) bb = a;
    // |U|, clamped to the scratch capacity (only reachable with inputs that
    // violate the documented k_cap contract)
    geo_sh[0] = min(g.hb + (bb - a) + (g.n_blk - g.tb), dm.u_cap);
    geo_sh[1] = a;
  }
  __syncthreads();
  const int nU = geo_sh[0], a_sel = geo_sh[1];
  const int c0 = chunk * CB;
  const size_t ohead = ((size_t)i * dm.Hq + qh0) * p_cap + chunk;
  if (c0 >= nU) {  // empty slot: lse = -inf, O = 0
    for (int x = tid; x < G * D; x += 256)
      o_part[(ohead + (size_t)(x / D) * p_cap) * D + (x % D)] = 0.0f;
    if (tid < G) lse_part[ohead + (size_t)tid * p_cap] = -INFINITY;
    return;
  }
  const int nb = min(CB, nU - c0);
  const int mid = nU - g.hb - (g.n_blk - g.tb);  // selected blocks in [hb, tb)
  if (tid < nb) {
    const int j = c0 + tid;
    int blk;
    bool selected;
    if (j < g.hb) {
      blk = j;
    } else if (j < g.hb + mid) {
      blk = sel[a_sel + j - g.hb];
    } else {
      blk = g.tb + (j - g.hb - mid);
    }
    if (j >= g.hb && j < g.hb + mid) {
      selected = true;
    } else {
      int k = min(max(blk_cnt[(size_t)i * dm.Hkv + h], 0), k_cap);
      int p = lower_bound(sel, k, blk);
      selected = p < k && sel[p] == blk;
    }
    unsigned long long m = 0ull;
    if (blk >= 0 && blk < g.n_blk) {
      const int lo = blk * S, cnt = min(S, N - lo);
      for (int r = 0; r < cnt; ++r) {
        const int t = lo + r;
        if (selected || t < g.ns || t >= g.wlo) m |= 1ull << r;
      }
    } else {
      blk = 0;
    }
    blk_sh[tid] = blk;
    mask_sh[tid] = m;
  }
  __syncthreads();

  // query of this lane's channels (fixed for the whole kernel)
  const int lg = lane / LPR, cl = lane % LPR;
  float qv[G][8];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const uint4 w = *reinterpret_cast<const uint4 *>(
        q + ((size_t)i * dm.Hq + qh0 + gg) * D + 8 * cl);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[gg][2 * e] = bf16_lo(ws[e]) * dm.scale_log2;
      qv[gg][2 * e + 1] = bf16_hi(ws[e]) * dm.scale_log2;
    }
  }

  const int n_slots = nb * S;
  const int32_t *pt = L.pt + (size_t)seq * dm.pages_per_seq;
  // pass 1: scaled logits (log2 units) into p_sh; masked slots get -inf
  for (int base = 0; base < n_slots; base += RPS) {
    const int t = base + wv * RPW + lg;
    float acc[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) acc[gg] = 0.0f;
    bool on = false;
    if (t < n_slots) {
      const int jj = t / S, r = t - jj * S;
      on = (mask_sh[jj] >> r) & 1ull;
      if (on) {
        const int pos = blk_sh[jj] * S + r;
        const int page = pt[pos / kPage];
        const uint4 w = *reinterpret_cast<const uint4 *>(
            L.k + (((size_t)page * dm.Hkv + h) * kPage + (pos % kPage)) * D + 8 * cl);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = bf16_lo(ws[e]), k1 = bf16_hi(ws[e]);
#pragma unroll
          for (int gg = 0; gg < G; ++gg) {
            acc[gg] = fmaf(qv[gg][2 * e], k0, acc[gg]);
            acc[gg] = fmaf(qv[gg][2 * e + 1], k1, acc[gg]);
          }
        }
      }
    }
#pragma unroll
    for (int gg = 0; gg < G; ++gg) acc[gg] = group_sum<LPR>(acc[gg]);
    if (t < n_slots && cl == 0) {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) p_sh[t][gg] = on ? acc[gg] : -INFINITY;
    }
  }
  __syncthreads();

  // softmax statistics per head over the chunk
  float mloc[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float x = -INFINITY;
    for (int t = tid; t < n_slots; t += 256) x = fmaxf(x, p_sh[t][gg]);
    x = wave_max(x);
    if (lane == 0) stat_sh[0][wv][gg] = x;
  }
  __syncthreads();
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
    mloc[gg] = fmaxf(fmaxf(stat_sh[0][0][gg], stat_sh[0][1][gg]),
                     fmaxf(stat_sh[0][2][gg], stat_sh[0][3][gg]));
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float x = 0.0f;
    for (int t = tid; t < n_slots; t += 256) {
      const float s = p_sh[t][gg];
      const float p = s == -INFINITY ? 0.0f : exp2f(s - mloc[gg]);
      p_sh[t][gg] = p;
      x += p;
    }
    x = wave_sum(x);
    if (lane == 0) stat_sh[1][wv][gg] = x;
  }
  __syncthreads();
  float zsum[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
    zsum[gg] = (stat_sh[1][0][gg] + stat_sh[1][1][gg]) +
               (stat_sh[1][2][gg] + stat_sh[1][3][gg]);
  // per-block mass sums (MAW)
  if (tid < nb * G) {
    const int jj = tid / G, gg = tid % G;
    float x = 0.0f;
    for (int r = 0; r < S; ++r) x += p_sh[jj * S + r][gg];
    bsum_sh[jj][gg] = x;
  }

  // pass 2: O = sum_t p_t v_t
  float o[G][8];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gg][e] = 0.0f;
  for (int base = 0; base < n_slots; base += RPS) {
    const int t = base + wv * RPW + lg;
    if (t < n_slots) {
      const int jj = t / S, r = t - jj * S;
      if ((mask_sh[jj] >> r) & 1ull) {
        const int pos = blk_sh[jj] * S + r;
        const int page = pt[pos / kPage];
        const uint4 w = *reinterpret_cast<const uint4 *>(
            L.v + (((size_t)page * dm.Hkv + h) * kPage + (pos % kPage)) * D + 8 * cl);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        float pw[G];
#pragma unroll
        for (int gg = 0; gg < G; ++gg) pw[gg] = p_sh[t][gg];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = bf16_lo(ws[e]), v1 = bf16_hi(ws[e]);
#pragma unroll
          for (int gg = 0; gg < G; ++gg) {
            o[gg][2 * e] = fmaf(pw[gg], v0, o[gg][2 * e]);
            o[gg][2 * e + 1] = fmaf(pw[gg], v1, o[gg][2 * e + 1]);
          }
        }
      }
    }
  }
  // reduce over the row groups of the wave (lanes with equal cl)
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[gg][e];
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      o[gg][e] = x;
    }
  if (lg == 0) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_sh[wv][gg][8 * cl + e] = o[gg][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int gg = x / D, c = x - gg * D;
    const float v = (red_sh[0][gg][c] + red_sh[1][gg][c]) +
                    (red_sh[2][gg][c] + red_sh[3][gg][c]);
    const float z = zsum[gg];
    o_part[(ohead + (size_t)gg * p_cap) * D + c] = z > 0.0f ? v / z : 0.0f;
  }
  constexpr float kLn2 = 0.69314718055994530942f;
  if (tid < G) {
    const float z = zsum[tid];
    lse_part[ohead + (size_t)tid * p_cap] =
        z > 0.0f ? (mloc[tid] + log2f(z)) * kLn2 : -INFINITY;
  }
  if (tid < nb * G) {
    const int jj = tid / G, gg = tid % G;
    const float z = bsum_sh[jj][gg];
    sc.lmass[((size_t)seq * dm.Hq + qh0 + gg) * dm.u_cap + c0 + jj] =
        z > 0.0f ? (mloc[gg] + log2f(z)) * kLn2 : -INFINITY;
    if (gg == 0) sc.ublk[((size_t)seq * dm.Hkv + h) * dm.u_cap + c0 + jj] = blk_sh[jj];
  }
  if (chunk == 0 && tid == 0) sc.ucnt[(size_t)seq * dm.Hkv + h] = nU;
}

// ---------------------------------------------------------------------------
// fuse: exact LSE fusion of the split-K partials of each query head ([HGCA]
// What carries the argument, max-subtracted form), then the MAW update of
// every block of the (seq, KV head): MAW <- r MAW + (1-r) a, with a the
// group-mean softmax mass of the block ([LFPS] decay r; [HGCA] MAW).
template <int D, int G>
__global__ __launch_bounds__(256) void k_fuse(
    float *__restrict__ maw_all, const HeadInfo *__restrict__ heads,
    SeqBatch b, Dims dm, Scratch sc, int with_maw,
    const float *__restrict__ o_part, const float *__restrict__ lse_part,
    int p_cap, float *__restrict__ o, float *__restrict__ lse) {
  __shared__ float lse_sh[G];
  __shared__ float m_sh[G];
  const int h = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int qh0 = h * G;
  // per-head max and lse: wave gg handles head gg (and gg+4, ...)
  for (int gg = wv; gg < G; gg += 4) {
    const float *lp = lse_part + ((size_t)i * dm.Hq + qh0 + gg) * p_cap;
    float m = -INFINITY;
    for (int p = lane; p < p_cap; p += 64) m = fmaxf(m, lp[p]);
    m = wave_max(m);
    float z = 0.0f;
    if (m != -INFINITY)
      for (int p = lane; p < p_cap; p += 64) {
        const float l = lp[p];
        if (l != -INFINITY) z += expf(l - m);
      }
    z = wave_sum(z);
    if (lane == 0) {
      m_sh[gg] = m;
      lse_sh[gg] = m == -INFINITY ? -INFINITY : m + logf(z);
    }
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int gg = x / D, c = x - gg * D;
    const float L = lse_sh[gg];
    const size_t hb = ((size_t)i * dm.Hq + qh0 + gg) * p_cap;
    float acc = 0.0f;
    if (L != -INFINITY)
      for (int p = 0; p < p_cap; ++p) {
        const float l = lse_part[hb + p];
        if (l != -INFINITY) acc = fmaf(expf(l - L), o_part[(hb + p) * D + c], acc);
      }
    o[((size_t)i * dm.Hq + qh0 + gg) * D + c] = acc;
  }
  if (tid < G) lse[(size_t)i * dm.Hq + qh0 + tid] = lse_sh[tid];
  if (!with_maw) return;

  const HeadInfo hi = heads[h];
  const int N = b.len[i], seq = b.seq[i];
  const int n_blk = (N + hi.S - 1) / hi.S;
  const int nU = min(sc.ucnt[(size_t)seq * dm.Hkv + h], dm.u_cap);
  const int32_t *ub = sc.ublk + ((size_t)seq * dm.Hkv + h) * dm.u_cap;
  float *mw = maw_all + hi.maw_off + (size_t)seq * hi.nbmax;
  const float r = dm.maw_decay;
  for (int blk = tid; blk < n_blk; blk += 256) {
    const int u = lower_bound(ub, nU, blk);
    float a = 0.0f;
    if (u < nU && ub[u] == blk) {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float L = lse_sh[gg];
        const float lm = sc.lmass[((size_t)seq * dm.Hq + qh0 + gg) * dm.u_cap + u];
        if (L != -INFINITY && lm != -INFINITY) a += expf(lm - L);
      }
      a *= 1.0f / (float)G;
    }
    mw[blk] = fmaf(r, mw[blk], (1.0f - r) * a);
  }
}

__global__ void k_fill_f32(float *p, size_t n, float v) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; idx < n; idx += (size_t)gridDim.x * blockDim.x) p[idx] = v;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_append(const LayerDev &L, const HeadInfo *d_heads,
                         const Dims &dm, const AppendBatch &b, int max_new,
                         int max_touch_blocks, const uint16_t *k_new,
                         const uint16_t *v_new, hipStream_t st) {
  if (b.n <= 0 || max_new <= 0) return hipSuccess;
  const int tpw = 16;
  dim3 g1((max_new + tpw - 1) / tpw, b.n);
  dim3 g2((max_touch_blocks * (dm.d / 4) + 255) / 256, dm.Hkv, b.n);
  if (dm.d == 128) {
    hipLaunchKernelGGL(k_append_kv<128>, g1, dim3(256), 0, st, L.k, L.v, L.pt, b,
                       dm.Hkv, dm.pages_per_seq, tpw, k_new, v_new);
    hipLaunchKernelGGL(k_append_summ<128>, g2, dim3(256), 0, st, L.summ, d_heads,
                       b, dm.Hkv, k_new);
  } else {
    hipLaunchKernelGGL(k_append_kv<64>, g1, dim3(256), 0, st, L.k, L.v, L.pt, b,
                       dm.Hkv, dm.pages_per_seq, tpw, k_new, v_new);
    hipLaunchKernelGGL(k_append_summ<64>, g2, dim3(256), 0, st, L.summ, d_heads,
                       b, dm.Hkv, k_new);
  }
  return hipGetLastError();
}

template <int D, int G>
static void launch_score_t(dim3 grid, const LayerDev &L, const HeadInfo *d_heads,
                           const SeqBatch &b, const Dims &dm, const Scratch &sc,
                           hipStream_t st) {
  hipLaunchKernelGGL((k_score<D, G>), grid, dim3(64), 0, st, L.summ, L.maw,
                     d_heads, b, dm, sc.qpm, sc.keys, sc.flags);
}

template <int D>
static hipError_t launch_score_d(dim3 grid, const LayerDev &L,
                                 const HeadInfo *d_heads, const SeqBatch &b,
                                 const Dims &dm, const Scratch &sc,
                                 hipStream_t st) {
  switch (dm.G) {
    case 1: launch_score_t<D, 1>(grid, L, d_heads, b, dm, sc, st); break;
    case 2: launch_score_t<D, 2>(grid, L, d_heads, b, dm, sc, st); break;
    case 3: launch_score_t<D, 3>(grid, L, d_heads, b, dm, sc, st); break;
    case 4: launch_score_t<D, 4>(grid, L, d_heads, b, dm, sc, st); break;
    case 5: launch_score_t<D, 5>(grid, L, d_heads, b, dm, sc, st); break;
    case 6: launch_score_t<D, 6>(grid, L, d_heads, b, dm, sc, st); break;
    case 7: launch_score_t<D, 7>(grid, L, d_heads, b, dm, sc, st); break;
    case 8: launch_score_t<D, 8>(grid, L, d_heads, b, dm, sc, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_select(const LayerDev &L, const HeadInfo *d_heads,
                         const Dims &dm, const Scratch &sc, const SeqBatch &b,
                         int max_blocks, const uint16_t *q, int32_t *blk_idx,
                         int32_t *blk_cnt, int32_t k_cap, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  const int nq = b.n * dm.Hq * dm.d;
  hipLaunchKernelGGL(k_qprep, dim3((nq + 255) / 256), dim3(256), 0, st, q,
                     sc.qpm, nq);
  dim3 grid((max(max_blocks, 1) + 63) / 64, dm.Hkv, b.n);
  hipError_t e = dm.d == 128 ? launch_score_d<128>(grid, L, d_heads, b, dm, sc, st)
                             : launch_score_d<64>(grid, L, d_heads, b, dm, sc, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk, dim3(dm.Hkv, b.n), dim3(256), 0, st, d_heads, b, dm,
                     sc.keys, sc.flags, blk_idx, blk_cnt, k_cap);
  return hipGetLastError();
}

template <int D, int G>
static void launch_attend_t(const LayerDev &L, const HeadInfo *d_heads,
                            const Dims &dm, const Scratch &sc,
                            const SeqBatch &b, const uint16_t *q,
                            const int32_t *blk_idx, const int32_t *blk_cnt,
                            int32_t k_cap, float *o_part, float *lse_part,
                            int32_t p_cap, hipStream_t st) {
  hipLaunchKernelGGL((k_attend<D, G>), dim3(p_cap, dm.Hkv, b.n), dim3(256), 0, st,
                     L, d_heads, b, dm, sc, q, blk_idx, blk_cnt, k_cap, o_part,
                     lse_part, p_cap);
}

template <int D>
static hipError_t launch_attend_d(const LayerDev &L, const HeadInfo *d_heads,
                                  const Dims &dm, const Scratch &sc,
                                  const SeqBatch &b, const uint16_t *q,
                                  const int32_t *blk_idx, const int32_t *blk_cnt,
                                  int32_t k_cap, float *o_part, float *lse_part,
                                  int32_t p_cap, hipStream_t st) {
#define SD_ATT(GG)                                                            \
  case GG:                                                                    \
    launch_attend_t<D, GG>(L, d_heads, dm, sc, b, q, blk_idx, blk_cnt, k_cap, \
                           o_part, lse_part, p_cap, st);                      \
    break;
  switch (dm.G) {
    SD_ATT(1) SD_ATT(2) SD_ATT(3) SD_ATT(4) SD_ATT(5) SD_ATT(6) SD_ATT(7) SD_ATT(8)
    default: return hipErrorInvalidValue;
  }
#undef SD_ATT
  return hipSuccess;
}

hipError_t launch_attend(const LayerDev &L, const HeadInfo *d_heads,
                         const Dims &dm, const Scratch &sc, const SeqBatch &b,
                         const uint16_t *q, const int32_t *blk_idx,
                         const int32_t *blk_cnt, int32_t k_cap, float *o_part,
                         float *lse_part, int32_t p_cap, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  hipError_t e = dm.d == 128
                     ? launch_attend_d<128>(L, d_heads, dm, sc, b, q, blk_idx, blk_cnt,
                                            k_cap, o_part, lse_part, p_cap, st)
                     : launch_attend_d<64>(L, d_heads, dm, sc, b, q, blk_idx, blk_cnt,
                                           k_cap, o_part, lse_part, p_cap, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fuse_d(const LayerDev *L, const HeadInfo *d_heads,
                                const Dims &dm, const Scratch &sc,
                                const SeqBatch &b, bool with_maw,
                                const float *o_part, const float *lse_part,
                                int32_t p_cap, float *o, float *lse,
                                hipStream_t st) {
  float *maw = L ? L->maw : nullptr;
  dim3 grid(dm.Hkv, b.n);
#define SD_FUSE(GG)                                                                 \
  case GG:                                                                          \
    hipLaunchKernelGGL((k_fuse<D, GG>), grid, dim3(256), 0, st, maw, d_heads, b, dm, \
                       sc, with_maw ? 1 : 0, o_part, lse_part, p_cap, o, lse);      \
    break;
  switch (dm.G) {
    SD_FUSE(1) SD_FUSE(2) SD_FUSE(3) SD_FUSE(4) SD_FUSE(5) SD_FUSE(6) SD_FUSE(7) SD_FUSE(8)
    default: return hipErrorInvalidValue;
  }
#undef SD_FUSE
  return hipSuccess;
}

hipError_t launch_fuse(const LayerDev *L, const HeadInfo *d_heads,
                       const Dims &dm, const Scratch &sc, const SeqBatch &b,
                       bool with_maw, const float *o_part,
                       const float *lse_part, int32_t p_cap, float *o,
                       float *lse, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  hipError_t e = dm.d == 128
                     ? launch_fuse_d<128>(L, d_heads, dm, sc, b, with_maw, o_part,
                                          lse_part, p_cap, o, lse, st)
                     : launch_fuse_d<64>(L, d_heads, dm, sc, b, with_maw, o_part,
                                         lse_part, p_cap, o, lse, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, size_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace sd
