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
//
// Work decomposition of one (sequence, KV head) "unit":
//   * score tiles: 256 blocks per workgroup; the last tile to finish (atomic
//     arrival counter) runs the unit's top-k;
//   * attention parts: P workgroups per unit share the unit's attended pages
//     (the dense pages, then the pages of the selected blocks without their
//     dense tokens, so every token of T = D U selected counts once); each
//     streams its pages and writes one partial (O, lse);
//   * fusion: the P partials merged with the LSE identity, then the MAW
//     update of every block.
// The fused step and the separate ABI calls run these same device functions
// with the same P, so their results are bitwise identical.
#include <algorithm>
#include <cfloat>
#include <cmath>

#include "sd_internal.h"

namespace sd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }
// x / m for x >= 0 and m in {1, 2, 3, 4} (pages per block): a shift, or a
// multiply-high by ceil(2^33 / 3) for m = 3 (exact for every 32-bit x).
__device__ __forceinline__ int div_m(int x, int m) {
  return m == 3 ? (int)(__umulhi((uint32_t)x, 0xAAAAAAABu) >> 1) : (int)((uint32_t)x >> (m >> 1));
}
// x / S for x >= 0 and a block size S = 16 m.
__device__ __forceinline__ int div_S(int x, int S) { return div_m((int)((uint32_t)x >> 4), S >> 4); }

// Data that one workgroup publishes to the last-arriving workgroup of the same
// unit inside one launch is written and read with relaxed device-scope atomic
// accesses, which the gfx950 memory model keeps coherent across the XCDs
// without L2 write-back or invalidation; a wait for the workgroup's memory
// operations (vmcnt 0) orders them before its arrival increment.
template <class T>
__device__ __forceinline__ void st_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads and stores are done
}
// Arrival of one workgroup of a unit; true in the last one to arrive.  Every
// thread of the workgroup must call it.
__device__ __forceinline__ bool arrive_last(uint32_t *counter, unsigned expected, int *flag) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *flag = prev == expected - 1;
  }
  __syncthreads();
  return *flag != 0;
}

// Arrival of one workgroup that needs no answer: its memory operations are
// done before the increment.  Every thread of the workgroup must call it.
__device__ __forceinline__ void arrive(uint32_t *counter) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bound of every wait inside a launch.
constexpr unsigned long long kWaitTicks = 20000000ull;  // 0.2 s of the 100 MHz clock

}  // namespace

// Per-phase timestamps of the one-launch step, built only with SD_TIMELINE
// (a measurement build; the product library has none of this): thread 0 of
// each workgroup stores wall_clock64(), a 100 MHz counter common to the whole
// device, at the phase boundaries of its role, indexed by its flat workgroup
// number.  sd_timeline_read copies them out.
#ifdef SD_TIMELINE
constexpr int kTlSlots = 8;
constexpr int kTlMaxWG = 16384;
__device__ unsigned long long sd_tl_buf[kTlMaxWG * kTlSlots];
#define SD_TL(slot)                                                                  \
  do {                                                                               \
    if (threadIdx.x == 0) {                                                          \
      const unsigned wg_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z); \
      if (wg_ < (unsigned)kTlMaxWG) sd_tl_buf[wg_ * kTlSlots + (slot)] = wall_clock64(); \
    }                                                                                \
  } while (0)
#else
#define SD_TL(slot) \
  do {              \
  } while (0)
#endif

namespace {

__device__ __forceinline__ int lower_bound(const int32_t *a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// k = ceil(ppm * N / (1e6 * S)) in 64-bit integers (budget as a token
// fraction of N, whole blocks; [FLX] Figure 2 and Figure 8).
__device__ __forceinline__ int budget_blocks(int ppm, int N, int S) {
  long long den = 1000000LL * S;
  return (int)(((long long)ppm * N + den - 1) / den);
}

// Geometry of one unit.  D = [0, ns) U [wlo, N) ([FLX] sinks, [HGCA] recent
// window); blocks [0, hb) touch the sinks, blocks [tb, n_blk) the window.
// Candidates lie in [0, n_sc): a block from n_sc on lies wholly in the
// window; only [0, n_sc) is scored and ranked.
struct UG {
  int N, S, n_blk, ns, wlo, hb, tb, n_dt, kk, n_sc;
};
// Blocks that can hold a candidate: [0, ceil(wlo / S)) with a window, else
// all of them.
__device__ __forceinline__ int scored_blocks(int N, int S, const Dims &dm) {
  const int n_blk = div_S(N + S - 1, S);
  return (dm.window > 0 && N > 0) ? min(n_blk, div_S(max(0, N - dm.window) + S - 1, S)) : n_blk;
}
__device__ __forceinline__ UG unit_geom(int N, const HeadInfo &hi, const Dims &dm) {
  UG g;
  const int S = hi.S;
  g.N = N;
  g.S = S;
  g.n_blk = div_S(N + S - 1, S);
  g.ns = min(dm.n_sink, N);
  g.wlo = max(0, N - dm.window);
  g.hb = div_S(g.ns + S - 1, S);
  g.tb = (dm.window > 0 && N > 0) ? div_S(g.wlo, S) : g.n_blk;
  if (g.hb >= g.tb) {  // every block touches D
    g.hb = g.n_blk;
    g.tb = g.n_blk;
  }
  g.n_dt = g.hb + (g.n_blk - g.tb);
  g.n_sc = scored_blocks(N, S, dm);
  const int n_cand = g.ns < g.wlo ? div_S(g.wlo + S - 1, S) - div_S(g.ns, S) : 0;
  g.kk = min(n_cand, budget_blocks(hi.ppm, N, S));
  return g;
}

// A unit selects nothing (k = 0) when its head's budget is 0 (a streaming
// head, which attends to its sinks and recent window only; [FLX] streaming
// heads) or when no block has a token outside the dense set.  Cheap: no
// division, so the score tiles can decide before any work.
__device__ __forceinline__ bool selects_nothing(const HeadInfo &hi, int N, const Dims &dm) {
  return hi.ppm == 0 || min(dm.n_sink, N) >= max(0, N - dm.window);
}

__device__ __forceinline__ bool is_candidate(const UG &g, int i) {
  if (g.ns >= g.wlo) return false;
  const int lo = i * g.S, hi = min(lo + g.S, g.N);
  return !(hi <= g.ns || lo >= g.wlo);
}
__device__ __forceinline__ int dense_count(const UG &g) {
  return g.ns + (g.N - g.wlo) - max(0, g.ns - g.wlo);
}
// Dense-touching block of dense slot j.
__device__ __forceinline__ int dense_block(const UG &g, int j) {
  return j < g.hb ? j : g.tb + (j - g.hb);
}
__device__ __forceinline__ uint32_t order_key(float u) {
  if (u == 0.0f) u = 0.0f;  // -0 and +0 are the same score
  const uint32_t b = __float_as_uint(u);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Shared memory of the roles (one launch may host several roles).
constexpr int kTileList = 64;  // keys a score tile lists per lane register for the fast top-k
constexpr int kFastK = 2 * kTileList;  // the fast top-k's largest k (lists of two registers)
// The four-wave top-k ranks units of (kTopkRegRows * 64, 256 * kWideM]
// blocks; its thread t holds blocks [t m, t m + m), m = ceil(n / 256).
static_assert(kWideM <= 64, "a thread's blocks span at most two mask words");
struct TopkSmem {
  int32_t ulist[kTopkUnc];  // uncertain blocks of the top-k, in index order
  uint32_t ukey[kTopkUnc];  // their exact keys
  uint32_t tk[kScoreTile];  // keys of a score tile (fast top-k)
  double ue[kFastK * SD_MAX_GROUP];  // exact scores of the fast top-k's band, per head
  unsigned long long bm[kFastTiles * kScoreTile / 64];  // chosen blocks (fast top-k)
  unsigned long long srt[4][kTileList];  // the waves' sorted keys (tile list)
  float qs[SD_MAX_GROUP * 128];
  double ud[16];
  uint32_t red[16];
  int nlist, nin, kr2, ok;
  int last;
};

template <int G>
struct FuseSmem {
  float w[G][kFuseSlots];   // per-slot LSE weights
  float lse[G];
  float dm[4 * G], dz[4 * G];  // MAW: per wave, running max and sum of the dense log-masses
  float pm[kFuseDenseLds];     // MAW: mass of each dense page under the dense partial
};

// ---------------------------------------------------------------------------
// append: scatter new K/V rows into their pages ([SPIN] page substrate;
// [HGCA] append process, Figure 2).
template <int D>
__device__ void append_scatter(const Ctx &c, const AppendBatch &b, int i,
                               int wg_x, int tok_per_wg,
                               const uint16_t *__restrict__ k_new,
                               const uint16_t *__restrict__ v_new) {
  const int n_new = b.n_new[i];
  const int t0 = wg_x * tok_per_wg;
  if (t0 >= n_new) return;
  const int seq = b.seq[i];
  const int nt = min(tok_per_wg, n_new - t0);
  constexpr int V8 = D / 8;
  const int Hkv = c.dm.Hkv;
  const int per_tok = Hkv * V8;
  const uint4 *ks = reinterpret_cast<const uint4 *>(k_new) + (size_t)(b.src_row[i] + t0) * per_tok;
  const uint4 *vs = reinterpret_cast<const uint4 *>(v_new) + (size_t)(b.src_row[i] + t0) * per_tok;
  for (int idx = threadIdx.x; idx < nt * per_tok; idx += blockDim.x) {
    const int t = idx / per_tok, r = idx - t * per_tok;
    const int h = r / V8, c8 = r - h * V8;
    const int pos = b.old_len[i] + t0 + t;
    const int page = c.L.pt[(size_t)seq * c.dm.pages_per_seq + pos / kPage];
    // K page: channel group c8 of the 16 tokens is 256 contiguous bytes
    const size_t dst = (((size_t)page * Hkv + h) * V8 + c8) * kPage + (pos % kPage);
    reinterpret_cast<uint4 *>(c.L.k)[dst] = ks[idx];
    // V page transposed: element (channel ch, token t) at ch * 16 + t
    const uint4 vv = vs[idx];
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
    uint16_t *vt = c.L.v + ((size_t)page * Hkv + h) * D * kPage + (size_t)(8 * c8) * kPage +
                   (pos % kPage);
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(size_t)e * kPage] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

// append: exact per-block min/max key summaries of every touched block.
// Thread = (touched block, channel quad); tokens are folded in logical order,
// starting from the stored summary if the block already held tokens.  Layout
// per (seq, head): [d/4][nbmax][4 x (min, max)] bf16, so that scoring reads
// 16 contiguous bytes per lane with consecutive lanes on consecutive blocks.
template <int D>
__device__ void append_summ(const Ctx &c, const AppendBatch &b, int i, int h,
                            int idx, const uint16_t *__restrict__ k_new) {
  const int n_new = b.n_new[i];
  if (n_new <= 0) return;
  const HeadInfo hi = c.heads[h];
  const int S = hi.S, Hkv = c.dm.Hkv;
  const int old_len = b.old_len[i], new_len = old_len + n_new;
  const int first = old_len / S, last = (new_len - 1) / S;
  const int n_touch = last - first + 1;
  constexpr int C4 = D / 4;
  if (idx >= n_touch * C4) return;
  const int tb = idx / C4, c4 = idx - tb * C4;
  const int blk = first + tb;
  const int seq = b.seq[i];
  uint16_t *sp = c.L.summ + hi.summ_off + (size_t)seq * C4 * hi.nbmax * 8 +
                 ((size_t)c4 * hi.nbmax + blk) * 8;
  const int t_lo = max(blk * S, old_len), t_hi = min(blk * S + S, new_len);
  float mn[4], mx[4];
  uint16_t bmn[4], bmx[4];
  int t = t_lo;
  if (blk * S < old_len) {
    const uint4 w = *reinterpret_cast<const uint4 *>(sp);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bmn[j] = (uint16_t)(ws[j] & 0xffffu);
      bmx[j] = (uint16_t)(ws[j] >> 16);
    }
  } else {
    const uint16_t *src0 = k_new + ((size_t)(b.src_row[i] + t_lo - old_len) * Hkv + h) * D + 4 * c4;
    const uint2 w = *reinterpret_cast<const uint2 *>(src0);
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t x = (uint16_t)((ws[j >> 1] >> (16 * (j & 1))) & 0xffffu);
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
    const uint2 w = *reinterpret_cast<const uint2 *>(src);
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t x = (uint16_t)((ws[j >> 1] >> (16 * (j & 1))) & 0xffffu);
      const float f = __uint_as_float((uint32_t)x << 16);
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
// Wave-level helpers of the scoring and the top-k.
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ __forceinline__ int count_lanes(bool p) { return __popcll(__ballot(p)); }
// Wave min / max of an unsigned value (uniform result): DPP inside rows of
// 16 lanes, then the four row results.
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  v = min(v, dppu<0xB1>(v));   // quad_perm [1,0,3,2]
  v = min(v, dppu<0x4E>(v));   // quad_perm [2,3,0,1]
  v = min(v, dppu<0x141>(v));  // row_half_mirror
  v = min(v, dppu<0x140>(v));  // row_mirror
  const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, dppu<0xB1>(v));
  v = max(v, dppu<0x4E>(v));
  v = max(v, dppu<0x141>(v));
  v = max(v, dppu<0x140>(v));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}
// Largest t in [lo, hi] with count_ge(t) >= k, given count_ge(lo) >= k: the
// k-th largest of the counted values.
template <class CountF>
__device__ __forceinline__ uint32_t bisect_kth(uint32_t lo, uint32_t hi, int k, CountF count_ge) {
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1) + 1u;  // lo < mid <= hi
    if (count_ge(mid) >= k) lo = mid; else hi = mid - 1u;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// score, approximate pass ([LFPS] block-based Quest bound, R2):
//   U_h(i) = sum_c max(q_hc m_ic, q_hc M_ic) = sum_c q-_hc m_ic + q+_hc M_ic
// with q- = min(q,0), q+ = max(q,0) (exact in bf16), so the bound of 16
// blocks x 16 (padded) heads is a bf16 MFMA product: A = [q-, q+] per
// channel, B = the (min, max) summaries exactly as stored (one 16-byte
// summary chunk of 4 channels is one lane's 8 k-values).  The fp32 result A_i
// (group max over the KV head's query heads, R1) carries an error bound
// eps_i from a second MFMA over absolute values; the top-k then re-scores
// exactly, in double and in channel order, every block whose approximate
// score lies within the band of the k-th.
__device__ __forceinline__ uint32_t key_to_bits(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float(key_to_bits(k));
}

// fp32 error bound of the approximate score: partial sums of 64 products of
// bf16 values (one chain of two MFMAs each, error <= gamma_64 times their
// magnitude) added in fp32 (at most 4 partials: gamma_4), with total
// magnitude E: 2 * (gamma_64 + gamma_4) * E (gamma_n = n u / (1 - n u),
// u = 2^-24, and a factor 2 of margin), plus one float rounding of the exact
// score.
__device__ __forceinline__ float score_eps(float E, float A) {
  return 8.2e-6f * E + 1.2e-7f * fabsf(A) + 1e-30f;
}

// Exact score of one block for one query head: sum_c max(q_c m_c, q_c M_c)
// in double in channel order, the plain sequential double sum.  The larger
// product is q_c M_c for q_c >= 0 and q_c m_c otherwise (m_c <= M_c; with
// q_c = 0 both are zeros, which leave the sum unchanged), and a product of
// two bf16 values is exact in double, so one fma per channel rounds as the
// product-then-add of the definition.
__device__ __forceinline__ float upper_term(float qv, uint32_t mm) {
  return qv >= 0.0f ? bf16_hi(mm) : bf16_lo(mm);
}
// Lane exchanges, bitonic sorting and merging of 64 keys held one per lane
// (key = order key << 32 | ~block: unique, so no ties).
// Lane l receives lane l ^ J's value.  J < 16: DPP inside 16-lane rows
// (quad permutations; row_ror:n gives lane l the value of lane l - n mod 16,
// so J = 4 takes row_ror:4 or row_ror:12 by lane).  J = 16, 32: the gfx950
// permlane swaps, which with both operands v return, in every lane, the
// values of the lower and the upper lane of the pair (l, l ^ J).
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true);  // row_ror:4
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0xF, true);  // row_ror:12
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else {
    static_assert(J == 16 || J == 32, "lane distance");
    const auto r = J == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & J) ? r[0] : r[1];
  }
}
template <int J>
__device__ __forceinline__ unsigned long long key_xor(unsigned long long v) {
  return ((unsigned long long)lane_xor<J>((uint32_t)(v >> 32)) << 32) | lane_xor<J>((uint32_t)v);
}
// DPP exchanges inside 16-lane rows (gfx9 encodings): every lane of a row
// receives the row's max / sum.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dppf<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dppf<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dppf<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dppf<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dppf<0xB1>(x);
  x += dppf<0x4E>(x);
  x += dppf<0x141>(x);
  x += dppf<0x140>(x);
  return x;
}
// Whole-wave reductions (every lane receives the result): the row reduction,
// then the rows combined by the swaps at distance 16 and 32.
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  x = fmaxf(x, __uint_as_float(lane_xor<16>(__float_as_uint(x))));
  return fmaxf(x, __uint_as_float(lane_xor<32>(__float_as_uint(x))));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  x += __uint_as_float(lane_xor<16>(__float_as_uint(x)));
  return x + __uint_as_float(lane_xor<32>(__float_as_uint(x)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, lane_xor<1>(x));
  x = max(x, lane_xor<2>(x));
  x = max(x, lane_xor<4>(x));
  x = max(x, lane_xor<8>(x));
  x = max(x, lane_xor<16>(x));
  return max(x, lane_xor<32>(x));
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += (int)lane_xor<1>((uint32_t)x);
  x += (int)lane_xor<2>((uint32_t)x);
  x += (int)lane_xor<4>((uint32_t)x);
  x += (int)lane_xor<8>((uint32_t)x);
  x += (int)lane_xor<16>((uint32_t)x);
  return x + (int)lane_xor<32>((uint32_t)x);
}
// Half-cleaner of a bitonic run of 64 into descending halves: the lower lane
// of each pair (l, l ^ J) keeps the larger key (keys are unique).
template <int J>
__device__ __forceinline__ unsigned long long half_clean(unsigned long long v) {
  const unsigned long long o = key_xor<J>(v);
  return (v > o) == ((threadIdx.x & J) == 0) ? v : o;
}
// Lane l receives lane 63 - l's key: row_mirror reverses each 16-lane row,
// the swaps at distance 16 and 32 reverse the order of the rows.
__device__ __forceinline__ uint32_t lane_rev(uint32_t v) {
  v = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);  // row_mirror
  return lane_xor<32>(lane_xor<16>(v));
}
// The 64 largest of two descending lists of 64 keys (one per lane), in
// descending order: max(a, b reversed) is bitonic and holds them; a cascade of
// half-cleaners sorts it.
__device__ __forceinline__ unsigned long long merge_top64(unsigned long long a, unsigned long long b) {
  const unsigned long long br =
      ((unsigned long long)lane_rev((uint32_t)(b >> 32)) << 32) | lane_rev((uint32_t)b);
  unsigned long long v = a > br ? a : br;
  v = half_clean<32>(v);
  v = half_clean<16>(v);
  v = half_clean<8>(v);
  v = half_clean<4>(v);
  v = half_clean<2>(v);
  v = half_clean<1>(v);
  return v;
}
// The 64 smallest of the same two lists, descending: min(a, b reversed).
__device__ __forceinline__ unsigned long long merge_bottom64(unsigned long long a,
                                                             unsigned long long b) {
  const unsigned long long br =
      ((unsigned long long)lane_rev((uint32_t)(b >> 32)) << 32) | lane_rev((uint32_t)b);
  unsigned long long v = a > br ? br : a;
  v = half_clean<32>(v);
  v = half_clean<16>(v);
  v = half_clean<8>(v);
  v = half_clean<4>(v);
  v = half_clean<2>(v);
  v = half_clean<1>(v);
  return v;
}
__device__ __forceinline__ unsigned long long key_rev(unsigned long long v) {
  return ((unsigned long long)lane_rev((uint32_t)(v >> 32)) << 32) | lane_rev((uint32_t)v);
}
// Lists of 128 keys in two registers, descending: rank l in h (lane l), rank
// 64 + l in lo.  The 128 largest of two such lists: the elementwise maximum
// of one list and the other reversed is bitonic and holds them; the
// half-cleaner at distance 64 pairs the two registers lane by lane, then each
// register is sorted by the cleaners at distances 32 .. 1.
__device__ __forceinline__ void merge_top128(unsigned long long &ah, unsigned long long &al,
                                             unsigned long long bh, unsigned long long bl) {
  const unsigned long long rbl = key_rev(bl), rbh = key_rev(bh);
  const unsigned long long mh = ah > rbl ? ah : rbl, ml = al > rbh ? al : rbh;
  unsigned long long h = mh > ml ? mh : ml, lo = mh > ml ? ml : mh;
  h = half_clean<32>(h);
  lo = half_clean<32>(lo);
  h = half_clean<16>(h);
  lo = half_clean<16>(lo);
  h = half_clean<8>(h);
  lo = half_clean<8>(lo);
  h = half_clean<4>(h);
  lo = half_clean<4>(lo);
  h = half_clean<2>(h);
  lo = half_clean<2>(lo);
  h = half_clean<1>(h);
  lo = half_clean<1>(lo);
  ah = h;
  al = lo;
}
// One compare-exchange step of a bitonic sort into descending order: lane l
// and lane l ^ J compare; in a run of K lanes sorted descending (l & K = 0)
// the lower lane keeps the larger key, in an ascending run the smaller.
template <int K, int J>
__device__ __forceinline__ unsigned long long bitonic_step(unsigned long long v) {
  const unsigned long long o = key_xor<J>(v);
  const int l = threadIdx.x & 63;
  const bool keep_max = ((l & J) == 0) == ((l & K) == 0);
  return (v > o) == keep_max ? v : o;
}
__device__ __forceinline__ unsigned long long sort64_desc(unsigned long long v) {
  v = bitonic_step<2, 1>(v);
  v = bitonic_step<4, 2>(v);
  v = bitonic_step<4, 1>(v);
  v = bitonic_step<8, 4>(v);
  v = bitonic_step<8, 2>(v);
  v = bitonic_step<8, 1>(v);
  v = bitonic_step<16, 8>(v);
  v = bitonic_step<16, 4>(v);
  v = bitonic_step<16, 2>(v);
  v = bitonic_step<16, 1>(v);
  v = bitonic_step<32, 16>(v);
  v = bitonic_step<32, 8>(v);
  v = bitonic_step<32, 4>(v);
  v = bitonic_step<32, 2>(v);
  v = bitonic_step<32, 1>(v);
  v = half_clean<32>(v);  // the final merge: a descending run of 64
  v = half_clean<16>(v);
  v = half_clean<8>(v);
  v = half_clean<4>(v);
  v = half_clean<2>(v);
  v = half_clean<1>(v);
  return v;
}

// List of one score tile for the fast top-k (no MAW flags, kk <= kTileList):
// the tile's 64 largest approximate keys, descending.  Blocks past the end of
// the unit and blocks that are not candidates have order key 0 and sort
// last.  Every block among the unit's 64 largest keys is among its own
// tile's 64 largest, so merging the tiles' lists gives the unit's 64 largest.
// Each wave sorts its 64 keys across its lanes; wave 0 merges the four
// sorted lists and publishes the result.  Every thread of the workgroup calls
// it, after a barrier that follows the tile's keys' writes to sm.tk.
__device__ __forceinline__ void tile_list(const Ctx &c, int seq, int h, int tile, TopkSmem &sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const size_t unit = (size_t)seq * c.dm.Hkv + h;
  const int b = wv * 64 + lane;  // block tile * kScoreTile + b
  unsigned long long v =
      ((unsigned long long)sm.tk[b] << 32) | (uint32_t)~(uint32_t)(tile * kScoreTile + b);
  v = sort64_desc(v);
  if (wv > 0) sm.srt[wv][lane] = v;
  __syncthreads();
  if (wv == 0) {
    const unsigned long long m01 = merge_top64(v, sm.srt[1][lane]);
    const unsigned long long m23 = merge_top64(sm.srt[2][lane], sm.srt[3][lane]);
    st_dev(&c.sc.cand[unit * c.dm.key_stride + (size_t)tile * kTileList + lane],
           merge_top64(m01, m23));
  }
}
// The same for kTileList < k <= kFastK: the tile's 128 largest keys,
// descending, as two lists of 64 (ranks l and 64 + l of lane l) at
// [128 t, 128 t + 128) of the unit's candidate lists.
__device__ __forceinline__ void tile_list128(const Ctx &c, int seq, int h, int tile, TopkSmem &sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const size_t unit = (size_t)seq * c.dm.Hkv + h;
  const int b = wv * 64 + lane;
  unsigned long long v =
      ((unsigned long long)sm.tk[b] << 32) | (uint32_t)~(uint32_t)(tile * kScoreTile + b);
  v = sort64_desc(v);
  if (wv > 0) sm.srt[wv][lane] = v;
  __syncthreads();
  if (wv == 0) {
    const unsigned long long w1 = sm.srt[1][lane], w2 = sm.srt[2][lane], w3 = sm.srt[3][lane];
    unsigned long long ah = merge_top64(v, w1), al = merge_bottom64(v, w1);
    merge_top128(ah, al, merge_top64(w2, w3), merge_bottom64(w2, w3));
    unsigned long long *cl = c.sc.cand + unit * c.dm.key_stride + (size_t)tile * kFastK;
    st_dev(&cl[lane], ah);
    st_dev(&cl[kTileList + lane], al);
  }
}

// fast_ok: also write the tile's candidate list for the fast top-k (tile <
// kFastTiles).  PQH: one key per query head (each head ranks its own bounds;
// the keys, bounds and flag counts of query head j of the unit sit at unit
// index unit * G + j), no list.
template <int D, int G, bool PQH = false>
__device__ __attribute__((always_inline)) bool score_tile(const Ctx &c, int i, int seq, int h, const HeadInfo &hi,
                           int N, int n_blk, int tile, const uint16_t *__restrict__ q,
                           TopkSmem &sm, bool fast_ok, UG &g) {
  uint32_t *red = sm.red;
  constexpr int MM = D / 16;    // MFMAs per 16 blocks (k = 2d values, 32 per MFMA)
  constexpr int GPW = kScoreTile / 64;  // 16-block groups per wave
  constexpr int C4 = D / 4;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, lgrp = lane >> 4;
  const int base = tile * kScoreTile + wv * 16 * GPW;
  const uint4 *sp = reinterpret_cast<const uint4 *>(c.L.summ + hi.summ_off +
                                                    (size_t)seq * C4 * hi.nbmax * 8);
  // the first kTileAhead 16-block groups are loaded before anything else;
  // each later group is issued once the group kTileAhead before it has been
  // scored, so a wave keeps kTileAhead groups in flight (block indices are
  // clamped, so the loads of a wave past the last block stay in bounds)
  constexpr int AHEAD = kTileAhead < GPW ? kTileAhead : GPW;
  uint4 kf[GPW][MM];
  const int nb_last = max(n_blk - 1, 0);
  auto load_group = [&](int gi) {
    const int blk = min(base + gi * 16 + r16, nb_last);
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) kf[gi][mm] = sp[(size_t)(4 * mm + lgrp) * hi.nbmax + blk];
  };
#pragma unroll
  for (int gi = 0; gi < AHEAD; ++gi) load_group(gi);
  const int qh0 = h * G;
  const uint16_t *qrow = q + ((size_t)i * c.dm.Hq + qh0 + min(r16, G - 1)) * D;
  uint2 qw[MM];
#pragma unroll
  for (int mm = 0; mm < MM; ++mm)
    qw[mm] = *reinterpret_cast<const uint2 *>(qrow + 4 * (4 * mm + lgrp));
  // MAW of the lane's blocks, for the flag (lanes of channel group 0 own the
  // keys)
  const bool need_maw = c.dm.maw_beta > 0.0f;
  const float *mwp = c.L.maw + hi.maw_off + (size_t)seq * hi.nbmax;
  float mwv[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int blk = base + gi * 16 + r16;
    mwv[gi] = (need_maw && (lgrp == 0 || PQH) && blk < n_blk) ? mwp[blk] : 0.0f;
  }
  __builtin_amdgcn_sched_barrier(0);
  g = unit_geom(N, hi, c.dm);
  const bool publish = !PQH && fast_ok && g.kk <= kFastK;
  // A operand: lane = head r16 (zero rows past G), channel quad 4*mm + lgrp,
  // pairs (q-, q+) matching the (min, max) pairs of the summaries
  uint4 qa[MM];
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) {
    const uint32_t x[2] = {qw[mm].x, qw[mm].y};
    uint32_t o4[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t lo = x[t] & 0xffffu, hi16 = x[t] >> 16;
      const uint32_t lo_neg = (lo & 0x8000u) ? lo : 0u, lo_pos = (lo & 0x8000u) ? 0u : lo;
      const uint32_t hi_neg = (hi16 & 0x8000u) ? hi16 : 0u, hi_pos = (hi16 & 0x8000u) ? 0u : hi16;
      o4[2 * t] = lo_neg | (lo_pos << 16);
      o4[2 * t + 1] = hi_neg | (hi_pos << 16);
    }
    qa[mm] = r16 < G ? make_uint4(o4[0], o4[1], o4[2], o4[3]) : make_uint4(0, 0, 0, 0);
  }
  const uint32_t absm = 0x7fff7fffu;
  float emax = 0.0f;
  float eh[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // PQH: bounds of heads 4 lgrp + jr
  int n_flag = 0;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    if (gi >= 1 && gi - 1 + AHEAD < GPW) {  // group gi - 1 is scored
      __builtin_amdgcn_sched_barrier(0);
      load_group(gi - 1 + AHEAD);
      __builtin_amdgcn_sched_barrier(0);
    }
    // partial sums over 64 (min, max) values (two chained MFMAs), added in
    // fp32: a tighter error bound than one chain over all 2d values
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acce = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m2 = 0; m2 < MM; m2 += 2) {
      f32x4 pa = {0.f, 0.f, 0.f, 0.f}, pe = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = m2; mm < m2 + 2; ++mm) {
        const uint4 a = qa[mm], b = kf[gi][mm];
        pa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), pa, 0, 0, 0);
        const uint4 aa = make_uint4(a.x & absm, a.y & absm, a.z & absm, a.w & absm);
        const uint4 ba = make_uint4(b.x & absm, b.y & absm, b.z & absm, b.w & absm);
        pe = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aa),
                                                     __builtin_bit_cast(bf16x8, ba), pe, 0, 0, 0);
      }
      acc += pa;
      acce += pe;
    }
    // lane (r16, lgrp) holds block r16 for heads 4*lgrp + jr
    if constexpr (PQH) {
      const int blk = base + gi * 16 + r16;
      if (blk < g.n_sc) {
        const bool cand = is_candidate(g, blk);
        const bool fl = c.dm.maw_beta > 0.0f &&
                        (double)mwv[gi] * (double)dense_count(g) > (double)c.dm.maw_beta * (double)hi.S;
        n_flag += (fl && cand && lgrp == 0) ? 1 : 0;
        const int slot = key_slot(blk, g.n_sc);
#pragma unroll
        for (int jr = 0; jr < 4; ++jr) {
          const int hd = 4 * lgrp + jr;
          if (hd < G) {
            unsigned long long kv = cand ? order_key(acc[jr]) : 0u;
            if (fl) kv |= 1ull << 32;
            if (cand) eh[jr] = fmaxf(eh[jr], score_eps(acce[jr], acc[jr]));
            st_dev(&c.sc.keyflag[(((size_t)seq * c.dm.Hkv + h) * G + hd) * c.dm.key_stride + slot], kv);
          }
        }
      }
      continue;
    }
    float A = -INFINITY, E = 0.0f;
#pragma unroll
    for (int jr = 0; jr < 4; ++jr)
      if (lgrp * 4 + jr < G) {
        A = fmaxf(A, acc[jr]);
        E = fmaxf(E, acce[jr]);
      }
    if constexpr (G > 4) {
      A = fmaxf(A, __shfl_xor(A, 16, 64));
      E = fmaxf(E, __shfl_xor(E, 16, 64));
    }
    const int blk = base + gi * 16 + r16;
    unsigned long long kv = 0u;
    if (lgrp == 0 && blk < g.n_sc) {
      const size_t ko = ((size_t)seq * c.dm.Hkv + h) * c.dm.key_stride + key_slot(blk, g.n_sc);
      const bool cand = is_candidate(g, blk);
      kv = cand ? order_key(A) : 0u;
      if (cand) emax = fmaxf(emax, score_eps(E, A));
      if (c.dm.maw_beta > 0.0f) {
        if ((double)mwv[gi] * (double)dense_count(g) > (double)c.dm.maw_beta * (double)hi.S) {
          kv |= 1ull << 32;
          n_flag += cand ? 1 : 0;
        }
      }
      st_dev(&c.sc.keyflag[ko], kv);
    }
    if (publish && lgrp == 0) sm.tk[wv * 16 * GPW + gi * 16 + r16] = (uint32_t)kv;
  }
  if constexpr (PQH) {
    // per query head: the largest bound over the tile (rows of 16 lanes share
    // lgrp, so a row maximum gathers one head's blocks), then over the waves
    const int nf = wave_sum_i(n_flag);
#pragma unroll
    for (int jr = 0; jr < 4; ++jr) {
      const float e = row_max16(eh[jr]);
      if (r16 == 0 && 4 * lgrp + jr < G) sm.ukey[wv * 8 + 4 * lgrp + jr] = __float_as_uint(e);
    }
    if (lane == 0) red[4 + wv] = (uint32_t)nf;
    __syncthreads();
    if (threadIdx.x < G) {
      const int hd = threadIdx.x;
      uint32_t *acc = &c.sc.unit_acc[4 * (((size_t)seq * c.dm.Hkv + h) * G + hd)];
      const uint32_t e = max(max(sm.ukey[hd], sm.ukey[8 + hd]), max(sm.ukey[16 + hd], sm.ukey[24 + hd]));
      __hip_atomic_fetch_max(acc, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t f = red[4] + red[5] + red[6] + red[7];
      if (f) __hip_atomic_fetch_add(acc + 1, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return false;
  }
  // the unit's largest error bound (non-negative floats order as their bits)
  // and its flagged candidates, accumulated over the tiles
  uint32_t eb = __float_as_uint(emax);
  eb = wave_max_u32(eb);
  const int nf = wave_sum_i(n_flag);
  if (lane == 0) {
    red[wv] = eb;
    red[4 + wv] = (uint32_t)nf;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t *acc = &c.sc.unit_acc[4 * ((size_t)seq * c.dm.Hkv + h)];
    __hip_atomic_fetch_max(acc, max(max(red[0], red[1]), max(red[2], red[3])), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t f = red[4] + red[5] + red[6] + red[7];
    if (f) __hip_atomic_fetch_add(acc + 1, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  SD_TL(1);  // keys written
  if (publish) {
    if (g.kk <= kTileList)
      tile_list(c, seq, h, tile, sm);
    else
      tile_list128(c, seq, h, tile, sm);
  }
  return publish;
}

template <int D>
__device__ double exact_score_seq(const Ctx &c, int seq, const HeadInfo &hi, int blk,
                                  const float *qs /* LDS [D] of this head */) {
  constexpr int C4 = D / 4;
  const uint4 *sp = reinterpret_cast<const uint4 *>(c.L.summ + hi.summ_off +
                                                    (size_t)seq * C4 * hi.nbmax * 8) + blk;
  double acc = 0.0;
  for (int c4 = 0; c4 < C4; ++c4) {
    const uint4 w = sp[(size_t)c4 * hi.nbmax];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float qv = qs[4 * c4 + j];
      acc = fma((double)qv, (double)upper_term(qv, ws[j]), acc);
    }
  }
  return acc;
}

__device__ __forceinline__ double dpp_quad_f64(double x, int which) {
  const unsigned long long b = __double_as_longlong(x);
  int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
  if (which == 1) {
    lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false);
  } else {
    lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false);
  }
  return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ int dpp_quad_i32(int x, int which) {
  return which == 1 ? __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false)
                    : __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
}

// The same sum by the four lanes of a quad (lane % 4 = part; part p sums
// channels [p D/4, (p+1) D/4)), returned in all four lanes.  Every product
// p_c = q_c s_c has at most 16 significant bits, so it is a multiple of
// 2^(e_c - 16) with |p_c| < 2^e_c; when sum_c |p_c| < 2^(min_c e_c + 36)
// (half the 2^53 range, covering the rounding of that bound) every partial
// sum in any order is exact, hence equal to the sequential sum.  Otherwise
// the sequential sum is taken.  Every lane of the wave must call it.
template <int D>
__device__ double exact_score_quad(const Ctx &c, int seq, const HeadInfo &hi, int blk,
                                   const float *qs /* LDS [D] of this head */, bool on) {
  constexpr int C4 = D / 4, P4 = C4 / 4;  // channel quads per part
  const int part = threadIdx.x & 3;
  const uint4 *sp = reinterpret_cast<const uint4 *>(c.L.summ + hi.summ_off +
                                                    (size_t)seq * C4 * hi.nbmax * 8) + blk;
  uint4 w[P4];
#pragma unroll
  for (int t = 0; t < P4; ++t)
    w[t] = on ? sp[(size_t)(part * P4 + t) * hi.nbmax] : make_uint4(0, 0, 0, 0);
  double ps = 0.0, sabs = 0.0;
  int emin = 4096;
#pragma unroll
  for (int t = 0; t < P4; ++t) {
    const uint32_t ws[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float qv = qs[4 * (part * P4 + t) + j];
      const double pr = (double)qv * (double)upper_term(qv, ws[j]);
      ps += pr;
      sabs += fabs(pr);
      emin = min(emin, pr != 0.0 ? __builtin_amdgcn_frexp_exp(pr) : 4096);
    }
  }
  ps += dpp_quad_f64(ps, 1);
  ps += dpp_quad_f64(ps, 2);
  sabs += dpp_quad_f64(sabs, 1);
  sabs += dpp_quad_f64(sabs, 2);
  emin = min(emin, dpp_quad_i32(emin, 1));
  emin = min(emin, dpp_quad_i32(emin, 2));
  // frexp exponents: |p| < 2^e; sabs < 2^(emin + 36) <=> frexp_exp(sabs) <= emin + 36
  const bool exact = sabs == 0.0 || __builtin_amdgcn_frexp_exp(sabs) <= emin + 36;
  if (on && !exact) ps = exact_score_seq<D>(c, seq, hi, blk, qs);
  return ps;
}

// Exact group scores of NB blocks per lane quad (the quad's lanes split the
// channels): every block's summary is loaded once, then each head's sum is
// taken as in exact_score_quad (the quad's partial sums where that order is
// exact, else the plain sum in channel order); best: the maximum over the G
// heads (qs: LDS [G][D]).  Every lane of the wave takes part.
template <int D, int G, int NB>
__device__ __forceinline__ void exact_group_quads(const Ctx &c, int seq, const HeadInfo &hi,
                                                  const int (&blk)[NB], const bool (&on)[NB],
                                                  const float *qs, double (&best)[NB]) {
  constexpr int C4 = D / 4, P4 = C4 / 4;
  const int part = threadIdx.x & 3;
  const uint4 *sp = reinterpret_cast<const uint4 *>(c.L.summ + hi.summ_off +
                                                    (size_t)seq * C4 * hi.nbmax * 8);
  uint4 w[NB][P4];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int t = 0; t < P4; ++t)
      w[n][t] = on[n] ? sp[(size_t)(part * P4 + t) * hi.nbmax + blk[n]] : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int n = 0; n < NB; ++n) best[n] = -INFINITY;
#pragma unroll 1
  for (int hh = 0; hh < G; ++hh) {
    const float *qh = qs + hh * D;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      double ps = 0.0, sabs = 0.0;
      int emin = 4096;
#pragma unroll
      for (int t = 0; t < P4; ++t) {
        const uint32_t ws[4] = {w[n][t].x, w[n][t].y, w[n][t].z, w[n][t].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float qv = qh[4 * (part * P4 + t) + j];
          const double pr = (double)qv * (double)upper_term(qv, ws[j]);
          ps += pr;
          sabs += fabs(pr);
          emin = min(emin, pr != 0.0 ? __builtin_amdgcn_frexp_exp(pr) : 4096);
        }
      }
      ps += dpp_quad_f64(ps, 1);
      ps += dpp_quad_f64(ps, 2);
      sabs += dpp_quad_f64(sabs, 1);
      sabs += dpp_quad_f64(sabs, 2);
      emin = min(emin, dpp_quad_i32(emin, 1));
      emin = min(emin, dpp_quad_i32(emin, 2));
      const bool exact = sabs == 0.0 || __builtin_amdgcn_frexp_exp(sabs) <= emin + 36;
      if (on[n] && !exact) ps = exact_score_seq<D>(c, seq, hi, blk[n], qh);
      best[n] = fmax(best[n], ps);
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k of one unit, in one wave, ordered by (MAW flag desc, exact fp32 score
// desc, index asc) ([FLX] per-head top-k; [HGCA] MAW threshold first; R5,
// R11).
//
// Block j sits in lane j % 64 of row j / 64 as one word: 0 = not selectable,
// 1 = taken by the flag tier, otherwise the order key of its approximate
// score (keys of finite or infinite floats are >= 0x007fffff).  Rows below
// kTopkRegRows stay in registers; later rows live in LDS, or in the global
// scratch beyond the LDS the launch reserved.
//   1. bisection on the key value narrows [a, b], which always holds the
//      k-th largest approximate key T_a (one ballot + popcount per row and
//      step), until b - a is within the unit's error bound eps;
//   2. band: A > b + 2 eps is in, A < a - 2 eps out (every approximate score
//      lies within eps of its exact score, so the k-th exact score lies
//      within eps of T_a); both edges are rounded outwards to float keys so
//      that the tests are integer compares.  Blocks inside the band are
//      listed in index order and re-scored exactly, one lane per (block,
//      head);
//   3. the kr2 still missing are the largest exact keys of that list (ties
//      to the lower index), found by bisection; they are marked in an LDS
//      bitmask of rows;
//   4. ordered compaction with ballots: ascending block indices.
template <int D, int G>
__device__ __attribute__((always_inline)) void topk_unit(const Ctx &c, int seq, size_t unit, size_t out,
                          const HeadInfo &hi,
                          const UG &g, const uint16_t *__restrict__ q,
                          int32_t *__restrict__ blk_idx, int32_t *__restrict__ blk_cnt,
                          int k_cap, TopkSmem &sm, uint32_t *lrows, int lrows_words,
                          unsigned long long *dmask /* LDS, one word per row */,
                          unsigned long long *tagd = nullptr, uint32_t epoch = 0) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int n = g.n_sc, rows = cdiv(n, 64);
  const size_t uo = unit * c.dm.key_stride;
  const unsigned long long *gkf = c.sc.keyflag + uo;
  constexpr int kRegWords = kTopkRegRows * 64;
  // words of the rows past the registers
  const bool mem_lds = rows * 64 - kRegWords <= lrows_words;
  uint32_t *gw = c.sc.keys + uo;
  auto mem_ld = [&](int j) -> uint32_t { return mem_lds ? lrows[j - kRegWords] : ld_dev(&gw[j]); };
  auto mem_st = [&](int j, uint32_t v) {
    if (mem_lds) lrows[j - kRegWords] = v; else st_dev(&gw[j], v);
  };
  // uncertain list: LDS up to kTopkUnc entries, global scratch after
  int32_t *gul = c.sc.ulist + uo;
  uint32_t *guk = c.sc.ukeys + uo;
  auto ul_ld = [&](int p) -> int { return p < kTopkUnc ? sm.ulist[p] : ld_dev(&gul[p]); };
  auto ul_st = [&](int p, int v) { if (p < kTopkUnc) sm.ulist[p] = v; else st_dev(&gul[p], v); };
  auto uk_ld = [&](int p) -> uint32_t { return p < kTopkUnc ? sm.ukey[p] : ld_dev(&guk[p]); };
  auto uk_st = [&](int p, uint32_t v) { if (p < kTopkUnc) sm.ukey[p] = v; else st_dev(&guk[p], v); };

  // 0. every load in flight together: the score tiles' accumulators (error
  // bound, flagged candidates), the register rows, the group's query
  const uint32_t eps_bits = ld_dev(&c.sc.unit_acc[4 * unit]);
  const uint32_t f_raw = ld_dev(&c.sc.unit_acc[4 * unit + 1]);
  const int jl = max(n - 1, 0);
  unsigned long long kv[kTopkRegRows];
#pragma unroll
  for (int r = 0; r < kTopkRegRows; ++r) kv[r] = ld_dev(&gkf[min(r * 64 + lane, jl)]);
  constexpr int QPL = (G * D + 63) / 64;
  const uint16_t *qg = q + out * G * D;
  uint16_t qv[QPL];
#pragma unroll
  for (int r = 0; r < QPL; ++r) qv[r] = qg[min(r * 64 + lane, G * D - 1)];

  const bool use_flag = c.dm.maw_beta > 0.0f;
  const int F = use_flag ? (int)f_raw : 0;
  const int kk = g.kk;
  // every flagged candidate is taken when they do not fill k on their own
  // (the unflagged ones are ranked for the rest); otherwise only the flagged
  // candidates are ranked
  const bool take_flagged = F < kk;
  const uint32_t want = take_flagged ? 0u : 1u;
  const int k_sub = take_flagged ? kk - F : kk;
  auto word_of = [&](unsigned long long x) -> uint32_t {
    const uint32_t key = (uint32_t)x;
    if (key == 0u) return 0u;
    const uint32_t fl = use_flag ? (uint32_t)(x >> 32) & 1u : 0u;
    return fl == want ? key : (take_flagged ? 1u : 0u);
  };
  for (int r = lane; r < max(rows, kTopkRegRows); r += 64) dmask[r] = 0ull;
#pragma unroll
  for (int r = 0; r < QPL; ++r) {
    const int x = r * 64 + lane;
    if (x < G * D) sm.qs[x] = __uint_as_float((uint32_t)qv[r] << 16);
  }
  uint32_t w[kTopkRegRows];
  uint32_t lo = 0xffffffffu, hi_k = 0u;
  uint32_t gm[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // maxima of rows r mod 8
#pragma unroll
  for (int r = 0; r < kTopkRegRows; ++r) {
    w[r] = r * 64 + lane < n ? word_of(kv[r]) : 0u;
    gm[r & 7] = max(gm[r & 7], w[r]);
    if (w[r] >= 2u) {
      lo = min(lo, w[r]);
      hi_k = max(hi_k, w[r]);
    }
  }
  for (int r0 = kTopkRegRows; r0 < rows; r0 += 8) {
    unsigned long long kb[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) kb[x] = ld_dev(&gkf[min((r0 + x) * 64 + lane, jl)]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int j = (r0 + x) * 64 + lane;
      if (r0 + x < rows) {
        const uint32_t v = j < n ? word_of(kb[x]) : 0u;
        mem_st(j, v);
#pragma unroll
        for (int y = 0; y < 8; ++y)
          if (((r0 + x) & 7) == y) gm[y] = max(gm[y], v);
        if (v >= 2u) {
          lo = min(lo, v);
          hi_k = max(hi_k, v);
        }
      }
    }
  }
  wait_vmem();
  auto count_ge = [&](uint32_t t) -> int {
    unsigned long long m[kTopkRegRows];
#pragma unroll
    for (int r = 0; r < kTopkRegRows; ++r) m[r] = __ballot(w[r] >= t);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < kTopkRegRows; ++r) cnt += __popcll(m[r]);
    for (int r = kTopkRegRows; r < rows; ++r) cnt += count_lanes(mem_ld(r * 64 + lane) >= t);
    return cnt;
  };

  // 1-3. band and decisions.  Uncertain: kb_lo <= w <= kb_hi; in: w > kb_hi.
  uint32_t kb_lo = 0xffffffffu, kb_hi = 0xffffffffu;
  if (k_sub > 0) {
    const double eps = (double)__uint_as_float(eps_bits);
    uint32_t a = wave_min_u(lo), b = wave_max_u(hi_k);
    // invariant: #words >= a is cnt_a >= k_sub, #words > b is cnt_b1 < k_sub
    const int n_cand = g.ns < g.wlo ? div_S(g.wlo + g.S - 1, g.S) - div_S(g.ns, g.S) : 0;
    int cnt_a = take_flagged ? n_cand - F : F, cnt_b1 = 0;
    // lower bound on T_a: the k_sub-th largest of the maxima of the row
    // groups (r mod NG; distinct blocks' keys), when there are enough of them
    if (k_sub <= 512) {
      const int NG = k_sub <= 256 ? 4 : 8;
      if (NG == 4) {
#pragma unroll
        for (int y = 0; y < 4; ++y) gm[y] = max(gm[y], gm[y + 4]), gm[y + 4] = 0u;
      }
      int nv = 0;
      uint32_t glo = 0xffffffffu, ghi = 0u;
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        nv += count_lanes(gm[y] >= 2u);
        if (gm[y] >= 2u) glo = min(glo, gm[y]);
        ghi = max(ghi, gm[y]);
      }
      if (nv >= k_sub) {
        uint32_t ga = wave_min_u(glo), gb = wave_max_u(ghi);
        for (int it = 0; it < 10 && ga < gb; ++it) {
          const uint32_t mid = ga + ((gb - ga) >> 1) + 1u;
          int cg = 0;
#pragma unroll
          for (int y = 0; y < 4; ++y) cg += count_lanes(gm[y] >= mid);
          if (NG == 8) {
#pragma unroll
            for (int y = 4; y < 8; ++y) cg += count_lanes(gm[y] >= mid);
          }
          if (cg >= k_sub) ga = mid; else gb = mid - 1u;
        }
        a = ga;
        cnt_a = count_ge(a);
      }
    }
    auto wide = [&]() {
      return a < b && (double)key_to_float(b) - (double)key_to_float(a) > eps;
    };
    if (wide() && cnt_a - cnt_b1 <= kTopkUnc) {
      // the words in [a, b], up to 8 per lane; then
      // count_ge(t) = above + #(x >= t) for a < t <= b + 1
      const int above = cnt_b1;
      int base = 0;
      auto gather = [&](uint32_t v) {
        const bool in = v >= a && v <= b;
        const unsigned long long m = __ballot(in);
        if (in && base + lanes_below(m) < kTopkUnc) sm.ukey[base + lanes_below(m)] = v;
        base += __popcll(m);
      };
#pragma unroll
      for (int r = 0; r < kTopkRegRows; ++r) gather(w[r]);
      for (int r = kTopkRegRows; r < rows; ++r) gather(mem_ld(r * 64 + lane));
      const int xr = cdiv(min(base, kTopkUnc), 64);
      uint32_t x[kTopkUnc / 64];
#pragma unroll
      for (int y = 0; y < kTopkUnc / 64; ++y)
        x[y] = y * 64 + lane < min(base, kTopkUnc) ? sm.ukey[y * 64 + lane] : 0u;
      while (wide()) {
        const uint32_t mid = a + ((b - a) >> 1) + 1u;
        int cm = above;
#pragma unroll
        for (int y = 0; y < kTopkUnc / 64; ++y)
          if (y < xr) cm += count_lanes(x[y] >= mid);
        if (cm >= k_sub) { a = mid; cnt_a = cm; } else { b = mid - 1u; cnt_b1 = cm; }
      }
    }
    while (wide()) {
      const uint32_t mid = a + ((b - a) >> 1) + 1u;  // a < mid <= b
      const int cm = count_ge(mid);
      if (cm >= k_sub) { a = mid; cnt_a = cm; } else { b = mid - 1u; cnt_b1 = cm; }
    }
    kb_hi = order_key(__double2float_rd((double)key_to_float(b) + 2.0 * eps));
    kb_lo = order_key(__double2float_ru((double)key_to_float(a) - 2.0 * eps));
    // list the uncertain blocks in index order; count the sure ones
    int n_in = 0, n_unc = 0;
    auto list_row = [&](int j, uint32_t v) {
      const bool unc = v >= kb_lo && v <= kb_hi;
      const unsigned long long m = __ballot(unc);
      if (unc) ul_st(n_unc + lanes_below(m), j);
      n_unc += __popcll(m);
      n_in += count_lanes(v > kb_hi);
    };
#pragma unroll
    for (int r = 0; r < kTopkRegRows; ++r) list_row(r * 64 + lane, w[r]);
    for (int r = kTopkRegRows; r < rows; ++r) list_row(r * 64 + lane, mem_ld(r * 64 + lane));
    wait_vmem();
    const int kr2 = k_sub - n_in;  // >= 1: T_a's own block is uncertain
    // exact keys of the uncertain blocks, one lane quad per (block, head)
    constexpr int BPR = 16 / G;  // blocks per round
    for (int u0 = 0; u0 < n_unc; u0 += BPR) {
      const int pair = lane >> 2, uu = u0 + pair / G, gg = pair % G;
      const bool on = pair < BPR * G && uu < n_unc;
      const double U = exact_score_quad<D>(c, seq, hi, on ? ul_ld(uu) : 0,
                                           sm.qs + (on ? gg : 0) * D, on);
      if ((lane & 3) == 0) sm.ud[pair] = U;
      if (lane < BPR && u0 + lane < n_unc) {
        double best = sm.ud[lane * G];
        for (int x = 1; x < G; ++x) best = sm.ud[lane * G + x] > best ? sm.ud[lane * G + x] : best;
        uk_st(u0 + lane, order_key((float)best));
      }
    }
    wait_vmem();
    // the kr2 largest exact keys of the list, ties to the lower index
    if (n_unc <= 64) {
      // rank of each entry: larger keys, then equal keys listed earlier
      const uint32_t e = lane < n_unc ? sm.ukey[lane] : 0u;
      int rank = 0;
      for (int p = 0; p < n_unc; ++p) {
        const uint32_t ep = (uint32_t)__builtin_amdgcn_readlane((int)e, p);
        rank += (ep > e || (ep == e && p < lane)) ? 1 : 0;
      }
      if (lane < n_unc && rank < kr2) {
        const int j = sm.ulist[lane];
        atomicOr(&dmask[j >> 6], 1ull << (j & 63));
      }
    } else {
    const int urows = cdiv(n_unc, 64);
    const uint32_t e0 = lane < n_unc ? uk_ld(lane) : 0u;
    uint32_t lo2 = lane < n_unc ? e0 : 0xffffffffu, hi2 = e0;
    for (int r = 1; r < urows; ++r) {
      const int p = r * 64 + lane;
      if (p < n_unc) {
        const uint32_t e = uk_ld(p);
        lo2 = min(lo2, e);
        hi2 = max(hi2, e);
      }
    }
    lo2 = wave_min_u(lo2);
    hi2 = wave_max_u(hi2);
    auto ucount_ge = [&](uint32_t t) -> int {
      int cnt = count_lanes(e0 >= t);
      for (int r = 1; r < urows; ++r) {
        const int p = r * 64 + lane;
        cnt += count_lanes(p < n_unc && uk_ld(p) >= t);
      }
      return cnt;
    };
    const uint32_t T2 = bisect_kth(lo2, hi2, kr2, ucount_ge);
    const int kr2_eq = kr2 - (T2 == 0xffffffffu ? 0 : ucount_ge(T2 + 1u));
    int eqb = 0;
    for (int r = 0; r < urows; ++r) {
      const int p = r * 64 + lane;
      const uint32_t e = r == 0 ? e0 : (p < n_unc ? uk_ld(p) : 0u);
      const bool eq = p < n_unc && e == T2;
      const unsigned long long me = __ballot(eq);
      const bool take = (p < n_unc && e > T2) || (eq && eqb + lanes_below(me) < kr2_eq);
      eqb += __popcll(me);
      if (take) {
        const int j = ul_ld(p);
        atomicOr(&dmask[j >> 6], 1ull << (j & 63));
      }
    }
    }
  }

  // 4. ordered compaction
  int32_t *dst = blk_idx + out * k_cap;
  int ob = 0;
  auto emit_row = [&](int r, uint32_t v, unsigned long long dm) {
    const bool ch = v == 1u || v > kb_hi || ((dm >> lane) & 1ull);
    const unsigned long long mc = __ballot(ch);
    const int o = ob + lanes_below(mc);
    if (ch && o < k_cap) {
      st_dev(&dst[o], r * 64 + lane);
      if (tagd && o < c.dm.kcap)
        st_dev(&tagd[o], ((unsigned long long)epoch << 32) | (uint32_t)(r * 64 + lane));
    }
    ob += __popcll(mc);
  };
  {
    unsigned long long dm[kTopkRegRows];
#pragma unroll
    for (int r = 0; r < kTopkRegRows; ++r) dm[r] = dmask[r];
#pragma unroll
    for (int r = 0; r < kTopkRegRows; ++r) emit_row(r, w[r], dm[r]);
  }
  for (int r = kTopkRegRows; r < rows; ++r) emit_row(r, mem_ld(r * 64 + lane), dmask[r]);
  if (lane == 0) {
    st_dev(&blk_cnt[out], kk);
    st_dev(&c.sc.unit_acc[4 * unit], 0u);  // cleared for the next step
    st_dev(&c.sc.unit_acc[4 * unit + 1], 0u);
    st_dev(&c.sc.unit_acc[4 * unit + 2], eps_bits);  // the bound this selection used
  }
}

// Workgroup helpers of the wide top-k (every thread calls them; red holds 8
// words of LDS, used in two halves by alternate calls).
__device__ __forceinline__ int wg_sum(int x, uint32_t *red, int &slot) {
  const int wv = threadIdx.x >> 6;
  x = wave_sum_i(x);
  uint32_t *r = red + 4 * slot;
  slot ^= 1;
  if ((threadIdx.x & 63) == 0) r[wv] = (uint32_t)x;
  __syncthreads();
  return (int)(r[0] + r[1] + r[2] + r[3]);
}
// exclusive prefix of x over the threads in index order, and the total
__device__ __forceinline__ int wg_scan(int x, uint32_t *red, int &slot, int &total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = x;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31),
            r2 = __builtin_amdgcn_readlane(incl, 47);
  incl += (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
  uint32_t *r = red + 4 * slot;
  slot ^= 1;
  if (lane == 63) r[wv] = (uint32_t)incl;
  __syncthreads();
  int before = 0;
  for (int v = 0; v < wv; ++v) before += (int)r[v];
  total = (int)(r[0] + r[1] + r[2] + r[3]);
  return before + incl - x;
}

// Full top-k of a long unit by all four waves (the same order and result as
// topk_unit): thread t holds the words of blocks [t m, t m + m), m =
// ceil(n / 256) <= kWideM, in registers.  The k-th largest word is bracketed
// by bisection with workgroup counts until the bracket is within eps; the
// band is listed in index order by a workgroup scan, re-scored exactly (lane
// quads of all waves) and ranked; the chosen blocks are put in ascending
// order by a second scan, through LDS when they fit so that the stores are
// coalesced.
template <int D, int G>
__device__ __attribute__((always_inline)) void topk_wide(const Ctx &c, int seq, size_t unit, size_t out,
                          const HeadInfo &hi,
                          const UG &g, const uint16_t *__restrict__ q,
                          int32_t *__restrict__ blk_idx, int32_t *__restrict__ blk_cnt,
                          int k_cap, TopkSmem &sm,
                          unsigned long long *dmask /* LDS, one word per row */,
                          int32_t *stage /* LDS, stage_words entries */, int stage_words,
                          unsigned long long *tagd = nullptr, uint32_t epoch = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = g.n_sc, rows = cdiv(n, 64);
  const int m = cdiv(n, 256), j0 = tid * m;
  const size_t uo = unit * c.dm.key_stride;
  const unsigned long long *gkf = c.sc.keyflag + uo;
  int32_t *gul = c.sc.ulist + uo;
  uint32_t *guk = c.sc.ukeys + uo;
  auto ul_ld = [&](int p) -> int { return p < kTopkUnc ? sm.ulist[p] : ld_dev(&gul[p]); };
  auto ul_st = [&](int p, int v) { if (p < kTopkUnc) sm.ulist[p] = v; else st_dev(&gul[p], v); };
  auto uk_ld = [&](int p) -> uint32_t { return p < kTopkUnc ? sm.ukey[p] : ld_dev(&guk[p]); };
  auto uk_st = [&](int p, uint32_t v) { if (p < kTopkUnc) sm.ukey[p] = v; else st_dev(&guk[p], v); };
  uint32_t *red = sm.red;
  int slot = 0;

  // 0. one batch of loads: the accumulators, the thread's keys, the query
  const uint32_t eps_bits = ld_dev(&c.sc.unit_acc[4 * unit]);
  const uint32_t f_raw = ld_dev(&c.sc.unit_acc[4 * unit + 1]);
  unsigned long long kv[kWideM];
#pragma unroll
  for (int x = 0; x < kWideM; ++x) kv[x] = (x < m && j0 + x < n) ? ld_dev(&gkf[x * 256 + tid]) : 0ull;
  constexpr int QT = (G * D + 255) / 256;
  const uint16_t *qg = q + out * G * D;
  uint16_t qv[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) qv[t] = qg[min(tid + 256 * t, G * D - 1)];

  const bool use_flag = c.dm.maw_beta > 0.0f;
  const int F = use_flag ? (int)f_raw : 0;
  const int kk = g.kk;
  const bool take_flagged = F < kk;
  const uint32_t want = take_flagged ? 0u : 1u;
  const int k_sub = take_flagged ? kk - F : kk;
  // the thread's blocks as bit masks (bit x: block j0 + x), so that the
  // single passes below are short loops over set bits rather than unrolled
  // code over all kWideM words: onem = always chosen (word 1), gtm = above
  // the band, bandm = in the band
  uint32_t w[kWideM];
  uint32_t lo = 0xffffffffu, hi_k = 0u;
  unsigned long long onem = 0ull, gtm = 0ull, bandm = 0ull;
#pragma unroll
  for (int x = 0; x < kWideM; ++x) {
    const uint32_t key = (uint32_t)kv[x];
    const uint32_t fl = use_flag ? (uint32_t)(kv[x] >> 32) & 1u : 0u;
    w[x] = key == 0u ? 0u : (fl == want ? key : (take_flagged ? 1u : 0u));
    onem |= w[x] == 1u ? (1ull << x) : 0ull;
    if (w[x] >= 2u) {
      lo = min(lo, w[x]);
      hi_k = max(hi_k, w[x]);
    }
  }
  for (int r = tid; r < rows; r += 256) dmask[r] = 0ull;
#pragma unroll
  for (int t = 0; t < QT; ++t)
    if (tid + 256 * t < G * D) sm.qs[tid + 256 * t] = __uint_as_float((uint32_t)qv[t] << 16);
  // workgroup counts of the words >= t1, t2, t3 (t1 <= t2 <= t3 > 1): the
  // first two packed in 16-bit halves (at most 10240 each), over the first
  // MM >= m words of each thread; LDS words red[8 s3 .. 8 s3 + 7], alternate
  // calls alternating
  int s3 = 0;
  auto count3 = [&](auto MMc, uint32_t t1, uint32_t t2, uint32_t t3, int &c1, int &c2, int &c3) {
    constexpr int MM = decltype(MMc)::value;
    int x12 = 0, x3 = 0;
#pragma unroll
    for (int x = 0; x < MM; ++x) {
      x12 += (w[x] >= t1 ? 1 : 0) + (w[x] >= t2 ? 0x10000 : 0);
      x3 += w[x] >= t3 ? 1 : 0;
    }
    x12 = wave_sum_i(x12);
    x3 = wave_sum_i(x3);
    uint32_t *r = red + 8 * s3;
    s3 ^= 1;
    if (lane == 0) {
      r[wv] = (uint32_t)x12;
      r[4 + wv] = (uint32_t)x3;
    }
    __syncthreads();
    const uint32_t s12 = r[0] + r[1] + r[2] + r[3];
    c1 = (int)(s12 & 0xffffu);
    c2 = (int)(s12 >> 16);
    c3 = (int)(r[4] + r[5] + r[6] + r[7]);
  };

  uint32_t kb_lo = 0xffffffffu, kb_hi = 0xffffffffu;
  if (k_sub > 0) {
    // 1. bracket [a, b] of the k_sub-th largest word T_a: #(>= a) >= k_sub >
    // #(> b), narrowed until within eps by a four-way search (three counts a
    // step); the band edges as in topk_unit
    const double eps = (double)__uint_as_float(eps_bits);
    lo = wave_min_u(lo);
    hi_k = wave_max_u(hi_k);
    if (lane == 0) {
      red[8 + wv] = lo;
      red[12 + wv] = hi_k;
    }
    __syncthreads();
    uint32_t a = min(min(red[8], red[9]), min(red[10], red[11]));
    uint32_t b = max(max(red[12], red[13]), max(red[14], red[15]));
    while (a < b && (double)key_to_float(b) - (double)key_to_float(a) > eps) {
      // a < t1 <= t2 <= t3 <= b at about the quarters of [a, b]
      const uint64_t span = (uint64_t)(b - a);
      const uint32_t t1 = a + (uint32_t)((span + 3u) / 4u);
      const uint32_t t2 = a + (uint32_t)((2u * span + 3u) / 4u);
      const uint32_t t3 = a + (uint32_t)((3u * span + 3u) / 4u);
      int c1, c2, c3;
      if (m <= 8)
        count3(std::integral_constant<int, 8>(), t1, t2, t3, c1, c2, c3);
      else if (m <= 16)
        count3(std::integral_constant<int, 16>(), t1, t2, t3, c1, c2, c3);
      else
        count3(std::integral_constant<int, kWideM>(), t1, t2, t3, c1, c2, c3);
      if (c3 >= k_sub) {
        a = t3;
      } else if (c2 >= k_sub) {
        a = t2;
        b = t3 - 1u;
      } else if (c1 >= k_sub) {
        a = t1;
        b = t2 - 1u;
      } else {
        b = t1 - 1u;
      }
    }
    __syncthreads();  // the counts' LDS words are free again
    kb_hi = order_key(__double2float_rd((double)key_to_float(b) + 2.0 * eps));
    kb_lo = order_key(__double2float_ru((double)key_to_float(a) - 2.0 * eps));
    // 2. the band in index order; the sure ones counted
#pragma unroll
    for (int x = 0; x < kWideM; ++x) {
      bandm |= (w[x] >= kb_lo && w[x] <= kb_hi) ? (1ull << x) : 0ull;
      gtm |= w[x] > kb_hi ? (1ull << x) : 0ull;
    }
    int n_unc = 0;
    int p = wg_scan(__popcll(bandm), red, slot, n_unc);
    const int n_in = wg_sum(__popcll(gtm), red, slot);
    for (unsigned long long bm = bandm; bm != 0ull; bm &= bm - 1ull)
      ul_st(p++, j0 + (int)__builtin_ctzll(bm));
    wait_vmem();
    __syncthreads();
    const int kr2 = k_sub - n_in;  // >= 1: T_a's own block is in the band
    // 3. exact keys of the band: one lane quad per (block, head), 64 / G
    // whole blocks a pass; then the best head per block
    constexpr int BPP = 64 / G;
    for (int b0 = 0; b0 < n_unc; b0 += BPP) {
      const int pair = tid >> 2, u = b0 + pair / G, gg = pair % G;
      const bool on = pair < BPP * G && u < n_unc;
      const double U = exact_score_quad<D>(c, seq, hi, on ? ul_ld(u) : 0, sm.qs + gg * D, on);
      if (on && (tid & 3) == 0) sm.ue[pair] = U;
      __syncthreads();
      if (tid < BPP && b0 + tid < n_unc) {
        double best = sm.ue[tid * G];
        for (int x = 1; x < G; ++x) best = sm.ue[tid * G + x] > best ? sm.ue[tid * G + x] : best;
        uk_st(b0 + tid, order_key((float)best));
      }
      __syncthreads();
    }
    wait_vmem();
    __syncthreads();
    // 4. the kr2 largest exact keys, ties to the lower index (list order)
    if (wv == 0) {
      if (n_unc <= 64) {
        const uint32_t e = lane < n_unc ? uk_ld(lane) : 0u;
        int rank = 0;
        for (int q2 = 0; q2 < n_unc; ++q2) {
          const uint32_t eq2 = (uint32_t)__builtin_amdgcn_readlane((int)e, q2);
          rank += (eq2 > e || (eq2 == e && q2 < lane)) ? 1 : 0;
        }
        if (lane < n_unc && rank < kr2) {
          const int j = ul_ld(lane);
          atomicOr(&dmask[j >> 6], 1ull << (j & 63));
        }
      } else {
        const int urows = cdiv(n_unc, 64);
        uint32_t lo2 = 0xffffffffu, hi2 = 0u;
        for (int r = 0; r < urows; ++r) {
          const int pp = r * 64 + lane;
          if (pp < n_unc) {
            const uint32_t e = uk_ld(pp);
            lo2 = min(lo2, e);
            hi2 = max(hi2, e);
          }
        }
        lo2 = wave_min_u(lo2);
        hi2 = wave_max_u(hi2);
        auto ucount_ge = [&](uint32_t t) -> int {
          int cnt = 0;
          for (int r = 0; r < urows; ++r) {
            const int pp = r * 64 + lane;
            cnt += count_lanes(pp < n_unc && uk_ld(pp) >= t);
          }
          return cnt;
        };
        const uint32_t T2 = bisect_kth(lo2, hi2, kr2, ucount_ge);
        const int kr2_eq = kr2 - (T2 == 0xffffffffu ? 0 : ucount_ge(T2 + 1u));
        int eqb = 0;
        for (int r = 0; r < urows; ++r) {
          const int pp = r * 64 + lane;
          const uint32_t e = pp < n_unc ? uk_ld(pp) : 0u;
          const bool eq = pp < n_unc && e == T2;
          const unsigned long long me = __ballot(eq);
          const bool take = (pp < n_unc && e > T2) || (eq && eqb + lanes_below(me) < kr2_eq);
          eqb += __popcll(me);
          if (take) {
            const int j = ul_ld(pp);
            atomicOr(&dmask[j >> 6], 1ull << (j & 63));
          }
        }
      }
    }
  }
  __syncthreads();

  // 5. ordered compaction: the thread's chosen blocks at their places.  Its
  // m <= 64 blocks touch at most two words of the band's mask, read once.
  const int r0 = j0 >> 6, sh = j0 & 63;
  const unsigned long long dm0 = r0 < rows ? dmask[r0] : 0ull;
  const unsigned long long dm1 = r0 + 1 < rows ? dmask[r0 + 1] : 0ull;
  const unsigned long long dmb = sh == 0 ? dm0 : ((dm0 >> sh) | (dm1 << (64 - sh)));
  const int nv = max(0, min(m, n - j0));  // the thread's blocks that exist
  const unsigned long long validm = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
  const unsigned long long chm = (onem | gtm | dmb) & validm;  // bit x: block j0 + x chosen
  const int my_ch = __popcll(chm);
  int tot = 0;
  int o = wg_scan(my_ch, red, slot, tot);
  int32_t *dst = blk_idx + out * k_cap;
  const bool staged = tot <= stage_words;  // the same for every thread
  for (unsigned long long cm = chm; cm != 0ull; cm &= cm - 1ull) {
    const int j = j0 + (int)__builtin_ctzll(cm);
    if (staged) {
      stage[o] = j;
    } else if (o < k_cap) {
      st_dev(&dst[o], j);
      if (tagd && o < c.dm.kcap) st_dev(&tagd[o], ((unsigned long long)epoch << 32) | (uint32_t)j);
    }
    ++o;
  }
  if (staged) {
    __syncthreads();
    for (int p = tid; p < tot; p += 256) {
      const int j = stage[p];
      if (p < k_cap) st_dev(&dst[p], j);
      if (tagd && p < c.dm.kcap) st_dev(&tagd[p], ((unsigned long long)epoch << 32) | (uint32_t)j);
    }
  }
  if (tid == 0) {
    st_dev(&blk_cnt[out], kk);
    st_dev(&c.sc.unit_acc[4 * unit], 0u);  // cleared for the next step
    st_dev(&c.sc.unit_acc[4 * unit + 1], 0u);
    st_dev(&c.sc.unit_acc[4 * unit + 2], eps_bits);  // the bound this selection used
  }
}

// Value of lane ^ J within the wave (J = 1, 2, 4, 8 by DPP inside 16-lane
// rows; 16 and 32 through ds_bpermute).
// The fast top-k's outputs (wave 0): the chosen blocks of the LDS bitmap in
// ascending order, the count, and the unit's accumulators cleared for the
// next step.
__device__ __forceinline__ void fast_out(const Ctx &c, size_t unit, size_t out, int nw, int kk,
                                         int k_cap, int32_t *__restrict__ blk_idx,
                                         int32_t *__restrict__ blk_cnt, TopkSmem &sm,
                                         uint32_t eps_bits) {
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  // ascending order: exclusive prefix of the words' popcounts, then each
  // lane writes the chosen blocks of its word
  unsigned long long wbits = lane < nw ? sm.bm[lane] : 0ull;
  const int cw = __popcll(wbits);
  // inclusive prefix: DPP shifts inside 16-lane rows, then the row totals
  int incl = cw;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31),
            r2 = __builtin_amdgcn_readlane(incl, 47);
  incl += (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
  int o = incl - cw;
  int32_t *dst = blk_idx + out * k_cap;
  while (wbits) {
    const int bb = lane * 64 + (__ffsll((long long)wbits) - 1);
    if (o < k_cap) st_dev(&dst[o], bb);
    ++o;
    wbits &= wbits - 1ull;
  }
  if (lane == 0) {
    st_dev(&blk_cnt[out], kk);
    st_dev(&c.sc.unit_acc[4 * unit], 0u);  // cleared for the next step
    st_dev(&c.sc.unit_acc[4 * unit + 1], 0u);
    st_dev(&c.sc.unit_acc[4 * unit + 2], eps_bits);  // the bound this selection used
  }
}

// Fast top-k of one unit from the score tiles' lists (no MAW flags, kk <=
// kTileList; every thread of the workgroup calls it and gets the same
// result).  The steps of topk_unit run on the listed keys, which hold the
// unit's top kk:
//   1. the lists, each descending, are merged pairwise keeping the 64
//      largest keys (bitonic half-cleaners; DPP and permlane exchanges),
//      which gives the kk-th largest approximate key T;
//   2. band: keys above T + 2 eps are in, below T - 2 eps out (eps: the
//      unit's error bound); the blocks in between are re-scored exactly by
//      the four waves, one lane quad per (block, head);
//   3. the kk - (blocks in) best of them by (exact key desc, index asc);
//   4. in the one-launch step, the tagged selection for the attention parts
//      is written in key order as soon as it is known (the surely selected
//      blocks at once, the band's picks after the re-score), then the count;
//      the caller's list is written in ascending block order, read off an
//      LDS bitmap of the chosen blocks.
// Returns false, before writing anything, when the band reaches past the 64
// largest keys; the caller then runs topk_unit.
template <int D, int G>
__device__ __attribute__((always_inline)) bool topk_fast(const Ctx &c, int seq, size_t unit,
                                                         size_t out, const HeadInfo &hi, const UG &g,
                                                         const uint16_t *__restrict__ q,
                                                         int32_t *__restrict__ blk_idx,
                                                         int32_t *__restrict__ blk_cnt, int k_cap,
                                                         TopkSmem &sm,
                                                         unsigned long long *tagd = nullptr,
                                                         unsigned long long *rtag = nullptr,
                                                         uint32_t epoch = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_tiles = max(1, cdiv(g.n_sc, kScoreTile));
  const unsigned long long etag = (unsigned long long)epoch << 32;
  const unsigned long long *cl = c.sc.cand + unit * c.dm.key_stride;
  const int kk = g.kk;
  const int nw = cdiv(g.n_sc, 64);
  // one batch of loads: lists and counts (wave 0), error bound, the query
  unsigned long long e[kFastTiles];
#pragma unroll
  for (int r = 0; r < kFastTiles; ++r)
    e[r] = (wv == 0 && r < n_tiles) ? ld_dev(&cl[(size_t)r * kTileList + lane]) : 0ull;
  const uint32_t eps_bits = ld_dev(&c.sc.unit_acc[4 * unit]);
  const uint16_t *qg = q + out * G * D;
  constexpr int QT = (G * D + 255) / 256;
  uint16_t qv[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) qv[t] = qg[min(tid + 256 * t, G * D - 1)];
#pragma unroll
  for (int t = 0; t < QT; ++t)
    if (tid + 256 * t < G * D) sm.qs[tid + 256 * t] = __uint_as_float((uint32_t)qv[t] << 16);

  if (wv == 0) {
    bool ok = true;
    int n_in = 0, n_unc = 0;
    if (lane < nw) sm.bm[lane] = 0ull;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    if (ok && kk > 0) {
      const double eps = (double)__uint_as_float(eps_bits);
      // the 64 largest listed keys, descending: pairwise merges of the lists
#pragma unroll
      for (int w = 1; w < kFastTiles; w <<= 1)
#pragma unroll
        for (int r = 0; r + w < kFastTiles; r += 2 * w)
          if (r + w < n_tiles) e[r] = merge_top64(e[r], e[r + w]);
      const unsigned long long m = e[0];
      const uint32_t kx = (uint32_t)(m >> 32);
      const uint32_t T = (uint32_t)__builtin_amdgcn_readlane((int)kx, kk - 1);
      const uint32_t kb_hi = order_key(__double2float_rd((double)key_to_float(T) + 2.0 * eps));
      const uint32_t kb_lo = order_key(__double2float_ru((double)key_to_float(T) - 2.0 * eps));
      // a band reaching below the 64 kept keys could miss blocks
      const uint32_t k63 = (uint32_t)__builtin_amdgcn_readlane((int)kx, 63);
      const bool whole = k63 < 2u || k63 < kb_lo;
      const int blk = (int)~(uint32_t)m;
      const bool in = kx >= 2u && kx > kb_hi;
      const bool unc = kx >= 2u && kx >= kb_lo && kx <= kb_hi;
      if (in) atomicOr(&sm.bm[blk >> 6], 1ull << (blk & 63));
      const unsigned long long mu = __ballot(unc);
      if (unc) sm.ulist[lanes_below(mu)] = blk;
      n_unc = __popcll(mu);
      n_in = count_lanes(in);
      ok = whole;
      ok = ok && n_in <= kk && n_in + n_unc >= kk;
      if (ok && tagd) {
        // the tagged selection goes out in key order: the surely selected
        // blocks at once, with the band when it is taken whole; the count
        // follows the last entry (the band's picks may come after the
        // exact re-score)
        const bool whole_band = n_in + n_unc == kk;
        const unsigned long long mi = __ballot(in);
        const int pos = in ? lanes_below(mi) : n_in + lanes_below(mu);
        if ((in || (whole_band && unc)) && pos < c.dm.kcap) st_dev(&tagd[pos], etag | (uint32_t)blk);
        if (lane == 0 && (whole_band || n_in == kk)) st_dev(rtag, etag | (uint32_t)kk);
      }
    }
    if (lane == 0) {
      sm.ok = ok;
      sm.nin = n_in;
      sm.nlist = n_unc;
    }
  }
  __syncthreads();
  if (!sm.ok) {
    SD_TL(6);  // the fast top-k gave up: the full top-k runs
    return false;
  }
  const int n_unc = sm.nlist, kr2 = kk - sm.nin;
  if (kr2 > 0 && kr2 == n_unc) {  // every band block is taken: no exact keys needed
    if (wv == 0 && lane < n_unc) {
      const int blk = sm.ulist[lane];
      atomicOr(&sm.bm[blk >> 6], 1ull << (blk & 63));
    }
  } else if (kr2 > 0) {
    SD_TL(7);  // the band's exact re-score starts
    // exact keys of the band, one lane quad per (block, head), in passes of 64
    for (int p0 = 0; p0 < n_unc * G; p0 += 64) {
      const int pair = p0 + (tid >> 2);
      const bool on = pair < n_unc * G;
      const int u = on ? pair / G : 0, gg = on ? pair - u * G : 0;
      const double U = exact_score_quad<D>(c, seq, hi, on ? sm.ulist[u] : 0, sm.qs + gg * D, on);
      if (on && (tid & 3) == 0) sm.ue[pair] = U;
    }
    __syncthreads();
    if (wv == 0) {
      unsigned long long ek = 0ull;
      if (lane < n_unc) {
        double best = sm.ue[lane * G];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) best = sm.ue[lane * G + gg] > best ? sm.ue[lane * G + gg] : best;
        ek = ((unsigned long long)order_key((float)best) << 32) | (uint32_t)~(uint32_t)sm.ulist[lane];
      }
      int rank = 0;
      for (int t = 0; t < n_unc; ++t) {
        const unsigned long long o =
            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(ek >> 32), t) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)ek, t);
        rank += o > ek ? 1 : 0;
      }
      if (lane < n_unc && rank < kr2) {
        const int blk = sm.ulist[lane];
        atomicOr(&sm.bm[blk >> 6], 1ull << (blk & 63));
        if (tagd && sm.nin + rank < c.dm.kcap) st_dev(&tagd[sm.nin + rank], etag | (uint32_t)blk);
      }
      if (tagd && lane == 0) st_dev(rtag, etag | (uint32_t)kk);
    }
  }
  if (wv == 0) fast_out(c, unit, out, nw, kk, k_cap, blk_idx, blk_cnt, sm, eps_bits);
  return true;
}

// Fast top-k for kTileList < k <= kFastK: the steps of topk_fast on the
// tiles' 128-key lists (ranks l and 64 + l in lane l's two registers), merged
// pairwise keeping the 128 largest; the band must end above the 128th merged
// key, else (false, before writing anything) the caller runs topk_unit.
template <int D, int G>
__device__ __attribute__((always_inline)) bool topk_fast128(const Ctx &c, int seq, size_t unit,
                                                            size_t out, const HeadInfo &hi, const UG &g,
                                                            const uint16_t *__restrict__ q,
                                                            int32_t *__restrict__ blk_idx,
                                                            int32_t *__restrict__ blk_cnt, int k_cap,
                                                            TopkSmem &sm,
                                                            unsigned long long *tagd = nullptr,
                                                            unsigned long long *rtag = nullptr,
                                                            uint32_t epoch = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_tiles = max(1, cdiv(g.n_sc, kScoreTile));
  const unsigned long long etag = (unsigned long long)epoch << 32;
  const unsigned long long *cl = c.sc.cand + unit * c.dm.key_stride;
  const int kk = g.kk;  // kTileList < kk <= kFastK
  const int nw = cdiv(g.n_sc, 64);
  // one batch of loads: lists (wave 0), error bound, the query
  unsigned long long eh[kFastTiles], el[kFastTiles];
#pragma unroll
  for (int r = 0; r < kFastTiles; ++r) {
    const bool on = wv == 0 && r < n_tiles;
    eh[r] = on ? ld_dev(&cl[(size_t)r * kFastK + lane]) : 0ull;
    el[r] = on ? ld_dev(&cl[(size_t)r * kFastK + kTileList + lane]) : 0ull;
  }
  const uint32_t eps_bits = ld_dev(&c.sc.unit_acc[4 * unit]);
  const uint16_t *qg = q + out * G * D;
  constexpr int QT = (G * D + 255) / 256;
  uint16_t qv[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) qv[t] = qg[min(tid + 256 * t, G * D - 1)];
#pragma unroll
  for (int t = 0; t < QT; ++t)
    if (tid + 256 * t < G * D) sm.qs[tid + 256 * t] = __uint_as_float((uint32_t)qv[t] << 16);

  if (wv == 0) {
    if (lane < nw) sm.bm[lane] = 0ull;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const double eps = (double)__uint_as_float(eps_bits);
#pragma unroll
    for (int w = 1; w < kFastTiles; w <<= 1)
#pragma unroll
      for (int r = 0; r + w < kFastTiles; r += 2 * w)
        if (r + w < n_tiles) merge_top128(eh[r], el[r], eh[r + w], el[r + w]);
    const uint32_t kh = (uint32_t)(eh[0] >> 32), kl = (uint32_t)(el[0] >> 32);
    const uint32_t T = (uint32_t)__builtin_amdgcn_readlane((int)kl, kk - 1 - kTileList);
    const uint32_t kb_hi = order_key(__double2float_rd((double)key_to_float(T) + 2.0 * eps));
    const uint32_t kb_lo = order_key(__double2float_ru((double)key_to_float(T) - 2.0 * eps));
    // a band reaching below the 128 kept keys could miss blocks
    const uint32_t k127 = (uint32_t)__builtin_amdgcn_readlane((int)kl, kTileList - 1);
    const bool whole = k127 < 2u || k127 < kb_lo;
    const int bh = (int)~(uint32_t)eh[0], bl = (int)~(uint32_t)el[0];
    const bool inh = kh >= 2u && kh > kb_hi, inl = kl >= 2u && kl > kb_hi;
    const bool unh = kh >= 2u && kh >= kb_lo && kh <= kb_hi;
    const bool unl = kl >= 2u && kl >= kb_lo && kl <= kb_hi;
    if (inh) atomicOr(&sm.bm[bh >> 6], 1ull << (bh & 63));
    if (inl) atomicOr(&sm.bm[bl >> 6], 1ull << (bl & 63));
    // the band in key order (every key of h is above every key of lo)
    const unsigned long long muh = __ballot(unh), mul = __ballot(unl);
    const int nuh = __popcll(muh);
    if (unh) sm.ulist[lanes_below(muh)] = bh;
    if (unl) sm.ulist[nuh + lanes_below(mul)] = bl;
    const int n_unc = nuh + __popcll(mul);
    const unsigned long long mih = __ballot(inh), mil = __ballot(inl);
    const int nih = __popcll(mih), n_in = nih + __popcll(mil);
    const bool ok = whole && n_in <= kk && n_in + n_unc >= kk;
    if (ok && tagd) {
      // the tagged selection in key order, as in topk_fast
      const bool whole_band = n_in + n_unc == kk;
      const int ph = inh ? lanes_below(mih) : n_in + lanes_below(muh);
      const int pl = inl ? nih + lanes_below(mil) : n_in + nuh + lanes_below(mul);
      if ((inh || (whole_band && unh)) && ph < c.dm.kcap) st_dev(&tagd[ph], etag | (uint32_t)bh);
      if ((inl || (whole_band && unl)) && pl < c.dm.kcap) st_dev(&tagd[pl], etag | (uint32_t)bl);
      if (lane == 0 && (whole_band || n_in == kk)) st_dev(rtag, etag | (uint32_t)kk);
    }
    if (lane == 0) {
      sm.ok = ok;
      sm.nin = n_in;
      sm.nlist = n_unc;
    }
  }
  __syncthreads();
  if (!sm.ok) {
    SD_TL(6);  // the fast top-k gave up: the full top-k runs
    return false;
  }
  const int n_unc = sm.nlist, kr2 = kk - sm.nin;
  if (kr2 > 0 && kr2 == n_unc) {  // every band block is taken: no exact keys needed
    if (wv == 0)
      for (int u = lane; u < n_unc; u += 64) {
        const int blk = sm.ulist[u];
        atomicOr(&sm.bm[blk >> 6], 1ull << (blk & 63));
      }
  } else if (kr2 > 0) {
    SD_TL(7);  // the band's exact re-score starts
    // exact keys of the band, one lane quad per (block, head), in passes of 64
    for (int p0 = 0; p0 < n_unc * G; p0 += 64) {
      const int pair = p0 + (tid >> 2);
      const bool on = pair < n_unc * G;
      const int u = on ? pair / G : 0, gg = on ? pair - u * G : 0;
      const double U = exact_score_quad<D>(c, seq, hi, on ? sm.ulist[u] : 0, sm.qs + gg * D, on);
      if (on && (tid & 3) == 0) sm.ue[pair] = U;
    }
    __syncthreads();
    if (wv == 0) {
      // exact keys of the listed blocks, two per lane (u = lane, 64 + lane),
      // ranked by (exact key desc, index asc)
      unsigned long long ek[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int u = lane + kTileList * x;
        ek[x] = 0ull;
        if (u < n_unc) {
          double best = sm.ue[u * G];
#pragma unroll
          for (int gg = 1; gg < G; ++gg) best = sm.ue[u * G + gg] > best ? sm.ue[u * G + gg] : best;
          ek[x] = ((unsigned long long)order_key((float)best) << 32) | (uint32_t)~(uint32_t)sm.ulist[u];
        }
      }
      int rank[2] = {0, 0};
      for (int t = 0; t < n_unc; ++t) {
        const unsigned long long src = t < kTileList ? ek[0] : ek[1];
        const int tl = t & (kTileList - 1);
        const unsigned long long o =
            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(src >> 32), tl) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)src, tl);
        rank[0] += o > ek[0] ? 1 : 0;
        rank[1] += o > ek[1] ? 1 : 0;
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int u = lane + kTileList * x;
        if (u < n_unc && rank[x] < kr2) {
          const int blk = sm.ulist[u];
          atomicOr(&sm.bm[blk >> 6], 1ull << (blk & 63));
          if (tagd && sm.nin + rank[x] < c.dm.kcap)
            st_dev(&tagd[sm.nin + rank[x]], etag | (uint32_t)blk);
        }
      }
      if (tagd && lane == 0) st_dev(rtag, etag | (uint32_t)kk);
    }
  }
  if (wv == 0) fast_out(c, unit, out, nw, kk, k_cap, blk_idx, blk_cnt, sm, eps_bits);
  return true;
}

// ---------------------------------------------------------------------------

__device__ __forceinline__ unsigned long long bit_range(int a, int b) {
  if (b <= a) return 0ull;
  const unsigned long long hi = b >= 64 ? ~0ull : ((1ull << b) - 1ull);
  const unsigned long long lo = (1ull << a) - 1ull;  // a < b <= 64
  return hi & ~lo;
}

// ---------------------------------------------------------------------------
// Page lists of the attention.  The attended set of a unit is T = D U the
// selected blocks ([HGCA] What carries the argument: dense recent window plus
// selected entries; union, so no token is counted twice), cut into 16-token
// pages: first the pages holding dense tokens (sink pages [0, sp), then window
// pages [wp, np)), each with its dense-token mask, then the pages of the
// selected blocks in selection order, each with the mask of its tokens that
// are not dense.  Position t of the unit's list is also the slot of the
// page's log softmax mass (selected pages from lm_sel0 on).
struct DenseList {
  int sp, wp, np, n;
};
__device__ __forceinline__ DenseList dense_list(const UG &g) {
  DenseList d;
  d.np = cdiv(g.N, kPage);
  d.sp = cdiv(g.ns, kPage);
  d.wp = g.wlo < g.N ? max(d.sp, g.wlo / kPage) : d.np;
  d.n = d.sp + (d.np - d.wp);
  return d;
}
// Attention parts a unit uses out of a launch's P: one per about kPartPages
// of its attended pages (dense pages, then k blocks' pages), at least one.
// Both call forms take the same number, so they give the same bits; a unit
// with fewer pages than the launch's longest does not hold workgroups that
// have nothing to do.
// Blocks the attention visits at most: k, or with one set per query head
// the union of the G sets, min(candidates, G k).
__device__ __forceinline__ int union_blocks(const UG &g, const Dims &dm) {
  if (!dm.pqh) return g.kk;
  const int n_cand = g.ns < g.wlo ? div_S(g.wlo + g.S - 1, g.S) - div_S(g.ns, g.S) : 0;
  return min(n_cand, dm.G * g.kk);
}
__device__ __forceinline__ int unit_parts(const UG &g, int P, const Dims &dm) {
  const int pages = dense_list(g).n + union_blocks(g, dm) * (g.S / kPage);
  return min(P, max(1, cdiv(pages, kPartPages)));
}
__device__ __forceinline__ int dense_page(const DenseList &d, int e) {
  return e < d.sp ? e : d.wp + (e - d.sp);
}
// position of page pn in the dense list, or -1
__device__ __forceinline__ int dense_pos(const DenseList &d, int pn) {
  return pn < d.sp ? pn : ((pn >= d.wp && pn < d.np) ? d.sp + (pn - d.wp) : -1);
}
__device__ __forceinline__ int page_valid16(const UG &g, int pn) {
  return (int)bit_range(0, min(max(g.N - pn * kPage, 0), kPage));
}
__device__ __forceinline__ int page_dense16(const UG &g, int pn) {
  const int b = pn * kPage;
  const int lo = min(max(g.wlo - b, 0), kPage), hi = min(max(g.N - b, 0), kPage);
  return (int)(bit_range(0, min(max(g.ns - b, 0), kPage)) | bit_range(lo, hi));
}

// ---------------------------------------------------------------------------
// Attention of one (unit, part): softmax attention of the G query heads of a
// KV head over its share of the unit's pages ([HGCA] What carries the
// argument: each partial carries its own normalisation statistics; split-K
// decoding).  Wave w of part p takes list positions 4p + w + i * 4P.  Pages
// stream through two register stages of two pages each: the loads of the
// next stage are in flight while the current one computes.  Per stage:
//   q.K: one v_mfma_f32_16x16x32_bf16 tile per page and 32 channels (rows =
//        heads padded to 16, columns = the page's 16 tokens);
//   softmax: online (running max and sum per head, O rescaled), DPP row
//        reductions;
//   p.V: the weights go through LDS into the MFMA A layout (row = head, 8
//        tokens per lane), split into bf16 hi + lo parts; V pages are stored
//        transposed ([channel][16 tokens]), so a lane's 8 tokens of one
//        channel are one 16-byte load in the MFMA B layout; two MFMAs per
//        16 output channels accumulate O in fp32.
// The four waves merge their (max, sum, O) once at the end.
// The step's new token of one unit when its append runs inside the step
// launch (the block holding it lies wholly in the recent window, so no score
// depends on it): the attention takes its K and V from the caller's rows, and
// the unit's fusion, which runs after every part, writes it into its page and
// folds it into the block summary.  pg < 0: no such token.
struct NewTok {
  int pg = -1, slot = 0;                      // physical page, place in the page
  const uint16_t *k = nullptr, *v = nullptr;  // rows [D] of this (sequence, KV head)
};

template <int D, int G>
struct AttLds {
  float p[4][16][32];  // per wave: the stage's weights, [head row][token]
  float wo[4][G][D];   // per wave: unnormalised O at the end
  float wm[4][G];      // per wave: running max (log2 units)
  float wz[4][G];      // per wave: running sum
};

template <int D>
struct KVStage {
  uint4 k[2][D / 32];  // K of the two pages: lane = token r16, channels lgrp*D/4 + 8m
  uint4 v[D / 16];     // V: lane = channel 16 nt + r16, tokens 8 lgrp .. 8 lgrp + 7
};

template <int D>
struct AttWave {
  float m[4], z[4];  // heads 4 lgrp + j: running max (log2 units), sum
  f32x4 o[D / 16];   // unnormalised O: rows 4 lgrp + j, channel 16 nt + r16
};

template <int D>
__device__ __forceinline__ void load_stage(const Ctx &c, int h, int pg0, int pg1,
                                           KVStage<D> &st, const NewTok &tok) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, lgrp = lane >> 4;
#pragma unroll
  for (int pi = 0; pi < 2; ++pi) {
    const int pg = pi ? pg1 : pg0;
    // the lane of the step's new token reads its K from the caller's row
    // MFMA m, lane (token r16, lgrp): channel group 4 m + lgrp, so that one
    // load instruction reads 1 KB of the page's K contiguously; the lane of
    // the step's new token reads its K from the caller's row
    const bool nt = pg == tok.pg && r16 == tok.slot;
    const uint16_t *kb = nt ? tok.k : c.L.k + ((size_t)pg * c.dm.Hkv + h) * kPage * D + r16 * 8;
    const int gstride = nt ? 8 : kPage * 8;  // elements from one channel group to the next
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
      st.k[pi][m] = *reinterpret_cast<const uint4 *>(kb + (size_t)(4 * m + lgrp) * gstride);
  }
  const uint16_t *vp = c.L.v + (((size_t)(lgrp >= 2 ? pg1 : pg0) * c.dm.Hkv + h) * D + r16) * kPage +
                       8 * (lgrp & 1);
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt)
    st.v[nt] = *reinterpret_cast<const uint4 *>(vp + (size_t)nt * 16 * kPage);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// One stage of a wave: pages with token masks mk0, mk1 (uniform; bits 0-15
// the page's tokens, bit 16 + h set when query head h attends none of them,
// which only a per-query-head selection does), log-mass slots s0, s1 (-1:
// none).  lmb: log-mass rows of the unit's heads.  Rows of
// padding heads (past G) carry finite values that are never stored.
template <int D, int G>
__device__ __forceinline__ void compute_stage(const Ctx &c, KVStage<D> &st, int mk0, int mk1,
                                              int s0, int s1, const uint4 (&qa)[D / 32],
                                              const uint4 &ones, AttWave<D> &W, float (*pl)[32],
                                              float *lmb, int newp, const NewTok &tok) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, lgrp = lane >> 4;
  constexpr int NT = D / 16;
  constexpr float kLn2 = 0.69314718055994530942f;
  float sc[2][4];
#pragma unroll
  for (int pi = 0; pi < 2; ++pi) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[m]),
                                                    __builtin_bit_cast(bf16x8, st.k[pi][m]),
                                                    acc, 0, 0, 0);
    const int mk = pi ? mk1 : mk0;
    const bool on = ((mk >> r16) & 1) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc[pi][j] = (on && !((mk >> (16 + 4 * lgrp + j)) & 1)) ? acc[j] * c.dm.scale_log2 : -INFINITY;
  }
  float al[4], mnv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mn = fmaxf(W.m[j], row_max16(fmaxf(sc[0][j], sc[1][j])));
    const bool none = mn == -INFINITY;
    // exp2 of a non-positive argument (or -inf): the hardware v_exp_f32
    al[j] = none ? 1.0f : __builtin_amdgcn_exp2f(W.m[j] - mn);
    pl[4 * lgrp + j][r16] = none ? 0.0f : __builtin_amdgcn_exp2f(sc[0][j] - mn);
    pl[4 * lgrp + j][16 + r16] = none ? 0.0f : __builtin_amdgcn_exp2f(sc[1][j] - mn);
    W.m[j] = mn;
    mnv[j] = mn;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) W.o[nt][j] *= al[j];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  // A operands: lane (head r16, tokens 8 lgrp .. 8 lgrp + 7); hi = weight
  // truncated to bf16, lo = the exact remainder rounded to bf16
  uint4 ahi, alo;
  {
    const float4 x0 = *reinterpret_cast<const float4 *>(&pl[r16][8 * lgrp]);
    const float4 x1 = *reinterpret_cast<const float4 *>(&pl[r16][8 * lgrp + 4]);
    const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t b0 = __float_as_uint(f[2 * t]) & 0xffff0000u;
      const uint32_t b1 = __float_as_uint(f[2 * t + 1]) & 0xffff0000u;
      hw[t] = (b0 >> 16) | b1;
      lw[t] = bf16_rne_bits(f[2 * t] - __uint_as_float(b0)) |
              (bf16_rne_bits(f[2 * t + 1] - __uint_as_float(b1)) << 16);
    }
    ahi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    alo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  // page newp (0 or 1, uniform) of the stage holds the step's new token: the
  // lanes whose 8 tokens include it take its V from the caller's row (one
  // stage per unit)
  if (newp >= 0 && (lgrp >= 2 ? 1 : 0) == newp && (lgrp & 1) == (tok.slot >> 3)) {
    const int e = tok.slot & 7, sh = 16 * (e & 1);
    const uint32_t keep = ~(0xffffu << sh);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t x = (uint32_t)tok.v[16 * nt + r16] << sh;
      uint4 &vv = st.v[nt];
      vv.x = (e >> 1) == 0 ? (vv.x & keep) | x : vv.x;
      vv.y = (e >> 1) == 1 ? (vv.y & keep) | x : vv.y;
      vv.z = (e >> 1) == 2 ? (vv.z & keep) | x : vv.z;
      vv.w = (e >> 1) == 3 ? (vv.w & keep) | x : vv.w;
    }
  }
  // masked tokens have zero weight; their V is zeroed too, so that stale or
  // unwritten slots cannot turn the products into NaN
  if ((mk0 & mk1) != 0xffff) {
    const int m8 = ((lgrp >= 2 ? mk1 : mk0) >> (8 * (lgrp & 1))) & 0xff;
    uint32_t wm[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      wm[t] = (((m8 >> (2 * t)) & 1) ? 0x0000ffffu : 0u) | (((m8 >> (2 * t + 1)) & 1) ? 0xffff0000u : 0u);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      st.v[nt].x &= wm[0];
      st.v[nt].y &= wm[1];
      st.v[nt].z &= wm[2];
      st.v[nt].w &= wm[3];
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    W.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ahi),
                                                      __builtin_bit_cast(bf16x8, st.v[nt]),
                                                      W.o[nt], 0, 0, 0);
    W.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo),
                                                      __builtin_bit_cast(bf16x8, st.v[nt]),
                                                      W.o[nt], 0, 0, 0);
  }
  // sums of the same bf16 weights by MFMA against constant columns: column 0
  // both pages, column 1 page 0, column 2 page 1
  f32x4 zs = {0.f, 0.f, 0.f, 0.f};
  zs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ahi),
                                               __builtin_bit_cast(bf16x8, ones), zs, 0, 0, 0);
  zs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo),
                                               __builtin_bit_cast(bf16x8, ones), zs, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    W.z[j] = fmaf(W.z[j], al[j], zs[j]);  // meaningful in lanes r16 == 0
    const int hd = 4 * lgrp + j, sl = r16 == 1 ? s0 : s1;
    if ((r16 == 1 || r16 == 2) && hd < G && sl >= 0) {
      const float zp = zs[j];
      st_dev(&lmb[(size_t)hd * c.dm.lm_cap + sl],
             zp > 0.0f ? (mnv[j] + __builtin_amdgcn_logf(zp)) * kLn2 : -INFINITY);
    }
  }
}

// One wave over its positions of a page list of `total` entries: positions
// gw + i NW.  resolve(t, pg, mk, sl) gives the page id, token mask and
// log-mass slot of list position t; up to 64 positions are resolved at once,
// one per lane.
template <int D, int G, class Resolve>
__device__ __forceinline__ void wave_pages(const Ctx &c, int h, int gw, int NW, int total,
                                           Resolve resolve, const uint4 (&qa)[D / 32], AttWave<D> &W,
                                           float (*pl)[32], float *lmb, const NewTok &tok,
                                           int tl_slot = -1) {
  const int lane = threadIdx.x & 63;
  const int nw = total > gw ? cdiv(total - gw, NW) : 0;
  for (int b0 = 0; b0 < nw; b0 += 64) {
    const int n = min(64, nw - b0);
    int pg = 0, mk = 0, sl = -1;
    if (lane < n) resolve(gw + (b0 + lane) * NW, pg, mk, sl);
    auto PG = [&](int t) { return __builtin_amdgcn_readlane(pg, min(t, n - 1)); };
    auto MK = [&](int t) { return t < n ? __builtin_amdgcn_readlane(mk, t) : 0; };
    auto SL = [&](int t) { return t < n ? __builtin_amdgcn_readlane(sl, t) : -1; };
    const int ns = cdiv(n, 2);
    // constant B columns of the weight sums: lane (column r16, tokens 8 lgrp ..)
    const int r16 = lane & 15, lgrp = lane >> 4;
    const uint32_t one2 = (r16 == 0 || (r16 == 1 && lgrp < 2) || (r16 == 2 && lgrp >= 2))
                              ? 0x3f803f80u : 0u;
    const uint4 ones = make_uint4(one2, one2, one2, one2);
    // which page of stage t (pages 2t, 2t + 1) holds the step's new token
    auto NP = [&](int t) { return PG(2 * t) == tok.pg ? 0 : (PG(2 * t + 1) == tok.pg ? 1 : -1); };
    KVStage<D> A, B;
    load_stage<D>(c, h, PG(0), PG(1), A, tok);
    if (tl_slot >= 0 && b0 == 0) SD_TL(tl_slot);  // (measurement build) page ids read
    for (int s = 0;; s += 2) {
      load_stage<D>(c, h, PG(2 * s + 2), PG(2 * s + 3), B, tok);
      compute_stage<D, G>(c, A, MK(2 * s), MK(2 * s + 1), SL(2 * s), SL(2 * s + 1), qa, ones, W,
                          pl, lmb, NP(s), tok);
      if (s + 1 >= ns) break;
      load_stage<D>(c, h, PG(2 * s + 4), PG(2 * s + 5), A, tok);
      compute_stage<D, G>(c, B, MK(2 * s + 2), MK(2 * s + 3), SL(2 * s + 2), SL(2 * s + 3), qa,
                          ones, W, pl, lmb, NP(s + 1), tok);
      if (s + 2 >= ns) break;
    }
  }
}

// Where a part finds the unit's selection.
struct SelIn {
  const int32_t *blk = nullptr;              // separate call: the caller's list
  int cnt = 0;                               //   and its count
  const unsigned long long *tag = nullptr;   // one-launch step: tagged entries
  const unsigned long long *rtag = nullptr;  //   and the tagged count
  uint32_t epoch = 0;
};

template <int D, int G>
__device__ __attribute__((always_inline)) void attend_part(const Ctx &c, int i, int seq, int h,
                                                           const UG &g, int part, int P,
                                                           const uint16_t *__restrict__ q,
                                                           const SelIn &si,
                                                           float *__restrict__ o_part,
                                                           float *__restrict__ lse_part, int p_cap,
                                                           AttLds<D, G> &sm,
                                                           int32_t *ptl /* LDS or null */,
                                                           int *s_cnt, const NewTok &tok,
                                                           const HeadInfo &hi,
                                                           uint32_t *dctr = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r16 = lane & 15, lgrp = lane >> 4;
  constexpr int NT = D / 16;
  const int qh0 = h * G, NW = 4 * P, gw = 4 * part + wv;
  const int PPB = g.S / kPage;
  const int32_t *pts = c.L.pt + (size_t)seq * c.dm.pages_per_seq;
  uint4 qa[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
    qa[m] = r16 < G ? *reinterpret_cast<const uint4 *>(q + ((size_t)i * c.dm.Hq + qh0 + r16) * D +
                                                       8 * (4 * m + lgrp))
                    : make_uint4(0, 0, 0, 0);
  AttWave<D> W;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    W.m[j] = -INFINITY;
    W.z[j] = 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) W.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float(*pl)[32] = sm.p[wv];
  float *lmb = c.sc.lm_pg + ((size_t)seq * c.dm.Hq + qh0) * c.dm.lm_cap;

  if (ptl) {
    // the page table to LDS (one batch of loads); the selected pages read it
    // after the barriers below
    constexpr int PER = (kPtLds + 255) / 256;
    const int np = cdiv(g.N, kPage);
    int32_t v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int x = tid + 256 * k;
      v[k] = x < np ? pts[x] : 0;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int x = tid + 256 * k;
      if (x < np) ptl[x] = v[k];
    }
  }
  // dense pages
  const DenseList dl = dense_list(g);
  wave_pages<D, G>(
      c, h, gw, NW, dl.n,
      [&](int t, int &pg, int &mk, int &sl) {
        const int pn = dense_page(dl, t);
        pg = pts[pn];
        mk = page_dense16(g, pn);
        sl = t;
      },
      qa, W, pl, lmb, tok, 6);

  SD_TL(1);  // dense pages done (wave 0)
  // the selection.  Each lane's first selected page's entry is read while
  // the count is awaited; when its tag is this step's the page resolves
  // without a second round trip
  const int t_pre = gw + lane * NW;
  const unsigned long long e_pre =
      si.tag ? ld_dev(&si.tag[min(div_m(t_pre, PPB), c.dm.kcap - 1)]) : 0ull;
  int cnt = si.cnt;
  if (si.rtag) {
    if (tid == 0) {
      int n = -1;
      const unsigned long long t0 = wall_clock64();
      for (;;) {
        const unsigned long long rt = ld_dev(si.rtag);
        if ((uint32_t)(rt >> 32) == si.epoch) {
          n = (int)(uint32_t)rt;
          break;
        }
        if (wall_clock64() - t0 > kWaitTicks) {
          st_dev(&c.sc.err[0], 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      *s_cnt = n;
    }
    __syncthreads();
    cnt = *s_cnt;
  }
  SD_TL(2);  // selection count seen
  // one-launch step: every part, and the unit's top-k, arrive once the dense
  // pages' log-masses are written (by now their stores are long done); the
  // unit's MAW worker then updates MAW, off the parts' path
  if (dctr) arrive(dctr);
  if (cnt > 0 && g.N > 0) {
    wave_pages<D, G>(
        c, h, gw, NW, cnt * PPB,
        [&](int t, int &pg, int &mk, int &sl) {
          const int j = div_m(t, PPB), pp = t - j * PPB;
          int blk, hx = 0;
          if (si.tag) {  // published before the count; the tag confirms it
            unsigned long long e = t == t_pre && (uint32_t)(e_pre >> 32) == si.epoch
                                       ? e_pre : ld_dev(&si.tag[j]);
            const unsigned long long t0 = wall_clock64();
            while ((uint32_t)(e >> 32) != si.epoch && wall_clock64() - t0 < kWaitTicks)
              e = ld_dev(&si.tag[j]);
            if ((uint32_t)(e >> 32) == si.epoch) {
              blk = (int)(uint32_t)e;
            } else {  // gave up: the step's outputs are invalid
              blk = -1;
              st_dev(&c.sc.err[0], 1u);
            }
          } else if (c.dm.pqh) {  // the group's union: block | head mask << 24
            const int e = si.blk[j];
            blk = e & 0xffffff;
            hx = ~(e >> 24) & 0xff;  // query heads that did not select it
          } else {
            blk = si.blk[j];
          }
          // an entry outside [0, n_blk) attends nothing (its pages' masks are
          // empty; the page read is a valid one of the sequence)
          const bool in_range = blk >= 0 && blk < g.n_blk;
          const int pn = in_range ? blk * PPB + pp : 0;
          const int pl_ = min(pn, dl.np - 1);  // pages past N are never read
          pg = ptl ? ptl[pl_] : pts[pl_];
          mk = in_range ? (page_valid16(g, pn) & ~page_dense16(g, pn)) | (hx << 16) : 0;
          // (the learn-from-the-past tables take every attended page's
          // mass; MAW only the dense pages')
          sl = c.dm.lfps ? c.dm.lm_sel0 + t : -1;
        },
        qa, W, pl, lmb, tok);
  }

  SD_TL(3);  // selected pages done (wave 0)
  // merge the four waves into the part's partial
  if (r16 == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hd = 4 * lgrp + j;
      if (hd < G) {
        sm.wm[wv][hd] = W.m[j];
        sm.wz[wv][hd] = W.z[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hd = 4 * lgrp + j;
    if (hd < G) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sm.wo[wv][hd][16 * nt + r16] = W.o[nt][j];
    }
  }
  __syncthreads();
  constexpr float kLn2 = 0.69314718055994530942f;
  const size_t ohead = ((size_t)i * c.dm.Hq + qh0) * p_cap + part;
  for (int x = tid; x < G * D; x += 256) {
    const int gg = x / D, ch = x - gg * D;
    const float M = fmaxf(fmaxf(sm.wm[0][gg], sm.wm[1][gg]), fmaxf(sm.wm[2][gg], sm.wm[3][gg]));
    float Z = 0.0f, v = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(sm.wm[w][gg] - M);
        Z = fmaf(f, sm.wz[w][gg], Z);
        v = fmaf(f, sm.wo[w][gg][ch], v);
      }
    st_dev(&o_part[(ohead + (size_t)gg * p_cap) * D + ch], Z > 0.0f ? v / Z : 0.0f);
    if (ch == 0)
      st_dev(&lse_part[ohead + (size_t)gg * p_cap], Z > 0.0f ? (M + log2f(Z)) * kLn2 : -INFINITY);
  }
}

// Slots [P, p_cap) of a unit's partials are unused: lse = -inf, O = 0.
template <int D, int G>
__device__ __forceinline__ void empty_slots(const Ctx &c, int i, int h, int P, int p_cap,
                                            float *__restrict__ o_part,
                                            float *__restrict__ lse_part) {
  const size_t hb = ((size_t)i * c.dm.Hq + (size_t)h * G) * p_cap;
  const int n = p_cap - P;
  for (int x = threadIdx.x; x < G * n * D; x += 256) {
    const int gg = x / (n * D), r = x - gg * n * D, u = r / D, ch = r - u * D;
    st_dev(&o_part[(hb + (size_t)gg * p_cap + P + u) * D + ch], 0.0f);
  }
  for (int x = threadIdx.x; x < G * n; x += 256)
    st_dev(&lse_part[hb + (size_t)(x / n) * p_cap + P + x % n], -INFINITY);
}

// ---------------------------------------------------------------------------
// fusion ([HGCA] What carries the argument: the exact log-sum-exp merge of
// partials, with the maximum subtracted as the referee's minor comment on
// section 3.3 asks): for each query head, lse = m + log sum_u exp(lse_u - m)
// with m the largest partial lse (empty slots, lse = -inf, drop out), and
// O = sum_u exp(lse_u - lse) O_u.
// e^x and ln x from the hardware base-2 exponential and logarithm (about one
// ulp each; the fp32 rounding of x log2(e) adds |x| 2^-24 relative, under
// 1e-5 for the partial weights here)
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}
__device__ __forceinline__ float fast_log(float x) {
  return __builtin_amdgcn_logf(x) * 0.69314718055994531f;
}
constexpr int kFusePre = 8;  // partial slots whose O values are preloaded

template <int D, int G>
__device__ __attribute__((always_inline)) void fuse_unit(const Ctx &c, int i, int h, int n_slots,
                                                         const float *__restrict__ o_part,
                                                         const float *__restrict__ lse_part,
                                                         int p_cap, float *__restrict__ o,
                                                         float *__restrict__ lse, FuseSmem<G> &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qh0 = h * G;
  n_slots = min(n_slots, kFuseSlots);  // (the host keeps every call within it)
  // ---- one batch of loads ---------------------------------------------------
  constexpr int R = kFuseSlots / 64;
  float l0[R], l1[R];  // lse of heads wv and wv + 4
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int u = lane + 64 * r;
    const bool on = u < n_slots;
    l0[r] = (on && wv < G) ? ld_dev(&lse_part[((size_t)i * c.dm.Hq + qh0 + wv) * p_cap + u])
                           : -INFINITY;
    l1[r] = (on && wv + 4 < G) ? ld_dev(&lse_part[((size_t)i * c.dm.Hq + qh0 + wv + 4) * p_cap + u])
                               : -INFINITY;
  }
  // O: thread tid < G D / 4 sums 4 channels of one head, each slot's read as
  // two 8-byte loads (the partials are 16-byte aligned)
  constexpr int NO = G * D / 4;
  static_assert(NO <= 256, "one thread per 4 output channels");
  const bool o_on = tid < NO;
  const int ogg = (4 * min(tid, NO - 1)) / D, och = 4 * min(tid, NO - 1) - ogg * D;
  const unsigned long long *op2 = reinterpret_cast<const unsigned long long *>(
      o_part + ((size_t)i * c.dm.Hq + qh0 + ogg) * p_cap * D + och);
  auto ld_o = [&](int u, bool on) -> float4 {
    if (!on) return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const unsigned long long a = ld_dev(op2 + (size_t)u * (D / 2)), b = ld_dev(op2 + (size_t)u * (D / 2) + 1);
    return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                       __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
  };
  float4 ov[kFusePre];
#pragma unroll
  for (int u = 0; u < kFusePre; ++u) ov[u] = ld_o(u, o_on && u < n_slots);

  // ---- per-head lse and slot weights ----------------------------------------
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int gg = wv + 4 * pass;
    if (gg >= G) continue;
    float l[R];
#pragma unroll
    for (int r = 0; r < R; ++r) l[r] = pass ? l1[r] : l0[r];
    float m = l[0];
#pragma unroll
    for (int r = 1; r < R; ++r) m = fmaxf(m, l[r]);
    m = wave_max(m);
    float z = 0.0f;
    if (m != -INFINITY)
#pragma unroll
      for (int r = 0; r < R; ++r) z += l[r] == -INFINITY ? 0.0f : fast_exp(l[r] - m);
    z = wave_sum(z);
    const float L = m == -INFINITY ? -INFINITY : m + fast_log(z);
    if (lane == 0) sm.lse[gg] = L;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = lane + 64 * r;
      sm.w[gg][u] = (L == -INFINITY || l[r] == -INFINITY) ? 0.0f : fast_exp(l[r] - L);
    }
  }
  __syncthreads();
  // ---- O = sum_u w_u O_u (zero weights select 0), each channel in slot order
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto add_slot = [&](int u, const float4 &v) {
    const float wgt = sm.w[ogg][u];
    const bool z = wgt == 0.0f;
    acc.x = fmaf(wgt, z ? 0.0f : v.x, acc.x);
    acc.y = fmaf(wgt, z ? 0.0f : v.y, acc.y);
    acc.z = fmaf(wgt, z ? 0.0f : v.z, acc.z);
    acc.w = fmaf(wgt, z ? 0.0f : v.w, acc.w);
  };
#pragma unroll
  for (int u = 0; u < kFusePre; ++u)
    if (u < n_slots) add_slot(u, ov[u]);
  for (int u0 = kFusePre; u0 < n_slots; u0 += 8) {  // the rest, 8 slots in flight
    float4 v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = ld_o(u0 + t, o_on && u0 + t < n_slots);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (u0 + t < n_slots) add_slot(u0 + t, v[t]);
  }
  if (o_on) {
    float *od = o + ((size_t)i * c.dm.Hq + qh0 + ogg) * D + och;
    od[0] = acc.x;
    od[1] = acc.y;
    od[2] = acc.z;
    od[3] = acc.w;
  }
  if (tid < G) lse[(size_t)i * c.dm.Hq + qh0 + tid] = sm.lse[tid];
}

// MAW update of one unit ([HGCA] What carries the argument: MAW, a moving
// average of attention weights, against beta over the GPU-side entries;
// referee report on section 3.2.2 / Algorithm 1: the average is fed by the
// GPU-side window's attention weights alone and an entry's average is frozen
// once it has left the window, blocks leaving whole; [LFPS] decay r = 0.95):
// per head, lse_D = log sum of exp(log-mass) over the dense pages (the dense
// partial's own normaliser); each block whose tokens all lie in D - a block
// that is not a candidate - takes MAW <- r MAW + (1 - r) a, a = (1/G)
// sum_h sum of exp(log-mass - lse_D) over the block's pages; every other
// block keeps its value.  Candidates are the only blocks whose MAW the score
// tiles read, and these are never written here, so this may run at any time
// after every part of the unit has written its dense pages' log-masses.
// With tok (the step's append folded into the launch, after every part has
// read the dense pages) it also writes the new token into its page (V
// transposed) and folds it into its block's summary (min/max in logical
// order, as the append kernel does).  LDS: pm [kFuseDenseLds], dm and dz
// [4 G] floats.  Every thread of the workgroup calls it.
template <int D, int G>
__device__ __attribute__((always_inline)) void dense_maw(const Ctx &c, int seq, int h,
                                                         const HeadInfo &hi, const UG &g,
                                                         const NewTok &tok, float *pm, float *dm,
                                                         float *dz) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const DenseList dl = dense_list(g);
  const float *lmb = c.sc.lm_pg + ((size_t)seq * c.dm.Hq + (size_t)h * G) * c.dm.lm_cap;
  float *mw = c.L.maw + hi.maw_off + (size_t)seq * hi.nbmax;
  constexpr int C4 = D / 4;
  // ---- one batch of loads: the dense pages' log-masses (one page per
  // thread; windows of more than 4096 tokens load the rest below), the MAW of
  // the block of dense slot tid, the new token and its block's summary
  float lmv[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
    lmv[gg] = tid < dl.n ? ld_dev(&lmb[(size_t)gg * c.dm.lm_cap + tid]) : -INFINITY;
  const int blk0 = tid < g.n_dt ? dense_block(g, tid) : 0;
  const bool upd0 = tid < g.n_dt && !is_candidate(g, blk0);
  const float mw0 = upd0 ? mw[blk0] : 0.0f;
  const bool app = tok.k != nullptr;
  const int pos = g.N - 1, blk_new = app ? div_S(pos, g.S) : 0;
  const bool had = app && pos > blk_new * g.S;  // the block held tokens before
  uint16_t *sp_new = c.L.summ + hi.summ_off + (size_t)seq * C4 * hi.nbmax * 8 +
                     ((size_t)min(tid, C4 - 1) * hi.nbmax + blk_new) * 8;
  uint4 k8 = make_uint4(0, 0, 0, 0), s_old = make_uint4(0, 0, 0, 0);
  uint2 k4 = make_uint2(0, 0);
  uint16_t v1 = 0;
  if (app) {
    if (tid < D / 8) k8 = reinterpret_cast<const uint4 *>(tok.k)[tid];
    if (tid < D) v1 = tok.v[tid];
    if (tid < C4) {
      k4 = reinterpret_cast<const uint2 *>(tok.k)[tid];
      if (had) s_old = *reinterpret_cast<const uint4 *>(sp_new);
    }
  }
  // ---- per head, lse_D: each thread folds its pages into a running (max,
  // sum), then the waves', then the workgroup's
  float mt[G], zt[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    mt[gg] = lmv[gg];
    zt[gg] = lmv[gg] == -INFINITY ? 0.0f : 1.0f;
  }
  for (int t = tid + 256; t < dl.n; t += 256)
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float x = ld_dev(&lmb[(size_t)gg * c.dm.lm_cap + t]);
      if (x == -INFINITY) continue;
      if (x > mt[gg]) {
        zt[gg] = zt[gg] * fast_exp(mt[gg] - x) + 1.0f;  // (exp(-inf) = 0)
        mt[gg] = x;
      } else {
        zt[gg] += fast_exp(x - mt[gg]);
      }
    }
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float M = wave_max(mt[gg]);
    const float z = wave_sum(M == -INFINITY || mt[gg] == -INFINITY ? 0.0f
                                                                   : zt[gg] * fast_exp(mt[gg] - M));
    if (lane == 0) {
      dm[wv * G + gg] = M;
      dz[wv * G + gg] = z;
    }
  }
  __syncthreads();
  float lse_d[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float M = fmaxf(fmaxf(dm[gg], dm[G + gg]), fmaxf(dm[2 * G + gg], dm[3 * G + gg]));
    float z = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        z += dm[w * G + gg] == -INFINITY ? 0.0f : dz[w * G + gg] * fast_exp(dm[w * G + gg] - M);
    lse_d[gg] = M == -INFINITY ? -INFINITY : M + fast_log(z);
  }
  // mass of each dense page under the dense partial, summed over the heads
  for (int t = tid; t < dl.n; t += 256) {
    float a = 0.0f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float x = t < 256 ? lmv[gg] : ld_dev(&lmb[(size_t)gg * c.dm.lm_cap + t]);
      a += (x == -INFINITY || lse_d[gg] == -INFINITY) ? 0.0f : fast_exp(x - lse_d[gg]);
    }
    pm[t] = a;
  }
  __syncthreads();
  const float r = c.dm.maw_decay, omr = 1.0f - r, inv_g = 1.0f / (float)G;
  const int PPB = g.S / kPage;
  for (int x = tid; x < g.n_dt; x += 256) {
    const int blk = x == tid ? blk0 : dense_block(g, x);
    if (is_candidate(g, blk)) continue;  // a token outside D: frozen
    float a = 0.0f;
    for (int pp = 0; pp < PPB; ++pp) {
      const int t = dense_pos(dl, blk * PPB + pp);
      if (t >= 0) a += pm[t];
    }
    const float m_old = x == tid ? mw0 : mw[blk];
    mw[blk] = __fadd_rn(__fmul_rn(r, m_old), __fmul_rn(omr, a * inv_g));
  }
  if (app) {
    if (tid < D / 8)
      reinterpret_cast<uint4 *>(c.L.k)[(((size_t)tok.pg * c.dm.Hkv + h) * (D / 8) + tid) * kPage +
                                       tok.slot] = k8;
    if (tid < D) c.L.v[(((size_t)tok.pg * c.dm.Hkv + h) * D + tid) * kPage + tok.slot] = v1;
    if (tid < C4) {
      const uint32_t kw[2] = {k4.x, k4.y}, ow[4] = {s_old.x, s_old.y, s_old.z, s_old.w};
      uint32_t nw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = (kw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        uint32_t mn = x, mx = x;
        if (had) {
          const uint32_t omn = ow[j] & 0xffffu, omx = ow[j] >> 16;
          const float fx = __uint_as_float(x << 16);
          mn = fx < __uint_as_float(omn << 16) ? x : omn;
          mx = fx > __uint_as_float(omx << 16) ? x : omx;
        }
        nw[j] = mn | (mx << 16);
      }
      *reinterpret_cast<uint4 *>(sp_new) = make_uint4(nw[0], nw[1], nw[2], nw[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// kernels

// append: K/V scatter and summary roles by workgroup index.
template <int D>
__global__ __launch_bounds__(256) void k_prep(Ctx c, AppendBatch b, int tok_per_wg,
                                              int n_scatter_x, int n_summ_x,
                                              const uint16_t *__restrict__ k_new,
                                              const uint16_t *__restrict__ v_new) {
  int wg = blockIdx.x;
  const int n_scatter = n_scatter_x * b.n;
  const int n_summ = n_summ_x * c.dm.Hkv * b.n;
  if (wg < n_scatter) {
    append_scatter<D>(c, b, wg / n_scatter_x, wg % n_scatter_x, tok_per_wg, k_new, v_new);
    return;
  }
  wg -= n_scatter;
  if (wg < n_summ) {
    const int x = wg % n_summ_x, hh = (wg / n_summ_x) % c.dm.Hkv, i = wg / (n_summ_x * c.dm.Hkv);
    append_summ<D>(c, b, i, hh, x * 256 + threadIdx.x, k_new);
    return;
  }
}

// select: score tiles; the last tile of a unit to arrive runs its top-k.
template <int D, int G>
__global__ __launch_bounds__(256) void k_select(Ctx c, SeqBatch b, int tiles_x,
                                                int32_t *__restrict__ blk_idx,
                                                int32_t *__restrict__ blk_cnt, int k_cap,
                                                const uint16_t *__restrict__ q,
                                                int lrows_words) {
  // dynamic LDS: TopkSmem + lrows_words top-k words + one 64-bit mask per row
  extern __shared__ __align__(16) unsigned char smem_raw[];
  TopkSmem &smem_topk = *reinterpret_cast<TopkSmem *>(smem_raw);
  const int wg = blockIdx.x;
  const int tile = wg % tiles_x, h = (wg / tiles_x) % c.dm.Hkv, i = wg / (tiles_x * c.dm.Hkv);
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  const int n_blk = div_S(N + hi.S - 1, hi.S);
  const int n_tiles = max(1, cdiv(scored_blocks(N, hi.S, c.dm), kScoreTile));
  if (tile >= n_tiles) return;
  const int rows_h = c.dm.pqh ? G : 1;  // selections per KV head
  if (selects_nothing(hi, N, c.dm)) {  // no scoring: the count is 0
    if (tile == 0 && threadIdx.x < rows_h)
      st_dev(&blk_cnt[((size_t)i * c.dm.Hkv + h) * rows_h + threadIdx.x], 0);
    return;
  }
  UG g;
  if (c.dm.pqh) {  // the query heads' top-ks run in the next launch (k_topk_heads)
    score_tile<D, G, true>(c, i, seq, h, hi, N, n_blk, tile, q, smem_topk, false, g);
    return;
  }
  score_tile<D, G>(c, i, seq, h, hi, N, n_blk, tile, q, smem_topk, false, g);
  uint32_t *ctr = &c.sc.arrive[((size_t)seq * c.dm.Hkv + h) * 4];
  if (!arrive_last(ctr, (unsigned)n_tiles, &smem_topk.last)) return;
  uint32_t *lrows = reinterpret_cast<uint32_t *>(smem_raw + sizeof(TopkSmem));
  unsigned long long *dmask = reinterpret_cast<unsigned long long *>(lrows + lrows_words);
  const size_t unit = (size_t)seq * c.dm.Hkv + h, out = (size_t)i * c.dm.Hkv + h;
  if (wide_unit(g.n_sc)) {
    topk_wide<D, G>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap, smem_topk, dmask,
                    reinterpret_cast<int32_t *>(lrows), lrows_words);
  } else {
    topk_unit<D, G>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap, smem_topk, lrows,
                    lrows_words, dmask);
  }
  if (threadIdx.x == 0) st_dev(ctr, 0u);
}

// Top-k of one query head with one selection per query head (grid: G query
// heads x KV heads x sequences, after k_select has scored every block per
// query head): that head's own keys, bound and exact scores, a group of one.
template <int D, int G>
__global__ __launch_bounds__(256) void k_topk_heads(Ctx c, SeqBatch b, int32_t *__restrict__ blk_idx,
                                                    int32_t *__restrict__ blk_cnt, int k_cap,
                                                    const uint16_t *__restrict__ q,
                                                    int lrows_words) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  TopkSmem &smem_topk = *reinterpret_cast<TopkSmem *>(smem_raw);
  const int j = blockIdx.x % G, h = (blockIdx.x / G) % c.dm.Hkv, i = blockIdx.x / (G * c.dm.Hkv);
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  if (selects_nothing(hi, N, c.dm)) return;  // (k_select wrote the count 0)
  const UG g = unit_geom(N, hi, c.dm);
  const size_t unit = ((size_t)seq * c.dm.Hkv + h) * G + j, out = ((size_t)i * c.dm.Hkv + h) * G + j;
  uint32_t *lrows = reinterpret_cast<uint32_t *>(smem_raw + sizeof(TopkSmem));
  unsigned long long *dmask = reinterpret_cast<unsigned long long *>(lrows + lrows_words);
  if (wide_unit(g.n_sc))
    topk_wide<D, 1>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap, smem_topk, dmask,
                    reinterpret_cast<int32_t *>(lrows), lrows_words);
  else
    topk_unit<D, 1>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap, smem_topk, lrows,
                    lrows_words, dmask);
}

// ---------------------------------------------------------------------------
// Learn-from-the-past selection ([LFPS] What carries the argument and Figure 4;
// at block granularity): per (sequence, KV head) a vertical table pv over
// blocks and a slash table ps over block offsets from the newest block b.
// Candidates C: blocks above the threshold tau = mean + a (max - mean) of
// either table, grown by the offsets {-1, 0, 1, 2}, kept when above a table's
// mean and holding a token outside D.  Only the blocks of C are scored, each
// exactly (fp64 in channel order, the plain sum where the products' exponents
// could make the quad's order round differently); the k = min(|C|, budget)
// best by (score desc, index asc) are written ascending.  One workgroup per
// unit.
constexpr int kLfpsLds = 6144;  // table candidates a workgroup keeps in LDS
struct LfpsSmem {
  int32_t list[kLfpsLds];  // C, ascending (global scratch past kLfpsLds)
  uint32_t key[kLfpsLds];  // order keys of their exact group scores
  float qs[SD_MAX_GROUP * 128];
  double rd[8];
  float rf[8];
  uint32_t red[16];
};

__device__ __forceinline__ double wg_sum_f64(double x, double *rd) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) rd[threadIdx.x >> 6] = x;
  __syncthreads();
  return (rd[0] + rd[1]) + (rd[2] + rd[3]);
}
__device__ __forceinline__ float wg_max_f32(float x, float *rf) {
  x = wave_max(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) rf[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(rf[0], rf[1]), fmaxf(rf[2], rf[3]));
}

template <int D, int G>
__global__ __launch_bounds__(256) void k_lfps_select(Ctx c, SeqBatch b, int32_t *__restrict__ blk_idx,
                                                     int32_t *__restrict__ blk_cnt, int k_cap,
                                                     const uint16_t *__restrict__ q) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  LfpsSmem &sm = *reinterpret_cast<LfpsSmem *>(smem_raw);
  uint32_t *c0w = reinterpret_cast<uint32_t *>(smem_raw + sizeof(LfpsSmem));  // bit rows
  const int tid = threadIdx.x;
  const int h = blockIdx.x % c.dm.Hkv, i = blockIdx.x / c.dm.Hkv;
  // wpu workgroups per unit (blockIdx.y): each works out C, scores its share
  // of C's passes of 128 blocks (pass x belongs to workgroup x % wpu) and
  // writes their keys to the unit's global scratch; the last to arrive takes
  // the k-th key and writes the selection
  const int wpu = gridDim.y, wi = blockIdx.y;
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  const size_t unit = (size_t)seq * c.dm.Hkv + h, out = (size_t)i * c.dm.Hkv + h;
  if (selects_nothing(hi, N, c.dm)) {
    if (tid == 0) st_dev(&blk_cnt[out], 0);
    return;
  }
  const UG g = unit_geom(N, hi, c.dm);
  const int nb = g.n_blk, bb = nb - 1;
  const float *pv = c.L.phi + 2 * hi.maw_off + (size_t)seq * 2 * hi.nbmax;
  const float *ps = pv + hi.nbmax;
  int32_t *gl = c.sc.ulist + unit * c.dm.key_stride;
  uint32_t *gk = c.sc.ukeys + unit * c.dm.key_stride;
  auto lst_ld = [&](int p) -> int { return p < kLfpsLds ? sm.list[p] : ld_dev(&gl[p]); };
  auto key_ld = [&](int p) -> uint32_t { return p < kLfpsLds ? sm.key[p] : ld_dev(&gk[p]); };
  auto key_st = [&](int p, uint32_t v) { if (p < kLfpsLds) sm.key[p] = v; else st_dev(&gk[p], v); };
  const uint16_t *qg = q + out * G * D;
  for (int x = tid; x < G * D; x += 256) sm.qs[x] = __uint_as_float((uint32_t)qg[x] << 16);
  // 1. mean and maximum of each table over [0, b] (eight loads in flight per
  // thread and table)
  constexpr int LB = 8;
  double sv = 0.0, ss = 0.0;
  float mv = -INFINITY, ms = -INFINITY;
  for (int t0 = tid; t0 <= bb; t0 += 256 * LB) {
    float a[LB], e[LB];
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int t = t0 + 256 * u;
      a[u] = t <= bb ? pv[t] : 0.0f;
      e[u] = t <= bb ? ps[t] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      if (t0 + 256 * u > bb) break;
      sv += (double)a[u];
      ss += (double)e[u];
      mv = fmaxf(mv, a[u]);
      ms = fmaxf(ms, e[u]);
    }
  }
  sv = wg_sum_f64(sv, sm.rd);
  ss = wg_sum_f64(ss, sm.rd + 4);
  mv = wg_max_f32(mv, sm.rf);
  ms = wg_max_f32(ms, sm.rf + 4);
  const double mu_v = sv / (double)nb, mu_s = ss / (double)nb;
  const double a = (double)c.dm.lfps_a;
  const double tau_v = mu_v + a * ((double)mv - mu_v), tau_s = mu_s + a * ((double)ms - mu_s);
  // 2. over [0, b], as bits: C0 (above a threshold) and "above a mean"
  const int words = (nb + 31) >> 5;
  uint32_t *abw = c0w + words;
  for (int w = tid; w < 2 * words; w += 256) c0w[w] = 0u;
  __syncthreads();
  for (int t0 = tid; t0 <= bb; t0 += 256 * LB) {
    float a[LB], e[LB];
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int t = t0 + 256 * u;
      a[u] = t <= bb ? pv[t] : 0.0f;
      e[u] = t <= bb ? ps[bb - t] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int t = t0 + 256 * u;
      if (t > bb) break;
      if ((double)a[u] > tau_v || (double)e[u] > tau_s) atomicOr(&c0w[t >> 5], 1u << (t & 31));
      if ((double)a[u] > mu_v || (double)e[u] > mu_s) atomicOr(&abw[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  auto c0 = [&](int x) -> bool { return x >= 0 && x <= bb && ((c0w[x >> 5] >> (x & 31)) & 1u); };
  auto in_c = [&](int x) -> bool {
    return is_candidate(g, x) && (c0(x + 1) || c0(x) || c0(x - 1) || c0(x - 2)) &&
           ((abw[x >> 5] >> (x & 31)) & 1u);
  };
  // 3. C in block order: thread t takes blocks [t m, t m + m) of the scored ones
  const int n_sc = g.n_sc, m = cdiv(n_sc, 256), j0 = tid * m;
  int mine = 0;
  for (int x = j0; x < min(j0 + m, n_sc); ++x) mine += in_c(x) ? 1 : 0;
  int slot = 0, nC = 0;
  int o = wg_scan(mine, sm.red, slot, nC);
  for (int x = j0; x < min(j0 + m, n_sc); ++x) {
    if (!in_c(x)) continue;
    // (past the LDS list each entry is written once, by its pass's owner)
    if (o < kLfpsLds) sm.list[o] = x;
    else if ((o >> 7) % wpu == wi) st_dev(&gl[o], x);
    ++o;
  }
  __syncthreads();
  if (tid == 0 && wi == 0) st_dev(&c.sc.unit_acc[4 * unit + 3], (uint32_t)nC);  // |C|, for inspection
  const int kq = min(g.kk, nC);
  if (kq == 0) {
    if (tid == 0 && wi == 0) st_dev(&blk_cnt[out], 0);
    return;
  }
  // 4. exact group scores: one lane quad per two blocks, each block's summary
  // loaded once for all the group's heads; this workgroup's passes
  for (int p0 = 128 * wi; p0 < nC; p0 += 128 * wpu) {
    int blk[2];
    bool on[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int p = p0 + 64 * n + (tid >> 2);
      on[n] = p < nC;
      blk[n] = on[n] ? lst_ld(p) : 0;
    }
    double best[2];
    exact_group_quads<D, G, 2>(c, seq, hi, blk, on, sm.qs, best);
#pragma unroll
    for (int n = 0; n < 2; ++n)
      if (on[n] && (tid & 3) == 0) {
        const int p = p0 + 64 * n + (tid >> 2);
        const uint32_t kv = order_key((float)best[n]);
        if (wpu == 1) key_st(p, kv); else st_dev(&gk[p], kv);
      }
  }
  if (wpu > 1) {
    // the last workgroup of the unit to arrive has every key: those within
    // the LDS list come to LDS, the rest are read from the scratch
    uint32_t *ctr = &c.sc.arrive[unit * 4];
    if (!arrive_last(ctr, (unsigned)wpu, reinterpret_cast<int *>(&sm.red[15]))) return;
    if (tid == 0) st_dev(ctr, 0u);
    for (int p = tid; p < min(nC, kLfpsLds); p += 256) sm.key[p] = ld_dev(&gk[p]);
  }
  __syncthreads();
  // 5. the kq-th largest key T: keys above T are in, of the keys equal to T
  // the lowest blocks (first in the list) fill the rest
  const int mm = cdiv(nC, 256), q0 = tid * mm, q1 = min(q0 + mm, nC);
  auto count_ge = [&](uint32_t t) {
    int n = 0;
    for (int p = q0; p < q1; ++p) n += key_ld(p) >= t ? 1 : 0;
    return wg_sum(n, sm.red, slot);
  };
  uint32_t lo = 0u, hi_k = 0xffffffffu;  // count_ge(lo) >= kq > count_ge(hi_k + 1)
  while (lo < hi_k) {
    const uint32_t mid = lo + ((hi_k - lo) >> 1) + 1u;
    if (count_ge(mid) >= kq) lo = mid; else hi_k = mid - 1u;
  }
  const uint32_t T = lo;
  const int n_gt = T == 0xffffffffu ? 0 : count_ge(T + 1u);
  const int need = kq - n_gt;  // keys equal to T to take, by block order
  int eq = 0, gt = 0;
  for (int p = q0; p < q1; ++p) {
    const uint32_t k = key_ld(p);
    eq += k == T ? 1 : 0;
    gt += k > T ? 1 : 0;
  }
  int eq_tot = 0;
  const int eq_before = wg_scan(eq, sm.red, slot, eq_tot);
  const int take_eq = max(0, min(eq, need - eq_before));
  int tot = 0;
  int pos = wg_scan(gt + take_eq, sm.red, slot, tot);
  int32_t *dst = blk_idx + out * k_cap;
  int e_seen = eq_before;
  for (int p = q0; p < q1; ++p) {
    const uint32_t k = key_ld(p);
    bool take = k > T;
    if (k == T) take = e_seen++ < need;
    if (take) {
      if (pos < k_cap) st_dev(&dst[pos], lst_ld(p));
      ++pos;
    }
  }
  if (tid == 0) st_dev(&blk_cnt[out], kq);
}

// The tables' update after a step's fusion ([LFPS] What carries the argument:
// both tables decay by r and take the step's attention weights): the mass
// each block received under the softmax over the attended set, averaged over
// the group's query heads, from the log-masses of the dense pages and of the
// selected pages (sel: the selection the attention call took) and each head's
// lse; then pv[x] <- r pv[x] + (1 - r) a[x], ps[o] <- r ps[o] + (1 - r) a[b - o]
// over [0, b].  ablk: LDS, one float per block.
template <int D, int G>
__device__ void lfps_update_unit(const Ctx &c, int seq, int h, const HeadInfo &hi, const UG &g,
                                 const int32_t *sel, int cnt, const float *lse_h, float *ablk) {
  const int tid = threadIdx.x, nb = g.n_blk, bb = nb - 1, PPB = g.S / kPage;
  const float *lmb = c.sc.lm_pg + ((size_t)seq * c.dm.Hq + (size_t)h * G) * c.dm.lm_cap;
  float *pv = c.L.phi + 2 * hi.maw_off + (size_t)seq * 2 * hi.nbmax;
  float *ps = pv + hi.nbmax;
  for (int x = tid; x < nb; x += 256) ablk[x] = 0.0f;
  __syncthreads();
  const DenseList dl = dense_list(g);
  const float inv_g = 1.0f / (float)G;
  auto mass = [&](int slot_) {
    float a = 0.0f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float x = ld_dev(&lmb[(size_t)gg * c.dm.lm_cap + slot_]);
      a += (x == -INFINITY || lse_h[gg] == -INFINITY) ? 0.0f : fast_exp(x - lse_h[gg]);
    }
    return a * inv_g;
  };
  for (int t = tid; t < dl.n; t += 256) {
    const int blk = div_S(dense_page(dl, t) * kPage, g.S);
    atomicAdd(&ablk[blk], mass(t));
  }
  for (int t = tid; t < cnt * PPB; t += 256) {
    const int blk = sel[t / PPB];
    if (blk >= 0 && blk < nb) atomicAdd(&ablk[blk], mass(c.dm.lm_sel0 + t));
  }
  __syncthreads();
  const float r = c.dm.maw_decay, omr = 1.0f - r;
  for (int x = tid; x <= bb; x += 256) {
    pv[x] = __fadd_rn(__fmul_rn(r, pv[x]), __fmul_rn(omr, ablk[x]));
    ps[x] = __fadd_rn(__fmul_rn(r, ps[x]), __fmul_rn(omr, ablk[bb - x]));
  }
}

// Table init from the last s prefill positions ([LFPS] Assumptions & free
// parameters, s = 32, Eq. (4)): position p_u = N - s + u attends causally to
// [0, p_u] (dense); k_lfps_init_mass writes its block masses (group mean)
// to scratch A, then k_lfps_init_tables applies the s updates in order.
// Grid of the first: (s, Hkv, sequences); two passes over the tokens: the
// heads' max and sum, then the masses.
template <int D, int G>
__global__ __launch_bounds__(256) void k_lfps_init_mass(Ctx c, SeqBatch b, const uint16_t *__restrict__ qp,
                                                        int s_steps, float *__restrict__ A) {
  extern __shared__ __align__(16) float ablk[];
  __shared__ float qs[G * D];
  __shared__ float rf[8];
  const int tid = threadIdx.x;
  const int u = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  const int pos = N - s_steps + u;
  const size_t arow = (((size_t)i * c.dm.Hkv + h) * s_steps + u) * c.dm.key_stride;
  if (pos < 0) return;
  const int nb = div_S(pos, hi.S) + 1;
  for (int x = tid; x < G * D; x += 256)
    qs[x] = __uint_as_float(
        (uint32_t)qp[(((size_t)i * s_steps + u) * c.dm.Hq + (size_t)h * G) * D + x] << 16);
  for (int x = tid; x < nb; x += 256) ablk[x] = 0.0f;
  __syncthreads();
  const int32_t *pts = c.L.pt + (size_t)seq * c.dm.pages_per_seq;
  auto logits = [&](int j, float (&sc)[G]) {
    const uint16_t *kr = c.L.k + ((size_t)pts[j >> 4] * c.dm.Hkv + h) * kPage * D + (j & 15) * 8;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) sc[gg] = 0.0f;
    for (int ch = 0; ch < D; ch += 8) {
      const uint4 w = *reinterpret_cast<const uint4 *>(kr + (size_t)(ch / 8) * kPage * 8);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float k0 = bf16_lo(ws[e]), k1 = bf16_hi(ws[e]);
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
          sc[gg] = fmaf(qs[gg * D + ch + 2 * e + 1], k1, fmaf(qs[gg * D + ch + 2 * e], k0, sc[gg]));
      }
    }
#pragma unroll
    for (int gg = 0; gg < G; ++gg) sc[gg] *= c.dm.scale_log2;  // log2 units
  };
  float mx[G], z[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) mx[gg] = -INFINITY, z[gg] = 0.0f;
  for (int j = tid; j <= pos; j += 256) {
    float sc[G];
    logits(j, sc);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      if (sc[gg] > mx[gg]) {
        z[gg] = z[gg] * exp2f(mx[gg] - sc[gg]) + 1.0f;
        mx[gg] = sc[gg];
      } else {
        z[gg] += exp2f(sc[gg] - mx[gg]);
      }
    }
  }
  float lse[G];  // log2 units
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float M = wg_max_f32(mx[gg], rf);
    float zz = mx[gg] == -INFINITY ? 0.0f : z[gg] * exp2f(mx[gg] - M);
    zz = wave_sum(zz);
    __syncthreads();
    if ((tid & 63) == 0) rf[4 + (tid >> 6)] = zz;
    __syncthreads();
    lse[gg] = M + log2f((rf[4] + rf[5]) + (rf[6] + rf[7]));
  }
  const float inv_g = 1.0f / (float)G;
  for (int j = tid; j <= pos; j += 256) {
    float sc[G];
    logits(j, sc);
    float a = 0.0f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) a += exp2f(sc[gg] - lse[gg]);
    atomicAdd(&ablk[div_S(j, hi.S)], a * inv_g);
  }
  __syncthreads();
  for (int x = tid; x < nb; x += 256) A[arow + x] = ablk[x];
}

// The s updates in order (grid: Hkv, sequences).
__global__ __launch_bounds__(256) void k_lfps_init_tables(Ctx c, SeqBatch b, int s_steps,
                                                          const float *__restrict__ A) {
  const int h = blockIdx.x, i = blockIdx.y;
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  float *pv = c.L.phi + 2 * hi.maw_off + (size_t)seq * 2 * hi.nbmax;
  float *ps = pv + hi.nbmax;
  const int nb_all = div_S(N + hi.S - 1, hi.S);
  const float r = c.dm.maw_decay, omr = 1.0f - r;
  for (int x = threadIdx.x; x < hi.nbmax; x += 256) pv[x] = ps[x] = 0.0f;
  __syncthreads();
  for (int u = 0; u < s_steps; ++u) {
    const int pos = N - s_steps + u;
    if (pos < 0) continue;
    const int bb = div_S(pos, hi.S);
    const float *a = A + (((size_t)i * c.dm.Hkv + h) * s_steps + u) * c.dm.key_stride;
    for (int x = threadIdx.x; x <= bb && x < nb_all; x += 256) {
      pv[x] = __fadd_rn(__fmul_rn(r, pv[x]), __fmul_rn(omr, a[x]));
      ps[x] = __fadd_rn(__fmul_rn(r, ps[x]), __fmul_rn(omr, a[bb - x]));
    }
    __syncthreads();
  }
}

// Union of a KV head's per-query-head selections (one workgroup per
// (KV head, sequence)): a byte of head bits per scored block in LDS, set from
// the G lists, then compacted in block order into block | mask << 24 entries
// with a workgroup scan.  Entries outside the scored blocks are dropped (a
// block past them lies wholly in the window: it has no token outside D).
template <int G>
__global__ __launch_bounds__(256) void k_union(Ctx c, SeqBatch b, const int32_t *__restrict__ blk_idx,
                                               const int32_t *__restrict__ blk_cnt, int k_cap) {
  extern __shared__ __align__(16) uint32_t hb[];  // ceil(max_scored / 4) words
  __shared__ uint32_t red[8];
  const int tid = threadIdx.x;
  const int h = blockIdx.x, i = blockIdx.y;
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  const int n_sc = min(scored_blocks(N, hi.S, c.dm), b.max_scored);
  const int words = (n_sc + 3) >> 2;
  for (int w = tid; w < words; w += 256) hb[w] = 0u;
  __syncthreads();
  for (int j = 0; j < G; ++j) {
    const size_t row = ((size_t)i * c.dm.Hkv + h) * G + j;
    const int cnt = min(max(blk_cnt[row], 0), k_cap);
    for (int e = tid; e < cnt; e += 256) {
      const int blk = blk_idx[row * k_cap + e];
      if (blk >= 0 && blk < n_sc) atomicOr(&hb[blk >> 2], 1u << (8 * (blk & 3) + j));
    }
  }
  __syncthreads();
  const int m = (n_sc + 255) >> 8, j0 = tid * m;
  auto mask_of = [&](int blk) -> uint32_t { return (hb[blk >> 2] >> (8 * (blk & 3))) & 0xffu; };
  int mine = 0;
  for (int x = 0; x < m; ++x)
    if (j0 + x < n_sc && mask_of(j0 + x)) ++mine;
  int slot = 0, total = 0;
  int o = wg_scan(mine, red, slot, total);
  const size_t unit = (size_t)seq * c.dm.Hkv + h;
  int32_t *dst = c.sc.uni + unit * c.dm.ucap;
  for (int x = 0; x < m; ++x) {
    const int blk = j0 + x;
    const uint32_t mk = blk < n_sc ? mask_of(blk) : 0u;
    if (mk) {
      if (o < c.dm.ucap) st_dev(&dst[o], (int32_t)((uint32_t)blk | (mk << 24)));
      ++o;
    }
  }
  if (tid == 0) st_dev(&c.sc.ucnt[unit], min(total, c.dm.ucap));
}

// attend, separate-call form: P workgroups per unit, of which the unit's
// parts (unit_parts) write one partial each; part 0 also empties the other
// slots up to p_cap.
template <int D, int G>
__global__ __launch_bounds__(256, 2) void k_attend(Ctx c, SeqBatch b, int P,
                                                   const uint16_t *__restrict__ q,
                                                   const int32_t *__restrict__ blk_idx,
                                                   const int32_t *__restrict__ blk_cnt, int k_cap,
                                                   float *__restrict__ o_part,
                                                   float *__restrict__ lse_part, int p_cap) {
  __shared__ AttLds<D, G> sm;
  __shared__ int s_cnt;
  const int part = blockIdx.x % P, u = blockIdx.x / P;
  const int h = u % c.dm.Hkv, i = u / c.dm.Hkv;
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i];
  const UG g = unit_geom(b.len[i], hi, c.dm);
  const int PU = unit_parts(g, P, c.dm);
  if (part >= PU) return;
  SelIn si;
  if (c.dm.pqh) {  // the union of the group's sets (k_union)
    const size_t unit = (size_t)seq * c.dm.Hkv + h;
    si.blk = c.sc.uni + unit * c.dm.ucap;
    si.cnt = min(max(c.sc.ucnt[unit], 0), union_blocks(g, c.dm));
  } else {
    si.blk = blk_idx + ((size_t)i * c.dm.Hkv + h) * k_cap;
    si.cnt = min(min(max(blk_cnt[(size_t)i * c.dm.Hkv + h], 0), k_cap), hi.kcap);
  }
  if (part == 0) empty_slots<D, G>(c, i, h, PU, p_cap, o_part, lse_part);
  attend_part<D, G>(c, i, seq, h, g, part, PU, q, si, o_part, lse_part, p_cap, sm, nullptr,
                    &s_cnt, NewTok(), hi);
}

// One decode step in one launch.  Workgroups by index: score tiles (the last
// of a unit runs its top-k and publishes the selection, tagged with the step
// number), then P attention parts per unit (a unit uses unit_parts of them,
// the rest exit at once), then one MAW worker per unit.  A part streams its
// dense pages from the start, then waits for the selection and streams its
// selected pages; the last part of a unit to finish fuses the partials.  The
// MAW worker updates MAW once the parts' dense pages and the top-k are done.
// Workgroups start in index order on each XCD; a part waits on a score tile,
// which never waits, and a MAW worker on parts and score tiles, which never
// wait on it, so no wait is on a workgroup that cannot start; each wait is
// also bounded in time (after kWaitTicks it gives up and raises the error
// flag).
template <int D, int G>
__global__ __launch_bounds__(256, 2) void k_step(Ctx c, SeqBatch b, int tiles_x, int P,
                                                 int32_t *__restrict__ blk_idx,
                                                 int32_t *__restrict__ blk_cnt, int k_cap,
                                                 const uint16_t *__restrict__ q,
                                                 float *__restrict__ o_part,
                                                 float *__restrict__ lse_part, int p_cap,
                                                 float *__restrict__ o, float *__restrict__ lse,
                                                 int lrows_words, uint32_t epoch, int ptl_cap,
                                                 const uint16_t *__restrict__ k_new,
                                                 const uint16_t *__restrict__ v_new) {
  // dynamic LDS: max(TopkSmem + top-k words and row masks, AttLds + ptl_cap
  // page-table entries, FuseSmem)
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int s_flag, s_cnt;
  TopkSmem &smem_topk = *reinterpret_cast<TopkSmem *>(smem_raw);
  AttLds<D, G> &smem_att = *reinterpret_cast<AttLds<D, G> *>(smem_raw);
  FuseSmem<G> &smem_fuse = *reinterpret_cast<FuseSmem<G> *>(smem_raw);
  SD_TL(0);  // first instruction
  // grid (KV head, sequence, role index): workgroups are dispatched with
  // blockIdx.x fastest, so the flat order is role-major.  Score tiles come
  // first, tile-major: consecutive workgroups (spread over the CUs first) are
  // different units' tiles of the same index, so the summary loads spread
  // evenly and the short last tiles of units are dispatched last.  The
  // attention parts follow, part-major.
  const int h = blockIdx.x, i = blockIdx.y;
  const bool score = (int)blockIdx.z < tiles_x;
  const int idx = score ? (int)blockIdx.z : (int)blockIdx.z - tiles_x;
  const HeadInfo hi = c.heads[h];
  const int seq = b.seq[i], N = b.len[i];
  const size_t unit = (size_t)seq * c.dm.Hkv + h;
  // the step's appended token of this unit, if its append runs in this
  // launch (then N >= 1)
  auto new_tok = [&](int n) {
    NewTok t;
    if (k_new) {
      t.k = k_new + ((size_t)i * c.dm.Hkv + h) * D;
      t.v = v_new + ((size_t)i * c.dm.Hkv + h) * D;
      t.slot = (n - 1) & (kPage - 1);
      t.pg = c.L.pt[(size_t)seq * c.dm.pages_per_seq + ((n - 1) >> 4)];
    }
    return t;
  };
  if (score) {
    const int n_blk = div_S(N + hi.S - 1, hi.S);
    const int n_tiles = max(1, cdiv(scored_blocks(N, hi.S, c.dm), kScoreTile));
    if (idx >= n_tiles || selects_nothing(hi, N, c.dm)) return;  // (the parts cover k = 0)
    // the score tiles, the top-k and the fusion are on every unit's critical
    // path: their waves get issue priority over the attention parts'
    __builtin_amdgcn_s_setprio(2);
    // without MAW flags each tile also lists its candidates for the fast top-k
    UG g;
    const bool fast = score_tile<D, G>(c, i, seq, h, hi, N, n_blk, idx, q, smem_topk,
                                       c.dm.maw_beta <= 0.0f && n_tiles <= kFastTiles, g);
    SD_TL(2);  // tile list published
    uint32_t *ctr = &c.sc.arrive[unit * 4];
    const bool last_tile = arrive_last(ctr, (unsigned)n_tiles, &s_flag);
    SD_TL(3);  // arrived
    if (!last_tile) return;
    __builtin_amdgcn_s_setprio(3);
    uint32_t *lrows = reinterpret_cast<uint32_t *>(smem_raw + sizeof(TopkSmem));
    unsigned long long *tagd = c.sc.seltag + unit * c.dm.kcap;
    // the fast top-k publishes the count itself, right after the entries
    const size_t out = (size_t)i * c.dm.Hkv + h;
    const bool fast_done =
        fast && (g.kk <= kTileList
                     ? topk_fast<D, G>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap,
                                       smem_topk, tagd, &c.sc.rtag[unit], epoch)
                     : topk_fast128<D, G>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap,
                                          smem_topk, tagd, &c.sc.rtag[unit], epoch));
    if (!fast_done) {
      unsigned long long *dmask = reinterpret_cast<unsigned long long *>(lrows + lrows_words);
      if (wide_unit(g.n_sc))
        topk_wide<D, G>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap, smem_topk, dmask,
                        reinterpret_cast<int32_t *>(lrows), lrows_words, tagd, epoch);
      else
        topk_unit<D, G>(c, seq, unit, out, hi, g, q, blk_idx, blk_cnt, k_cap, smem_topk, lrows,
                        lrows_words, dmask, tagd, epoch);
    }
    SD_TL(4);  // top-k done
    if (threadIdx.x == 0) {
      // the entries carry their own tags, so the count need not wait for them
      st_dev(ctr, 0u);
      if (!fast_done || g.kk == 0)
        st_dev(&c.sc.rtag[unit], ((unsigned long long)epoch << 32) |
                                     (uint32_t)min(min(g.kk, k_cap), hi.kcap));
    }
    // the unit's MAW worker waits for this arrival too: the tiles have read
    // the MAW values and summaries that its update writes
    arrive(&c.sc.arrive[unit * 4 + 2]);
    return;
  }
  if ((int)blockIdx.z == tiles_x + P) {
    // the unit's MAW worker: once every part has written its dense pages'
    // log-masses and the top-k has arrived, the MAW update and the folded
    // append's writes.  It waits on workgroups of lower index only.
    const UG g = unit_geom(N, hi, c.dm);
    const bool no_sel = selects_nothing(hi, N, c.dm);
    const unsigned expected = (unsigned)unit_parts(g, P, c.dm) + (no_sel ? 0u : 1u);
    uint32_t *dctr = &c.sc.arrive[unit * 4 + 2];
    if (threadIdx.x == 0) {
      int ok = 1;
      const unsigned long long t0 = wall_clock64();
      while (ld_dev(dctr) < expected) {
        if (wall_clock64() - t0 > kWaitTicks) {
          st_dev(&c.sc.err[0], 1u);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      s_flag = ok;
    }
    __syncthreads();
    SD_TL(6);  // arrivals seen
    if (!s_flag) return;
    float *pm = reinterpret_cast<float *>(smem_raw);
    dense_maw<D, G>(c, seq, h, hi, g, new_tok(N), pm, pm + kFuseDenseLds,
                    pm + kFuseDenseLds + 4 * G);
    if (threadIdx.x == 0) st_dev(dctr, 0u);
    SD_TL(7);  // MAW updated
    return;
  }
  const UG g = unit_geom(N, hi, c.dm);
  const int PU = unit_parts(g, P, c.dm);
  if (idx >= PU) return;
  // attention part idx of the unit; the sequence's page table goes to LDS
  // for the selected pages
  int32_t *ptl = cdiv(g.N, kPage) <= ptl_cap
                     ? reinterpret_cast<int32_t *>(smem_raw + ((sizeof(AttLds<D, G>) + 15) & ~15))
                     : nullptr;
  if (idx == 0) empty_slots<D, G>(c, i, h, PU, p_cap, o_part, lse_part);
  // a unit that selects nothing has no score tiles: its parts take the dense
  // pages only and part 0 writes the count
  const bool no_sel = selects_nothing(hi, N, c.dm);
  if (no_sel && idx == 0 && threadIdx.x == 0) st_dev(&blk_cnt[(size_t)i * c.dm.Hkv + h], 0);
  SelIn si;
  si.tag = no_sel ? nullptr : c.sc.seltag + unit * c.dm.kcap;
  si.rtag = no_sel ? nullptr : &c.sc.rtag[unit];
  si.cnt = 0;
  si.epoch = epoch;
  attend_part<D, G>(c, i, seq, h, g, idx, PU, q, si, o_part, lse_part, p_cap, smem_att, ptl,
                    &s_cnt, new_tok(N), hi, &c.sc.arrive[unit * 4 + 2]);
  uint32_t *fctr = &c.sc.arrive[unit * 4 + 1];
  const bool last_part = arrive_last(fctr, (unsigned)PU, &s_flag);
  SD_TL(4);  // partial written, arrived
  if (!last_part) return;
  __builtin_amdgcn_s_setprio(3);
  fuse_unit<D, G>(c, i, h, PU, o_part, lse_part, p_cap, o, lse, smem_fuse);
  SD_TL(5);  // fused
  if (threadIdx.x == 0) st_dev(fctr, 0u);
}

// fuse, separate-call form: one workgroup per unit over the partial slots of
// its parts out of the attend call's P (layer call: the dense pages' masses
// from the attend call) or over every slot of p_cap (pure fusion).
template <int D, int G>
__global__ __launch_bounds__(256) void k_fuse(Ctx c, SeqBatch b, int with_maw, int P,
                                              const float *__restrict__ o_part,
                                              const float *__restrict__ lse_part, int p_cap,
                                              float *__restrict__ o, float *__restrict__ lse,
                                              const int32_t *__restrict__ sel_idx,
                                              const int32_t *__restrict__ sel_cnt, int k_cap) {
  __shared__ FuseSmem<G> sm;
  extern __shared__ __align__(16) float ablk[];  // the tables' block masses (lfps)
  const int h = blockIdx.x, i = blockIdx.y;
  const HeadInfo hi = c.heads[h];
  if (with_maw) {
    const UG g = unit_geom(b.len[i], hi, c.dm);
    fuse_unit<D, G>(c, i, h, unit_parts(g, P, c.dm), o_part, lse_part, p_cap, o, lse, sm);
    if (c.dm.lfps && g.N > 0) {
      const size_t row = (size_t)i * c.dm.Hkv + h;
      const int cnt = min(min(max(sel_cnt[row], 0), k_cap), hi.kcap);
      lfps_update_unit<D, G>(c, b.seq[i], h, hi, g, sel_idx + row * k_cap, cnt, sm.lse, ablk);
      __syncthreads();
    }
    dense_maw<D, G>(c, b.seq[i], h, hi, g, NewTok(), sm.pm, sm.dm, sm.dz);
  } else {
    fuse_unit<D, G>(c, i, h, p_cap, o_part, lse_part, p_cap, o, lse, sm);
  }
}

__global__ void k_fill_f32(float *p, size_t n, float v) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; idx < n; idx += (size_t)gridDim.x * blockDim.x) p[idx] = v;
}
__global__ void k_fill_u32(uint32_t *p, size_t n, uint32_t v) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; idx < n; idx += (size_t)gridDim.x * blockDim.x) p[idx] = v;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers

#define SD_DISPATCH_G(GG_VAR, ...)                        \
  switch (GG_VAR) {                                       \
    case 1: { constexpr int G_ = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int G_ = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int G_ = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int G_ = 4; __VA_ARGS__; } break; \
    case 5: { constexpr int G_ = 5; __VA_ARGS__; } break; \
    case 6: { constexpr int G_ = 6; __VA_ARGS__; } break; \
    case 7: { constexpr int G_ = 7; __VA_ARGS__; } break; \
    case 8: { constexpr int G_ = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                 \
  }

#define SD_DISPATCH_DG(DIM, GG_VAR, ...)   \
  if ((DIM) == 128) {                      \
    constexpr int D_ = 128;                \
    SD_DISPATCH_G(GG_VAR, __VA_ARGS__)     \
  } else {                                 \
    constexpr int D_ = 64;                 \
    SD_DISPATCH_G(GG_VAR, __VA_ARGS__)     \
  }

hipError_t launch_append(const Ctx &c, const AppendBatch &b, int max_new,
                         int max_touch_blocks, const uint16_t *k_new,
                         const uint16_t *v_new, hipStream_t st) {
  const int tpw = 16;
  const int n_scatter_x = max_new > 0 ? (max_new + tpw - 1) / tpw : 0;
  const int n_summ_x = max_new > 0 ? (max_touch_blocks * (c.dm.d / 4) + 255) / 256 : 0;
  const int grid = n_scatter_x * b.n + n_summ_x * c.dm.Hkv * b.n;
  if (grid == 0) return hipSuccess;
  if (c.dm.d == 128)
    hipLaunchKernelGGL(k_prep<128>, dim3(grid), dim3(256), 0, st, c, b, tpw, n_scatter_x,
                       n_summ_x, k_new, v_new);
  else
    hipLaunchKernelGGL(k_prep<64>, dim3(grid), dim3(256), 0, st, c, b, tpw, n_scatter_x,
                       n_summ_x, k_new, v_new);
  return hipGetLastError();
}

// top-k words past the register rows go to LDS while the launch stays within
// 64 KiB of LDS per workgroup, else to the global scratch
static int topk_lds(int max_blocks, size_t *bytes) {
  const int rows = max(1, (max_blocks + 63) / 64);
  const int extra = max(0, rows - kTopkRegRows) * 64;
  const size_t fixed = sizeof(TopkSmem) + sizeof(unsigned long long) * (size_t)max(rows, kTopkRegRows);
  const int lrows_words = fixed + sizeof(uint32_t) * (size_t)extra <= 65536 ? extra : 0;
  *bytes = fixed + sizeof(uint32_t) * (size_t)lrows_words;
  return lrows_words;
}

hipError_t launch_select(const Ctx &c, const SeqBatch &b, int max_blocks, const uint16_t *q,
                         int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  const int tiles_x = max(1, (b.max_scored + kScoreTile - 1) / kScoreTile);
  const int grid = tiles_x * c.dm.Hkv * b.n;
  size_t topk_bytes;
  const int lrows_words = topk_lds(max_blocks, &topk_bytes);
  if (topk_bytes > 65536) return hipErrorInvalidValue;
  SD_DISPATCH_DG(c.dm.d, c.dm.G, {
    hipLaunchKernelGGL((k_select<D_, G_>), dim3(grid), dim3(256), topk_bytes, st, c, b, tiles_x,
                       blk_idx, blk_cnt, k_cap, q, lrows_words);
    if (c.dm.pqh)
      hipLaunchKernelGGL((k_topk_heads<D_, G_>), dim3(G_ * c.dm.Hkv * b.n), dim3(256), topk_bytes,
                         st, c, b, blk_idx, blk_cnt, k_cap, q, lrows_words);
  });
  return hipGetLastError();
}

hipError_t launch_union(const Ctx &c, const SeqBatch &b, const int32_t *blk_idx,
                        const int32_t *blk_cnt, int32_t k_cap, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  const size_t lds = sizeof(uint32_t) * (size_t)max(1, (b.max_scored + 3) / 4);
  if (lds > 65536) return hipErrorInvalidValue;
  dim3 grid(c.dm.Hkv, b.n);
  SD_DISPATCH_G(c.dm.G, hipLaunchKernelGGL((k_union<G_>), grid, dim3(256), lds, st, c, b,
                                           blk_idx, blk_cnt, k_cap));
  return hipGetLastError();
}

hipError_t launch_attend(const Ctx &c, const SeqBatch &b, int P, const uint16_t *q,
                         const int32_t *blk_idx, const int32_t *blk_cnt, int32_t k_cap,
                         float *o_part, float *lse_part, int32_t p_cap, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  if (P < 1 || P > p_cap) return hipErrorInvalidValue;
  const int grid = P * c.dm.Hkv * b.n;
  SD_DISPATCH_DG(c.dm.d, c.dm.G,
                 hipLaunchKernelGGL((k_attend<D_, G_>), dim3(grid), dim3(256), 0, st, c, b, P,
                                    q, blk_idx, blk_cnt, k_cap, o_part, lse_part, p_cap));
  return hipGetLastError();
}

int step_capacity(const Ctx &c, int max_blocks, int ptl_cap) {
  size_t topk_bytes;
  topk_lds(max_blocks, &topk_bytes);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  hipError_t e = hipSuccess;
  SD_DISPATCH_DG(c.dm.d, c.dm.G, {
    const size_t att = ((sizeof(AttLds<D_, G_>) + 15) & ~size_t(15)) + sizeof(int32_t) * ptl_cap;
    const size_t smem = std::max(std::max(att, sizeof(FuseSmem<G_>)), topk_bytes);
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<D_, G_>, 256, smem);
  });
  return e == hipSuccess ? per_cu * cus : 0;
}

hipError_t launch_step(const Ctx &c, const SeqBatch &b, int max_blocks, int P, const uint16_t *q,
                       int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, float *o_part,
                       float *lse_part, int32_t p_cap, float *o, float *lse, uint32_t epoch,
                       int ptl_cap, const uint16_t *k_new, const uint16_t *v_new,
                       hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  if (P < 1 || P > p_cap) return hipErrorInvalidValue;
  const int tiles_x = max(1, (b.max_scored + kScoreTile - 1) / kScoreTile);
  const dim3 grid(c.dm.Hkv, b.n, tiles_x + P + 1);  // + the MAW workers
  size_t topk_bytes;
  const int lrows_words = topk_lds(max_blocks, &topk_bytes);
  if (topk_bytes > 65536) return hipErrorInvalidValue;
  SD_DISPATCH_DG(c.dm.d, c.dm.G, {
    const size_t att = ((sizeof(AttLds<D_, G_>) + 15) & ~size_t(15)) + sizeof(int32_t) * ptl_cap;
    const size_t smem = std::max(std::max(att, sizeof(FuseSmem<G_>)), topk_bytes);
    hipLaunchKernelGGL((k_step<D_, G_>), grid, dim3(256), smem, st, c, b, tiles_x, P,
                       blk_idx, blk_cnt, k_cap, q, o_part, lse_part, p_cap, o, lse, lrows_words,
                       epoch, ptl_cap, k_new, v_new);
  });
  return hipGetLastError();
}

hipError_t launch_fuse(const Ctx &c, const SeqBatch &b, bool with_maw, int P,
                       const float *o_part, const float *lse_part, int32_t p_cap,
                       float *o, float *lse, const int32_t *sel_idx, const int32_t *sel_cnt,
                       int32_t k_cap, int max_blocks, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  dim3 grid(c.dm.Hkv, b.n);
  const size_t lds = (with_maw && c.dm.lfps) ? sizeof(float) * (size_t)max(1, max_blocks) : 0;
  if (lds > 40960) return hipErrorInvalidValue;
  SD_DISPATCH_DG(c.dm.d, c.dm.G,
                 hipLaunchKernelGGL((k_fuse<D_, G_>), grid, dim3(256), lds, st, c, b,
                                    with_maw ? 1 : 0, P, o_part, lse_part, p_cap, o, lse,
                                    sel_idx, sel_cnt, k_cap));
  return hipGetLastError();
}

hipError_t launch_lfps_select(const Ctx &c, const SeqBatch &b, int max_blocks, const uint16_t *q,
                              int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, hipStream_t st) {
  if (b.n <= 0) return hipSuccess;
  const size_t lds = sizeof(LfpsSmem) + sizeof(uint32_t) * 2 * (size_t)((max_blocks + 31) / 32 + 1);
  if (lds > 65536) return hipErrorInvalidValue;
  // workgroups per unit: one per 512 blocks of the longest unit, at most 16
  // (units of up to 1024 blocks keep one)
  const int wpu = b.max_scored <= 1024 ? 1 : std::min(16, (b.max_scored + 511) / 512);
  SD_DISPATCH_DG(c.dm.d, c.dm.G,
                 hipLaunchKernelGGL((k_lfps_select<D_, G_>), dim3(c.dm.Hkv * b.n, wpu), dim3(256),
                                    lds, st, c, b, blk_idx, blk_cnt, k_cap, q));
  return hipGetLastError();
}

hipError_t launch_lfps_init(const Ctx &c, const SeqBatch &b, int max_blocks, const uint16_t *q_prefill,
                            int s_steps, float *A, hipStream_t st) {
  if (b.n <= 0 || s_steps <= 0) return hipSuccess;
  const size_t lds = sizeof(float) * (size_t)max(1, max_blocks);
  if (lds > 49152) return hipErrorInvalidValue;
  SD_DISPATCH_DG(c.dm.d, c.dm.G,
                 hipLaunchKernelGGL((k_lfps_init_mass<D_, G_>), dim3(s_steps, c.dm.Hkv, b.n),
                                    dim3(256), lds, st, c, b, q_prefill, s_steps, A));
  hipLaunchKernelGGL(k_lfps_init_tables, dim3(c.dm.Hkv, b.n), dim3(256), 0, st, c, b, s_steps, A);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
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

#ifdef SD_TIMELINE
// Copy of the step timeline (bytes <= kTlMaxWG * kTlSlots * 8) to host memory,
// then zeroed.  Declared in include/sparse_decode_timeline.h.
extern "C" int32_t sd_timeline_read(void *host_dst, size_t bytes, int32_t *slots,
                                    int32_t *max_wg) {
  if (slots) *slots = sd::kTlSlots;
  if (max_wg) *max_wg = sd::kTlMaxWG;
  const size_t all = sizeof(unsigned long long) * sd::kTlSlots * sd::kTlMaxWG;
  if (!host_dst || bytes > all) return SD_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(sd::sd_tl_buf), bytes) != hipSuccess)
    return SD_EHIP;
  static unsigned long long zeros[sd::kTlSlots * 1024];
  for (size_t off = 0; off < all; off += sizeof zeros)
    if (hipMemcpyToSymbol(HIP_SYMBOL(sd::sd_tl_buf), zeros, std::min(sizeof zeros, all - off), off) !=
        hipSuccess)
      return SD_EHIP;
  return SD_OK;
}
#endif
