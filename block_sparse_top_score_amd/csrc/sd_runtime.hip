// sd_runtime.hip - host runtime behind the C ABI of libsparse_decode.so:
// configuration checks, device allocation, per-layer page pools and page
// tables, per-call validation and kernel launches.  No exception crosses the
// ABI; every failure is a negative status plus a message in sd_last_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <vector>

#include "sd_internal.h"

using namespace sd;

// Scratch of the allocation-free step (sparse_decode_step_noalloc): one
// array per GPU, in the code object's device memory for as long as the
// process runs.  Host code never passes `scratch` itself to a kernel (its
// host-side name is a stand-in, not a device address): the device address is
// resolved once per device with hipGetSymbolAddress at context set-up and
// kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[SD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];    // device address of `scratch`, per device
hipError_t g_scratch_err[kMaxDevices];  // result of resolving it (hipSuccess once done)
bool g_scratch_tried[kMaxDevices];

// Where the allocation-free step keeps each scratch array inside `scratch`
// (byte offsets, 256-aligned).  The arrays that must start each call at zero
// (arrival counters, score accumulators, selection hand-off tags) come first,
// so one fill clears them.
struct StaticLayout {
  size_t arrive, unit_acc, rtag, seltag, clear_bytes;
  size_t keyflag, cand, keys, ulist, ukeys, lm_pg, total;
};

struct Layer {
  LayerDev dev{};
  int32_t *h_pt = nullptr;           // pinned host mirror of the page table
  std::vector<int32_t> len;          // tokens per sequence
  std::vector<int32_t> free_pages;   // stack; back() is handed out next
};

}  // namespace

struct sd_ctx {
  sd_config cfg{};
  std::vector<int32_t> S, ppm;
  int D = 0, Hq = 0, Hkv = 0, G = 0, pps = 0, max_S = 0;
  bool pqh = false;  // one selection per query head
  bool lfps = false;  // selection among the learn-from-the-past table candidates
  // the selection the last attend call took (the table update reads it)
  const int32_t *pend_idx = nullptr, *pend_cnt = nullptr;
  int32_t pend_kcap = 0;
  int sel_rows = 0;  // selections per sequence: Hq with pqh, else Hkv
  hipStream_t stream = nullptr;
  int device = 0;
  std::vector<HeadInfo> heads;
  HeadInfo *d_heads = nullptr;
  Dims dims{};
  Scratch sc{};
  std::vector<Layer> layers;
  int32_t k_cap = 0, p_cap = 0;
  uint32_t epoch = 0;  // step launches so far (never 0 once used)
  // attend -> fuse hand-over state
  int pend_layer = -2;
  std::vector<int32_t> pend_seqs;
  int32_t pend_pcap = 0;
  std::vector<int> pend_parts;  // P of each launch of the attend call
  // resident step workgroups by max_blocks (a fixed table: no allocation
  // after init)
  int cap_key[16] = {}, cap_val[16] = {}, n_cap = 0;
  std::vector<uint8_t> seen;     // [max_seqs] duplicate-id check, all 0 between calls
  void *static_scratch = nullptr;  // device address of `scratch` on this device
  StaticLayout slayout{};
  char err[512] = {};
  std::vector<void *> dev_allocs;
};

namespace {

sd_status fail(sd_ctx *c, sd_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) snprintf(c->err, sizeof c->err, "%s", buf);
  return st;
}

#define SD_HIP(ctx, call)                                                    \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess)                                                    \
      return fail(ctx, SD_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// k for a sequence of N tokens on head h (budget as parts per million of N,
// whole blocks, capped by the number of candidate blocks).
int64_t n_candidates(int64_t N, int S, int n_s, int W) {
  // blocks entirely inside the sinks: floor(ns/S); entirely inside the
  // window: n_blk - ceil(wlo/S); the rest hold a token outside D.
  int64_t ns = std::min<int64_t>(n_s, N), wlo = std::max<int64_t>(0, N - W);
  if (ns >= wlo) return 0;
  return cdiv(wlo, S) - ns / S;
}

int64_t k_of(int64_t N, int S, int ppm, int n_s, int W) {
  int64_t den = 1000000LL * S;
  int64_t k = (int64_t(ppm) * N + den - 1) / den;
  return std::min(k, n_candidates(N, S, n_s, W));
}

// splitmix64: seeded permutation of the free list.
uint64_t splitmix64(uint64_t &x) {
  uint64_t z = (x += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <class T>
sd_status dev_alloc(sd_ctx *c, T **p, size_t count) {
  *p = nullptr;
  if (count == 0) count = 1;
  hipError_t e = hipMalloc(reinterpret_cast<void **>(p), count * sizeof(T));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, SD_ENOMEM, "hipMalloc of %zu bytes failed: %s",
                count * sizeof(T), hipGetErrorString(e));
  }
  c->dev_allocs.push_back(*p);
  return SD_OK;
}

void free_all(sd_ctx *c) {
  for (void *p : c->dev_allocs) (void)hipFree(p);
  c->dev_allocs.clear();
  for (auto &L : c->layers)
    if (L.h_pt) (void)hipHostFree(L.h_pt);
  c->layers.clear();
}

// Sequence arguments shared by the decode calls.
sd_status check_seqs(sd_ctx *c, int32_t layer, int32_t n_seqs,
                     const int32_t *seq_ids) {
  if (layer < 0 || layer >= c->cfg.num_layers)
    return fail(c, SD_EINVAL, "layer %d out of range [0,%d)", layer,
                c->cfg.num_layers);
  if (n_seqs < 0) return fail(c, SD_EINVAL, "n_seqs %d < 0", n_seqs);
  if (n_seqs > 0 && !seq_ids) return fail(c, SD_EINVAL, "seq_ids is NULL");
  // c->seen is all zero between calls; the ids marked here are cleared again
  sd_status st = SD_OK;
  int i = 0;
  for (; i < n_seqs; ++i) {
    int s = seq_ids[i];
    if (s < 0 || s >= c->cfg.max_seqs) {
      st = fail(c, SD_EINVAL, "seq_ids[%d]=%d out of range [0,%d)", i, s, c->cfg.max_seqs);
      break;
    }
    if (c->seen[s]) {
      st = fail(c, SD_EINVAL, "seq id %d repeated in one call", s);
      break;
    }
    c->seen[s] = 1;
  }
  for (int j = 0; j < i; ++j) c->seen[seq_ids[j]] = 0;
  return st;
}

void fill_batch(const sd_ctx *c, int layer, const int32_t *seq_ids, int base,
                int n, SeqBatch *b, int *max_blocks) {
  b->n = n;
  int mb = 0, ms = 0;
  const int W = c->cfg.recent_window;
  for (int i = 0; i < n; ++i) {
    b->seq[i] = seq_ids[base + i];
    b->len[i] = c->layers[layer].len[seq_ids[base + i]];
    for (int h = 0; h < c->Hkv; ++h) {
      const int nb = (int)cdiv(b->len[i], c->S[h]);
      mb = std::max(mb, nb);
      // blocks from ceil((N - W) / S) on lie wholly in the recent window
      const int sc = (W > 0 && b->len[i] > 0)
                         ? std::min<int>(nb, (int)cdiv(std::max(0, b->len[i] - W), c->S[h]))
                         : nb;
      ms = std::max(ms, sc);
    }
  }
  b->max_scored = ms;
  if (max_blocks) *max_blocks = mb;
}

__attribute__((format(printf, 3, 4))) void report(char *err, size_t err_len,
                                                  const char *fmt, ...) {
  if (!err || !err_len) return;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(err, err_len, fmt, ap);
  va_end(ap);
}

}  // namespace

// ---------------------------------------------------------------------------
extern "C" {

sd_status sd_validate_config(const sd_config *cfg, char *err, size_t err_len) {
#define bad(...) (report(err, err_len, __VA_ARGS__), SD_EINVAL)
  if (!cfg) return bad("config is NULL");
  if (cfg->max_seqs < 1) return bad("max_seqs %d < 1", cfg->max_seqs);
  if (cfg->num_layers < 1) return bad("num_layers %d < 1", cfg->num_layers);
  if (cfg->num_kv_heads < 1 || cfg->num_kv_heads > SD_MAX_KV_HEADS)
    return bad("num_kv_heads %d outside [1,%d]", cfg->num_kv_heads, SD_MAX_KV_HEADS);
  if (cfg->num_q_heads < 1 || cfg->num_q_heads % cfg->num_kv_heads != 0)
    return bad("num_q_heads %d is not a positive multiple of num_kv_heads %d",
               cfg->num_q_heads, cfg->num_kv_heads);
  if (cfg->num_q_heads / cfg->num_kv_heads > SD_MAX_GROUP)
    return bad("group size %d > %d", cfg->num_q_heads / cfg->num_kv_heads,
               SD_MAX_GROUP);
  if (cfg->head_dim != 64 && cfg->head_dim != 128)
    return bad("head_dim %d not in {64,128}", cfg->head_dim);
  if (cfg->page_size != SD_PAGE_SIZE)
    return bad("page_size %d != %d", cfg->page_size, SD_PAGE_SIZE);
  if (cfg->num_pages < 1) return bad("num_pages %d < 1", cfg->num_pages);
  if (cfg->max_seq_len < 1) return bad("max_seq_len %d < 1", cfg->max_seq_len);
  if (cfg->sink_tokens < 0) return bad("sink_tokens %d < 0", cfg->sink_tokens);
  if (cfg->recent_window < 0) return bad("recent_window %d < 0", cfg->recent_window);
  if (!cfg->block_size || !cfg->budget_ppm)
    return bad("block_size / budget_ppm arrays are NULL");
  for (int h = 0; h < cfg->num_kv_heads; ++h) {
    int S = cfg->block_size[h];
    if (S < SD_PAGE_SIZE || S > SD_MAX_BLOCK || S % SD_PAGE_SIZE != 0)
      return bad("block_size[%d]=%d is not a multiple of %d in [%d,%d]", h, S,
                 SD_PAGE_SIZE, SD_PAGE_SIZE, SD_MAX_BLOCK);
    if (cfg->budget_ppm[h] < 0 || cfg->budget_ppm[h] > 1000000)
      return bad("budget_ppm[%d]=%d outside [0,1000000]", h, cfg->budget_ppm[h]);
  }
  if (!(cfg->softmax_scale >= 0.0f) || std::isinf(cfg->softmax_scale))
    return bad("softmax_scale must be finite and >= 0");
  if (!(cfg->maw_decay >= 0.0f && cfg->maw_decay < 1.0f))
    return bad("maw_decay %g outside [0,1)", (double)cfg->maw_decay);
  if (std::isnan(cfg->maw_beta) || std::isinf(cfg->maw_beta))
    return bad("maw_beta must be finite");
  if (cfg->select_per_query_head != 0 && cfg->select_per_query_head != 1)
    return bad("select_per_query_head %d not in {0,1}", cfg->select_per_query_head);
  if (cfg->lfps_select != 0 && cfg->lfps_select != 1)
    return bad("lfps_select %d not in {0,1}", cfg->lfps_select);
  if (cfg->lfps_select) {
    if (!(cfg->lfps_a >= 0.0f && cfg->lfps_a <= 1.0f))
      return bad("lfps_a %g outside [0,1]", (double)cfg->lfps_a);
    if (cfg->maw_beta > 0.0f) return bad("lfps_select ranks no MAW flags: maw_beta must be <= 0");
    if (cfg->select_per_query_head) return bad("lfps_select selects per KV head");
  }
  if (err && err_len) err[0] = 0;
  return SD_OK;
#undef bad
}

sd_status sparse_decode_init(const sd_config *cfg, sd_ctx **out) {
  if (!out) return SD_EINVAL;
  *out = nullptr;
  char msg[256];
  sd_status st = sd_validate_config(cfg, msg, sizeof msg);
  sd_ctx *c = new (std::nothrow) sd_ctx();
  if (!c) return SD_ENOMEM;
  if (st != SD_OK) {
    snprintf(c->err, sizeof c->err, "%s", msg);
    *out = c;  // caller can read the message, then destroy
    return st;
  }
  c->cfg = *cfg;
  c->Hq = cfg->num_q_heads;
  c->Hkv = cfg->num_kv_heads;
  c->G = c->Hq / c->Hkv;
  c->pqh = cfg->select_per_query_head == 1;
  c->lfps = cfg->lfps_select == 1;
  c->sel_rows = c->pqh ? c->Hq : c->Hkv;
  c->D = cfg->head_dim;
  c->pps = (int)cdiv(cfg->max_seq_len, kPage);
  c->S.assign(cfg->block_size, cfg->block_size + c->Hkv);
  c->max_S = *std::max_element(c->S.begin(), c->S.end());
  c->ppm.assign(cfg->budget_ppm, cfg->budget_ppm + c->Hkv);
  c->cfg.block_size = nullptr;
  c->cfg.budget_ppm = nullptr;
  c->stream = reinterpret_cast<hipStream_t>(cfg->stream);
  *out = c;
  if (hipGetDevice(&c->device) != hipSuccess)
    return fail(c, SD_EHIP, "no HIP device");

  const int max_seqs = cfg->max_seqs;
  // per-head geometry and capacities.  The attended pages of a unit: at most
  // lm_sel0 pages with dense tokens, then kcap * S / 16 pages of selected
  // blocks; partial slots: one per attention workgroup, P <= p_cap.
  c->heads.resize(c->Hkv);
  int64_t summ_elems = 0, maw_elems = 0;
  int key_stride = 1, sel_pages = 1;
  int64_t ucap = 1;
  const int lm_sel0 = (int)(cdiv(cfg->sink_tokens, kPage) + cdiv(cfg->recent_window, kPage) + 1);
  for (int h = 0; h < c->Hkv; ++h) {
    HeadInfo &hi = c->heads[h];
    hi.S = c->S[h];
    hi.ppm = c->ppm[h];
    hi.nbmax = (int)cdiv(cfg->max_seq_len, hi.S);
    hi.summ_off = summ_elems;
    hi.maw_off = maw_elems;
    summ_elems += (int64_t)max_seqs * (c->D / 4) * hi.nbmax * 8;
    maw_elems += (int64_t)max_seqs * hi.nbmax;
    key_stride = std::max(key_stride, hi.nbmax);
    // k grows with N: its largest value is at max_seq_len
    int64_t kc = std::min<int64_t>(cdiv((int64_t)hi.ppm * cfg->max_seq_len, 1000000LL * hi.S),
                                   hi.nbmax);
    hi.kcap = (int)std::max<int64_t>(kc, 1);
    // with one set per query head the attention reads the group's union
    const int64_t ku = c->pqh ? std::min<int64_t>((int64_t)c->G * hi.kcap, hi.nbmax) : hi.kcap;
    ucap = std::max<int64_t>(ucap, ku);
    const int spg = (int)ku * (hi.S / kPage);
    sel_pages = std::max(sel_pages, spg);
    c->k_cap = std::max(c->k_cap, hi.kcap);
    c->p_cap = std::max<int32_t>(c->p_cap, (int32_t)std::max<int64_t>(1, cdiv(lm_sel0 + spg, kPartPages)));
  }

  if (c->p_cap > kFuseSlots)
    return fail(c, SD_EUNSUPPORTED,
                "%d partial slots per head exceed the fusion limit %d (lower the budget "
                "or max_seq_len, or raise the block size)", c->p_cap, kFuseSlots);
  if (lm_sel0 > kFuseDenseLds)
    return fail(c, SD_EUNSUPPORTED,
                "sinks %d + recent window %d span up to %d pages, more than the %d the fusion "
                "holds", cfg->sink_tokens, cfg->recent_window, lm_sel0, kFuseDenseLds);
  sd_status s;
  if ((s = dev_alloc(c, &c->d_heads, c->Hkv)) != SD_OK) return s;
  SD_HIP(c, hipMemcpy(c->d_heads, c->heads.data(), sizeof(HeadInfo) * c->Hkv,
                      hipMemcpyHostToDevice));

  c->dims.Hq = c->Hq;
  c->dims.Hkv = c->Hkv;
  c->dims.G = c->G;
  c->dims.d = c->D;
  c->dims.pages_per_seq = c->pps;
  c->dims.n_sink = cfg->sink_tokens;
  c->dims.window = cfg->recent_window;
  float scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale
                                          : (float)(1.0 / std::sqrt((double)c->D));
  c->dims.scale_log2 = (float)((double)scale * 1.4426950408889634);
  c->dims.maw_decay = cfg->maw_decay > 0.0f ? cfg->maw_decay : 0.95f;
  c->dims.maw_beta = cfg->maw_beta;
  // whole groups of 256 blocks: the keys of a unit that the four-wave top-k
  // ranks are stored 256 apart (thread-transposed)
  key_stride = (int)cdiv(key_stride, 256) * 256;
  c->dims.key_stride = key_stride;
  c->dims.lm_sel0 = lm_sel0;
  // the dense pages' log-masses (MAW's input); with the tables also the
  // selected pages'
  c->dims.lm_cap = c->lfps ? lm_sel0 + sel_pages : lm_sel0;
  c->dims.kcap = c->k_cap;
  c->dims.pqh = c->pqh ? 1 : 0;
  c->dims.ucap = (int32_t)ucap;
  c->dims.lfps = c->lfps ? 1 : 0;
  c->dims.lfps_a = cfg->lfps_a;

  // scratch (the selection's per-unit arrays are per query head with one
  // set per query head)
  const size_t per_unit = (size_t)max_seqs * c->Hkv * key_stride;
  const size_t per_sel = (size_t)max_seqs * c->sel_rows * key_stride;
  if ((s = dev_alloc(c, &c->sc.keys, per_sel)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.keyflag, per_sel)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.ulist, per_sel)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.ukeys, per_sel)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.unit_acc, (size_t)max_seqs * c->sel_rows * 4)) != SD_OK) return s;
  SD_HIP(c, hipMemset(c->sc.unit_acc, 0, sizeof(uint32_t) * max_seqs * c->sel_rows * 4));
  if (c->pqh) {
    if ((s = dev_alloc(c, &c->sc.uni, (size_t)max_seqs * c->Hkv * ucap)) != SD_OK) return s;
    if ((s = dev_alloc(c, &c->sc.ucnt, (size_t)max_seqs * c->Hkv)) != SD_OK) return s;
  }
  if ((s = dev_alloc(c, &c->sc.lm_pg, (size_t)max_seqs * c->Hq * c->dims.lm_cap)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.arrive, (size_t)max_seqs * c->Hkv * 4)) != SD_OK) return s;
  SD_HIP(c, hipMemset(c->sc.arrive, 0, sizeof(uint32_t) * max_seqs * c->Hkv * 4));
  if ((s = dev_alloc(c, &c->sc.cand, per_unit)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.rtag, (size_t)max_seqs * c->Hkv)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.seltag, (size_t)max_seqs * c->Hkv * c->k_cap)) != SD_OK) return s;
  if ((s = dev_alloc(c, &c->sc.err, 1)) != SD_OK) return s;
  SD_HIP(c, hipMemset(c->sc.rtag, 0, sizeof(unsigned long long) * max_seqs * c->Hkv));
  SD_HIP(c, hipMemset(c->sc.seltag, 0, sizeof(unsigned long long) * max_seqs * c->Hkv * c->k_cap));
  SD_HIP(c, hipMemset(c->sc.err, 0, sizeof(uint32_t)));

  c->seen.assign(max_seqs, 0);

  // layout of the allocation-free step's scratch inside `scratch`, and the
  // array's device address on this device (resolved once per device)
  {
    const size_t units = (size_t)max_seqs * c->Hkv;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
      const size_t at = off;
      off = (off + bytes + 255) & ~size_t(255);
      return at;
    };
    StaticLayout &sl = c->slayout;
    sl.arrive = take(sizeof(uint32_t) * units * 4);
    sl.unit_acc = take(sizeof(uint32_t) * units * 4);
    sl.rtag = take(sizeof(unsigned long long) * units);
    sl.seltag = take(sizeof(unsigned long long) * units * c->k_cap);
    sl.clear_bytes = off;
    sl.keyflag = take(sizeof(unsigned long long) * per_unit);
    sl.cand = take(sizeof(unsigned long long) * per_unit);
    sl.keys = take(sizeof(uint32_t) * per_unit);
    sl.ulist = take(sizeof(int32_t) * per_unit);
    sl.ukeys = take(sizeof(uint32_t) * per_unit);
    sl.lm_pg = take(sizeof(float) * (size_t)max_seqs * c->Hq * c->dims.lm_cap);
    sl.total = off;
    if (c->device >= 0 && c->device < kMaxDevices) {
      std::lock_guard<std::mutex> lock(g_scratch_mu);
      if (!g_scratch_tried[c->device]) {
        void *ptr = nullptr;
        g_scratch_err[c->device] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (g_scratch_err[c->device] != hipSuccess) (void)hipGetLastError();
        g_scratch_dev[c->device] = g_scratch_err[c->device] == hipSuccess ? ptr : nullptr;
        g_scratch_tried[c->device] = true;
      }
      c->static_scratch = g_scratch_dev[c->device];
    }
  }

  // layers
  c->layers.resize(cfg->num_layers);
  const size_t pool = (size_t)cfg->num_pages * c->Hkv * kPage * c->D;
  for (int l = 0; l < cfg->num_layers; ++l) {
    Layer &L = c->layers[l];
    if ((s = dev_alloc(c, &L.dev.k, pool)) != SD_OK) return s;
    if ((s = dev_alloc(c, &L.dev.v, pool)) != SD_OK) return s;
    if ((s = dev_alloc(c, &L.dev.pt, (size_t)max_seqs * c->pps)) != SD_OK) return s;
    if ((s = dev_alloc(c, &L.dev.summ, (size_t)summ_elems)) != SD_OK) return s;
    if ((s = dev_alloc(c, &L.dev.maw, (size_t)maw_elems)) != SD_OK) return s;
    if (c->lfps) {
      if ((s = dev_alloc(c, &L.dev.phi, (size_t)maw_elems * 2)) != SD_OK) return s;
      SD_HIP(c, hipMemset(L.dev.phi, 0, sizeof(float) * maw_elems * 2));
    }
    SD_HIP(c, hipMemset(L.dev.pt, 0, sizeof(int32_t) * max_seqs * c->pps));
    SD_HIP(c, hipMemset(L.dev.maw, 0, sizeof(float) * maw_elems));
    SD_HIP(c, hipMemset(L.dev.summ, 0, sizeof(uint16_t) * summ_elems));
    hipError_t e = hipHostMalloc(reinterpret_cast<void **>(&L.h_pt),
                                 sizeof(int32_t) * max_seqs * c->pps, hipHostMallocDefault);
    if (e != hipSuccess) return fail(c, SD_ENOMEM, "hipHostMalloc failed");
    std::fill(L.h_pt, L.h_pt + (size_t)max_seqs * c->pps, 0);
    L.len.assign(max_seqs, 0);
    L.free_pages.resize(cfg->num_pages);
    // back() is handed out first: page 0, 1, 2, ... in order
    for (int p = 0; p < cfg->num_pages; ++p) L.free_pages[p] = cfg->num_pages - 1 - p;
    if (cfg->page_shuffle_seed) {
      uint64_t st64 = cfg->page_shuffle_seed * 0x100000001B3ull + (uint64_t)l;
      for (int p = cfg->num_pages - 1; p > 0; --p) {
        int j = (int)(splitmix64(st64) % (uint64_t)(p + 1));
        std::swap(L.free_pages[p], L.free_pages[j]);
      }
    }
  }
  SD_HIP(c, hipDeviceSynchronize());
  return SD_OK;
}

sd_status sparse_decode_destroy(sd_ctx *c) {
  if (!c) return SD_EINVAL;
  sd_status st = SD_OK;
  if (!c->dev_allocs.empty() && hipStreamSynchronize(c->stream) != hipSuccess)
    st = SD_EHIP;
  free_all(c);
  delete c;
  return st;
}

sd_status sd_caps(const sd_ctx *c, int32_t *k_cap, int32_t *p_cap) {
  if (!c) return SD_EINVAL;
  if (k_cap) *k_cap = c->k_cap;
  if (p_cap) *p_cap = c->p_cap;
  return SD_OK;
}

const char *sd_last_error(const sd_ctx *c) {
  if (!c) return "null context";
  return c->err;
}

sd_status sd_sync(sd_ctx *c) {
  if (!c) return SD_EINVAL;
  SD_HIP(c, hipStreamSynchronize(c->stream));
  uint32_t e = 0;
  SD_HIP(c, hipMemcpy(&e, c->sc.err, sizeof e, hipMemcpyDeviceToHost));
  if (e) {
    // a wait gave up: the hand-off counters may be left part-way; they start
    // from zero again for the next call
    SD_HIP(c, hipMemset(c->sc.err, 0, sizeof e));
    SD_HIP(c, hipMemset(c->sc.arrive, 0, sizeof(uint32_t) * c->cfg.max_seqs * c->Hkv * 4));
    SD_HIP(c, hipMemset(c->sc.unit_acc, 0, sizeof(uint32_t) * c->cfg.max_seqs * c->sel_rows * 4));
    return fail(c, SD_EHIP, "a decode step kernel timed out waiting for a unit's selection; "
                "its outputs are invalid");
  }
  return SD_OK;
}

sd_status sd_seq_len(const sd_ctx *c, int32_t layer, int32_t seq, int32_t *len) {
  if (!c || !len) return SD_EINVAL;
  if (layer < 0 || layer >= c->cfg.num_layers || seq < 0 || seq >= c->cfg.max_seqs)
    return SD_EINVAL;
  *len = c->layers[layer].len[seq];
  return SD_OK;
}

namespace {

Ctx kctx(const sd_ctx *c, int layer) {
  Ctx k{};
  if (layer >= 0) k.L = c->layers[layer].dev;
  k.heads = c->d_heads;
  k.dm = c->dims;
  k.sc = c->sc;
  return k;
}

// Host-side append: validate, take pages, push the touched page-table span,
// then (launch) the append kernel.  n_new == NULL: one token per sequence.
// Without launch the caller's step kernel writes the tokens and summaries.
sd_status do_append(sd_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                    const int32_t *n_new_arr, const void *k_bf16, const void *v_bf16,
                    bool launch = true) {
  Layer &L = c->layers[layer];
  auto n_new = [n_new_arr](int i) { return n_new_arr ? n_new_arr[i] : 1; };
  int64_t total = 0, pages_needed = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (n_new(i) < 0) return fail(c, SD_EINVAL, "n_new[%d]=%d < 0", i, n_new(i));
    int64_t nl = (int64_t)L.len[seq_ids[i]] + n_new(i);
    if (nl > c->cfg.max_seq_len)
      return fail(c, SD_EINVAL, "sequence %d would hold %lld tokens > max_seq_len %d",
                  seq_ids[i], (long long)nl, c->cfg.max_seq_len);
    total += n_new(i);
    pages_needed += cdiv(nl, kPage) - cdiv(L.len[seq_ids[i]], kPage);
  }
  if (total > 0 && (!k_bf16 || !v_bf16)) return fail(c, SD_EINVAL, "k/v pointers are NULL");
  if (total > 0 && (reinterpret_cast<uintptr_t>(k_bf16) % 16 != 0 ||
                    reinterpret_cast<uintptr_t>(v_bf16) % 16 != 0))
    return fail(c, SD_EINVAL, "k/v rows must be 16-byte aligned");
  if (pages_needed > (int64_t)L.free_pages.size())
    return fail(c, SD_ENOMEM, "page pool of layer %d exhausted: need %lld pages, %zu free",
                layer, (long long)pages_needed, L.free_pages.size());
  int64_t lo = INT64_MAX, hi = -1;
  for (int i = 0; i < n_seqs; ++i) {
    int seq = seq_ids[i];
    int64_t p0 = cdiv(L.len[seq], kPage), p1 = cdiv((int64_t)L.len[seq] + n_new(i), kPage);
    for (int64_t p = p0; p < p1; ++p) {
      L.h_pt[(size_t)seq * c->pps + p] = L.free_pages.back();
      L.free_pages.pop_back();
      lo = std::min<int64_t>(lo, (int64_t)seq * c->pps + p);
      hi = std::max<int64_t>(hi, (int64_t)seq * c->pps + p);
    }
  }
  if (hi >= 0)
    SD_HIP(c, hipMemcpyAsync(L.dev.pt + lo, L.h_pt + lo, sizeof(int32_t) * (hi - lo + 1),
                             hipMemcpyHostToDevice, c->stream));
  const Ctx kc = kctx(c, layer);
  int row = 0;
  for (int base = 0; launch && base < n_seqs; base += kLaunchSeqs) {
    AppendBatch b{};
    b.n = std::min(kLaunchSeqs, n_seqs - base);
    int max_new = 0, max_touch = 0;
    for (int i = 0; i < b.n; ++i) {
      int seq = seq_ids[base + i];
      b.seq[i] = seq;
      b.old_len[i] = L.len[seq];
      b.n_new[i] = n_new(base + i);
      b.src_row[i] = row;
      row += n_new(base + i);
      max_new = std::max(max_new, b.n_new[i]);
      if (b.n_new[i] > 0)
        for (int h = 0; h < c->Hkv; ++h) {
          int S = c->S[h];
          int t = (b.old_len[i] + b.n_new[i] - 1) / S - b.old_len[i] / S + 1;
          max_touch = std::max(max_touch, t);
        }
    }
    SD_HIP(c, launch_append(kc, b, max_new, max_touch, static_cast<const uint16_t *>(k_bf16),
                            static_cast<const uint16_t *>(v_bf16), c->stream));
  }
  for (int i = 0; i < n_seqs; ++i) L.len[seq_ids[i]] += n_new(i);
  return SD_OK;
}

int64_t k_of_seq(const sd_ctx *c, int64_t N, int h) {
  return k_of(N, c->S[h], c->ppm[h], c->cfg.sink_tokens, c->cfg.recent_window);
}

// Pages holding dense tokens (sinks, recent window) of a sequence of N tokens.
int64_t dense_pages(const sd_ctx *c, int64_t N) {
  const int64_t np = cdiv(N, kPage);
  const int64_t sp = cdiv(std::min<int64_t>(c->cfg.sink_tokens, N), kPage);
  const int64_t wlo = std::max<int64_t>(0, N - c->cfg.recent_window);
  const int64_t wp = wlo < N ? std::max<int64_t>(sp, wlo / kPage) : np;
  return sp + (np - wp);
}

// Attention workgroups per unit of one launch: about kPartPages attended
// pages each, for the unit with the most; fewer if the one-launch step would
// otherwise not fit on the device at once (a part that starts late finishes
// late).  The separate calls use the same P, so both give the same bits.
int parts_of(sd_ctx *c, int layer, const SeqBatch &b, int max_blocks) {
  int64_t P = 1;
  for (int i = 0; i < b.n; ++i)
    for (int h = 0; h < c->Hkv; ++h) {
      int64_t kb = k_of_seq(c, b.len[i], h);
      if (c->pqh)  // the union of the group's sets
        kb = std::min<int64_t>(kb * c->G, n_candidates(b.len[i], c->S[h], c->cfg.sink_tokens,
                                                       c->cfg.recent_window));
      const int64_t pages = dense_pages(c, b.len[i]) + kb * (c->S[h] / kPage);
      P = std::max<int64_t>(P, cdiv(pages, kPartPages));
    }
  int cap = -1;
  for (int t = 0; t < c->n_cap; ++t)
    if (c->cap_key[t] == max_blocks) cap = c->cap_val[t];
  if (cap < 0) {
    cap = step_capacity(kctx(c, layer), max_blocks, c->pps <= kPtLds ? c->pps : 0);
    if (c->n_cap < 16) {
      c->cap_key[c->n_cap] = max_blocks;
      c->cap_val[c->n_cap++] = cap;
    }
  }
  const int units = c->Hkv * b.n;
  const int tiles = std::max(1, (b.max_scored + kScoreTile - 1) / kScoreTile);
  // fewer parts, so that the whole step stays resident, pays when it costs
  // at most half of them; otherwise (long units, many tiles) the parts that do
  // not fit start as score tiles finish
  const int64_t resident = cap > 0 ? cap / units - tiles : P;
  if (2 * resident >= P) P = std::min<int64_t>(P, std::max<int64_t>(1, resident));
  return (int)std::min<int64_t>(P, c->p_cap);
}

sd_status check_kcap(sd_ctx *c, int layer, int n_seqs, const int32_t *seq_ids, int32_t k_cap) {
  const Layer &L = c->layers[layer];
  for (int i = 0; i < n_seqs; ++i)
    for (int h = 0; h < c->Hkv; ++h) {
      int64_t k = k_of_seq(c, L.len[seq_ids[i]], h);
      if (k > k_cap)
        return fail(c, SD_EINVAL, "k_cap %d < %lld blocks needed (seq %d, kv head %d)",
                    k_cap, (long long)k, seq_ids[i], h);
    }
  return SD_OK;
}

}  // namespace

sd_status append_kv(sd_ctx *c, int32_t layer, int32_t n_seqs,
                    const int32_t *seq_ids, const int32_t *n_new,
                    const void *k_bf16, const void *v_bf16) {
  if (!c) return SD_EINVAL;
  sd_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != SD_OK) return s;
  if (n_seqs > 0 && !n_new) return fail(c, SD_EINVAL, "n_new is NULL");
  return do_append(c, layer, n_seqs, seq_ids, n_new, k_bf16, v_bf16);
}

sd_status select_topk(sd_ctx *c, int32_t layer, int32_t n_seqs,
                      const int32_t *seq_ids, const void *q_bf16,
                      int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap) {
  if (!c) return SD_EINVAL;
  sd_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != SD_OK) return s;
  if (n_seqs == 0) return SD_OK;
  if (!q_bf16 || !blk_idx || !blk_cnt)
    return fail(c, SD_EINVAL, "q / blk_idx / blk_cnt pointer is NULL");
  if ((s = check_kcap(c, layer, n_seqs, seq_ids, k_cap)) != SD_OK) return s;
  const Ctx kc = kctx(c, layer);
  const uint16_t *q = static_cast<const uint16_t *>(q_bf16);
  for (int base = 0; base < n_seqs; base += kLaunchSeqs) {
    SeqBatch b;
    int mb = 0;
    fill_batch(c, layer, seq_ids, base, std::min(kLaunchSeqs, n_seqs - base), &b, &mb);
    const uint16_t *qb = q + (size_t)base * c->Hq * c->D;
    if (c->lfps)
      SD_HIP(c, launch_lfps_select(kc, b, mb, qb, blk_idx + (size_t)base * c->Hkv * k_cap,
                                   blk_cnt + (size_t)base * c->Hkv, k_cap, c->stream));
    else
      SD_HIP(c, launch_select(kc, b, mb, qb, blk_idx + (size_t)base * c->sel_rows * k_cap,
                              blk_cnt + (size_t)base * c->sel_rows, k_cap, c->stream));
  }
  return SD_OK;
}

sd_status sparse_attend(sd_ctx *c, int32_t layer, int32_t n_seqs,
                        const int32_t *seq_ids, const void *q_bf16,
                        const int32_t *blk_idx, const int32_t *blk_cnt,
                        int32_t k_cap, float *o_part, float *lse_part,
                        int32_t p_cap) {
  if (!c) return SD_EINVAL;
  sd_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != SD_OK) return s;
  if (n_seqs == 0) return SD_OK;
  if (!q_bf16 || !blk_idx || !blk_cnt || !o_part || !lse_part)
    return fail(c, SD_EINVAL, "a device pointer is NULL");
  if (k_cap < 1) return fail(c, SD_EINVAL, "k_cap %d < 1", k_cap);
  if (p_cap < c->p_cap)
    return fail(c, SD_EINVAL, "p_cap %d < %d partial slots per head (sd_caps)", p_cap, c->p_cap);
  const Ctx kc = kctx(c, layer);
  const uint16_t *q = static_cast<const uint16_t *>(q_bf16);
  c->pend_parts.clear();
  for (int base = 0; base < n_seqs; base += kLaunchSeqs) {
    SeqBatch b;
    int mb = 0;
    fill_batch(c, layer, seq_ids, base, std::min(kLaunchSeqs, n_seqs - base), &b, &mb);
    const int P = parts_of(c, layer, b, mb);
    c->pend_parts.push_back(P);
    if (c->pqh)
      SD_HIP(c, launch_union(kc, b, blk_idx + (size_t)base * c->sel_rows * k_cap,
                             blk_cnt + (size_t)base * c->sel_rows, k_cap, c->stream));
    SD_HIP(c, launch_attend(kc, b, P, q + (size_t)base * c->Hq * c->D,
                            blk_idx + (size_t)base * c->sel_rows * k_cap,
                            blk_cnt + (size_t)base * c->sel_rows, k_cap,
                            o_part + (size_t)base * c->Hq * p_cap * c->D,
                            lse_part + (size_t)base * c->Hq * p_cap, p_cap, c->stream));
  }
  c->pend_layer = layer;
  c->pend_seqs.assign(seq_ids, seq_ids + n_seqs);
  c->pend_pcap = p_cap;
  c->pend_idx = blk_idx;
  c->pend_cnt = blk_cnt;
  c->pend_kcap = k_cap;
  return SD_OK;
}

sd_status fuse_lse(sd_ctx *c, int32_t layer, int32_t n_seqs,
                   const int32_t *seq_ids, const float *o_part,
                   const float *lse_part, int32_t p_cap, float *o, float *lse) {
  if (!c) return SD_EINVAL;
  if (n_seqs < 0) return fail(c, SD_EINVAL, "n_seqs %d < 0", n_seqs);
  if (n_seqs == 0) return SD_OK;
  if (!o_part || !lse_part || !o || !lse)
    return fail(c, SD_EINVAL, "a device pointer is NULL");
  if (p_cap < 1) return fail(c, SD_EINVAL, "p_cap %d < 1", p_cap);
  if (reinterpret_cast<uintptr_t>(o_part) % 16 != 0)
    return fail(c, SD_EINVAL, "o_part must be 16-byte aligned");
  const bool with_maw = layer >= 0;
  if (layer < -1) return fail(c, SD_EINVAL, "layer %d < -1", layer);
  if (!with_maw && p_cap > kFuseSlots)
    return fail(c, SD_EUNSUPPORTED, "pure fusion of p_cap %d > %d partial slots per head",
                p_cap, kFuseSlots);
  if (with_maw) {
    sd_status s = check_seqs(c, layer, n_seqs, seq_ids);
    if (s != SD_OK) return s;
    if (c->pend_layer != layer || c->pend_pcap != p_cap ||
        c->pend_seqs != std::vector<int32_t>(seq_ids, seq_ids + n_seqs))
      return fail(c, SD_ESTATE,
                  "fuse_lse(layer %d) does not follow sparse_attend of the same layer, "
                  "sequences and p_cap", layer);
  }
  const Ctx kc = kctx(c, with_maw ? layer : -1);
  for (int base = 0; base < n_seqs; base += kLaunchSeqs) {
    SeqBatch b;
    const int n = std::min(kLaunchSeqs, n_seqs - base);
    int mb = 0;
    if (with_maw) {
      fill_batch(c, layer, seq_ids, base, n, &b, &mb);
    } else {
      b.n = n;
      b.max_scored = 0;
      for (int i = 0; i < n; ++i) b.seq[i] = b.len[i] = 0;
    }
    const int P = with_maw ? c->pend_parts[base / kLaunchSeqs] : p_cap;
    SD_HIP(c, launch_fuse(kc, b, with_maw, P, o_part + (size_t)base * c->Hq * p_cap * c->D,
                          lse_part + (size_t)base * c->Hq * p_cap, p_cap,
                          o + (size_t)base * c->Hq * c->D, lse + (size_t)base * c->Hq,
                          c->pend_idx ? c->pend_idx + (size_t)base * c->Hkv * c->pend_kcap : nullptr,
                          c->pend_cnt ? c->pend_cnt + (size_t)base * c->Hkv : nullptr,
                          c->pend_kcap, mb, c->stream));
  }
  if (with_maw) c->pend_layer = -2;
  return SD_OK;
}

sd_status sd_debug_set_lfps(sd_ctx *c, int32_t layer, int32_t seq,
                            const float *host_src, size_t bytes) {
  if (!c) return SD_EINVAL;
  size_t need = 0;
  const sd_status st = sd_debug_bytes(c, SD_DEBUG_LFPS, layer, seq, &need);
  if (st != SD_OK) return fail(c, st, "bad table request (layer %d, seq %d)", layer, seq);
  if (bytes != need || (need && !host_src))
    return fail(c, SD_EINVAL, "table upload needs %zu bytes, got %zu", need, bytes);
  SD_HIP(c, hipStreamSynchronize(c->stream));
  const int64_t len = c->layers[layer].len[seq];
  for (int h = 0; h < c->Hkv; ++h) {
    const HeadInfo &hi = c->heads[h];
    const int64_t nb = cdiv(len, hi.S);
    float *dst = c->layers[layer].dev.phi + 2 * hi.maw_off + (size_t)seq * 2 * hi.nbmax;
    if (nb) {
      SD_HIP(c, hipMemcpy(dst, host_src, sizeof(float) * nb, hipMemcpyHostToDevice));
      SD_HIP(c, hipMemcpy(dst + hi.nbmax, host_src + nb, sizeof(float) * nb,
                          hipMemcpyHostToDevice));
    }
    host_src += 2 * nb;
  }
  return SD_OK;
}

sd_status sd_lfps_init(sd_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                       const void *q_prefill, int32_t s_steps) {
  if (!c) return SD_EINVAL;
  if (!c->lfps) return fail(c, SD_EUNSUPPORTED, "sd_lfps_init needs lfps_select");
  sd_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != SD_OK) return s;
  if (n_seqs == 0) return SD_OK;
  if (!q_prefill) return fail(c, SD_EINVAL, "q_prefill is NULL");
  if (s_steps < 1) return fail(c, SD_EINVAL, "s_steps %d < 1", s_steps);
  for (int i = 0; i < n_seqs; ++i)
    if (c->layers[layer].len[seq_ids[i]] < s_steps)
      return fail(c, SD_EINVAL, "sequence %d holds %d tokens, fewer than s_steps %d", seq_ids[i],
                  c->layers[layer].len[seq_ids[i]], s_steps);
  const Ctx kc = kctx(c, layer);
  const uint16_t *q = static_cast<const uint16_t *>(q_prefill);
  const int n0 = std::min(kLaunchSeqs, n_seqs);
  float *A = nullptr;
  SD_HIP(c, hipMalloc(reinterpret_cast<void **>(&A),
                      sizeof(float) * (size_t)n0 * c->Hkv * s_steps * c->dims.key_stride));
  sd_status st = SD_OK;
  for (int base = 0; base < n_seqs && st == SD_OK; base += kLaunchSeqs) {
    SeqBatch b;
    int mb = 0;
    fill_batch(c, layer, seq_ids, base, std::min(kLaunchSeqs, n_seqs - base), &b, &mb);
    const hipError_t e = launch_lfps_init(kc, b, mb, q + (size_t)base * s_steps * c->Hq * c->D,
                                          s_steps, A, c->stream);
    if (e != hipSuccess) st = fail(c, SD_EHIP, "table init launch failed: %s", hipGetErrorString(e));
  }
  const hipError_t e1 = hipStreamSynchronize(c->stream);
  const hipError_t e2 = hipFree(A);
  if (st == SD_OK && (e1 != hipSuccess || e2 != hipSuccess))
    st = fail(c, SD_EHIP, "table init: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  return st;
}

}  // extern "C"

namespace {

// The one-launch step of both entry points: sc is the scratch its kernels
// use (the context's own, or the static array's); clear_first zeroes the
// arrays that must start at zero (the static array keeps whatever the last
// call on the GPU left in it).
sd_status decode_step_impl(sd_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                           const void *k_new, const void *v_new, const void *q_bf16,
                           int32_t *blk_idx, int32_t *blk_cnt, int32_t k_cap, float *o_part,
                           float *lse_part, int32_t p_cap, float *o, float *lse,
                           const Scratch &sc, uint32_t *clear, size_t clear_words) {
  sd_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != SD_OK) return s;
  if (c->pqh || c->lfps)
    return fail(c, SD_EUNSUPPORTED,
                "the one-launch step ranks every block per KV head; with %s use select_topk, "
                "sparse_attend and fuse_lse", c->pqh ? "select_per_query_head" : "lfps_select");
  if (n_seqs == 0) return SD_OK;
  if (!q_bf16 || !blk_idx || !blk_cnt || !o_part || !lse_part || !o || !lse)
    return fail(c, SD_EINVAL, "a device pointer is NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(c, SD_EINVAL, "k_new and v_new must both be given or both be NULL");
  if (reinterpret_cast<uintptr_t>(o_part) % 16 != 0)
    return fail(c, SD_EINVAL, "o_part must be 16-byte aligned");
  if (p_cap < c->p_cap)
    return fail(c, SD_EINVAL, "p_cap %d < %d partial slots per head (sd_caps)", p_cap, c->p_cap);
  // k after the optional one-token append
  {
    const Layer &L = c->layers[layer];
    const int add = k_new ? 1 : 0;
    for (int i = 0; i < n_seqs; ++i) {
      if ((int64_t)L.len[seq_ids[i]] + add > c->cfg.max_seq_len)
        return fail(c, SD_EINVAL, "sequence %d is full", seq_ids[i]);
      for (int h = 0; h < c->Hkv; ++h) {
        int64_t k = k_of_seq(c, L.len[seq_ids[i]] + add, h);
        if (k > k_cap)
          return fail(c, SD_EINVAL, "k_cap %d < %lld blocks needed (seq %d, kv head %d)",
                      k_cap, (long long)k, seq_ids[i], h);
      }
    }
  }
  const uint16_t *q = static_cast<const uint16_t *>(q_bf16);
  // the append runs inside the step launch when the new token's block lies
  // wholly in the recent window for every head (W >= S): no score then
  // depends on it; otherwise the append kernel runs first
  const bool fold = k_new && c->cfg.recent_window >= c->max_S;
  if (clear) SD_HIP(c, launch_fill_u32(clear, clear_words, 0u, c->stream));
  if (k_new && (s = do_append(c, layer, n_seqs, seq_ids, nullptr, k_new, v_new, !fold)) != SD_OK)
    return s;
  const uint16_t *kn = fold ? static_cast<const uint16_t *>(k_new) : nullptr;
  const uint16_t *vn = fold ? static_cast<const uint16_t *>(v_new) : nullptr;
  Ctx kc = kctx(c, layer);
  kc.sc = sc;
  for (int base = 0; base < n_seqs; base += kLaunchSeqs) {
    SeqBatch b;
    int mb = 0;
    const int n = std::min(kLaunchSeqs, n_seqs - base);
    fill_batch(c, layer, seq_ids, base, n, &b, &mb);
    const uint16_t *qb = q + (size_t)base * c->Hq * c->D;
    const int P = parts_of(c, layer, b, mb);
    int32_t *bi = blk_idx + (size_t)base * c->Hkv * k_cap;
    int32_t *bc = blk_cnt + (size_t)base * c->Hkv;
    float *op = o_part + (size_t)base * c->Hq * p_cap * c->D;
    float *lp = lse_part + (size_t)base * c->Hq * p_cap;
    if (++c->epoch == 0) c->epoch = 1;
    const size_t row0 = (size_t)base * c->Hkv * c->D;
    SD_HIP(c, launch_step(kc, b, mb, P, qb, bi, bc, k_cap, op, lp, p_cap,
                          o + (size_t)base * c->Hq * c->D, lse + (size_t)base * c->Hq,
                          c->epoch, c->pps <= kPtLds ? c->pps : 0, kn ? kn + row0 : nullptr,
                          vn ? vn + row0 : nullptr, c->stream));
  }
  c->pend_layer = -2;
  return SD_OK;
}

}  // namespace

extern "C" {

sd_status sparse_decode_step(sd_ctx *c, int32_t layer, int32_t n_seqs,
                             const int32_t *seq_ids, const void *k_new,
                             const void *v_new, const void *q_bf16, int32_t *blk_idx,
                             int32_t *blk_cnt, int32_t k_cap, float *o_part,
                             float *lse_part, int32_t p_cap, float *o, float *lse) {
  if (!c) return SD_EINVAL;
  return decode_step_impl(c, layer, n_seqs, seq_ids, k_new, v_new, q_bf16, blk_idx, blk_cnt,
                          k_cap, o_part, lse_part, p_cap, o, lse, c->sc, nullptr, 0);
}

sd_status sparse_decode_step_noalloc(sd_ctx *c, int32_t layer, int32_t n_seqs,
                                     const int32_t *seq_ids, const void *k_new,
                                     const void *v_new, const void *q_bf16, int32_t *blk_idx,
                                     int32_t *blk_cnt, int32_t k_cap, float *o_part,
                                     float *lse_part, int32_t p_cap, float *o, float *lse) {
  if (!c) return SD_EINVAL;
  if (!c->static_scratch) {
    const hipError_t e = (c->device >= 0 && c->device < kMaxDevices) ? g_scratch_err[c->device]
                                                                      : hipErrorInvalidDevice;
    return fail(c, SD_EHIP, "the static scratch array has no device address on device %d (%s)",
                c->device, hipGetErrorString(e));
  }
  const StaticLayout &sl = c->slayout;
  if (sl.total > (size_t)SD_STATIC_SCRATCH_BYTES)
    return fail(c, SD_EUNSUPPORTED,
                "this context's step needs %zu bytes of scratch, more than the %zu of the "
                "static array (fewer max_seqs or a shorter max_seq_len)",
                sl.total, (size_t)SD_STATIC_SCRATCH_BYTES);
  unsigned char *base = static_cast<unsigned char *>(c->static_scratch);
  Scratch sc = c->sc;  // err stays the context's own
  sc.arrive = reinterpret_cast<uint32_t *>(base + sl.arrive);
  sc.unit_acc = reinterpret_cast<uint32_t *>(base + sl.unit_acc);
  sc.rtag = reinterpret_cast<unsigned long long *>(base + sl.rtag);
  sc.seltag = reinterpret_cast<unsigned long long *>(base + sl.seltag);
  sc.keyflag = reinterpret_cast<unsigned long long *>(base + sl.keyflag);
  sc.cand = reinterpret_cast<unsigned long long *>(base + sl.cand);
  sc.keys = reinterpret_cast<uint32_t *>(base + sl.keys);
  sc.ulist = reinterpret_cast<int32_t *>(base + sl.ulist);
  sc.ukeys = reinterpret_cast<uint32_t *>(base + sl.ukeys);
  sc.lm_pg = reinterpret_cast<float *>(base + sl.lm_pg);
  return decode_step_impl(c, layer, n_seqs, seq_ids, k_new, v_new, q_bf16, blk_idx, blk_cnt,
                          k_cap, o_part, lse_part, p_cap, o, lse, sc,
                          reinterpret_cast<uint32_t *>(base), sl.clear_bytes / 4);
}

sd_status sd_release_seq(sd_ctx *c, int32_t seq) {
  if (!c) return SD_EINVAL;
  if (seq < 0 || seq >= c->cfg.max_seqs)
    return fail(c, SD_EINVAL, "seq id %d out of range", seq);
  SD_HIP(c, hipStreamSynchronize(c->stream));
  for (auto &L : c->layers) {
    int64_t np = cdiv(L.len[seq], kPage);
    for (int64_t p = np - 1; p >= 0; --p)
      L.free_pages.push_back(L.h_pt[(size_t)seq * c->pps + p]);
    L.len[seq] = 0;
    for (int h = 0; h < c->Hkv; ++h) {
      const HeadInfo &hi = c->heads[h];
      SD_HIP(c, launch_fill_f32(L.dev.maw + hi.maw_off + (size_t)seq * hi.nbmax,
                                hi.nbmax, 0.0f, c->stream));
      if (L.dev.phi)
        SD_HIP(c, launch_fill_f32(L.dev.phi + 2 * hi.maw_off + (size_t)seq * 2 * hi.nbmax,
                                  2 * hi.nbmax, 0.0f, c->stream));
    }
  }
  if (c->pend_layer >= 0 &&
      std::find(c->pend_seqs.begin(), c->pend_seqs.end(), seq) != c->pend_seqs.end())
    c->pend_layer = -2;
  SD_HIP(c, hipStreamSynchronize(c->stream));
  return SD_OK;
}

sd_status sd_debug_bytes(const sd_ctx *c, int32_t what, int32_t layer,
                         int32_t seq, size_t *bytes) {
  if (!c || !bytes) return SD_EINVAL;
  if (layer < 0 || layer >= c->cfg.num_layers || seq < 0 || seq >= c->cfg.max_seqs)
    return SD_EINVAL;
  const int64_t len = c->layers[layer].len[seq];
  size_t b = 0;
  switch (what) {
    case SD_DEBUG_PAGE_TABLE: b = sizeof(int32_t) * c->pps; break;
    case SD_DEBUG_SUMMARY:
      for (int h = 0; h < c->Hkv; ++h) b += sizeof(uint16_t) * cdiv(len, c->S[h]) * c->D * 2;
      break;
    case SD_DEBUG_MAW:
      for (int h = 0; h < c->Hkv; ++h) b += sizeof(float) * cdiv(len, c->S[h]);
      break;
    case SD_DEBUG_K:
    case SD_DEBUG_V: b = sizeof(uint16_t) * len * c->Hkv * c->D; break;
    case SD_DEBUG_LFPS_CAND:
      if (!c->lfps) return SD_EUNSUPPORTED;
      b = sizeof(int32_t) * c->Hkv;
      break;
    case SD_DEBUG_LFPS:
      if (!c->lfps) return SD_EUNSUPPORTED;
      for (int h = 0; h < c->Hkv; ++h) b += sizeof(float) * 2 * cdiv(len, c->S[h]);
      break;
    case SD_DEBUG_SCORES:
      if (c->pqh || c->lfps) return SD_EUNSUPPORTED;  // (other key layouts)
      for (int h = 0; h < c->Hkv; ++h) b += sizeof(float) * (1 + cdiv(len, c->S[h]));
      break;
    default: return SD_EINVAL;
  }
  *bytes = b;
  return SD_OK;
}

sd_status sd_debug_copy(sd_ctx *c, int32_t what, int32_t layer, int32_t seq,
                        void *host_dst, size_t bytes) {
  if (!c) return SD_EINVAL;
  size_t need = 0;
  if (sd_debug_bytes(c, what, layer, seq, &need) != SD_OK)
    return fail(c, SD_EINVAL, "bad debug request (what %d, layer %d, seq %d)", what, layer, seq);
  if (bytes != need || (need && !host_dst))
    return fail(c, SD_EINVAL, "debug copy needs %zu bytes, got %zu", need, bytes);
  SD_HIP(c, hipStreamSynchronize(c->stream));
  const Layer &L = c->layers[layer];
  const int64_t len = L.len[seq];
  const int D = c->D;
  if (what == SD_DEBUG_PAGE_TABLE) {
    SD_HIP(c, hipMemcpy(host_dst, L.dev.pt + (size_t)seq * c->pps, need, hipMemcpyDeviceToHost));
  } else if (what == SD_DEBUG_SUMMARY) {
    uint16_t *dst = static_cast<uint16_t *>(host_dst);
    for (int h = 0; h < c->Hkv; ++h) {
      const HeadInfo &hi = c->heads[h];
      const int64_t nb = cdiv(len, hi.S);
      std::vector<uint16_t> raw((size_t)(D / 4) * hi.nbmax * 8);
      SD_HIP(c, hipMemcpy(raw.data(), L.dev.summ + hi.summ_off + (size_t)seq * raw.size(),
                          raw.size() * sizeof(uint16_t), hipMemcpyDeviceToHost));
      for (int64_t b = 0; b < nb; ++b)
        for (int ch = 0; ch < D; ++ch) {
          const size_t src = ((size_t)(ch / 4) * hi.nbmax + b) * 8 + 2 * (ch % 4);
          dst[(b * D + ch) * 2 + 0] = raw[src];
          dst[(b * D + ch) * 2 + 1] = raw[src + 1];
        }
      dst += nb * D * 2;
    }
  } else if (what == SD_DEBUG_MAW) {
    float *dst = static_cast<float *>(host_dst);
    for (int h = 0; h < c->Hkv; ++h) {
      const HeadInfo &hi = c->heads[h];
      const int64_t nb = cdiv(len, hi.S);
      if (nb)
        SD_HIP(c, hipMemcpy(dst, L.dev.maw + hi.maw_off + (size_t)seq * hi.nbmax,
                            sizeof(float) * nb, hipMemcpyDeviceToHost));
      dst += nb;
    }
  } else if (what == SD_DEBUG_LFPS_CAND) {
    int32_t *dst = static_cast<int32_t *>(host_dst);
    for (int h = 0; h < c->Hkv; ++h)
      SD_HIP(c, hipMemcpy(dst + h, c->sc.unit_acc + 4 * ((size_t)seq * c->Hkv + h) + 3,
                          sizeof(int32_t), hipMemcpyDeviceToHost));
  } else if (what == SD_DEBUG_LFPS) {
    float *dst = static_cast<float *>(host_dst);
    for (int h = 0; h < c->Hkv; ++h) {
      const HeadInfo &hi = c->heads[h];
      const int64_t nb = cdiv(len, hi.S);
      const float *src = L.dev.phi + 2 * hi.maw_off + (size_t)seq * 2 * hi.nbmax;
      if (nb) {
        SD_HIP(c, hipMemcpy(dst, src, sizeof(float) * nb, hipMemcpyDeviceToHost));
        SD_HIP(c, hipMemcpy(dst + nb, src + hi.nbmax, sizeof(float) * nb, hipMemcpyDeviceToHost));
      }
      dst += 2 * nb;
    }
  } else if (what == SD_DEBUG_SCORES) {
    // the unit's keys as its score tiles wrote them (order key of the fp32
    // group score; 0 for a block that is not a candidate) and the bound its
    // top-k kept
    float *dst = static_cast<float *>(host_dst);
    const int64_t ks = c->dims.key_stride;
    std::vector<unsigned long long> kf((size_t)ks);
    const int64_t W = c->dims.window, ns = c->dims.n_sink;
    for (int h = 0; h < c->Hkv; ++h) {
      const HeadInfo &hi = c->heads[h];
      const int64_t nb = cdiv(len, hi.S);
      const size_t unit = (size_t)seq * c->Hkv + h;
      const bool none = hi.ppm == 0 || std::min(ns, len) >= std::max<int64_t>(0, len - W);
      const int64_t n_sc = (W > 0 && len > 0) ? std::min(nb, cdiv(std::max<int64_t>(0, len - W), hi.S))
                                              : nb;
      const float nan = std::numeric_limits<float>::quiet_NaN();
      for (int64_t b = 0; b <= nb; ++b) dst[b] = nan;
      if (!none && nb) {
        uint32_t eb = 0;
        SD_HIP(c, hipMemcpy(&eb, c->sc.unit_acc + 4 * unit + 2, sizeof(uint32_t),
                            hipMemcpyDeviceToHost));
        memcpy(&dst[0], &eb, sizeof(float));
        SD_HIP(c, hipMemcpy(kf.data(), c->sc.keyflag + unit * ks, sizeof(unsigned long long) * ks,
                            hipMemcpyDeviceToHost));
        for (int64_t b = 0; b < n_sc; ++b) {
          const uint32_t k = (uint32_t)kf[(size_t)key_slot((int)b, (int)n_sc)];
          if (k == 0u) continue;
          const uint32_t bits = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
          memcpy(&dst[1 + b], &bits, sizeof(float));
        }
      }
      dst += 1 + nb;
    }
  } else {
    const uint16_t *pool = what == SD_DEBUG_K ? L.dev.k : L.dev.v;
    uint16_t *dst = static_cast<uint16_t *>(host_dst);
    const size_t page_elems = (size_t)c->Hkv * kPage * D;
    std::vector<uint16_t> page(page_elems);
    for (int64_t p = 0; p < cdiv(len, kPage); ++p) {
      int pid = L.h_pt[(size_t)seq * c->pps + p];
      SD_HIP(c, hipMemcpy(page.data(), pool + (size_t)pid * page_elems,
                          page_elems * sizeof(uint16_t), hipMemcpyDeviceToHost));
      for (int r = 0; r < kPage && p * kPage + r < len; ++r)
        for (int h = 0; h < c->Hkv; ++h) {
          uint16_t *row = dst + (((size_t)(p * kPage + r)) * c->Hkv + h) * D;
          if (what == SD_DEBUG_K)  // K pages: [Hkv][d/8][16][8]
            for (int ch = 0; ch < D; ++ch)
              row[ch] = page[(((size_t)h * (D / 8) + ch / 8) * kPage + r) * 8 + ch % 8];
          else  // V pages are stored transposed: [Hkv][d][16]
            for (int ch = 0; ch < D; ++ch) row[ch] = page[((size_t)h * D + ch) * kPage + r];
        }
    }
  }
  return SD_OK;
}

sd_status sd_debug_set_maw(sd_ctx *c, int32_t layer, int32_t seq,
                           const float *host_src, size_t bytes) {
  if (!c) return SD_EINVAL;
  size_t need = 0;
  if (sd_debug_bytes(c, SD_DEBUG_MAW, layer, seq, &need) != SD_OK)
    return fail(c, SD_EINVAL, "bad MAW request (layer %d, seq %d)", layer, seq);
  if (bytes != need || (need && !host_src))
    return fail(c, SD_EINVAL, "MAW upload needs %zu bytes, got %zu", need, bytes);
  SD_HIP(c, hipStreamSynchronize(c->stream));
  const int64_t len = c->layers[layer].len[seq];
  for (int h = 0; h < c->Hkv; ++h) {
    const HeadInfo &hi = c->heads[h];
    const int64_t nb = cdiv(len, hi.S);
    if (nb)
      SD_HIP(c, hipMemcpy(c->layers[layer].dev.maw + hi.maw_off + (size_t)seq * hi.nbmax,
                          host_src, sizeof(float) * nb, hipMemcpyHostToDevice));
    host_src += nb;
  }
  return SD_OK;
}

}  // extern "C"
