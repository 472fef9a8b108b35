// C ABI of libvdm.so: argument validation, workspace layout and the launch
// sequences of the five calls declared in include/vdm.h. No kernels here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "vdm_hvd.hpp"
#include "vdm_internal.hpp"

namespace vdm {

static thread_local std::string g_err;

static vdm_status fail(vdm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static vdm_status fail(vdm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define VDM_HIP(call, what)                                                                          \
  do {                                                                                               \
    hipError_t e_ = (call);                                                                          \
    if (e_ != hipSuccess) return fail(VDM_ERR_HIP, "%s: %s", what, hipGetErrorString(e_));          \
  } while (0)

// VDM_HIP for a launch of timing kind `kind` (see vdm_timing)
#define VDM_HIP_T(kind, s, call, what) \
  do {                                 \
    Timed tm_((kind), (s));            \
    VDM_HIP(call, what);               \
  } while (0)

DevInfo dev_info() {
  static DevInfo cache[64];
  static bool have[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DevInfo{256, 65536};
  if (!have[dev]) {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) lds = 65536;
    cache[dev] = DevInfo{cus, lds};
    have[dev] = true;
  }
  return cache[dev];
}

// ------------------------------------------------------------------ launch timing
namespace {
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> free_events;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[VDM_TIME_KINDS];
  hipEvent_t get() {  // caller holds mu
    if (!free_events.empty()) {
      hipEvent_t e = free_events.back();
      free_events.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) == hipSuccess) return e;
    (void)hipGetLastError();
    return nullptr;
  }
};
Timing& timing() {
  static Timing t;
  return t;
}

// Records an event on `s` now and another when it goes out of scope, if timing is on.
class Timed {
 public:
  Timed(int kind, hipStream_t s) : kind_(kind), s_(s) {
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on) return;
    a_ = t.get();
    b_ = t.get();
    if (a_ && b_ && hipEventRecord(a_, s_) == hipSuccess) return;
    (void)hipGetLastError();  // a failed record must not be reported by the launch that follows
    if (a_) t.free_events.push_back(a_);
    if (b_) t.free_events.push_back(b_);
    a_ = b_ = nullptr;
  }
  ~Timed() {
    if (!a_) return;
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    if (hipEventRecord(b_, s_) == hipSuccess) {
      t.rec[kind_].emplace_back(a_, b_);
    } else {
      (void)hipGetLastError();
      t.free_events.push_back(a_);
      t.free_events.push_back(b_);
    }
  }
  Timed(const Timed&) = delete;
  Timed& operator=(const Timed&) = delete;

 private:
  int kind_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};
}  // namespace

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
static size_t esize(int dtype) { return dtype == VDM_BF16 ? 2 : 4; }

// Carves a workspace; with base == nullptr it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <typename P>
  P* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

static vdm_status check_decoder(const vdm_decoder* d) {
  if (!d) return fail(VDM_ERR_INVALID_ARG, "decoder is NULL");
  if (d->dtype != VDM_F32 && d->dtype != VDM_BF16) return fail(VDM_ERR_INVALID_ARG, "dtype %d unknown", d->dtype);
  if (d->n_freq != 8) return fail(VDM_ERR_UNSUPPORTED, "n_freq must be 8 (got %d)", d->n_freq);
  if (d->H < 1 || d->D != 64 * d->H) return fail(VDM_ERR_UNSUPPORTED, "D must be 64*H (D=%d H=%d)", d->D, d->H);
  const bool ok = (d->dtype == VDM_BF16 && (d->D == 64 || d->D == 256)) || (d->dtype == VDM_F32 && d->D == 64);
  if (!ok) return fail(VDM_ERR_UNSUPPORTED, "unsupported width D=%d for dtype %d", d->D, d->dtype);
  const int fc = decode_f_chunk(d->dtype, d->D);
  if (d->F < fc || d->F > 4096 || d->F % fc) return fail(VDM_ERR_UNSUPPORTED, "F=%d must be a multiple of %d in [%d, 4096]", d->F, fc, fc);
  if (!d->Wq || !d->Wk || !d->Wv || !d->Wo || !d->W1 || !d->W2 || !d->w_head)
    return fail(VDM_ERR_INVALID_ARG, "a decoder weight pointer is NULL");
  const size_t es = esize(d->dtype);
  if (!aligned(d->Wq, es) || !aligned(d->Wk, 16) || !aligned(d->Wv, 16) || !aligned(d->Wo, 16) ||
      !aligned(d->W1, 16) || !aligned(d->W2, 16) || !aligned(d->w_head, 4))
    return fail(VDM_ERR_INVALID_ARG, "misaligned decoder weights (Wq: element size; others: 16 bytes)");
  if (d->n_prims < 1 || d->n_prims > VDM_MAX_PRIMS) return fail(VDM_ERR_INVALID_ARG, "n_prims=%d", d->n_prims);
  for (int i = 0; i < d->n_prims; ++i)
    if (d->prims[i].kind != VDM_PRIM_SPHERE && d->prims[i].kind != VDM_PRIM_BOX)
      return fail(VDM_ERR_INVALID_ARG, "primitive %d has kind %d", i, d->prims[i].kind);
  if (!isfinite(d->net_scale)) return fail(VDM_ERR_INVALID_ARG, "net_scale is not finite");
  return VDM_OK;
}

static PrimSet prims_of(const vdm_decoder* d) {
  PrimSet p;
  memset(&p, 0, sizeof p);
  p.n = d->n_prims;
  for (int i = 0; i < d->n_prims; ++i) {
    p.p[i].kind = d->prims[i].kind;
    for (int c = 0; c < 3; ++c) {
      p.p[i].c[c] = d->prims[i].centre[c];
      p.p[i].s[c] = d->prims[i].size[c];
    }
  }
  return p;
}

static DecodeArgs base_args(const vdm_decoder* d) {
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.Wq = d->Wq;
  a.Wo = d->Wo;
  a.W1 = d->W1;
  a.W2 = d->W2;
  a.w_head = d->w_head;
  a.F = d->F;
  a.net_scale = d->net_scale;
  a.prims = prims_of(d);
  return a;
}

static int64_t mpad(int64_t M) { return (M + 31) / 32 * 32; }

// KV selection scratch: per-workgroup score rows (H rows per probe with per-head
// sets), then (bf16) the packed K
static int sel_sets(const vdm_decoder* d, bool heads) { return heads ? d->H : 1; }
static size_t select_ws_bytes(const vdm_decoder* d, int64_t M, bool heads = false) {
  const size_t kp = d->dtype == VDM_BF16 ? (size_t)mpad(M) * d->D * 2 : 0;
  return (select_scratch_bytes((int)M, sel_sets(d, heads)) + 255) / 256 * 256 + kp + 256;
}

// bf16 decoders stream Wo, W1, W2 in fragment-packed form from the workspace
static size_t packed_w_bytes(const vdm_decoder* d) {
  return d->dtype == VDM_BF16 ? ((size_t)d->D * d->D + 2 * (size_t)d->D * d->F) * 2 : 0;
}

static hipError_t pack_weights(const vdm_decoder* d, void* Wp, DecodeArgs& a, hipStream_t s) {
  if (d->dtype != VDM_BF16) return hipSuccess;
  char* p = static_cast<char*>(Wp);
  const size_t DD = (size_t)d->D * d->D * 2, DF = (size_t)d->D * d->F * 2;
  hipError_t e = launch_pack_w(d->Wo, d->D, d->D, p, s);
  if (e == hipSuccess) e = launch_pack_w(d->W1, d->F, d->D, p + DD, s);
  if (e == hipSuccess) e = launch_pack_w(d->W2, d->D, d->F, p + DD + DF, s);
  a.Wo = p;
  a.W1 = p + DD;
  a.W2 = p + DD + DF;
  return e;
}

// ------------------------------------------------------------------ dense workspace
struct DenseWs {
  void* Kp;
  void* Vt;
  void* Wp;
  float* kmax;
  Item* items;
  int32_t* n_items;
  SplitPlan split;  // tail split of the full-attention launch (parts = 1: none)
  float* part;
  int32_t* part_cnt;
};

// split: plan a tail split of the full-attention decode (decode_split_plan)
static size_t dense_ws(const vdm_decoder* d, int64_t M, int64_t N, bool sel, void* base, DenseWs* w,
                       bool split = true) {
  Carve c(base);
  DenseWs x;
  const size_t kv = (size_t)mpad(M) * d->D * esize(d->dtype);
  x.Kp = sel ? nullptr : c.take<char>(kv);
  x.Vt = sel ? nullptr : c.take<char>(kv);
  x.Wp = c.take<char>(packed_w_bytes(d));
  x.kmax = c.take<float>(256);
  x.items = sel ? c.take<Item>((size_t)(N > 0 ? N : 1) * sizeof(Item)) : nullptr;
  x.n_items = sel ? c.take<int32_t>(256) : nullptr;
  const int bq = decode_tile_queries(d->dtype, d->D);
  if (!sel && split) x.split = decode_split_plan(d->dtype, d->D, M, (N + bq - 1) / bq);
  x.part = x.split.parts > 1 ? c.take<float>(x.split.part_bytes) : nullptr;
  x.part_cnt = x.split.parts > 1 ? c.take<int32_t>(x.split.cnt_bytes) : nullptr;
  if (w) *w = x;
  return c.off + 256;
}

// batch of B vecsets: packed K/V per shape, kmax [B][H]
struct BatchWs {
  char* Kp;
  char* Vt;
  void* Wp;
  float* kmax;
  size_t kv;  // packed bytes per shape (K or V)
  unsigned long long* queue;  // the decode's work-unit counter
};

static size_t batch_ws(const vdm_decoder* d, int64_t B, int64_t M, void* base, BatchWs* w) {
  Carve c(base);
  BatchWs x;
  x.kv = ((size_t)mpad(M) * d->D * esize(d->dtype) + 255) / 256 * 256;
  x.Kp = c.take<char>(x.kv * B);
  x.Vt = c.take<char>(x.kv * B);
  x.Wp = c.take<char>(packed_w_bytes(d));
  x.kmax = c.take<float>((size_t)B * d->H * 4);
  x.queue = c.take<unsigned long long>(256);
  if (w) *w = x;
  return c.off + 256;
}

// ------------------------------------------------------------------ hierarchical workspace
struct HierWs {
  void* Kp;
  void* Vt;
  void* Wp;
  float* kmax;
  float* vol[VDM_MAX_LEVELS];
  uint64_t* active[VDM_MAX_LEVELS];
  uint64_t* kept[VDM_MAX_LEVELS];
  uint64_t* comp[VDM_MAX_LEVELS];
  uint64_t* tmp;
  uint64_t* newmask;
  int32_t* counts;
  int4* offs;
  int4* partial;
  int32_t* totals;  // [levels][4]: queries, items, occupied blocks
  int32_t* list;
  Item* items;
  int64_t list_cap, item_cap;  // entries of list and items
  int32_t* occ;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  float* sel_scores;
  int64_t* stats;
  int64_t* part;     // spread partial counters of the mask stages
  int64_t* bprefix;  // a batch's decode units per shape, prefixed (slice 0 of a batch)
  unsigned long long* queues;  // per level: the decode's work-unit counter (slice 0)
};

static size_t hier_ws(const vdm_decoder* d, const vdm_hier_params* p, int64_t M, void* base, HierWs* w) {
  Carve c(base);
  HierWs x;
  memset(&x, 0, sizeof x);
  const size_t kv = (size_t)mpad(M) * d->D * esize(d->dtype);
  x.Kp = c.take<char>(kv);
  x.Vt = c.take<char>(kv);
  x.Wp = c.take<char>(packed_w_bytes(d));
  x.kmax = c.take<float>(256);
  int64_t maxP3 = 0, maxNB3 = 0, maxWords = 0;
  for (int L = 0; L < p->levels; ++L) {
    const int64_t R = (int64_t)p->R0 << L, P = R + 1;
    const int64_t NB = nblocks8((int)P);
    if (L < p->levels - 1) x.vol[L] = c.take<float>((size_t)P * P * P * 4);
    x.active[L] = c.take<uint64_t>((size_t)mask_words((int)P) * 8);
    x.kept[L] = c.take<uint64_t>((size_t)mask_words((int)P) * 8);
    if (L > 0) x.comp[L] = c.take<uint64_t>((size_t)mask_words((int)P) * 8);
    maxP3 = P * P * P > maxP3 ? P * P * P : maxP3;
    maxNB3 = NB * NB * NB > maxNB3 ? NB * NB * NB : maxNB3;
    maxWords = mask_words((int)P) > maxWords ? mask_words((int)P) : maxWords;
  }
  const int bq = decode_tile_queries(d->dtype, d->D);
  x.tmp = c.take<uint64_t>((size_t)maxWords * 8);
  x.newmask = c.take<uint64_t>((size_t)maxWords * 8);
  x.counts = c.take<int32_t>((size_t)maxNB3 * 4);
  x.offs = c.take<int4>((size_t)maxNB3 * 16);
  x.partial = c.take<int4>((size_t)scan_partials(maxNB3) * 16);
  x.totals = c.take<int32_t>((size_t)VDM_MAX_LEVELS * 4 * 4);
  x.list_cap = maxP3;
  x.item_cap = maxNB3 * ((512 + bq - 1) / bq);
  x.list = c.take<int32_t>((size_t)x.list_cap * 4);
  x.items = c.take<Item>((size_t)x.item_cap * sizeof(Item));
  x.occ = c.take<int32_t>((size_t)maxNB3 * 4);
  if (p->use_kvsel) {
    const int ns = sel_sets(d, p->heads != 0);
    x.sel_idx = c.take<int32_t>((size_t)maxNB3 * ns * p->cap * 4);
    x.sel_cnt = c.take<int32_t>((size_t)maxNB3 * ns * 4);
    x.sel_scores = c.take<float>(select_scratch_bytes((int)M, ns));
  }
  x.stats = c.take<int64_t>((size_t)VDM_MAX_LEVELS * VDM_STAT_FIELDS * 8);
  x.part = c.take<int64_t>((size_t)stat_part_words() * 8);
  x.bprefix = c.take<int64_t>((size_t)(4096 + 1) * 8);
  x.queues = c.take<unsigned long long>((size_t)VDM_MAX_LEVELS * 8);
  if (w) *w = x;
  return c.off + 256;
}

static vdm_status check_hier(const vdm_decoder* d, const vdm_hier_params* p, int64_t M) {
  if (!p) return fail(VDM_ERR_INVALID_ARG, "params is NULL");
  if (p->levels < 1 || p->levels > VDM_MAX_LEVELS) return fail(VDM_ERR_INVALID_ARG, "levels=%d", p->levels);
  if (p->R0 < 1) return fail(VDM_ERR_INVALID_ARG, "R0=%d", p->R0);
  const int64_t Rf = (int64_t)p->R0 << (p->levels - 1);
  if (Rf > 1200) return fail(VDM_ERR_INVALID_ARG, "finest grid R=%lld exceeds 1200", (long long)Rf);
  if (p->dilation < 0 || p->dilation > 8) return fail(VDM_ERR_INVALID_ARG, "dilation=%d", p->dilation);
  if (isnan(p->tau)) return fail(VDM_ERR_INVALID_ARG, "tau is NaN");
  if (M < 1) return fail(VDM_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (p->use_kvsel) {
    if (p->block != 8) return fail(VDM_ERR_UNSUPPORTED, "KV selection blocks must be 8 points per axis");
    if (p->k < 1 || p->k > M || p->cap < p->k) return fail(VDM_ERR_INVALID_ARG, "k=%d cap=%d M=%lld", p->k, p->cap, (long long)M);
    if (!select_fits(M, p->k, p->cap, p->heads == 1))
      return fail(VDM_ERR_UNSUPPORTED, "KV selection: M=%lld (at most %d) with k=%d cap=%d", (long long)M,
                  select_max_tokens(p->heads == 1), p->k, p->cap);
    if (p->probes != 0 && p->probes != 1) return fail(VDM_ERR_INVALID_ARG, "probes=%d (0: corners, 1: random)", p->probes);
    if (p->heads != 0 && p->heads != 1) return fail(VDM_ERR_INVALID_ARG, "heads=%d (0: one set per block, 1: per head)", p->heads);
  }
  (void)d;
  return VDM_OK;
}

}  // namespace vdm

using namespace vdm;


// Bounds-checked builds: after a call's launches, wait for them and report the
// first failed device bounds check of any kernel file (VDM_BOUND). Release builds
// return the status unchanged.
static vdm_status debug_checked(vdm_status st, vdm_stream stream) {
#if VDM_DEBUG
  if (st != VDM_OK) return st;
  static const char* const what[BC_CHECKS] = {
      "",
      "work item query range",
      "work item selection row",
      "selection row count",
      "selected token id",
      "block selection row",
      "selection block id",
      "selection output slot",
      "query list slot",
      "work item slot",
      "occupied block slot",
      "support slot",
      "cell support range",
      "query index in cell order",
      "selection candidate slot"};
  hipError_t (*const take[])(unsigned*) = {debug_take_decode, debug_take_select, debug_take_hvd,
                                            debug_take_local,  debug_take_prep,   debug_take_surface};
  static const char* const file[] = {"decode", "select", "hvd", "local", "prep", "surface"};
  VDM_HIP(hipStreamSynchronize((hipStream_t)stream), "bounds-check synchronize");
  vdm_status out = VDM_OK;
  for (int f = 0; f < 6; ++f) {
    unsigned w = 0;
    VDM_HIP(take[f](&w), "bounds-check read");
    if (w != 0 && out == VDM_OK)
      out = fail(VDM_ERR_HIP, "bounds check failed in the %s kernels: %s (check %u)", file[f],
                 w < BC_CHECKS ? what[w] : "?", w);
  }
  return out;
#else
  (void)stream;
  return st;
#endif
}

extern "C" {

const char* vdm_last_error(void) { return g_err.c_str(); }
vdm_status vdm_timing(int32_t mode) {
  if (mode < 0 || mode > 2) return fail(VDM_ERR_INVALID_ARG, "timing mode %d is not 0, 1 or 2", mode);
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (mode == 2) {
    for (auto& r : t.rec) {
      for (auto& e : r) {
        t.free_events.push_back(e.first);
        t.free_events.push_back(e.second);
      }
      r.clear();
    }
  } else {
    t.on = mode == 1;
  }
  return VDM_OK;
}

vdm_status vdm_timing_read(int32_t kind, int64_t* launches, double* total_ms) {
  if (kind < 0 || kind >= VDM_TIME_KINDS) return fail(VDM_ERR_INVALID_ARG, "timing kind %d out of range", kind);
  if (!launches || !total_ms) return fail(VDM_ERR_INVALID_ARG, "null output pointer");
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  double sum = 0.0;
  for (auto& e : t.rec[kind]) {
    VDM_HIP(hipEventSynchronize(e.second), "timing event wait");
    float ms = 0.f;
    VDM_HIP(hipEventElapsedTime(&ms, e.first, e.second), "timing event read");
    sum += ms;
  }
  *launches = (int64_t)t.rec[kind].size();
  *total_ms = sum;
  return VDM_OK;
}

int32_t vdm_version(void) { return VDM_VERSION; }

vdm_status vdm_device_info(int32_t* compute_units, int32_t* peak_clock_khz) {
  int dev = 0, cus = 0, khz = 0;
  VDM_HIP(hipGetDevice(&dev), "no HIP device");
  VDM_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "device attribute");
  VDM_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev), "device attribute");
  if (compute_units) *compute_units = cus;
  if (peak_clock_khz) *peak_clock_khz = khz;
  return VDM_OK;
}

size_t vdm_dense_workspace_size(const vdm_decoder* dec, int64_t M, int64_t N, int32_t with_sel) {
  if (check_decoder(dec) != VDM_OK) return 0;
  if (M < 1 || N < 0) {
    fail(VDM_ERR_INVALID_ARG, "M=%lld N=%lld", (long long)M, (long long)N);
    return 0;
  }
  return dense_ws(dec, M, N, with_sel != 0, nullptr, nullptr);
}

size_t vdm_select_workspace_size(const vdm_decoder* dec, int64_t M) {
  if (check_decoder(dec) != VDM_OK) return 0;
  if (M < 1 || M > select_max_tokens(false)) {
    fail(VDM_ERR_INVALID_ARG, "M=%lld (1..%d)", (long long)M, select_max_tokens(false));
    return 0;
  }
  return select_ws_bytes(dec, M);
}

size_t vdm_select_heads_workspace_size(const vdm_decoder* dec, int64_t M) {
  if (check_decoder(dec) != VDM_OK) return 0;
  if (M < 1 || M > select_max_tokens(true)) {
    fail(VDM_ERR_INVALID_ARG, "M=%lld (1..%d)", (long long)M, select_max_tokens(true));
    return 0;
  }
  return select_ws_bytes(dec, M, true);
}

size_t vdm_hier_workspace_size(const vdm_decoder* dec, const vdm_hier_params* params, int64_t M) {
  if (check_decoder(dec) != VDM_OK || check_hier(dec, params, M) != VDM_OK) return 0;
  return hier_ws(dec, params, M, nullptr, nullptr);
}

static vdm_status hier_run(const vdm_decoder* dec, const vdm_hier_params* p, int B, const void* K, const void* V,
                           int64_t M, size_t kv_bytes, float* vol, int64_t vol_stride, int64_t* S, int64_t st_stride,
                           const vdm_hier_debug* dbg, void* ws, size_t ws_stride, hipStream_t s);

// ------------------------------------------------------------------ batched hierarchical decoding
// B shapes through the hierarchical pipeline on one stream: every mask stage of a
// level is one launch for all B shapes (hier_run), so the small per-level
// bookkeeping launches are shared instead of repeated per shape.
namespace {
size_t hier_batch_stride(const vdm_decoder* dec, const vdm_hier_params* p, int64_t M) {
  return (hier_ws(dec, p, M, nullptr, nullptr) + 255) / 256 * 256;
}
}  // namespace

size_t vdm_hier_batch_workspace_size(const vdm_decoder* dec, const vdm_hier_params* params, int32_t B, int64_t M) {
  if (B < 1 || B > 4096) {
    fail(VDM_ERR_INVALID_ARG, "B=%d (1..4096)", B);
    return 0;
  }
  if (check_decoder(dec) != VDM_OK || check_hier(dec, params, M) != VDM_OK) return 0;
  return hier_batch_stride(dec, params, M) * (size_t)B;
}

static vdm_status decode_hier_batch_body(const vdm_decoder* dec, const vdm_hier_params* p, int32_t B, const void* K,
                                 const void* V, int64_t M, float* vol, int64_t vol_elems, int64_t* stats, void* ws,
                                 size_t ws_bytes, vdm_stream stream) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (B < 1 || B > 4096) return fail(VDM_ERR_INVALID_ARG, "B=%d (1..4096)", B);
  st = check_hier(dec, p, M);
  if (st != VDM_OK) return st;
  const int64_t Pf = ((int64_t)p->R0 << (p->levels - 1)) + 1, P3 = Pf * Pf * Pf;
  if (!vol || vol_elems / B < P3) return fail(VDM_ERR_INVALID_ARG, "vol needs %d x %lld floats", B, (long long)P3);
  const size_t kv_bytes = (size_t)M * dec->D * esize(dec->dtype);
  if (!K || !V || !aligned(K, 16) || !aligned(V, 16) || kv_bytes % 16 != 0 || !aligned(vol, 4))
    return fail(VDM_ERR_INVALID_ARG, "K, V or vol NULL/misaligned (each shape's K/V must start 16-byte aligned)");
  const size_t stride = hier_batch_stride(dec, p, M);
  if (!ws || ws_bytes / (size_t)B < stride || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace needs %d x %zu bytes, 256-aligned (got %zu)", B, stride, ws_bytes);
  (void)hipGetLastError();
  // counters: the caller's [B][levels][fields], or each slice's own
  HierWs w;
  hier_ws(dec, p, M, ws, &w);
  int64_t* S = stats ? stats : w.stats;
  const int64_t sst = stats ? (int64_t)p->levels * VDM_STAT_FIELDS : (int64_t)(stride / 8);
  return hier_run(dec, p, B, K, V, M, kv_bytes, vol, P3, S, sst, nullptr, ws, stride, (hipStream_t)stream);
}

vdm_status vdm_decode_hier_batch(const vdm_decoder* dec, const vdm_hier_params* p, int32_t B, const void* K,
                                 const void* V, int64_t M, float* vol, int64_t vol_elems, int64_t* stats, void* ws,
                                 size_t ws_bytes, vdm_stream stream) {
  return debug_checked(decode_hier_batch_body(dec, p, B, K, V, M, vol, vol_elems, stats, ws, ws_bytes, stream), stream);
}

// ------------------------------------------------------------------ surface extraction
static vdm_status check_surface(int32_t R) {
  if (R < 1 || R > 893) return fail(VDM_ERR_INVALID_ARG, "R=%d (1 <= R <= 893)", R);
  return VDM_OK;
}

size_t vdm_surface_workspace_size(int32_t R) {
  if (check_surface(R) != VDM_OK) return 0;
  return surface_ws_layout(R).bytes;
}

static vdm_status extract_surface_body(const float* vol, int32_t R, const uint8_t* cell_mask, float* verts,
                               int64_t max_verts, int32_t* tris, int64_t max_tris, int64_t* vert_edges,
                               int64_t* counts, void* ws, size_t ws_bytes, vdm_stream stream) {
  vdm_status st = check_surface(R);
  if (st != VDM_OK) return st;
  if (!vol || !counts) return fail(VDM_ERR_INVALID_ARG, "vol or counts is NULL");
  if (max_verts < 0 || max_tris < 0) return fail(VDM_ERR_INVALID_ARG, "negative max_verts or max_tris");
  if ((max_verts > 0 && !verts) || (max_tris > 0 && !tris))
    return fail(VDM_ERR_INVALID_ARG, "verts or tris is NULL with a nonzero maximum");
  if (!aligned(vol, 4) || !aligned(counts, 8) || !aligned(verts, 4) || !aligned(tris, 4) || !aligned(vert_edges, 8))
    return fail(VDM_ERR_INVALID_ARG, "misaligned vol, verts, tris (4 bytes) or counts, vert_edges (8 bytes)");
  const size_t need = surface_ws_layout(R).bytes;
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed, got %zu", need, ws_bytes);
  (void)hipGetLastError();
  VDM_HIP_T(VDM_TIME_SURFACE, (hipStream_t)stream,
            launch_surface(vol, R, cell_mask, verts, max_verts, tris, max_tris, vert_edges, counts, (char*)ws,
                           (hipStream_t)stream),
            "surface launch");
  return VDM_OK;
}

vdm_status vdm_extract_surface(const float* vol, int32_t R, const uint8_t* cell_mask, float* verts,
                               int64_t max_verts, int32_t* tris, int64_t max_tris, int64_t* vert_edges,
                               int64_t* counts, void* ws, size_t ws_bytes, vdm_stream stream) {
  return debug_checked(extract_surface_body(vol, R, cell_mask, verts, max_verts, tris, max_tris, vert_edges, counts,
                                            ws, ws_bytes, stream), stream);
}

static vdm_status embed_queries_body(const vdm_decoder* dec, const float* xyz, int64_t N, void* Q, vdm_stream stream) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (N < 0 || N >= (1ll << 31)) return fail(VDM_ERR_INVALID_ARG, "N=%lld", (long long)N);
  if (N == 0) return VDM_OK;
  if (!xyz || !Q) return fail(VDM_ERR_INVALID_ARG, "xyz or Q is NULL");
  if (!aligned(xyz, 4) || !aligned(Q, 16)) return fail(VDM_ERR_INVALID_ARG, "misaligned xyz or Q");
  QuerySrc qs{0, 0, xyz, nullptr, 0};
  (void)hipGetLastError();
  VDM_HIP_T(VDM_TIME_EMBED, (hipStream_t)stream, launch_embed(dec->dtype, dec->D, qs, N, dec->Wq, Q, (hipStream_t)stream), "embed launch");
  return VDM_OK;
}

vdm_status vdm_embed_queries(const vdm_decoder* dec, const float* xyz, int64_t N, void* Q, vdm_stream stream) {
  return debug_checked(embed_queries_body(dec, xyz, N, Q, stream), stream);
}

static vdm_status project_kv_body(const vdm_decoder* dec, const void* Z, int64_t M, void* K, void* V, vdm_stream stream) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (M < 0 || M >= (1ll << 31) / dec->D) return fail(VDM_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (M == 0) return VDM_OK;
  if (!Z || !K || !V) return fail(VDM_ERR_INVALID_ARG, "Z, K or V is NULL");
  if (!aligned(Z, 16) || !aligned(K, 16) || !aligned(V, 16)) return fail(VDM_ERR_INVALID_ARG, "misaligned Z, K or V");
  (void)hipGetLastError();
  VDM_HIP_T(VDM_TIME_PROJECT_KV, (hipStream_t)stream, launch_project_kv(dec->dtype, Z, dec->Wk, dec->Wv, (int)M, dec->D, K, V, (hipStream_t)stream),
          "project_kv launch");
  return VDM_OK;
}

vdm_status vdm_project_kv(const vdm_decoder* dec, const void* Z, int64_t M, void* K, void* V, vdm_stream stream) {
  return debug_checked(project_kv_body(dec, Z, M, K, V, stream), stream);
}

// Checks shared by the dense decode calls (decoder, queries, K/V, output).
// *done = true when there is nothing to do (N = 0).
static vdm_status check_dense(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V, int64_t M,
                              const float* sdf, bool* done) {
  *done = false;
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (!q) return fail(VDM_ERR_INVALID_ARG, "queries is NULL");
  if (q->N < 0 || q->N >= (1ll << 31)) return fail(VDM_ERR_INVALID_ARG, "N=%lld", (long long)q->N);
  if (q->mode < VDM_Q_POINTS || q->mode > VDM_Q_GRID_LIST) return fail(VDM_ERR_INVALID_ARG, "query mode %d", q->mode);
  if (q->mode != VDM_Q_POINTS) {
    if (q->R < 1 || q->R > 1200) return fail(VDM_ERR_INVALID_ARG, "grid R=%d outside 1..1200", q->R);
    const int64_t P = q->R + 1;
    if (q->mode == VDM_Q_GRID && q->N != P * P * P)
      return fail(VDM_ERR_INVALID_ARG, "grid mode needs N=(R+1)^3=%lld (got %lld)", (long long)(P * P * P), (long long)q->N);
  }
  if (q->N == 0) {
    *done = true;
    return VDM_OK;
  }
  if (M < 1 || M >= (1ll << 31) / dec->D) return fail(VDM_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (!K || !V || !sdf) return fail(VDM_ERR_INVALID_ARG, "K, V or sdf is NULL");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(sdf, 4)) return fail(VDM_ERR_INVALID_ARG, "misaligned K, V or sdf");
  if (q->mode == VDM_Q_POINTS && (!q->xyz || !aligned(q->xyz, 4))) return fail(VDM_ERR_INVALID_ARG, "xyz NULL or misaligned");
  if (q->mode == VDM_Q_GRID_LIST && (!q->list || !aligned(q->list, 4)))
    return fail(VDM_ERR_INVALID_ARG, "list NULL or misaligned");
  return VDM_OK;
}

// Full-attention decode over a carved dense workspace: key norms, packed
// weights, packed K/V, then the decode launch. timed: record the decode launch
// for vdm_timing.
static vdm_status dense_full(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V, int64_t M,
                             float* sdf, const DenseWs& w, hipStream_t s, bool timed) {
  DecodeArgs a = base_args(dec);
  a.qs = QuerySrc{q->mode, q->R, q->xyz, q->list, 0};
  a.N = q->N;
  a.out = sdf;
  a.scatter = 0;
  a.kmax = w.kmax;
  VDM_HIP(launch_zero(w.kmax, 256, s), "zero launch");
  VDM_HIP(launch_key_norms(dec->dtype, K, (int)M, dec->H, w.kmax, s), "key norms launch");
  VDM_HIP(pack_weights(dec, w.Wp, a, s), "weight packing launch");
  VDM_HIP(launch_pack_kv(dec->dtype, K, V, (int)M, dec->D, (int)mpad(M), w.Kp, w.Vt, s), "pack_kv launch");
  a.Kp = w.Kp;
  a.Vt = w.Vt;
  a.M = (int)M;
  a.n_tiles = (q->N + decode_tile_queries(dec->dtype, dec->D) - 1) / decode_tile_queries(dec->dtype, dec->D);
  if (w.split.parts > 1) {
    a.split = w.split.parts;
    a.split_tiles = w.split.tiles;
    a.part = w.part;
    a.part_cnt = w.part_cnt;
    VDM_HIP(launch_zero(w.part_cnt, w.split.cnt_bytes, s), "zero launch");
  }
  // the work-unit counter: byte 128 of the key-norm slot (256 bytes, zeroed above)
  a.queue = reinterpret_cast<unsigned long long*>((char*)w.kmax + 128);
  if (timed)
    VDM_HIP_T(VDM_TIME_DECODE, s, launch_decode(dec->dtype, dec->D, false, a, s), "decode launch");
  else
    VDM_HIP(launch_decode(dec->dtype, dec->D, false, a, s), "decode launch");
  return VDM_OK;
}

// ------------------------------------------------------------------ no-allocation scratch
// The scratch of vdm_decode_dense_noalloc: one array per GPU, held until the
// process ends. Host code uses only its device address from hipGetSymbolAddress
// (per device, taken once with that device current), never the array's name.
static __device__ __align__(256) char scratch[VDM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NA_MAX_DEV = 64;
std::mutex g_na_mu;
void* g_na_ptr[NA_MAX_DEV];
}  // namespace

static vdm_status noalloc_scratch(void** out) {
  int dev = 0;
  VDM_HIP(hipGetDevice(&dev), "device query");
  if (dev < 0 || dev >= NA_MAX_DEV) return fail(VDM_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> g(g_na_mu);
  if (!g_na_ptr[dev]) {
    void* p = nullptr;
    VDM_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (!p) return fail(VDM_ERR_HIP, "scratch symbol address is NULL");
    g_na_ptr[dev] = p;
  }
  *out = g_na_ptr[dev];
  return VDM_OK;
}

static vdm_status decode_dense_body(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V, int64_t M,
                            const vdm_kvsel* sel, float* sdf, void* ws, size_t ws_bytes, vdm_stream stream) {
  bool done = false;
  vdm_status st = check_dense(dec, q, K, V, M, sdf, &done);
  if (st != VDM_OK || done) return st;
  if (sel) {
    if (q->mode != VDM_Q_GRID_LIST) return fail(VDM_ERR_INVALID_ARG, "token selection needs grid-list queries");
    if (sel->block < 1 || sel->cap < 1 || !sel->sel_idx || !sel->sel_cnt || (sel->heads != 0 && sel->heads != 1))
      return fail(VDM_ERR_INVALID_ARG, "bad kvsel (block=%d cap=%d heads=%d)", sel->block, sel->cap, sel->heads);
  }
  const size_t need = dense_ws(dec, M, q->N, sel != nullptr, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace needs %zu bytes, 256-aligned (got %zu)", need, ws_bytes);
  DenseWs w;
  dense_ws(dec, M, q->N, sel != nullptr, ws, &w);
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  if (!sel) return dense_full(dec, q, K, V, M, sdf, w, s, true);
  {
    DecodeArgs a = base_args(dec);
    a.qs = QuerySrc{q->mode, q->R, q->xyz, q->list, 0};
    a.N = q->N;
    a.out = sdf;
    a.scatter = 0;
    a.kmax = w.kmax;
    VDM_HIP(launch_zero(w.kmax, 256, s), "zero launch");
    VDM_HIP(launch_key_norms(dec->dtype, K, (int)M, dec->H, w.kmax, s), "key norms launch");
    VDM_HIP(pack_weights(dec, w.Wp, a, s), "weight packing launch");
    const int bq = decode_tile_queries(dec->dtype, dec->D);
    VDM_HIP(launch_zero(w.n_items, 256, s), "zero launch");
    VDM_HIP(launch_items_from_list(q->list, q->N, q->R, sel->block, sel->block_row, bq, w.items, w.n_items, sdf, s),
            "items launch");
    a.Kp = K;
    a.Vt = V;
    a.M = (int)M;
    a.items = w.items;
    a.n_tiles = q->N;
    a.d_n_items = w.n_items;
    a.sel_idx = sel->sel_idx;
    a.sel_cnt = sel->sel_cnt;
    a.cap = sel->cap;
    a.heads = sel->heads;
    // the work-item queue: byte 128 of the item count's 256-byte slot, zeroed with it
    a.queue = reinterpret_cast<unsigned long long*>((char*)w.n_items + 128);
    VDM_HIP_T(VDM_TIME_DECODE_GATHERED, s, launch_decode(dec->dtype, dec->D, true, a, s), "gathered decode launch");
  }
  return VDM_OK;
}

vdm_status vdm_decode_dense(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V, int64_t M,
                            const vdm_kvsel* sel, float* sdf, void* ws, size_t ws_bytes, vdm_stream stream) {
  return debug_checked(decode_dense_body(dec, q, K, V, M, sel, sdf, ws, ws_bytes, stream), stream);
}

static vdm_status decode_dense_noalloc_body(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V,
                                    int64_t M, float* sdf, vdm_stream stream) {
  bool done = false;
  vdm_status st = check_dense(dec, q, K, V, M, sdf, &done);
  if (st != VDM_OK || done) return st;
  const size_t need = dense_ws(dec, M, q->N, false, nullptr, nullptr, false);
  if (need > (size_t)VDM_NOALLOC_SCRATCH_BYTES)
    return fail(VDM_ERR_WORKSPACE, "M=%lld needs %zu bytes of scratch; the no-allocation decode holds %zu",
                (long long)M, need, (size_t)VDM_NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  st = noalloc_scratch(&base);
  if (st != VDM_OK) return st;
  DenseWs w;
  dense_ws(dec, M, q->N, false, base, &w, false);
  (void)hipGetLastError();
  return dense_full(dec, q, K, V, M, sdf, w, (hipStream_t)stream, false);
}

vdm_status vdm_decode_dense_noalloc(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V,
                                    int64_t M, float* sdf, vdm_stream stream) {
  return debug_checked(decode_dense_noalloc_body(dec, q, K, V, M, sdf, stream), stream);
}

size_t vdm_dense_batch_workspace_size(const vdm_decoder* dec, int32_t B, int64_t M) {
  if (check_decoder(dec) != VDM_OK) return 0;
  if (B < 1 || B > 4096 || M < 1 || M >= (1ll << 31) / dec->D) {
    fail(VDM_ERR_INVALID_ARG, "B=%d M=%lld", B, (long long)M);
    return 0;
  }
  return batch_ws(dec, B, M, nullptr, nullptr);
}

static vdm_status decode_dense_batch_body(const vdm_decoder* dec, const vdm_queries* q, int32_t B, const void* K,
                                  const void* V, int64_t M, float* sdf, void* ws, size_t ws_bytes,
                                  vdm_stream stream) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (B < 1 || B > 4096) return fail(VDM_ERR_INVALID_ARG, "B=%d (1..4096)", B);
  if (!q) return fail(VDM_ERR_INVALID_ARG, "queries is NULL");
  if (q->N < 0 || q->N >= (1ll << 31)) return fail(VDM_ERR_INVALID_ARG, "N=%lld", (long long)q->N);
  if (q->mode < VDM_Q_POINTS || q->mode > VDM_Q_GRID_LIST) return fail(VDM_ERR_INVALID_ARG, "query mode %d", q->mode);
  if (q->mode != VDM_Q_POINTS) {
    if (q->R < 1 || q->R > 1200) return fail(VDM_ERR_INVALID_ARG, "grid R=%d outside 1..1200", q->R);
    const int64_t P = q->R + 1;
    if (q->mode == VDM_Q_GRID && q->N != P * P * P)
      return fail(VDM_ERR_INVALID_ARG, "grid mode needs N=(R+1)^3=%lld (got %lld)", (long long)(P * P * P), (long long)q->N);
  }
  if (q->N == 0) return VDM_OK;
  if (M < 1 || M >= (1ll << 31) / dec->D) return fail(VDM_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (!K || !V || !sdf) return fail(VDM_ERR_INVALID_ARG, "K, V or sdf is NULL");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(sdf, 4)) return fail(VDM_ERR_INVALID_ARG, "misaligned K, V or sdf");
  if ((M * dec->D * (int64_t)esize(dec->dtype)) % 16 != 0)
    return fail(VDM_ERR_INVALID_ARG, "each shape's K/V must start 16-byte aligned (M * D * element size)");
  if (q->mode == VDM_Q_POINTS && (!q->xyz || !aligned(q->xyz, 4))) return fail(VDM_ERR_INVALID_ARG, "xyz NULL or misaligned");
  if (q->mode == VDM_Q_GRID_LIST && (!q->list || !aligned(q->list, 4)))
    return fail(VDM_ERR_INVALID_ARG, "list NULL or misaligned");
  const size_t need = batch_ws(dec, B, M, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace needs %zu bytes, 256-aligned (got %zu)", need, ws_bytes);
  BatchWs w;
  batch_ws(dec, B, M, ws, &w);
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  DecodeArgs a = base_args(dec);
  a.qs = QuerySrc{q->mode, q->R, q->xyz, q->list, 0};
  a.N = q->N;
  a.out = sdf;
  a.scatter = 0;
  a.kmax = w.kmax;
  const size_t shape_bytes = (size_t)M * dec->D * esize(dec->dtype);
  VDM_HIP(launch_zero(w.kmax, ((size_t)B * dec->H * 4 + 7) / 8 * 8, s), "zero launch");  // (within its 256-byte slot)
  VDM_HIP(pack_weights(dec, w.Wp, a, s), "weight packing launch");
  // every shape's key norms and packed K/V, one launch each for the batch
  VDM_HIP(launch_key_norms(dec->dtype, K, (int)M, dec->H, w.kmax, s, B, (int64_t)shape_bytes, (int64_t)dec->H * 4),
          "key norms launch");
  VDM_HIP(launch_pack_kv(dec->dtype, K, V, (int)M, dec->D, (int)mpad(M), w.Kp, w.Vt, s, B, (int64_t)shape_bytes,
                         (int64_t)w.kv),
          "pack_kv launch");
  a.Kp = w.Kp;
  a.Vt = w.Vt;
  a.M = (int)M;
  a.batch = B;
  a.kv_stride = (int64_t)w.kv;
  a.out_stride = q->N;
  VDM_HIP(launch_zero(w.queue, 256, s), "zero launch");
  a.queue = w.queue;
  VDM_HIP_T(VDM_TIME_DECODE, s, launch_decode(dec->dtype, dec->D, false, a, s), "batched decode launch");
  return VDM_OK;
}

vdm_status vdm_decode_dense_batch(const vdm_decoder* dec, const vdm_queries* q, int32_t B, const void* K,
                                  const void* V, int64_t M, float* sdf, void* ws, size_t ws_bytes,
                                  vdm_stream stream) {
  return debug_checked(decode_dense_batch_body(dec, q, B, K, V, M, sdf, ws, ws_bytes, stream), stream);
}

}  // extern "C"

static vdm_status select_kv(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap, int32_t probes,
                            uint64_t seed, const void* K, int64_t M, const int32_t* blocks, int64_t nblk,
                            int32_t* sel_idx, int32_t* sel_cnt, void* ws, size_t ws_bytes, vdm_stream stream,
                            bool heads) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (R < 1 || R > 1200 || block < 1) return fail(VDM_ERR_INVALID_ARG, "R=%d block=%d", R, block);
  if (M < 1 || M > select_max_tokens(heads))
    return fail(M < 1 ? VDM_ERR_INVALID_ARG : VDM_ERR_UNSUPPORTED, "M=%lld (1..%d)", (long long)M, select_max_tokens(heads));
  if (k < 1 || k > M || cap < k) return fail(VDM_ERR_INVALID_ARG, "k=%d cap=%d M=%lld", k, cap, (long long)M);
  if (!select_fits(M, k, cap, heads))
    return fail(VDM_ERR_UNSUPPORTED, "k=%d cap=%d with M=%lld: k * ceil(M / 4096) must be <= 1024, and 8 k <= 1024 unless cap >= 8 k",
                k, cap, (long long)M);
  if (probes != 0 && probes != 1) return fail(VDM_ERR_INVALID_ARG, "probes=%d (0: corners, 1: random)", probes);
  const int64_t NB = (R + block) / block;
  if (nblk < 0 || (!blocks && nblk != NB * NB * NB))
    return fail(VDM_ERR_INVALID_ARG, "nblk=%lld (all blocks: %lld)", (long long)nblk, (long long)(NB * NB * NB));
  if (nblk == 0) return VDM_OK;
  if (!K || !sel_idx || !sel_cnt || !aligned(K, 16)) return fail(VDM_ERR_INVALID_ARG, "K, sel_idx or sel_cnt NULL/misaligned");
  const size_t need = select_ws_bytes(dec, M, heads);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  char* kp = static_cast<char*>(ws) + (select_scratch_bytes((int)M, sel_sets(dec, heads)) + 255) / 256 * 256;
  if (dec->dtype == VDM_BF16)
    VDM_HIP(launch_pack_kv(dec->dtype, K, nullptr, (int)M, dec->D, (int)mpad(M), kp, nullptr, s), "pack K launch");
  SelectArgs a;
  memset(&a, 0, sizeof a);
  a.R = R;
  a.block = block;
  a.k = k;
  a.cap = cap;
  a.probes = probes;
  a.seed = seed;
  a.M = (int)M;
  a.H = dec->H;
  a.D = dec->D;
  a.Wq = dec->Wq;
  a.K = K;
  a.Kp = kp;
  a.blocks = blocks;
  a.n_blocks = nblk;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.scores = (float*)ws;
  a.per_head = heads ? 1 : 0;
  VDM_HIP_T(VDM_TIME_SELECT, s, launch_select(dec->dtype, a, s), "select launch");
  return VDM_OK;
}

extern "C" {

static vdm_status select_kv_body(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap, int32_t probes,
                         uint64_t seed, const void* K, int64_t M, const int32_t* blocks, int64_t nblk, int32_t* sel_idx,
                         int32_t* sel_cnt, void* ws, size_t ws_bytes, vdm_stream stream) {
  return select_kv(dec, R, block, k, cap, probes, seed, K, M, blocks, nblk, sel_idx, sel_cnt, ws, ws_bytes, stream,
                   false);
}

vdm_status vdm_select_kv(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap, int32_t probes,
                         uint64_t seed, const void* K, int64_t M, const int32_t* blocks, int64_t nblk, int32_t* sel_idx,
                         int32_t* sel_cnt, void* ws, size_t ws_bytes, vdm_stream stream) {
  return debug_checked(select_kv_body(dec, R, block, k, cap, probes, seed, K, M, blocks, nblk, sel_idx, sel_cnt, ws,
                                      ws_bytes, stream), stream);
}

static vdm_status select_kv_heads_body(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap,
                               int32_t probes, uint64_t seed, const void* K, int64_t M, const int32_t* blocks,
                               int64_t nblk, int32_t* sel_idx, int32_t* sel_cnt, void* ws, size_t ws_bytes,
                               vdm_stream stream) {
  return select_kv(dec, R, block, k, cap, probes, seed, K, M, blocks, nblk, sel_idx, sel_cnt, ws, ws_bytes, stream,
                   true);
}

vdm_status vdm_select_kv_heads(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap,
                               int32_t probes, uint64_t seed, const void* K, int64_t M, const int32_t* blocks,
                               int64_t nblk, int32_t* sel_idx, int32_t* sel_cnt, void* ws, size_t ws_bytes,
                               vdm_stream stream) {
  return debug_checked(select_kv_heads_body(dec, R, block, k, cap, probes, seed, K, M, blocks, nblk, sel_idx,
                                            sel_cnt, ws, ws_bytes, stream), stream);
}


}  // extern "C"

// The hierarchical level loop for B shapes at once: shape b uses K, V at byte
// offset b * kv_bytes, its volume at vol + b * vol_stride floats, its counters at
// S + b * st_stride int64 and workspace slice ws + b * ws_stride bytes (each
// slice laid out by hier_ws). Every mask stage is one launch for all B shapes
// (gridDim.y = B), and so are the selection and the decode of a level. The packed
// epilogue weights of slice 0 serve every shape. dbg: B = 1 only.
static vdm_status hier_run(const vdm_decoder* dec, const vdm_hier_params* p, int B, const void* K, const void* V,
                           int64_t M, size_t kv_bytes, float* vol, int64_t vol_stride, int64_t* S, int64_t st_stride,
                           const vdm_hier_debug* dbg, void* ws, size_t ws_stride, hipStream_t s) {
  HierWs w;
  hier_ws(dec, p, M, ws, &w);
  const int bq = decode_tile_queries(dec->dtype, dec->D);
  const bool kv = p->use_kvsel != 0;
  const int64_t wst = (int64_t)ws_stride, sst = st_stride * 8, vst = vol_stride * 4;
  auto off = [](const void* q, int64_t bytes) { return (const char*)q + bytes; };
  auto shape_of = [&](auto* q, int b) { return (decltype(q))((char*)q + (int64_t)b * wst); };

  VDM_HIP(launch_stats_init(bp(S, sst), p->levels, p->R0, B, s), "stats init");
  VDM_HIP(launch_zero_b(BP<void>{w.part, wst}, (size_t)stat_part_words() * 8, B, s), "zero launch");
  VDM_HIP(launch_zero_b(BP<void>{w.kmax, wst}, 256, B, s), "zero launch");
  VDM_HIP(launch_zero(w.queues, (size_t)VDM_MAX_LEVELS * 8, s), "zero launch");
  // every shape's key norms and packed K/V (packed K only with KV selection, which
  // streams it; bf16), one launch each for the batch
  VDM_HIP(launch_key_norms(dec->dtype, K, (int)M, dec->H, w.kmax, s, B, (int64_t)kv_bytes, wst), "key norms launch");
  if (!kv)
    VDM_HIP(launch_pack_kv(dec->dtype, K, V, (int)M, dec->D, (int)mpad(M), w.Kp, w.Vt, s, B, (int64_t)kv_bytes, wst),
            "pack_kv launch");
  else if (dec->dtype == VDM_BF16)
    VDM_HIP(launch_pack_kv(dec->dtype, K, nullptr, (int)M, dec->D, (int)mpad(M), w.Kp, nullptr, s, B,
                           (int64_t)kv_bytes, wst),
            "pack K launch");
  DecodeArgs packed = base_args(dec);
  VDM_HIP(pack_weights(dec, w.Wp, packed, s), "weight packing launch");

  // the level's volume of shape 0 and its stride (the last level is the caller's)
  auto vol_of = [&](int L) { return L == p->levels - 1 ? vol : w.vol[L]; };
  auto vstride = [&](int L) { return L == p->levels - 1 ? vst : wst; };
  // list, items and occupied blocks of level L are in w.list / w.items / w.occ
  // The selection, then the decode, each one launch for all shapes: with B > 1
  // they take their groups of blocks, tiles or work items shape by shape from a
  // device-side prefix of the shapes' counts.
  auto decode_level = [&](int L) -> vdm_status {
    const int R = p->R0 << L;
    {
      int32_t* tot = w.totals + 4 * L;  // shape 0's counts: queries, work items, occupied blocks
      const void* Kb = K;
      if (kv) {
        SelectArgs sa;
        memset(&sa, 0, sizeof sa);
        sa.R = R;
        sa.block = 8;
        sa.k = p->k;
        sa.cap = p->cap;
        sa.probes = p->probes;
        sa.seed = p->seed + (uint64_t)R;  // a different stream per level
        sa.M = (int)M;
        sa.H = dec->H;
        sa.D = dec->D;
        sa.Wq = dec->Wq;
        sa.K = Kb;
        sa.Kp = w.Kp;
        sa.blocks = w.occ;
        sa.n_blocks = 0;
        sa.d_n_blocks = tot + 2;
        sa.sel_idx = w.sel_idx;
        sa.sel_cnt = w.sel_cnt;
        sa.stat_selected = S + L * VDM_STAT_FIELDS + VDM_STAT_SELECTED;
        sa.scores = w.sel_scores;  // (per workgroup, so slice 0's serves the batch)
        sa.per_head = p->heads;
        if (B > 1) {
          VDM_HIP_T(VDM_TIME_SCAN, s,
                    launch_batch_prefix(tot + 2, wst / 4, B, select_blocks_per_group(), w.bprefix, s),
                    "prefix launch");
          sa.batch = B;
          sa.grp_prefix = w.bprefix;
          sa.cnt_stride = wst / 4;
          sa.blocks_stride = wst;
          sa.k_stride = (int64_t)kv_bytes;
          sa.kp_stride = wst;
          sa.sel_stride = wst;
          sa.stat_stride = sst;
        }
        VDM_HIP_T(VDM_TIME_SELECT, s, launch_select(dec->dtype, sa, s), "select launch");
      }
    }
    int32_t* tot = w.totals + 4 * L;  // shape 0's counts: queries, work items
    DecodeArgs a = packed;
    a.qs = QuerySrc{VDM_Q_GRID_LIST, R, nullptr, w.list, 0};
    a.kmax = w.kmax;
    a.out = (float*)vol_of(L);
    a.scatter = 1;
    a.M = (int)M;
    a.d_N = tot;  // the level's query count (the list length)
    if (kv) {
      a.Kp = K;
      a.Vt = V;
      a.items = w.items;
      a.d_n_items = tot + 1;
      a.sel_idx = w.sel_idx;
      a.sel_cnt = w.sel_cnt;
      a.cap = p->cap;
      a.heads = p->heads;
    } else {
      a.Kp = w.Kp;
      a.Vt = w.Vt;
    }
    a.queue = w.queues + L;  // the level's work-unit counter (zeroed once, before level 0)
    if (B > 1) {
      VDM_HIP_T(VDM_TIME_SCAN, s,
                launch_batch_prefix(kv ? tot + 1 : tot, wst / 4, B, kv ? 1 : bq, w.bprefix, s), "prefix launch");
      a.batch = B;
      a.tile_prefix = w.bprefix;
      a.cnt_stride = wst / 4;
      a.list_stride = wst;
      a.items_stride = wst;
      a.sel_stride = wst;
      a.kmax_stride = wst / 4;
      a.kv_stride = kv ? (int64_t)kv_bytes : wst;
      a.out_stride = vstride(L) / 4;
    }
    VDM_HIP_T(kv ? VDM_TIME_DECODE_GATHERED : VDM_TIME_DECODE, s, launch_decode(dec->dtype, dec->D, kv, a, s),
              "decode launch");
    return VDM_OK;
  };

  auto BPt = [&](auto* q) { return bp(q, wst); };
  // level 0: every point, in blocked order
  {
    const int NB = nblocks8(p->R0 + 1);
    const int64_t nb3 = (int64_t)NB * NB * NB;
    VDM_HIP_T(VDM_TIME_MARK, s,
              launch_mark(BP<const uint64_t>{nullptr, 0}, 1, BP<const uint64_t>{nullptr, 0}, 1, p->R0, BPt(w.newmask),
                          BP<uint64_t>{nullptr, 0}, BPt(w.counts), B, s),
              "mark launch");
    VDM_HIP_T(VDM_TIME_SCAN, s,
              launch_scan(bp((const int32_t*)w.counts, wst), nb3, bq, BPt(w.partial), BPt(w.offs), BPt(w.occ),
                          BPt(w.totals), bp(S, sst), B, s),
              "scan launch");
    VDM_HIP_T(VDM_TIME_EMIT, s,
              launch_emit(bp((const uint64_t*)w.newmask, wst), bp((const int32_t*)w.counts, wst),
                          bp((const int4*)w.offs, wst), bp((const int32_t*)w.occ, wst),
                          bp((const int32_t*)w.totals, wst), p->R0, bq, BPt(w.list), w.list_cap, BPt(w.items),
                          w.item_cap, B, s),
              "emit launch");
    vdm_status st = decode_level(0);
    if (st != VDM_OK) return st;
  }
  for (int L = 0; L < p->levels; ++L) {
    const int R = p->R0 << L, P = R + 1, NB = nblocks8(P);
    int64_t* SL = S + L * VDM_STAT_FIELDS;
    VDM_HIP_T(VDM_TIME_CELL_TEST, s,
              launch_cell_test(bp((const float*)vol_of(L), vstride(L)), R,
                               bp((const uint64_t*)(L ? w.kept[L - 1] : nullptr), wst), p->tau, BPt(w.active[L]),
                               BPt(w.part), bp(SL + VDM_STAT_TESTED, sst), bp(SL + VDM_STAT_ACTIVE, sst), B, s),
              "cell test launch");
    if (dbg) {
      const int64_t p3 = (int64_t)P * P * P, nb3 = (int64_t)NB * NB * NB;
      if (dbg->vol[L] && L < p->levels - 1)
        VDM_HIP(hipMemcpyAsync(dbg->vol[L], vol_of(L), p3 * 4, hipMemcpyDeviceToDevice, s), "debug copy");
      if (dbg->vol[L] && L == p->levels - 1 && dbg->vol[L] != vol)
        VDM_HIP(hipMemcpyAsync(dbg->vol[L], vol, p3 * 4, hipMemcpyDeviceToDevice, s), "debug copy");
      if (dbg->active[L]) VDM_HIP(launch_bits_to_bytes(w.active[L], R, NB, dbg->active[L], s), "debug export");
      if (dbg->list[L]) VDM_HIP(hipMemcpyAsync(dbg->list[L], w.list, p3 * 4, hipMemcpyDeviceToDevice, s), "debug copy");
      if (kv && dbg->sel_blocks[L])
        VDM_HIP(hipMemcpyAsync(dbg->sel_blocks[L], w.occ, nb3 * 4, hipMemcpyDeviceToDevice, s), "debug copy");
      const int64_t ns = kv && p->heads ? dec->H : 1;
      if (kv && dbg->sel_cnt[L])
        VDM_HIP(hipMemcpyAsync(dbg->sel_cnt[L], w.sel_cnt, nb3 * ns * 4, hipMemcpyDeviceToDevice, s), "debug copy");
      if (kv && dbg->sel_idx[L])
        VDM_HIP(hipMemcpyAsync(dbg->sel_idx[L], w.sel_idx, nb3 * ns * p->cap * 4, hipMemcpyDeviceToDevice, s),
                "debug copy");
    }
    if (L == p->levels - 1) break;
    // kept = active dilated `dilation` times (ping-pong through tmp)
    if (p->dilation == 0) {
      VDM_HIP_T(VDM_TIME_DILATE, s,
                launch_dilate(bp((const uint64_t*)w.active[L], wst), BPt(w.kept[L]), R, 1, BPt(w.part),
                              bp(SL + VDM_STAT_KEPT, sst), B, s),
                "copy launch");
    } else {
      const uint64_t* src = w.active[L];
      for (int t = 0; t < p->dilation; ++t) {
        uint64_t* dst = ((p->dilation - 1 - t) % 2 == 0) ? w.kept[L] : w.tmp;
        VDM_HIP_T(VDM_TIME_DILATE, s,
                  launch_dilate(bp(src, wst), BPt(dst), R, 0, BPt(w.part),
                                t == p->dilation - 1 ? bp(SL + VDM_STAT_KEPT, sst) : BP<int64_t>{nullptr, 0}, B, s),
                  "dilate launch");
        src = dst;
      }
    }
    if (dbg && dbg->kept[L]) VDM_HIP(launch_bits_to_bytes(w.kept[L], R, NB, dbg->kept[L], s), "debug export");
    const int Rn = 2 * R, Pn = Rn + 1, NBn = nblocks8(Pn);
    VDM_HIP_T(VDM_TIME_MARK, s,
              launch_mark(bp((const uint64_t*)w.kept[L], wst), R, bp((const uint64_t*)(L ? w.comp[L] : nullptr), wst), 0,
                          Rn, BPt(w.newmask), BPt(w.comp[L + 1]), BPt(w.counts), B, s),
              "mark launch");
    VDM_HIP_T(VDM_TIME_SCAN, s,
              launch_scan(bp((const int32_t*)w.counts, wst), (int64_t)NBn * NBn * NBn, bq, BPt(w.partial), BPt(w.offs),
                          BPt(w.occ), BPt(w.totals + 4 * (L + 1)), bp(S + (L + 1) * VDM_STAT_FIELDS, sst), B, s),
              "scan launch");
    VDM_HIP_T(VDM_TIME_EMIT, s,
              launch_emit(bp((const uint64_t*)w.newmask, wst), bp((const int32_t*)w.counts, wst),
                          bp((const int4*)w.offs, wst), bp((const int32_t*)w.occ, wst),
                          bp((const int32_t*)(w.totals + 4 * (L + 1)), wst), Rn, bq, BPt(w.list), w.list_cap,
                          BPt(w.items), w.item_cap, B, s),
              "emit launch");
    VDM_HIP_T(VDM_TIME_FILL, s,
              launch_fill(bp((const float*)vol_of(L), vstride(L)), P, bp(vol_of(L + 1), vstride(L + 1)), Pn, B, s),
              "fill launch");
    vdm_status st = decode_level(L + 1);
    if (st != VDM_OK) return st;
  }
  return VDM_OK;
}

extern "C" {

static vdm_status decode_hier_body(const vdm_decoder* dec, const vdm_hier_params* p, const void* K, const void* V, int64_t M,
                           float* vol, int64_t vol_elems, int64_t* stats, const vdm_hier_debug* dbg, void* ws,
                           size_t ws_bytes, vdm_stream stream) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  st = check_hier(dec, p, M);
  if (st != VDM_OK) return st;
  const int64_t Rf = (int64_t)p->R0 << (p->levels - 1), Pf = Rf + 1;
  if (!vol || vol_elems < Pf * Pf * Pf)
    return fail(VDM_ERR_INVALID_ARG, "vol needs %lld floats", (long long)(Pf * Pf * Pf));
  if (!K || !V || !aligned(K, 16) || !aligned(V, 16) || !aligned(vol, 4))
    return fail(VDM_ERR_INVALID_ARG, "K, V or vol NULL/misaligned");
  const size_t need = hier_ws(dec, p, M, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace needs %zu bytes, 256-aligned (got %zu)", need, ws_bytes);
  HierWs w;
  hier_ws(dec, p, M, ws, &w);
  (void)hipGetLastError();
  int64_t* S = stats ? stats : w.stats;
  return hier_run(dec, p, 1, K, V, M, 0, vol, 0, S, 0, dbg, ws, 0, (hipStream_t)stream);
}

vdm_status vdm_decode_hier(const vdm_decoder* dec, const vdm_hier_params* p, const void* K, const void* V, int64_t M,
                           float* vol, int64_t vol_elems, int64_t* stats, const vdm_hier_debug* dbg, void* ws,
                           size_t ws_bytes, vdm_stream stream) {
  return debug_checked(decode_hier_body(dec, p, K, V, M, vol, vol_elems, stats, dbg, ws, ws_bytes, stream), stream);
}

// ------------------------------------------------------------------ local KNN decoder
}  // extern "C"

namespace vdm {

struct LocalWs {
  int32_t* counts;   // support buckets
  int32_t* fill;
  int32_t* starts;
  int32_t* cell_of;
  uint32_t* occ;
  float4* spos;
  int32_t* qcounts;  // query buckets (processing order)
  int32_t* qfill;
  int32_t* qstarts;
  int32_t* qcell;
  int32_t* order;
  int32_t* nbr;
  void* h;
  void* Wp;
};

static size_t local_ws(const vdm_local_decoder* d, int64_t M, int64_t N, void* base, LocalWs* w) {
  Carve c(base);
  LocalWs x;
  constexpr size_t NC = (size_t)LOCAL_G * LOCAL_G * LOCAL_G;
  const size_t n1 = (size_t)(N > 0 ? N : 1);
  x.counts = c.take<int32_t>(NC * 4);
  x.fill = c.take<int32_t>(NC * 4);
  x.starts = c.take<int32_t>((NC + 1) * 4);
  x.cell_of = c.take<int32_t>((size_t)M * 4);
  x.occ = c.take<uint32_t>((size_t)LOCAL_G * LOCAL_G * 4);
  x.spos = c.take<float4>((size_t)M * 16);
  x.qcounts = c.take<int32_t>(NC * 4);
  x.qfill = c.take<int32_t>(NC * 4);
  x.qstarts = c.take<int32_t>((NC + 1) * 4);
  x.qcell = c.take<int32_t>(n1 * 4);
  x.order = c.take<int32_t>(n1 * 4);
  x.nbr = c.take<int32_t>((size_t)(N > 0 ? N : 1) * LOCAL_K * 4);
  x.h = c.take<char>((size_t)(N > 0 ? N : 1) * LOCAL_C * 2);
  x.Wp = c.take<char>((size_t)2 * d->C * d->F * 2);
  if (w) *w = x;
  return c.off + 256;
}

static vdm_status check_local(const vdm_local_decoder* d) {
  if (!d) return fail(VDM_ERR_INVALID_ARG, "local decoder is NULL");
  if (d->C != LOCAL_C || d->K != LOCAL_K || d->hidden != LOCAL_HIDDEN)
    return fail(VDM_ERR_UNSUPPORTED, "local decoder needs C=%d K=%d hidden=%d (got %d, %d, %d)", LOCAL_C, LOCAL_K,
                LOCAL_HIDDEN, d->C, d->K, d->hidden);
  if (d->F < 256 || d->F > 4096 || d->F % 256)
    return fail(VDM_ERR_UNSUPPORTED, "F=%d must be a multiple of 256 in [256, 4096]", d->F);
  if (!d->A || !d->a || !d->B || !d->W1 || !d->W2 || !d->w_head)
    return fail(VDM_ERR_INVALID_ARG, "a local decoder weight pointer is NULL");
  if (!aligned(d->A, 4) || !aligned(d->a, 4) || !aligned(d->w_head, 4) || !aligned(d->B, 16) || !aligned(d->W1, 16) ||
      !aligned(d->W2, 16))
    return fail(VDM_ERR_INVALID_ARG, "misaligned local decoder weights (A, a, w_head: 4 bytes; B, W1, W2: 16)");
  if (d->n_prims < 1 || d->n_prims > VDM_MAX_PRIMS) return fail(VDM_ERR_INVALID_ARG, "n_prims=%d", d->n_prims);
  for (int i = 0; i < d->n_prims; ++i)
    if (d->prims[i].kind != VDM_PRIM_SPHERE && d->prims[i].kind != VDM_PRIM_BOX)
      return fail(VDM_ERR_INVALID_ARG, "primitive %d has kind %d", i, d->prims[i].kind);
  if (!isfinite(d->net_scale)) return fail(VDM_ERR_INVALID_ARG, "net_scale is not finite");
  return VDM_OK;
}

}  // namespace vdm

extern "C" {

size_t vdm_local_workspace_size(const vdm_local_decoder* dec, int64_t M, int64_t N) {
  if (check_local(dec) != VDM_OK) return 0;
  if (M < 1 || M >= (1ll << 31) / LOCAL_C || N < 0 || N >= (1ll << 31) / LOCAL_C) {
    fail(VDM_ERR_INVALID_ARG, "M=%lld N=%lld", (long long)M, (long long)N);
    return 0;
  }
  return local_ws(dec, M, N, nullptr, nullptr);
}

static vdm_status decode_local_body(const vdm_local_decoder* dec, const float* sup_xyz, const void* feats, int64_t M,
                            const float* xyz, int64_t N, float* sdf, int32_t* nbr, void* ws, size_t ws_bytes,
                            vdm_stream stream) {
  vdm_status st = check_local(dec);
  if (st != VDM_OK) return st;
  if (N < 0 || N >= (1ll << 31) / LOCAL_C) return fail(VDM_ERR_INVALID_ARG, "N=%lld", (long long)N);
  if (N == 0) return VDM_OK;
  if (M < dec->K || M >= (1ll << 31) / LOCAL_C)
    return fail(VDM_ERR_INVALID_ARG, "M=%lld (K=%d <= M < %lld)", (long long)M, dec->K, (1ll << 31) / LOCAL_C);
  if (!sup_xyz || !feats || !xyz || !sdf) return fail(VDM_ERR_INVALID_ARG, "sup_xyz, feats, xyz or sdf is NULL");
  if (!aligned(sup_xyz, 4) || !aligned(feats, 16) || !aligned(xyz, 4) || !aligned(sdf, 4) || !aligned(nbr, 4))
    return fail(VDM_ERR_INVALID_ARG, "misaligned sup_xyz, xyz, sdf, nbr (4 bytes) or feats (16 bytes)");
  const size_t need = local_ws(dec, M, N, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace needs %zu bytes, 256-aligned (got %zu)", need, ws_bytes);
  LocalWs w;
  local_ws(dec, M, N, ws, &w);
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  int32_t* nb = nbr ? nbr : w.nbr;
  constexpr size_t NC = (size_t)LOCAL_G * LOCAL_G * LOCAL_G;
  VDM_HIP(launch_zero(w.counts, NC * 4, s), "zero launch");
  VDM_HIP(launch_zero(w.fill, NC * 4, s), "zero launch");
  VDM_HIP(launch_zero(w.qcounts, NC * 4, s), "zero launch");
  VDM_HIP(launch_zero(w.qfill, NC * 4, s), "zero launch");
  VDM_HIP_T(VDM_TIME_LOCAL_GRID, s,
            launch_local_grid(sup_xyz, M, w.counts, w.starts, w.fill, w.cell_of, w.spos, nullptr, w.occ, s),
            "support grid launch");
  VDM_HIP_T(VDM_TIME_LOCAL_GRID, s,
            launch_local_grid(xyz, N, w.qcounts, w.qstarts, w.qfill, w.qcell, nullptr, w.order, nullptr, s),
            "query order launch");
  VDM_HIP_T(VDM_TIME_LOCAL_KNN, s, launch_local_knn(xyz, N, w.order, w.starts, w.occ, w.spos, nb, s), "knn launch");
  LocalFuseArgs fa;
  fa.sup_xyz = sup_xyz;
  fa.feats = feats;
  fa.M = (int)M;
  fa.xyz = xyz;
  fa.N = N;
  fa.nbr = nb;
  fa.A = dec->A;
  fa.a = dec->a;
  fa.B = dec->B;
  fa.h = w.h;
  VDM_HIP_T(VDM_TIME_LOCAL_FUSE, s, launch_local_fuse(fa, s), "fuse launch");
  const size_t CF = (size_t)dec->C * dec->F * 2;
  char* wp = static_cast<char*>(w.Wp);
  VDM_HIP(launch_pack_w(dec->W1, dec->F, dec->C, wp, s), "weight packing launch");
  VDM_HIP(launch_pack_w(dec->W2, dec->C, dec->F, wp + CF, s), "weight packing launch");
  HeadArgs ha;
  memset(&ha, 0, sizeof ha);
  ha.xyz = xyz;
  ha.N = N;
  ha.h = w.h;
  ha.W1 = wp;
  ha.W2 = wp + CF;
  ha.w_head = dec->w_head;
  ha.F = dec->F;
  ha.net_scale = dec->net_scale;
  ha.prims.n = dec->n_prims;
  for (int i = 0; i < dec->n_prims; ++i) {
    ha.prims.p[i].kind = dec->prims[i].kind;
    for (int c = 0; c < 3; ++c) {
      ha.prims.p[i].c[c] = dec->prims[i].centre[c];
      ha.prims.p[i].s[c] = dec->prims[i].size[c];
    }
  }
  ha.out = sdf;
  VDM_HIP_T(VDM_TIME_LOCAL_HEAD, s, launch_local_head(ha, s), "head launch");
  return VDM_OK;
}

vdm_status vdm_decode_local(const vdm_local_decoder* dec, const float* sup_xyz, const void* feats, int64_t M,
                            const float* xyz, int64_t N, float* sdf, int32_t* nbr, void* ws, size_t ws_bytes,
                            vdm_stream stream) {
  return debug_checked(decode_local_body(dec, sup_xyz, feats, M, xyz, N, sdf, nbr, ws, ws_bytes, stream), stream);
}

}  // extern "C"
