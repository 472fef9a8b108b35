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

// KV selection scratch: per-workgroup score rows, then (bf16) the packed K
static size_t select_ws_bytes(const vdm_decoder* d, int64_t M) {
  const size_t kp = d->dtype == VDM_BF16 ? (size_t)mpad(M) * d->D * 2 : 0;
  return (select_scratch_bytes((int)M) + 255) / 256 * 256 + kp + 256;
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
};

static size_t dense_ws(const vdm_decoder* d, int64_t M, int64_t N, bool sel, void* base, DenseWs* w) {
  Carve c(base);
  DenseWs x;
  const size_t kv = (size_t)mpad(M) * d->D * esize(d->dtype);
  x.Kp = sel ? nullptr : c.take<char>(kv);
  x.Vt = sel ? nullptr : c.take<char>(kv);
  x.Wp = c.take<char>(packed_w_bytes(d));
  x.kmax = c.take<float>(256);
  x.items = sel ? c.take<Item>((size_t)(N > 0 ? N : 1) * sizeof(Item)) : nullptr;
  x.n_items = sel ? c.take<int32_t>(256) : nullptr;
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
};

static size_t batch_ws(const vdm_decoder* d, int64_t B, int64_t M, void* base, BatchWs* w) {
  Carve c(base);
  BatchWs x;
  x.kv = ((size_t)mpad(M) * d->D * esize(d->dtype) + 255) / 256 * 256;
  x.Kp = c.take<char>(x.kv * B);
  x.Vt = c.take<char>(x.kv * B);
  x.Wp = c.take<char>(packed_w_bytes(d));
  x.kmax = c.take<float>((size_t)B * d->H * 4);
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
  int32_t* occ;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  float* sel_scores;
  int64_t* stats;
  int64_t* part;  // spread partial counters of the mask stages
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
  x.list = c.take<int32_t>((size_t)maxP3 * 4);
  x.items = c.take<Item>((size_t)maxNB3 * ((512 + bq - 1) / bq) * sizeof(Item));
  x.occ = c.take<int32_t>((size_t)maxNB3 * 4);
  if (p->use_kvsel) {
    x.sel_idx = c.take<int32_t>((size_t)maxNB3 * p->cap * 4);
    x.sel_cnt = c.take<int32_t>((size_t)maxNB3 * 4);
    x.sel_scores = c.take<float>(select_scratch_bytes((int)M));
  }
  x.stats = c.take<int64_t>((size_t)VDM_MAX_LEVELS * VDM_STAT_FIELDS * 8);
  x.part = c.take<int64_t>((size_t)stat_part_words() * 8);
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
    if (M > 4096) return fail(VDM_ERR_UNSUPPORTED, "KV selection supports M <= 4096");
    if (p->probes != 0 && p->probes != 1) return fail(VDM_ERR_INVALID_ARG, "probes=%d (0: corners, 1: random)", p->probes);
  }
  (void)d;
  return VDM_OK;
}

}  // namespace vdm

using namespace vdm;

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
  if (M < 1 || M > 4096) {
    fail(VDM_ERR_INVALID_ARG, "M=%lld (1..4096)", (long long)M);
    return 0;
  }
  return select_ws_bytes(dec, M);
}

size_t vdm_hier_workspace_size(const vdm_decoder* dec, const vdm_hier_params* params, int64_t M) {
  if (check_decoder(dec) != VDM_OK || check_hier(dec, params, M) != VDM_OK) return 0;
  return hier_ws(dec, params, M, nullptr, nullptr);
}

// ------------------------------------------------------------------ batched hierarchical decoding
// B shapes through the hierarchical pipeline on up to four streams of the device
// at once: the caller's stream and three side streams forked from it with an event
// and joined back. The per-level bookkeeping launches of one shape are too small to
// fill the chip; those of different shapes run side by side. No host
// synchronisation (the fork and join are stream-ordered events).
namespace {
constexpr int HB_SIDE = 3;  // side streams (four with the caller's: HIP's default number of hardware queues)
constexpr int HB_MAX_DEV = 64;
struct HierFork {
  std::mutex mu;  // one batched call per device at a time records and waits on these events
  bool ready = false;
  hipStream_t side[HB_SIDE];
  hipEvent_t fork, join[HB_SIDE];
};
HierFork g_fork[HB_MAX_DEV];

vdm_status hier_fork_init(HierFork& f) {
  if (f.ready) return VDM_OK;
  for (int i = 0; i < HB_SIDE; ++i) {
    VDM_HIP(hipStreamCreateWithFlags(&f.side[i], hipStreamNonBlocking), "side stream");
    VDM_HIP(hipEventCreateWithFlags(&f.join[i], hipEventDisableTiming), "join event");
  }
  VDM_HIP(hipEventCreateWithFlags(&f.fork, hipEventDisableTiming), "fork event");
  f.ready = true;
  return VDM_OK;
}

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

vdm_status vdm_decode_hier_batch(const vdm_decoder* dec, const vdm_hier_params* p, int32_t B, const void* K,
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
  hipStream_t s = (hipStream_t)stream;
  auto shape = [&](int b, hipStream_t sb) {
    return vdm_decode_hier(dec, p, (const char*)K + b * kv_bytes, (const char*)V + b * kv_bytes, M, vol + b * P3, P3,
                           stats ? stats + (int64_t)b * p->levels * VDM_STAT_FIELDS : nullptr, nullptr,
                           (char*)ws + b * stride, stride, (vdm_stream)sb);
  };
  if (B == 1) return shape(0, s);
  int dev = 0;
  VDM_HIP(hipGetDevice(&dev), "device query");
  if (dev < 0 || dev >= HB_MAX_DEV) return fail(VDM_ERR_UNSUPPORTED, "device %d", dev);
  HierFork& f = g_fork[dev];
  std::lock_guard<std::mutex> lock(f.mu);
  st = hier_fork_init(f);
  if (st != VDM_OK) return st;
  const int nside = B - 1 < HB_SIDE ? B - 1 : HB_SIDE;
  VDM_HIP(hipEventRecord(f.fork, s), "fork record");
  for (int i = 0; i < nside; ++i) VDM_HIP(hipStreamWaitEvent(f.side[i], f.fork, 0), "fork wait");
  vdm_status first = VDM_OK;
  for (int b = 0; b < B && first == VDM_OK; ++b) {
    const int q = b % (nside + 1);
    first = shape(b, q == 0 ? s : f.side[q - 1]);
  }
  // join every side stream, also after an error, so that nothing of this call is
  // left running unordered with the caller's stream
  for (int i = 0; i < nside; ++i) {
    VDM_HIP(hipEventRecord(f.join[i], f.side[i]), "join record");
    VDM_HIP(hipStreamWaitEvent(s, f.join[i], 0), "join wait");
  }
  return first;
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

vdm_status vdm_extract_surface(const float* vol, int32_t R, const uint8_t* cell_mask, float* verts,
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

vdm_status vdm_embed_queries(const vdm_decoder* dec, const float* xyz, int64_t N, void* Q, vdm_stream stream) {
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

vdm_status vdm_project_kv(const vdm_decoder* dec, const void* Z, int64_t M, void* K, void* V, vdm_stream stream) {
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

vdm_status vdm_decode_dense(const vdm_decoder* dec, const vdm_queries* q, const void* K, const void* V, int64_t M,
                            const vdm_kvsel* sel, float* sdf, void* ws, size_t ws_bytes, vdm_stream stream) {
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
  if (q->N == 0) return VDM_OK;
  if (M < 1 || M >= (1ll << 31) / dec->D) return fail(VDM_ERR_INVALID_ARG, "M=%lld", (long long)M);
  if (!K || !V || !sdf) return fail(VDM_ERR_INVALID_ARG, "K, V or sdf is NULL");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(sdf, 4)) return fail(VDM_ERR_INVALID_ARG, "misaligned K, V or sdf");
  if (q->mode == VDM_Q_POINTS && (!q->xyz || !aligned(q->xyz, 4))) return fail(VDM_ERR_INVALID_ARG, "xyz NULL or misaligned");
  if (q->mode == VDM_Q_GRID_LIST && (!q->list || !aligned(q->list, 4)))
    return fail(VDM_ERR_INVALID_ARG, "list NULL or misaligned");
  if (sel) {
    if (q->mode != VDM_Q_GRID_LIST) return fail(VDM_ERR_INVALID_ARG, "token selection needs grid-list queries");
    if (sel->block < 1 || sel->cap < 1 || !sel->sel_idx || !sel->sel_cnt)
      return fail(VDM_ERR_INVALID_ARG, "bad kvsel (block=%d cap=%d)", sel->block, sel->cap);
  }
  const size_t need = dense_ws(dec, M, q->N, sel != nullptr, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace needs %zu bytes, 256-aligned (got %zu)", need, ws_bytes);
  DenseWs w;
  dense_ws(dec, M, q->N, sel != nullptr, ws, &w);
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  DecodeArgs a = base_args(dec);
  a.qs = QuerySrc{q->mode, q->R, q->xyz, q->list, 0};
  a.N = q->N;
  a.out = sdf;
  a.scatter = 0;
  a.kmax = w.kmax;
  VDM_HIP(launch_zero(w.kmax, 256, s), "zero launch");
  VDM_HIP(launch_key_norms(dec->dtype, K, (int)M, dec->H, w.kmax, s), "key norms launch");
  VDM_HIP(pack_weights(dec, w.Wp, a, s), "weight packing launch");
  if (!sel) {
    VDM_HIP(launch_pack_kv(dec->dtype, K, V, (int)M, dec->D, (int)mpad(M), w.Kp, w.Vt, s), "pack_kv launch");
    a.Kp = w.Kp;
    a.Vt = w.Vt;
    a.M = (int)M;
    a.n_tiles = (q->N + decode_tile_queries(dec->dtype, dec->D) - 1) / decode_tile_queries(dec->dtype, dec->D);
    VDM_HIP_T(VDM_TIME_DECODE, s, launch_decode(dec->dtype, dec->D, false, a, s), "decode launch");
  } else {
    const int bq = decode_tile_queries(dec->dtype, dec->D);
    VDM_HIP(launch_zero(w.n_items, 256, s), "zero launch");
    VDM_HIP(launch_items_from_list(q->list, q->N, q->R, sel->block, sel->block_row, bq, w.items, w.n_items, s),
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
    VDM_HIP_T(VDM_TIME_DECODE_GATHERED, s, launch_decode(dec->dtype, dec->D, true, a, s), "gathered decode launch");
  }
  return VDM_OK;
}

size_t vdm_dense_batch_workspace_size(const vdm_decoder* dec, int32_t B, int64_t M) {
  if (check_decoder(dec) != VDM_OK) return 0;
  if (B < 1 || B > 4096 || M < 1 || M >= (1ll << 31) / dec->D) {
    fail(VDM_ERR_INVALID_ARG, "B=%d M=%lld", B, (long long)M);
    return 0;
  }
  return batch_ws(dec, B, M, nullptr, nullptr);
}

vdm_status vdm_decode_dense_batch(const vdm_decoder* dec, const vdm_queries* q, int32_t B, const void* K,
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
  for (int b = 0; b < B; ++b) {
    const char* Kb = (const char*)K + b * shape_bytes;
    const char* Vb = (const char*)V + b * shape_bytes;
    VDM_HIP(launch_key_norms(dec->dtype, Kb, (int)M, dec->H, w.kmax + (size_t)b * dec->H, s), "key norms launch");
    VDM_HIP(launch_pack_kv(dec->dtype, Kb, Vb, (int)M, dec->D, (int)mpad(M), w.Kp + b * w.kv, w.Vt + b * w.kv, s),
            "pack_kv launch");
  }
  a.Kp = w.Kp;
  a.Vt = w.Vt;
  a.M = (int)M;
  a.batch = B;
  a.kv_stride = (int64_t)w.kv;
  a.out_stride = q->N;
  VDM_HIP_T(VDM_TIME_DECODE, s, launch_decode(dec->dtype, dec->D, false, a, s), "batched decode launch");
  return VDM_OK;
}

vdm_status vdm_select_kv(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap, int32_t probes,
                         uint64_t seed, const void* K, int64_t M, const int32_t* blocks, int64_t nblk, int32_t* sel_idx,
                         int32_t* sel_cnt, void* ws, size_t ws_bytes, vdm_stream stream) {
  vdm_status st = check_decoder(dec);
  if (st != VDM_OK) return st;
  if (R < 1 || R > 1200 || block < 1) return fail(VDM_ERR_INVALID_ARG, "R=%d block=%d", R, block);
  if (M < 1 || M > 4096) return fail(M < 1 ? VDM_ERR_INVALID_ARG : VDM_ERR_UNSUPPORTED, "M=%lld (1..4096)", (long long)M);
  if (k < 1 || k > M || cap < k) return fail(VDM_ERR_INVALID_ARG, "k=%d cap=%d M=%lld", k, cap, (long long)M);
  if (probes != 0 && probes != 1) return fail(VDM_ERR_INVALID_ARG, "probes=%d (0: corners, 1: random)", probes);
  const int64_t NB = (R + block) / block;
  if (nblk < 0 || (!blocks && nblk != NB * NB * NB))
    return fail(VDM_ERR_INVALID_ARG, "nblk=%lld (all blocks: %lld)", (long long)nblk, (long long)(NB * NB * NB));
  if (nblk == 0) return VDM_OK;
  if (!K || !sel_idx || !sel_cnt || !aligned(K, 16)) return fail(VDM_ERR_INVALID_ARG, "K, sel_idx or sel_cnt NULL/misaligned");
  const size_t need = select_ws_bytes(dec, M);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(VDM_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  char* kp = static_cast<char*>(ws) + (select_scratch_bytes((int)M) + 255) / 256 * 256;
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
  VDM_HIP_T(VDM_TIME_SELECT, s, launch_select(dec->dtype, a, s), "select launch");
  return VDM_OK;
}

vdm_status vdm_decode_hier(const vdm_decoder* dec, const vdm_hier_params* p, const void* K, const void* V, int64_t M,
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
  hipStream_t s = (hipStream_t)stream;
  int64_t* S = stats ? stats : w.stats;
  const int bq = decode_tile_queries(dec->dtype, dec->D);
  const bool kv = p->use_kvsel != 0;

  VDM_HIP(launch_stats_init(S, p->levels, p->R0, s), "stats init");
  VDM_HIP(launch_zero(w.part, (size_t)stat_part_words() * 8, s), "zero launch");
  VDM_HIP(launch_zero(w.kmax, 256, s), "zero launch");
  VDM_HIP(launch_key_norms(dec->dtype, K, (int)M, dec->H, w.kmax, s), "key norms launch");
  if (!kv)
    VDM_HIP(launch_pack_kv(dec->dtype, K, V, (int)M, dec->D, (int)mpad(M), w.Kp, w.Vt, s), "pack_kv launch");
  else if (dec->dtype == VDM_BF16)  // the selection streams packed K
    VDM_HIP(launch_pack_kv(dec->dtype, K, nullptr, (int)M, dec->D, (int)mpad(M), w.Kp, nullptr, s), "pack K launch");
  DecodeArgs packed = base_args(dec);
  VDM_HIP(pack_weights(dec, w.Wp, packed, s), "weight packing launch");

  auto vol_of = [&](int L) { return L == p->levels - 1 ? vol : w.vol[L]; };
  // list, items and occupied blocks of level L are in w.list / w.items / w.occ
  auto decode_level = [&](int L) -> vdm_status {
    const int R = p->R0 << L;
    int32_t* tot = w.totals + 4 * L;
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
      sa.K = K;
      sa.Kp = w.Kp;
      sa.blocks = w.occ;
      sa.n_blocks = 0;
      sa.d_n_blocks = tot + 2;
      sa.sel_idx = w.sel_idx;
      sa.sel_cnt = w.sel_cnt;
      sa.stat_selected = S + L * VDM_STAT_FIELDS + VDM_STAT_SELECTED;
      sa.scores = w.sel_scores;
      VDM_HIP_T(VDM_TIME_SELECT, s, launch_select(dec->dtype, sa, s), "select launch");
    }
    DecodeArgs a = packed;
    a.qs = QuerySrc{VDM_Q_GRID_LIST, R, nullptr, w.list, 0};
    a.kmax = w.kmax;
    a.out = vol_of(L);
    a.scatter = 1;
    a.M = (int)M;
    if (kv) {
      a.Kp = K;
      a.Vt = V;
      a.items = w.items;
      a.d_n_items = tot + 1;
      a.sel_idx = w.sel_idx;
      a.sel_cnt = w.sel_cnt;
      a.cap = p->cap;
    } else {
      a.Kp = w.Kp;
      a.Vt = w.Vt;
      a.d_N = tot;
    }
    VDM_HIP_T(kv ? VDM_TIME_DECODE_GATHERED : VDM_TIME_DECODE, s, launch_decode(dec->dtype, dec->D, kv, a, s), "decode launch");
    return VDM_OK;
  };

  // level 0: every point, in blocked order
  {
    const int NB = nblocks8(p->R0 + 1);
    const int64_t nb3 = (int64_t)NB * NB * NB;
    VDM_HIP_T(VDM_TIME_MARK, s, launch_mark(nullptr, 1, nullptr, 1, p->R0, w.newmask, nullptr, w.counts, s), "mark launch");
    VDM_HIP_T(VDM_TIME_SCAN, s, launch_scan(w.counts, nb3, bq, w.partial, w.offs, w.occ, w.totals, S, s), "scan launch");
    VDM_HIP_T(VDM_TIME_EMIT, s, launch_emit(w.newmask, w.counts, w.offs, w.occ, w.totals, p->R0, bq, w.list, w.items, s),
              "emit launch");
    st = decode_level(0);
    if (st != VDM_OK) return st;
  }
  for (int L = 0; L < p->levels; ++L) {
    const int R = p->R0 << L, P = R + 1, NB = nblocks8(P);
    int64_t* SL = S + L * VDM_STAT_FIELDS;
    VDM_HIP_T(VDM_TIME_CELL_TEST, s, launch_cell_test(vol_of(L), R, L ? w.kept[L - 1] : nullptr, p->tau, w.active[L], w.part, SL + VDM_STAT_TESTED,
                             SL + VDM_STAT_ACTIVE, s),
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
      if (kv && dbg->sel_cnt[L])
        VDM_HIP(hipMemcpyAsync(dbg->sel_cnt[L], w.sel_cnt, nb3 * 4, hipMemcpyDeviceToDevice, s), "debug copy");
      if (kv && dbg->sel_idx[L])
        VDM_HIP(hipMemcpyAsync(dbg->sel_idx[L], w.sel_idx, nb3 * p->cap * 4, hipMemcpyDeviceToDevice, s), "debug copy");
    }
    if (L == p->levels - 1) break;
    // kept = active dilated `dilation` times (ping-pong through tmp)
    if (p->dilation == 0) {
      VDM_HIP_T(VDM_TIME_DILATE, s, launch_dilate(w.active[L], w.kept[L], R, 1, w.part, SL + VDM_STAT_KEPT, s), "copy launch");
    } else {
      const uint64_t* src = w.active[L];
      for (int t = 0; t < p->dilation; ++t) {
        uint64_t* dst = ((p->dilation - 1 - t) % 2 == 0) ? w.kept[L] : w.tmp;
        VDM_HIP_T(VDM_TIME_DILATE, s, launch_dilate(src, dst, R, 0, w.part, t == p->dilation - 1 ? SL + VDM_STAT_KEPT : nullptr, s), "dilate launch");
        src = dst;
      }
    }
    if (dbg && dbg->kept[L]) VDM_HIP(launch_bits_to_bytes(w.kept[L], R, NB, dbg->kept[L], s), "debug export");
    const int Rn = 2 * R, Pn = Rn + 1, NBn = nblocks8(Pn);
    VDM_HIP_T(VDM_TIME_MARK, s, launch_mark(w.kept[L], R, L ? w.comp[L] : nullptr, 0, Rn, w.newmask, w.comp[L + 1], w.counts, s),
            "mark launch");
    VDM_HIP_T(VDM_TIME_SCAN, s, launch_scan(w.counts, (int64_t)NBn * NBn * NBn, bq, w.partial, w.offs, w.occ, w.totals + 4 * (L + 1),
                        S + (L + 1) * VDM_STAT_FIELDS, s),
            "scan launch");
    VDM_HIP_T(VDM_TIME_EMIT, s,
              launch_emit(w.newmask, w.counts, w.offs, w.occ, w.totals + 4 * (L + 1), Rn, bq, w.list, w.items, s),
              "emit launch");
    VDM_HIP_T(VDM_TIME_FILL, s, launch_fill(vol_of(L), P, vol_of(L + 1), Pn, s), "fill launch");
    st = decode_level(L + 1);
    if (st != VDM_OK) return st;
  }
  return VDM_OK;
}

}  // extern "C"
