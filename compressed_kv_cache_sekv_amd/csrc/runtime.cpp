// Host runtime of the SeKV C ABI (include/sekv.h): contexts, index build /
// import / export, routing and decode orchestration, and the pinned-tier
// gather into the HBM staging ring (sizing on the device, placement and
// capacity check on the host, the copy itself by a kernel reading the mapped
// pinned pool).
//
// SeKV article (aitrends.kr/articles/75020): section 방법론 (Method) and its
// Fig. 2 describe the two tiers (summaries and anchors on the GPU, truncated
// SVD factors on the CPU) and the asynchronous CPU->GPU transfer of the routed
// spans' factors; section 한계점 (Limitations) names the CPU-GPU bandwidth
// dependency, which is why the gather is timed and counted on its own.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <unordered_set>
#include <vector>

#include "sekv.h"
#include "common.h"

using namespace sekv;

namespace {

thread_local std::string g_err;

sekv_status fail(sekv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// On a failing HIP call: reset the runtime's last-error state (so that the
// caller's next HIP call does not report this failure again), then return.
#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) {                                                              \
      (void)hipGetLastError();                                                           \
      return fail(e_ == hipErrorOutOfMemory ? SEKV_ENOMEM : SEKV_EHIP, "%s: %s (%s:%d)", \
                  #expr, hipGetErrorString(e_), __FILE__, __LINE__);                     \
    }                                                                                    \
  } while (0)

constexpr uint32_t CTX_MAGIC = 0x53454b43u;   // "SEKC"
constexpr uint32_t IDX_MAGIC = 0x53454b49u;   // "SEKI"
constexpr uint32_t DEAD_MAGIC = 0xdeadbeefu;

// Handles handed out and not yet destroyed or freed.  A call checks its
// handles here before reading them, so a destroyed context or a freed index
// is refused (SEKV_ESTATE) without touching freed memory.
std::mutex g_live_mu;
std::unordered_set<const void*> g_live;
bool is_live(const void* p) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return p && g_live.count(p) != 0;
}
void set_live(const void* p, bool on) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  if (on) g_live.insert(p);
  else g_live.erase(p);
}

// Work decomposition of the decode kernel: at most kStepsPerItem resident
// 32-row steps (two per wave) and kSpansPerItem compressed spans of the
// sequence per workgroup (where the items run in many waves of workgroups,
// larger items amortise each one's start-up chain; 32 and 64 measured slower
// on the batch of 32 sequences); the larger count sets the items of a KV
// head, raised until the items fill the attention kernel's resident
// workgroup slots, keeping at least kMinFillSpans spans of the sequence per
// item.
constexpr int kStepsPerItem = 8;
constexpr int kSpansPerItem = 48;
static_assert(kSpansPerItem <= kMaxSpanList, "items hold at most one span per lane");
constexpr int kMinFillSpans = 16;

// Device buffer owned by the library.
struct DBuf {
  void* p = nullptr;
  size_t n = 0;
  void release() {
    if (p) (void)hipFree(p);
    p = nullptr;
    n = 0;
  }
};

hipError_t dalloc(DBuf& b, size_t bytes) {
  b.release();
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc(&b.p, bytes);
  if (e == hipSuccess) b.n = bytes;
  else b.p = nullptr;
  return e;
}

hipError_t dgrow(DBuf& b, size_t bytes) {
  if (b.p && b.n >= bytes) return hipSuccess;
  return dalloc(b, bytes);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

// Scratch of sekv_decode_attend_noalloc: the softmax partials of the attention
// items live in this file-scope device array (one copy per GPU, held until the
// process ends) instead of index-owned memory.  Host code never uses the
// array's name as an address: sekv_create takes the device address of each
// GPU's copy once, with that GPU current, and keeps it in g_scratch.
constexpr size_t kScratchBytes = size_t(40) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[kMaxScratchDevices];

// Event pairs bracketing kernel launches (instrumentation).
struct Timer {
  std::vector<hipEvent_t> ev;   // 2 per launch, reused across periods
  size_t used = 0;
  hipError_t begin(hipStream_t st, size_t* slot) {
    if (used + 2 > ev.size()) {
      for (int i = 0; i < 2; ++i) {
        hipEvent_t e;
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) return r;
        ev.push_back(e);
      }
    }
    *slot = used;
    used += 2;
    return hipEventRecord(ev[*slot], st);
  }
  hipError_t end(hipStream_t st, size_t slot) { return hipEventRecord(ev[slot + 1], st); }
  // two events for a launch that records them itself
  hipError_t reserve(size_t* slot) {
    if (used + 2 > ev.size()) {
      for (int i = 0; i < 2; ++i) {
        hipEvent_t e;
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) return r;
        ev.push_back(e);
      }
    }
    *slot = used;
    used += 2;
    return hipSuccess;
  }
  hipError_t drain(double* ms, int64_t* n) {
    double t = 0.0;
    for (size_t i = 0; i < used; i += 2) {
      hipError_t r = hipEventSynchronize(ev[i + 1]);
      if (r != hipSuccess) return r;
      float x = 0.f;
      r = hipEventElapsedTime(&x, ev[i], ev[i + 1]);
      if (r != hipSuccess) return r;
      t += x;
    }
    if (ms) *ms = t;
    if (n) *n = (int64_t)(used / 2);
    used = 0;
    return hipSuccess;
  }
  void release() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    used = 0;
  }
};

struct sekv_ctx {
  uint32_t magic = CTX_MAGIC;
  int device = 0;
  hipStream_t stream = nullptr;
  bool timing = false;
  Timer t_route, t_attend;
};

struct sekv_index {
  uint32_t magic = IDX_MAGIC;
  sekv_ctx* ctx = nullptr;
  int B = 0, L = 0, Hq = 0, Hkv = 0, D = 0, R = 0, dp = 0, G = 0, tier = 0;
  int max_spans = 0, Wd = 0, max_raw = 0;
  int64_t total_spans = 0, total_raw = 0, total_tok = 0;
  int64_t pool_bytes = 0, max_layer_bytes = 0;
  int64_t kres_elems = 0, s_elems = 0;
  std::vector<BMeta> meta;
  std::vector<int32_t> h_span_len;      // concatenated span lengths
  std::vector<float> h_logn;            // ln n_S (host copy of what d_logn holds)
  // factor blobs: layer l's region at layer_off[l]; within it (b, g, span)
  // order, sequence b's blobs from region_off[l][b] (b = B: the layer's end)
  std::vector<int64_t> layer_off;       // [L + 1]
  std::vector<int64_t> region_off;      // [L][B + 1]
  std::vector<uint2> h_bref;            // [L][Hkv][total_spans] blob references
  // device
  DBuf d_meta, d_span_start, d_span_len, d_logn, d_bref, d_layer_off, d_raw_pos;
  DBuf d_kres, d_vres, d_s, d_W;
  DBuf d_pool;                 // HBM tier
  uint8_t* h_pool = nullptr;   // pinned tier (host address)
  const uint8_t* d_host_pool = nullptr;   // the same pool's device address
  DBuf d_ring;                 // pinned tier: the call's layers, blobs at their pool offsets
  DBuf d_gstat;                // pinned tier: per (l, b, g) union spans and bytes (sekv_stats)
  int64_t ring_bytes = 0;
  std::vector<int2> h_gstat;
  // decode work
  std::vector<WorkItem> items;
  std::vector<int32_t> bg_first;
  DBuf d_items, d_bg_first, d_part;
  // routing scratch: scores ranked by the budget kernels; alpha for calibration
  DBuf d_score, d_packed, d_alpha, d_tau_inf;
  // pinned tier: the copy stream the gathers of multi-layer calls run on, the
  // events that order them against the attention, and gather timing events
  hipStream_t copy = nullptr;
  hipEvent_t ev_call = nullptr, ev_ready[2] = {nullptr, nullptr}, ev_free[2] = {nullptr, nullptr};
  std::vector<hipEvent_t> gev;
};

namespace {

// The kernels read q, K, V and W with 16-byte vector loads and the masks as
// 64-bit words.
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

sekv_status check_ctx(const sekv_ctx* c) {
  if (!c) return fail(SEKV_EINVAL, "null context");
  if (!is_live(c) || c->magic != CTX_MAGIC) return fail(SEKV_ESTATE, "context is not live");
  return SEKV_OK;
}

sekv_status check_idx(const sekv_ctx* c, const sekv_index* x) {
  sekv_status st = check_ctx(c);
  if (st) return st;
  if (!x) return fail(SEKV_EINVAL, "null index");
  if (!is_live(x) || x->magic != IDX_MAGIC) return fail(SEKV_ESTATE, "index is not live");
  if (x->ctx != c) return fail(SEKV_ESTATE, "index belongs to another context");
  return SEKV_OK;
}

sekv_status check_shape(const sekv_build_params* p, bool need_build_fields) {
  if (!p) return fail(SEKV_EINVAL, "null params");
  if (p->B < 1 || p->L < 1 || p->Hq < 1 || p->Hkv < 1 || p->T < 1)
    return fail(SEKV_EINVAL, "B, L, Hq, Hkv, T must be >= 1");
  if (p->Hq % p->Hkv) return fail(SEKV_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->dprime < 1 || p->dprime > 64) return fail(SEKV_EUNSUPPORTED, "dprime must be in [1, 64]");
  if (p->R < 1 || p->R > p->d) return fail(SEKV_EINVAL, "R must be in [1, d]");
  if (!attend_supported(p->d, p->Hq / p->Hkv, p->R))
    return fail(SEKV_EUNSUPPORTED, "unsupported shape d=%d G=%d R=%d (d in {64,128}, G in {1,2,4,8}, R in {16,32,64})",
                p->d, p->Hq / p->Hkv, p->R);
  if (p->tier != SEKV_TIER_HBM && p->tier != SEKV_TIER_PINNED_HOST) return fail(SEKV_EINVAL, "bad tier");
  if (p->ring_bytes < 0) return fail(SEKV_EINVAL, "ring_bytes < 0");
  if (need_build_fields) {
    if (p->l_min < 1) return fail(SEKV_EINVAL, "l_min must be >= 1");
    if (!(p->alpha_sp == p->alpha_sp) || std::isinf(p->alpha_sp)) return fail(SEKV_EINVAL, "alpha_sp must be finite");
    if (std::isnan(p->gate_eps)) return fail(SEKV_EINVAL, "gate_eps is NaN");
    if (p->oversample < 0 || p->oversample > 16) return fail(SEKV_EINVAL, "oversample must be in [0, 16]");
    if (p->power_iters < 0 || p->power_iters > 8) return fail(SEKV_EINVAL, "power_iters must be in [0, 8]");
  }
  const int64_t smax = ((int64_t)p->T + 1) / (p->l_min > 0 ? (int64_t)p->l_min + 1 : 2);
  if ((smax + 63) / 64 > kMaxWords) return fail(SEKV_EUNSUPPORTED, "T too large for l_min (more than 65536 spans possible)");
  return SEKV_OK;
}

// Fill shape fields and the per-sequence layout from span counts/lengths.
// n_spans, n_raw: per b; lens: concatenated span lengths.
sekv_status plan_layout(sekv_index* x, const sekv_build_params* p, const std::vector<int32_t>& n_spans,
                 const std::vector<int32_t>& n_raw, const std::vector<int32_t>& lens) {
  for (int b = 0; b < p->B; ++b)
    if (n_spans[b] > 64 * kMaxWords)
      return fail(SEKV_EUNSUPPORTED, "%d spans in sequence %d: the routing masks hold at most %d per sequence",
                  n_spans[b], b, 64 * kMaxWords);
  x->B = p->B; x->L = p->L; x->Hq = p->Hq; x->Hkv = p->Hkv; x->D = p->d; x->R = p->R;
  x->dp = p->dprime; x->G = p->Hq / p->Hkv; x->tier = p->tier;
  x->meta.assign(x->B, BMeta{});
  x->h_span_len = lens;
  int64_t sb = 0, rb = 0, tb = 0, res = 0, sel = 0;
  x->max_spans = 0; x->max_raw = 0;
  for (int b = 0; b < x->B; ++b) {
    BMeta& m = x->meta[b];
    m.n_spans = n_spans[b];
    m.n_raw = n_raw[b];
    m.n_res = m.n_spans + m.n_raw;
    m.n_res_pad = (int32_t)round_up(std::max(m.n_res, 1), 64);
    m.s_pad = (int32_t)round_up(std::max(m.n_spans, 1), 64);
    m.span_base = sb;
    m.raw_base = rb;
    m.tok_base = tb;
    m.res_base = res;
    m.s_base = sel;
    for (int S = 0; S < m.n_spans; ++S) tb += lens[sb + S];
    sb += m.n_spans;
    rb += m.n_raw;
    res += (int64_t)x->L * x->Hkv * m.n_res_pad * x->D;
    sel += (int64_t)x->L * x->Hq * dp_pad4(x->dp) * m.s_pad;
    x->max_spans = std::max(x->max_spans, m.n_spans);
    x->max_raw = std::max(x->max_raw, m.n_raw);
  }
  x->total_spans = sb;
  x->total_raw = rb;
  x->total_tok = tb;
  x->kres_elems = res;
  x->s_elems = sel;
  x->Wd = std::max(1, (x->max_spans + 63) / 64);
  // decode work items: nj per (b, g), each with an equal slice of the
  // resident steps and an equal share of the routed union; nj covers the
  // larger of the two (at most kSpansPerItem union spans and kStepsPerItem
  // steps an item)
  const int spi = kSpansPerItem, spw = kStepsPerItem;
  // workgroups of the attention kernel resident at once on this device: the
  // items of one launch (one layer) share them out per (b, g).  One wave of
  // workgroups that fills them measured fastest (items of fewer routed spans
  // shorten each wave's chain of blob round trips; a second wave of
  // workgroups costs more than it saves).
  int fill = 0;
  if (attend_supported(x->D, x->G, x->R)) {
    int slots = 0;
    HIP_TRY(attend_slots(x->D, x->G, x->R, x->Wd, x->ctx->device, &slots));
    fill = slots / std::max(1, x->B * x->Hkv);
  }
  x->items.clear();
  x->bg_first.assign((size_t)2 * x->B * x->Hkv, 0);
  int slot = 0;
  for (int b = 0; b < x->B; ++b) {
    const BMeta& m = x->meta[b];
    const int nsteps = m.n_res_pad / 32;
    const int nfac = m.n_spans ? (m.n_spans + spi - 1) / spi : 0;
    const int nres = (nsteps + spw - 1) / spw;
    const int nfill = std::min(fill, (m.n_spans + kMinFillSpans - 1) / kMinFillSpans);
    const int nj = std::max(std::max(std::max(nfac, nres), nfill), 1);
    if ((m.n_spans + nj - 1) / nj > kMaxSpanList || (int64_t)nj * m.n_spans >= (1LL << 31))
      return fail(SEKV_EUNSUPPORTED, "%d spans in sequence %d exceed the decode work plan", m.n_spans, b);
    for (int g = 0; g < x->Hkv; ++g) {
      x->bg_first[2 * ((size_t)b * x->Hkv + g)] = slot;
      x->bg_first[2 * ((size_t)b * x->Hkv + g) + 1] = nj;
      for (int j = 0; j < nj; ++j)
        x->items.push_back(WorkItem{b, g, j, nj, (int)((int64_t)j * nsteps / nj),
                                    (int)((int64_t)(j + 1) * nsteps / nj), slot++, 0});
    }
  }
  return SEKV_OK;
}

// Place the factor blobs of a planned index from their stored ranks (ranks:
// [L][Hkv][total_spans], rk | rv << 16): per layer, sequences in order, KV
// heads in order, spans in order, each blob on a 256-byte boundary.
sekv_status plan_blobs(sekv_index* x, const std::vector<uint32_t>& ranks) {
  const int64_t tot = x->total_spans;
  x->h_bref.assign((size_t)x->L * x->Hkv * tot, make_uint2(0u, 0u));
  x->layer_off.assign((size_t)x->L + 1, 0);
  x->region_off.assign((size_t)x->L * (x->B + 1), 0);
  x->max_layer_bytes = 0;
  int64_t base = 0;
  for (int l = 0; l < x->L; ++l) {
    x->layer_off[l] = base;
    int64_t off = 0;
    for (int b = 0; b < x->B; ++b) {
      const BMeta& m = x->meta[b];
      x->region_off[(size_t)l * (x->B + 1) + b] = off;
      for (int g = 0; g < x->Hkv; ++g)
        for (int S = 0; S < m.n_spans; ++S) {
          const size_t i = ((size_t)l * x->Hkv + g) * tot + m.span_base + S;
          const uint32_t rr = ranks[i];
          const int rk = (int)(rr & 0xffffu), rv = (int)(rr >> 16);
          if (rk < 16 || rv < 16 || rk > x->R || rv > x->R || (rk & 15) || (rv & 15))
            return fail(SEKV_EHIP, "stored rank (%d, %d) of span %d (b=%d, l=%d, g=%d) outside the R=%d tiles", rk, rv,
                        S, b, l, g, x->R);
          if ((off >> 8) > 0xffffffffLL) return fail(SEKV_EUNSUPPORTED, "one layer's factors exceed 1 TiB");
          x->h_bref[i] = make_uint2((uint32_t)(off >> 8), rr);
          off += Blob::bytes(rk, rv, x->D, x->h_span_len[m.span_base + S]);
        }
    }
    x->region_off[(size_t)l * (x->B + 1) + x->B] = off;
    x->max_layer_bytes = std::max(x->max_layer_bytes, off);
    base += off;
  }
  x->layer_off[x->L] = base;
  x->pool_bytes = base;
  return SEKV_OK;
}

// Allocate and clear the device (and pinned) storage of a planned index.
sekv_status alloc_index(sekv_index* x, int64_t ring_bytes_req) {
  const size_t nsp = (size_t)std::max<int64_t>(x->total_spans, 1);
  HIP_TRY(dalloc(x->d_meta, sizeof(BMeta) * x->B));
  HIP_TRY(dalloc(x->d_span_start, 4 * nsp));
  HIP_TRY(dalloc(x->d_span_len, 4 * nsp));
  HIP_TRY(dalloc(x->d_logn, 4 * nsp));
  HIP_TRY(dalloc(x->d_bref, sizeof(uint2) * std::max<size_t>(x->h_bref.size(), 1)));
  HIP_TRY(dalloc(x->d_layer_off, sizeof(int64_t) * x->layer_off.size()));
  HIP_TRY(dalloc(x->d_raw_pos, 4 * (size_t)std::max<int64_t>(x->total_raw, 1)));
  HIP_TRY(dalloc(x->d_kres, 2 * (size_t)x->kres_elems));
  HIP_TRY(dalloc(x->d_vres, 2 * (size_t)x->kres_elems));
  HIP_TRY(dalloc(x->d_s, 4 * (size_t)x->s_elems));
  HIP_TRY(dalloc(x->d_W, 4 * (size_t)x->L * x->Hq * x->dp * x->D));
  hipStream_t st = x->ctx->stream;
  HIP_TRY(hipMemsetAsync(x->d_kres.p, 0, x->d_kres.n, st));
  HIP_TRY(hipMemsetAsync(x->d_vres.p, 0, x->d_vres.n, st));
  HIP_TRY(hipMemsetAsync(x->d_s.p, 0, x->d_s.n, st));
  if (x->tier == SEKV_TIER_HBM) {
    HIP_TRY(dalloc(x->d_pool, (size_t)std::max<int64_t>(x->pool_bytes, 256)));
    HIP_TRY(hipMemsetAsync(x->d_pool.p, 0, x->d_pool.n, st));
  } else {
    const size_t pb = (size_t)std::max<int64_t>(x->pool_bytes, 256);
    hipError_t e = hipHostMalloc((void**)&x->h_pool, pb, hipHostMallocPortable | hipHostMallocMapped);
    if (e != hipSuccess) {
      x->h_pool = nullptr;
      (void)hipGetLastError();
      return fail(SEKV_ENOMEM, "pinned host pool of %zu bytes: %s", pb, hipGetErrorString(e));
    }
    memset(x->h_pool, 0, pb);
    void* dp = nullptr;
    HIP_TRY(hipHostGetDevicePointer(&dp, x->h_pool, 0));
    x->d_host_pool = (const uint8_t*)dp;
    // two layer slots by default: a multi-layer call gathers one layer ahead
    x->ring_bytes = ring_bytes_req > 0 ? ring_bytes_req : 2 * std::max<int64_t>((x->max_layer_bytes + 255) & ~255LL, 256);
    HIP_TRY(dalloc(x->d_ring, (size_t)x->ring_bytes));
  }
  HIP_TRY(hipMemcpyAsync(x->d_meta.p, x->meta.data(), sizeof(BMeta) * x->B, hipMemcpyHostToDevice, st));
  HIP_TRY(hipMemcpyAsync(x->d_span_len.p, x->h_span_len.data(), 4 * x->h_span_len.size(), hipMemcpyHostToDevice, st));
  // ln n_S of the pseudo rows, computed here for built and imported indexes alike
  x->h_logn.resize(x->h_span_len.size());
  for (size_t i = 0; i < x->h_span_len.size(); ++i) x->h_logn[i] = logf((float)x->h_span_len[i]);
  if (!x->h_logn.empty())
    HIP_TRY(hipMemcpyAsync(x->d_logn.p, x->h_logn.data(), 4 * x->h_logn.size(), hipMemcpyHostToDevice, st));
  if (!x->h_bref.empty())
    HIP_TRY(hipMemcpyAsync(x->d_bref.p, x->h_bref.data(), sizeof(uint2) * x->h_bref.size(), hipMemcpyHostToDevice, st));
  HIP_TRY(hipMemcpyAsync(x->d_layer_off.p, x->layer_off.data(), sizeof(int64_t) * x->layer_off.size(),
                         hipMemcpyHostToDevice, st));
  HIP_TRY(dalloc(x->d_items, sizeof(WorkItem) * std::max<size_t>(x->items.size(), 1)));
  HIP_TRY(dalloc(x->d_bg_first, 4 * x->bg_first.size()));
  HIP_TRY(hipMemcpyAsync(x->d_items.p, x->items.data(), sizeof(WorkItem) * x->items.size(), hipMemcpyHostToDevice, st));
  HIP_TRY(hipMemcpyAsync(x->d_bg_first.p, x->bg_first.data(), 4 * x->bg_first.size(), hipMemcpyHostToDevice, st));
  if (x->tier == SEKV_TIER_PINNED_HOST) {
    HIP_TRY(hipStreamCreateWithFlags(&x->copy, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&x->ev_call, hipEventDisableTiming));
    for (int k = 0; k < 2; ++k) {
      HIP_TRY(hipEventCreateWithFlags(&x->ev_ready[k], hipEventDisableTiming));
      HIP_TRY(hipEventCreateWithFlags(&x->ev_free[k], hipEventDisableTiming));
    }
  }
  return SEKV_OK;
}

void free_index(sekv_index* x) {
  if (!x) return;
  set_live(x, false);
  if (x->ctx && is_live(x->ctx) && x->ctx->magic == CTX_MAGIC) (void)hipStreamSynchronize(x->ctx->stream);
  if (x->copy) (void)hipStreamSynchronize(x->copy);
  DBuf* bufs[] = {&x->d_meta, &x->d_span_start, &x->d_span_len, &x->d_logn, &x->d_bref, &x->d_layer_off,
                  &x->d_raw_pos, &x->d_kres, &x->d_vres, &x->d_s, &x->d_W, &x->d_pool,
                  &x->d_ring, &x->d_gstat, &x->d_items, &x->d_bg_first, &x->d_part,
                  &x->d_score, &x->d_packed, &x->d_alpha, &x->d_tau_inf};
  for (DBuf* b : bufs) b->release();
  if (x->h_pool) (void)hipHostFree(x->h_pool);
  if (x->copy) (void)hipStreamDestroy(x->copy);
  for (hipEvent_t e : {x->ev_call, x->ev_ready[0], x->ev_ready[1], x->ev_free[0], x->ev_free[1]})
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : x->gev) (void)hipEventDestroy(e);
  x->magic = DEAD_MAGIC;
  delete x;
}

struct IndexGuard {
  sekv_index* x;
  ~IndexGuard() { if (x) free_index(x); }
};

sekv_status set_device(sekv_ctx* c) {
  HIP_TRY(hipSetDevice(c->device));
  return SEKV_OK;
}

// Per-span routing scratch of lc layers: the scores (budget kernels) or alpha
// (calibration).
sekv_status ensure_route_scratch(sekv_index* x, int lc, DBuf& buf) {
  const size_t rows = (size_t)x->B * lc * x->Hq;
  HIP_TRY(dgrow(buf, rows * x->Wd * 64 * sizeof(float)));
  return SEKV_OK;
}

// Streamed bytes of an index (resident rows, summary keys, factor pool)
// above which the kernels load them with the non-temporal hint: half of the
// 256 MB Infinity Cache.  A smaller index is re-read from the cache step
// after step (a single 32K layer: 39.9 thousand query-tokens/s with plain
// loads, 36.1 with the hint); a larger one evicts itself anyway, and the
// hint keeps the shared tables cached instead (128K, 32 layers: 763 -> 796;
// 70B-shaped batch at 64K: 12.5 -> 12.7 thousand).
constexpr int64_t kStreamHintBytes = 128ll << 20;
int stream_hint(const sekv_index* x) {
  return 2 * 2 * x->kres_elems + 4 * x->s_elems + x->pool_bytes > kStreamHintBytes ? 1 : 0;
}

sekv_status check_layers(const sekv_index* x, int lb, int lc) {
  if (lb < 0 || lc < 1 || lb + lc > x->L)
    return fail(SEKV_EINVAL, "layer range [%d, %d) outside [0, %d)", lb, lb + lc, x->L);
  return SEKV_OK;
}

}  // namespace

// ============================================================== lifecycle ===

extern "C" sekv_status sekv_create(int32_t device, void* stream, sekv_ctx** out) {
  if (!out) return fail(SEKV_EINVAL, "null out");
  *out = nullptr;
  int n = 0;
  HIP_TRY(hipGetDeviceCount(&n));
  if (device < 0 || device >= n) return fail(SEKV_EINVAL, "device %d not in [0, %d)", device, n);
  HIP_TRY(hipSetDevice(device));
  if (device < kMaxScratchDevices) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[device]) {
      void* ptr = nullptr;
      HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
      g_scratch[device] = ptr;
    }
  }
  sekv_ctx* c = new sekv_ctx();
  c->device = device;
  c->stream = (hipStream_t)stream;
  set_live(c, true);
  *out = c;
  return SEKV_OK;
}

extern "C" void sekv_destroy(sekv_ctx* c) {
  if (!c || !is_live(c) || c->magic != CTX_MAGIC) return;
  set_live(c, false);
  (void)hipSetDevice(c->device);
  (void)hipStreamSynchronize(c->stream);
  c->t_route.release();
  c->t_attend.release();
  c->magic = DEAD_MAGIC;
  delete c;
}

extern "C" sekv_status sekv_timing_enable(sekv_ctx* c, int32_t enable) {
  sekv_status st = check_ctx(c);
  if (st) return st;
  if ((st = set_device(c))) return st;
  double ms;
  int64_t n;
  HIP_TRY(c->t_route.drain(&ms, &n));
  HIP_TRY(c->t_attend.drain(&ms, &n));
  c->timing = enable != 0;
  return SEKV_OK;
}

extern "C" sekv_status sekv_timing_read(sekv_ctx* c, double* route_ms, int64_t* route_n, double* attend_ms,
                                        int64_t* attend_n) {
  sekv_status st = check_ctx(c);
  if (st) return st;
  if ((st = set_device(c))) return st;
  HIP_TRY(c->t_route.drain(route_ms, route_n));
  HIP_TRY(c->t_attend.drain(attend_ms, attend_n));
  return SEKV_OK;
}

extern "C" const char* sekv_last_error(void) { return g_err.c_str(); }

extern "C" int32_t sekv_max_spans(int32_t T, int32_t l_min) {
  if (T < 1 || l_min < 1) return 0;
  return (int32_t)(((int64_t)T + 1) / ((int64_t)l_min + 1));
}

extern "C" sekv_status sekv_validate_params(const sekv_build_params* p) { return check_shape(p, true); }

extern "C" sekv_status sekv_rsvd_batched(sekv_ctx* c, int32_t count, const void* A, const int64_t* row_off,
                                         const int32_t* rows, int32_t max_rows, int32_t d, int32_t R,
                                         int32_t oversample, int32_t power_iters, uint64_t seed,
                                         float* U, float* sigma, float* Vt) {
  sekv_status st = check_ctx(c);
  if (st) return st;
  if (count < 0) return fail(SEKV_EINVAL, "count < 0");
  if (count == 0) return SEKV_OK;
  if (!A || !row_off || !rows || !U || !sigma || !Vt) return fail(SEKV_EINVAL, "null pointer argument");
  if (d != 64 && d != 128) return fail(SEKV_EUNSUPPORTED, "d must be 64 or 128");
  if (R < 1 || R > 64 || R > d) return fail(SEKV_EINVAL, "R must be in [1, min(64, d)]");
  if (oversample < 0 || oversample > 16) return fail(SEKV_EINVAL, "oversample must be in [0, 16]");
  if (power_iters < 0 || power_iters > 8) return fail(SEKV_EINVAL, "power_iters must be in [0, 8]");
  if (max_rows < 1) return fail(SEKV_EINVAL, "max_rows must be >= 1");
  if ((st = set_device(c))) return st;
  PackArgs pa{};
  pa.A = (const bf16_t*)A;
  pa.mat_row_off = row_off;
  pa.mat_rows = rows;
  pa.out_U = U;
  pa.out_S = sigma;
  pa.out_Vt = Vt;
  pa.count = count;
  pa.max_rows = max_rows;
  pa.D = d;
  pa.R = R;
  pa.oversample = oversample;
  pa.power_iters = power_iters;
  pa.seed = seed;
  HIP_TRY(launch_rsvd_batched(pa, c->stream));
  return SEKV_OK;
}

extern "C" sekv_status sekv_index_get_info(const sekv_index* x, sekv_index_info* info) {
  if (!x || !info) return fail(SEKV_EINVAL, "null argument");
  if (!is_live(x) || x->magic != IDX_MAGIC) return fail(SEKV_ESTATE, "index is not live");
  info->B = x->B; info->L = x->L; info->Hq = x->Hq; info->Hkv = x->Hkv; info->d = x->D;
  info->R = x->R; info->dprime = x->dp; info->tier = x->tier;
  info->max_spans = x->max_spans;
  info->mask_words = x->Wd;
  info->total_spans = x->total_spans;
  info->total_raw = x->total_raw;
  info->total_span_tokens = x->total_tok;
  info->resident_bytes = 2 * 2 * x->kres_elems + 4 * x->s_elems + 4LL * x->L * x->Hq * x->dp * x->D;
  info->factor_bytes = x->pool_bytes;
  info->ring_bytes = x->ring_bytes;
  return SEKV_OK;
}

extern "C" sekv_status sekv_index_counts(const sekv_index* x, int32_t* n_spans, int32_t* n_raw) {
  if (!x || !n_spans || !n_raw) return fail(SEKV_EINVAL, "null argument");
  if (!is_live(x) || x->magic != IDX_MAGIC) return fail(SEKV_ESTATE, "index is not live");
  for (int b = 0; b < x->B; ++b) {
    n_spans[b] = x->meta[b].n_spans;
    n_raw[b] = x->meta[b].n_raw;
  }
  return SEKV_OK;
}

extern "C" void sekv_index_free(sekv_index* x) {
  if (!x || !is_live(x) || x->magic != IDX_MAGIC) return;
  if (x->ctx && is_live(x->ctx) && x->ctx->magic == CTX_MAGIC) (void)hipSetDevice(x->ctx->device);
  free_index(x);
}

// ================================================================ prefill ===

extern "C" sekv_status sekv_build_index(sekv_ctx* c, const sekv_build_params* p, const void* K,
                                        const void* V, const float* H, const float* W,
                                        const float* gates, sekv_index** out) {
  sekv_status st = check_ctx(c);
  if (st) return st;
  if (!out) return fail(SEKV_EINVAL, "null out");
  *out = nullptr;
  if ((st = check_shape(p, true))) return st;
  if (!K || !V || !H || !W) return fail(SEKV_EINVAL, "null K, V, H or W");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(W, 16))
    return fail(SEKV_EINVAL, "K, V and W must be 16-byte aligned");
  if ((st = set_device(c))) return st;
  hipStream_t stream = c->stream;
  const int B = p->B, T = p->T;
  const int S_max = sekv_max_spans(T, p->l_min);

  // ---- span split into scratch
  DBuf sst, sln, raw, cnt, scr;
  struct Rel { DBuf* b[5]; ~Rel() { for (DBuf* x : b) x->release(); } } rel{{&sst, &sln, &raw, &cnt, &scr}};
  HIP_TRY(dalloc(sst, 4 * (size_t)B * std::max(S_max, 1)));
  HIP_TRY(dalloc(sln, 4 * (size_t)B * std::max(S_max, 1)));
  HIP_TRY(dalloc(raw, 4 * (size_t)B * T));
  HIP_TRY(dalloc(cnt, 8 * (size_t)B));
  HIP_TRY(dalloc(scr, 4 * (size_t)B * 2 * (T / 2 + 2)));
  SplitArgs sa{};
  sa.H = H;
  sa.span_start = (int32_t*)sst.p;
  sa.span_len = (int32_t*)sln.p;
  sa.raw_pos = (int32_t*)raw.p;
  sa.counts = (int32_t*)cnt.p;
  sa.scratch = (int32_t*)scr.p;
  sa.B = B; sa.T = T; sa.S_max = S_max; sa.l_min = p->l_min; sa.alpha_sp = p->alpha_sp;
  HIP_TRY(launch_span_split(sa, stream));
  std::vector<int32_t> counts(2 * B);
  HIP_TRY(hipMemcpyAsync(counts.data(), cnt.p, 8 * (size_t)B, hipMemcpyDeviceToHost, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  std::vector<int32_t> n_spans(B), n_raw(B);
  int64_t tot_sp = 0;
  for (int b = 0; b < B; ++b) {
    n_spans[b] = counts[2 * b];
    n_raw[b] = counts[2 * b + 1];
    if (n_spans[b] < 0 || n_spans[b] > S_max || n_raw[b] < 0 || n_raw[b] > T)
      return fail(SEKV_EHIP, "span split produced inconsistent counts for b=%d", b);
    tot_sp += n_spans[b];
  }
  std::vector<int32_t> lens((size_t)tot_sp);
  {
    int64_t o = 0;
    for (int b = 0; b < B; ++b) {
      if (n_spans[b])
        HIP_TRY(hipMemcpyAsync(lens.data() + o, (int32_t*)sln.p + (size_t)b * S_max, 4 * (size_t)n_spans[b],
                               hipMemcpyDeviceToHost, stream));
      o += n_spans[b];
    }
    HIP_TRY(hipStreamSynchronize(stream));
  }
  sekv_index* x = new sekv_index();
  x->ctx = c;
  IndexGuard guard{x};
  if ((st = plan_layout(x, p, n_spans, n_raw, lens))) return st;
  // stored ranks of every span factorization (gates below gate_eps drop their
  // components), which place the blobs and size the pool
  {
    DBuf rk;
    struct RelR { DBuf* b; ~RelR() { b->release(); } } relr{&rk};
    const size_t nr = (size_t)B * p->L * p->Hkv * std::max(S_max, 1);
    HIP_TRY(dalloc(rk, 4 * nr));
    RankArgs ra{};
    ra.gates = gates;
    ra.span_len = (const int32_t*)sln.p;
    ra.counts = (const int32_t*)cnt.p;
    ra.ranks = (uint32_t*)rk.p;
    ra.B = B; ra.L = p->L; ra.Hkv = p->Hkv; ra.R = p->R; ra.S_max = S_max; ra.gate_eps = p->gate_eps;
    HIP_TRY(launch_ranks(ra, stream));
    std::vector<uint32_t> hr(nr);
    HIP_TRY(hipMemcpyAsync(hr.data(), rk.p, 4 * nr, hipMemcpyDeviceToHost, stream));
    HIP_TRY(hipStreamSynchronize(stream));
    std::vector<uint32_t> ranks((size_t)p->L * p->Hkv * x->total_spans);
    for (int b = 0; b < B; ++b)
      for (int l = 0; l < p->L; ++l)
        for (int g = 0; g < p->Hkv; ++g)
          for (int S = 0; S < n_spans[b]; ++S)
            ranks[((size_t)l * p->Hkv + g) * x->total_spans + x->meta[b].span_base + S] =
                hr[(((size_t)b * p->L + l) * p->Hkv + g) * S_max + S];
    if ((st = plan_blobs(x, ranks))) return st;
  }
  if ((st = alloc_index(x, p->ring_bytes))) return st;
  // compact span tables and raw positions
  for (int b = 0; b < B; ++b) {
    const BMeta& m = x->meta[b];
    if (m.n_spans) {
      HIP_TRY(hipMemcpyAsync((int32_t*)x->d_span_start.p + m.span_base, (int32_t*)sst.p + (size_t)b * S_max,
                             4 * (size_t)m.n_spans, hipMemcpyDeviceToDevice, stream));
    }
    if (m.n_raw)
      HIP_TRY(hipMemcpyAsync((int32_t*)x->d_raw_pos.p + m.raw_base, (int32_t*)raw.p + (size_t)b * T,
                             4 * (size_t)m.n_raw, hipMemcpyDeviceToDevice, stream));
  }
  HIP_TRY(hipMemcpyAsync(x->d_W.p, W, x->d_W.n, hipMemcpyDeviceToDevice, stream));

  PackArgs pa{};
  pa.K = (const bf16_t*)K;
  pa.V = (const bf16_t*)V;
  pa.H = H;
  pa.W = W;
  pa.gates = gates;
  pa.meta = (const BMeta*)x->d_meta.p;
  pa.span_start = (const int32_t*)x->d_span_start.p;
  pa.span_len = (const int32_t*)x->d_span_len.p;
  pa.raw_pos = (const int32_t*)x->d_raw_pos.p;
  pa.bref = (const uint2*)x->d_bref.p;
  pa.total_spans = x->total_spans;
  pa.gate_eps = p->gate_eps;
  pa.kres = (bf16_t*)x->d_kres.p;
  pa.vres = (bf16_t*)x->d_vres.p;
  pa.s = (float*)x->d_s.p;
  pa.B = B; pa.L = p->L; pa.Hq = p->Hq; pa.Hkv = p->Hkv; pa.D = p->d; pa.T = T; pa.R = p->R;
  pa.dp = p->dprime; pa.S_max = S_max; pa.max_raw = x->max_raw; pa.max_spans = x->max_spans;
  pa.oversample = p->oversample; pa.power_iters = p->power_iters; pa.seed = p->seed;
  HIP_TRY(launch_pack_raw(pa, stream));
  HIP_TRY(launch_summaries(pa, stream));
  if (x->tier == SEKV_TIER_HBM) {
    for (int l = 0; l < p->L; ++l) {
      pa.layer = l;
      pa.pool = (uint8_t*)x->d_pool.p + x->layer_off[l];
      HIP_TRY(launch_rsvd(pa, stream));
    }
    HIP_TRY(hipStreamSynchronize(stream));
  } else {
    // pinned tier: layer l's factors go to HBM stage l % 2 and are copied to
    // the pinned pool on a second stream while layer l + 1 is factored into
    // the other stage (cleared first: the blob layout differs between layers
    // where the stored ranks do)
    struct Overlap {
      DBuf stage[2];
      hipStream_t copy = nullptr;
      hipEvent_t done[2] = {nullptr, nullptr}, copied[2] = {nullptr, nullptr};
      ~Overlap() {
        if (copy) (void)hipStreamSynchronize(copy);
        for (int k = 0; k < 2; ++k) {
          if (done[k]) (void)hipEventDestroy(done[k]);
          if (copied[k]) (void)hipEventDestroy(copied[k]);
          stage[k].release();
        }
        if (copy) (void)hipStreamDestroy(copy);
      }
    } ov;
    const int nst = p->L > 1 ? 2 : 1;
    for (int k = 0; k < nst; ++k) {
      HIP_TRY(dalloc(ov.stage[k], (size_t)std::max<int64_t>(x->max_layer_bytes, 256)));
      HIP_TRY(hipEventCreateWithFlags(&ov.done[k], hipEventDisableTiming));
      HIP_TRY(hipEventCreateWithFlags(&ov.copied[k], hipEventDisableTiming));
    }
    HIP_TRY(hipStreamCreateWithFlags(&ov.copy, hipStreamNonBlocking));
    for (int l = 0; l < p->L; ++l) {
      const int k = l % nst;
      pa.layer = l;
      pa.pool = (uint8_t*)ov.stage[k].p;
      const size_t lbytes = (size_t)(x->layer_off[l + 1] - x->layer_off[l]);
      if (l >= nst) HIP_TRY(hipStreamWaitEvent(stream, ov.copied[k], 0));   // stage k drained
      if (lbytes) HIP_TRY(hipMemsetAsync(ov.stage[k].p, 0, lbytes, stream));
      HIP_TRY(launch_rsvd(pa, stream));
      HIP_TRY(hipEventRecord(ov.done[k], stream));
      HIP_TRY(hipStreamWaitEvent(ov.copy, ov.done[k], 0));
      if (lbytes)
        HIP_TRY(hipMemcpyAsync(x->h_pool + x->layer_off[l], ov.stage[k].p, lbytes, hipMemcpyDeviceToHost, ov.copy));
      HIP_TRY(hipEventRecord(ov.copied[k], ov.copy));
    }
    HIP_TRY(hipStreamSynchronize(ov.copy));
    HIP_TRY(hipStreamSynchronize(stream));
  }
  guard.x = nullptr;
  set_live(x, true);
  *out = x;
  return SEKV_OK;
}

extern "C" sekv_status sekv_index_import(sekv_ctx* c, const sekv_build_params* p, const sekv_host_index* h,
                                         sekv_index** out) {
  sekv_status st = check_ctx(c);
  if (st) return st;
  if (!out) return fail(SEKV_EINVAL, "null out");
  *out = nullptr;
  if ((st = check_shape(p, false))) return st;
  if (!h || !h->n_spans || !h->n_raw || !h->k_res || !h->v_res || !h->s || !h->W)
    return fail(SEKV_EINVAL, "null host index member");
  const int B = p->B, T = p->T, D = p->d, R = p->R, L = p->L, Hkv = p->Hkv, Hq = p->Hq, dp = p->dprime;
  std::vector<int32_t> n_spans(h->n_spans, h->n_spans + B), n_raw(h->n_raw, h->n_raw + B);
  int64_t tot_sp = 0, tot_raw = 0;
  for (int b = 0; b < B; ++b) {
    if (n_spans[b] < 0 || n_raw[b] < 0) return fail(SEKV_EINVAL, "negative count at b=%d", b);
    if (n_spans[b] > 64 * kMaxWords)
      return fail(SEKV_EUNSUPPORTED, "%d spans in sequence %d: the routing masks hold at most %d per sequence",
                  n_spans[b], b, 64 * kMaxWords);
    tot_sp += n_spans[b];
    tot_raw += n_raw[b];
  }
  if (tot_sp && (!h->span_start || !h->span_len || !h->uk || !h->uv || !h->vkt || !h->vvt || !h->smk || !h->smv))
    return fail(SEKV_EINVAL, "null span arrays");
  if (tot_raw && !h->raw_pos) return fail(SEKV_EINVAL, "null raw_pos");
  // the tables must partition [0, T) per sequence
  {
    int64_t so = 0, ro = 0;
    std::vector<uint8_t> seen(T);
    for (int b = 0; b < B; ++b) {
      std::fill(seen.begin(), seen.end(), 0);
      int64_t cov = 0;
      for (int S = 0; S < n_spans[b]; ++S) {
        const int a0 = h->span_start[so + S], n = h->span_len[so + S];
        if (n < 1 || a0 < 0 || (int64_t)a0 + n > T) return fail(SEKV_EINVAL, "span %d of b=%d out of range", S, b);
        for (int t = a0; t < a0 + n; ++t) {
          if (seen[t]) return fail(SEKV_EINVAL, "token %d of b=%d covered twice", t, b);
          seen[t] = 1;
        }
        cov += n;
      }
      for (int i = 0; i < n_raw[b]; ++i) {
        const int t = h->raw_pos[ro + i];
        if (t < 0 || t >= T || seen[t]) return fail(SEKV_EINVAL, "raw token %d of b=%d invalid", t, b);
        seen[t] = 1;
      }
      if (cov + n_raw[b] != T) return fail(SEKV_EINVAL, "spans and raw tokens of b=%d do not cover T", b);
      so += n_spans[b];
      ro += n_raw[b];
    }
  }
  if ((st = set_device(c))) return st;
  std::vector<int32_t> lens(h->span_len, h->span_len + tot_sp);
  sekv_index* x = new sekv_index();
  x->ctx = c;
  IndexGuard guard{x};
  if ((st = plan_layout(x, p, n_spans, n_raw, lens))) return st;
  // stored ranks: components up to the last one with nonzero sigma * m (the
  // rest contribute nothing), in 16-wide tiles
  {
    std::vector<uint32_t> ranks((size_t)L * Hkv * x->total_spans, 0u);
    int64_t spo = 0;
    auto kept = [&](const float* sm) {
      int c = 0;
      for (int i = 0; i < R; ++i)
        if (sm[i] != 0.f) c = i + 1;
      return stored_rank(c);
    };
    for (int b = 0; b < B; ++b) {
      const BMeta& m = x->meta[b];
      for (int l = 0; l < L; ++l)
        for (int g = 0; g < Hkv; ++g)
          for (int S = 0; S < m.n_spans; ++S) {
            const int64_t rsp = spo + ((int64_t)l * Hkv + g) * m.n_spans + S;
            ranks[((size_t)l * Hkv + g) * x->total_spans + m.span_base + S] =
                (uint32_t)kept(h->smk + rsp * R) | ((uint32_t)kept(h->smv + rsp * R) << 16);
          }
      spo += (int64_t)L * Hkv * m.n_spans;
    }
    if ((st = plan_blobs(x, ranks))) return st;
  }
  if ((st = alloc_index(x, p->ring_bytes))) return st;
  hipStream_t stream = c->stream;
  // pack into the native layouts on the host
  std::vector<bf16_t> kres((size_t)x->kres_elems, 0), vres((size_t)x->kres_elems, 0);
  std::vector<float> s((size_t)x->s_elems, 0.f);
  std::vector<uint8_t> pool;
  uint8_t* pool_dst;
  if (x->tier == SEKV_TIER_HBM) {
    pool.assign((size_t)x->pool_bytes, 0);
    pool_dst = pool.data();
  } else {
    pool_dst = x->h_pool;
  }
  int64_t kro = 0, so = 0, tko = 0, spo = 0;
  for (int b = 0; b < B; ++b) {
    const BMeta& m = x->meta[b];
    const int NS = m.n_spans, NR = m.n_res;
    int64_t ntok = 0;
    for (int S = 0; S < NS; ++S) ntok += lens[m.span_base + S];
    for (int lg = 0; lg < L * Hkv; ++lg) {
      const int64_t dst = m.res_base + (int64_t)lg * m.n_res_pad * D;
      for (int r = 0; r < NR; ++r)
        for (int d = 0; d < D; ++d) {
          const int64_t src = kro + ((int64_t)lg * NR + r) * D + d;
          kres[dst + krow_off(r, d, D)] = h->k_res[src];
          vres[dst + vrow_off(r, d, D)] = h->v_res[src];
        }
    }
    kro += (int64_t)L * Hkv * NR * D;
    for (int lh = 0; lh < L * Hq; ++lh)
      for (int j = 0; j < dp; ++j)
        for (int S = 0; S < NS; ++S)
          s[m.s_base + (int64_t)lh * dp_pad4(dp) * m.s_pad + skey_index(S, j, dp_pad4(dp))] =
              h->s[so + ((int64_t)lh * dp + j) * NS + S];
    so += (int64_t)L * Hq * dp * NS;
    for (int l = 0; l < L; ++l)
      for (int g = 0; g < Hkv; ++g) {
        const int lg = l * Hkv + g;
        int64_t toff = 0;
        for (int S = 0; S < NS; ++S) {
          const int n = lens[m.span_base + S], np = Blob::npad(n);
          const uint2 rf = x->h_bref[(size_t)lg * x->total_spans + m.span_base + S];
          const int rk = bref_rk(rf), rv = bref_rv(rf);
          uint8_t* blob = pool_dst + x->layer_off[l] + (int64_t)rf.x * 256;
          bf16_t* vkt = (bf16_t*)(blob + Blob::off_vkt());
          bf16_t* vv = (bf16_t*)(blob + Blob::off_vv(rk, D));
          float* smk = (float*)(blob + Blob::off_smk(rk, rv, D));
          float* smv = (float*)(blob + Blob::off_smv(rk, rv, D));
          bf16_t* uk = (bf16_t*)(blob + Blob::off_uk(rk, rv, D));
          bf16_t* uvt = (bf16_t*)(blob + Blob::off_uvt(rk, rv, D, n));
          const int64_t rsp = spo + (int64_t)lg * NS + S;   // [L][Hkv][NS] index
          for (int i = 0; i < rk; ++i) {
            for (int d = 0; d < D; ++d) vkt[krow_off(i, d, D)] = h->vkt[(rsp * R + i) * D + d];
            smk[i] = h->smk[rsp * R + i];
          }
          for (int i = 0; i < rv; ++i) {
            for (int d = 0; d < D; ++d) vv[a16_off(d, i, rv)] = h->vvt[(rsp * R + i) * D + d];
            smv[i] = h->smv[rsp * R + i];
          }
          const int64_t ub = tko + (int64_t)lg * ntok + toff;  // [L][Hkv][sum n][R] row
          for (int t = 0; t < n; ++t) {
            for (int i = 0; i < rk; ++i) uk[a16_off(t, i, rk)] = h->uk[(ub + t) * R + i];
            for (int i = 0; i < rv; ++i) uvt[a16_off(i, t, np)] = h->uv[(ub + t) * R + i];
          }
          toff += n;
        }
      }
    tko += (int64_t)L * Hkv * ntok;
    spo += (int64_t)L * Hkv * NS;
  }
  HIP_TRY(hipMemcpyAsync(x->d_kres.p, kres.data(), 2 * kres.size(), hipMemcpyHostToDevice, stream));
  HIP_TRY(hipMemcpyAsync(x->d_vres.p, vres.data(), 2 * vres.size(), hipMemcpyHostToDevice, stream));
  HIP_TRY(hipMemcpyAsync(x->d_s.p, s.data(), 4 * s.size(), hipMemcpyHostToDevice, stream));
  if (tot_sp) {
    HIP_TRY(hipMemcpyAsync(x->d_span_start.p, h->span_start, 4 * (size_t)tot_sp, hipMemcpyHostToDevice, stream));
  }
  if (tot_raw) HIP_TRY(hipMemcpyAsync(x->d_raw_pos.p, h->raw_pos, 4 * (size_t)tot_raw, hipMemcpyHostToDevice, stream));
  HIP_TRY(hipMemcpyAsync(x->d_W.p, h->W, x->d_W.n, hipMemcpyHostToDevice, stream));
  if (x->tier == SEKV_TIER_HBM)
    HIP_TRY(hipMemcpyAsync(x->d_pool.p, pool.data(), pool.size(), hipMemcpyHostToDevice, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  guard.x = nullptr;
  set_live(x, true);
  *out = x;
  return SEKV_OK;
}

namespace {

// Export of sequences [bb, bb + bc) and layers [lb, lb + lc): the logical
// layout with bc sequences and lc in place of L.
sekv_status export_part(sekv_ctx* c, const sekv_index* x, int bb, int bc, int lb, int lc,
                        const sekv_host_index_out* h) {
  sekv_status st = check_idx(c, x);
  if (st) return st;
  if (!h) return fail(SEKV_EINVAL, "null host index");
  if ((st = check_layers(x, lb, lc))) return st;
  if (bb < 0 || bc < 1 || bb + bc > x->B)
    return fail(SEKV_EINVAL, "sequence range [%d, %d) outside [0, %d)", bb, bb + bc, x->B);
  if ((st = set_device(c))) return st;
  hipStream_t stream = c->stream;
  const int D = x->D, R = x->R, L = lc, Hkv = x->Hkv, Hq = x->Hq, dp = x->dp;
  const bool want_res = h->k_res || h->v_res;
  const bool want_fac = h->uk || h->uv || h->vkt || h->vvt || h->smk || h->smv;
  const BMeta& m0 = x->meta[bb];
  const BMeta& m1 = x->meta[bb + bc - 1];
  // device ranges of the sequences: resident rows, summary keys, span tables,
  // and each layer's factor region
  const int64_t res0 = m0.res_base, res1 = m1.res_base + (int64_t)x->L * Hkv * m1.n_res_pad * D;
  const int64_t s0 = m0.s_base, s1 = m1.s_base + (int64_t)x->L * Hq * dp_pad4(dp) * m1.s_pad;
  const int64_t sp0 = m0.span_base, sp1 = m1.span_base + m1.n_spans;
  const int64_t rw0 = m0.raw_base, rw1 = m1.raw_base + m1.n_raw;
  std::vector<bf16_t> kres(want_res ? (size_t)(res1 - res0) : 0), vres(want_res ? (size_t)(res1 - res0) : 0);
  std::vector<float> s(h->s ? (size_t)(s1 - s0) : 0);
  std::vector<int32_t> sst((size_t)std::max<int64_t>(sp1 - sp0, 1)), rp((size_t)std::max<int64_t>(rw1 - rw0, 1));
  // the sequences' factor blobs, layer by layer: layer lb + l's region from
  // region_off[lb + l][bb] copied to pool[ppos[l]]
  std::vector<uint8_t> pool;
  std::vector<int64_t> ppos((size_t)lc + 1, 0);
  auto reg = [&](int l, int b) { return x->region_off[(size_t)l * (x->B + 1) + b]; };
  for (int l = 0; l < lc; ++l) ppos[l + 1] = ppos[l] + (reg(lb + l, bb + bc) - reg(lb + l, bb));
  if (want_fac) {
    pool.resize((size_t)std::max<int64_t>(ppos[lc], 1));
    for (int l = 0; l < lc; ++l) {
      const int64_t n = ppos[l + 1] - ppos[l];
      if (n <= 0) continue;
      const size_t src = (size_t)(x->layer_off[lb + l] + reg(lb + l, bb));
      if (x->tier == SEKV_TIER_HBM)
        HIP_TRY(hipMemcpyAsync(pool.data() + ppos[l], (const uint8_t*)x->d_pool.p + src, (size_t)n,
                               hipMemcpyDeviceToHost, stream));
      else
        memcpy(pool.data() + ppos[l], x->h_pool + src, (size_t)n);
    }
  }
  if (want_res) {
    HIP_TRY(hipMemcpyAsync(kres.data(), (const bf16_t*)x->d_kres.p + res0, 2 * kres.size(), hipMemcpyDeviceToHost,
                           stream));
    HIP_TRY(hipMemcpyAsync(vres.data(), (const bf16_t*)x->d_vres.p + res0, 2 * vres.size(), hipMemcpyDeviceToHost,
                           stream));
  }
  if (h->s)
    HIP_TRY(hipMemcpyAsync(s.data(), (const float*)x->d_s.p + s0, 4 * s.size(), hipMemcpyDeviceToHost, stream));
  if (sp1 > sp0)
    HIP_TRY(hipMemcpyAsync(sst.data(), (const int32_t*)x->d_span_start.p + sp0, 4 * (size_t)(sp1 - sp0),
                           hipMemcpyDeviceToHost, stream));
  if (rw1 > rw0)
    HIP_TRY(hipMemcpyAsync(rp.data(), (const int32_t*)x->d_raw_pos.p + rw0, 4 * (size_t)(rw1 - rw0),
                           hipMemcpyDeviceToHost, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  if (h->span_start) std::copy(sst.begin(), sst.begin() + (sp1 - sp0), h->span_start);
  if (h->span_len) std::copy(x->h_span_len.begin() + sp0, x->h_span_len.begin() + sp1, h->span_len);
  if (h->raw_pos) std::copy(rp.begin(), rp.begin() + (rw1 - rw0), h->raw_pos);
  int64_t kro = 0, so = 0, tko = 0, spo = 0;
  for (int b = bb; b < bb + bc; ++b) {
    const BMeta& m = x->meta[b];
    const int NS = m.n_spans, NR = m.n_res;
    int64_t ntok = 0;
    for (int S = 0; S < NS; ++S) ntok += x->h_span_len[m.span_base + S];
    for (int lg = 0; want_res && lg < L * Hkv; ++lg) {
      const int64_t src = m.res_base - res0 + ((int64_t)lb * Hkv + lg) * m.n_res_pad * D;
      for (int r = 0; r < NR; ++r)
        for (int d = 0; d < D; ++d) {
          const int64_t dst = kro + ((int64_t)lg * NR + r) * D + d;
          if (h->k_res) h->k_res[dst] = kres[src + krow_off(r, d, D)];
          if (h->v_res) h->v_res[dst] = vres[src + vrow_off(r, d, D)];
        }
    }
    kro += (int64_t)L * Hkv * NR * D;
    if (h->s)
      for (int lh = 0; lh < L * Hq; ++lh)
        for (int j = 0; j < dp; ++j)
          for (int S = 0; S < NS; ++S)
            h->s[so + ((int64_t)lh * dp + j) * NS + S] =
                s[m.s_base - s0 + ((int64_t)lb * Hq + lh) * dp_pad4(dp) * m.s_pad + skey_index(S, j, dp_pad4(dp))];
    so += (int64_t)L * Hq * dp * NS;
    for (int l = 0; (want_fac || h->rank) && l < L; ++l)
      for (int g = 0; g < Hkv; ++g) {
        const int lg = l * Hkv + g;
        int64_t toff = 0;
        for (int S = 0; S < NS; ++S) {
          const int n = x->h_span_len[m.span_base + S], np = Blob::npad(n);
          const uint2 rf = x->h_bref[((size_t)(lb + l) * Hkv + g) * x->total_spans + m.span_base + S];
          const int rk = bref_rk(rf), rv = bref_rv(rf);
          const int64_t rsp = spo + (int64_t)lg * NS + S;
          if (h->rank) {
            h->rank[2 * rsp] = rk;
            h->rank[2 * rsp + 1] = rv;
          }
          if (!want_fac) continue;
          // components past the stored ones are zero
          const uint8_t* blob = pool.data() + ppos[l] + ((int64_t)rf.x * 256 - reg(lb + l, bb));
          const bf16_t* vkt = (const bf16_t*)(blob + Blob::off_vkt());
          const bf16_t* vv = (const bf16_t*)(blob + Blob::off_vv(rk, D));
          const float* smk = (const float*)(blob + Blob::off_smk(rk, rv, D));
          const float* smv = (const float*)(blob + Blob::off_smv(rk, rv, D));
          const bf16_t* uk = (const bf16_t*)(blob + Blob::off_uk(rk, rv, D));
          const bf16_t* uvt = (const bf16_t*)(blob + Blob::off_uvt(rk, rv, D, n));
          for (int i = 0; i < R; ++i)
            for (int d = 0; d < D; ++d) {
              if (h->vkt) h->vkt[(rsp * R + i) * D + d] = i < rk ? vkt[krow_off(i, d, D)] : 0;
              if (h->vvt) h->vvt[(rsp * R + i) * D + d] = i < rv ? vv[a16_off(d, i, rv)] : 0;
            }
          for (int i = 0; i < R; ++i) {
            if (h->smk) h->smk[rsp * R + i] = i < rk ? smk[i] : 0.f;
            if (h->smv) h->smv[rsp * R + i] = i < rv ? smv[i] : 0.f;
          }
          const int64_t ub = tko + (int64_t)lg * ntok + toff;
          for (int t = 0; t < n; ++t)
            for (int i = 0; i < R; ++i) {
              if (h->uk) h->uk[(ub + t) * R + i] = i < rk ? uk[a16_off(t, i, rk)] : 0;
              if (h->uv) h->uv[(ub + t) * R + i] = i < rv ? uvt[a16_off(i, t, np)] : 0;
            }
          toff += n;
        }
      }
    tko += (int64_t)L * Hkv * ntok;
    spo += (int64_t)L * Hkv * NS;
  }
  return SEKV_OK;
}

}  // namespace

extern "C" sekv_status sekv_index_export(sekv_ctx* c, const sekv_index* x, const sekv_host_index_out* h) {
  sekv_status st = check_idx(c, x);
  if (st) return st;
  return export_part(c, x, 0, x->B, 0, x->L, h);
}

extern "C" sekv_status sekv_index_export_part(sekv_ctx* c, const sekv_index* x, int32_t seq_begin,
                                              int32_t seq_count, int32_t layer_begin, int32_t layer_count,
                                              const sekv_host_index_out* h) {
  return export_part(c, x, seq_begin, seq_count, layer_begin, layer_count, h);
}

// ================================================================= decode ===

extern "C" sekv_status sekv_route(sekv_ctx* c, const sekv_index* xc, int32_t lb, int32_t lc, const void* q,
                                  const float* tau, int32_t cap, uint64_t* mask, float* alpha) {
  sekv_index* x = const_cast<sekv_index*>(xc);
  sekv_status st = check_idx(c, x);
  if (st) return st;
  if ((st = check_layers(x, lb, lc))) return st;
  if (!q || !tau || !mask) return fail(SEKV_EINVAL, "null q, tau or mask");
  if (!aligned(q, 16) || !aligned(mask, 8)) return fail(SEKV_EINVAL, "q must be 16-byte and mask 8-byte aligned");
  if (cap < 0) return fail(SEKV_EINVAL, "cap < 0");
  if (alpha && ((uintptr_t)alpha & 15)) return fail(SEKV_EINVAL, "alpha must be 16-byte aligned");
  if ((st = set_device(c))) return st;
  if (cap > 0 && ((st = ensure_route_scratch(x, lc, x->d_score)) || (st = ensure_route_scratch(x, lc, x->d_packed))))
    return st;
  RouteArgs ra{};
  ra.q = (const bf16_t*)q;
  ra.tau = tau;
  ra.W = (const float*)x->d_W.p;
  ra.s = (const float*)x->d_s.p;
  ra.meta = (const BMeta*)x->d_meta.p;
  ra.mask = mask;
  ra.alpha = alpha;
  ra.score = cap > 0 ? (float*)x->d_score.p : nullptr;
  ra.packed = cap > 0 ? (uint32_t*)x->d_packed.p : nullptr;
  ra.layer_begin = lb; ra.layer_count = lc;
  ra.B = x->B; ra.L = x->L; ra.Hq = x->Hq; ra.Hkv = x->Hkv; ra.D = x->D; ra.dp = x->dp; ra.Wd = x->Wd;
  ra.cap = cap;
  ra.stream = stream_hint(x);
  size_t slot = 0;
  if (c->timing) HIP_TRY(c->t_route.begin(c->stream, &slot));
  HIP_TRY(launch_route(ra, c->stream));
  if (cap > 0) HIP_TRY(launch_route_cap(ra, c->stream));
  if (c->timing) HIP_TRY(c->t_route.end(c->stream, slot));
  return SEKV_OK;
}

extern "C" sekv_status sekv_route_pooled(sekv_ctx* c, const sekv_index* xc, int32_t lb, int32_t lc, const void* q,
                                         const float* tau, int32_t budget, uint64_t* mask, float* alpha) {
  sekv_index* x = const_cast<sekv_index*>(xc);
  sekv_status st = check_idx(c, x);
  if (st) return st;
  if ((st = check_layers(x, lb, lc))) return st;
  if (!q || !tau || !mask) return fail(SEKV_EINVAL, "null q, tau or mask");
  if (!aligned(q, 16) || !aligned(mask, 8)) return fail(SEKV_EINVAL, "q must be 16-byte and mask 8-byte aligned");
  if (budget < 0) return fail(SEKV_EINVAL, "budget < 0");
  if (alpha && ((uintptr_t)alpha & 15)) return fail(SEKV_EINVAL, "alpha must be 16-byte aligned");
  if ((st = set_device(c))) return st;
  if (budget > 0 && ((st = ensure_route_scratch(x, lc, x->d_score)) || (st = ensure_route_scratch(x, lc, x->d_packed))))
    return st;
  RouteArgs ra{};
  ra.q = (const bf16_t*)q;
  ra.tau = tau;
  ra.W = (const float*)x->d_W.p;
  ra.s = (const float*)x->d_s.p;
  ra.meta = (const BMeta*)x->d_meta.p;
  ra.mask = mask;
  ra.alpha = alpha;
  ra.score = budget > 0 ? (float*)x->d_score.p : nullptr;
  ra.packed = budget > 0 ? (uint32_t*)x->d_packed.p : nullptr;
  ra.layer_begin = lb; ra.layer_count = lc;
  ra.B = x->B; ra.L = x->L; ra.Hq = x->Hq; ra.Hkv = x->Hkv; ra.D = x->D; ra.dp = x->dp; ra.Wd = x->Wd;
  ra.cap = 0;
  ra.budget = budget;
  ra.stream = stream_hint(x);
  size_t slot = 0;
  if (c->timing) HIP_TRY(c->t_route.begin(c->stream, &slot));
  HIP_TRY(launch_route(ra, c->stream));
  if (budget > 0) HIP_TRY(launch_route_pool(ra, c->stream));
  if (c->timing) HIP_TRY(c->t_route.end(c->stream, slot));
  return SEKV_OK;
}

extern "C" sekv_status sekv_calibrate_tau(sekv_ctx* c, const sekv_index* xc, int32_t lb, int32_t lc,
                                          const void* q_cal, float frac, float* tau_out) {
  sekv_index* x = const_cast<sekv_index*>(xc);
  sekv_status st = check_idx(c, x);
  if (st) return st;
  if ((st = check_layers(x, lb, lc))) return st;
  if (!q_cal || !tau_out) return fail(SEKV_EINVAL, "null q_cal or tau_out");
  if (!aligned(q_cal, 16)) return fail(SEKV_EINVAL, "q_cal must be 16-byte aligned");
  if (!(frac >= 0.f && frac <= 1.f)) return fail(SEKV_EINVAL, "frac must be in [0, 1]");
  if (x->total_spans < 2) return fail(SEKV_EINVAL, "calibration needs at least 2 spans");
  if ((st = set_device(c))) return st;
  if ((st = ensure_route_scratch(x, lc, x->d_alpha))) return st;
  const size_t ntau = (size_t)lc * x->Hq;
  if (!x->d_tau_inf.p || x->d_tau_inf.n < 4 * ntau) {
    HIP_TRY(dalloc(x->d_tau_inf, 4 * ntau));
    std::vector<float> inf(ntau, INFINITY);
    HIP_TRY(hipMemcpyAsync(x->d_tau_inf.p, inf.data(), 4 * ntau, hipMemcpyHostToDevice, c->stream));
    HIP_TRY(hipStreamSynchronize(c->stream));
  }
  DBuf mk;
  struct Rel { DBuf* b; ~Rel() { b->release(); } } rel{&mk};
  HIP_TRY(dalloc(mk, 8 * (size_t)x->B * lc * x->Hq * x->Wd));
  RouteArgs ra{};
  ra.q = (const bf16_t*)q_cal;
  ra.tau = (const float*)x->d_tau_inf.p;
  ra.W = (const float*)x->d_W.p;
  ra.s = (const float*)x->d_s.p;
  ra.meta = (const BMeta*)x->d_meta.p;
  ra.mask = (uint64_t*)mk.p;
  ra.alpha = (float*)x->d_alpha.p;
  ra.score = nullptr;
  ra.layer_begin = lb; ra.layer_count = lc;
  ra.B = x->B; ra.L = x->L; ra.Hq = x->Hq; ra.Hkv = x->Hkv; ra.D = x->D; ra.dp = x->dp; ra.Wd = x->Wd;
  ra.cap = 0;
  HIP_TRY(launch_route(ra, c->stream));
  CalibArgs ca{};
  ca.alpha = (const float*)x->d_alpha.p;
  ca.meta = (const BMeta*)x->d_meta.p;
  ca.tau_out = tau_out;
  ca.layer_count = lc; ca.B = x->B; ca.Hq = x->Hq; ca.Wd = x->Wd; ca.frac = frac;
  HIP_TRY(launch_calibrate(ca, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));  // the temporary mask is freed on return
  return SEKV_OK;
}

namespace {

// Softmax-partial bytes of one decode call over lc layers.
size_t part_bytes(const sekv_index* x, int lc) {
  return sizeof(float) * (size_t)lc * std::max<size_t>(x->items.size(), 1) * x->G * (x->D + 2);
}

// The staging ring of the pinned tier holds one or two layer slots, each a
// mirror of one layer's factor region (blobs at their offsets within it).
int64_t ring_slot_bytes(const sekv_index* x) { return (x->max_layer_bytes + 255) & ~255LL; }
int ring_slots(const sekv_index* x) {
  const int64_t sb = std::max<int64_t>(ring_slot_bytes(x), 256);
  return (int)std::min<int64_t>(2, x->ring_bytes / sb);
}

sekv_status check_ring(const sekv_index* x) {
  if (x->tier == SEKV_TIER_PINNED_HOST && ring_slots(x) < 1)
    return fail(SEKV_ECAPACITY, "staging ring of %lld bytes holds less than one layer's factors (%lld bytes)",
                (long long)x->ring_bytes, (long long)ring_slot_bytes(x));
  return SEKV_OK;
}

// Gather (pinned tier), attention items writing their partials to `part`,
// merge into out.  Asynchronous unless stats are asked for on the pinned tier
// (then the union sizes and the gather times are read back).
//
// Pinned tier: layer li of the call is gathered into ring slot li % slots and
// attended from there.  With two slots and more than one layer the gathers run
// on the index's copy stream, one layer ahead: layer li + 1 crosses PCIe while
// layer li is attended ([Method] Fig. 2: asynchronous transfer overlapped with
// the pipeline), and the gather into a slot waits for the attention of the
// layer that used it before.
sekv_status decode_run(sekv_ctx* c, sekv_index* x, int lb, int lc, const void* q, const uint64_t* mask, float* out,
                       sekv_stats* stats, float* part, int2* gstat, bool timed) {
  if (stats) memset(stats, 0, sizeof *stats);
  const int n_items = (int)x->items.size();
  hipStream_t st = c->stream;
  const bool pinned = x->tier == SEKV_TIER_PINNED_HOST;
  AttendArgs aa{};
  aa.q = (const bf16_t*)q;
  aa.mask = mask;
  aa.meta = (const BMeta*)x->d_meta.p;
  aa.items = (const WorkItem*)x->d_items.p;
  aa.kres = (const bf16_t*)x->d_kres.p;
  aa.vres = (const bf16_t*)x->d_vres.p;
  aa.logn = (const float*)x->d_logn.p;
  aa.span_len = (const int32_t*)x->d_span_len.p;
  aa.bref = (const uint2*)x->d_bref.p;
  aa.layer_off = (const int64_t*)x->d_layer_off.p;
  aa.pool = (const uint8_t*)x->d_pool.p;
  aa.pool_layer0 = 0;
  aa.part = part;
  aa.total_spans = x->total_spans;
  aa.layer_begin = lb; aa.layer_count = lc; aa.n_items = n_items;
  aa.lc_first = 0; aa.lc_count = lc;
  aa.B = x->B; aa.L = x->L; aa.Hq = x->Hq; aa.Hkv = x->Hkv; aa.W = x->Wd;
  aa.max_spans = std::max(x->max_spans, 1);
  aa.scale = 1.0f / sqrtf((float)x->D);
  aa.stream = stream_hint(x);
  auto attend = [&]() -> sekv_status {
    if (n_items <= 0) return SEKV_OK;
    if (timed) {
      size_t slot = 0;
      HIP_TRY(c->t_attend.reserve(&slot));
      HIP_TRY(launch_attend(aa, x->D, x->G, x->R, st, c->t_attend.ev[slot], c->t_attend.ev[slot + 1]));
    } else {
      HIP_TRY(launch_attend(aa, x->D, x->G, x->R, st));
    }
    return SEKV_OK;
  };
  sekv_status rs;
  if (!pinned) {
    if ((rs = attend())) return rs;
  } else {
    GatherArgs ga{};
    ga.mask = mask;
    ga.meta = (const BMeta*)x->d_meta.p;
    ga.span_len = (const int32_t*)x->d_span_len.p;
    ga.bref = (const uint2*)x->d_bref.p;
    ga.layer_off = (const int64_t*)x->d_layer_off.p;
    ga.host_pool = x->d_host_pool;
    ga.stat = gstat;
    ga.total_spans = x->total_spans;
    ga.layer_begin = lb; ga.layer_count = lc; ga.B = x->B; ga.Hq = x->Hq; ga.Hkv = x->Hkv;
    ga.W = x->Wd; ga.G = x->G; ga.D = x->D;
    ga.nsplit = std::max(1, (x->max_spans + gather_share() - 1) / gather_share());
    const int slots = ring_slots(x);
    const bool overlap = slots >= 2 && lc >= 2;
    hipStream_t gs = overlap ? x->copy : st;
    if (stats && x->gev.size() < (size_t)2 * lc) {
      while (x->gev.size() < (size_t)2 * lc) {
        hipEvent_t e = nullptr;
        HIP_TRY(hipEventCreate(&e));
        x->gev.push_back(e);
      }
    }
    if (overlap) {   // the copy stream starts after the work already on the call's stream (the masks)
      HIP_TRY(hipEventRecord(x->ev_call, st));
      HIP_TRY(hipStreamWaitEvent(gs, x->ev_call, 0));
    }
    for (int li = 0; li < lc; ++li) {
      const int k = li % slots;
      const int l = lb + li;
      uint8_t* ring = (uint8_t*)x->d_ring.p + (size_t)k * ring_slot_bytes(x);
      ga.ring = ring;
      ga.ring_layer0 = l;
      ga.lc_first = li; ga.lc_count = 1;
      if (overlap && li >= slots) HIP_TRY(hipStreamWaitEvent(gs, x->ev_free[k], 0));
      if (stats) HIP_TRY(hipEventRecord(x->gev[2 * li], gs));
      HIP_TRY(launch_gather(ga, gs));
      if (stats) HIP_TRY(hipEventRecord(x->gev[2 * li + 1], gs));
      if (overlap) {
        HIP_TRY(hipEventRecord(x->ev_ready[k], gs));
        HIP_TRY(hipStreamWaitEvent(st, x->ev_ready[k], 0));
      }
      aa.pool = ring;
      aa.pool_layer0 = l;
      aa.lc_first = li; aa.lc_count = 1;
      if ((rs = attend())) return rs;
      if (overlap) HIP_TRY(hipEventRecord(x->ev_free[k], st));
    }
  }
  MergeArgs mg{};
  mg.part = part;
  mg.items = (const WorkItem*)x->d_items.p;
  mg.bg_first = (const int32_t*)x->d_bg_first.p;
  mg.out = out;
  mg.layer_count = lc; mg.n_items = n_items; mg.B = x->B; mg.Hq = x->Hq; mg.Hkv = x->Hkv;
  HIP_TRY(launch_merge(mg, x->D, x->G, st));
  if (pinned && stats && gstat) {
    const size_t nreg = (size_t)lc * x->B * x->Hkv;
    x->h_gstat.resize(nreg);
    HIP_TRY(hipMemcpyAsync(x->h_gstat.data(), gstat, sizeof(int2) * nreg, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    uint64_t un = 0, by = 0;
    for (const int2& v : x->h_gstat) {
      un += (uint64_t)v.x;
      by += (uint64_t)v.y << 8;
    }
    double ms = 0.0;
    for (int li = 0; li < lc; ++li) {
      float m = 0.f;
      HIP_TRY(hipEventElapsedTime(&m, x->gev[2 * li], x->gev[2 * li + 1]));
      ms += m;
    }
    stats->union_spans = un;
    stats->pcie_bytes = by;
    stats->pcie_copies = (uint64_t)lc;
    stats->pcie_ms = ms;
  }
  return SEKV_OK;
}

}  // namespace

extern "C" sekv_status sekv_decode_attend(sekv_ctx* c, const sekv_index* xc, int32_t lb, int32_t lc,
                                          const void* q, const uint64_t* mask, float* out, sekv_stats* stats) {
  sekv_index* x = const_cast<sekv_index*>(xc);
  sekv_status st = check_idx(c, x);
  if (st) return st;
  if ((st = check_layers(x, lb, lc))) return st;
  if (!q || !mask || !out) return fail(SEKV_EINVAL, "null q, mask or out");
  if (!aligned(q, 16) || !aligned(mask, 8)) return fail(SEKV_EINVAL, "q must be 16-byte and mask 8-byte aligned");
  if ((st = check_ring(x))) return st;
  if ((st = set_device(c))) return st;
  HIP_TRY(dgrow(x->d_part, part_bytes(x, lc)));
  int2* gstat = nullptr;
  if (stats && x->tier == SEKV_TIER_PINNED_HOST) {
    HIP_TRY(dgrow(x->d_gstat, sizeof(int2) * (size_t)lc * x->B * x->Hkv));
    gstat = (int2*)x->d_gstat.p;
  }
  return decode_run(c, x, lb, lc, q, mask, out, stats, (float*)x->d_part.p, gstat, c->timing);
}

extern "C" sekv_status sekv_decode_attend_noalloc(sekv_ctx* c, const sekv_index* xc, int32_t lb, int32_t lc,
                                                  const void* q, const uint64_t* mask, float* out,
                                                  sekv_stats* stats) {
  sekv_index* x = const_cast<sekv_index*>(xc);
  sekv_status st = check_idx(c, x);
  if (st) return st;
  if ((st = check_layers(x, lb, lc))) return st;
  if (!q || !mask || !out) return fail(SEKV_EINVAL, "null q, mask or out");
  if (!aligned(q, 16) || !aligned(mask, 8)) return fail(SEKV_EINVAL, "q must be 16-byte and mask 8-byte aligned");
  if (x->tier != SEKV_TIER_HBM)
    return fail(SEKV_EUNSUPPORTED, "the no-allocation decode serves the HBM tier only");
  const size_t need = part_bytes(x, lc);
  if (need > kScratchBytes)
    return fail(SEKV_ECAPACITY, "this call needs %zu bytes of partials; the no-allocation scratch holds %zu "
                                "(call fewer layers at once)", need, kScratchBytes);
  if (c->device >= kMaxScratchDevices || !g_scratch[c->device])
    return fail(SEKV_ESTATE, "no scratch address for device %d", c->device);
  if ((st = set_device(c))) return st;
  return decode_run(c, x, lb, lc, q, mask, out, stats, (float*)g_scratch[c->device], nullptr, false);
}
