// libpe: context, host store, orchestration and the C ABI declared in include/pe.h.
//
// SGLang "Paged Experts" docs page: "The K-slot table and the host store"
// (K-row slot tables on the GPU, every expert in a page-locked host store whose
// rows have the slots' layout), "A step: waves, page-in, merge" and "Captured
// decode" (one device-planned wave with no host synchronisation when
// tokens x top_k <= K, host-planned waves otherwise, one shared LRU state).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/pe.h"
#include "pe_kernels.h"
#include "pe_layout.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define PE_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(PE_ERR_HIP, "%s failed: %s (line %d)", #call, hipGetErrorString(e_), \
                  __LINE__);                                                          \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct BlobLayout {
  size_t w13, w2, s13, s2;              // sub-tensor bytes
  size_t off_w13, off_w2, off_s13, off_s2;
  size_t algorithmic, copied, stride;
};

// One contiguous blob per expert: W13 | W2 | S13 | S2, each 256-byte aligned.
// Keeping every sub-tensor of an expert in one blob means one page-in moves all
// of them; no part of an expert can be left behind in a slot.
bool blob_layout(int wtype, int H, int I, BlobLayout* b) {
  const size_t n13 = (size_t)2 * I * H, n2 = (size_t)H * I;
  switch (wtype) {
    case PE_W_BF16: b->w13 = 2 * n13; b->w2 = 2 * n2; b->s13 = 0; b->s2 = 0; break;
    case PE_W_FP8_B128:
      b->w13 = n13; b->w2 = n2;
      b->s13 = (size_t)(2 * I / 128) * (H / 128) * 4;
      b->s2 = (size_t)(H / 128) * (I / 128) * 4;
      break;
    case PE_W_INT4_G128:
      b->w13 = n13 / 2; b->w2 = n2 / 2;
      b->s13 = (size_t)2 * I * (H / 128) * 2;
      b->s2 = (size_t)H * (I / 128) * 2;
      break;
    case PE_W_INT8_G128:
      b->w13 = n13; b->w2 = n2;
      b->s13 = (size_t)2 * I * (H / 128) * 2;
      b->s2 = (size_t)H * (I / 128) * 2;
      break;
    case PE_W_MXFP4_B32:
      b->w13 = n13 / 2; b->w2 = n2 / 2;
      b->s13 = (size_t)2 * I * (H / 32);
      b->s2 = (size_t)H * (I / 32);
      break;
    default: return false;
  }
  b->off_w13 = 0;
  b->off_w2 = align_up(b->off_w13 + b->w13, 256);
  b->off_s13 = align_up(b->off_w2 + b->w2, 256);
  b->off_s2 = align_up(b->off_s13 + b->s13, 256);
  b->copied = align_up(b->off_s2 + b->s2, 256);
  b->stride = align_up(b->copied, 4096);
  b->algorithmic = b->w13 + b->w2 + b->s13 + b->s2;
  return true;
}

// Page-in grid: a one-expert copy (9.4 MB) is fastest with few blocks and two 16-byte
// loads in flight per thread (about 169 us, 56 GB/s, back to back), and a small grid
// leaves most CUs to the expert kernels that overlap it.
constexpr int kPageInGrid = 128;
// Copier workgroups of a device-planned step, which page in the missing experts
// and compute their gate/up projection on the way (96 divides the gate/up row
// blocks of every format at hidden 2048 / inter 768: 192, 96 and 48).
constexpr int kStreamWgs = 96;

static_assert(pe::kStaticScratchBytes == PE_STATIC_SCRATCH_BYTES, "the fixed scratch size is stated in pe.h");

}  // namespace

struct pe_ctx {
  pe_config cfg{};
  pe::Dims d{};
  pe::LayerLayout ll{};
  pe::WorkLayout wl{};
  pe::Offsets o{};
  BlobLayout b{};
  bool unpaged = false;
  int mfma_min = pe::kNoMfma;         // = d.mfma_min
  uint8_t* host_store = nullptr;       // page-locked, mapped: [L][E][stride]
  uint8_t* host_store_dev = nullptr;   // its device-visible address
  uint8_t* slots = nullptr;            // device: [L][K][stride]
  size_t layer_words = 0;              // ll.total + wl.total, rounded: a layer's block, then its work lists
  int32_t* blocks = nullptr;           // device: [L][layer_words]
  uint16_t* h = nullptr;               // device: [max_entries][I] bf16
  float* merged = nullptr;             // device: [max_entries][H] fp32
  unsigned long long* stats = nullptr; // device: [ST_COUNT]
  // Page-locked, mapped, coherent host staging of host-planned steps: the routed
  // ids and the host mirror of each layer's block and work lists.  A step's
  // first launch writes the ids and the block's LRU state into them through
  // their device addresses; the host plans in the mirror, and one more launch
  // reads the block and work lists back from it.
  int32_t* st_ids = nullptr;           // [max_entries]
  int32_t* st_blk = nullptr;           // [L][layer_words]
  int32_t* st_ids_dev = nullptr;       // device-visible addresses of the two
  int32_t* st_blk_dev = nullptr;
  // The read-back's completion word (page-locked, mapped, coherent): the launch
  // stores the step's sequence number there once its writes are visible, and
  // the host polls it instead of synchronising the stream.
  uint32_t* st_flag = nullptr;
  uint32_t* st_flag_dev = nullptr;
  uint32_t gather_seq = 0;
  pe::HostPlanSummary* sum = nullptr;
  // plan log (PE_FLAG_PLAN_LOG): per layer a ring of log_cap records
  pe::PlanLogLayout pl{};
  int log_cap = 0;
  int32_t* plan_log = nullptr;         // device: [L][log_cap][pl.total]
  uint32_t* log_seq = nullptr;         // device: [L] steps logged per layer
  unsigned long long host_counts[pe::ST_COUNT] = {};
  // Second stream (default priority): runs the experts that were already
  // resident while the page-in is in flight; forked and joined with events.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // measurement mode
  bool timing = false;
  std::vector<hipEvent_t> ev_free;
  struct Pending { int stage; hipEvent_t a, b; };
  std::vector<Pending> pending;
  double stage_ms[PE_NUM_STAGES] = {};
  unsigned long long stage_n[PE_NUM_STAGES] = {};
};

namespace {

void free_ctx(pe_ctx* c) {
  if (!c) return;
  for (auto& p : c->pending) { (void)hipEventDestroy(p.a); (void)hipEventDestroy(p.b); }
  for (hipEvent_t e : c->ev_free) (void)hipEventDestroy(e);
  if (c->host_store) (void)hipHostFree(c->host_store);
  if (c->st_ids) (void)hipHostFree(c->st_ids);
  if (c->st_blk) (void)hipHostFree(c->st_blk);
  if (c->st_flag) (void)hipHostFree(c->st_flag);
  for (void* p : {(void*)c->slots, (void*)c->blocks, (void*)c->h, (void*)c->merged,
                  (void*)c->stats, (void*)c->plan_log, (void*)c->log_seq})
    if (p) (void)hipFree(p);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->side) (void)hipStreamDestroy(c->side);
  delete c->sum;
  delete c;
}

int use_device(const pe_ctx* c) {
  int cur = -1;
  PE_HIP(hipGetDevice(&cur));
  if (cur != c->cfg.device) PE_HIP(hipSetDevice(c->cfg.device));
  return PE_OK;
}

// Where a step's activations go: the context's buffers, or the fixed scratch area.
struct Act {
  uint16_t* h;
  float* merged;
};

pe::ExpertArgs expert_args(pe_ctx* c, const Act& act, int layer, int wave, const void* x, const float* w,
                           int part = 0) {
  pe::ExpertArgs a{};
  a.part = part;
  a.slots = c->slots + (size_t)layer * c->d.K * c->b.stride;
  a.slot_stride = c->b.stride;
  a.off_w13 = c->b.off_w13; a.off_w2 = c->b.off_w2; a.off_s13 = c->b.off_s13; a.off_s2 = c->b.off_s2;
  a.work = c->blocks + (size_t)layer * c->layer_words + c->ll.total;
  a.o = c->o;
  a.MW = c->d.max_waves;
  a.wave = wave;
  a.x = static_cast<const uint16_t*>(x);
  a.topk_w = w;
  a.h = act.h;
  a.merged = act.merged;
  a.H = c->d.H; a.I = c->d.I; a.k = c->d.k;
  a.lean = 0;
  a.mfma_min = c->mfma_min;
  return a;
}

hipEvent_t take_event(pe_ctx* c) {
  if (!c->ev_free.empty()) {
    hipEvent_t e = c->ev_free.back();
    c->ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Fold finished event pairs into the per-stage sums; with `wait`, all of them.
int drain_timing(pe_ctx* c, bool wait) {
  size_t keep = 0;
  for (size_t i = 0; i < c->pending.size(); ++i) {
    auto& p = c->pending[i];
    if (!wait && hipEventQuery(p.b) != hipSuccess) { c->pending[keep++] = p; continue; }
    PE_HIP(hipEventSynchronize(p.b));
    float ms = 0.f;
    PE_HIP(hipEventElapsedTime(&ms, p.a, p.b));
    c->stage_ms[p.stage] += ms;
    c->stage_n[p.stage] += 1;
    c->ev_free.push_back(p.a);
    c->ev_free.push_back(p.b);
  }
  c->pending.resize(keep);
  return PE_OK;
}

// Brackets one stage's launches with events when timing is on (and `on`).
struct StageTimer {
  pe_ctx* c;
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr;
  StageTimer(pe_ctx* c_, int stage_, hipStream_t s_, bool on = true) : c(c_), stage(stage_), s(s_) {
    if (!c->timing || !on) return;
    a = take_event(c);
    if (a && hipEventRecord(a, s) != hipSuccess) a = nullptr;
  }
  ~StageTimer() {
    if (!a) return;
    hipEvent_t b = take_event(c);
    if (!b || hipEventRecord(b, s) != hipSuccess) { c->ev_free.push_back(a); return; }
    c->pending.push_back({stage, a, b});
    if (c->pending.size() > 4096) (void)drain_timing(c, false);
    if (c->pending.size() > 8192) (void)drain_timing(c, true);
  }
};

// A host-planned wave's GEMV and MFMA ranges in the work lists (first, first
// paged-in, end), which its launches then take as arguments instead of
// reading the work arena's header.
struct WaveRanges { int g0, gsplit, g1, t0, tsplit, t1; };

// Expert kernels (gate/up then down; GEMV items, then MFMA tiles) of one part
// of one wave.  `items`/`tiles` bound the launches' grids; `max_m` bounds the
// GEMV experts' token counts; `wr`, if given, are the wave's ranges.
void set_ranges(pe::ExpertArgs& a, const WaveRanges& wr) {
  a.hdr_known = 1;
  a.g0 = wr.g0; a.gsplit = wr.gsplit; a.g1 = wr.g1;
  a.t0 = wr.t0; a.tsplit = wr.tsplit; a.t1 = wr.t1;
}

void run_experts(pe_ctx* c, const Act& act, bool tm_on, int layer, int wave, int part, const void* x,
                 const float* w, int items, int max_m, int tiles, hipStream_t s, const WaveRanges* wr = nullptr) {
  pe::ExpertArgs a = expert_args(c, act, layer, wave, x, w, part);
  if (wr) set_ranges(a, *wr);
  if (items > 0) {
    {
      StageTimer tm(c, PE_STAGE_GATE_UP, s, tm_on);
      pe::launch_gemv_gate_up(c->cfg.wtype, a, items, max_m, s);
    }
    StageTimer tm(c, PE_STAGE_DOWN, s, tm_on);
    pe::launch_gemv_down(c->cfg.wtype, a, items, max_m, s);
  }
  if (tiles > 0) {
    {
      StageTimer tm(c, PE_STAGE_GATE_UP, s, tm_on);
      pe::launch_mfma_gate_up(c->cfg.wtype, a, tiles, s);
    }
    StageTimer tm(c, PE_STAGE_DOWN, s, tm_on);
    pe::launch_mfma_down(c->cfg.wtype, a, tiles, s);
  }
}

// The LDS a one-wave down projection + top-k sum launch (launch_down_sum) takes
// for n routed entries at most (row blocks of up to 16 rows: per entry 16 fp32
// results plus its id, sorted position and router weight).  Steps whose
// launch would need more than one workgroup may take run the down kernel into
// the merged buffer and the separate top-k sum instead: the same arithmetic.
bool down_sum_fits(int n) { return (size_t)n * 76 + 64 <= 64 * 1024; }

}  // namespace

extern "C" {

const char* pe_strerror(int status) {
  switch (status) {
    case PE_OK: return "ok";
    case PE_ERR_INVALID_ARG: return "invalid argument";
    case PE_ERR_UNSUPPORTED: return "unsupported";
    case PE_ERR_OOM_HOST_PIN: return "cannot pin host memory";
    case PE_ERR_OOM_DEVICE: return "out of device memory";
    case PE_ERR_HIP: return "HIP runtime error";
    case PE_ERR_NOT_CAPTURABLE: return "host-planned step under stream capture";
    default: return "unknown status";
  }
}

const char* pe_last_error(void) { return g_err.c_str(); }

namespace {
// The format's divisibility rule for hidden and inter: whole 16-byte chunks
// per row (bf16: 8), whole scale groups (FP8 / int4 / int8: 128), and whole
// 32-column MXFP4 blocks with 2-byte aligned row scales (64).
int check_multiples(int wtype, int hidden, int inter) {
  if (wtype == PE_W_MXFP4_B32) {
    if (hidden % 64 || inter % 64) return fail(PE_ERR_INVALID_ARG, "MXFP4 needs hidden and inter multiples of 64");
  } else if (wtype != PE_W_BF16 && (hidden % 128 || inter % 128)) {
    return fail(PE_ERR_INVALID_ARG, "quantized formats need hidden and inter multiples of 128");
  }
  return PE_OK;
}
}  // namespace

int pe_expert_bytes(int wtype, int hidden, int inter, size_t* algorithmic, size_t* copied) {
  if (hidden <= 0 || inter <= 0) return fail(PE_ERR_INVALID_ARG, "hidden and inter must be positive");
  if (int rc = check_multiples(wtype, hidden, inter)) return rc;
  BlobLayout b;
  if (!blob_layout(wtype, hidden, inter, &b)) return fail(PE_ERR_INVALID_ARG, "unknown weight type %d", wtype);
  if (algorithmic) *algorithmic = b.algorithmic;
  if (copied) *copied = b.copied;
  return PE_OK;
}

int pe_suggest_k(int wtype, int hidden, int inter, int num_layers, int num_experts, int top_k,
                 double budget_bytes) {
  size_t alg = 0, copied = 0;
  const int rc = pe_expert_bytes(wtype, hidden, inter, &alg, &copied);
  if (rc) return rc;
  if (num_layers < 1 || num_experts < 1 || top_k < 1 || top_k > num_experts || !(budget_bytes >= 0))
    return fail(PE_ERR_INVALID_ARG, "bad sizing arguments");
  const double per_slot = (double)copied * num_layers;
  const double k = budget_bytes / per_slot;
  const int K = k >= num_experts ? num_experts : (int)k;
  if (K < top_k)
    return fail(PE_ERR_INVALID_ARG, "budget holds %d slots per layer, fewer than top_k=%d", K, top_k);
  return K;
}

int pe_create(const pe_config* cfg, pe_ctx** out) {
  if (!out) return fail(PE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(PE_ERR_INVALID_ARG, "cfg is NULL");
  const pe_config& g = *cfg;
  const bool unpaged = (g.flags & PE_FLAG_UNPAGED) != 0;
  if (g.num_layers < 1) return fail(PE_ERR_INVALID_ARG, "num_layers must be >= 1");
  if (g.num_experts < 1 || g.num_experts > pe::kMaxExperts)
    return fail(PE_ERR_INVALID_ARG, "num_experts must be in [1, %d]", pe::kMaxExperts);
  if (g.top_k < 1 || g.top_k > g.num_experts) return fail(PE_ERR_INVALID_ARG, "top_k must be in [1, E]");
  const int K = unpaged ? g.num_experts : g.num_resident;
  if (K < g.top_k) return fail(PE_ERR_INVALID_ARG, "num_resident K=%d must be at least top_k=%d", K, g.top_k);
  if (K > g.num_experts) return fail(PE_ERR_INVALID_ARG, "num_resident K=%d exceeds num_experts", K);
  if (g.max_tokens < 1) return fail(PE_ERR_INVALID_ARG, "max_tokens must be >= 1");
  if (g.hidden <= 0 || g.inter <= 0 || g.hidden % 8 || g.inter % 8)
    return fail(PE_ERR_INVALID_ARG, "hidden and inter must be positive multiples of 8");
  if (g.hidden > 4096 || g.inter > 4096)
    return fail(PE_ERR_UNSUPPORTED, "hidden and inter above 4096 are not supported");
  if (g.wtype < PE_W_BF16 || g.wtype > PE_W_MXFP4_B32)
    return fail(PE_ERR_INVALID_ARG, "unknown weight type %d", g.wtype);
  if (int rc = check_multiples(g.wtype, g.hidden, g.inter)) return rc;
  if (g.flags & ~(PE_FLAG_PAGEIN_DMA | PE_FLAG_FORCE_HOST_PLAN | PE_FLAG_UNPAGED | PE_FLAG_PLAN_LOG))
    return fail(PE_ERR_INVALID_ARG, "unknown flags 0x%x", g.flags);
  const bool plan_log = (g.flags & PE_FLAG_PLAN_LOG) != 0;
  if (plan_log && (g.plan_log_steps < 1 || g.plan_log_steps > (1 << 24)))
    return fail(PE_ERR_INVALID_ARG, "PE_FLAG_PLAN_LOG needs plan_log_steps in [1, 2^24]");
  if ((long long)g.max_tokens * g.top_k > (1 << 24))
    return fail(PE_ERR_UNSUPPORTED, "max_tokens * top_k too large");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || g.device < 0 || g.device >= ndev)
    return fail(PE_ERR_INVALID_ARG, "device %d not available", g.device);

  pe_ctx* c = new pe_ctx;
  c->cfg = g;
  c->cfg.num_resident = K;
  c->unpaged = unpaged;
  c->d = pe::make_dims(g.num_layers, g.num_experts, K, g.top_k, g.hidden, g.inter, g.max_tokens);
  c->ll = pe::make_layer_layout(c->d);
  c->wl = pe::make_work_layout(c->d);
  c->layer_words = c->ll.total + c->wl.total;     // both multiples of 64 words
  c->o = pe::make_offsets(c->ll, c->wl);
  blob_layout(g.wtype, g.hidden, g.inter, &c->b);
  // The MFMA kernels stage K in blocks of 64 (bf16, MXFP4) or 128 (scaled formats).
  const int mm = pe::mfma_multiple(g.wtype);
  c->mfma_min = (g.hidden % mm == 0 && g.inter % mm == 0) ? pe::kMfmaMinTokens : pe::kNoMfma;
  c->d.mfma_min = c->mfma_min;
  c->pl = pe::make_plan_log_layout(c->d, c->ll);
  c->log_cap = plan_log ? g.plan_log_steps : 0;
  c->sum = new pe::HostPlanSummary;
  int rc = use_device(c);
  if (rc) { free_ctx(c); return rc; }

  const pe::Dims& d = c->d;
  if (!unpaged) {
    size_t bytes = (size_t)d.L * d.E * c->b.stride;
    if (hipHostMalloc(reinterpret_cast<void**>(&c->host_store), bytes, hipHostMallocMapped) != hipSuccess) {
      c->host_store = nullptr;
      (void)hipGetLastError();
      free_ctx(c);
      return fail(PE_ERR_OOM_HOST_PIN, "cannot pin %zu bytes of host memory for the expert store", bytes);
    }
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, c->host_store, 0) != hipSuccess) {
      free_ctx(c);
      return fail(PE_ERR_HIP, "hipHostGetDevicePointer failed for the host store");
    }
    c->host_store_dev = static_cast<uint8_t*>(dp);
  }
  struct { void** p; size_t bytes; } dev[] = {
      {reinterpret_cast<void**>(&c->slots), (size_t)d.L * d.K * c->b.stride},
      {reinterpret_cast<void**>(&c->blocks), (size_t)d.L * c->layer_words * 4},
      {reinterpret_cast<void**>(&c->h), (size_t)d.max_entries * d.I * 2},
      {reinterpret_cast<void**>(&c->merged), (size_t)d.max_entries * d.H * 4},
      {reinterpret_cast<void**>(&c->stats), pe::ST_COUNT * 8},
      {reinterpret_cast<void**>(&c->plan_log), (size_t)d.L * c->log_cap * c->pl.total * 4},
      {reinterpret_cast<void**>(&c->log_seq), (size_t)d.L * 4},
  };
  for (auto& a : dev) {
    if (a.bytes == 0) continue;
    if (hipMalloc(a.p, a.bytes) != hipSuccess) {
      *a.p = nullptr;
      (void)hipGetLastError();
      free_ctx(c);
      return fail(PE_ERR_OOM_DEVICE, "cannot allocate %zu bytes of device memory", a.bytes);
    }
  }
  struct { int32_t** p; size_t words; } pin[] = {
      {&c->st_ids, (size_t)d.max_entries}, {&c->st_blk, (size_t)d.L * c->layer_words},
      {reinterpret_cast<int32_t**>(&c->st_flag), 64}};
  for (auto& a : pin) {
    if (hipHostMalloc(reinterpret_cast<void**>(a.p), a.words * 4, hipHostMallocMapped | hipHostMallocCoherent) !=
        hipSuccess) {
      *a.p = nullptr;
      (void)hipGetLastError();
      free_ctx(c);
      return fail(PE_ERR_OOM_HOST_PIN, "cannot pin staging buffers");
    }
  }
  {
    void* a = nullptr;
    void* b = nullptr;
    void* f = nullptr;
    if (hipHostGetDevicePointer(&a, c->st_ids, 0) != hipSuccess ||
        hipHostGetDevicePointer(&b, c->st_blk, 0) != hipSuccess ||
        hipHostGetDevicePointer(&f, c->st_flag, 0) != hipSuccess) {
      free_ctx(c);
      return fail(PE_ERR_HIP, "hipHostGetDevicePointer failed for the staging buffers");
    }
    c->st_ids_dev = static_cast<int32_t*>(a);
    c->st_blk_dev = static_cast<int32_t*>(b);
    c->st_flag_dev = static_cast<uint32_t*>(f);
    *c->st_flag = 0;
  }
  if (hipMemset(c->stats, 0, pe::ST_COUNT * 8) != hipSuccess ||
      hipMemset(c->blocks, 0, (size_t)d.L * c->layer_words * 4) != hipSuccess ||
      (c->log_seq && hipMemset(c->log_seq, 0, (size_t)d.L * 4) != hipSuccess)) {
    free_ctx(c);
    return fail(PE_ERR_HIP, "initialising device buffers failed");
  }
  if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess) {
    free_ctx(c);
    return fail(PE_ERR_HIP, "creating the side stream and its events failed");
  }
  pe::launch_reset_lru(c->blocks, c->layer_words, 0, d.L, c->o, d.E, d.K, unpaged, nullptr);
  if (hipDeviceSynchronize() != hipSuccess) {
    free_ctx(c);
    return fail(PE_ERR_HIP, "resetting the LRU state failed: %s", hipGetErrorString(hipGetLastError()));
  }
  // The fixed scratch area of pe_forward_static: its address on this device,
  // looked up once per device while the device is current.
  if (!pe::static_scratch(g.device)) {
    free_ctx(c);
    return fail(PE_ERR_HIP, "hipGetSymbolAddress failed for the fixed scratch area");
  }
  *out = c;
  return PE_OK;
}

void pe_destroy(pe_ctx* ctx) {
  if (!ctx) return;
  (void)use_device(ctx);
  (void)hipDeviceSynchronize();
  free_ctx(ctx);
}

int pe_load_expert(pe_ctx* c, int layer, int expert, const void* w13, const void* w2, const void* s13,
                   const void* s2) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  if (layer < 0 || layer >= c->d.L || expert < 0 || expert >= c->d.E)
    return fail(PE_ERR_INVALID_ARG, "layer %d / expert %d out of range", layer, expert);
  if (!w13 || !w2) return fail(PE_ERR_INVALID_ARG, "w13 and w2 are required");
  const bool quant = c->cfg.wtype != PE_W_BF16;
  if (quant && (!s13 || !s2)) return fail(PE_ERR_INVALID_ARG, "scales are required for quantized formats");
  const BlobLayout& b = c->b;
  if (c->unpaged) {
    int rc = use_device(c);
    if (rc) return rc;
    uint8_t* dst = c->slots + ((size_t)layer * c->d.K + expert) * b.stride;
    PE_HIP(hipMemcpy(dst + b.off_w13, w13, b.w13, hipMemcpyHostToDevice));
    PE_HIP(hipMemcpy(dst + b.off_w2, w2, b.w2, hipMemcpyHostToDevice));
    if (quant) {
      PE_HIP(hipMemcpy(dst + b.off_s13, s13, b.s13, hipMemcpyHostToDevice));
      PE_HIP(hipMemcpy(dst + b.off_s2, s2, b.s2, hipMemcpyHostToDevice));
    }
    return PE_OK;
  }
  uint8_t* dst = c->host_store + ((size_t)layer * c->d.E + expert) * b.stride;
  memcpy(dst + b.off_w13, w13, b.w13);
  memcpy(dst + b.off_w2, w2, b.w2);
  if (quant) {
    memcpy(dst + b.off_s13, s13, b.s13);
    memcpy(dst + b.off_s2, s2, b.s2);
  }
  return PE_OK;
}

int pe_reset_lru(pe_ctx* c, int layer, void* stream) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  if (layer < -1 || layer >= c->d.L) return fail(PE_ERR_INVALID_ARG, "layer %d out of range", layer);
  int rc = use_device(c);
  if (rc) return rc;
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->d.L : layer + 1;
  pe::launch_reset_lru(c->blocks, c->layer_words, l0, l1, c->o, c->d.E, c->d.K, c->unpaged,
                       static_cast<hipStream_t>(stream));
  PE_HIP(hipGetLastError());
  return PE_OK;
}

namespace {

// Poll the read-back's completion word until it holds `want`, for at most about
// 200 ms (a step's read-back normally lands within microseconds); false if it
// did not.
bool poll_flag(const uint32_t* flag, uint32_t want) {
  if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == want) return true;
  const auto t0 = std::chrono::steady_clock::now();
  for (unsigned i = 1;; ++i) {
    if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == want) return true;
    __builtin_ia32_pause();
    if ((i & 1023) == 0 && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(200)) return false;
  }
}

// Append the record of the step that just ended to the layer's plan log.
void log_step(pe_ctx* c, const int32_t* blk, int layer, int T, hipStream_t s) {
  if (!c->log_cap) return;
  pe::launch_plan_log(blk, c->o, c->d.K, (int)c->ll.n_waves, (int)c->pl.plan_words, T,
                      c->plan_log + (size_t)layer * c->log_cap * c->pl.total, c->log_cap, (int)c->pl.total,
                      c->log_seq + layer, s);
}

// One forward step of one layer (pe_forward and pe_forward_static): `act` holds
// the step's activation buffers; the stage timers record events only if `tm_on`.
int forward_impl(pe_ctx* c, int layer, const void* x, const int32_t* topk_ids, const float* topk_w, int T,
                 void* out, void* stream, const Act& act, bool tm_on) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const pe::Dims& d = c->d;
  const int n = T * d.k;
  int32_t* blk = c->blocks + (size_t)layer * c->layer_words;
  int32_t* work_l = blk + c->ll.total;
  uint8_t* slots_l = c->slots + (size_t)layer * d.K * c->b.stride;
  const uint8_t* host_l = c->unpaged ? nullptr : c->host_store_dev + (size_t)layer * d.E * c->b.stride;
  const bool device_plan = n <= d.K && !(c->cfg.flags & PE_FLAG_FORCE_HOST_PLAN);

  // An expert's entries take the MFMA kernels iff the step has at least
  // mfma_min tokens and the expert at least mfma_min entries: the choice depends
  // only on the step's size and the expert's entry count, never on K or the wave
  // split, so paged and unpaged runs share every expert's arithmetic.
  const int mfma_min = T >= c->mfma_min ? c->mfma_min : pe::kNoMfma;

  if (device_plan) {
    // One wave, on the caller's stream only (a second stream would put graph
    // branches on other hardware queues, whose cross-queue dependencies cost more
    // than they hide).  No host synchronisation: capturable.
    const int items = std::min(n, d.K);
    if (!c->unpaged && mfma_min == pe::kNoMfma && d.E <= 256) {
      // Launch A: planning + page-in workgroups (each makes the same LRU decision
      // in LDS from the current state copy; one publishes it and writes the new
      // state into the other copy) that compute the missing experts' gate/up
      // projection from the rows as they stream in, alongside the gate/up
      // projection of the experts already resident.  Launch B: every expert's
      // down projection and the fixed-order top-k sum, which also makes the new
      // state copy current.
      pe::ExpertArgs a = expert_args(c, act, layer, 0, x, topk_w, 1);
      a.lean = 1;
      a.ids = topk_ids;
      a.T = T;
      a.E = d.E;
      a.blk = blk;
      a.mfma_min = mfma_min;
      {
        StageTimer tm(c, PE_STAGE_PAGE_IN, s, tm_on);
        pe::launch_step_a(c->cfg.wtype, blk, topk_ids, n, d, c->o, mfma_min, work_l, c->stats, host_l,
                          slots_l, c->b.stride, c->b.copied, kStreamWgs, a, items, T, s);
      }
      pe::ExpertArgs all = expert_args(c, act, layer, 0, x, topk_w, 0);
      all.ids = topk_ids;
      all.T = T;
      all.E = d.E;
      {
        StageTimer tm(c, PE_STAGE_DOWN, s, tm_on);
        pe::launch_down_sum(c->cfg.wtype, all, T, static_cast<uint16_t*>(out), blk + c->ll.cur, s);
      }
      log_step(c, blk, layer, T, s);
      PE_HIP(hipGetLastError());
      return PE_OK;
    }
    // Unpaged, or experts with many entries: plan (+ plain page-in), then the
    // GEMV and MFMA expert kernels over the published lists, then the top-k sum.
    // Surplus MFMA workgroups exit on the device tile count.
    const int tiles = mfma_min != pe::kNoMfma ? pe::ceil_div(n, pe::kTileM) + items : 0;
    {
      StageTimer tm(c, PE_STAGE_PAGE_IN, s, tm_on);
      pe::launch_plan_page_in(blk, topk_ids, n, d, c->o, mfma_min, work_l, c->stats, host_l, slots_l,
                              c->b.stride, c->b.copied, !c->unpaged, kPageInGrid, s);
    }
    run_experts(c, act, tm_on, layer, 0, 0, x, topk_w, items, T, tiles, s);
    {
      StageTimer tm(c, PE_STAGE_TOPK_SUM, s, tm_on);
      pe::launch_topk_sum(act.merged, topk_ids, T, d.k, d.E, d.H, static_cast<uint16_t*>(out),
                          blk + c->ll.cur, s);
    }
    log_step(c, blk, layer, T, s);
    PE_HIP(hipGetLastError());
    return PE_OK;
  }

  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  PE_HIP(hipStreamIsCapturing(s, &cap));
  if (cap != hipStreamCaptureStatusNone)
    return fail(PE_ERR_NOT_CAPTURABLE, "T*top_k=%d > K=%d needs host planning, which cannot be captured", n, d.K);

  // Host-planned step.  One launch writes the routed ids and the layer's LRU
  // state (both state copies and the current-copy index, whoever changed them
  // last: a device-planned step, a replayed graph or a reset) into page-locked
  // host memory; that is the one synchronisation.  The host plans every wave in
  // its mirror of the block, one launch reads the block (state, plans, slot map)
  // and the work lists back into device memory, and the waves run in order.
  int32_t* mirror = c->st_blk + (size_t)layer * c->layer_words;
  int32_t* mirror_dev = c->st_blk_dev + (size_t)layer * c->layer_words;
  if (++c->gather_seq == 0) c->gather_seq = 1;     // 0 is the word's initial value
  const uint32_t want = c->gather_seq;
  pe::launch_gather_state(blk, (int)c->ll.state_prefix, topk_ids, n, mirror_dev, c->st_ids_dev, c->st_flag_dev,
                          want, s);
  PE_HIP(hipGetLastError());
  if (!poll_flag(c->st_flag, want)) {
    // not seen within the polling budget: wait for the stream the ordinary way
    PE_HIP(hipStreamSynchronize(s));
    if (__atomic_load_n(c->st_flag, __ATOMIC_ACQUIRE) != want)
      return fail(PE_ERR_HIP, "the routed ids and LRU state were not read back (step %u)", want);
  }
  pe::HostPlanSummary& sm = *c->sum;
  pe::Dims dp = d;
  dp.mfma_min = mfma_min;
  if (pe::host_plan_step(dp, c->ll, c->wl, c->st_ids, n, mirror, mirror + c->ll.total, &sm) != 0)
    return fail(PE_ERR_INVALID_ARG, "step needs more waves than the context holds");
  // The plan (the block with state, plans and slot map, and the work lists that
  // follow it) goes to device memory in one copy.  When the first wave is a
  // streamed GEMV wave, that wave's launch makes the copy with one extra
  // workgroup and reads its own work lists from the host's copy: one launch
  // fewer between the host's plan and the GPU's work.
  const bool dma = (c->cfg.flags & PE_FLAG_PAGEIN_DMA) != 0;
  const size_t up_bytes = align_up((c->ll.total + c->wl.entries + (size_t)n) * 4, 16);
  const bool fold = sm.n_waves > 0 && !c->unpaged && !dma && sm.tiles[0] == 0;
  if (!fold) {
    const int grid = (int)std::min<size_t>(16, std::max<size_t>(1, up_bytes / 8192));
    pe::launch_copy(blk, mirror_dev, up_bytes, grid, s);
  }
  bool summed = false;     // the top-k sum already ran with the last down projection
  WaveRanges wr{0, 0, 0, 0, 0, 0};
  for (int w = 0; w < sm.n_waves; ++w) {
    const int cnt = mirror[c->ll.plan_count + w];
    const int g_all = sm.gemv_items[w], g_hit = sm.gemv_hits[w];
    const int t_all = sm.tiles[w], t_hit = sm.tile_hits[w];
    wr.g0 = wr.g1; wr.gsplit = wr.g0 + g_hit; wr.g1 = wr.g0 + g_all;
    wr.t0 = wr.t1; wr.tsplit = wr.t0 + t_hit; wr.t1 = wr.t0 + t_all;
    if (!c->unpaged && !dma && t_all == 0) {
      // GEMV experts only: one launch pages in the missing experts with their
      // gate/up projection fused in while the resident ones run theirs, then
      // one launch runs the wave's down projection.
      pe::ExpertArgs a = expert_args(c, act, layer, w, x, topk_w, 1);
      set_ranges(a, wr);
      const bool up = fold && w == 0;
      if (up) a.work = mirror_dev + c->ll.total;
      {
        StageTimer tm(c, PE_STAGE_PAGE_IN, s, tm_on);
        pe::launch_wave_a(c->cfg.wtype, a, g_hit, sm.max_gemv_tokens, kStreamWgs, host_l, c->b.stride,
                          c->b.copied, up ? mirror_dev : nullptr, up ? blk : nullptr, up ? up_bytes : 0, s);
      }
      a = expert_args(c, act, layer, w, x, topk_w, 0);     // device work lists from here on
      set_ranges(a, wr);
      StageTimer tm(c, PE_STAGE_DOWN, s, tm_on);
      if (sm.n_waves == 1 && mfma_min == pe::kNoMfma && down_sum_fits(n)) {
        // one wave of few tokens: its down projection and the top-k sum in one
        // launch, as in a device-planned step (the same arithmetic as the
        // down kernel followed by the sum over the merged buffer)
        a.ids = topk_ids;
        a.T = T;
        a.E = d.E;
        pe::launch_down_sum(c->cfg.wtype, a, sm.max_gemv_tokens, static_cast<uint16_t*>(out), nullptr, s);
        summed = true;
      } else {
        pe::launch_gemv_down(c->cfg.wtype, a, g_all, sm.max_gemv_tokens, s);
      }
      continue;
    }
    const bool fork = !c->unpaged && cnt > 0 && (g_hit > 0 || t_hit > 0);
    if (fork) {
      PE_HIP(hipEventRecord(c->ev_fork, s));
      PE_HIP(hipStreamWaitEvent(c->side, c->ev_fork, 0));
      run_experts(c, act, tm_on, layer, w, 1, x, topk_w, g_hit, sm.max_gemv_tokens, t_hit, c->side, &wr);
      PE_HIP(hipEventRecord(c->ev_join, c->side));
    }
    if (!c->unpaged && cnt > 0) {
      StageTimer tm(c, PE_STAGE_PAGE_IN, s, tm_on);
      if (dma) {
        const int32_t* pe_ = mirror + c->ll.plan_expert + (size_t)w * d.K;
        const int32_t* ps_ = mirror + c->ll.plan_slot + (size_t)w * d.K;
        for (int r = 0; r < cnt; ++r)
          PE_HIP(hipMemcpyAsync(slots_l + (size_t)ps_[r] * c->b.stride,
                                c->host_store + ((size_t)layer * d.E + pe_[r]) * c->b.stride, c->b.copied,
                                hipMemcpyHostToDevice, s));
      } else {
        pe::launch_page_in(blk, c->o, w, d.K, host_l, slots_l, c->b.stride, c->b.copied, kPageInGrid, s);
      }
    }
    if (fork) {
      run_experts(c, act, tm_on, layer, w, 2, x, topk_w, g_all - g_hit, sm.max_gemv_tokens, t_all - t_hit, s, &wr);
      PE_HIP(hipStreamWaitEvent(s, c->ev_join, 0));    // before the next wave may evict these slots
    } else {
      run_experts(c, act, tm_on, layer, w, 0, x, topk_w, g_all, sm.max_gemv_tokens, t_all, s, &wr);
    }
  }
  if (!summed) {
    StageTimer tm(c, PE_STAGE_TOPK_SUM, s, tm_on);
    pe::launch_topk_sum(act.merged, topk_ids, T, d.k, d.E, d.H, static_cast<uint16_t*>(out), nullptr, s);
  }
  log_step(c, blk, layer, T, s);
  PE_HIP(hipGetLastError());
  c->host_counts[pe::ST_STEPS] += 1;
  c->host_counts[pe::ST_HOST_PLANNED] += 1;
  c->host_counts[pe::ST_WAVES] += sm.n_waves;
  c->host_counts[pe::ST_PAGE_INS] += sm.page_ins;
  c->host_counts[pe::ST_DISTINCT] += sm.distinct;
  c->host_counts[pe::ST_ENTRIES] += sm.valid_entries;
  c->host_counts[pe::ST_BAD_IDS] += sm.bad_ids;
  return PE_OK;
}

// Argument checks shared by pe_forward and pe_forward_static; 1 if T = 0 (no-op).
int check_forward(pe_ctx* c, int layer, const void* x, const int32_t* topk_ids, const float* topk_w, int T,
                  void* out) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  if (layer < 0 || layer >= c->d.L) return fail(PE_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (T < 0 || T > c->d.max_tokens) return fail(PE_ERR_INVALID_ARG, "T=%d outside [0, %d]", T, c->d.max_tokens);
  if (T == 0) return 1;
  if (!x || !topk_ids || !topk_w || !out) return fail(PE_ERR_INVALID_ARG, "NULL tensor pointer");
  return use_device(c);
}

}  // namespace

int pe_forward(pe_ctx* c, int layer, const void* x, const int32_t* topk_ids, const float* topk_w, int T,
               void* out, void* stream) {
  const int rc = check_forward(c, layer, x, topk_ids, topk_w, T, out);
  if (rc) return rc < 0 ? rc : PE_OK;
  return forward_impl(c, layer, x, topk_ids, topk_w, T, out, stream, Act{c->h, c->merged}, true);
}

int pe_forward_static(pe_ctx* c, int layer, const void* x, const int32_t* topk_ids, const float* topk_w, int T,
                      void* out, void* stream) {
  const int rc = check_forward(c, layer, x, topk_ids, topk_w, T, out);
  if (rc) return rc < 0 ? rc : PE_OK;
  // h [n][I] bf16, then the merged buffer [n][H] fp32, 256-byte aligned
  const size_t n = (size_t)T * c->d.k;
  const size_t h_bytes = align_up(n * c->d.I * 2, 256);
  const size_t need = h_bytes + n * c->d.H * 4;
  if (need > pe::kStaticScratchBytes)
    return fail(PE_ERR_INVALID_ARG,
                "pe_forward_static: %zu entries need %zu bytes of scratch, more than the fixed %zu "
                "(%zu entries fit at this hidden and inter size)",
                n, need, pe::kStaticScratchBytes,
                (size_t)((pe::kStaticScratchBytes - 256) / (2 * (size_t)c->d.I + 4 * (size_t)c->d.H)));
  char* base = static_cast<char*>(pe::static_scratch(c->cfg.device));
  if (!base) return fail(PE_ERR_HIP, "the fixed scratch area has no address on device %d", c->cfg.device);
  const Act act{reinterpret_cast<uint16_t*>(base), reinterpret_cast<float*>(base + h_bytes)};
  return forward_impl(c, layer, x, topk_ids, topk_w, T, out, stream, act, false);
}

int pe_max_captured_batch(const pe_ctx* c) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  return c->d.K / c->d.k;
}

int pe_max_waves(const pe_ctx* c) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  return c->d.max_waves;
}

int pe_get_lru_state(pe_ctx* c, int layer, int32_t* slot_expert, uint32_t* last_use, uint32_t* tick,
                     void* stream) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  if (layer < 0 || layer >= c->d.L) return fail(PE_ERR_INVALID_ARG, "layer %d out of range", layer);
  int rc = use_device(c);
  if (rc) return rc;
  PE_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  std::vector<int32_t> blk(c->ll.state_prefix);
  PE_HIP(hipMemcpy(blk.data(), c->blocks + (size_t)layer * c->layer_words, blk.size() * 4, hipMemcpyDeviceToHost));
  const int32_t* st = blk.data() + c->ll.state(blk[c->ll.cur] & 1);
  if (slot_expert) memcpy(slot_expert, st + c->ll.slot_expert, (size_t)c->d.K * 4);
  if (last_use) memcpy(last_use, st + c->ll.last_use, (size_t)c->d.K * 4);
  if (tick) *tick = (uint32_t)st[c->ll.tick];
  return PE_OK;
}

int pe_get_plan(pe_ctx* c, int layer, int wave, int32_t* count, int32_t* experts, int32_t* slots,
                int32_t* evicted, int32_t* n_waves, void* stream) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  if (layer < 0 || layer >= c->d.L || wave < 0 || wave >= c->d.max_waves)
    return fail(PE_ERR_INVALID_ARG, "layer %d / wave %d out of range", layer, wave);
  int rc = use_device(c);
  if (rc) return rc;
  PE_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  std::vector<int32_t> blk(c->ll.slot_of);
  PE_HIP(hipMemcpy(blk.data(), c->blocks + (size_t)layer * c->layer_words, blk.size() * 4, hipMemcpyDeviceToHost));
  const int K = c->d.K;
  if (count) *count = blk[c->ll.plan_count + wave];
  if (experts) memcpy(experts, blk.data() + c->ll.plan_expert + (size_t)wave * K, (size_t)K * 4);
  if (slots) memcpy(slots, blk.data() + c->ll.plan_slot + (size_t)wave * K, (size_t)K * 4);
  if (evicted) memcpy(evicted, blk.data() + c->ll.plan_evicted + (size_t)wave * K, (size_t)K * 4);
  if (n_waves) *n_waves = blk[c->ll.n_waves];
  return PE_OK;
}

int pe_get_slot_map(pe_ctx* c, int layer, int32_t* slot_of, int T, void* stream) {
  if (!c || !slot_of) return fail(PE_ERR_INVALID_ARG, "NULL argument");
  if (layer < 0 || layer >= c->d.L || T < 0 || T > c->d.max_tokens)
    return fail(PE_ERR_INVALID_ARG, "layer %d / T %d out of range", layer, T);
  int rc = use_device(c);
  if (rc) return rc;
  PE_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  PE_HIP(hipMemcpy(slot_of, c->blocks + (size_t)layer * c->layer_words + c->ll.slot_of, (size_t)T * c->d.k * 4,
                   hipMemcpyDeviceToHost));
  return PE_OK;
}

int pe_plan_log_record_words(const pe_ctx* c) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  return (int)c->pl.total;
}

int pe_get_plan_log(pe_ctx* c, int layer, int32_t* records, int max_records, int* n_records, void* stream) {
  if (!c || !records || !n_records) return fail(PE_ERR_INVALID_ARG, "NULL argument");
  if (!c->log_cap) return fail(PE_ERR_INVALID_ARG, "the context keeps no plan log (create it with PE_FLAG_PLAN_LOG)");
  if (layer < 0 || layer >= c->d.L || max_records < 0)
    return fail(PE_ERR_INVALID_ARG, "layer %d / max_records %d out of range", layer, max_records);
  int rc = use_device(c);
  if (rc) return rc;
  PE_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  uint32_t seq = 0;
  PE_HIP(hipMemcpy(&seq, c->log_seq + layer, 4, hipMemcpyDeviceToHost));
  const uint32_t cap = (uint32_t)c->log_cap;
  const uint32_t n = std::min(std::min(seq, cap), (uint32_t)max_records);
  const size_t rw = c->pl.total;
  const int32_t* ring = c->plan_log + (size_t)layer * cap * rw;
  // records seq - n .. seq - 1 sit at ring positions (seq - n + i) % cap: at most two runs
  uint32_t done = 0;
  while (done < n) {
    const uint32_t pos = (seq - n + done) % cap;
    const uint32_t run = std::min(n - done, cap - pos);
    PE_HIP(hipMemcpy(records + (size_t)done * rw, ring + (size_t)pos * rw, (size_t)run * rw * 4,
                     hipMemcpyDeviceToHost));
    done += run;
  }
  *n_records = (int)n;
  return PE_OK;
}

int pe_get_stats(pe_ctx* c, pe_stats* out) {
  if (!c || !out) return fail(PE_ERR_INVALID_ARG, "NULL argument");
  int rc = use_device(c);
  if (rc) return rc;
  unsigned long long dv[pe::ST_COUNT];
  PE_HIP(hipDeviceSynchronize());
  PE_HIP(hipMemcpy(dv, c->stats, sizeof dv, hipMemcpyDeviceToHost));
  unsigned long long t[pe::ST_COUNT];
  for (int i = 0; i < pe::ST_COUNT; ++i) t[i] = dv[i] + c->host_counts[i];
  out->steps = t[pe::ST_STEPS];
  out->device_planned = t[pe::ST_DEVICE_PLANNED];
  out->host_planned = t[pe::ST_HOST_PLANNED];
  out->waves = t[pe::ST_WAVES];
  out->page_ins = c->unpaged ? 0 : t[pe::ST_PAGE_INS];
  out->page_in_bytes = out->page_ins * c->b.copied;
  out->distinct = t[pe::ST_DISTINCT];
  out->entries = t[pe::ST_ENTRIES];
  out->bad_ids = t[pe::ST_BAD_IDS];
  return PE_OK;
}

int pe_reset_stats(pe_ctx* c) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  int rc = use_device(c);
  if (rc) return rc;
  PE_HIP(hipDeviceSynchronize());
  PE_HIP(hipMemset(c->stats, 0, pe::ST_COUNT * 8));
  for (auto& v : c->host_counts) v = 0;
  return PE_OK;
}

int pe_link_probe(pe_ctx* c, size_t bytes, int use_kernel, int reps, double* gbps, void* stream) {
  if (!c || !gbps || bytes < 16 || bytes % 16 || reps < 1) return fail(PE_ERR_INVALID_ARG, "bad probe arguments");
  int rc = use_device(c);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* hbuf = nullptr;
  void* dbuf = nullptr;
  if (hipHostMalloc(&hbuf, bytes, hipHostMallocMapped) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PE_ERR_OOM_HOST_PIN, "probe: cannot pin %zu bytes", bytes);
  }
  memset(hbuf, 0x5A, bytes);
  if (hipMalloc(&dbuf, bytes) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipHostFree(hbuf);
    return fail(PE_ERR_OOM_DEVICE, "probe: cannot allocate %zu device bytes", bytes);
  }
  void* hdev = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int status = PE_OK;
  double best = 0.0;
  do {
    if (hipHostGetDevicePointer(&hdev, hbuf, 0) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
        hipEventCreate(&e1) != hipSuccess) {
      status = fail(PE_ERR_HIP, "probe: HIP setup failed");
      break;
    }
    for (int r = 0; r <= reps && status == PE_OK; ++r) {   // r == 0 warms up
      if (hipEventRecord(e0, s) != hipSuccess) { status = fail(PE_ERR_HIP, "probe: event record"); break; }
      if (use_kernel) pe::launch_copy(dbuf, hdev, bytes, kPageInGrid, s);
      else if (hipMemcpyAsync(dbuf, hbuf, bytes, hipMemcpyHostToDevice, s) != hipSuccess) {
        status = fail(PE_ERR_HIP, "probe: hipMemcpyAsync");
        break;
      }
      float ms = 0.f;
      if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
        status = fail(PE_ERR_HIP, "probe: timing failed: %s", hipGetErrorString(hipGetLastError()));
        break;
      }
      if (r > 0 && ms > 0.f) best = std::max(best, bytes / (ms * 1e-3) / 1e9);
    }
  } while (false);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(dbuf);
  (void)hipHostFree(hbuf);
  if (status == PE_OK) *gbps = best;
  return status;
}

int pe_set_timing(pe_ctx* c, int enable) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  int rc = use_device(c);
  if (rc) return rc;
  rc = drain_timing(c, true);
  if (rc) return rc;
  c->timing = enable != 0;
  for (int i = 0; i < PE_NUM_STAGES; ++i) { c->stage_ms[i] = 0.0; c->stage_n[i] = 0; }
  return PE_OK;
}

int pe_get_timing(pe_ctx* c, uint64_t* launches, double* total_ms) {
  if (!c) return fail(PE_ERR_INVALID_ARG, "ctx is NULL");
  int rc = use_device(c);
  if (rc) return rc;
  rc = drain_timing(c, true);
  if (rc) return rc;
  for (int i = 0; i < PE_NUM_STAGES; ++i) {
    if (launches) launches[i] = c->stage_n[i];
    if (total_ms) total_ms[i] = c->stage_ms[i];
  }
  return PE_OK;
}

int pe_plan_host(int num_experts, int num_resident, int top_k, int T, const int32_t* topk_ids,
                 int32_t* slot_expert, uint32_t* last_use, uint32_t* tick, int max_waves, int32_t* n_waves,
                 int32_t* counts, int32_t* experts, int32_t* slots, int32_t* evicted, int32_t* slot_of) {
  if (num_experts < 1 || num_experts > pe::kMaxExperts || top_k < 1 || num_resident < top_k ||
      num_resident > num_experts || T < 1 || max_waves < 1)
    return fail(PE_ERR_INVALID_ARG, "bad planner dimensions");
  if (!topk_ids || !slot_expert || !last_use || !tick || !n_waves || !counts || !experts || !slots || !evicted ||
      !slot_of)
    return fail(PE_ERR_INVALID_ARG, "NULL argument");
  pe::Dims d = pe::make_dims(1, num_experts, num_resident, top_k, 8, 8, T);
  d.max_waves = max_waves;
  const pe::LayerLayout ll = pe::make_layer_layout(d);
  const pe::WorkLayout wl = pe::make_work_layout(d);
  std::vector<int32_t> blk(ll.total, 0), work(wl.total, 0);
  const int K = num_resident, E = num_experts;
  blk[ll.cur] = 0;
  int32_t* st = blk.data() + ll.state(0);
  st[ll.tick] = (int32_t)*tick;
  for (int e = 0; e < E; ++e) st[ll.expert_slot + e] = -1;
  for (int j = 0; j < K; ++j) {
    const int e = slot_expert[j];
    if (e >= E) return fail(PE_ERR_INVALID_ARG, "slot_expert[%d] = %d out of range", j, e);
    st[ll.slot_expert + j] = e;
    st[ll.last_use + j] = (int32_t)last_use[j];
    if (e >= 0) {
      if (st[ll.expert_slot + e] >= 0) return fail(PE_ERR_INVALID_ARG, "expert %d in two slots", e);
      st[ll.expert_slot + e] = j;
    }
  }
  pe::HostPlanSummary* sm = new pe::HostPlanSummary;
  const int rc = pe::host_plan_step(d, ll, wl, topk_ids, T * top_k, blk.data(), work.data(), sm);
  delete sm;
  if (rc != 0) return fail(PE_ERR_INVALID_ARG, "step needs more than %d waves", max_waves);
  for (int j = 0; j < K; ++j) {
    slot_expert[j] = st[ll.slot_expert + j];
    last_use[j] = (uint32_t)st[ll.last_use + j];
  }
  *tick = (uint32_t)st[ll.tick];
  *n_waves = blk[ll.n_waves];
  for (int w = 0; w < max_waves; ++w) counts[w] = w < *n_waves ? blk[ll.plan_count + w] : 0;
  memcpy(experts, blk.data() + ll.plan_expert, (size_t)max_waves * K * 4);
  memcpy(slots, blk.data() + ll.plan_slot, (size_t)max_waves * K * 4);
  memcpy(evicted, blk.data() + ll.plan_evicted, (size_t)max_waves * K * 4);
  memcpy(slot_of, blk.data() + ll.slot_of, (size_t)T * top_k * 4);
  return PE_OK;
}

}  // extern "C"
