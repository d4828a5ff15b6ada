// C ABI of libmoe: model and pool handles, weight upload, the decode and
// stack entry points, and the pool's miss path (pinned host blob ->
// hipMemcpyAsync on a side stream -> HBM slot).
//
// Pages: routed experts streamed on demand into a bounded slot pool with LFU +
// recency eviction while the dense core (router, shared experts) stays
// resident (cheshm.ai news article, paragraph on how it works; paotong.dev
// commentary, paragraphs on the resident set and the bounded pool); a miss
// reads the expert's record with one call at base + index * stride
// (paotong.dev, paragraph on the fetch path; alphalab.site field test,
// section on SSD reads). Here the blob is pinned host memory and the read is
// a host-to-device copy into the victim slot.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "blob_file.h"
#include "common.h"
#include "kernels.h"
#include "launch.h"
#include "pool_policy.h"
#include "prefill.h"
#include "scalar.h"

using namespace moe;

namespace {

constexpr uint64_t kModelMagic = 0x4d4f454d4f44454cull;  // "MOEMODEL"
constexpr uint64_t kPoolMagic = 0x4d4f45504f4f4c21ull;

std::mutex g_live_mu;
std::set<const void*> g_live;

void live_add(const void* p) {
  std::lock_guard<std::mutex> g(g_live_mu);
  g_live.insert(p);
}
void live_del(const void* p) {
  std::lock_guard<std::mutex> g(g_live_mu);
  g_live.erase(p);
}
bool live_has(const void* p) {
  std::lock_guard<std::mutex> g(g_live_mu);
  return g_live.count(p) != 0;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                 \
  do {                                      \
    hipError_t e_ = (expr);                 \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// Optional per-launch timing: a hipEvent pair around every kernel launch.
}  // namespace

LaunchEvents& moe::launch_events() {
  thread_local LaunchEvents ev{nullptr, nullptr};
  return ev;
}

namespace {

enum KernelKind {
  K_ROUTER, K_ROUTE, K_GATEUP, K_DOWN, K_EXPERT, K_REDUCE,
  K_PF_XPREP, K_PF_ROUTER, K_PF_ROUTE, K_PF_COUNT, K_PF_SCAN, K_PF_SCATTER, K_PF_GATEUP, K_PF_DOWN, K_PF_COMBINE,
  K_EXPERT_MISS,
  K_COUNT
};
const char* const kKindName[K_COUNT] = {"router",         "route",          "gateup",         "down",
                                        "expert",         "reduce",
                                        "prefill_xprep",  "prefill_router", "prefill_route",  "prefill_count",
                                        "prefill_scan",   "prefill_scatter", "prefill_gateup", "prefill_down",
                                        "prefill_combine", "expert_miss"};

struct Profiler {
  bool on = false;
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> spare;
  uint64_t launches[K_COUNT] = {};
  double ms[K_COUNT] = {};

  hipEvent_t get() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  hipError_t harvest() {
    for (auto& r : pending) {
      hipError_t e = hipEventSynchronize(r.b);
      if (e != hipSuccess) return e;
      float t = 0.f;
      e = hipEventElapsedTime(&t, r.a, r.b);
      if (e != hipSuccess) return e;
      launches[r.kind] += 1;
      ms[r.kind] += t;
      spare.push_back(r.a);
      spare.push_back(r.b);
    }
    pending.clear();
    return hipSuccess;
  }
  // Launch `fn` (returning hipError_t) bracketed by events when profiling.
  template <class F>
  hipError_t run(int kind, hipStream_t s, F&& fn) {
    if (!on) return fn();
    if (pending.size() >= 4096) {
      hipError_t e = harvest();
      if (e != hipSuccess) return e;
    }
    Rec r{kind, get(), get()};
    if (!r.a || !r.b) return hipErrorOutOfMemory;
    // fn launches exactly one kernel; that launch takes the kernel's own
    // begin/end timestamps into the pair (see launch.h).
    launch_events() = LaunchEvents{r.a, r.b};
    const hipError_t e = fn();
    const bool consumed = launch_events().start == nullptr;
    launch_events() = LaunchEvents{};
    if (e != hipSuccess || !consumed) {
      spare.push_back(r.a);
      spare.push_back(r.b);
      return e;
    }
    pending.push_back(r);
    return hipSuccess;
  }
  void release() {
    harvest();
    for (auto e : spare) hipEventDestroy(e);
    spare.clear();
  }
};

}  // namespace

struct moe_model {
  uint64_t magic = kModelMagic;
  moe_config cfg{};
  int32_t storage = MOE_STORE_DEVICE;
  int device = 0;
  Geometry geo{};
  size_t rec_bytes = 0, stride = 0, shared_stride = 0;
  uint8_t* experts = nullptr;       // device (STORE_DEVICE) or pinned host (STORE_HOST); NULL for STORE_FILE
  size_t experts_bytes = 0;         // L * E * stride: the store, or the file's blob region
  BlobFile file;                    // STORE_FILE: the blob file
  uint8_t* shared = nullptr;        // device [L] records
  float* wr_rows = nullptr;         // device [L][E+1][H]
  uint16_t* wr_split = nullptr;     // device [L][3][E+1][H] bf16: wr_rows = hi + mid + lo exactly
  float* bias = nullptr;            // device [L][E]
  float* logits = nullptr;          // device [E+1]
  float* h = nullptr;               // device [(k+1)][I]
  float* h_scalar = nullptr;        // device [(k+1)][I]: h of the scalar expert kernels
  int32_t kernels = MOE_KERNELS_FAST;
  float* rbuf = nullptr;            // device [H]
  uint16_t* xbuf = nullptr;         // device [2][H]
  int32_t* route_idx = nullptr;     // device [route_cap][k]
  float* route_w = nullptr;         // device [route_cap][k]
  float* route_gamma = nullptr;     // device [route_cap]
  size_t route_cap = 0;             // steps
  size_t route_steps = 0;           // steps recorded by the last call
  std::vector<uint8_t> layer_set;
  void* prefill = nullptr;          // prefill workspace (prefill.hip)
  Profiler prof;
  // captured decode sequences, replayed with hipGraphLaunch (kernel arguments
  // are baked in, so an entry is keyed by every pointer and size it used)
  struct GraphEntry {
    int kind, layer, n;
    const void* x;
    void* out;
    hipGraphExec_t exec;
    hipEvent_t done;  // recorded after the entry's latest launch
    uint64_t stamp;
  };
  std::vector<GraphEntry> graphs;
  hipStream_t cap_stream = nullptr;
  uint64_t graph_clock = 0;
};

struct moe_pool {
  uint64_t magic = kPoolMagic;
  moe_model* model = nullptr;
  int64_t n_slots = 0;
  uint8_t* arena = nullptr;         // device [n_slots][stride]
  PoolTable table{1};
  // Misses are spread round-robin over several copy streams (default
  // priority) so that their host->device transfers run side by side.
  static constexpr int kCopyStreams = 4;
  hipStream_t copy_stream[kCopyStreams] = {};
  hipEvent_t copies_done[kCopyStreams] = {};
  hipEvent_t route_ready = nullptr;
  int32_t* host_route = nullptr;    // pinned, mapped [k]
  int32_t* host_route_dev = nullptr;
  // storage-backed misses (STORE_FILE): pinned staging buffers, one per miss
  // of a step (k of them, stride bytes each), filled by pread on the read
  // workers, then copied to the slot like a host-blob miss
  uint8_t* staging = nullptr;
  uint8_t* bounce = nullptr;        // direct I/O: k ordinary 4096-aligned buffers the reads land in first
  ReadWorkers* readers = nullptr;
  uint64_t storage_reads = 0, storage_bytes = 0;
};

namespace {

moe_status check_model(moe_model* m, const char* fn) {
  if (!m) return fail(MOE_EINVAL, std::string(fn) + ": model is NULL");
  if (!live_has(m) || m->magic != kModelMagic) return fail(MOE_ESTATE, std::string(fn) + ": not a live model handle");
  return MOE_OK;
}

moe_status check_pool(const moe_pool* p, const char* fn) {
  if (!p) return fail(MOE_EINVAL, std::string(fn) + ": pool is NULL");
  if (!live_has(p) || p->magic != kPoolMagic) return fail(MOE_ESTATE, std::string(fn) + ": not a live pool handle");
  return MOE_OK;
}

// Every graph may still be executing: callers synchronise the device first.
void drop_graphs(moe_model* m) {
  for (auto& g : m->graphs) {
    hipGraphExecDestroy(g.exec);
    hipEventDestroy(g.done);
  }
  m->graphs.clear();
}

moe_status ensure_route_cap(moe_model* m, size_t steps) {
  if (steps <= m->route_cap) return MOE_OK;
  size_t cap = std::max<size_t>(steps, 2 * m->route_cap);
  HIP_TRY(hipDeviceSynchronize(), "route log resize");
  drop_graphs(m);  // captured kernels point at the old buffers
  hipFree(m->route_idx);
  hipFree(m->route_w);
  hipFree(m->route_gamma);
  m->route_idx = nullptr;
  m->route_w = nullptr;
  m->route_gamma = nullptr;
  m->route_cap = 0;
  const size_t k = (size_t)m->cfg.top_k;
  if (hipMalloc(&m->route_idx, cap * k * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&m->route_w, cap * k * sizeof(float)) != hipSuccess ||
      hipMalloc(&m->route_gamma, cap * sizeof(float)) != hipSuccess)
    return fail(MOE_ENOMEM, "route log allocation failed");
  m->route_cap = cap;
  return MOE_OK;
}

StepBuffers step_buffers(moe_model* m, const uint16_t* x, size_t step) {
  StepBuffers b;
  b.x = x;
  b.logits = m->logits;
  b.route_idx = m->route_idx + step * (size_t)m->cfg.top_k;
  b.route_w = m->route_w + step * (size_t)m->cfg.top_k;
  b.route_gamma = m->route_gamma + step;
  b.h = m->h;
  b.partial = m->h;  // the fused path's partial rows share the buffer
  return b;
}

ExpertSource resident_source(moe_model* m, int layer) {
  ExpertSource s{};
  s.base = m->experts;
  s.stride = m->stride;
  s.gid_base = (int64_t)layer * m->cfg.n_experts;
  s.use_table = 0;
  return s;
}

const float* layer_wr(moe_model* m, int layer) {
  return m->wr_rows + (size_t)layer * (m->cfg.n_experts + 1) * m->cfg.hidden;
}
const uint16_t* layer_wr_split(moe_model* m, int layer) {
  return m->wr_split + (size_t)layer * 3 * (m->cfg.n_experts + 1) * m->cfg.hidden;
}

// bf16 bits of v rounded to nearest, ties to even (finite v).
uint16_t bf16_rne_bits(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float v;
  std::memcpy(&v, &u, 4);
  return v;
}
const float* layer_bias(moe_model* m, int layer) { return m->bias + (size_t)layer * m->cfg.n_experts; }
const uint8_t* layer_shared(moe_model* m, int layer) { return m->shared + (size_t)layer * m->shared_stride; }

// The expert kernels of one token-layer (after routing): fused expert +
// reduce where the shape allows, else gate/up + down; with the scalar kernels
// selected, their plainly written equivalent + reduce.
moe_status expert_steps(moe_model* m, int layer, const StepBuffers& b, const ExpertSource& src,
                        const ResidualArgs& r, hipStream_t s) {
  if (m->kernels == MOE_KERNELS_SCALAR) {
    // three launches, so outside the per-launch profiler
    if (!fused_expert_supported(m->geo))
      return fail(MOE_EINVAL, "scalar decode kernels need hidden <= 2048 (the fused path's shapes)");
    HIP_TRY(launch_expert_scalar(m->geo, m->experts, m->stride, src.gid_base, layer_shared(m, layer), b, m->h_scalar,
                                 s),
            "scalar expert launch");
    HIP_TRY(m->prof.run(K_REDUCE, s, [&] { return launch_reduce(m->geo, b, r, s); }), "reduce launch");
    return MOE_OK;
  }
  if (fused_expert_supported(m->geo)) {
    HIP_TRY(m->prof.run(K_EXPERT, s, [&] { return launch_expert(m->geo, src, layer_shared(m, layer), b, s); }),
            "expert launch");
    HIP_TRY(m->prof.run(K_REDUCE, s, [&] { return launch_reduce(m->geo, b, r, s); }), "reduce launch");
    return MOE_OK;
  }
  HIP_TRY(m->prof.run(K_GATEUP, s, [&] { return launch_gateup(m->geo, src, layer_shared(m, layer), b, s); }),
          "gate/up launch");
  HIP_TRY(m->prof.run(K_DOWN, s, [&] { return launch_down(m->geo, src, layer_shared(m, layer), b, r, s); }),
          "down launch");
  return MOE_OK;
}

// One token through one layer on the decode kernels.
moe_status decode_step(moe_model* m, int layer, const StepBuffers& b, const ExpertSource& src,
                       const ResidualArgs& r, hipStream_t s) {
  HIP_TRY(m->prof.run(K_ROUTER, s, [&] { return launch_router(m->geo, layer_wr(m, layer), layer_bias(m, layer), b, s); }),
          "router launch");
  return expert_steps(m, layer, b, src, r, s);
}

moe_status check_forward_args(moe_model* m, int32_t layer, const void* x, int32_t n_tok, const void* out,
                              const char* fn) {
  moe_status st = check_model(m, fn);
  if (st) return st;
  if (layer < 0 || layer >= m->cfg.n_layers) return fail(MOE_EINVAL, std::string(fn) + ": layer out of range");
  if (n_tok < 0 || n_tok > 65536) return fail(MOE_EINVAL, std::string(fn) + ": n_tok must be in [0, 65536]");
  if (n_tok > 0 && (!x || !out)) return fail(MOE_EINVAL, std::string(fn) + ": NULL pointer");
  if (m->storage != MOE_STORE_DEVICE)
    return fail(MOE_ESTATE, std::string(fn) + ": experts are in host or file storage; use moe_stack_decode with a pool");
  if (n_tok > 0 && !m->layer_set[(size_t)layer])
    return fail(MOE_ESTATE, std::string(fn) + ": moe_model_set_layer was not called for this layer");
  return MOE_OK;
}

// Token sequences at least this long are captured once into a HIP graph and
// replayed (host launch work drops out of the per-token chain).
constexpr int kGraphMinTokens = 64;
constexpr size_t kGraphCacheSize = 8;

template <class F>
moe_status run_graph(moe_model* m, int kind, int layer, const void* x, void* out, int n, hipStream_t user,
                     F&& enqueue) {
  moe_model::GraphEntry* hit = nullptr;
  for (auto& g : m->graphs)
    if (g.kind == kind && g.layer == layer && g.n == n && g.x == x && g.out == out) hit = &g;
  if (!hit) {
    if (!m->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking), "capture stream");
    HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal), "graph capture begin");
    moe_status st = enqueue(m->cap_stream);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(m->cap_stream, &graph);
    if (st) {
      if (graph) hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return hip_fail(e, "graph capture end");
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "graph instantiate");
    hipEvent_t done = nullptr;
    e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
    if (e != hipSuccess) {
      hipGraphExecDestroy(exec);
      return hip_fail(e, "graph event");
    }
    if (m->graphs.size() >= kGraphCacheSize) {
      auto lru = std::min_element(m->graphs.begin(), m->graphs.end(),
                                  [](const moe_model::GraphEntry& a, const moe_model::GraphEntry& b) {
                                    return a.stamp < b.stamp;
                                  });
      // the evicted graph's last launch may still be running on some stream
      e = hipEventSynchronize(lru->done);
      hipGraphExecDestroy(lru->exec);
      hipEventDestroy(lru->done);
      m->graphs.erase(lru);
      if (e != hipSuccess) {
        hipGraphExecDestroy(exec);
        hipEventDestroy(done);
        return hip_fail(e, "graph eviction wait");
      }
    }
    m->graphs.push_back({kind, layer, n, x, out, exec, done, 0});
    hit = &m->graphs.back();
  }
  hit->stamp = ++m->graph_clock;
  HIP_TRY(hipGraphLaunch(hit->exec, user), "graph launch");
  HIP_TRY(hipEventRecord(hit->done, user), "graph event record");
  return MOE_OK;
}

// ------------------------------------------------------------ no-alloc path ---
// Scratch of moe_layer_forward_noalloc: one file-scope device array, of which
// every GPU the library runs on holds its own copy until the process ends.
// Host code never uses the array's name as an address: the device address
// of each GPU's copy comes from hipGetSymbolAddress with that GPU current.
constexpr size_t kNoAllocScratchBytes = 64ull << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of the scratch array (looked up
// once per device), or NULL with the error set.
moe_status scratch_on_current_device(uint8_t** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "moe_layer_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: device index out of range");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "moe_layer_forward_noalloc: hipGetSymbolAddress");
    if (!p) return fail(MOE_EHIP, "moe_layer_forward_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Misses of one step from the blob file: one pread per missing record into
// its pinned staging buffer (all of them in flight on the read workers), and
// each record's host->device copy into its slot issued as soon as its read
// has landed. A direct (O_DIRECT) file reads whole strides: record offsets
// and strides are multiples of 4096.
moe_status read_misses(moe_model* m, moe_pool* pool, const int64_t* gids, const int64_t* slots, const uint8_t* miss,
                       ExpertSource& src, int* n_miss) {
  const int k = m->cfg.top_k;
  std::vector<uint64_t> off;
  std::vector<void*> dst, bounce;
  std::vector<size_t> bytes;
  std::vector<int> which;
  const size_t len = m->file.direct() ? m->stride : m->rec_bytes;
  for (int j = 0; j < k; ++j) {
    src.table[j] = slots[j];
    if (!miss[j]) continue;
    off.push_back((uint64_t)gids[j] * m->stride);
    dst.push_back(pool->staging + which.size() * m->stride);
    if (pool->bounce) bounce.push_back(pool->bounce + which.size() * m->stride);
    bytes.push_back(len);
    which.push_back(j);
  }
  *n_miss = (int)which.size();
  if (which.empty()) return MOE_OK;
  // the staging buffers were last read by the previous step's copies
  for (int c = 0; c < moe_pool::kCopyStreams; ++c)
    HIP_TRY(hipEventSynchronize(pool->copies_done[c]), "staging reuse wait");
  pool->readers->start(&m->file, off, dst, bytes, bounce);
  for (size_t i = 0; i < which.size(); ++i) {
    std::string err;
    if (!pool->readers->wait(i, &err)) {
      pool->readers->drain();
      return fail(MOE_EHIP, "moe_stack_decode: expert read from the blob file failed: " + err);
    }
    const int c = (int)(i % moe_pool::kCopyStreams);
    const hipError_t e = hipMemcpyAsync(pool->arena + (size_t)slots[which[i]] * m->stride, dst[i], m->rec_bytes,
                                        hipMemcpyHostToDevice, pool->copy_stream[c]);
    if (e != hipSuccess) {
      pool->readers->drain();
      return hip_fail(e, "miss copy");
    }
  }
  pool->storage_reads += which.size();
  pool->storage_bytes += which.size() * len;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_model_create(const moe_config* cfg, int32_t storage, moe_model** out) {
  clear_error();
  if (!out) return fail(MOE_EINVAL, "moe_model_create: out is NULL");
  *out = nullptr;
  std::string why = check_config(cfg);
  if (!why.empty()) return fail(MOE_EINVAL, "moe_model_create: " + why);
  if (storage != MOE_STORE_DEVICE && storage != MOE_STORE_HOST && storage != MOE_STORE_FILE)
    return fail(MOE_EINVAL, "moe_model_create: storage must be MOE_STORE_DEVICE, MOE_STORE_HOST or MOE_STORE_FILE");
  Geometry g{};
  g.H = cfg->hidden;
  g.I = cfg->inter;
  g.E = cfg->n_experts;
  g.k = cfg->top_k;
  g.bits = cfg->bits;
  g.norm_topk = cfg->norm_topk;
  RecordLayout lay = record_layout(*cfg, cfg->inter);
  g.gate_codes = lay.gate_codes;
  g.up_codes = lay.up_codes;
  g.down_codes = lay.down_codes;
  g.gate_sc = lay.gate_sc;
  g.up_sc = lay.up_sc;
  g.down_sc = lay.down_sc;
  if (!decode_shape_supported(g))
    return fail(MOE_EINVAL, "moe_model_create: shape not supported (n_experts <= 1024, (top_k+1)*inter <= 15360)");

  moe_model* m = new moe_model();
  m->cfg = *cfg;
  m->storage = storage;
  m->geo = g;
  m->rec_bytes = record_bytes(*cfg, cfg->inter);
  m->stride = record_stride(*cfg, cfg->inter);
  m->shared_stride = record_stride(*cfg, cfg->shared_inter);
  m->layer_set.assign((size_t)cfg->n_layers, 0);
  hipGetDevice(&m->device);
  const size_t L = cfg->n_layers, E = cfg->n_experts, H = cfg->hidden;
  m->experts_bytes = L * E * m->stride;
  bool ok = true;
  hipError_t e = hipSuccess;
  if (storage == MOE_STORE_DEVICE) {
    e = hipMalloc(&m->experts, m->experts_bytes);
    ok = ok && e == hipSuccess;
    if (ok) ok = hipMemset(m->experts, 0, m->experts_bytes) == hipSuccess;
  } else if (storage == MOE_STORE_HOST) {
    e = hipHostMalloc(&m->experts, m->experts_bytes, hipHostMallocDefault);
    ok = ok && e == hipSuccess;
  }  // MOE_STORE_FILE: the records stay in the blob file (moe_model_open_blob)
  ok = ok && hipMalloc(&m->shared, L * m->shared_stride) == hipSuccess;
  ok = ok && hipMalloc(&m->wr_rows, L * (E + 1) * H * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&m->wr_split, L * 3 * (E + 1) * H * sizeof(uint16_t)) == hipSuccess;
  ok = ok && hipMalloc(&m->bias, L * E * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&m->logits, (E + 1) * sizeof(float)) == hipSuccess;
  {
    // decode scratch: h of the two-kernel path, or the fused path's partial rows
    const size_t slots = (size_t)cfg->top_k + 1;
    const size_t n_h = slots * cfg->inter;
    const size_t n_part = slots * ((size_t)cfg->inter / 32) * cfg->hidden;  // 32-row I slices
    ok = ok && hipMalloc(&m->h, std::max(n_h, n_part) * sizeof(float)) == hipSuccess;
    ok = ok && hipMalloc(&m->h_scalar, n_h * sizeof(float)) == hipSuccess;
  }
  ok = ok && hipMalloc(&m->rbuf, H * sizeof(float)) == hipSuccess;
  ok = ok && hipMalloc(&m->xbuf, 2 * H * sizeof(uint16_t)) == hipSuccess;
  if (ok) ok = hipMemset(m->bias, 0, L * E * sizeof(float)) == hipSuccess;
  if (ok) ok = hipMemset(m->shared, 0, L * m->shared_stride) == hipSuccess;
  if (ok) ok = hipMemset(m->wr_rows, 0, L * (E + 1) * H * sizeof(float)) == hipSuccess;
  if (ok) ok = hipMemset(m->wr_split, 0, L * 3 * (E + 1) * H * sizeof(uint16_t)) == hipSuccess;
  if (ok) ok = hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    live_add(m);
    moe_model_destroy(m);
    return fail(MOE_ENOMEM, "moe_model_create: allocation failed");
  }
  live_add(m);
  moe_status st = ensure_route_cap(m, 1);
  if (st) {
    moe_model_destroy(m);
    return st;
  }
  *out = m;
  return MOE_OK;
}

moe_status moe_model_set_layer(moe_model* m, int32_t layer, const float* router_w, const float* router_bias,
                               const void* shared_record, const float* shared_gate) {
  clear_error();
  moe_status st = check_model(m, "moe_model_set_layer");
  if (st) return st;
  if (layer < 0 || layer >= m->cfg.n_layers) return fail(MOE_EINVAL, "moe_model_set_layer: layer out of range");
  if (!router_w || !shared_record || !shared_gate) return fail(MOE_EINVAL, "moe_model_set_layer: NULL pointer");
  const size_t E = m->cfg.n_experts, H = m->cfg.hidden;
  std::vector<float> rows((E + 1) * H);
  for (size_t h = 0; h < H; ++h)
    for (size_t e = 0; e < E; ++e) rows[e * H + h] = router_w[h * E + e];
  std::memcpy(rows.data() + E * H, shared_gate, H * sizeof(float));
  HIP_TRY(hipMemcpy((void*)layer_wr(m, layer), rows.data(), rows.size() * sizeof(float), hipMemcpyHostToDevice),
          "moe_model_set_layer: router upload");
  // The batched router's operand: each fp32 weight as three bf16 whose sum is
  // the weight exactly (leading 8 significand bits, then those of the two
  // rounding residuals; both subtractions are exact in fp32).
  std::vector<uint16_t> split(3 * rows.size());
  for (size_t i = 0; i < rows.size(); ++i) {
    const uint16_t hi = bf16_rne_bits(rows[i]);
    const float r1 = rows[i] - bf16_value(hi);
    const uint16_t mid = bf16_rne_bits(r1);
    const uint16_t lo = bf16_rne_bits(r1 - bf16_value(mid));
    split[i] = hi;
    split[rows.size() + i] = mid;
    split[2 * rows.size() + i] = lo;
  }
  HIP_TRY(hipMemcpy((void*)layer_wr_split(m, layer), split.data(), split.size() * sizeof(uint16_t),
                    hipMemcpyHostToDevice),
          "moe_model_set_layer: router split upload");
  if (router_bias) {
    HIP_TRY(hipMemcpy((void*)layer_bias(m, layer), router_bias, E * sizeof(float), hipMemcpyHostToDevice),
            "moe_model_set_layer: bias upload");
  } else {
    HIP_TRY(hipMemset((void*)layer_bias(m, layer), 0, E * sizeof(float)), "moe_model_set_layer: bias clear");
  }
  const size_t sb = record_bytes(m->cfg, m->cfg.shared_inter);
  HIP_TRY(hipMemcpy((void*)layer_shared(m, layer), shared_record, sb, hipMemcpyHostToDevice),
          "moe_model_set_layer: shared expert upload");
  HIP_TRY(hipDeviceSynchronize(), "moe_model_set_layer");
  m->layer_set[(size_t)layer] = 1;
  return MOE_OK;
}

moe_status moe_model_set_experts(moe_model* m, int64_t first_gid, int64_t n, const void* records) {
  clear_error();
  moe_status st = check_model(m, "moe_model_set_experts");
  if (st) return st;
  const int64_t total = (int64_t)m->cfg.n_layers * m->cfg.n_experts;
  if (first_gid < 0 || n < 0 || first_gid + n > total)
    return fail(MOE_EINVAL, "moe_model_set_experts: gid range outside [0, L*E)");
  if (n == 0) return MOE_OK;
  if (!records) return fail(MOE_EINVAL, "moe_model_set_experts: records is NULL");
  if (m->storage == MOE_STORE_FILE)
    return fail(MOE_ESTATE, "moe_model_set_experts: a file-backed model reads its records from the blob file");
  uint8_t* dst = m->experts + (size_t)first_gid * m->stride;
  const size_t bytes = (size_t)n * m->stride;
  if (m->storage == MOE_STORE_DEVICE) {
    HIP_TRY(hipMemcpy(dst, records, bytes, hipMemcpyHostToDevice), "moe_model_set_experts: upload");
  } else {
    std::memcpy(dst, records, bytes);
  }
  return MOE_OK;
}

moe_status moe_model_host_blob(moe_model* m, void** ptr, size_t* bytes) {
  clear_error();
  moe_status st = check_model(m, "moe_model_host_blob");
  if (st) return st;
  if (!ptr || !bytes) return fail(MOE_EINVAL, "moe_model_host_blob: NULL pointer");
  if (m->storage != MOE_STORE_HOST) return fail(MOE_ESTATE, "moe_model_host_blob: model keeps experts in HBM");
  *ptr = m->experts;
  *bytes = m->experts_bytes;
  return MOE_OK;
}

moe_status moe_model_open_blob(moe_model* m, const char* path, uint64_t base, int32_t flags) {
  clear_error();
  moe_status st = check_model(m, "moe_model_open_blob");
  if (st) return st;
  if (!path) return fail(MOE_EINVAL, "moe_model_open_blob: path is NULL");
  if (flags != 0 && flags != MOE_FILE_DIRECT) return fail(MOE_EINVAL, "moe_model_open_blob: unknown flags");
  if (m->storage != MOE_STORE_FILE)
    return fail(MOE_ESTATE, "moe_model_open_blob: the model was not created with MOE_STORE_FILE");
  std::string err;
  if (!m->file.open(path, base, m->experts_bytes, flags == MOE_FILE_DIRECT, &err))
    return fail(MOE_EINVAL, "moe_model_open_blob: " + err);
  return MOE_OK;
}

void moe_model_destroy(moe_model* m) {
  if (!m || !live_has(m) || m->magic != kModelMagic) return;
  hipDeviceSynchronize();
  m->file.close();
  if (m->storage == MOE_STORE_HOST) hipHostFree(m->experts);
  else hipFree(m->experts);
  hipFree(m->shared);
  hipFree(m->wr_rows);
  hipFree(m->wr_split);
  hipFree(m->bias);
  hipFree(m->logits);
  hipFree(m->h);
  hipFree(m->h_scalar);
  hipFree(m->rbuf);
  hipFree(m->xbuf);
  hipFree(m->route_idx);
  hipFree(m->route_w);
  hipFree(m->route_gamma);
  prefill_free(m->prefill);
  m->prof.release();
  drop_graphs(m);
  if (m->cap_stream) hipStreamDestroy(m->cap_stream);
  m->magic = 0;
  live_del(m);
  delete m;
}

moe_status moe_layer_decode(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                            void* stream) {
  clear_error();
  moe_status st = check_forward_args(m, layer, x, n_tok, out, "moe_layer_decode");
  if (st) return st;
  if (n_tok == 0) {
    m->route_steps = 0;
    return MOE_OK;
  }
  st = ensure_route_cap(m, (size_t)n_tok);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto enqueue = [&](hipStream_t q) -> moe_status {
    const size_t H = m->cfg.hidden;
    const ExpertSource src = resident_source(m, layer);
    for (int t = 0; t < n_tok; ++t) {
      StepBuffers b = step_buffers(m, x + (size_t)t * H, (size_t)t);
      ResidualArgs r{out + (size_t)t * H, nullptr, nullptr, nullptr};
      moe_status e = decode_step(m, layer, b, src, r, q);
      if (e) return e;
    }
    return MOE_OK;
  };
  st = (n_tok >= kGraphMinTokens && !m->prof.on) ? run_graph(m, 1 + m->kernels, layer, x, out, n_tok, s, enqueue)
                                                   : enqueue(s);
  if (st) return st;
  m->route_steps = (size_t)n_tok;
  return MOE_OK;
}

// Batches of at least this many tokens take the bucketed grouped-GEMM path.
// Measured on the 80B-shaped layer (one MI355X): 4 tokens 64 us token by
// token against 81 us batched, 8 tokens 127 against 99, 64 tokens 1022
// against 255; the batched path's fixed cost (~70 us) is about five tokens'
// worth of the per-token chain.
constexpr int kBatchedMinTokens = 8;

moe_status moe_layer_forward(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                             void* stream) {
  clear_error();
  moe_status st = check_forward_args(m, layer, x, n_tok, out, "moe_layer_forward");
  if (st) return st;
  if (n_tok == 0) {
    m->route_steps = 0;
    return MOE_OK;
  }
  if (n_tok >= kBatchedMinTokens && prefill_supported(m->cfg)) {
    st = ensure_route_cap(m, (size_t)n_tok);
    if (st) return st;
    PrefillArgs a{};
    a.cfg = m->cfg;
    a.geo = m->geo;
    a.experts = m->experts + (size_t)layer * m->cfg.n_experts * m->stride;
    a.stride = m->stride;
    a.shared = layer_shared(m, layer);
    a.wr_rows = layer_wr(m, layer);
    a.wr_split = layer_wr_split(m, layer);
    a.bias = layer_bias(m, layer);
    a.x = x;
    a.n_tok = n_tok;
    a.out = out;
    a.route_idx = m->route_idx;
    a.route_w = m->route_w;
    a.route_gamma = m->route_gamma;
    a.scalar = m->kernels == MOE_KERNELS_SCALAR;
    st = prefill_reserve(&m->prefill, m->cfg, n_tok);
    if (st) return fail(st, "moe_layer_forward: prefill workspace allocation failed");
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = m->prefill;
    using Stage = hipError_t (*)(void*, const PrefillArgs&, hipStream_t);
    static const Stage kStages[] = {prefill_xprep, prefill_router,  prefill_route,  prefill_count,  prefill_scan,
                                    prefill_scatter, prefill_gateup, prefill_down, prefill_combine};
    for (int i = 0; i < 9; ++i)
      HIP_TRY(m->prof.run(K_PF_XPREP + i, s, [&] { return kStages[i](ws, a, s); }), "moe_layer_forward: prefill stage");
    m->route_steps = (size_t)n_tok;
    return MOE_OK;
  }
  return moe_layer_decode(m, layer, x, n_tok, out, stream);
}

moe_status moe_layer_forward_noalloc(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                                     void* stream) {
  clear_error();
  moe_status st = check_forward_args(m, layer, x, n_tok, out, "moe_layer_forward_noalloc");
  if (st) return st;
  if (!prefill_supported(m->cfg))
    return fail(MOE_EINVAL, "moe_layer_forward_noalloc: the layer shape has no batched path (int4, H % 256 == 0)");
  m->route_steps = 0;  // this call's routing stays in the scratch array
  if (n_tok == 0) return MOE_OK;
  const size_t need = prefill_placed_bytes(m->cfg, n_tok);
  if (need > kNoAllocScratchBytes) {
    int most = n_tok;
    while (most > 0 && prefill_placed_bytes(m->cfg, most) > kNoAllocScratchBytes) most = most * 15 / 16;
    while (prefill_placed_bytes(m->cfg, most + 1) <= kNoAllocScratchBytes) ++most;
    return fail(MOE_EINVAL, "moe_layer_forward_noalloc: " + std::to_string(n_tok) + " tokens need " +
                                std::to_string(need) + " bytes of scratch, more than its " +
                                std::to_string(kNoAllocScratchBytes) + "; this layer shape takes at most " +
                                std::to_string(most) + " tokens per call");
  }
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "moe_layer_forward_noalloc: hipGetDevice");
  if (dev != m->device) return fail(MOE_ESTATE, "moe_layer_forward_noalloc: the model lives on another device");
  uint8_t* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st) return st;
  PrefillWorkspace ws{};
  PrefillArgs a{};
  prefill_place(&ws, m->cfg, n_tok, base, &a.route_idx, &a.route_w, &a.route_gamma);
  a.cfg = m->cfg;
  a.geo = m->geo;
  a.experts = m->experts + (size_t)layer * m->cfg.n_experts * m->stride;
  a.stride = m->stride;
  a.shared = layer_shared(m, layer);
  a.wr_rows = layer_wr(m, layer);
  a.wr_split = layer_wr_split(m, layer);
  a.bias = layer_bias(m, layer);
  a.x = x;
  a.n_tok = n_tok;
  a.out = out;
  a.scalar = m->kernels == MOE_KERNELS_SCALAR;
  hipStream_t s = static_cast<hipStream_t>(stream);
  using Stage = hipError_t (*)(void*, const PrefillArgs&, hipStream_t);
  static const Stage kStages[] = {prefill_xprep, prefill_router,  prefill_route,  prefill_count,  prefill_scan,
                                  prefill_scatter, prefill_gateup, prefill_down, prefill_combine};
  for (const Stage stage : kStages) HIP_TRY(stage(&ws, a, s), "moe_layer_forward_noalloc: prefill stage");
  return MOE_OK;
}

moe_status moe_stack_decode(moe_model* m, moe_pool* pool, const uint16_t* x0, int32_t n_tok, float* out,
                            void* stream) {
  clear_error();
  moe_status st = check_model(m, "moe_stack_decode");
  if (st) return st;
  if (n_tok < 0 || n_tok > 65536) return fail(MOE_EINVAL, "moe_stack_decode: n_tok must be in [0, 65536]");
  if (n_tok > 0 && (!x0 || !out)) return fail(MOE_EINVAL, "moe_stack_decode: NULL pointer");
  if (pool) {
    st = check_pool(pool, "moe_stack_decode");
    if (st) return st;
    if (pool->model != m) return fail(MOE_ESTATE, "moe_stack_decode: pool belongs to another model");
    if (m->kernels != MOE_KERNELS_FAST)
      return fail(MOE_EINVAL, "moe_stack_decode: the scalar kernels read resident experts only; no pool");
  } else if (m->storage != MOE_STORE_DEVICE) {
    return fail(MOE_ESTATE, "moe_stack_decode: experts are in host or file storage; a pool is required");
  }
  for (int l = 0; l < m->cfg.n_layers; ++l)
    if (!m->layer_set[(size_t)l]) return fail(MOE_ESTATE, "moe_stack_decode: a layer was not set");
  if (n_tok == 0) {
    m->route_steps = 0;
    return MOE_OK;
  }
  const int L = m->cfg.n_layers, k = m->cfg.top_k, E = m->cfg.n_experts;
  const size_t H = m->cfg.hidden;
  st = ensure_route_cap(m, (size_t)n_tok * L);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int64_t> gids((size_t)k), slots((size_t)k);
  std::vector<uint8_t> miss((size_t)k);
  for (int t = 0; t < n_tok; ++t) {
    for (int l = 0; l < L; ++l) {
      const size_t step = (size_t)t * L + l;
      const uint16_t* xl = (l == 0) ? x0 + (size_t)t * H : m->xbuf + (size_t)(l & 1) * H;
      StepBuffers b = step_buffers(m, xl, step);
      ResidualArgs r{};
      r.out = (l == L - 1) ? out + (size_t)t * H : m->rbuf;
      r.r_in = (l == 0) ? nullptr : m->rbuf;
      r.x_res = (l == 0) ? x0 + (size_t)t * H : nullptr;
      r.x_next = (l == L - 1) ? nullptr : m->xbuf + (size_t)((l + 1) & 1) * H;
      if (!pool) {
        st = decode_step(m, l, b, resident_source(m, l), r, s);
        if (st) return st;
        continue;
      }
      // pool: top-k on the device, then the host decides hits, misses and victims
      HIP_TRY(m->prof.run(K_ROUTER, s, [&] { return launch_router(m->geo, layer_wr(m, l), layer_bias(m, l), b, s); }),
              "router launch");
      HIP_TRY(m->prof.run(K_ROUTE, s,
                          [&] {
                            return launch_route(m->geo, b.logits, 0, 1, b.route_idx, b.route_w, b.route_gamma,
                                                pool->host_route_dev, s);
                          }),
              "route launch");
      HIP_TRY(hipEventRecord(pool->route_ready, s), "event record");
      HIP_TRY(hipEventSynchronize(pool->route_ready), "route sync");
      for (int j = 0; j < k; ++j) gids[(size_t)j] = (int64_t)l * E + pool->host_route[j];
      pool->table.step(gids.data(), k, slots.data(), miss.data());
      ExpertSource src{};
      src.base = pool->arena;
      src.stride = m->stride;
      src.use_table = 1;
      // Victim slots are free to overwrite: the host waited for this layer's
      // route, recorded after every earlier kernel on the stream.
      int n_miss = 0;
      if (m->storage == MOE_STORE_FILE) {
        st = read_misses(m, pool, gids.data(), slots.data(), miss.data(), src, &n_miss);
        if (st) return st;
      } else {
        for (int j = 0; j < k; ++j) {
          src.table[j] = slots[(size_t)j];
          if (miss[(size_t)j]) {
            const int c = n_miss++ % moe_pool::kCopyStreams;
            HIP_TRY(hipMemcpyAsync(pool->arena + (size_t)slots[(size_t)j] * m->stride,
                                   m->experts + (size_t)gids[(size_t)j] * m->stride, m->rec_bytes,
                                   hipMemcpyHostToDevice, pool->copy_stream[c]),
                    "miss copy");
          }
        }
      }
      // The fused path runs the hit experts and the shared expert at once,
      // while the miss copies are in flight, and the missed experts after the
      // copies land; the reduce sums every slot's partial rows in the same
      // fixed order either way. (Other shapes run every slot after the copies.)
      const bool split = fused_expert_supported(m->geo) && n_miss > 0;
      if (split) {
        ExpertSource hits = src;
        for (int j = 0; j <= k; ++j)
          if (j == k || !miss[(size_t)j]) hits.sel[hits.n_sel++] = j;
        HIP_TRY(m->prof.run(K_EXPERT, s, [&] { return launch_expert(m->geo, hits, layer_shared(m, l), b, s); }),
                "expert launch");
      }
      for (int c = 0; c < moe_pool::kCopyStreams && c < n_miss; ++c) {
        HIP_TRY(hipEventRecord(pool->copies_done[c], pool->copy_stream[c]), "event record");
        HIP_TRY(hipStreamWaitEvent(s, pool->copies_done[c], 0), "stream wait");
      }
      if (split) {
        ExpertSource misses = src;
        for (int j = 0; j < k; ++j)
          if (miss[(size_t)j]) misses.sel[misses.n_sel++] = j;
        HIP_TRY(m->prof.run(K_EXPERT_MISS, s,
                            [&] { return launch_expert(m->geo, misses, layer_shared(m, l), b, s); }),
                "expert launch");
        HIP_TRY(m->prof.run(K_REDUCE, s, [&] { return launch_reduce(m->geo, b, r, s); }), "reduce launch");
      } else {
        st = expert_steps(m, l, b, src, r, s);
        if (st) return st;
      }
    }
  }
  if (pool) HIP_TRY(hipStreamSynchronize(s), "moe_stack_decode: final sync");
  m->route_steps = (size_t)n_tok * L;
  return MOE_OK;
}

moe_status moe_debug_routing(moe_model* m, int32_t* idx, float* w, size_t cap, size_t* n_steps) {
  clear_error();
  moe_status st = check_model(m, "moe_debug_routing");
  if (st) return st;
  if (!n_steps) return fail(MOE_EINVAL, "moe_debug_routing: n_steps is NULL");
  HIP_TRY(hipDeviceSynchronize(), "moe_debug_routing: sync");
  *n_steps = m->route_steps;
  const size_t n = std::min(cap, m->route_steps);
  const size_t k = (size_t)m->cfg.top_k;
  if (n && idx) HIP_TRY(hipMemcpy(idx, m->route_idx, n * k * sizeof(int32_t), hipMemcpyDeviceToHost), "copy idx");
  if (n && w) HIP_TRY(hipMemcpy(w, m->route_w, n * k * sizeof(float), hipMemcpyDeviceToHost), "copy w");
  return MOE_OK;
}

moe_status moe_model_set_kernels(moe_model* m, int32_t kernels) {
  clear_error();
  moe_status st = check_model(m, "moe_model_set_kernels");
  if (st) return st;
  if (kernels != MOE_KERNELS_FAST && kernels != MOE_KERNELS_SCALAR)
    return fail(MOE_EINVAL, "moe_model_set_kernels: kernels must be MOE_KERNELS_FAST or MOE_KERNELS_SCALAR");
  m->kernels = kernels;
  return MOE_OK;
}

moe_status moe_profile_enable(moe_model* m, int32_t enable) {
  clear_error();
  moe_status st = check_model(m, "moe_profile_enable");
  if (st) return st;
  if (enable != 0 && enable != 1) return fail(MOE_EINVAL, "moe_profile_enable: enable must be 0 or 1");
  m->prof.on = enable != 0;
  return MOE_OK;
}

moe_status moe_profile_read(moe_model* m, moe_kernel_time_t* out, size_t cap, size_t* n) {
  clear_error();
  moe_status st = check_model(m, "moe_profile_read");
  if (st) return st;
  if (!n) return fail(MOE_EINVAL, "moe_profile_read: n is NULL");
  HIP_TRY(m->prof.harvest(), "moe_profile_read: event wait");
  *n = K_COUNT;
  for (size_t i = 0; i < K_COUNT && i < cap && out; ++i) {
    std::memset(out[i].name, 0, sizeof(out[i].name));
    std::strncpy(out[i].name, kKindName[i], sizeof(out[i].name) - 1);
    out[i].launches = m->prof.launches[i];
    out[i].total_ms = m->prof.ms[i];
  }
  for (int i = 0; i < K_COUNT; ++i) {
    m->prof.launches[i] = 0;
    m->prof.ms[i] = 0.0;
  }
  return MOE_OK;
}

moe_status moe_pool_create(moe_model* m, size_t budget_bytes, moe_pool** out) {
  clear_error();
  if (!out) return fail(MOE_EINVAL, "moe_pool_create: out is NULL");
  *out = nullptr;
  moe_status st = check_model(m, "moe_pool_create");
  if (st) return st;
  if (m->storage == MOE_STORE_DEVICE) return fail(MOE_ESTATE, "moe_pool_create: the model keeps its experts in HBM");
  if (m->storage == MOE_STORE_FILE && !m->file.is_open())
    return fail(MOE_ESTATE, "moe_pool_create: open the blob file first (moe_model_open_blob)");
  const int64_t slots = (int64_t)(budget_bytes / m->stride);
  if (slots < m->cfg.top_k)
    return fail(MOE_EINVAL, "moe_pool_create: budget holds " + std::to_string(slots) + " slots, fewer than top_k");
  moe_pool* p = new moe_pool();
  p->model = m;
  p->n_slots = slots;
  p->table = PoolTable(slots);
  bool ok = hipMalloc(&p->arena, (size_t)slots * m->stride) == hipSuccess;
  for (int c = 0; c < moe_pool::kCopyStreams; ++c) {
    ok = ok && hipStreamCreateWithFlags(&p->copy_stream[c], hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&p->copies_done[c], hipEventDisableTiming) == hipSuccess;
  }
  ok = ok && hipEventCreateWithFlags(&p->route_ready, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipHostMalloc(&p->host_route, kMaxTopK * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess;
  ok = ok && hipHostGetDevicePointer((void**)&p->host_route_dev, p->host_route, 0) == hipSuccess;
  if (ok && m->storage == MOE_STORE_FILE) {
    ok = hipHostMalloc(&p->staging, (size_t)m->cfg.top_k * m->stride, hipHostMallocDefault) == hipSuccess;
    if (ok && m->file.direct()) {
      void* b = nullptr;
      ok = posix_memalign(&b, kDirectAlign, (size_t)m->cfg.top_k * m->stride) == 0;
      p->bounce = static_cast<uint8_t*>(b);
    }
    // completed events, so the first step's staging wait returns at once
    for (int c = 0; ok && c < moe_pool::kCopyStreams; ++c)
      ok = hipEventRecord(p->copies_done[c], p->copy_stream[c]) == hipSuccess;
    if (ok) p->readers = new ReadWorkers(std::min(m->cfg.top_k, 8));
  }
  live_add(p);
  if (!ok) {
    moe_pool_destroy(p);
    return fail(MOE_ENOMEM, "moe_pool_create: allocation failed");
  }
  *out = p;
  return MOE_OK;
}

moe_status moe_pool_reset(moe_pool* p) {
  clear_error();
  moe_status st = check_pool(p, "moe_pool_reset");
  if (st) return st;
  p->table.reset();
  p->storage_reads = p->storage_bytes = 0;
  return MOE_OK;
}

moe_status moe_pool_stats(const moe_pool* p, moe_pool_stats_t* out) {
  clear_error();
  moe_status st = check_pool(p, "moe_pool_stats");
  if (st) return st;
  if (!out) return fail(MOE_EINVAL, "moe_pool_stats: out is NULL");
  out->accesses = p->table.accesses;
  out->hits = p->table.hits;
  out->misses = p->table.misses;
  out->evictions = p->table.evictions;
  out->h2d_bytes = p->table.misses * (uint64_t)p->model->rec_bytes;
  out->requested_bytes = p->table.accesses * (uint64_t)p->model->rec_bytes;
  out->storage_reads = p->storage_reads;
  out->storage_bytes = p->storage_bytes;
  out->direct_io = p->model->storage == MOE_STORE_FILE && p->model->file.direct() ? 1 : 0;
  return MOE_OK;
}

moe_status moe_pool_trace(const moe_pool* p, uint8_t* hit, int64_t* victim, size_t cap, size_t* n) {
  clear_error();
  moe_status st = check_pool(p, "moe_pool_trace");
  if (st) return st;
  if (!n) return fail(MOE_EINVAL, "moe_pool_trace: n is NULL");
  *n = p->table.trace_hit.size();
  const size_t c = std::min(cap, *n);
  if (hit) std::copy(p->table.trace_hit.begin(), p->table.trace_hit.begin() + (ptrdiff_t)c, hit);
  if (victim) std::copy(p->table.trace_victim.begin(), p->table.trace_victim.begin() + (ptrdiff_t)c, victim);
  return MOE_OK;
}

void moe_pool_destroy(moe_pool* p) {
  if (!p || !live_has(p) || p->magic != kPoolMagic) return;
  hipDeviceSynchronize();
  hipFree(p->arena);
  for (int c = 0; c < moe_pool::kCopyStreams; ++c) {
    if (p->copy_stream[c]) hipStreamDestroy(p->copy_stream[c]);
    if (p->copies_done[c]) hipEventDestroy(p->copies_done[c]);
  }
  if (p->route_ready) hipEventDestroy(p->route_ready);
  if (p->host_route) hipHostFree(p->host_route);
  delete p->readers;
  if (p->staging) hipHostFree(p->staging);
  free(p->bounce);
  p->magic = 0;
  live_del(p);
  delete p;
}

}  // extern "C"
