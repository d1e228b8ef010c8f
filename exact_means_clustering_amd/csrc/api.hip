// C ABI of the k-means library: argument validation, workspace carve-up and
// the stream-ordered Lloyd loop.  See include/flashkm.h for the contract.
#include "kernels.h"
#include "workspace.h"

#include "flashkm.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <tuple>
#include <vector>

using namespace fkm;

namespace {

int hip_fail(hipError_t e, const char* what) { return fail(KM_EHIP, "%s: %s", what, hipGetErrorString(e)); }

#define KM_HIP(expr, what)                           \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool supported_d(int D) { return D == 16 || D == 32 || D == 64 || D == 128 || D == 256; }

int check_shape(int dtype, int64_t N, int32_t D, int32_t K, int32_t B) {
  if (dtype != KM_F32 && dtype != KM_F16 && dtype != KM_BF16) return fail(KM_EUNSUPPORTED, "unsupported dtype %d", dtype);
  if (!supported_d(D)) return fail(KM_EUNSUPPORTED, "unsupported D=%d (supported: 16, 32, 64, 128, 256)", D);
  if (B < 1) return fail(KM_EINVAL, "B=%d must be >= 1", B);
  if (K < 1) return fail(KM_EINVAL, "K=%d must be >= 1", K);
  if (N < K) return fail(KM_EINVAL, "need N >= K (N=%lld, K=%d)", (long long)N, K);
  if (N * (int64_t)B >= (int64_t)1 << 31) return fail(KM_EINVAL, "B*N must be < 2^31");
  if ((int64_t)B * K >= (int64_t)1 << 31) return fail(KM_EINVAL, "B*K must be < 2^31");
  return KM_OK;
}

int check_ws(const void* ws, size_t ws_bytes, const Layout& L) {
  if (ws_bytes < L.total)
    return fail(KM_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, L.total);
  if (!ws) return fail(KM_EINVAL, "workspace pointer is null");
  if (((uintptr_t)ws & 255) != 0) return fail(KM_EINVAL, "workspace must be 256-byte aligned");
  return KM_OK;
}

// prep + assign (+ inertia) on stream s
int run_assign(const void* X, int dt, int64_t N, int D, int B, const float* C, int K, int32_t* labels,
               float* min_d2, double* inertia, double* hist, Work& w, hipStream_t s) {
  KM_HIP(launch_prep(dt, D, C, w.chat, w.hb, B, K, s), "centroid prep launch");
  const AssignConfig cfg = assign_pick(dt, D, N, B, K);
  KM_HIP(launch_assign(dt, D, cfg, X, w.chat, w.hb, N, K, B, labels, min_d2, w.part, s), "assign launch");
  if (inertia) KM_HIP(launch_inertia_reduce(w.part, (int)cfg.parts(N), B, inertia, hist, false, s), "inertia launch");
  return KM_OK;
}

// argsort + segment offsets and means on stream s
int run_update(const void* X, int dt, int64_t N, int D, int B, const int32_t* labels, int K, const float* C_prev,
               float* C_new, int32_t* counts, Work& w, hipStream_t s) {
  const uint2* sorted = nullptr;
  const int64_t n = N * B;
  const uint32_t nseg = (uint32_t)((int64_t)B * K);
  KM_HIP(launch_argsort_labels(labels, N, B, K, w.sort, &sorted, s), "argsort launch");
  SegOut o{C_prev, C_new, counts ? counts : w.cnt, nullptr, nullptr};
  KM_HIP(launch_segment_reduce(dt, D, X, sorted, w.off, n, nseg, o, w.seg, s), "segment reduce launch");
  return KM_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---- the Lloyd loop and its graph replay ------------------------------------
struct FitArgs {
  const void* X;
  int dt;
  int64_t N;
  int D, B;
  const float* C0;
  int K, iters;
  int32_t* labels;
  float* C_out;
  double* inertia;
  double* hist;
  void* ws;
  size_t ws_bytes;
  int dev;
  // the assign configuration chosen for the shape when the call was made:
  // part of the key, so a replay never runs a configuration the tuning table
  // or the environment no longer selects
  AssignConfig cfg;
  auto tie() const {
    return std::tie(X, dt, N, D, B, C0, K, iters, labels, C_out, inertia, hist, ws, ws_bytes, dev, cfg.pb, cfg.waves);
  }
  bool operator==(const FitArgs& o) const { return tie() == o.tie(); }
};

// iters x (assign, argsort, segment reductions) on stream s.  Two
// stand-alone launches of kmeans_assign / kmeans_update are folded into
// neighbours: the inertia reduction runs as extra blocks of the first sort
// histogram, and the centroid preparation for iteration t+1 is done by the
// update of iteration t as it finishes each cluster (a kernel prepares C0).
int enqueue_fit(const FitArgs& a, Work& w, hipStream_t s) {
  const int64_t n = a.N * a.B;
  const uint32_t nseg = (uint32_t)((int64_t)a.B * a.K);
  const AssignConfig cfg = a.cfg;
  const int64_t nwg = cfg.parts(a.N);
  KM_HIP(launch_prep(a.dt, a.D, a.C0, w.chat, w.hb, a.B, a.K, s), "centroid prep launch");
  for (int t = 0; t < a.iters; ++t) {
    const float* Cs = t == 0 ? a.C0 : a.C_out;
    KM_HIP(launch_assign(a.dt, a.D, cfg, a.X, w.chat, w.hb, a.N, a.K, a.B, a.labels, nullptr, w.part, s),
           "assign launch");
    InertiaJob side;
    side.part = w.part;
    side.nwg = (int)nwg;
    side.B = a.B;
    side.inertia = a.inertia;
    side.hist = a.hist ? a.hist + (int64_t)t * a.B : nullptr;
    const uint2* sorted = nullptr;
    KM_HIP(launch_argsort_labels(a.labels, a.N, a.B, a.K, w.sort, &sorted, s, &side), "argsort launch");
    SegOut o{Cs, a.C_out, w.cnt, nullptr, nullptr};
    o.chat = w.chat;
    o.hb = w.hb;
    o.K = (uint32_t)a.K;
    o.Kp = (uint32_t)kpad(a.K);
    KM_HIP(launch_segment_reduce(a.dt, a.D, a.X, sorted, w.off, n, nseg, o, w.seg, s), "segment reduce launch");
  }
  return KM_OK;
}

// A fit is a fixed sequence of 6 to 10 kernels per iteration whose
// arguments are only pointers and sizes, so it is captured once into a HIP
// graph and replayed: one graph launch enqueues every kernel, which removes
// the per-launch host overhead that dominates small problems.  Graphs are
// kept for the last few distinct argument lists (a replay binds the same
// buffers; their contents may change freely between calls).  Capture runs on
// a private stream (default priority) and records kernels only.
// FLASHKM_FIT_GRAPH=0 selects direct launches.
constexpr size_t kGraphCache = 8;
struct GraphEntry {
  FitArgs key;
  hipGraphExec_t exec;
};
std::mutex& graph_mutex() {
  static std::mutex m;
  return m;
}
std::vector<GraphEntry>& graph_cache() {
  static std::vector<GraphEntry> c;
  return c;
}
bool graphs_enabled() {
  const char* e = getenv("FLASHKM_FIT_GRAPH");
  return !(e && e[0] == '0');
}

int fit_graph(const FitArgs& a, Work& w, hipStream_t s) {
  std::lock_guard<std::mutex> lock(graph_mutex());
  auto& cache = graph_cache();
  for (const GraphEntry& g : cache)
    if (g.key == a) {
      KM_HIP(hipGraphLaunch(g.exec, s), "graph launch");
      return KM_OK;
    }
  // device queries the launches need happen now, not during the capture
  KM_HIP(assign_prime(a.dt, a.D, a.cfg), "assign configuration query");
  static hipStream_t capture[64] = {};
  if (a.dev < 0 || a.dev >= 64) return fail(KM_EINVAL, "device index %d out of range", a.dev);
  if (!capture[a.dev]) KM_HIP(hipStreamCreateWithFlags(&capture[a.dev], hipStreamNonBlocking), "stream create");
  hipStream_t cs = capture[a.dev];
  KM_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal), "graph capture begin");
  const int rc = enqueue_fit(a, w, cs);
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(cs, &graph);
  if (rc != KM_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  if (ec != hipSuccess) return hip_fail(ec, "graph capture end");
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) return hip_fail(ei, "graph instantiate");
  if (cache.size() == kGraphCache) {
    (void)hipGraphExecDestroy(cache.front().exec);
    cache.erase(cache.begin());
  }
  cache.push_back(GraphEntry{a, exec});
  KM_HIP(hipGraphLaunch(exec, s), "graph launch");
  return KM_OK;
}

// ---- the assignment stage without a caller workspace ------------------------
// Scratch of kmeans_assign_noalloc: the rounded centroids, their biases and
// the per-workgroup inertia partials live in this file-scope device array
// (one copy per GPU, held until the process ends).  Host code never uses
// the array's name as an address: the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocScratch = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratch];

// Regions of the scratch for an assignment of this shape (256-byte aligned).
struct NoAllocLayout {
  size_t chat, hb, part, total;
};
NoAllocLayout noalloc_layout(int64_t N, int D, int K, int B, int dt) {
  NoAllocLayout L{};
  size_t o = 0;
  L.chat = o;  o = al256(o + (size_t)B * K * D * dtype_size(dt));
  L.hb = o;    o = al256(o + (size_t)B * kpad(K) * 4);
  L.part = o;  o = al256(o + (size_t)B * assign_max_parts(N) * 8);
  L.total = o;
  return L;
}

int scratch_address(void** out) {
  static std::mutex m;
  static void* addr[64] = {};
  int dev = 0;
  KM_HIP(hipGetDevice(&dev), "device query");
  if (dev < 0 || dev >= 64) return fail(KM_EINVAL, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(m);
  if (!addr[dev]) {
    void* p = nullptr;
    KM_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (!p) return fail(KM_EHIP, "scratch symbol address is null");
    addr[dev] = p;
  }
  *out = addr[dev];
  return KM_OK;
}

}  // namespace

extern "C" {

int kmeans_assign_noalloc(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* C, int32_t K,
                          int32_t* labels, float* min_d2, double* inertia, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (!X || !C || !labels) return fail(KM_EINVAL, "X, C and labels must be non-null");
  if (!aligned(X, 16) || !aligned(C, 4) || !aligned(labels, 4) || !aligned(min_d2, 4) || !aligned(inertia, 8))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const NoAllocLayout L = noalloc_layout(N, D, K, B, dtype);
  if (L.total > kNoAllocScratch)
    return fail(KM_EWORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu", L.total,
                kNoAllocScratch);
  void* base = nullptr;
  if (int rc = scratch_address(&base)) return rc;
  char* b = static_cast<char*>(base);
  Work w{};
  w.chat = b + L.chat;
  w.hb = reinterpret_cast<float*>(b + L.hb);
  w.part = reinterpret_cast<double*>(b + L.part);
  return run_assign(X, dtype, N, D, B, C, K, labels, min_d2, inertia, nullptr, w, (hipStream_t)stream);
}

size_t kmeans_workspace_bytes(int64_t N, int32_t D, int32_t K, int32_t B, int32_t dtype) {
  if (check_shape(dtype, N, D, K, B) != KM_OK) return 0;
  return make_layout(N, D, K, B, dtype).total;
}

int kmeans_assign(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* C, int32_t K,
                  int32_t* labels, float* min_d2, double* inertia, void* ws, size_t ws_bytes, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (!X || !C || !labels) return fail(KM_EINVAL, "X, C and labels must be non-null");
  if (!aligned(X, 16) || !aligned(C, 4) || !aligned(labels, 4) || !aligned(min_d2, 4) || !aligned(inertia, 8))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  return run_assign(X, dtype, N, D, B, C, K, labels, min_d2, inertia, nullptr, w, (hipStream_t)stream);
}

int kmeans_assign_top2(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* C, int32_t K,
                       int32_t* labels2, float* d2, void* ws, size_t ws_bytes, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (K < 2) return fail(KM_EINVAL, "top-2 assignment needs K >= 2 (K=%d)", K);
  if (!X || !C || !labels2) return fail(KM_EINVAL, "X, C and labels2 must be non-null");
  if (!aligned(X, 16) || !aligned(C, 4) || !aligned(labels2, 4) || !aligned(d2, 4))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  KM_HIP(launch_prep(dtype, D, C, w.chat, w.hb, B, K, s), "centroid prep launch");
  KM_HIP(launch_assign_top2(dtype, D, X, w.chat, w.hb, N, K, B, labels2, d2, s), "top-2 assign launch");
  return KM_OK;
}

int kmeans_assign_soft(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* C, int32_t K,
                       const float* log_w, float sigma2, int32_t* labels, float* log_density, double* total,
                       void* ws, size_t ws_bytes, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (!(sigma2 > 0.f) || !(sigma2 < INFINITY)) return fail(KM_EINVAL, "sigma2 must be positive and finite");
  if (!X || !C || !labels || !log_density) return fail(KM_EINVAL, "X, C, labels and log_density must be non-null");
  if (!aligned(X, 16) || !aligned(C, 4) || !aligned(log_w, 4) || !aligned(labels, 4) || !aligned(log_density, 4) ||
      !aligned(total, 8))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  KM_HIP(launch_prep(dtype, D, C, w.chat, w.hb, B, K, s, log_w, sigma2), "centroid prep launch");
  const SoftArgs sa{log_w, 1.4426950408889634f / sigma2, 0.5f / sigma2};
  KM_HIP(launch_assign_soft(dtype, D, X, w.chat, w.hb, N, K, B, labels, log_density, w.part, sa, s),
         "soft assign launch");
  if (total) {
    KM_HIP(launch_inertia_reduce(w.part, (int)mode_config(dtype, D).parts(N), B, total, nullptr, false, s),
           "total launch");
  }
  return KM_OK;
}

int kmeans_gauss_sum(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* Y, int32_t K,
                     const float* w, float sigma2, float* gsum, double* total, void* ws, size_t ws_bytes,
                     void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (!(sigma2 > 0.f) || !(sigma2 < INFINITY)) return fail(KM_EINVAL, "sigma2 must be positive and finite");
  if (!X || !Y || !w || !gsum) return fail(KM_EINVAL, "X, Y, w and gsum must be non-null");
  if (!aligned(X, 16) || !aligned(Y, 4) || !aligned(w, 4) || !aligned(gsum, 4) || !aligned(total, 8))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work wk = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  KM_HIP(launch_prep(dtype, D, Y, wk.chat, wk.hb, B, K, s), "source prep launch");
  KM_HIP(launch_pad_weights(w, wk.wpad, B, K, s), "weight pad launch");
  // the kernel also writes each point's nearest source, which this entry point
  // does not return: it lands in the first sort buffer (B*N pairs of words),
  // since the counts region holds only B*K entries and K may be below N
  int32_t* lab = reinterpret_cast<int32_t*>(wk.sort.kv[0]);
  const SoftArgs sa{nullptr, 1.4426950408889634f / sigma2, 0.5f / sigma2, wk.wpad};
  KM_HIP(launch_assign_gauss(dtype, D, X, wk.chat, wk.hb, N, K, B, lab, gsum, wk.part, sa, s), "gauss sum launch");
  if (total) {
    KM_HIP(launch_inertia_reduce(wk.part, (int)mode_config(dtype, D).parts(N), B, total, nullptr, false, s),
           "total launch");
  }
  return KM_OK;
}

int kmeans_seed(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, int32_t K, int32_t method,
                const double* u, int32_t* idx, float* C, float* d2, void* ws, size_t ws_bytes, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (method != 0 && method != 1) return fail(KM_EINVAL, "method must be 0 (random) or 1 (k-means++), got %d", method);
  if (!X || !u || !idx || !C) return fail(KM_EINVAL, "X, u, idx and C must be non-null");
  if (!aligned(X, 16) || !aligned(u, 8) || !aligned(idx, 4) || !aligned(C, 4) || !aligned(d2, 4))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  // running D2 [B,N] fp32 in the first sort buffer (B*N*8 bytes), block sums in the partials
  KM_HIP(launch_seed(dtype, D, X, N, B, K, method, u, idx, C, reinterpret_cast<float*>(w.sort.kv[0]), w.part, d2,
                     (hipStream_t)stream),
         "seeding launch");
  return KM_OK;
}

int kmeans_tune(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* C, int32_t K,
                int32_t* labels, void* ws, size_t ws_bytes, void* stream, int32_t* pb, int32_t* waves, float* ms) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (!X || !C || !labels) return fail(KM_EINVAL, "X, C and labels must be non-null");
  if (!aligned(X, 16) || !aligned(C, 4) || !aligned(labels, 4))
    return fail(KM_EINVAL, "misaligned pointer (X needs 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  struct Events {
    hipEvent_t a = nullptr, b = nullptr;
    ~Events() {
      if (a) (void)hipEventDestroy(a);
      if (b) (void)hipEventDestroy(b);
    }
  } ev;
  KM_HIP(hipEventCreate(&ev.a), "event create");
  KM_HIP(hipEventCreate(&ev.b), "event create");
  KM_HIP(launch_prep(dtype, D, C, w.chat, w.hb, B, K, s), "centroid prep launch");
  AssignConfig cand[8];
  const int nc = assign_configs(dtype, D, cand, 8);
  AssignConfig best{0, 0};
  float best_ms = 0.f;
  for (int i = 0; i < nc; ++i) {
    KM_HIP(assign_prime(dtype, D, cand[i]), "assign configuration query");
    KM_HIP(launch_assign(dtype, D, cand[i], X, w.chat, w.hb, N, K, B, labels, nullptr, w.part, s), "assign launch");
    KM_HIP(hipEventRecord(ev.a, s), "event record");
    for (int r = 0; r < 2; ++r)
      KM_HIP(launch_assign(dtype, D, cand[i], X, w.chat, w.hb, N, K, B, labels, nullptr, w.part, s), "assign launch");
    KM_HIP(hipEventRecord(ev.b, s), "event record");
    KM_HIP(hipEventSynchronize(ev.b), "event synchronize");
    float t = 0.f;
    KM_HIP(hipEventElapsedTime(&t, ev.a, ev.b), "event elapsed time");
    t *= 0.5f;
    if (best.pb == 0 || t < best_ms) best = cand[i], best_ms = t;
  }
  tune_record(dtype, D, N, B, K, best);
  if (pb) *pb = best.pb;
  if (waves) *waves = best.waves;
  if (ms) *ms = best_ms;
  return KM_OK;
}

int kmeans_update(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const int32_t* labels, int32_t K,
                  const float* C_prev, float* C_new, int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (!X || !labels || !C_prev || !C_new) return fail(KM_EINVAL, "X, labels, C_prev and C_new must be non-null");
  if (!aligned(X, 16) || !aligned(C_prev, 16) || !aligned(C_new, 16) || !aligned(labels, 4) || !aligned(counts, 4))
    return fail(KM_EINVAL, "misaligned pointer (X and the centroid buffers need 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  return run_update(X, dtype, N, D, B, labels, K, C_prev, C_new, counts, w, (hipStream_t)stream);
}

int kmeans_fit(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, const float* C0, int32_t K,
               int32_t iters, int32_t* labels, float* C_out, double* inertia, double* inertia_hist, void* ws,
               size_t ws_bytes, void* stream) {
  err_buf()[0] = 0;
  if (int rc = check_shape(dtype, N, D, K, B)) return rc;
  if (iters < 1) return fail(KM_EINVAL, "iters=%d must be >= 1", iters);
  if (!X || !C0 || !labels || !C_out || !inertia)
    return fail(KM_EINVAL, "X, C0, labels, C_out and inertia must be non-null");
  if (!aligned(X, 16) || !aligned(C0, 16) || !aligned(C_out, 16) || !aligned(labels, 4) || !aligned(inertia, 8) ||
      !aligned(inertia_hist, 8))
    return fail(KM_EINVAL, "misaligned pointer (X and the centroid buffers need 16 bytes)");
  const Layout L = make_layout(N, D, K, B, dtype);
  if (int rc = check_ws(ws, ws_bytes, L)) return rc;
  Work w = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  KM_HIP(hipGetDevice(&dev), "device query");
  const FitArgs a{X,     dtype,   N,            D,  B,        C0,  K,
                  iters, labels,  C_out,        inertia,      inertia_hist, ws,  ws_bytes,
                  dev,   assign_pick(dtype, D, N, B, K)};
  return graphs_enabled() ? fit_graph(a, w, s) : enqueue_fit(a, w, s);
}

const char* kmeans_last_error(void) { return err_buf(); }

}  // extern "C"
