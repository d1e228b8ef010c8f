// Out-of-core Lloyd iteration: chunked-stream overlap (Flash-KMeans paper page,
// abstract; article section "Flash-KMeans が変える点", third point: when the
// points do not fit in device memory, the host-to-device transfer of the
// next chunk overlaps the computation on the current one).
//
// Two device slots hold point chunks.  A copy stream moves chunk c+1 into
// its slot while the compute stream assigns chunk c, sorts its labels and
// adds its per-cluster sums into fp64 accumulators (chunk order fixed, so the
// result is deterministic).  Labels of each chunk go back to the host on the
// copy stream (in the last iteration, whose labels are the result).  After
// the last chunk of an iteration the means are formed once from the fp64
// sums.
#include "kernels.h"
#include "workspace.h"

#include "flashkm.h"

#include <vector>

using namespace fkm;

namespace {

// Per-chunk timeline of the last streamed fit on this thread: rows of
// kTimelineCols doubles (iteration, chunk, then the start and end in ms,
// relative to the fit's first event, of the chunk's host-to-device copy,
// of its compute and of its labels' device-to-host copy).
constexpr int kTimelineCols = 8;
constexpr int64_t kTimelineMaxChunks = 16384;  // longer fits record no timeline
std::vector<double>& timeline() {
  static thread_local std::vector<double> t;
  return t;
}

struct Res {
  hipStream_t cs = nullptr, xs = nullptr;
  hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
  std::vector<hipEvent_t> marks;  // timing events of the timeline (origin first, then 6 per chunk)
  void* dev[16] = {};
  int ndev = 0;
  void* alloc(size_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes < 256 ? 256 : bytes) != hipSuccess) return nullptr;
    dev[ndev++] = p;
    return p;
  }
  ~Res() {
    if (cs) (void)hipStreamSynchronize(cs);
    if (xs) (void)hipStreamSynchronize(xs);
    for (int i = 0; i < ndev; ++i) (void)hipFree(dev[i]);
    for (int i = 0; i < 2; ++i) {
      if (copied[i]) (void)hipEventDestroy(copied[i]);
      if (done[i]) (void)hipEventDestroy(done[i]);
      if (freed[i]) (void)hipEventDestroy(freed[i]);
    }
    for (hipEvent_t e : marks) (void)hipEventDestroy(e);
    if (cs) (void)hipStreamDestroy(cs);
    if (xs) (void)hipStreamDestroy(xs);
  }
};

int bad(int code, const char* msg) { return fail(code, "%s", msg); }

}  // namespace

#define KS_HIP(expr, what)                                                             \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) {                                                            \
      char m_[256];                                                                    \
      snprintf(m_, sizeof(m_), "%s: %s", what, hipGetErrorString(e_));                 \
      return bad(KM_EHIP, m_);                                           \
    }                                                                                  \
  } while (0)

extern "C" int kmeans_fit_streamed(const void* X_host, int32_t dtype, int64_t N, int32_t D, const float* C0,
                                   int32_t K, int32_t iters, size_t device_x_budget, int32_t* labels_host,
                                   float* C_out, double* inertia_host, double* inertia_hist_host, void* stream) {
  err_buf()[0] = 0;
  if (dtype != KM_F32 && dtype != KM_F16 && dtype != KM_BF16) return bad(KM_EUNSUPPORTED, "unsupported dtype");
  if (!(D == 16 || D == 32 || D == 64 || D == 128 || D == 256))
    return bad(KM_EUNSUPPORTED, "unsupported D (supported: 16, 32, 64, 128, 256)");
  if (K < 1 || N < K) return bad(KM_EINVAL, "need 1 <= K <= N");
  if (iters < 1) return bad(KM_EINVAL, "iters must be >= 1");
  if (!X_host || !C0 || !labels_host || !C_out || !inertia_host)
    return bad(KM_EINVAL, "X_host, C0, labels_host, C_out and inertia_host must be non-null");
  if (((uintptr_t)X_host & 15) != 0) return bad(KM_EINVAL, "X_host must be 16-byte aligned");
  {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, X_host) != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return bad(KM_EINVAL, "X_host must be page-locked host memory (hipHostMalloc / pinned tensor)");
    }
  }
  const int sz = dtype_size(dtype);
  const size_t row_bytes = (size_t)D * sz;
  int64_t chunk = (int64_t)(device_x_budget / 2 / row_bytes);
  if (chunk > ((int64_t)1 << 30)) chunk = (int64_t)1 << 30;
  if (chunk < 1) return bad(KM_EINVAL, "device_x_budget is smaller than two rows");
  if (chunk > N) chunk = N;
  const int64_t nch = (N + chunk - 1) / chunk;

  Res r;
  timeline().clear();
  KS_HIP(hipStreamSynchronize((hipStream_t)stream), "caller stream sync");
  KS_HIP(hipStreamCreateWithFlags(&r.cs, hipStreamNonBlocking), "stream create");
  KS_HIP(hipStreamCreateWithFlags(&r.xs, hipStreamNonBlocking), "stream create");
  for (int i = 0; i < 2; ++i) {
    KS_HIP(hipEventCreateWithFlags(&r.copied[i], hipEventDisableTiming), "event create");
    KS_HIP(hipEventCreateWithFlags(&r.done[i], hipEventDisableTiming), "event create");
    KS_HIP(hipEventCreateWithFlags(&r.freed[i], hipEventDisableTiming), "event create");
  }

  // device buffers
  void* xslot[2];
  int32_t* lslot[2];
  for (int i = 0; i < 2; ++i) {
    xslot[i] = r.alloc(al256((size_t)chunk * row_bytes));
    lslot[i] = (int32_t*)r.alloc(al256((size_t)chunk * 4));
    if (!xslot[i] || !lslot[i]) return bad(KM_ENOMEM, "device slot allocation failed");
  }
  // Every chunk but the last has `chunk` rows.  The workspace is laid out
  // for each of the two row counts (sort tiles and segment chunks change
  // size at 2^21 rows, so a layout for more rows need not cover fewer) in
  // one allocation of the larger size; a chunk uses its own layout.  The
  // stages of one chunk run in order on the compute stream, so the two
  // carvings never hold live data at once, and the centroid preparation
  // sits at the same offsets in both.
  const int64_t last = N - (nch - 1) * chunk;
  const Layout LF = make_layout(chunk, D, K, 1, dtype), LL = make_layout(last, D, K, 1, dtype);
  const size_t ws_bytes = LF.total > LL.total ? LF.total : LL.total;
  void* ws = r.alloc(ws_bytes);
  double* S_acc = (double*)r.alloc((size_t)K * D * 8);
  int64_t* n_acc = (int64_t*)r.alloc((size_t)K * 8);
  double* J_dev = (double*)r.alloc((size_t)iters * 8);
  if (!ws || !S_acc || !n_acc || !J_dev) return bad(KM_ENOMEM, "device workspace allocation failed");

  Work wf = carve(ws, LF), wl = carve(ws, LL);
  Work& w = wf;  // centroid preparation and partials: same offsets in both layouts

  const char* xh = (const char*)X_host;
  // timeline marks: an origin, then per chunk the copy in, the compute and
  // the labels' copy out, each bracketed by two timing events on its stream
  const bool record = (int64_t)iters * nch <= kTimelineMaxChunks;
  auto mark = [&](hipStream_t st) -> int {
    if (!record) return KM_OK;
    hipEvent_t e = nullptr;
    KS_HIP(hipEventCreate(&e), "event create");
    r.marks.push_back(e);
    KS_HIP(hipEventRecord(e, st), "event record");
    return KM_OK;
  };
  if (int rc = mark(r.xs)) return rc;
  // both slots start free
  for (int i = 0; i < 2; ++i) KS_HIP(hipEventRecord(r.freed[i], r.xs), "event record");

  for (int t = 0; t < iters; ++t) {
    const float* Cs = t == 0 ? C0 : C_out;
    KS_HIP(launch_prep(dtype, D, Cs, w.chat, w.hb, 1, K, r.cs), "centroid prep launch");
    KS_HIP(launch_zero_bytes(S_acc, (size_t)K * D * 8, r.cs), "zero launch");
    KS_HIP(launch_zero_bytes(n_acc, (size_t)K * 8, r.cs), "zero launch");
    KS_HIP(launch_zero_bytes(J_dev + t, 8, r.cs), "zero launch");

    auto h2d = [&](int64_t c) -> int {
      const int sl = (int)(c & 1);
      const int64_t rows = (c + 1) * chunk <= N ? chunk : N - c * chunk;
      KS_HIP(hipStreamWaitEvent(r.xs, r.freed[sl], 0), "stream wait");
      if (int rc = mark(r.xs)) return rc;
      KS_HIP(hipMemcpyAsync(xslot[sl], xh + (size_t)c * chunk * row_bytes, (size_t)rows * row_bytes,
                            hipMemcpyHostToDevice, r.xs),
             "H2D copy");
      if (int rc = mark(r.xs)) return rc;
      KS_HIP(hipEventRecord(r.copied[sl], r.xs), "event record");
      return KM_OK;
    };
    if (int rc = h2d(0)) return rc;
    for (int64_t c = 0; c < nch; ++c) {
      const int sl = (int)(c & 1);
      const int64_t rows = (c + 1) * chunk <= N ? chunk : N - c * chunk;
      Work& wc = rows == chunk ? wf : wl;
      if (c + 1 < nch)
        if (int rc = h2d(c + 1)) return rc;
      KS_HIP(hipStreamWaitEvent(r.cs, r.copied[sl], 0), "stream wait");
      if (int rc = mark(r.cs)) return rc;
      const AssignConfig cfg = assign_pick(dtype, D, rows, 1, K);
      KS_HIP(launch_assign(dtype, D, cfg, xslot[sl], wc.chat, wc.hb, rows, K, 1, lslot[sl], nullptr, wc.part, r.cs),
             "assign launch");
      KS_HIP(launch_inertia_reduce(wc.part, (int)cfg.parts(rows), 1, J_dev + t, nullptr, true, r.cs),
             "inertia launch");
      const uint2* sorted = nullptr;
      KS_HIP(launch_argsort_labels(lslot[sl], rows, 1, K, wc.sort, &sorted, r.cs), "argsort launch");
      SegOut so{nullptr, nullptr, nullptr, S_acc, n_acc};
      KS_HIP(launch_segment_reduce(dtype, D, xslot[sl], sorted, wc.off, rows, (uint32_t)K, so, wc.seg, r.cs),
             "segment reduce launch");
      if (int rc = mark(r.cs)) return rc;
      KS_HIP(hipEventRecord(r.done[sl], r.cs), "event record");
      KS_HIP(hipStreamWaitEvent(r.xs, r.done[sl], 0), "stream wait");
      if (int rc = mark(r.xs)) return rc;
      // only the last iteration's labels are returned, so earlier iterations
      // keep the copy stream for the points (their labels-out windows are empty)
      if (t == iters - 1)
        KS_HIP(hipMemcpyAsync(labels_host + c * chunk, lslot[sl], (size_t)rows * 4, hipMemcpyDeviceToHost, r.xs),
               "labels D2H copy");
      if (int rc = mark(r.xs)) return rc;
      KS_HIP(hipEventRecord(r.freed[sl], r.xs), "event record");
    }
    KS_HIP(launch_mean_from_sums(S_acc, n_acc, D, K, Cs, C_out, r.cs), "mean launch");
  }
  KS_HIP(hipStreamSynchronize(r.cs), "compute stream sync");
  KS_HIP(hipStreamSynchronize(r.xs), "copy stream sync");
  KS_HIP(hipMemcpy(inertia_host, J_dev + (iters - 1), 8, hipMemcpyDeviceToHost), "inertia copy");
  if (inertia_hist_host) KS_HIP(hipMemcpy(inertia_hist_host, J_dev, (size_t)iters * 8, hipMemcpyDeviceToHost), "inertia copy");
  if (record) {
    // marks: origin, then per chunk in issue order: the next chunk's copy in
    // (issued before this chunk's compute, except chunk 0 of an iteration,
    // issued first), compute start / end, labels out start / end
    std::vector<double>& tl = timeline();
    tl.assign((size_t)iters * nch * kTimelineCols, 0.0);
    size_t m = 1;
    auto ms = [&](size_t i, double* out) -> int {
      float v = 0.f;
      KS_HIP(hipEventElapsedTime(&v, r.marks[0], r.marks[i]), "event elapsed time");
      *out = v;
      return KM_OK;
    };
    for (int t = 0; t < iters; ++t) {
      for (int64_t c = 0; c < nch; ++c) {
        double* row = &tl[((size_t)t * nch + c) * kTimelineCols];
        row[0] = t;
        row[1] = (double)c;
      }
      // chunk 0's copy in, then per chunk: [chunk c+1's copy in], compute, labels out
      if (int rc = ms(m++, &tl[(size_t)t * nch * kTimelineCols + 2])) return rc;
      if (int rc = ms(m++, &tl[(size_t)t * nch * kTimelineCols + 3])) return rc;
      for (int64_t c = 0; c < nch; ++c) {
        double* row = &tl[((size_t)t * nch + c) * kTimelineCols];
        if (c + 1 < nch) {
          double* nxt = row + kTimelineCols;
          if (int rc = ms(m++, &nxt[2])) return rc;
          if (int rc = ms(m++, &nxt[3])) return rc;
        }
        for (int j = 4; j < 8; ++j)
          if (int rc = ms(m++, &row[j])) return rc;
      }
    }
  }
  return KM_OK;
}

extern "C" int kmeans_stream_timeline(double* rows, int32_t cap, int32_t* count) {
  err_buf()[0] = 0;
  if (!count || cap < 0 || (cap > 0 && !rows)) return bad(KM_EINVAL, "count must be non-null and rows hold cap rows");
  const std::vector<double>& tl = timeline();
  const int64_t n = (int64_t)tl.size() / kTimelineCols;
  for (int64_t i = 0; i < n && i < cap; ++i)
    for (int j = 0; j < kTimelineCols; ++j) rows[i * kTimelineCols + j] = tl[(size_t)i * kTimelineCols + j];
  *count = (int32_t)n;
  return KM_OK;
}
