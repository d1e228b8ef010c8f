/*
 * flashkm.h — C ABI of the MI355X (gfx950) exact Lloyd k-means library.
 *
 * The operations follow "Flash-KMeans: Fast and Memory-Efficient Exact
 * K-Means" (paper page, abstract) and the article "Hacker Newsが捉えた
 * Flash-KMeans、Exact K-MeansをGPUのonline primitiveへ" (section
 * "Flash-KMeans が変える点"):
 *   - an assignment stage that fuses the point-to-centroid distance
 *     computation with a running argmin, so no N x K distance matrix is ever
 *     written to memory (FlashAssign);
 *   - a centroid update stage that first builds the cluster-sorted inverse
 *     mapping of the labels and then reduces each cluster's contiguous
 *     segment of points, with no global atomics (sort-inverse update);
 *   - chunked streaming of a host-resident point set that overlaps the
 *     host-to-device copies with compute (chunked-stream overlap).
 * The iteration itself is the unchanged, exact Lloyd iteration.
 *
 * Conventions shared by every entry point
 *   Shapes: X is [B, N, D] row-major (B independent instances of N points;
 *     B = 1 is the plain unbatched problem).  Centroids are [B, K, D] fp32
 *     row-major.  Labels are [B, N] int32 with values in [0, K) local to the
 *     instance.  Counts are [B, K] int32.  Inertia is [B] fp64.
 *   dtype (km_dtype) is the storage type of X.  Assignment uses the
 *     centroids rounded to nearest-even into that type (the fp32 centroid
 *     state itself is never rounded); squared centroid norms come from the
 *     rounded values; accumulation is fp32.  Ties go to the lowest index.
 *   Supported D: 16, 32, 64, 128, 256.  1 <= K <= N, B >= 1, B*N < 2^31.
 *   In-core pointers are DEVICE pointers (hipMalloc / torch CUDA tensors),
 *     contiguous; X, and the centroid buffers of kmeans_update and
 *     kmeans_fit (C_prev, C_new, C0, C_out), must be 16-byte aligned,
 *     everything else naturally aligned.  The caller owns every buffer.
 *     The in-core entry points never allocate or free memory: scratch space
 *     comes from the caller's workspace `ws` of at least
 *     kmeans_workspace_bytes(...) bytes.
 *   stream is a hipStream_t passed as void* (NULL = the null stream).
 *     In-core calls only enqueue work on it; results are valid once the
 *     stream has been synchronised.  Calls that share a workspace must be
 *     ordered on one stream.
 *   Errors: arguments are validated before anything is enqueued; on any
 *     failure the call returns a non-zero km_status, enqueues nothing (for
 *     validation errors) and kmeans_last_error() describes it.  HIP launch
 *     or API failures return KM_EHIP.  Device-side faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI and
 *     the library prints nothing.  Non-finite inputs give unspecified labels
 *     and centroids (memory safety is kept).
 *   Determinism: identical inputs on the same device give bitwise identical
 *     outputs; no result depends on atomics or scheduling order.
 */
#ifndef FLASHKM_H
#define FLASHKM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KM_API __attribute__((visibility("default")))
#else
#define KM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KM_F32 = 0, KM_F16 = 1, KM_BF16 = 2 } km_dtype;

typedef enum {
  KM_OK = 0,
  KM_EINVAL = 1,       /* bad argument (null pointer, K > N, iters < 1, ...) */
  KM_EUNSUPPORTED = 2, /* unsupported D or dtype                            */
  KM_EWORKSPACE = 3,   /* workspace smaller than kmeans_workspace_bytes()   */
  KM_EHIP = 4,         /* a HIP runtime call or kernel launch failed        */
  KM_ENOMEM = 5        /* kmeans_fit_streamed could not allocate its slots  */
} km_status;

/* Bytes of device workspace the in-core entry points need for this shape.
 * Returns 0 for an invalid or unsupported shape.  The same workspace serves
 * kmeans_assign, kmeans_update and kmeans_fit. */
KM_API size_t kmeans_workspace_bytes(int64_t N, int32_t D, int32_t K, int32_t B, int32_t dtype);

/* Assignment stage (FlashAssign; paper page abstract, "assignment stage";
 * article section "Flash-KMeans が変える点", first point).
 *   labels[b,i]  = argmin_k || x_bi - round(C_bk) ||^2   (lowest k on ties)
 *   min_d2[b,i]  = that minimum squared distance (fp32)   [nullable]
 *   inertia[b]   = sum_i min_d2[b,i], accumulated in fp64 [nullable]
 * X [B,N,D] dtype; C [B,K,D] fp32; labels [B,N] int32 (required). */
KM_API int kmeans_assign(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                  const float* C, int32_t K,
                  int32_t* labels, float* min_d2, double* inertia,
                  void* ws, size_t ws_bytes, void* stream);

/* The assignment stage for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): kmeans_assign with the same arguments and results, minus the
 * workspace.  Its scratch is a 32 MiB array inside the library, one per
 * GPU, held from the library's load until the process ends: the rounded
 * centroids (B*K*D*sizeof(dtype) bytes), their biases (B*ceil(K/256)*1 KiB)
 * and the per-wave inertia partials ((B*ceil(N/32) + 8)*8 bytes), each
 * rounded up to 256 bytes.  A shape that needs more is rejected with
 * KM_EWORKSPACE before anything is enqueued.  Nothing is allocated or freed.
 * Every call on one GPU uses that GPU's single array: calls that overlap on
 * one GPU (different streams or threads without ordering) race and give
 * unspecified results.  Every region a call reads is written earlier in the
 * same call, so no clearing is needed between calls.  Asynchronous. */
KM_API int kmeans_assign_noalloc(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                                 const float* C, int32_t K,
                                 int32_t* labels, float* min_d2, double* inertia, void* stream);

/* Centroid update stage (sort-inverse update; paper page abstract, "centroid
 * update stage"; article section "Flash-KMeans が変える点", second point).
 *   counts[b,k] = #{i : labels[b,i] = k}
 *   C_new[b,k]  = (1/counts) * sum_{i: labels[b,i]=k} x_bi     if counts > 0
 *               = C_prev[b,k]                                 otherwise
 * Sums are fp32 within fixed chunks of the cluster-sorted order and fp64
 * across chunks; each mean is rounded once to fp32 (an fp32 division for a
 * cluster inside one chunk, an fp64 one otherwise).  C_new may alias C_prev.
 * Labels outside [0,K) are a caller error: results are unspecified but every
 * memory access stays in bounds. */
KM_API int kmeans_update(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                  const int32_t* labels, int32_t K,
                  const float* C_prev, float* C_new, int32_t* counts,
                  void* ws, size_t ws_bytes, void* stream);

/* The exact Lloyd iteration (paper page abstract; article section 論文の要点):
 * exactly `iters` rounds of assign-then-update starting from C0.
 * Returns labels and inertia of the LAST assignment, and C_out = the
 * centroids after the LAST update.  inertia [B] fp64 device (required);
 * inertia_hist [iters, B] fp64 device (nullable) receives every round's
 * inertia.  C_out may alias C0.  Resuming is fit(X, C_t, iters - t).
 * Every round equals one kmeans_assign followed by one kmeans_update bit for
 * bit (internally the inertia sum and the next round's centroid preparation
 * ride along with the update's kernels).
 * The first call with a given argument list (pointers, sizes, iters, device,
 * and the assignment tile configuration chosen for the shape at the time of
 * the call, see kmeans_tune) captures the whole fit into a HIP graph; later
 * calls with the same list replay it with one graph launch (the last 8 lists
 * are kept; the buffers' contents may change between calls).  Results are
 * identical to direct launches, which the environment variable
 * FLASHKM_FIT_GRAPH=0 selects. */
KM_API int kmeans_fit(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
               const float* C0, int32_t K, int32_t iters,
               int32_t* labels, float* C_out, double* inertia, double* inertia_hist,
               void* ws, size_t ws_bytes, void* stream);

/* Out-of-core Lloyd iteration (chunked-stream overlap; paper page abstract;
 * article section "Flash-KMeans が変える点", third point).  B = 1.
 *   X_host         [N,D] dtype in PAGE-LOCKED host memory (hipHostMalloc or
 *                  a pinned torch tensor); it never has to fit on the device.
 *   C0, C_out      [K,D] fp32 DEVICE pointers (may alias).
 *   labels_host    [N] int32 host memory (pinned recommended).
 *   inertia_host   [1] fp64 host; inertia_hist_host [iters] fp64 host or NULL.
 *   device_x_budget  bytes of device memory the point chunks may occupy
 *                  (two slots of half the budget each).
 * Same results as kmeans_fit for labels and inertia of a given centroid
 * state; centroid sums are combined chunk by chunk in fp64 (in chunk order),
 * so centroids agree with the in-core path to rounding.  Synchronous: all
 * outputs are final on return.  This entry point allocates (and frees) its
 * own device slots and workspace; KM_ENOMEM if that fails. */
KM_API int kmeans_fit_streamed(const void* X_host, int32_t dtype, int64_t N, int32_t D,
                        const float* C0, int32_t K, int32_t iters, size_t device_x_budget,
                        int32_t* labels_host, float* C_out, double* inertia_host,
                        double* inertia_hist_host, void* stream);

/* Per-chunk timeline of the last kmeans_fit_streamed call on the calling
 * thread, to show the copy / compute overlap (article section "Flash-KMeans
 * が変える点", third point).  One row of 8 doubles per chunk and iteration,
 * in issue order: iteration, chunk, then the start and end (ms, relative to
 * the fit's first event, from HIP events recorded on the copy and compute
 * streams) of the chunk's host-to-device copy, of its compute (assign, sort,
 * segment sums) and of its labels' device-to-host copy (only the last
 * iteration copies labels; earlier iterations' windows are empty).  The first
 * min(cap, *count) rows go to `rows` (host, nullable when cap = 0) and
 * *count receives their number (0 if no streamed fit ran on this thread, or
 * if it had more than 16,384 chunk iterations, which record no timeline).
 * Does not touch the GPU. */
KM_API int kmeans_stream_timeline(double* rows, int32_t cap, int32_t* count);

/* Multi-assignment epilogue (the "Flash-GMM: A Memory-Efficient Kernel for
 * Scalable Soft Clustering" page, abstract: border vectors assigned to more
 * than one cluster).  The assignment kernel with a top-2 running state:
 *   labels2[b,i,0..1] = the two smallest (d_ik, k) pairs, d_ik the squared
 *                       distance to the dtype-rounded centroid (exact ties:
 *                       lower index first),
 *   d2[b,i,0..1]      = those two distances, computed directly (nullable).
 * Needs K >= 2.  Arguments otherwise as kmeans_assign; asynchronous. */
KM_API int kmeans_assign_top2(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                              const float* C, int32_t K, int32_t* labels2, float* d2,
                              void* ws, size_t ws_bytes, void* stream);

/* Soft-assignment epilogue (same page, abstract: Gaussian-mixture soft
 * clustering in one pass without materialising the N x K responsibility
 * matrix).  Components are isotropic with the shared variance sigma2 > 0,
 * centred at the dtype-rounded centroids, with log-weights log_w [B,K] fp32
 * (NULL = all zero); the constant (2 pi sigma2)^(-D/2) is left out.  With
 * a_ik = log_w_k - ||x_i - c_k||^2 / (2 sigma2):
 *   log_density[b,i] = log sum_k exp(a_ik)          (fp32; responsibilities
 *                      are r_ik = exp(a_ik - log_density[b,i])),
 *   labels[b,i]      = the most responsible component (lowest k on ties),
 *   total[b]         = sum_i log_density[b,i] in fp64 (nullable).
 * The kernel keeps a running maximum and a running sum of exponentials per
 * point (base 2, fp32) and anchors the result on the directly computed
 * distance of the most responsible centroid.  Asynchronous. */
KM_API int kmeans_assign_soft(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                              const float* C, int32_t K, const float* log_w, float sigma2,
                              int32_t* labels, float* log_density, double* total,
                              void* ws, size_t ws_bytes, void* stream);

/* Gauss kernel sums with the same fused tile ("Fast Gauss Sums via Flash
 * Attention" page, abstract: Gaussian kernel sums with arbitrary signed
 * weights; the FlashDiffusion card on the same listing, abstract: dense
 * Gaussian kernel blocks evaluated in fused tiles, never materialised).
 *   gsum[b,i] = sum_k w[b,k] exp(-||x_bi - y_bk||^2 / (2 sigma2))   (fp32)
 *   total[b]  = sum_i gsum[b,i] in fp64 (nullable)
 * X [B,N,D] dtype (targets), Y [B,K,D] fp32 sources rounded to dtype like
 * centroids, w [B,K] fp32 weights of any sign, sigma2 > 0; K <= N as for the
 * assignment.  The kernel keeps a running maximum score and the signed sum
 * sum_k w_k 2^(t_k - t_max) per target, anchored on the direct distance of
 * the nearest source.  Asynchronous. */
KM_API int kmeans_gauss_sum(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                            const float* Y, int32_t K, const float* w, float sigma2,
                            float* gsum, double* total,
                            void* ws, size_t ws_bytes, void* stream);

/* Initial centroids on the device.  The pages name k-means++ seeding only
 * as outside the method's inner loop (article, section なぜ Hacker News の
 * スレッドが重要だったか); this is the standard D^2 sampling, driven by
 * uniforms the caller draws (u [B,K] fp64 in [0,1), device):
 *   method 0 (random):   idx[b,j] = floor(u[b,j] * N)            (with replacement)
 *   method 1 (k-means++): idx[b,0] = floor(u[b,0] * N); for j >= 1 idx[b,j] is
 *     the smallest row i with sum_{i'<=i} D2_bi' > u[b,j] * sum_i D2_bi, where
 *     D2_bi is row i's squared distance to its nearest earlier pick (fp32,
 *     computed directly; sums in fp64 in a fixed order); floor(u N) when all
 *     D2 are zero.
 *   C[b,j,:] = row idx[b,j] of X as fp32 (exact); d2 [B,N] fp32 (nullable)
 *   receives every row's squared distance to its nearest pick.
 * k-means++ is sequential in j: 2 kernel launches per pick, each streaming X
 * once.  Arguments otherwise as kmeans_assign; asynchronous.  Deterministic;
 * where the cumulative sum lies within rounding of u * sum, the pick may
 * differ from an exact-arithmetic one by that rounding. */
KM_API int kmeans_seed(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B, int32_t K,
                       int32_t method, const double* u, int32_t* idx, float* C, float* d2,
                       void* ws, size_t ws_bytes, void* stream);

/* Shape-keyed configuration of the assignment kernel, with a per-shape
 * tuning cache (the pages' point about configuration tuning under dynamic
 * shapes: paper page abstract and the article section "Flash-KMeans が変える
 * 点", third point, which avoids re-tuning for every new shape).
 * Assignment kernels are compiled ahead of time for a few tile
 * configurations per row size: pb point blocks of 32 per wave and `waves`
 * waves per workgroup.  Every configuration computes bit-identical labels
 * (the same products in the same order); they differ only in speed.  The
 * choice for a shape (dtype, D, N, B, K) is, in order: the environment
 * variable FLASHKM_ASSIGN_CONFIG="pb,waves" if compiled for the row size;
 * the tuning table's entry for exactly that shape; a built-in rule.
 *
 * kmeans_tune times every compiled configuration on this shape (prep once,
 * then per configuration one warm-up and two timed assign launches on
 * `stream`, HIP events), records the fastest in the process-wide table and
 * returns it in *pb / *waves with its time per launch in *ms (each output
 * nullable).  labels [B,N] receives a valid assignment.  Arguments as for
 * kmeans_assign.  Synchronous (waits on its events).
 *
 * kmeans_tune_save / kmeans_tune_load write / read the table as text, one
 * entry per line "dtype D N B K pb waves" ('#' starts a comment).  Loading
 * adds or replaces entries; a malformed line, an unsupported shape or a
 * configuration not compiled for the row size fails with KM_EINVAL (naming
 * the line) and adds nothing from that file.  FLASHKM_TUNE_CACHE=<path> loads
 * a table once, at the first configuration choice.  These two calls do not
 * touch the GPU.  The table is shared by all threads (internally locked). */
KM_API int kmeans_tune(const void* X, int32_t dtype, int64_t N, int32_t D, int32_t B,
                       const float* C, int32_t K, int32_t* labels,
                       void* ws, size_t ws_bytes, void* stream,
                       int32_t* pb, int32_t* waves, float* ms);
KM_API int kmeans_tune_save(const char* path);
/* The configurations compiled for rows of D elements of `dtype`, the set
 * kmeans_tune chooses from and a tuning-table line may name: the first
 * min(cap, *count) pairs go to pb[i], waves[i] (host arrays, nullable when
 * cap = 0) and *count receives their number.  KM_EUNSUPPORTED for a dtype or
 * D the library does not support.  Does not touch the GPU. */
KM_API int kmeans_assign_configs(int32_t dtype, int32_t D, int32_t* pb, int32_t* waves, int32_t cap,
                                 int32_t* count);
KM_API int kmeans_tune_load(const char* path);

/* Text of the last error set on the calling thread ("" if none). */
KM_API const char* kmeans_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHKM_H */
