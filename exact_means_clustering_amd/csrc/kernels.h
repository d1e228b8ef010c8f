// Host-side launchers for the k-means kernels (internal; the public ABI is
// include/flashkm.h).  Every launcher enqueues on `s` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkm {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

inline int dtype_size(int dt) { return dt == DT_F32 ? 4 : 2; }

// ---- assignment stage ------------------------------------------------------
// Tile configuration of the assign kernel: `pb` blocks of 32 points held in
// registers per wave, `waves` waves per workgroup sharing one LDS centroid
// tile.  A workgroup covers waves * 32 * pb points.
struct AssignConfig {
  int pb;
  int waves;
  int rows() const { return waves * 32 * pb; }
  // inertia partials per instance: one per wave and job of rows() points
  int64_t parts(int64_t N) const { return (N + rows() - 1) / rows() * waves; }
};
// Configuration for a shape (dtype, D, N per instance, B instances, K): the
// environment variable FLASHKM_ASSIGN_CONFIG="pb,waves" when that pair is
// compiled for the row size, else the tuning table's entry for the shape,
// else a built-in rule.
AssignConfig assign_pick(int dt, int D, int64_t N, int B, int K);
// Is `c` compiled for rows of D elements of dtype dt?
bool assign_config_compiled(int dt, int D, AssignConfig c);
// The configurations compiled for the row size (at most cap); returns the count.
int assign_configs(int dt, int D, AssignConfig* out, int cap);
// Tuning table (thread-safe): exact-shape lookup and record.
bool tune_lookup(int dt, int D, int64_t N, int B, int K, AssignConfig* cfg);
void tune_record(int dt, int D, int64_t N, int B, int K, AssignConfig cfg);
// Largest number of inertia partials per instance over every configuration
// (waves * ceil(N / (waves * 32 * pb)) <= ceil(N / 32) + 8).
inline int64_t assign_max_parts(int64_t N) { return (N + 31) / 32 + 8; }

// Centroid count padded for the bias array: a multiple of every assign tile.
__host__ __device__ inline int64_t kpad(int K) { return ((int64_t)K + 255) / 256 * 256; }
// Chat[b,k] = RNE(C[b,k] -> dtype) and hb[b * kpad(K) + k] = -0.5 * ||Chat[b,k]||^2
// for k < K; hb[b * kpad(K) + k] = -inf for K <= k < kpad(K).
// With log_w (soft assignment) the bias also carries sigma2 * log_w[b * K + k].
hipError_t launch_prep(int dt, int D, const float* C, void* Chat, float* hb, int64_t B, int K, hipStream_t s,
                       const float* log_w = nullptr, float sigma2 = 0.f);

// Fused distance + running argmin.  part[b * P + j * waves + w] receives wave
// w's fp64 sum of min_d2 over its points of job j (P = cfg.parts(N)).
hipError_t launch_assign(int dt, int D, AssignConfig cfg, const void* X, const void* Chat, const float* hb,
                         int64_t N, int K, int B, int32_t* labels, float* min_d2, double* part, hipStream_t s);

// Two nearest centroids of every point: labels2 [B,N,2] (nearer first, ties
// to the lower index), d2 [B,N,2] their direct squared distances (nullable).
hipError_t launch_assign_top2(int dt, int D, const void* X, const void* Chat, const float* hb, int64_t N, int K, int B,
                              int32_t* labels2, float* d2, hipStream_t s);
// Gaussian-mixture soft assignment (the bias must come from launch_prep with
// the log-weights and sigma2): labels = most responsible component, logp =
// log sum_k w_k exp(-||x - c_k||^2 / (2 sigma2)), part = per-workgroup sums.
struct SoftArgs {
  const float* log_w;  // [B,K] or null (all zero)
  float scale2;        // log2(e) / sigma2
  float inv2s2;        // 1 / (2 sigma2)
  const float* wpad;   // Gauss sums: weights [B, kpad(K)], zero past K
};
hipError_t launch_assign_soft(int dt, int D, const void* X, const void* Chat, const float* hb, int64_t N, int K, int B,
                              int32_t* labels, float* logp, double* part, SoftArgs soft, hipStream_t s);
// Gauss kernel sums gsum[b,i] = sum_k w_k exp(-||x - c_k||^2 / (2 sigma2)) (bias
// from launch_prep without log-weights; soft.wpad from launch_pad_weights);
// labels = nearest source, part = per-workgroup sums.
hipError_t launch_assign_gauss(int dt, int D, const void* X, const void* Chat, const float* hb, int64_t N, int K,
                               int B, int32_t* labels, float* gsum, double* part, SoftArgs soft, hipStream_t s);
// wpad[b * kpad(K) + k] = w[b * K + k] for k < K, 0 beyond.
hipError_t launch_pad_weights(const float* w, float* wpad, int64_t B, int K, hipStream_t s);
// Configuration of the top-2 and soft launches (rows per workgroup: rows()).
AssignConfig mode_config(int dt, int D);

// Runs the per-device queries an assign launch with `cfg` needs (grid size),
// without launching, so that later launches make no device query (for
// instance while a stream is being captured into a graph).
hipError_t assign_prime(int dt, int D, AssignConfig cfg);

// inertia[b] = sum_w part[b * nwg + w] in a fixed order (added to the old
// value when `accumulate`); also copied to hist[b] if non-null.
hipError_t launch_inertia_reduce(const double* part, int nwg, int B, double* inertia, double* hist,
                                 bool accumulate, hipStream_t s);
// The same reduction as extra blocks of another launch (inertia_reduce_block
// in common.h: one 256-thread workgroup per instance).
struct InertiaJob {
  const double* part = nullptr;  // [B, nwg] per-wave partials (null: no job)
  int nwg = 0;
  int B = 0;
  double* inertia = nullptr;     // [B]
  double* hist = nullptr;        // [B] copy, nullable
};

// ---- inverse mapping (stable LSD radix argsort) -------------------------------
constexpr int kSortTile = 4096;       // keys per sort workgroup
constexpr int kSortTileSmall = 1024;  // for small problems, so the sort grid still fills the chip
inline int sort_tile(int64_t n) { return n <= ((int64_t)1 << 21) ? kSortTileSmall : kSortTile; }
inline int64_t sort_blocks(int64_t n) { return (n + sort_tile(n) - 1) / sort_tile(n); }
// A pass whose scatter sums the per-tile counts itself, with no scan kernel,
// covers at most this many tiles (per segment, for a segmented pass).
constexpr int64_t kScanFreeTiles = 64;
// B > 1 instances with K <= 256 sort in one segmented pass (each instance by
// its label) when an instance spans at most kScanFreeTiles tiles and the
// per-instance tiles number at most twice the plain ones (tiles at least
// half full on average, so many tiny instances keep the plain passes and a
// histogram that grows with the keys, not with the instance count).
inline bool sort_segmented(int64_t N, int B, int K) {
  const int64_t ntb = (N + sort_tile(N * B) - 1) / sort_tile(N * B);
  return B > 1 && K <= 256 && ntb <= kScanFreeTiles && ntb * B <= 2 * sort_blocks(N * B);
}
// Tiles the sort's histogram must hold: a segmented pass tiles each
// instance separately, so its ragged tails can add up to B - 1 tiles.
inline int64_t sort_hist_tiles(int64_t N, int B, int K) {
  const int64_t plain = sort_blocks(N * B);
  const int64_t seg = sort_segmented(N, B, K) ? (N + sort_tile(N * B) - 1) / sort_tile(N * B) * B : 0;
  return plain > seg ? plain : seg;
}
// Bits of the sort key b*K + label (B*K distinct keys).
inline int sort_key_bits(int B, int K) {
  const uint64_t nseg = (uint64_t)B * (uint64_t)K;
  int bits = 1;
  while (bits < 32 && (1ull << bits) < nseg) ++bits;
  return bits;
}
// Keys of 9 to 11 bits that the segmented pass does not take are sorted in
// one pass with a digit that wide, on the small tiles, while the histogram
// (2^bits counts per tile) stays within 2^20 words: there the saved launches
// outweigh the wider histogram, scan and scatter (measured: 4% faster at
// 2^20 keys with 10 bits, 15-20% at 2^15 to 2^18 keys; 32% slower at 2^21
// keys with 11 bits).  Returns the digit bits, or 0.
constexpr int kSortWideBits = 11;
inline int sort_wide_bits(int64_t N, int B, int K) {
  const int bits = sort_key_bits(B, K);
  const bool fits = bits > 8 && bits <= kSortWideBits && sort_tile(N * B) == kSortTileSmall &&
                    ((int64_t)1 << bits) * sort_blocks(N * B) <= ((int64_t)1 << 20);
  return fits && !sort_segmented(N, B, K) ? bits : 0;
}
// Words of the sort's histogram: 256 per tile, or 2^bits per tile for a
// wide pass.
inline int64_t sort_hist_words(int64_t N, int B, int K) {
  const int64_t narrow = 256 * sort_hist_tiles(N, B, K);
  const int wb = sort_wide_bits(N, B, K);
  const int64_t wide = wb ? ((int64_t)1 << wb) * sort_blocks(N * B) : 0;
  return narrow > wide ? narrow : wide;
}

// Sort elements are (key, row) pairs packed in one 8-byte word, so a pass
// reads and writes each element with a single access (a two-pass sort below
// 2^24 rows keeps its intermediate as 4-byte words in the first half of kv[0]).
struct SortBuffers {
  uint2* kv[2];     // [n] each: ping-pong pair buffers
  uint32_t* hist;   // [hist_words], at least sort_hist_words(N, B, K) for the shape it was laid out for
  int64_t hist_words;  // capacity of hist: a call takes only a pass whose histogram fits
  uint32_t* dtot;   // [2^kSortWideBits] digit totals
};
// Sorts rows by key = b*K + clamp(labels[b*N+i], 0, K-1) (stable).  On return
// *sorted points at the buffer holding the sorted (key, row) pairs.
// `side` (nullable) is an inertia reduction that runs as extra blocks of the
// first pass's histogram launch.
hipError_t launch_argsort_labels(const int32_t* labels, int64_t N, int B, int K, SortBuffers& buf,
                                 const uint2** sorted, hipStream_t s, const InertiaJob* side = nullptr);

// ---- segment-local reductions ----------------------------------------------
#ifndef FKM_SEG_ROWS
constexpr int kSegRows = 512;    // rows of the sorted order per wave chunk (level 1)
#else
constexpr int kSegRows = FKM_SEG_ROWS;
#endif
constexpr int kSegRowsSmall = 128;  // chunk rows for small problems, so the level-1 grid still fills the chip
constexpr int kSegGroup = 8;        // level-1 chunks per level-2 group
// Rows per level-1 chunk for n sorted rows.
static_assert((kSegRows & (kSegRows - 1)) == 0 && (kSegRowsSmall & (kSegRowsSmall - 1)) == 0 &&
                  (kSegGroup & (kSegGroup - 1)) == 0,
              "segment units are powers of two (levels 2 and 3 divide by shifting)");
inline int seg_rows(int64_t n) { return n <= ((int64_t)1 << 21) ? kSegRowsSmall : kSegRows; }
inline int64_t seg_chunks(int64_t n) { return (n + seg_rows(n) - 1) / seg_rows(n); }
inline int64_t seg_groups(int64_t n) { return (seg_chunks(n) + kSegGroup - 1) / kSegGroup; }

struct SegBuffers {
  float* frag;     // [nchunks * 2 * D] fp32
  double* gfrag;   // [ngroups * 2 * D] fp64
};
// Where each finished segment goes.  Means mode (S_acc == nullptr):
// C_new[k] = segment sum / count, counts[k] = count, and an empty segment
// copies C_prev[k] with count 0.  Accumulate mode (S_acc != nullptr):
// S_acc[k] += segment sum (fp64) and n_acc[k] += count; empty segments are
// left alone.  Every segment is finished by exactly one wave, so neither
// mode needs atomics.
struct SegOut {
  const float* C_prev;
  float* C_new;
  int32_t* counts;
  double* S_acc;
  int64_t* n_acc;
  // Means mode, optional: the assignment's centroid preparation fused into
  // the update.  Every cluster with rows also gets chat[k] = RNE(C_new[k])
  // in the input type and hb[b * Kp + l] = -0.5 ||chat[k]||^2 for key
  // k = b * K + l, exactly as launch_prep computes them; an empty cluster
  // keeps C_prev, so its entries (already prepared from C_prev) stay.
  void* chat = nullptr;
  float* hb = nullptr;
  uint32_t K = 0, Kp = 0;
};
// Also writes the segment offsets off[k] = #{rows with key < k}, k in [0, nseg].
hipError_t launch_segment_reduce(int dt, int D, const void* X, const uint2* sorted, int32_t* off, int64_t n,
                                 uint32_t nseg, const SegOut& out, SegBuffers& buf, hipStream_t s);

// ---- seeding ------------------------------------------------------------------
// Initial centroids of B instances: method 0 = rows floor(u N); method 1 =
// k-means++ D^2 sampling driven by u [B,K] (fp64 uniforms in [0,1)).  idx
// [B,K] the chosen rows, C [B,K,D] those rows in fp32.  d2_scratch [B,N]
// fp32 and part [B, ceil(N/256)] fp64 are scratch; d2_out [B,N] (nullable)
// receives each row's squared distance to its nearest pick.
hipError_t launch_seed(int dt, int D, const void* X, int64_t N, int B, int K, int method, const double* u,
                       int32_t* idx, float* C, float* d2_scratch, double* part, float* d2_out, hipStream_t s);

// ---- streamed path helpers ---------------------------------------------------
// C_new[k] = S[k] / n[k] (fp64 divide, rounded once to fp32) when n[k] > 0,
// else C_prev[k]; counts are not produced.
hipError_t launch_mean_from_sums(const double* S, const int64_t* n, int D, int64_t K, const float* C_prev,
                                 float* C_new, hipStream_t s);
hipError_t launch_zero_bytes(void* p, size_t bytes, hipStream_t s);

}  // namespace fkm
