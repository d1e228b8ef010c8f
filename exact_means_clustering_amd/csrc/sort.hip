// Inverse mapping for the sort-inverse update (Flash-KMeans paper page,
// abstract: the update first builds an explicit inverse mapping from clusters
// to their points; article section "Flash-KMeans が変える点", second point).
//
// A stable least-significant-digit radix argsort of the cluster keys
// (key = b*K + label) with 8-bit digits, then the segment offsets
// off[k] = #{rows with key < k}.  Each digit pass is reduce-then-scan:
//   hist    per-workgroup digit counts, stored digit-major [256][nblk];
//   scan    exclusive scan of each digit row, plus the digit totals;
//   scatter stable rank of every key inside its workgroup tile, written to
//           digit base + workgroup offset + rank.
// Ranks come from wave-level digit matching (eight ballots give each lane the
// mask of lanes holding the same digit), so there are no atomics on hot
// digits and the output order is fully determined: equal keys keep their row
// order.  No workgroup ever waits on another.
#include "common.h"
#include "kernels.h"

namespace fkm {

namespace {

constexpr int kT = 256;
constexpr int kIPT = kSortTile / kT;  // keys per thread per tile (16)

// Key of row i.  For the first pass keys come from the labels; later passes
// read the previous pass's output.
struct LabelKeys {
  const int32_t* labels;
  int64_t N;      // rows per instance
  uint32_t K;     // centroids per instance
  int B;          // instances
  double invN;    // 1.0 / N, for the instance index
  __device__ __forceinline__ uint32_t operator()(int64_t i) const {
    const int32_t l = labels[i];
    const uint32_t lab = (uint32_t)l < K ? (uint32_t)l : K - 1;  // out-of-range labels clamp (caller error)
    if (B == 1) return lab;
    // instance index i / N: a floating estimate corrected to the exact floor
    int64_t b = (int64_t)((double)i * invN);
    if ((b + 1) * N <= i) ++b;
    if (b * N > i) --b;
    return (uint32_t)b * K + lab;
  }
};
struct BufKeys {
  const uint32_t* keys;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const { return keys[i]; }
};

// Mask of the active lanes of this wave whose 8-bit digit equals mine.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = (d >> bit) & 1u;
    const uint64_t bb = __ballot(on);
    m &= on ? bb : ~bb;
  }
  return m;
}

template <class KeyFn>
__global__ __launch_bounds__(kT) void radix_hist_kernel(KeyFn key, int64_t n, int shift, uint32_t* __restrict__ hist,
                                                        int64_t nblk) {
  __shared__ uint32_t cnt[256];
  const int t = threadIdx.x;
  const int lane = t & 63;
  cnt[t] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll 4
  for (int r = 0; r < kIPT; ++r) {
    const int64_t i = base + r * kT + t;
    const bool valid = i < n;
    const uint32_t d = valid ? (key(i) >> shift) & 255u : 0u;
    const uint64_t m = match_digit(d, valid);
    // the lowest lane of each digit group adds the group size
    if (valid && (m & ((1ull << lane) - 1ull)) == 0) atomicAdd(&cnt[d], (uint32_t)__popcll(m));
  }
  __syncthreads();
  hist[(int64_t)t * nblk + blockIdx.x] = cnt[t];
}

// One workgroup per digit: exclusive scan of hist[d][0..nblk) in place,
// dtot[d] = row total.
__global__ __launch_bounds__(kT) void radix_scan_kernel(uint32_t* __restrict__ hist, int64_t nblk,
                                                        uint32_t* __restrict__ dtot) {
  __shared__ uint32_t tmp[4];
  uint32_t* row = hist + (int64_t)blockIdx.x * nblk;
  uint32_t running = 0;
  constexpr int PER = 4;
  for (int64_t c0 = 0; c0 < nblk; c0 += (int64_t)kT * PER) {
    uint32_t v[PER];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t i = c0 + (int64_t)threadIdx.x * PER + j;
      v[j] = i < nblk ? row[i] : 0u;
      s += v[j];
    }
    uint32_t tot;
    uint32_t pre = block_exclusive_scan_256(s, tmp, &tot);
    pre += running;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t i = c0 + (int64_t)threadIdx.x * PER + j;
      if (i < nblk) row[i] = pre;
      pre += v[j];
    }
    running += tot;
  }
  if (threadIdx.x == 0) dtot[blockIdx.x] = running;
}

template <class KeyFn>
__global__ __launch_bounds__(kT) void radix_scatter_kernel(KeyFn key, const uint32_t* __restrict__ vals_in, int64_t n,
                                                           int shift, const uint32_t* __restrict__ hist,
                                                           const uint32_t* __restrict__ dtot, int64_t nblk,
                                                           uint32_t* __restrict__ keys_out,
                                                           uint32_t* __restrict__ vals_out) {
  __shared__ uint32_t dbase[256];
  __shared__ uint32_t running[256];
  __shared__ uint32_t wc[2][4][256];  // per round parity, per wave, per digit: count | (round+1) << 16
  __shared__ uint32_t tmp[4];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;

  uint32_t tot;
  const uint32_t dpre = block_exclusive_scan_256(dtot[t], tmp, &tot);
  dbase[t] = dpre + hist[(int64_t)t * nblk + blockIdx.x];
  running[t] = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) wc[q][ww][t] = 0;
  __syncthreads();

  const int64_t base = (int64_t)blockIdx.x * kSortTile;
  for (int r = 0; r < kIPT; ++r) {
    const int64_t i = base + r * kT + t;
    const bool valid = i < n;
    const uint32_t k = valid ? key(i) : 0u;
    const uint32_t v = valid ? (vals_in ? vals_in[i] : (uint32_t)i) : 0u;
    const uint32_t d = (k >> shift) & 255u;
    const uint64_t m = match_digit(d, valid);
    const uint32_t lrank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    const uint32_t tag = (uint32_t)(r + 1) << 16;
    uint32_t(*wr)[256] = wc[r & 1];
    if (valid && lrank == 0) wr[w][d] = (uint32_t)__popcll(m) | tag;
    __syncthreads();
    if (valid) {
      uint32_t pre = 0;
      for (int ww = 0; ww < w; ++ww) {
        const uint32_t c = wr[ww][d];
        if ((c & 0xFFFF0000u) == tag) pre += c & 0xFFFFu;
      }
      const uint32_t pos = dbase[d] + running[d] + pre + lrank;
      keys_out[pos] = k;
      vals_out[pos] = v;
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const uint32_t c = wr[ww][t];
      if ((c & 0xFFFF0000u) == tag) add += c & 0xFFFFu;
    }
    running[t] += add;
    // the next round's first barrier orders this update before its reads
  }
}

__global__ __launch_bounds__(kT) void segment_offsets_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                             uint32_t nseg, int32_t* __restrict__ off) {
  const int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i >= n) return;
  const int64_t k = keys[i] < nseg ? (int64_t)keys[i] : (int64_t)nseg;
  const int64_t kp = i == 0 ? -1 : (keys[i - 1] < nseg ? (int64_t)keys[i - 1] : (int64_t)nseg);
  for (int64_t kk = kp + 1; kk <= k; ++kk) off[kk] = (int32_t)i;
  if (i == n - 1)
    for (int64_t kk = k + 1; kk <= (int64_t)nseg; ++kk) off[kk] = (int32_t)n;
}

template <class KeyFn>
hipError_t one_pass(KeyFn key, const uint32_t* vals_in, int64_t n, int shift, SortBuffers& buf, uint32_t* keys_out,
                    uint32_t* vals_out, hipStream_t s) {
  const int64_t nblk = sort_blocks(n);
  radix_hist_kernel<KeyFn><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(key, n, shift, buf.hist, nblk);
  radix_scan_kernel<<<dim3(256), dim3(kT), 0, s>>>(buf.hist, nblk, buf.dtot);
  radix_scatter_kernel<KeyFn><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(key, vals_in, n, shift, buf.hist, buf.dtot,
                                                                       nblk, keys_out, vals_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_argsort_labels(const int32_t* labels, int64_t N, int B, int K, SortBuffers& buf,
                                 const uint32_t** sorted_keys, const uint32_t** perm, hipStream_t s) {
  const int64_t n = N * (int64_t)B;
  const uint64_t nseg = (uint64_t)B * (uint64_t)K;
  int bits = 1;
  while (bits < 32 && (1ull << bits) < nseg) ++bits;
  const int passes = (bits + 7) / 8;
  LabelKeys lk{labels, N, (uint32_t)K, B, 1.0 / (double)N};
  hipError_t e = one_pass(lk, nullptr, n, 0, buf, buf.keys[0], buf.vals[0], s);
  if (e != hipSuccess) return e;
  int cur = 0;
  for (int p = 1; p < passes; ++p) {
    BufKeys bk{buf.keys[cur]};
    e = one_pass(bk, buf.vals[cur], n, 8 * p, buf, buf.keys[cur ^ 1], buf.vals[cur ^ 1], s);
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  *sorted_keys = buf.keys[cur];
  *perm = buf.vals[cur];
  return hipSuccess;
}

hipError_t launch_segment_offsets(const uint32_t* sorted_keys, int64_t n, uint32_t nseg, int32_t* off,
                                  hipStream_t s) {
  const int64_t grid = (n + kT - 1) / kT;
  segment_offsets_kernel<<<dim3((unsigned)grid), dim3(kT), 0, s>>>(sorted_keys, n, nseg, off);
  return hipGetLastError();
}

}  // namespace fkm
