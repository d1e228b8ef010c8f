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
// mask of lanes holding the same digit) and per-wave counters, so the output
// order is fully determined: equal keys keep their row order.  Histogram
// counts use LDS atomics (exact integers, so order-free).  No workgroup ever
// waits on another.
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
  cnt[t] = 0;
  __syncthreads();
  const int64_t tile = xcd_tile(blockIdx.x, nblk);
  const int64_t base = tile * kSortTile;
  uint32_t d[kIPT];
#pragma unroll
  for (int r = 0; r < kIPT; ++r) {
    const int64_t i = base + r * kT + t;
    d[r] = i < n ? (key(i) >> shift) & 255u : 256u;
  }
  // LDS atomics: the counts are exact integers, so their order is irrelevant
#pragma unroll
  for (int r = 0; r < kIPT; ++r)
    if (d[r] < 256u) atomicAdd(&cnt[d[r]], 1u);
  __syncthreads();
  hist[(int64_t)t * nblk + tile] = cnt[t];
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

// Stable scatter of one tile.  Each wave ranks a contiguous quarter of the
// tile (64 keys per round, in row order): a key's rank among equal digits of
// its wave = keys of that digit in the wave's earlier rounds (a per-wave LDS
// counter; LDS operations of one wave complete in order, so no barrier is
// needed between rounds) + equal digits in lower lanes.  One barrier later
// the per-wave counts become per-wave offsets, every key lands in an LDS copy
// of the tile sorted by digit, and the tile is written out digit run by digit
// run, so consecutive threads write consecutive addresses.
template <class KeyFn>
__global__ __launch_bounds__(kT) void radix_scatter_kernel(KeyFn key, const uint32_t* __restrict__ vals_in, int64_t n,
                                                           int shift, const uint32_t* __restrict__ hist,
                                                           const uint32_t* __restrict__ dtot, int64_t nblk,
                                                           uint32_t* __restrict__ keys_out,
                                                           uint32_t* __restrict__ vals_out) {
  constexpr int KW = kSortTile / 4;   // keys per wave
  constexpr int RW = KW / 64;         // rounds per wave
  __shared__ uint32_t lkey[kSortTile];
  __shared__ uint32_t lval[kSortTile];
  __shared__ uint32_t gbase[256];     // global position of LDS slot 0 of digit d's run, minus lstart[d]
  __shared__ uint32_t lstart[256];    // first LDS slot of digit d
  __shared__ uint32_t wcnt[4][256];   // per-wave digit counts, then per-wave offsets
  __shared__ uint32_t tmp[4];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int64_t blk = xcd_tile(blockIdx.x, nblk);  // the tile this workgroup sorts

  // this tile's count of digit t, from the scanned (exclusive) histogram row
  const uint32_t h0 = hist[(int64_t)t * nblk + blk];
  const uint32_t h1 = blk + 1 < nblk ? hist[(int64_t)t * nblk + blk + 1] : dtot[t];
  uint32_t tot;
  const uint32_t dpre = block_exclusive_scan_256(dtot[t], tmp, &tot);
  const uint32_t ls = block_exclusive_scan_256(h1 - h0, tmp, &tot);
  lstart[t] = ls;
  gbase[t] = dpre + h0 - ls;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) wcnt[ww][t] = 0;
  __syncthreads();

  const int64_t base = blk * kSortTile + (int64_t)w * KW;
  uint32_t kr[RW], vr[RW], rr[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t i = base + r * 64 + lane;
    const bool valid = i < n;
    kr[r] = valid ? key(i) : 0u;
    vr[r] = valid ? (vals_in ? vals_in[i] : (uint32_t)i) : 0u;
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t i = base + r * 64 + lane;
    const bool valid = i < n;
    const uint32_t d = (kr[r] >> shift) & 255u;
    const uint64_t m = match_digit(d, valid);
    const uint32_t lrank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    const uint32_t before = wcnt[w][d];
    rr[r] = before + lrank;
    if (valid && lrank == 0) wcnt[w][d] = before + (uint32_t)__popcll(m);
  }
  __syncthreads();
  {  // per-wave counts -> exclusive per-wave offsets (thread t owns digit t)
    uint32_t run = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const uint32_t c = wcnt[ww][t];
      wcnt[ww][t] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t i = base + r * 64 + lane;
    if (i < n) {
      const uint32_t d = (kr[r] >> shift) & 255u;
      const uint32_t slot = lstart[d] + wcnt[w][d] + rr[r];
      lkey[slot] = kr[r];
      lval[slot] = vr[r];
    }
  }
  __syncthreads();
  const int64_t rem = n - blk * kSortTile;
  const int cnt = rem < kSortTile ? (int)rem : kSortTile;
  for (int i = t; i < cnt; i += kT) {
    const uint32_t k = lkey[i];
    const uint32_t pos = gbase[(k >> shift) & 255u] + (uint32_t)i;
    keys_out[pos] = k;
    vals_out[pos] = lval[i];
  }
}

// off[k] for every k in [0, nseg]: row i writes the offsets of the keys in
// (key[i-1], key[i]]; the last row also closes (key[n-1], nseg].  Keys that
// no row carries are empty clusters: when `counts` is given they get count 0
// and keep their previous centroid (C_new[k] = C_prev[k]).
__global__ __launch_bounds__(kT) void segment_offsets_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                             uint32_t nseg, int32_t* __restrict__ off,
                                                             EmptyOut eo) {
  // four consecutive rows per thread (one 16-byte key load; the buffer is
  // 256-byte aligned and i0 is a multiple of 4)
  const int64_t i0 = ((int64_t)blockIdx.x * kT + threadIdx.x) * 4;
  if (i0 >= n) return;
  auto clampk = [&](uint32_t v) -> int64_t { return v < nseg ? (int64_t)v : (int64_t)nseg; };
  uint32_t kv[4];
  if (i0 + 3 < n) {
    const uint4 q = *reinterpret_cast<const uint4*>(keys + i0);
    kv[0] = q.x, kv[1] = q.y, kv[2] = q.z, kv[3] = q.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) kv[j] = i0 + j < n ? keys[i0 + j] : 0u;
  }
  auto empty = [&](int64_t kk) {
    eo.counts[kk] = 0;
    if (eo.C_new != eo.C_prev) {  // D is a multiple of 4: copy the row as float4
      const float4* src = reinterpret_cast<const float4*>(eo.C_prev + kk * eo.D);
      float4* dst = reinterpret_cast<float4*>(eo.C_new + kk * eo.D);
#pragma unroll 8
      for (int d = 0; d < eo.D / 4; ++d) dst[d] = src[d];
    }
  };
  int64_t kp = i0 == 0 ? -1 : clampk(keys[i0 - 1]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = i0 + j;
    if (i >= n) break;
    const int64_t k = clampk(kv[j]);
    for (int64_t kk = kp + 1; kk <= k; ++kk) off[kk] = (int32_t)i;
    if (eo.counts)
      for (int64_t kk = kp + 1; kk < k; ++kk) empty(kk);
    if (i == n - 1) {
      for (int64_t kk = k + 1; kk <= (int64_t)nseg; ++kk) off[kk] = (int32_t)n;
      if (eo.counts)
        for (int64_t kk = k + 1; kk < (int64_t)nseg; ++kk) empty(kk);
    }
    kp = k;
  }
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
                                  const EmptyOut& eo, hipStream_t s) {
  const int64_t grid = (n + 4 * kT - 1) / (4 * kT);
  segment_offsets_kernel<<<dim3((unsigned)grid), dim3(kT), 0, s>>>(sorted_keys, n, nseg, off, eo);
  return hipGetLastError();
}

}  // namespace fkm
