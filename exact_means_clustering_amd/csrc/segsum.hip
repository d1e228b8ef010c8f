// Segment-local reductions of the sort-inverse update (Flash-KMeans paper
// page, abstract: scatters become segment-level localized reductions;
// article section "Flash-KMeans が変える点", second point: no atomic write
// contention on hot clusters).
//
// After the argsort, cluster k owns the contiguous sorted positions
// [off[k], off[k+1]).  The sorted order is cut into fixed chunks of kSegRows
// positions, one wave each:
//   level 1  a wave sums, per segment piece inside its chunk, the gathered
//            rows X[perm[j]] in fp32 (4 rows in flight per 64 lanes for
//            D*SZ = 256 B).  A segment that lies inside the chunk is finished
//            on the spot; the chunk's first / last piece of a segment that
//            crosses the chunk edge goes to fragment slot 0 / 1.
//   level 2  one wave per group of kSegGroup chunks adds (fp64) the chunk
//            fragments of every segment that crosses a chunk edge; segments
//            inside the group are finished, the others leave group fragments.
//   level 3  one wave per group finishes the segment (if any) that crosses
//            into the group from the left and ends inside it.
// Every segment is finished by exactly one wave in a fixed order, so the
// update is deterministic and uses no atomics.  Fragment slot rule (used to
// find a segment's piece in unit u of size U): the piece is in slot 1 iff u
// is the unit where the segment starts and the segment does not start on
// the unit boundary; otherwise slot 0.
#include "common.h"
#include "kernels.h"

namespace fkm {

namespace {

__device__ __forceinline__ int frag_slot(int64_t u, int64_t U, int64_t s) {
  return (u == s / U && s != u * U) ? 1 : 0;
}

// Finish a segment: means mode writes C_new / counts, accumulate mode adds
// into S_acc / n_acc.  `v` holds the segment sum for dims lane + 64*j.
template <int PER>
__device__ __forceinline__ void finish(const SegOut& o, int64_t k, int D, int lane, const double* v, int64_t cnt) {
  if (o.S_acc) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      if (d < D) o.S_acc[k * D + d] += v[j];
    }
    if (lane == 0) o.n_acc[k] += cnt;
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      if (d < D) o.C_new[k * D + d] = (float)(v[j] / (double)cnt);
    }
    if (lane == 0) o.counts[k] = (int32_t)cnt;
  }
}

// ---------------------------------------------------------------------------
// level 1: gather + fp32 sums per chunk
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void seg_level1_kernel(const typename T::raw* __restrict__ X,
                                                         const uint32_t* __restrict__ perm,
                                                         const uint32_t* __restrict__ keys,
                                                         const int32_t* __restrict__ off, int64_t n, SegOut o,
                                                         float* __restrict__ frag) {
  constexpr int VEC = Vec<T>::N;           // elements per 16-byte word
  constexpr int LPR = D * T::SZ / 16;      // lanes per row
  constexpr int SL = 64 / LPR;             // rows in flight per wave
  static_assert(LPR >= 1 && LPR <= 64, "row size");
  const int lane = lane_id();
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t r0 = c * kSegRows;
  if (r0 >= n) return;
  const int64_t r1 = r0 + kSegRows < n ? r0 + kSegRows : n;
  const int q = lane / LPR, g = lane % LPR;
  const int64_t kf = keys[r0], kl = keys[r1 - 1];

  for (int64_t k = kf; k <= kl; ++k) {
    const int64_t s = off[k], e = off[k + 1];
    const int64_t a = s > r0 ? s : r0;
    const int64_t z = e < r1 ? e : r1;
    if (a >= z) continue;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    int64_t j = a + q;
    // four rows per lane in flight
    for (; j + 3 * SL < z; j += 4 * SL) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t row = perm[j + u * SL];
        v[u] = reinterpret_cast<const uint4*>(X + (int64_t)row * D)[g];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float f[VEC];
        Vec<T>::unpack(v[u], f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += f[i];
      }
    }
    for (; j < z; j += SL) {
      const uint32_t row = perm[j];
      float f[VEC];
      Vec<T>::unpack(reinterpret_cast<const uint4*>(X + (int64_t)row * D)[g], f);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += f[i];
    }
    // combine the SL row slots (fixed butterfly order)
#pragma unroll
    for (int o2 = LPR; o2 < 64; o2 <<= 1)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += __shfl_xor(acc[i], o2);
    if (q == 0) {
      if (s >= r0 && e <= r1) {
        const int64_t cnt = e - s;
        if (o.S_acc) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) o.S_acc[k * D + g * VEC + i] += (double)acc[i];
          if (g == 0) o.n_acc[k] += cnt;
        } else {
          const float fc = (float)cnt;
#pragma unroll
          for (int i = 0; i < VEC; ++i) o.C_new[k * D + g * VEC + i] = acc[i] / fc;
          if (g == 0) o.counts[k] = (int32_t)cnt;
        }
      } else {
        const int slot = (k == kf) ? 0 : 1;
        float* fp = frag + (c * 2 + slot) * D + g * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) fp[i] = acc[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// level 2: per group of chunks, combine chunk fragments (fp64)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void seg_level2_kernel(const uint32_t* __restrict__ keys,
                                                         const int32_t* __restrict__ off, int64_t n, SegOut o,
                                                         const float* __restrict__ frag, double* __restrict__ gfrag) {
  constexpr int PER = (D + 63) / 64;
  constexpr int64_t U = kSegRows;
  constexpr int64_t UG = (int64_t)kSegRows * kSegGroup;
  const int lane = lane_id();
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t gr0 = g * UG;
  if (gr0 >= n) return;
  const int64_t gr1 = gr0 + UG < n ? gr0 + UG : n;
  const int64_t kf = keys[gr0], kl = keys[gr1 - 1];
  for (int64_t k = kf; k <= kl; ++k) {
    const int64_t s = off[k], e = off[k + 1];
    if (s >= e) continue;
    if (s / U == (e - 1) / U) continue;  // finished at level 1
    const int64_t a = s > gr0 ? s : gr0;
    const int64_t z = e < gr1 ? e : gr1;
    if (a >= z) continue;
    double acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.0;
    const int64_t u0 = a / U, u1 = (z - 1) / U;
#pragma unroll 4
    for (int64_t u = u0; u <= u1; ++u) {
      const float* fp = frag + (u * 2 + frag_slot(u, U, s)) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int d = lane + 64 * j;
        if (d < D) acc[j] += (double)fp[d];
      }
    }
    if (s >= gr0 && e <= gr1) {
      finish<PER>(o, k, D, lane, acc, e - s);
    } else {
      double* gp = gfrag + (g * 2 + ((k == kf) ? 0 : 1)) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int d = lane + 64 * j;
        if (d < D) gp[d] = acc[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// level 3: the segment crossing into group g from the left and ending in it
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void seg_level3_kernel(const uint32_t* __restrict__ keys,
                                                         const int32_t* __restrict__ off, int64_t n, SegOut o,
                                                         const double* __restrict__ gfrag) {
  constexpr int PER = (D + 63) / 64;
  constexpr int64_t UG = (int64_t)kSegRows * kSegGroup;
  __shared__ double part[4][PER * 64];
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int64_t g = blockIdx.x;
  const int64_t gr0 = g * UG;
  const int64_t gr1 = gr0 + UG < n ? gr0 + UG : n;
  const int64_t k = keys[gr0];
  const int64_t s = off[k], e = off[k + 1];
  if (!(s < gr0 && e <= gr1)) return;  // uniform over the workgroup
  // the four waves take interleaved groups; partials combine in a fixed order
  const int64_t g0 = s / UG;
  double acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0;
#pragma unroll 2
  for (int64_t gg = g0 + w; gg <= g; gg += 4) {
    const double* gp = gfrag + (gg * 2 + frag_slot(gg, UG, s)) * D;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      if (d < D) acc[j] += gp[d];
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) part[w][lane + 64 * j] = acc[j];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      acc[j] = (part[0][d] + part[1][d]) + (part[2][d] + part[3][d]);
    }
    finish<PER>(o, k, D, lane, acc, e - s);
  }
}

// empty segments: C_new[k] = C_prev[k], counts[k] = 0 (means mode only)
__global__ __launch_bounds__(256) void seg_empty_kernel(const int32_t* __restrict__ off, int64_t nseg, int D,
                                                        const float* __restrict__ C_prev, float* __restrict__ C_new,
                                                        int32_t* __restrict__ counts) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= nseg) return;
  if (off[k + 1] > off[k]) return;
  counts[k] = 0;
  if (C_new != C_prev)
    for (int d = 0; d < D; ++d) C_new[k * D + d] = C_prev[k * D + d];
}

__global__ __launch_bounds__(256) void mean_from_sums_kernel(const double* __restrict__ S,
                                                             const int64_t* __restrict__ cnt, int D, int64_t K,
                                                             const float* __restrict__ C_prev,
                                                             float* __restrict__ C_new) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= K * D) return;
  const int64_t k = i / D;
  C_new[i] = cnt[k] > 0 ? (float)(S[i] / (double)cnt[k]) : C_prev[i];
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t n16, uint8_t* __restrict__ tail,
                                                   int tail_bytes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
  if (i < tail_bytes) tail[i] = 0;
}

template <class T, int D>
hipError_t seg_reduce_t(const void* X, const uint32_t* perm, const uint32_t* keys, const int32_t* off, int64_t n,
                        uint32_t nseg, const SegOut& o, SegBuffers& buf, hipStream_t s) {
  const int64_t nchunks = seg_chunks(n);
  const int64_t ngroups = seg_groups(n);
  seg_level1_kernel<T, D><<<dim3((unsigned)((nchunks + 3) / 4)), dim3(256), 0, s>>>(
      reinterpret_cast<const typename T::raw*>(X), perm, keys, off, n, o, buf.frag);
  if (nchunks > 1) {
    seg_level2_kernel<D><<<dim3((unsigned)((ngroups + 3) / 4)), dim3(256), 0, s>>>(keys, off, n, o, buf.frag,
                                                                                  buf.gfrag);
    if (ngroups > 1) seg_level3_kernel<D><<<dim3((unsigned)ngroups), dim3(256), 0, s>>>(keys, off, n, o, buf.gfrag);
  }
  if (!o.S_acc)
    seg_empty_kernel<<<dim3((unsigned)((nseg + 255) / 256)), dim3(256), 0, s>>>(off, nseg, D, o.C_prev, o.C_new,
                                                                               o.counts);
  return hipGetLastError();
}

template <class T>
hipError_t seg_reduce_d(int D, const void* X, const uint32_t* perm, const uint32_t* keys, const int32_t* off,
                        int64_t n, uint32_t nseg, const SegOut& o, SegBuffers& buf, hipStream_t s) {
  switch (D) {
    case 16: return seg_reduce_t<T, 16>(X, perm, keys, off, n, nseg, o, buf, s);
    case 32: return seg_reduce_t<T, 32>(X, perm, keys, off, n, nseg, o, buf, s);
    case 64: return seg_reduce_t<T, 64>(X, perm, keys, off, n, nseg, o, buf, s);
    case 128: return seg_reduce_t<T, 128>(X, perm, keys, off, n, nseg, o, buf, s);
    case 256: return seg_reduce_t<T, 256>(X, perm, keys, off, n, nseg, o, buf, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_segment_reduce(int dt, int D, const void* X, const uint32_t* perm, const uint32_t* sorted_keys,
                                 const int32_t* off, int64_t n, uint32_t nseg, const SegOut& out, SegBuffers& buf,
                                 hipStream_t s) {
  switch (dt) {
    case DT_F32: return seg_reduce_d<F32>(D, X, perm, sorted_keys, off, n, nseg, out, buf, s);
    case DT_F16: return seg_reduce_d<F16>(D, X, perm, sorted_keys, off, n, nseg, out, buf, s);
    case DT_BF16: return seg_reduce_d<BF16>(D, X, perm, sorted_keys, off, n, nseg, out, buf, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_mean_from_sums(const double* S, const int64_t* n, int D, int64_t K, const float* C_prev,
                                 float* C_new, hipStream_t s) {
  const int64_t tot = K * D;
  mean_from_sums_kernel<<<dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s>>>(S, n, D, K, C_prev, C_new);
  return hipGetLastError();
}

hipError_t launch_zero_bytes(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int tail = (int)(bytes % 16);
  const int64_t work = n16 > tail ? n16 : tail;
  zero_kernel<<<dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s>>>(
      reinterpret_cast<uint4*>(p), n16, reinterpret_cast<uint8_t*>(p) + n16 * 16, tail);
  return hipGetLastError();
}

}  // namespace fkm
