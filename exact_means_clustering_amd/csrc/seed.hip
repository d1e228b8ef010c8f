// On-device seeding of the initial centroids: random rows, or k-means++ D^2
// sampling.  The pages name k-means++ seeding only as outside the method's
// inner loop (article "Hacker Newsが捉えたFlash-KMeans…", section なぜ Hacker
// News のスレッドが重要だったか); this is the standard D^2 sampling, driven by
// uniforms the caller supplies:
//   c_0 = row floor(u_0 N);  for j >= 1, with D2_i the squared distance of row
//   i to its nearest chosen row, c_j = the smallest row i whose cumulative D2
//   exceeds u_j * sum(D2)  (row floor(u_j N) when the sum is zero).
// Each round is two kernels: a streaming D2 update against the newest pick
// (one 256-row block per workgroup, rows read coalesced; the block's fp64 sum
// comes from the same inclusive scan the pick uses), then one workgroup per
// instance that finds the block and the row of the inverse CDF.  Sums are in
// a fixed order, so the picks are deterministic.
#include "common.h"
#include "kernels.h"

namespace fkm {

namespace {

constexpr int kSeedRows = 256;  // rows per D2 block (one per thread in the scans)

// Inclusive fp64 prefix sum over a 256-thread block (4 waves, fixed order).
// tmp holds 4 doubles.  *total receives the block sum.
__device__ __forceinline__ double block_inclusive_scan_f64(double v, double* tmp, double* total) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  double wpre = 0.0;
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (i < w) wpre += tmp[i];
  const double tot = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  *total = tot;
  return wpre + inc;
}

// D2[b, i] = min(D2[b, i], ||x_bi - x_b,center||^2) (or the distance alone on
// the first round) for the 256 rows of block blockIdx.x of instance
// blockIdx.y; part[b * nblk + blk] = the block's sum (inclusive-scan total).
template <class T, int D>
__global__ __launch_bounds__(256) void seed_d2_kernel(const typename T::raw* __restrict__ X, int64_t N, int K,
                                                      const int32_t* __restrict__ idx, int j, int first,
                                                      float* __restrict__ d2, double* __restrict__ part,
                                                      int64_t nblk) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D * T::SZ / 16;  // lanes per row
  constexpr int SL = 64 / LPR;         // rows per wave step
  __shared__ float rowd[kSeedRows];
  __shared__ double tmp[4];
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int q = lane / LPR, g = lane % LPR;
  const int64_t b = blockIdx.y;
  const int64_t blk = blockIdx.x;
  const typename T::raw* Xb = X + b * N * D;
  const int64_t center = idx[b * K + j];
  float cf[VEC];
  Vec<T>::unpack(reinterpret_cast<const uint4*>(Xb + center * D)[g], cf);
  // wave w covers rows [w*64, w*64+64) of the block, SL rows per step
  for (int r0 = w * 64; r0 < w * 64 + 64; r0 += SL) {
    const int r = r0 + q;
    const int64_t i = blk * kSeedRows + r;
    float part_d = 0.f;
    if (i < N) {
      float xf[VEC];
      Vec<T>::unpack(reinterpret_cast<const uint4*>(Xb + i * D)[g], xf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float df = xf[e] - cf[e];
        part_d = fmaf(df, df, part_d);
      }
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) part_d += __shfl_xor(part_d, o);
    if (g == 0) {
      float v = 0.f;
      if (i < N) {
        v = first ? part_d : fminf(d2[b * N + i], part_d);
        d2[b * N + i] = v;
      }
      rowd[r] = v;
    }
  }
  __syncthreads();
  double total;
  (void)block_inclusive_scan_f64((double)rowd[threadIdx.x], tmp, &total);
  if (threadIdx.x == 0) part[b * nblk + blk] = total;
}

// Pick c_j of instance blockIdx.y (sampled == 0: row floor(u N)) and copy it
// into C[b, j, :] as fp32.
template <class T, int D>
__global__ __launch_bounds__(256) void seed_pick_kernel(const typename T::raw* __restrict__ X, int64_t N, int K,
                                                        const double* __restrict__ u, int j, int sampled,
                                                        const float* __restrict__ d2,
                                                        const double* __restrict__ part, int64_t nblk,
                                                        int32_t* __restrict__ idx, float* __restrict__ C) {
  __shared__ double tmp[4];
  __shared__ int64_t pick_s;
  __shared__ int first_s;
  const int t = threadIdx.x;
  const int64_t b = blockIdx.y;
  const double uj = u[b * K + j];
  int64_t uni = (int64_t)(uj * (double)N);
  uni = uni < 0 ? 0 : (uni > N - 1 ? N - 1 : uni);
  if (t == 0) pick_s = uni;
  if (sampled) {
    // 1. blocks [t*per, (t+1)*per) summed in order by thread t; scan over threads
    const int64_t per = (nblk + 255) / 256;
    const double* pb = part + b * nblk;
    double v = 0.0;
    for (int64_t k = t * per; k < (t + 1) * per && k < nblk; ++k) v += pb[k];
    double total;
    const double inc = block_inclusive_scan_f64(v, tmp, &total);
    const double target = uj * total;
    // 2. the first thread whose inclusive sum exceeds the target (rounding
    //    can put the target at the total: then the last thread with a
    //    positive sum, and below its last positive block and row)
    __shared__ int lastv_s;
    if (t == 0) {
      first_s = 256;
      lastv_s = -1;
    }
    __syncthreads();
    if (total > 0.0 && inc > target) atomicMin(&first_s, t);
    if (total > 0.0 && v > 0.0) atomicMax(&lastv_s, t);
    __syncthreads();
    const int ft = first_s < 256 ? first_s : lastv_s;
    // the exact exclusive prefix of each thread: the previous thread's inclusive sum
    __shared__ double incs[256];
    incs[t] = inc;
    __syncthreads();
    const double excl = t > 0 ? incs[t - 1] : 0.0;
    if (total > 0.0 && ft >= 0) {
      // 3. that thread's first block whose cumulative sum exceeds the target;
      //    the local prefix is summed exactly as v was, so excl + (local sum
      //    at the thread's last block) reproduces inc and the search ends
      __shared__ int64_t blk_s;
      __shared__ double before_s;
      if (t == ft) {
        double local = 0.0, local_nz = 0.0;
        const int64_t last = (t + 1) * per < nblk ? (t + 1) * per : nblk;
        int64_t found = -1, lastnz = t * per;
        for (int64_t k = t * per; k < last; ++k) {
          const double nl = local + pb[k];
          if (pb[k] > 0.0) lastnz = k, local_nz = local;
          if (excl + nl > target) {
            found = k;
            break;
          }
          local = nl;
        }
        blk_s = found >= 0 ? found : lastnz;
        before_s = excl + (found >= 0 ? local : local_nz);
      }
      __syncthreads();
      const int64_t blk = blk_s;
      // 4. the row inside the block, by the same scan that summed the block
      const int64_t i = blk * kSeedRows + t;
      const float dv = i < N ? d2[b * N + i] : 0.f;
      double btot;
      const double rinc = before_s + block_inclusive_scan_f64((double)dv, tmp, &btot);
      __shared__ int row_s, lastpos_s;
      if (t == 0) {
        row_s = 256;
        lastpos_s = -1;
      }
      __syncthreads();
      if (dv > 0.f && rinc > target) atomicMin(&row_s, t);
      if (dv > 0.f) atomicMax(&lastpos_s, t);
      __syncthreads();
      // rounding can leave the target past the block's last row: take the last row with D2 > 0
      if (t == 0) pick_s = blk * kSeedRows + (row_s < 256 ? row_s : (lastpos_s >= 0 ? lastpos_s : 0));
    }
  }
  __syncthreads();
  const int64_t pick = pick_s;
  if (t == 0) idx[b * K + j] = (int32_t)pick;
  const typename T::raw* row = X + (b * N + pick) * D;
  for (int d = t; d < D; d += 256) C[(b * K + j) * D + d] = T::to_f32(row[d]);
}

template <class T, int D>
hipError_t seed_t(const void* Xv, int64_t N, int B, int K, int method, const double* u, int32_t* idx, float* C,
                  float* d2, double* part, float* d2_out, hipStream_t s) {
  const auto* X = reinterpret_cast<const typename T::raw*>(Xv);
  const int64_t nblk = (N + kSeedRows - 1) / kSeedRows;
  const dim3 gb((unsigned)nblk, (unsigned)B), g1(1, (unsigned)B), th(256);
  // with the caller's D2 buffer the running D2 lives there directly
  if (d2_out) d2 = d2_out;
  seed_pick_kernel<T, D><<<g1, th, 0, s>>>(X, N, K, u, 0, 0, d2, part, nblk, idx, C);
  for (int j = 1; j < K; ++j) {
    if (method == 1) seed_d2_kernel<T, D><<<gb, th, 0, s>>>(X, N, K, idx, j - 1, j == 1, d2, part, nblk);
    seed_pick_kernel<T, D><<<g1, th, 0, s>>>(X, N, K, u, j, method == 1, d2, part, nblk, idx, C);
  }
  if (d2_out) {
    // the distance of every row to its nearest pick, after the last one
    if (method == 1) {
      seed_d2_kernel<T, D><<<gb, th, 0, s>>>(X, N, K, idx, K - 1, K == 1, d2, part, nblk);
    } else {
      for (int jj = 0; jj < K; ++jj)
        seed_d2_kernel<T, D><<<gb, th, 0, s>>>(X, N, K, idx, jj, jj == 0, d2, part, nblk);
    }
  }
  return hipGetLastError();
}

template <class T, int D> struct SeedF {
  static hipError_t run(const void* X, int64_t N, int B, int K, int method, const double* u, int32_t* idx, float* C,
                        float* d2, double* part, float* d2_out, hipStream_t s) {
    return seed_t<T, D>(X, N, B, K, method, u, idx, C, d2, part, d2_out, s);
  }
};

template <template <class, int> class F, class... A>
hipError_t dispatch_seed(int dt, int D, A&&... a) {
  auto byd = [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    switch (D) {
      case 16: return F<T, 16>::run(a...);
      case 32: return F<T, 32>::run(a...);
      case 64: return F<T, 64>::run(a...);
      case 128: return F<T, 128>::run(a...);
      case 256: return F<T, 256>::run(a...);
      default: return hipErrorInvalidValue;
    }
  };
  switch (dt) {
    case DT_F32: return byd(F32{});
    case DT_F16: return byd(F16{});
    case DT_BF16: return byd(BF16{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_seed(int dt, int D, const void* X, int64_t N, int B, int K, int method, const double* u,
                       int32_t* idx, float* C, float* d2_scratch, double* part, float* d2_out, hipStream_t s) {
  return dispatch_seed<SeedF>(dt, D, X, N, B, K, method, u, idx, C, d2_scratch, part, d2_out, s);
}

}  // namespace fkm
