// Device-side building blocks shared by the k-means kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fkm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types.  `raw` is the storage word, KPL the elements one lane feeds
// to one 32x32 MFMA step, SZ the storage bytes per element.
// ---------------------------------------------------------------------------

// Round-to-nearest-even fp32 -> bf16 on the bit pattern (bf16 is the upper
// half of an IEEE binary32; add half an ulp of the kept part, plus one when
// the kept part is odd, then truncate).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct BF16 {
  using raw = uint16_t;
  static constexpr int SZ = 2;
  static constexpr int KPL = 8;
  __device__ static raw from_f32(float f) { return f32_to_bf16_rne(f); }
  __device__ static float to_f32(raw r) { return bf16_to_f32(r); }
  // 8 elements packed in a 16-byte word
  __device__ static void unpack8(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

struct F16 {
  using raw = uint16_t;
  static constexpr int SZ = 2;
  static constexpr int KPL = 8;
  __device__ static raw from_f32(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
  __device__ static float to_f32(raw r) { return (float)__builtin_bit_cast(_Float16, r); }
  __device__ static void unpack8(const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
      o[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
};

struct F32 {
  using raw = float;
  static constexpr int SZ = 4;
  static constexpr int KPL = 1;
  __device__ static raw from_f32(float f) { return f; }
  __device__ static float to_f32(raw r) { return r; }
  __device__ static void unpack4(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};

// Elements held in one 16-byte word: unpack to fp32, and add them into N
// fp32 accumulators (add_if: only when `take`).  For the 16-bit types the
// add is a two-element dot product with (1, -0) or (-0, 1): the products are
// exact, so each accumulator receives exactly one rounded fp32 addition of
// its element, the same value as an unpack followed by an fp32 add, in half
// the instructions.  The -0 halves keep the multipliers from matching an
// inline constant, whose packed 16-bit reading differs between the compiler
// and the hardware for bf16 operands; as 32-bit literals their meaning is
// exact.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// sq_add(x, c, acc): acc plus the squared differences of the elements of
// x and c, added with fused multiply-adds in element order (for the 16-bit
// types each difference is the exact difference rounded once to fp32).
template <class T> struct Vec;
template <class T>
__device__ __forceinline__ float sq_add_unpacked(const uint4& x, const uint4& c, float acc) {
  float xv[T::N], cv[T::N];
  T::unpack(x, xv);
  T::unpack(c, cv);
#pragma unroll
  for (int e = 0; e < T::N; ++e) {
    const float df = xv[e] - cv[e];
    acc = fmaf(df, df, acc);
  }
  return acc;
}
template <> struct Vec<BF16> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& v, float* o) { BF16::unpack8(v, o); }
  __device__ __forceinline__ static float sq_add(const uint4& x, const uint4& c, float acc) {
    return sq_add_unpacked<Vec<BF16>>(x, c, acc);
  }
  __device__ __forceinline__ static void add_with(const uint4& v, float* acc, uint32_t lo, uint32_t hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const bf16x2 blo = __builtin_bit_cast(bf16x2, lo), bhi = __builtin_bit_cast(bf16x2, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 a = __builtin_bit_cast(bf16x2, w[i]);
      acc[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(a, blo, acc[2 * i], false);
      acc[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(a, bhi, acc[2 * i + 1], false);
    }
  }
  __device__ __forceinline__ static void add(const uint4& v, float* acc) { add_with(v, acc, 0x80003F80u, 0x3F808000u); }
  __device__ __forceinline__ static void add_if(const uint4& v, float* acc, bool take) {
    add_with(v, acc, take ? 0x80003F80u : 0u, take ? 0x3F808000u : 0u);
  }
};
template <> struct Vec<F16> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& v, float* o) { F16::unpack8(v, o); }
  // x - c of the low / high halves of two words: a mixed-precision fma
  // x * 1 + (-c) on the f16 halves, one instruction for the two conversions
  // and the subtraction, with the same single rounding
  __device__ __forceinline__ static float diff_lo(uint32_t x, uint32_t c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,1]" : "=v"(d) : "v"(x), "v"(c));
    return d;
  }
  __device__ __forceinline__ static float diff_hi(uint32_t x, uint32_t c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(x), "v"(c));
    return d;
  }
  __device__ __forceinline__ static float sq_add(const uint4& x, const uint4& c, float acc) {
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d0 = diff_lo(xw[i], cw[i]);
      acc = fmaf(d0, d0, acc);
      const float d1 = diff_hi(xw[i], cw[i]);
      acc = fmaf(d1, d1, acc);
    }
    return acc;
  }
  __device__ __forceinline__ static void add_with(const uint4& v, float* acc, uint32_t lo, uint32_t hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const f16x2 blo = __builtin_bit_cast(f16x2, lo), bhi = __builtin_bit_cast(f16x2, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 a = __builtin_bit_cast(f16x2, w[i]);
      acc[2 * i] = __builtin_amdgcn_fdot2(a, blo, acc[2 * i], false);
      acc[2 * i + 1] = __builtin_amdgcn_fdot2(a, bhi, acc[2 * i + 1], false);
    }
  }
  __device__ __forceinline__ static void add(const uint4& v, float* acc) { add_with(v, acc, 0x80003C00u, 0x3C008000u); }
  __device__ __forceinline__ static void add_if(const uint4& v, float* acc, bool take) {
    add_with(v, acc, take ? 0x80003C00u : 0u, take ? 0x3C008000u : 0u);
  }
};
template <> struct Vec<F32> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& v, float* o) { F32::unpack4(v, o); }
  __device__ __forceinline__ static float sq_add(const uint4& x, const uint4& c, float acc) {
    return sq_add_unpacked<Vec<F32>>(x, c, acc);
  }
  __device__ __forceinline__ static void add(const uint4& v, float* acc) {
    acc[0] += __uint_as_float(v.x);
    acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z);
    acc[3] += __uint_as_float(v.w);
  }
  __device__ __forceinline__ static void add_if(const uint4& v, float* acc, bool take) {
    acc[0] += take ? __uint_as_float(v.x) : 0.f;
    acc[1] += take ? __uint_as_float(v.y) : 0.f;
    acc[2] += take ? __uint_as_float(v.z) : 0.f;
    acc[3] += take ? __uint_as_float(v.w) : 0.f;
  }
};

// One 32x32 MFMA step.  `a` / `b` are the lane's row fragments as 16-byte
// words; step s consumes KPL elements starting at element s*KPL.  Callers
// invoke it from fully unrolled loops so `s` is a compile-time constant.
template <class T> struct Mfma;
template <> struct Mfma<BF16> {
  __device__ __forceinline__ static f32x16 step(const uint4* a, const uint4* b, int s, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                   __builtin_bit_cast(bf16x8, b[s]), c, 0, 0, 0);
  }
};
template <> struct Mfma<F16> {
  __device__ __forceinline__ static f32x16 step(const uint4* a, const uint4* b, int s, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[s]),
                                                  __builtin_bit_cast(f16x8, b[s]), c, 0, 0, 0);
  }
};
__device__ __forceinline__ float word(const uint4& v, int c) {
  return __uint_as_float(c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w);
}
template <> struct Mfma<F32> {
  __device__ __forceinline__ static f32x16 step(const uint4* a, const uint4* b, int s, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(word(a[s >> 2], s & 3), word(b[s >> 2], s & 3), c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Wave / block helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// inertia[b] (+= when accumulating) = fixed-order sum of part[b, 0..nwg) by
// one 256-thread workgroup: thread t sums the pairs part[b, 2 (t + 256 i) + {0, 1}]
// in order of i into two running sums (one per pair element), adds them, each
// wave adds its lanes, then thread 0 adds the four wave sums in order.  The
// pairs are 16-byte loads issued kBatch at a time, so one workgroup reads the
// ~10^5 partials of a large instance in a few microseconds.
__device__ __forceinline__ void inertia_reduce_block(const double* __restrict__ part, int nwg, int64_t b,
                                                     double* __restrict__ inertia, double* __restrict__ hist,
                                                     bool accumulate) {
  constexpr int kBatch = 12;
  __shared__ double ws[4];
  const double* p = part + b * nwg;
  const int n2 = nwg >> 1;
  double v0 = 0.0, v1 = 0.0;
  int i = threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    const double2* q = reinterpret_cast<const double2*>(p);
    for (; i + 256 * (kBatch - 1) < n2; i += 256 * kBatch) {
      double2 t[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) t[u] = q[i + 256 * u];
      __builtin_amdgcn_sched_barrier(0);  // every load of the batch issues before the first add
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        v0 += t[u].x;
        v1 += t[u].y;
      }
    }
    for (; i < n2; i += 256) {
      const double2 t = q[i];
      v0 += t.x;
      v1 += t.y;
    }
  } else {
    for (; i < n2; i += 256) {
      v0 += p[2 * i];
      v1 += p[2 * i + 1];
    }
  }
  if ((nwg & 1) && threadIdx.x == 0) v0 += p[nwg - 1];
  double v = v0 + v1;
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = ((ws[0] + ws[1]) + ws[2]) + ws[3];
    if (accumulate) tot += inertia[b];
    inertia[b] = tot;
    if (hist) hist[b] = tot;
  }
}

// Centroid preparation of one row by one wave: lane l holds the fp32
// centroid values c[j] of dims l + 64 j.  Writes the row rounded to the
// input type and returns sum_d RNE(c_d)^2, summed per lane in dim order and
// then across the wave (lane 0's value is the one used).  Both the
// preparation kernel and the update's fused preparation call this, so their
// results are identical.
template <class T, int D>
__device__ __forceinline__ float prep_row(const float (&c)[(D + 63) / 64], typename T::raw* __restrict__ chat_row,
                                          int lane) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < (D + 63) / 64; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
      const typename T::raw r = T::from_f32(c[j]);
      chat_row[d] = r;
      const float v = T::to_f32(r);
      ss = fmaf(v, v, ss);
    }
  }
  return wave_sum_f32(ss);
}

// 16-byte load marked non-temporal (data read once: streamed past the caches
// instead of displacing reusable lines).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroups are dispatched to the chip's 8 XCDs (each with its own L2) in
// round-robin order of their index.  xcd_tile maps workgroup b of n to a
// tile so that the workgroups of one XCD take one contiguous range of tiles:
// neighbouring tiles then share that XCD's L2 (partial cache lines written
// by adjacent tiles merge there).  It is a bijection on [0, n) whatever the
// dispatch really does; only locality depends on it.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t n) {
  constexpr int kXcd = 8;
  const int64_t q = n / kXcd, r = n % kXcd;
  const int64_t x = b % kXcd, i = b / kXcd;
  return x * q + (x < r ? x : r) + i;
}

// Exclusive prefix sum over a 256-thread block (4 waves).  `tmp` must hold 4
// words.  Returns the exclusive prefix of `v`; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan_256(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  uint32_t wpre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t t = tmp[i];
    if (i < w) wpre += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wpre + inc - v;
}

}  // namespace fkm
