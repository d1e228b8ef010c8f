// Inverse mapping for the sort-inverse update (Flash-KMeans paper page,
// abstract: the update first builds an explicit inverse mapping from clusters
// to their points; article section "Flash-KMeans が変える点", second point).
//
// A stable least-significant-digit radix argsort of the cluster keys
// (key = b*K + label) with 8-bit digits.  Each digit pass is reduce-then-scan:
//   hist    per-workgroup digit counts, stored digit-major [256][nblk];
//   scan    exclusive scan of each digit row, plus the digit totals;
//   scatter stable rank of every key inside its workgroup tile, written to
//           digit base + workgroup offset + rank.
// Elements travel as (key, row) pairs packed in 8 bytes, so every pass reads
// and writes each element with one access and a digit run of a tile is one
// contiguous piece of the output; between the two passes of keys below 2^16
// over fewer than 2^24 rows they travel in 4 bytes (high key byte and row).
// Ranks come from wave-level digit matching (eight ballots give each lane the
// mask of lanes holding the same digit) and per-wave counters, so the output
// order is fully determined: equal keys keep their row order.  Histogram
// counts use LDS atomics (exact integers, so order-free).  No workgroup ever
// waits on another.
// With few tiles a pass drops its scan kernel: the histogram is stored
// tile-major and each scatter workgroup sums the counts it needs.  Batched
// keys with K <= 256 take a single segmented pass: the instances arrive one
// after another, so tiles that stay inside one instance and sort by the label
// alone produce the order of b*K + label.  Other keys of 9 to 11 bits take a
// single pass whose digit is the whole key (2^bits counts per tile).
#include "common.h"
#include "kernels.h"

namespace fkm {

namespace {

constexpr int kT = 256;

// Source of the (key, row) pair at position i of a pass's input.  The first
// pass makes it from the labels (row = i); later passes read the previous
// pass's output.
struct LabelSrc {
  const int32_t* labels;
  int64_t N;      // rows per instance
  uint32_t K;     // centroids per instance
  int B;          // instances
  double invN;    // 1.0 / N, for the instance index
  // key of label value l at position i
  __device__ __forceinline__ uint32_t key(int32_t l, int64_t i) const {
    const uint32_t lab = (uint32_t)l < K ? (uint32_t)l : K - 1;  // out-of-range labels clamp (caller error)
    if (B == 1) return lab;
    // instance index i / N: a floating estimate corrected to the exact floor
    int64_t b = (int64_t)((double)i * invN);
    if ((b + 1) * N <= i) ++b;
    if (b * N > i) --b;
    return (uint32_t)b * K + lab;
  }
  __device__ __forceinline__ uint2 operator()(int64_t i) const { return make_uint2(key(labels[i], i), (uint32_t)i); }
  // A segmented pass's tile lies inside one instance, whose key offset koff
  // = b * K the tile already knows: the key is koff + the clamped label, with
  // no per-element instance division.
  __device__ __forceinline__ uint2 in_instance(int64_t i, uint32_t koff) const {
    const uint32_t l = (uint32_t)labels[i];
    return make_uint2(koff + (l < K ? l : K - 1), (uint32_t)i);
  }
};
struct PairSrc {
  const uint2* kv;
  __device__ __forceinline__ uint2 operator()(int64_t i) const { return kv[i]; }
};
// The high pass of a two-pass sort of keys below 2^16 over fewer than 2^24
// rows reads 4-byte elements (high key byte << 24 | row) that the low pass
// wrote in low-byte order: the low byte of the element at position i is the
// low-digit bucket holding i, found from the low pass's digit totals.  As a
// plain source it yields the key with its low byte zero, which is all the
// histogram of the high digit needs.
struct PackedSrc {
  const uint32_t* kv;
  const uint32_t* lo_tot;  // the low pass's 256 digit totals
  __device__ __forceinline__ uint2 operator()(int64_t i) const {
    const uint32_t v = kv[i];
    return make_uint2((v >> 24) << 8, v & 0xFFFFFFu);
  }
};
template <class Src>
constexpr bool is_label_src = false;
template <>
constexpr bool is_label_src<LabelSrc> = true;
template <class Src>
constexpr bool is_pair_src = false;
template <>
constexpr bool is_pair_src<PairSrc> = true;
template <class Src>
constexpr bool is_packed_src = false;
template <>
constexpr bool is_packed_src<PackedSrc> = true;

// Segment geometry of a segmented pass (segN elements per segment, ntb
// tiles each, key offset kseg per segment); unused by a plain pass.
struct Segs {
  int64_t segN = 0, ntb = 1;
  uint32_t kseg = 0;
};
// Where tile g lies: its elements are row0 + [first, min(first + TILE, lim)),
// g0 is the segment's first tile and koff its key offset.
struct TilePos {
  int64_t row0, first, lim, g0, blk;
  uint32_t koff;
};
template <bool SEG, int TILE>
__device__ __forceinline__ TilePos tile_pos_t(int64_t g, int64_t n, const Segs& s) {
  if constexpr (SEG) {
    const int64_t sb = g / s.ntb;
    const int64_t blk = g - sb * s.ntb;
    return TilePos{sb * s.segN, blk * TILE, s.segN, sb * s.ntb, blk, (uint32_t)sb * s.kseg};
  } else {
    return TilePos{0, g * TILE, n, 0, g, 0u};
  }
}

// Mask of the active lanes of this wave whose RB-bit digit equals mine.
// Per bit, t is all ones where this lane's bit is set, and the lanes whose
// bit agrees are ~(ballot ^ t), applied to the two 32-bit halves of the mask
// with one three-input bit operation each (truth table 0x90: src0 & ~(src1 ^
// src2)): four vector instructions per bit, with every bit's extract and
// ballot issued ahead of the mask updates.  The empty asm statement keeps
// the compiler from re-deriving each ballot's condition with a shift.  (A
// per-lane select between the ballot and its complement cost the compiler
// nine instructions per bit; the scatter spends most of its issue cycles on
// the vector ALU.)
template <int RB>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid) {
  const uint64_t v = __ballot(valid);
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint32_t t[RB];
  uint64_t bb[RB];
#pragma unroll
  for (int bit = 0; bit < RB; ++bit) {
    t[bit] = (uint32_t)__builtin_amdgcn_sbfe((int)d, bit, 1);
    asm volatile("" : "+v"(t[bit]));
  }
#pragma unroll
  for (int bit = 0; bit < RB; ++bit) bb[bit] = __ballot(t[bit] != 0u);
#pragma unroll
  for (int bit = 0; bit < RB; ++bit) {
    lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)bb[bit], t[bit], 0x90);
    hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(bb[bit] >> 32), t[bit], 0x90);
  }
  return ((uint64_t)hi << 32) | lo;
}

// Blocks put in front of the histogram tiles for a side job.
__host__ __device__ inline int64_t side_blocks(const InertiaJob& side) {
  return side.part ? ((int64_t)side.B + 7) / 8 * 8 : 0;
}

// Count d of tile b goes to hist[d * dstride + b * tstride] (digit-major
// for the scan kernel, tile-major when the scatter sums the counts itself).
// The first side.B blocks run the side job (an inertia reduction), so it
// overlaps the counting instead of trailing it; the tiles start at block
// side_blocks(side), a multiple of 8, so each tile stays on the XCD it has
// without a side job.
// SEG: the n elements are consecutive segments of segN, each cut into ntb
// tiles of its own (the last one ragged), and the digit is taken from
// key - segment * kseg, so one pass sorts every segment by its local key.
// RB: digit bits (8, or up to 11 for a key sorted in one wide pass).
template <class Src, int TILE, bool SEG, int RB = 8>
__global__ __launch_bounds__(kT) void radix_hist_kernel(Src src, int64_t n, int shift, uint32_t* __restrict__ hist,
                                                        int64_t nblk, int64_t dstride, int64_t tstride,
                                                        Segs seg, InertiaJob side) {
  constexpr uint32_t R = 1u << RB;
  constexpr int DPT = (int)R / kT;  // digits per thread
  const int64_t extra = side_blocks(side);
  if ((int64_t)blockIdx.x < extra) {
    if ((int64_t)blockIdx.x < side.B)
      inertia_reduce_block(side.part, side.nwg, (int64_t)blockIdx.x, side.inertia, side.hist, false);
    return;
  }
  __shared__ uint32_t cnt[R];
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < DPT; ++j) cnt[t + kT * j] = 0;
  __syncthreads();
  const int64_t tile = xcd_tile((int64_t)blockIdx.x - extra, nblk);
  const TilePos p = tile_pos_t<SEG, TILE>(tile, n, seg);
  constexpr int kIPT = TILE / kT;  // keys per thread
  uint32_t d[kIPT];
  bool vec = false;
  if constexpr (is_label_src<Src> && !SEG && kIPT % 4 == 0) {
    // a whole tile of 16-byte aligned labels: four labels per load (4-byte
    // loads move half the bytes per instruction); which thread counts which
    // key does not matter
    const int32_t* lp = src.labels + p.row0 + p.first;
    vec = p.first + TILE <= p.lim && (reinterpret_cast<uintptr_t>(lp) & 15) == 0;
    if (vec) {
#pragma unroll
      for (int r4 = 0; r4 < kIPT / 4; ++r4) {
        const int li = (r4 * kT + t) * 4;
        const int4 l4 = *reinterpret_cast<const int4*>(lp + li);
        const int64_t i = p.row0 + p.first + li;
        d[4 * r4 + 0] = ((src.key(l4.x, i) - p.koff) >> shift) & (R - 1);
        d[4 * r4 + 1] = ((src.key(l4.y, i + 1) - p.koff) >> shift) & (R - 1);
        d[4 * r4 + 2] = ((src.key(l4.z, i + 2) - p.koff) >> shift) & (R - 1);
        d[4 * r4 + 3] = ((src.key(l4.w, i + 3) - p.koff) >> shift) & (R - 1);
      }
    }
  }
  if constexpr (is_pair_src<Src> && !SEG && kIPT % 2 == 0) {
    // a whole tile: two pairs per 16-byte load (the pair buffers are
    // 256-byte aligned and tiles start at multiples of TILE)
    vec = p.first + TILE <= p.lim;
    if (vec) {
      const uint4* kp = reinterpret_cast<const uint4*>(src.kv + p.row0 + p.first);
#pragma unroll
      for (int r2 = 0; r2 < kIPT / 2; ++r2) {
        const uint4 q = kp[r2 * kT + t];
        d[2 * r2 + 0] = ((q.x - p.koff) >> shift) & (R - 1);
        d[2 * r2 + 1] = ((q.z - p.koff) >> shift) & (R - 1);
      }
    }
  }
  if constexpr (is_packed_src<Src> && !SEG && kIPT % 4 == 0) {
    // a whole tile: four packed elements per 16-byte load, the digit is the
    // top byte
    static_assert(RB == 8, "packed elements carry an 8-bit digit");
    vec = p.first + TILE <= p.lim;
    if (vec) {
      const uint4* kp = reinterpret_cast<const uint4*>(src.kv + p.first);
#pragma unroll
      for (int r4 = 0; r4 < kIPT / 4; ++r4) {
        const uint4 q = kp[r4 * kT + t];
        d[4 * r4 + 0] = q.x >> 24;
        d[4 * r4 + 1] = q.y >> 24;
        d[4 * r4 + 2] = q.z >> 24;
        d[4 * r4 + 3] = q.w >> 24;
      }
    }
  }
  if (!vec) {
#pragma unroll
    for (int r = 0; r < kIPT; ++r) {
      const int64_t li = p.first + r * kT + t;
      uint2 kv;
      if constexpr (is_label_src<Src> && SEG) kv = li < p.lim ? src.in_instance(p.row0 + li, p.koff) : make_uint2(0u, 0u);
      else kv = li < p.lim ? src(p.row0 + li) : make_uint2(0u, 0u);
      d[r] = li < p.lim ? ((kv.x - p.koff) >> shift) & (R - 1) : R;
    }
  }
  // LDS atomics: the counts are exact integers, so their order is irrelevant.
  // When all 64 keys of a wave's round share one digit (a skewed label
  // distribution makes whole tiles of one cluster), one lane adds 64: 64
  // lanes hitting one counter would serialise.
  const int lane = t & 63;
#pragma unroll
  for (int r = 0; r < kIPT; ++r) {
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(d[r]);
    if (__ballot(d[r] == d0) == ~0ull) {
      if (lane == 0 && d0 < R) atomicAdd(&cnt[d0], 64u);
    } else if (d[r] < R) {
      atomicAdd(&cnt[d[r]], 1u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < DPT; ++j) hist[(int64_t)(t + kT * j) * dstride + tile * tstride] = cnt[t + kT * j];
}

// One workgroup per digit: exclusive scan of hist[d][0..nblk) in place,
// dtot[d] = row total.  Each thread takes kScanPer consecutive counts per
// round (16-byte loads and stores where the row allows), so the 2048 tiles of
// 2^23 keys are one round.
constexpr int kScanPer = 8;
__global__ __launch_bounds__(kT) void radix_scan_kernel(uint32_t* __restrict__ hist, int64_t nblk,
                                                        uint32_t* __restrict__ dtot) {
  __shared__ uint32_t tmp[4];
  uint32_t* row = hist + (int64_t)blockIdx.x * nblk;
  // the histogram region is 256-byte aligned, so the row is 16-byte aligned
  // when nblk is a multiple of 4
  const bool vec = (nblk & 3) == 0;
  uint32_t running = 0;
  for (int64_t c0 = 0; c0 < nblk; c0 += (int64_t)kT * kScanPer) {
    const int64_t i0 = c0 + (int64_t)threadIdx.x * kScanPer;
    const bool whole = vec && i0 + kScanPer <= nblk;
    uint32_t v[kScanPer];
    if (whole) {
#pragma unroll
      for (int j = 0; j < kScanPer; j += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(row + i0 + j);
        v[j] = q.x, v[j + 1] = q.y, v[j + 2] = q.z, v[j + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j) v[j] = i0 + j < nblk ? row[i0 + j] : 0u;
    }
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) s += v[j];
    uint32_t tot;
    uint32_t pre = block_exclusive_scan_256(s, tmp, &tot) + running;
    uint32_t out[kScanPer];
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      out[j] = pre;
      pre += v[j];
    }
    if (whole) {
#pragma unroll
      for (int j = 0; j < kScanPer; j += 4)
        *reinterpret_cast<uint4*>(row + i0 + j) = make_uint4(out[j], out[j + 1], out[j + 2], out[j + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j)
        if (i0 + j < nblk) row[i0 + j] = out[j];
    }
    running += tot;
  }
  if (threadIdx.x == 0) dtot[blockIdx.x] = running;
}

// With few tiles (kScanFreeTiles or fewer) the scatter reads the raw
// per-tile counts (tile-major, so each load is one contiguous kilobyte) and
// forms its own prefix, so the pass needs no scan kernel.

// Stable scatter of one tile.  Each wave ranks a contiguous quarter of the
// tile (64 keys per round, in row order): a key's rank among equal digits of
// its wave = keys of that digit in the wave's earlier rounds (a per-wave LDS
// counter; LDS operations of one wave complete in order, so no barrier is
// needed between rounds) + equal digits in lower lanes.  One barrier later
// the per-wave counts become per-wave offsets, every key lands in an LDS copy
// of the tile sorted by digit, and the tile is written out digit run by digit
// run, so consecutive threads write consecutive addresses.
// SEG (scan-free only): the tile sums the counts of its own segment's tiles
// and writes into that segment's part of the output.
// RB > 8 (scanned only): a wide digit of up to 11 bits, so a key of that
// many bits is sorted in one pass; thread t then owns the DPT consecutive
// digits t*DPT .. t*DPT + DPT - 1 (with 8 bits, digit t).
// PACK: the low pass of a two-pass sort of keys below 2^16 over fewer than
// 2^24 rows writes each element in 4 bytes, (key >> 8) << 24 | row, to out
// read as 32-bit words (a PackedSrc for the high pass).
template <class Src, int TILE, bool SCANNED, bool SEG, int RB = 8, bool PACK = false>
__global__ __launch_bounds__(kT) void radix_scatter_kernel(Src src, int64_t n, int shift,
                                                           const uint32_t* __restrict__ hist,
                                                           const uint32_t* __restrict__ dtot, int64_t nblk,
                                                           Segs seg, uint2* __restrict__ out) {
  static_assert(!(SCANNED && SEG), "a segmented pass sums its own counts");
  static_assert(RB == 8 || (SCANNED && !SEG), "wide digits use the scanned histogram");
  static_assert(!is_packed_src<Src> || (SCANNED && !SEG && RB == 8 && !PACK), "packed input: scanned high pass");
  constexpr uint32_t R = 1u << RB;
  constexpr int DPT = (int)R / kT;    // digits per thread
  constexpr int KW = TILE / 4;        // keys per wave
  constexpr int RW = KW / 64;         // rounds per wave
  __shared__ uint2 lkv[TILE];
  __shared__ uint32_t gbase[R];       // global position of LDS slot 0 of digit d's run, minus lstart[d]
  __shared__ uint32_t lstart[R];      // first LDS slot of digit d
  __shared__ uint32_t wcnt[4][R];     // per-wave digit counts, then per-wave offsets
  __shared__ uint32_t tmp[4];
  __shared__ uint32_t lo_start[is_packed_src<Src> ? 256 : 1];  // packed input: first position of each low digit
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int64_t g = xcd_tile(blockIdx.x, nblk);  // the tile this workgroup sorts
  const TilePos p = tile_pos_t<SEG, TILE>(g, n, seg);
  const int64_t blk = p.blk;                      // its index inside the segment
  const int64_t tiles = SEG ? seg.ntb : nblk;     // tiles of the segment

  // the tile's elements are loaded first, so their latency overlaps the
  // histogram loads and scans below
  const int64_t first = p.first + (int64_t)w * KW;
  uint2 e[RW];
  uint32_t rr[RW];
  // 16-byte loads (narrower loads move fewer bytes per instruction): in the
  // first pass lane l takes the labels of rows 4 (64 r4 + l) + {0..3} of the
  // wave's quarter, four per load where the tile is whole and aligned; in
  // later passes the pairs of rows 2 (64 r2 + l) + {0, 1}, two per load.
  // They go back to row order through this wave's quarter of lkv after the
  // histogram loads are issued.
  constexpr bool kLab = is_label_src<Src> && !SEG && RW % 4 == 0;
  constexpr bool kPair = is_pair_src<Src> && !SEG && RW % 2 == 0;
  constexpr bool kPk = is_packed_src<Src>;
  static_assert(!kPk || RW % 4 == 0, "packed input: whole 16-byte loads per lane");
  int4 l4[kLab ? RW / 4 : 1];
  uint4 q2[kPair ? RW / 2 : 1];
  uint4 k4[kPk ? RW / 4 : 1];
  if constexpr (kPk) {
    // packed input: lane l takes the elements of rows 4 (64 r4 + l) + {0..3}
    // of the wave's quarter, like the labels of the first pass
    const uint32_t* kp = src.kv + first;
    const bool vec = p.first + TILE <= p.lim;
#pragma unroll
    for (int r4 = 0; r4 < RW / 4; ++r4) {
      const int li = (r4 * 64 + lane) * 4;
      if (vec) {
        k4[r4] = *reinterpret_cast<const uint4*>(kp + li);
      } else {
        uint32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = first + li + j < p.lim ? kp[li + j] : 0u;
        k4[r4] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  } else if constexpr (kPair) {
    const uint2* kp = src.kv + p.row0 + first;
    const bool vec = p.first + TILE <= p.lim;
#pragma unroll
    for (int r2 = 0; r2 < RW / 2; ++r2) {
      const int li = (r2 * 64 + lane) * 2;
      if (vec) {
        q2[r2] = *reinterpret_cast<const uint4*>(kp + li);
      } else {
        const uint2 a = first + li < p.lim ? kp[li] : make_uint2(0u, 0u);
        const uint2 b = first + li + 1 < p.lim ? kp[li + 1] : make_uint2(0u, 0u);
        q2[r2] = make_uint4(a.x, a.y, b.x, b.y);
      }
    }
  } else if constexpr (kLab) {
    const int32_t* lp = src.labels + p.row0 + first;
    const bool vec = p.first + TILE <= p.lim && (reinterpret_cast<uintptr_t>(lp) & 15) == 0;
#pragma unroll
    for (int r4 = 0; r4 < RW / 4; ++r4) {
      const int li = (r4 * 64 + lane) * 4;
      if (vec) {
        l4[r4] = *reinterpret_cast<const int4*>(lp + li);
      } else {
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = first + li + j < p.lim ? lp[li + j] : 0;
        l4[r4] = make_int4(v[0], v[1], v[2], v[3]);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t li = first + r * 64 + lane;
      if constexpr (is_label_src<Src> && SEG) e[r] = li < p.lim ? src.in_instance(p.row0 + li, p.koff) : make_uint2(0u, 0u);
      else e[r] = li < p.lim ? src(p.row0 + li) : make_uint2(0u, 0u);
    }
  }

  // this tile's first position among, and count of, each digit it owns
  // (h0[j], cn[j]) and the digit's total (dt[j]): from the scanned
  // (exclusive) histogram rows, or summed here from the raw counts of the
  // segment's tiles
  uint32_t h0[DPT], cn[DPT], dt[DPT];
  if constexpr (SCANNED) {
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
      const int64_t d = (int64_t)t * DPT + j;
      h0[j] = hist[d * nblk + blk];
      const uint32_t h1 = blk + 1 < nblk ? hist[d * nblk + blk + 1] : dtot[d];
      cn[j] = h1 - h0[j];
      dt[j] = dtot[d];
    }
  } else {
    // tile-major counts: tile j's count of digit t is hist[j * 256 + t]
    uint32_t c[kScanFreeTiles];
#pragma unroll
    for (int j = 0; j < kScanFreeTiles; ++j) c[j] = j < tiles ? hist[(p.g0 + j) * 256 + t] : 0u;
    uint32_t before = 0, all = 0, own = 0;
#pragma unroll
    for (int j = 0; j < kScanFreeTiles; ++j) {
      before += j < blk ? c[j] : 0u;
      own += j == blk ? c[j] : 0u;
      all += c[j];
    }
    h0[0] = before;
    cn[0] = own;
    dt[0] = all;
  }
  // packed input: the low digits' first positions (an exclusive scan of the
  // low pass's totals), and the low digits of this tile's first and last
  // positions, which bound every element's low digit
  uint32_t lo_a = 0, lo_b = 0;
  if constexpr (kPk) {
    uint32_t tot;
    lo_start[t] = block_exclusive_scan_256(src.lo_tot[t], tmp, &tot);
    __syncthreads();
    const int64_t last = (p.first + TILE < p.lim ? p.first + TILE : p.lim) - 1;
    lo_a = (uint32_t)__syncthreads_count(t >= 1 && lo_start[t] <= (uint32_t)p.first);
    lo_b = (uint32_t)__syncthreads_count(t >= 1 && lo_start[t] <= (uint32_t)last);
  }
  if constexpr (kPair) {
    uint2* tw = lkv + w * KW;
#pragma unroll
    for (int r2 = 0; r2 < RW / 2; ++r2) *reinterpret_cast<uint4*>(tw + (r2 * 64 + lane) * 2) = q2[r2];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t li = first + r * 64 + lane;
      e[r] = li < p.lim ? tw[r * 64 + lane] : make_uint2(0u, 0u);
    }
  }
  if constexpr (kLab) {
    uint32_t* tw = reinterpret_cast<uint32_t*>(lkv) + w * KW;
#pragma unroll
    for (int r4 = 0; r4 < RW / 4; ++r4) *reinterpret_cast<int4*>(tw + (r4 * 64 + lane) * 4) = l4[r4];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t li = first + r * 64 + lane;
      e[r] = li < p.lim ? make_uint2(src.key((int32_t)tw[r * 64 + lane], p.row0 + li), (uint32_t)(p.row0 + li))
                        : make_uint2(0u, 0u);
    }
  }
  if constexpr (kPk) {
    uint32_t* tw = reinterpret_cast<uint32_t*>(lkv) + w * KW;
#pragma unroll
    for (int r4 = 0; r4 < RW / 4; ++r4) *reinterpret_cast<uint4*>(tw + (r4 * 64 + lane) * 4) = k4[r4];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t li = first + r * 64 + lane;
      const uint32_t v = tw[r * 64 + lane];
      // the low digit holding position li: the last digit whose first
      // position is at most li (an empty digit's first position equals the
      // next one's, so it is never the last)
      uint32_t a = lo_a, b = lo_b;
      while (a < b) {
        const uint32_t m = (a + b + 1) >> 1;
        if (lo_start[m] <= (uint32_t)li) a = m;
        else b = m - 1;
      }
      e[r] = li < p.lim ? make_uint2(((v >> 24) << 8) | a, v & 0xFFFFFFu) : make_uint2(0u, 0u);
    }
  }
  uint32_t sdt = 0, scn = 0;
#pragma unroll
  for (int j = 0; j < DPT; ++j) sdt += dt[j], scn += cn[j];
  uint32_t tot;
  uint32_t dpre = block_exclusive_scan_256(sdt, tmp, &tot);
  uint32_t ls = block_exclusive_scan_256(scn, tmp, &tot);
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int d = t * DPT + j;
    lstart[d] = ls;
    gbase[d] = (uint32_t)p.row0 + dpre + h0[j] - ls;
    dpre += dt[j];
    ls += cn[j];
  }
#pragma unroll
  for (int ww = 0; ww < 4; ++ww)
#pragma unroll
    for (int j = 0; j < DPT; ++j) wcnt[ww][t * DPT + j] = 0;
  __syncthreads();

#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const bool valid = first + r * 64 + lane < p.lim;
    const uint32_t d = ((e[r].x - p.koff) >> shift) & (R - 1);
    const uint64_t m = match_digit<RB>(d, valid);
    const uint32_t lrank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    const uint32_t before = wcnt[w][d];
    rr[r] = before + lrank;
    if (valid && lrank == 0) wcnt[w][d] = before + (uint32_t)__popcll(m);
  }
  __syncthreads();
  // per-wave counts -> exclusive per-wave offsets (thread t owns its digits)
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int d = t * DPT + j;
    uint32_t run = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const uint32_t c = wcnt[ww][d];
      wcnt[ww][d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    if (first + r * 64 + lane < p.lim) {
      const uint32_t d = ((e[r].x - p.koff) >> shift) & (R - 1);
      lkv[lstart[d] + wcnt[w][d] + rr[r]] = e[r];
    }
  }
  __syncthreads();
  const int64_t rem = p.lim - p.first;
  const int cnt = rem < TILE ? (int)rem : TILE;
  for (int i = t; i < cnt; i += kT) {
    const uint2 v = lkv[i];
    const uint32_t pos = gbase[((v.x - p.koff) >> shift) & (R - 1)] + (uint32_t)i;
    if constexpr (PACK) reinterpret_cast<uint32_t*>(out)[pos] = ((v.x >> 8) << 24) | v.y;
    else out[pos] = v;
  }
}

template <class Src, int TILE>
hipError_t one_pass_t(Src src, int64_t n, int shift, SortBuffers& buf, uint2* out, hipStream_t s,
                      const InertiaJob& side) {
  const int64_t nblk = (n + TILE - 1) / TILE;
  const int64_t extra = side_blocks(side);
  const bool scan_free = nblk <= kScanFreeTiles;
  radix_hist_kernel<Src, TILE, false><<<dim3((unsigned)(nblk + extra)), dim3(kT), 0, s>>>(
      src, n, shift, buf.hist, nblk, scan_free ? 1 : nblk, scan_free ? 256 : 1, Segs{}, side);
  if (scan_free) {
    radix_scatter_kernel<Src, TILE, false, false><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
        src, n, shift, buf.hist, buf.dtot, nblk, Segs{}, out);
  } else {
    radix_scan_kernel<<<dim3(256), dim3(kT), 0, s>>>(buf.hist, nblk, buf.dtot);
    radix_scatter_kernel<Src, TILE, true, false><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
        src, n, shift, buf.hist, buf.dtot, nblk, Segs{}, out);
  }
  return hipGetLastError();
}

template <class Src>
hipError_t one_pass(Src src, int64_t n, int shift, SortBuffers& buf, uint2* out, hipStream_t s,
                    const InertiaJob& side = InertiaJob{}) {
  return sort_tile(n) == kSortTileSmall ? one_pass_t<Src, kSortTileSmall>(src, n, shift, buf, out, s, side)
                                        : one_pass_t<Src, kSortTile>(src, n, shift, buf, out, s, side);
}

// Two 8-bit passes over n < 2^24 keys below 2^16 (scanned: more than
// kScanFreeTiles tiles).  The low pass writes each element in 4 bytes (high
// key byte and row) into kv[0], read as 32-bit words; the high pass reads
// them, restores the low byte from the element's position, and writes the
// sorted (key, row) pairs to out.  Half the bytes of the 8-byte intermediate
// are written, counted and read back.  The low pass's totals stay in
// dtot[256..511].
template <int TILE>
hipError_t packed_two_pass_t(const LabelSrc& ls, int64_t n, SortBuffers& buf, uint2* out, hipStream_t s,
                             const InertiaJob& side) {
  const int64_t nblk = (n + TILE - 1) / TILE;
  const int64_t extra = side_blocks(side);
  uint32_t* dlo = buf.dtot + 256;
  radix_hist_kernel<LabelSrc, TILE, false><<<dim3((unsigned)(nblk + extra)), dim3(kT), 0, s>>>(
      ls, n, 0, buf.hist, nblk, nblk, 1, Segs{}, side);
  radix_scan_kernel<<<dim3(256), dim3(kT), 0, s>>>(buf.hist, nblk, dlo);
  radix_scatter_kernel<LabelSrc, TILE, true, false, 8, true><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
      ls, n, 0, buf.hist, dlo, nblk, Segs{}, buf.kv[0]);
  const PackedSrc ps{reinterpret_cast<const uint32_t*>(buf.kv[0]), dlo};
  radix_hist_kernel<PackedSrc, TILE, false><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
      ps, n, 8, buf.hist, nblk, nblk, 1, Segs{}, InertiaJob{});
  radix_scan_kernel<<<dim3(256), dim3(kT), 0, s>>>(buf.hist, nblk, buf.dtot);
  radix_scatter_kernel<PackedSrc, TILE, true, false><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
      ps, n, 8, buf.hist, buf.dtot, nblk, Segs{}, out);
  return hipGetLastError();
}

// One pass over keys of RB (9 to 11) bits with RB-bit digits: histogram,
// one scan workgroup per digit, scatter.
template <class Src, int TILE, int RB>
hipError_t wide_pass_t(Src src, int64_t n, SortBuffers& buf, uint2* out, hipStream_t s, const InertiaJob& side) {
  const int64_t nblk = (n + TILE - 1) / TILE;
  const int64_t extra = side_blocks(side);
  radix_hist_kernel<Src, TILE, false, RB><<<dim3((unsigned)(nblk + extra)), dim3(kT), 0, s>>>(
      src, n, 0, buf.hist, nblk, nblk, 1, Segs{}, side);
  radix_scan_kernel<<<dim3(1u << RB), dim3(kT), 0, s>>>(buf.hist, nblk, buf.dtot);
  radix_scatter_kernel<Src, TILE, true, false, RB><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
      src, n, 0, buf.hist, buf.dtot, nblk, Segs{}, out);
  return hipGetLastError();
}

template <int RB>
hipError_t wide_pass(const LabelSrc& src, int64_t n, SortBuffers& buf, uint2* out, hipStream_t s,
                     const InertiaJob& side) {
  return wide_pass_t<LabelSrc, kSortTileSmall, RB>(src, n, buf, out, s, side);  // sort_wide_bits: small tiles only
}

// One segmented pass: B segments of N keys b*K + label with K <= 256, each
// tiled on its own, ntb = ceil(N / TILE) <= kScanFreeTiles tiles per segment,
// B * ntb tiles in all (the histogram holds sort_seg_blocks(N, B) tiles).
template <int TILE>
hipError_t seg_pass_t(const LabelSrc& src, int64_t N, int B, uint32_t K, SortBuffers& buf, uint2* out,
                      hipStream_t s, const InertiaJob& side) {
  const int64_t n = N * (int64_t)B;
  const Segs sg{N, (N + TILE - 1) / TILE, K};
  const int64_t nblk = sg.ntb * B;
  const int64_t extra = side_blocks(side);
  radix_hist_kernel<LabelSrc, TILE, true><<<dim3((unsigned)(nblk + extra)), dim3(kT), 0, s>>>(
      src, n, 0, buf.hist, nblk, 1, 256, sg, side);
  radix_scatter_kernel<LabelSrc, TILE, false, true><<<dim3((unsigned)nblk), dim3(kT), 0, s>>>(
      src, n, 0, buf.hist, buf.dtot, nblk, sg, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_argsort_labels(const int32_t* labels, int64_t N, int B, int K, SortBuffers& buf,
                                 const uint2** sorted, hipStream_t s, const InertiaJob* side) {
  const int64_t n = N * (int64_t)B;
  const int passes = (sort_key_bits(B, K) + 7) / 8;
  LabelSrc ls{labels, N, (uint32_t)K, B, 1.0 / (double)N};
  // A workspace laid out for more rows than this call sorts (the streamed
  // path's last chunk) may not hold the histogram of the one-pass variants,
  // whose size is not monotone in the row count: they are taken only if the
  // histogram fits, and the plain passes always fit a layout for at least n.
  const int64_t T = sort_tile(n);
  const bool seg_fits = 256 * ((N + T - 1) / T) * (int64_t)B <= buf.hist_words;
  if (passes > 1 && sort_segmented(N, B, K) && seg_fits) {
    // instances arrive one after another, so sorting each by its label alone
    // gives the order of the key b*K + label in one pass
    *sorted = buf.kv[0];
    return sort_tile(n) == kSortTileSmall
               ? seg_pass_t<kSortTileSmall>(ls, N, B, (uint32_t)K, buf, buf.kv[0], s, side ? *side : InertiaJob{})
               : seg_pass_t<kSortTile>(ls, N, B, (uint32_t)K, buf, buf.kv[0], s, side ? *side : InertiaJob{});
  }
  const int wb = sort_wide_bits(N, B, K);
  if (wb && ((int64_t)1 << wb) * sort_blocks(n) <= buf.hist_words) {
    // the whole key fits one digit of 9 to 11 bits: a single pass
    *sorted = buf.kv[0];
    const InertiaJob sj = side ? *side : InertiaJob{};
    return wb == 9    ? wide_pass<9>(ls, n, buf, buf.kv[0], s, sj)
           : wb == 10 ? wide_pass<10>(ls, n, buf, buf.kv[0], s, sj)
                      : wide_pass<11>(ls, n, buf, buf.kv[0], s, sj);
  }
  if (256 * sort_blocks(n) > buf.hist_words) return hipErrorInvalidValue;  // workspace laid out for fewer rows
  if (passes == 2 && n < ((int64_t)1 << 24) && sort_blocks(n) > kScanFreeTiles) {
    *sorted = buf.kv[1];
    const InertiaJob sj = side ? *side : InertiaJob{};
    return sort_tile(n) == kSortTileSmall ? packed_two_pass_t<kSortTileSmall>(ls, n, buf, buf.kv[1], s, sj)
                                          : packed_two_pass_t<kSortTile>(ls, n, buf, buf.kv[1], s, sj);
  }
  hipError_t e = one_pass(ls, n, 0, buf, buf.kv[0], s, side ? *side : InertiaJob{});
  if (e != hipSuccess) return e;
  int cur = 0;
  for (int p = 1; p < passes; ++p) {
    e = one_pass(PairSrc{buf.kv[cur]}, n, 8 * p, buf, buf.kv[cur ^ 1], s);
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  *sorted = buf.kv[cur];
  return hipSuccess;
}

}  // namespace fkm
