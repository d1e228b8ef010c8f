// Segment-local reductions of the sort-inverse update (Flash-KMeans paper
// page, abstract: scatters become segment-level localized reductions;
// article section "Flash-KMeans が変える点", second point: no atomic write
// contention on hot clusters).
//
// After the argsort, cluster k owns the contiguous sorted positions
// [off[k], off[k+1]).  The sorted order is cut into fixed chunks of
// seg_rows(n) positions, one wave each:
//   level 1  a wave writes the segment offsets off[k] of the segments that
//            start in its chunk, then sums, per segment piece inside the
//            chunk, the gathered rows X[perm[j]] in fp32 (4 rows per 64-lane
//            load for D*SZ = 256 B).  A segment that lies inside the chunk is
//            finished on the spot; the chunk's first / last piece of a
//            segment that crosses the chunk edge goes to fragment slot 0 / 1.
//            (Means mode: every cluster's count, off[k+1] - off[k], is then
//            written, and clusters no row carries are filled from C_prev, by
//            extra blocks of the level-2 launch, or by a separate pass.)
//   level 2  one workgroup per group of kSegGroup chunks adds (fp64) the chunk
//            fragments of every segment that crosses a chunk edge; segments
//            inside the group are finished, the others leave group fragments.
//   level 3  the segment (if any) that crosses into a group from the left
//            and ends inside it is finished by a workgroup of 16 waves.
// Every segment is finished by exactly one wave in a fixed order, so the
// update is deterministic and uses no atomics.  Fragment slot rule (used to
// find a segment's piece in unit u of size U): the piece is in slot 1 iff u
// is the unit where the segment starts and the segment does not start on
// the unit boundary; otherwise slot 0.
#include "common.h"
#include "kernels.h"

namespace fkm {

namespace {

// (Units are powers of two, U = 2^ulog, and positions are non-negative, so
// divisions by U are shifts: a 64-bit division is a long instruction
// sequence on the GPU.)
__device__ __forceinline__ int frag_slot(int64_t u, int ulog, int64_t s) {
  return (u == (s >> ulog) && s != (u << ulog)) ? 1 : 0;
}

// The fused centroid preparation of cluster k (means mode with o.chat):
// c[j] holds its new centroid at dims lane + 64 j.
template <class T, int D>
__device__ __forceinline__ void fused_prep(const SegOut& o, int64_t k, int lane, const float (&c)[(D + 63) / 64]) {
  const float ss = prep_row<T, D>(c, reinterpret_cast<typename T::raw*>(o.chat) + k * D, lane);
  if (lane == 0) {
    // B * K < 2^31, so a 32-bit division (a 64-bit one is a long sequence)
    const uint32_t b = (uint32_t)k / o.K;
    o.hb[(int64_t)b * o.Kp + ((uint32_t)k - b * o.K)] = -0.5f * ss;
  }
}

// Finish a segment: means mode writes C_new (and the fused preparation; the
// counts come from the offsets, in the fill blocks), accumulate mode adds
// into S_acc / n_acc.  `v` holds the segment sum for dims lane + 64*j.
template <class T, int D>
__device__ __forceinline__ void finish(const SegOut& o, int64_t k, int lane, const double* v, int64_t cnt) {
  constexpr int PER = (D + 63) / 64;
  if (o.S_acc) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      if (d < D) o.S_acc[k * D + d] += v[j];
    }
    if (lane == 0) o.n_acc[k] += cnt;
  } else {
    float c[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int d = lane + 64 * j;
      c[j] = d < D ? (float)(v[j] / (double)cnt) : 0.f;
      if (d < D) o.C_new[k * D + d] = c[j];
    }
    if (o.chat) fused_prep<T, D>(o, k, lane, c);
  }
}

// ---------------------------------------------------------------------------
// level 1: streaming gather + fp32 segmented sums per chunk
// ---------------------------------------------------------------------------
// One wave per chunk of U sorted positions.  The wave walks the chunk in
// steps of SL rows (one row per lane slot q, LPR lanes per row) and keeps
// kRing steps of row loads in flight whatever the segment boundaries.  Each
// lane slot accumulates its rows of the current segment in fp32; when the
// (wave-uniform) key changes, the slots are combined in a fixed butterfly
// and the piece is emitted: finished on the spot if the whole segment lies
// in the chunk, otherwise stored as the chunk's fragment (slot 0: the
// chunk's first segment, slot 1: its last).
//
// The chunk's keys and row ids are staged in LDS, wave-private (the kernel
// has no workgroup barrier), transposed as [q][step] so a lane reads the key
// and the row id of its slot's step with one LDS load each; a step's are read
// one step before they are needed.  The staging covers the ring's lookahead
// past the chunk: entries past the chunk's end hold its last row (every row
// load is issued unconditionally, which keeps each ring slot in fixed
// registers); whether a lane's row is real is decided by its position, and a
// row past the end adds zeros.
//
// The memory counter waits: a ring slot's row is consumed before the slot
// is refilled at the end of its step, so the ring keeps fixed registers
// across rounds (an old value still live while the slot's next load is in
// flight makes the register allocator rotate the ring at the loop edge, which
// needs every load to have landed), and no global store is issued inside the
// loop over a step's segment boundaries (the compiler would wait for every
// load in flight before that loop): the loop only waits for the oldest row.
// Steps of row loads kept in flight per wave: 4 for the 512-row chunks of
// large problems (update of 2^23 bf16 rows of 128 into 65,536 clusters:
// 0.516 against 0.519-0.520 ms with 8), 8 for the small chunks.
template <int U>
constexpr int ring_steps() {
#ifdef FKM_RING
  return FKM_RING;
#else
  return U >= 512 ? 4 : 8;
#endif
}

// Staging geometry of a level-1 chunk of U rows.
template <class T, int D, int U>
struct L1Geo {
  static constexpr int LPR = D * T::SZ / 16;                   // lanes per row
  static constexpr int SL = 64 / LPR;                          // rows per step (lane slots)
  static constexpr int NS = U / SL;                            // steps per chunk
  static constexpr int kRing = ring_steps<U>();
  // staged steps per slot: the chunk's rounds, the ring's lookahead, and the
  // one step further that the last step reads ahead
  static constexpr int NSP = (NS + kRing - 1) / kRing * kRing + kRing + 1;
  static constexpr int ENT = SL * NSP;                         // staged rows
  // finished pieces buffered per wave: one step can finish up to SL of them,
  // and the buffer is drained between steps once it could not take SL more
  // (two more for the 512-row chunks: 0.503 against 0.507 ms for the update
  // of 2^23 bf16 rows of 128 into 65,536 clusters)
  static constexpr int BUF = SL >= 4 ? 2 * SL + (U >= 512 ? 2 : 0) : 8;
  static_assert(LPR >= 1 && LPR <= 64 && U % SL == 0, "row and chunk sizes");
};

// ACC selects accumulate mode (o.S_acc / o.n_acc) at compile time, so the
// means-mode instance carries no read-modify-write code in its loop.
template <class T, int D, bool ACC, int U>
__global__ __launch_bounds__(256) void seg_level1_kernel(const typename T::raw* __restrict__ X,
                                                         const uint2* __restrict__ kv, int64_t n, uint32_t nseg,
                                                         int32_t* __restrict__ off, SegOut o,
                                                         float* __restrict__ frag) {
  using G = L1Geo<T, D, U>;
  constexpr int VEC = Vec<T>::N;           // elements per 16-byte word
  constexpr int LPR = G::LPR, SL = G::SL, NSP = G::NSP, kBuf = G::BUF, kRing = G::kRing;
  __shared__ __align__(16) uint32_t tkey[4][SL][NSP];
  __shared__ __align__(16) uint32_t trow[4][SL][NSP];
  __shared__ __align__(16) float bsum[4][kBuf][D];
  __shared__ uint32_t bkey[4][kBuf];
  __shared__ int32_t bkind[4][kBuf], bcnt[4][kBuf];
  const int lane = lane_id();
  // the wave index, and everything derived from it, is wave-uniform: keeping
  // it in scalar registers makes the per-step tests scalar branches
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t c = (int64_t)blockIdx.x * 4 + w;
  const int64_t r0 = c * U;
  if (r0 >= n) return;                     // every access below is wave-private: no barrier to reach
  const int cnt = (int)(n - r0 < U ? n - r0 : U);

  // Staging: chunk row e (rows at or past cnt read row cnt-1) goes to step
  // e / SL of slot e % SL; lane l stages rows l + 64 j (coalesced loads).
  const int64_t kbefore = r0 > 0 ? (int64_t)kv[r0 - 1].x : -1;  // key of the row before the chunk
  // key of the row after the chunk (the last row's own key if there is none)
  const uint32_t kafter = kv[r0 + cnt < n ? r0 + cnt : r0 + cnt - 1].x;
#pragma unroll 4
  for (int e = lane; e < G::ENT; e += 64) {
    const uint2 pr = kv[r0 + (e < cnt ? e : cnt - 1)];
    tkey[w][e % SL][e / SL] = pr.x;
    trow[w][e % SL][e / SL] = pr.y;
  }
  const uint32_t kf = __builtin_amdgcn_readfirstlane(tkey[w][0][0]);
  // does the chunk's first segment continue from the previous chunk?
  const bool cont_left = kbefore == (int64_t)kf;
  const int q = lane / LPR, g = lane % LPR;
  auto load_row = [&](uint32_t row) -> uint4 {
    return load_nt(reinterpret_cast<const uint4*>(X + (int64_t)row * D) + g);
  };

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  uint32_t cur = kf;
  int seg_start = 0;
  // Finished pieces wait in a wave-private LDS buffer and are written to
  // global memory between steps when it is nearly full, and after the loop.
  // Global stores share the load counter on this architecture: a store
  // issued inside the loop over a step's segment boundaries would make the
  // compiler wait for every row load in flight before that loop, and any
  // store makes the following ring waits also wait for its write
  // acknowledgement.  Entry kinds: 0 = a segment finished in this chunk,
  // 1 / 2 = the chunk's fragment slot 0 / 1.
  int nb = 0;  // buffered pieces (wave-uniform)
  auto drain = [&]() {
    for (int b = 0; b < nb; ++b) {
      const uint32_t k = __builtin_amdgcn_readfirstlane(bkey[w][b]);
      const int kind = __builtin_amdgcn_readfirstlane(bkind[w][b]);
      const int nk = __builtin_amdgcn_readfirstlane(bcnt[w][b]);
      for (int d = lane * 4; d < D; d += 256) {
        const float4 v = *reinterpret_cast<const float4*>(&bsum[w][b][d]);
        if (kind == 0) {
          if constexpr (ACC) {
            double* sa = o.S_acc + (int64_t)k * D + d;
            sa[0] += (double)v.x, sa[1] += (double)v.y, sa[2] += (double)v.z, sa[3] += (double)v.w;
          } else {
            const float fc = (float)nk;
            *reinterpret_cast<float4*>(o.C_new + (int64_t)k * D + d) =
                make_float4(v.x / fc, v.y / fc, v.z / fc, v.w / fc);
          }
        } else {
          *reinterpret_cast<float4*>(frag + (c * 2 + (kind - 1)) * D + d) = v;
        }
      }
      if constexpr (ACC) {
        if (lane == 0 && kind == 0) o.n_acc[k] += nk;
      }
      if constexpr (!ACC) {
        if (kind == 0 && o.chat) {
          // the same fp32 quotients as the stores above, at dims lane + 64 j
          const float fc = (float)nk;
          float cv[(D + 63) / 64];
#pragma unroll
          for (int j = 0; j < (D + 63) / 64; ++j) {
            const int d = lane + 64 * j;
            cv[j] = d < D ? bsum[w][b][d] / fc : 0.f;
          }
          fused_prep<T, D>(o, k, lane, cv);
        }
      }
    }
    nb = 0;
  };
  // emit the piece of segment k that ends before row `end` of the chunk;
  // only the chunk's last segment (the final flush) can continue into the
  // next chunk, and only its first can come from the previous one
  auto flush = [&](uint32_t k, int end, bool last) {
    // the slots' sums combine in place: the accumulators restart at zero
    float* s = acc;
#pragma unroll
    for (int o2 = LPR; o2 < 64; o2 <<= 1)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s[e] += __shfl_xor(s[e], o2);
    const bool left = k == kf && cont_left;
    const bool right = last && r0 + cnt < n && __builtin_amdgcn_readfirstlane(kafter) == k;
    if (q == 0) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) bsum[w][nb][g * VEC + e] = s[e];
    }
    if (lane == 0) {
      bkey[w][nb] = k;
      bkind[w][nb] = (left || right) ? (k == kf ? 1 : 2) : 0;
      bcnt[w][nb] = end - seg_start;
    }
    ++nb;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    seg_start = end;
  };

  // Segment offsets.  A row whose key k differs from the previous row's key
  // kp starts segment k: off[kk] = its position for every kk in (kp, k]
  // (keys no row carries get the start of the next present key), and the
  // last row of the order also sets off[kk] = n for kk in (k, nseg].  A lane
  // fills a short range itself; ranges of 64 or more keys are filled by the
  // whole wave, one coalesced store per 64 keys.  Large chunks write them
  // after their rows: a store issued before a ring wait makes that wait also
  // wait for the store's acknowledgement (0.507 against 0.514 ms for the
  // same update).  Small chunks write them while their first rows load
  // (their loop is too short to hide the stores at the end).
  auto key_at = [&](int r) -> uint32_t { return tkey[w][r % SL][r / SL]; };  // key of chunk row r
  auto write_offsets = [&]() {
    for (int e0 = 0; e0 < cnt; e0 += 64) {
      const int e = e0 + lane;
      int64_t a = 0, b = -1, a2 = 0, b2 = -1;
      int32_t val = 0;
      if (e < cnt) {
        const int64_t k = key_at(e);
        const int64_t kp = e > 0 ? (int64_t)key_at(e - 1) : kbefore;
        val = (int32_t)(r0 + e);
        if (k != kp) a = kp + 1, b = k;
        if (r0 + e == n - 1) a2 = k + 1, b2 = nseg;
      }
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int64_t lo = pass ? a2 : a, hi = pass ? b2 : b;
        const int32_t v = pass ? (int32_t)n : val;
        const bool longr = hi - lo >= 64;
        if (!longr)
          for (int64_t kk = lo; kk <= hi; ++kk) off[kk] = v;
        for (uint64_t lm = __ballot(longr); lm; lm &= lm - 1) {
          const int l = __ffsll((unsigned long long)lm) - 1;
          const int64_t la = __shfl(lo, l), lb = __shfl(hi, l);
          const int32_t lv = __shfl(v, l);
          for (int64_t kk = la + lane; kk <= lb; kk += 64) off[kk] = lv;
        }
      }
    }
  };

  const uint32_t* keys = &tkey[w][q][0];   // key of step i: keys[i]
  const uint32_t* rows = &trow[w][q][0];   // row id of step i: rows[i]
  uint4 ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing; ++u) ring[u] = load_row(rows[u]);
  if constexpr (U < 512) write_offsets();

  // Rounds of kRing steps; the steps past the chunk's end in the last round
  // add zeros to the (unchanged) last segment.
  const int nsteps = (cnt + SL - 1) / SL;
  uint32_t mk_next = keys[0], rn_next = rows[kRing];
  for (int i0 = 0; i0 < nsteps; i0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int i = i0 + u;                   // step
      const int row0 = i * SL;                // chunk row of the step's slot 0
      const uint32_t mk = mk_next, rn = rn_next;
      mk_next = keys[i + 1];
      rn_next = rows[i + 1 + kRing];
      const bool valid = row0 + q < cnt;
      uint4 v = ring[u];
      const int nv = cnt - row0;              // valid rows in this step (uniform)
      // key of the step's last valid row (uniform); no valid row: no boundary
      const uint32_t lk = nv > 0 ? __builtin_amdgcn_readlane(mk, ((nv < SL ? nv : SL) - 1) * LPR) : cur;
      if (lk == cur) {
        // whole step inside the current segment
        if (nv < SL && !valid) v = make_uint4(0, 0, 0, 0);
        Vec<T>::add(v, acc);
      } else {
        // the step ends `cur` and starts one or more new segments
        for (;;) {
          Vec<T>::add_if(v, acc, valid && mk == cur);
          if (cur == lk) break;
          const uint64_t above = __ballot(valid && mk > cur);
          const int fl = __ffsll((unsigned long long)above) - 1;
          flush(cur, row0 + fl / LPR, false);
          cur = __builtin_amdgcn_readlane(mk, fl);
        }
        if (nb > kBuf - SL) drain();
      }
      ring[u] = load_row(rn);
    }
  }
  flush(cur, cnt, true);
  drain();
  if constexpr (U >= 512) write_offsets();
}

// ---------------------------------------------------------------------------
// level 2: per group of chunks, combine chunk fragments (fp64)
// ---------------------------------------------------------------------------
// Means mode: every cluster's count is off[k+1] - off[k], written here for
// all clusters at once (coalesced, after the gather, so no count store
// competes with it); a cluster no row carries (count 0) keeps its previous
// centroid (its fused preparation, made from the previous centroid, stays as
// it is).  One thread per cluster, 256 per block.
__device__ __forceinline__ void empty_fill_block(int64_t blk, const int32_t* __restrict__ off, int64_t nseg, int D,
                                                 const float* __restrict__ C_prev, float* __restrict__ C_new,
                                                 int32_t* __restrict__ counts) {
  const int64_t k = blk * 256 + threadIdx.x;
  if (k >= nseg) return;
  const int32_t cnt = off[k + 1] - off[k];
  counts[k] = cnt;
  if (cnt != 0) return;
  if (C_new != C_prev) {  // D is a multiple of 4: copy the row as float4
    const float4* src = reinterpret_cast<const float4*>(C_prev + k * D);
    float4* dst = reinterpret_cast<float4*>(C_new + k * D);
#pragma unroll 8
    for (int d = 0; d < D / 4; ++d) dst[d] = src[d];
  }
}

// One workgroup of 4 waves per group.  The group's segments are scanned 64
// at a time (one coalesced load of their offsets); a ballot picks the ones
// that cross a chunk edge, and those are dealt round-robin to the 4 waves.
// In means mode the blocks past the groups run the empty-cluster fill,
// which needs only the offsets.
template <class T, int D>
__global__ __launch_bounds__(256) void seg_level2_kernel(const uint2* __restrict__ kv,
                                                         const int32_t* __restrict__ off, int64_t n, int64_t U,
                                                         int64_t ngroups, int64_t nseg, SegOut o,
                                                         const float* __restrict__ frag,
                                                         double* __restrict__ gfrag) {
  constexpr int PER = (D + 63) / 64;
  const int64_t UG = U * kSegGroup;
  const int ulog = __builtin_ctzll((unsigned long long)U);  // U is a power of two
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const int64_t g = blockIdx.x;
  if (g >= ngroups) {
    empty_fill_block(g - ngroups, off, nseg, D, o.C_prev, o.C_new, o.counts);
    return;
  }
  const int64_t gr0 = g * UG;
  if (gr0 >= n) return;
  const int64_t gr1 = gr0 + UG < n ? gr0 + UG : n;
  const int64_t kf = kv[gr0].x, kl = kv[gr1 - 1].x;
  int turn = 0;  // crossing segments seen so far in this group
  for (int64_t k0 = kf; k0 <= kl; k0 += 64) {
    const int64_t kk = k0 + lane;
    const bool valid = kk <= kl;
    const int64_t sv = valid ? off[kk] : 0, ev = valid ? off[kk + 1] : 0;
    // crosses a chunk edge (a segment inside one chunk was finished at level 1)
    const bool cross = valid && sv < ev && ((sv >> ulog) != ((ev - 1) >> ulog));
    uint64_t all = __ballot(cross);
    // this wave's share: every 4th crossing segment in order
    uint64_t mask = 0;
    for (uint64_t m = all; m; m &= m - 1, ++turn)
      if ((turn & 3) == w) mask |= m & (~m + 1);
    while (mask) {
      const int j = __ffsll((unsigned long long)mask) - 1;
      mask &= mask - 1;
      const int64_t k = k0 + j;
      const int64_t s = __shfl(sv, j), e = __shfl(ev, j);
      const int64_t a = s > gr0 ? s : gr0;
      const int64_t z = e < gr1 ? e : gr1;
      double acc[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) acc[q] = 0.0;
      const int64_t u0 = a >> ulog, u1 = (z - 1) >> ulog;
#pragma unroll 4
      for (int64_t u = u0; u <= u1; ++u) {
        const float* fp = frag + (u * 2 + frag_slot(u, ulog, s)) * D;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int d = lane + 64 * q;
          if (d < D) acc[q] += (double)fp[d];
        }
      }
      if (s >= gr0 && e <= gr1) {
        finish<T, D>(o, k, lane, acc, e - s);
      } else {
        double* gp = gfrag + (g * 2 + ((k == kf) ? 0 : 1)) * D;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int d = lane + 64 * q;
          if (d < D) gp[d] = acc[q];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// level 3: segments that cross a group edge
// ---------------------------------------------------------------------------
// A segment crossing into group g from the left and ending in it is owned by
// g.  One workgroup of kL3Waves waves covers kL3Waves groups: each wave checks
// its group's ownership and finishes an owned segment spanning at most
// kL3Waves groups by itself; longer segments are then summed by all waves
// together (interleaved by wave, combined in wave order).
constexpr int kL3Waves = 16;
template <class T, int D>
__global__ __launch_bounds__(kL3Waves * 64) void seg_level3_kernel(const uint2* __restrict__ kv,
                                                                   const int32_t* __restrict__ off, int64_t n,
                                                                   int64_t U, int64_t ngroups, SegOut o,
                                                                   const double* __restrict__ gfrag) {
  constexpr int PER = (D + 63) / 64;
  const int64_t UG = U * kSegGroup;
  const int glog = __builtin_ctzll((unsigned long long)UG);  // UG is a power of two
  __shared__ double part[kL3Waves][PER * 64];
  __shared__ int64_t own_k[kL3Waves], own_s[kL3Waves], own_e[kL3Waves];
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  {
    const int64_t g = (int64_t)blockIdx.x * kL3Waves + w;
    int64_t k = -1, s = 0, e = 0;
    if (g < ngroups) {
      const int64_t gr0 = g * UG;
      const int64_t gr1 = gr0 + UG < n ? gr0 + UG : n;
      const int64_t kk = kv[gr0].x;
      s = off[kk];
      e = off[kk + 1];
      if (s < gr0 && e <= gr1) k = kk;
    }
    if (k >= 0 && g - (s >> glog) < kL3Waves) {
      // short span: this wave alone, in group order
      double acc[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) acc[q] = 0.0;
#pragma unroll 4
      for (int64_t gg = s >> glog; gg <= g; ++gg) {
        const double* gp = gfrag + (gg * 2 + frag_slot(gg, glog, s)) * D;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int d = lane + 64 * q;
          if (d < D) acc[q] += gp[d];
        }
      }
      finish<T, D>(o, k, lane, acc, e - s);
      k = -1;
    }
    if (lane == 0) {
      own_k[w] = k;
      own_s[w] = s;
      own_e[w] = e;
    }
  }
  __syncthreads();
  for (int ow = 0; ow < kL3Waves; ++ow) {
    const int64_t k = own_k[ow];
    if (k < 0) continue;  // uniform over the workgroup: long segments only
    const int64_t s = own_s[ow], e = own_e[ow];
    const int64_t g_end = (int64_t)blockIdx.x * kL3Waves + ow;
    double acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) acc[q] = 0.0;
#pragma unroll 4
    for (int64_t gg = (s >> glog) + w; gg <= g_end; gg += kL3Waves) {
      const double* gp = gfrag + (gg * 2 + frag_slot(gg, glog, s)) * D;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int d = lane + 64 * q;
        if (d < D) acc[q] += gp[d];
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) part[w][lane + 64 * q] = acc[q];
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int d = lane + 64 * q;
        double v = 0.0;
#pragma unroll
        for (int i = 0; i < kL3Waves; ++i) v += part[i][d];
        acc[q] = v;
      }
      finish<T, D>(o, k, lane, acc, e - s);
    }
    __syncthreads();
  }
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

// The empty-cluster fill on its own (a problem of one chunk has no level 2).
__global__ __launch_bounds__(256) void empty_fill_kernel(const int32_t* __restrict__ off, int64_t nseg, int D,
                                                         const float* __restrict__ C_prev, float* __restrict__ C_new,
                                                         int32_t* __restrict__ counts) {
  empty_fill_block(blockIdx.x, off, nseg, D, C_prev, C_new, counts);
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t n16, uint8_t* __restrict__ tail,
                                                   int tail_bytes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
  if (i < tail_bytes) tail[i] = 0;
}

template <class T, int D, int U>
void seg_level1_launch(const void* X, const uint2* kv, int32_t* off, int64_t n, uint32_t nseg, const SegOut& o,
                       SegBuffers& buf, hipStream_t s) {
  const dim3 g1((unsigned)((seg_chunks(n) + 3) / 4));
  if (o.S_acc)
    seg_level1_kernel<T, D, true, U><<<g1, dim3(256), 0, s>>>(reinterpret_cast<const typename T::raw*>(X), kv, n,
                                                              nseg, off, o, buf.frag);
  else
    seg_level1_kernel<T, D, false, U><<<g1, dim3(256), 0, s>>>(reinterpret_cast<const typename T::raw*>(X), kv, n,
                                                               nseg, off, o, buf.frag);
}

template <class T, int D>
hipError_t seg_reduce_t(const void* X, const uint2* kv, int32_t* off, int64_t n, uint32_t nseg, const SegOut& o,
                        SegBuffers& buf, hipStream_t s) {
  const int64_t nchunks = seg_chunks(n);
  const int64_t ngroups = seg_groups(n);
  const int64_t U = seg_rows(n);
  if (U == kSegRowsSmall)
    seg_level1_launch<T, D, kSegRowsSmall>(X, kv, off, n, nseg, o, buf, s);
  else
    seg_level1_launch<T, D, kSegRows>(X, kv, off, n, nseg, o, buf, s);
  const int64_t fill_blocks = o.S_acc ? 0 : ((int64_t)nseg + 255) / 256;
  if (nchunks > 1) {
    // level 2, with the empty-cluster fill in the same launch
    seg_level2_kernel<T, D><<<dim3((unsigned)(ngroups + fill_blocks)), dim3(256), 0, s>>>(
        kv, off, n, U, ngroups, (int64_t)nseg, o, buf.frag, buf.gfrag);
    if (ngroups > 1)
      seg_level3_kernel<T, D><<<dim3((unsigned)((ngroups + kL3Waves - 1) / kL3Waves)), dim3(kL3Waves * 64), 0, s>>>(
          kv, off, n, U, ngroups, o, buf.gfrag);
  } else if (fill_blocks) {
    empty_fill_kernel<<<dim3((unsigned)fill_blocks), dim3(256), 0, s>>>(off, nseg, D, o.C_prev, o.C_new, o.counts);
  }
  return hipGetLastError();
}

template <class T>
hipError_t seg_reduce_d(int D, const void* X, const uint2* kv, int32_t* off, int64_t n, uint32_t nseg,
                        const SegOut& o, SegBuffers& buf, hipStream_t s) {
  switch (D) {
    case 16: return seg_reduce_t<T, 16>(X, kv, off, n, nseg, o, buf, s);
    case 32: return seg_reduce_t<T, 32>(X, kv, off, n, nseg, o, buf, s);
    case 64: return seg_reduce_t<T, 64>(X, kv, off, n, nseg, o, buf, s);
    case 128: return seg_reduce_t<T, 128>(X, kv, off, n, nseg, o, buf, s);
    case 256: return seg_reduce_t<T, 256>(X, kv, off, n, nseg, o, buf, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_segment_reduce(int dt, int D, const void* X, const uint2* sorted, int32_t* off, int64_t n,
                                 uint32_t nseg, const SegOut& out, SegBuffers& buf, hipStream_t s) {
  switch (dt) {
    case DT_F32: return seg_reduce_d<F32>(D, X, sorted, off, n, nseg, out, buf, s);
    case DT_F16: return seg_reduce_d<F16>(D, X, sorted, off, n, nseg, out, buf, s);
    case DT_BF16: return seg_reduce_d<BF16>(D, X, sorted, off, n, nseg, out, buf, s);
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
