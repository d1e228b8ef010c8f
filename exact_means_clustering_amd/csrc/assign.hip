// Assignment stage: centroid preparation and the fused distance + running
// argmin kernel ("FlashAssign" in the Flash-KMeans paper page, abstract, and
// the article section "Flash-KMeans が変える点", first point: the distance
// computation is fused with an online argmin so the N x K distance matrix is
// never written to memory).
//
// Score form.  For a point x and a rounded centroid c,
//     ||x - c||^2 = ||x||^2 - 2 (x.c - 0.5 ||c||^2),
// so the nearest centroid maximises s = x.c + hb with hb = -0.5 ||c||^2.
// The MFMA accumulator is seeded with hb (exact: a power-of-two scaling of
// the fp32 norm), so the matrix unit produces s directly and the epilogue is
// a pure running max.
//
// Layout.  A 32x32 MFMA output tile has the 32 tile centroids on its rows and
// 32 points on its columns: lane l owns point l%32 and the 16 centroid rows
// 8*(r/4) + 4*(l/32) + r%4 (r = accumulator register).  So each lane keeps a
// private (max, argmax) per point and needs no cross-lane work until the
// very end, where the two lane halves of a point merge once.
// The contraction index is permuted so that lane half h feeds the
// contiguous dims [h*D/2, (h+1)*D/2) of its row: point fragments are then
// single contiguous loads and stay in registers for the whole sweep, and
// centroid fragments are contiguous 16-byte LDS reads.
//
// Pipeline.  Centroids stream through a double-buffered LDS tile (16-byte
// chunks XOR-swizzled by row so a 32-row fragment read is free of bank
// conflicts), loaded straight from global memory into LDS; the loads of
// tile t+1 are issued before the MFMAs of tile t.  One barrier per tile.
#include "common.h"
#include "kernels.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>

namespace fkm {

// ---------------------------------------------------------------------------
// centroid preparation: Chat = RNE(C -> dtype), hb = -0.5 ||Chat||^2 (fp32)
// ---------------------------------------------------------------------------
// One wave per slot of the padded bias array [B][Kp]: slots k < K prepare
// centroid k of their instance, slots k >= K hold -inf (never chosen).
template <class T, int D>
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ C, typename T::raw* __restrict__ Ch,
                                                   float* __restrict__ hb, int64_t B, int K, int Kp,
                                                   const float* __restrict__ log_w, float sigma2) {
  const int lane = lane_id();
  const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slot >= B * Kp) return;
  const int64_t b = slot / Kp;
  const int k = (int)(slot - b * Kp);
  if (k >= K) {
    if (lane == 0) hb[slot] = -INFINITY;
    return;
  }
  const int64_t row = b * K + k;
  constexpr int PER = (D + 63) / 64;
  float c[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int d = lane + 64 * j;
    c[j] = d < D ? C[row * D + d] : 0.f;
  }
  const float ss = prep_row<T, D>(c, Ch + row * D, lane);
  // mixture log-weights enter the score as sigma2 * log w_k (soft assignment)
  if (lane == 0) hb[slot] = -0.5f * ss + (log_w ? sigma2 * log_w[row] : 0.f);
}

// ---------------------------------------------------------------------------
// fused assign
// ---------------------------------------------------------------------------
template <class T, int D, int PB, int W>
struct AssignCfg {
  static constexpr int RB = D * T::SZ;                 // bytes per row
#ifndef FKM_TK
  // centroids per LDS tile: 256 for 8-wave workgroups (one per CU, fewer
  // barriers), 128 otherwise; 64 for rows over 256 bytes
  static constexpr int TK = RB <= 256 ? (W == 8 ? 256 : 128) : 64;
#else
  static constexpr int TK = RB <= 256 ? FKM_TK : 64;
#endif
#ifndef FKM_SBG
  static constexpr int SBG = 1;                        // 32-centroid sub-blocks per MFMA group
#else
  static constexpr int SBG = FKM_SBG;
#endif
#ifndef FKM_DELAY
  static constexpr bool DELAY = true;                  // reduce group j-1 behind group j's MFMAs
#else
  static constexpr bool DELAY = FKM_DELAY;
#endif
#ifndef FKM_APF
  static constexpr bool APF = false;                   // prefetch the next group's A fragments
#else
  static constexpr bool APF = FKM_APF;
#endif
  static constexpr int NCH = RB / 16;                  // 16-byte chunks per row
  static constexpr int HV = NCH / 2;                   // chunks per lane-half fragment
  static constexpr int STEPS = (D / 2) / T::KPL;       // MFMA steps per 32x32 tile
  static constexpr int TILE_CH = TK * NCH;             // chunks per LDS tile
  static constexpr int THREADS = W * 64;
  static constexpr int DMA_INSTS = TILE_CH / 64;                  // 64-lane LDS loads per tile
  static constexpr int DMA_PER_WAVE = (DMA_INSTS + W - 1) / W;    // per wave (upper bound)
  static constexpr int ROWS = W * 32 * PB;                       // points per workgroup
  static_assert(NCH >= 2 && (NCH & (NCH - 1)) == 0, "row must be a power-of-two number of 16B chunks");
  static_assert(TILE_CH % 64 == 0 && TK % 4 == 0 && TK / 4 <= 64, "tile must be whole 64-lane LDS loads");
};

__device__ __forceinline__ float max16(const f32x16& a) {
  float m0 = fmaxf(fmaxf(a[0], a[1]), a[2]);
  float m1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  float m2 = fmaxf(fmaxf(a[6], a[7]), a[8]);
  float m3 = fmaxf(fmaxf(a[9], a[10]), a[11]);
  float m4 = fmaxf(fmaxf(a[12], a[13]), a[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)), fmaxf(m4, a[15]));
}

// Running top-2 update for one lane and one 32-centroid tile: the 16 scores
// are visited in increasing centroid index, and strict comparisons keep the
// lower index first on equal scores.  Written with value selects only (a
// score not above the second best changes nothing): with branches the
// compiler selects between the state variables by address and moves them
// to scratch memory.
__device__ __forceinline__ void insert_top2(const f32x16& acc, float& b1, int& i1, float& b2, int& i2, int base) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float v = acc[r];
    const int idx = base + 8 * (r >> 2) + (r & 3);
    const bool gt1 = v > b1;
    const bool gt2 = v > b2;
    const float nb2 = gt1 ? b1 : (gt2 ? v : b2);
    const int ni2 = gt1 ? i1 : (gt2 ? idx : i2);
    b1 = gt1 ? v : b1;
    i1 = gt1 ? idx : i1;
    b2 = nb2;
    i2 = ni2;
  }
}

// Running (max, argmax) update for one lane and one 32-centroid tile whose
// maximum score is `tmax`.  `base` is the centroid index of accumulator
// register 0 for this lane.  Centroid indices grow with the register index,
// and a tile only replaces the running best on a strictly larger score, so
// ties keep the lowest index.
__device__ __forceinline__ void improve(const f32x16& acc, float tmax, float& best, int& bidx, int base) {
  if (tmax > best) {
    int r = 15;
#pragma unroll
    for (int rr = 14; rr >= 0; --rr)
      if (acc[rr] == tmax) r = rr;
    best = tmax;
    bidx = base + 8 * (r >> 2) + (r & 3);
  }
}

// Epilogue modes (what the running per-point state is):
//   kArgmax  (best score, its index): labels, min_d2, inertia partials;
//   kTop2    the two best (score, index) pairs, ties to the lower index:
//            labels [B,N,2] and both direct distances in `dist` [B,N,2];
//   kSoft    for the Gaussian-mixture log density (the bias then carries
//            sigma2 * log w_k): the best score and index plus the running
//            sum l = sum_k 2^(t_k - t_best) with t_k = score_k * log2(e) / sigma2;
//            labels = most responsible component, dist = log density, part =
//            per-wave sums of it;
//   kGauss   the same running maximum, and the signed sum
//            sum_k w_k 2^(t_k - t_best) (weights from the padded array
//            soft.wpad, staged in LDS with the tile): dist = the Gauss sum
//            sum_k w_k exp(-||x - c_k||^2 / (2 sigma2)), part = its sums,
//            labels = the nearest source.
enum AssignMode : int { kArgmax = 0, kTop2 = 1, kSoft = 2, kGauss = 3 };

// RES (argmax, 8 waves, all K centroids in one tile): a workgroup takes a
// contiguous run of jobs, so consecutive jobs share an instance and its
// centroid tile stays in LDS (reloaded, behind a barrier, only where the run
// enters the next instance), and a job needs no workgroup barrier.  With one
// point block per wave the second tile buffer stages points instead: each
// wave copies its next job's 32 rows there (global->LDS, XOR-swizzled like
// the tile) while it computes the current job, so a job starts from LDS
// instead of waiting on HBM.  With two blocks (512 points, too many to stage)
// the points load straight into registers, as in the plain kernel.  Products,
// their order and the epilogue are those of the plain configuration.
template <class T, int D, int PB, int W, int MODE, bool RES = false>
__global__ __launch_bounds__(W * 64) void assign_kernel(const typename T::raw* __restrict__ X,
                                                        const typename T::raw* __restrict__ Ch,
                                                        const float* __restrict__ hb, int64_t N, int K, int B,
                                                        int32_t* __restrict__ labels, float* __restrict__ min_d2,
                                                        double* __restrict__ part, SoftArgs soft) {
  using Cfg = AssignCfg<T, D, PB, W>;
  constexpr int NCH = Cfg::NCH, HV = Cfg::HV, STEPS = Cfg::STEPS;
  constexpr int TK = Cfg::TK;
  // the delayed reduction holds a second set of accumulators: there is room
  // for it at one point block, and at two for the argmax epilogue only
  constexpr bool DELAY = Cfg::DELAY && (MODE == kArgmax || PB == 1) && PB <= 2;
  __shared__ uint4 tile[2][Cfg::TILE_CH];
  __shared__ __align__(16) float tb[2][TK];  // read back as float4
  __shared__ __align__(16) float tw[MODE == kGauss ? 2 : 1][MODE == kGauss ? TK : 4];  // kGauss: weights
  static_assert(!RES || (MODE == kArgmax && (PB > 1 || TK == Cfg::ROWS)),
                "resident tile: argmax only; one point block stages a job's rows in a tile buffer");

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int ntiles = (K + TK - 1) / TK;
  const int64_t nblk = (N + Cfg::ROWS - 1) / Cfg::ROWS;  // point blocks per instance

  // Persistent loop over (instance, point block).  Every workgroup does the
  // same amount of work per block, so the workgroups resident on an XCD sweep
  // the centroids in step and share each tile through that XCD's L2.  (RES:
  // a contiguous, balanced run of jobs per workgroup.)
  int64_t jbeg = blockIdx.x, jend = nblk * B, jstep = gridDim.x;
  if constexpr (RES) {
    const int64_t nj = nblk * B, q = nj / gridDim.x, r = nj % gridDim.x, g = blockIdx.x;
    jbeg = g * q + (g < r ? g : r);
    jend = jbeg + q + (g < r ? 1 : 0);
    jstep = 1;
  }
  // RES: wave w's 32 rows of job j go to rows [32 w, 32 w + 32) of tile[1],
  // chunk c of row m at chunk (c ^ (m % NCH)) of that row; lane l of the
  // instruction i writes chunk 64 i + l of the wave's slice.
  auto stage_points = [&](int64_t j) {
    const int bj = (int)(j / nblk);
    const int64_t pj = (j - (int64_t)bj * nblk) * Cfg::ROWS + (int64_t)w * 32;
    const typename T::raw* Xj = X + (int64_t)bj * N * D;
#pragma unroll
    for (int i = 0; i < 32 * NCH / 64; ++i) {
      const int qc = i * 64 + lane;
      const int lr = qc / NCH, pc = qc % NCH;
      const int m = w * 32 + lr;
      int64_t n = pj + lr;
      n = n < N ? n : N - 1;
      const uint4* src = reinterpret_cast<const uint4*>(Xj + n * D) + (pc ^ (m & (NCH - 1)));
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&tile[1][w * 32 * NCH + i * 64],
                                       16, 0, 0);
    }
  };
  // point fragments straight from global memory: lane half h of the wave's
  // block p takes dims [h*D/2, (h+1)*D/2) of point p0 + 32 p + col (rows past
  // N read row N-1; their results are not written)
  auto load_points = [&](const typename T::raw* Xb, int64_t p0, uint4 (&xf)[PB][HV]) {
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      int64_t n = p0 + p * 32 + col;
      n = n < N ? n : N - 1;
      const uint4* src = reinterpret_cast<const uint4*>(Xb + n * D) + h * HV;
#pragma unroll
      for (int v = 0; v < HV; ++v) xf[p][v] = src[v];
    }
  };
  int cur_b = -1;
  if constexpr (RES && PB == 1) {
    if (jbeg < jend) stage_points(jbeg);
  }
  // RES: a job's results (this lane's label and distance, lane 0's wave
  // partial) are stored at the next job, after its wait for the staged
  // points: loads and stores share one counter, so stores issued at the end
  // of a job would make that wait also wait for their acknowledgement.
  int64_t pend_o[PB], pend_pi = -1;  // output index of the pending results (-1: none)
  int pend_l[PB];
  float pend_d[PB];
#pragma unroll
  for (int p = 0; p < PB; ++p) pend_o[p] = -1, pend_l[p] = 0, pend_d[p] = 0.f;
  double pend_p = 0.0;
  auto store_pending = [&]() {
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      if (pend_o[p] >= 0) {
        labels[pend_o[p]] = pend_l[p];
        if (min_d2) min_d2[pend_o[p]] = pend_d[p];
      }
      pend_o[p] = -1;
    }
    if (lane == 0 && pend_pi >= 0) part[pend_pi] = pend_p;
    pend_pi = -1;
  };
  for (int64_t job = jbeg; job < jend; job += jstep) {
    const int b = (int)(job / nblk);
    const int64_t blk = job - (int64_t)b * nblk;
    const typename T::raw* Xb = X + (int64_t)b * N * D;
    const typename T::raw* Cb = Ch + (int64_t)b * K * D;
    const float* hbb = hb + (int64_t)b * kpad(K);
    const int64_t p0 = blk * Cfg::ROWS + (int64_t)w * (PB * 32);


    // Tile t goes straight from global memory into LDS buffer `buf`
    // (global_load_lds: lane l of a wave writes 16 bytes at the instruction's
    // LDS base + 16*l), so nothing is staged in registers.  The XOR swizzle is
    // applied on the global side: LDS chunk q of the tile (row m = q / NCH,
    // physical chunk q % NCH) receives logical chunk (q % NCH) ^ (m % NCH) of
    // centroid row m.  Rows past K read row K-1 (their bias is -inf).  The
    // bias slice comes from the -inf-padded array in 16-byte pieces.
    auto issue_tile = [&](int t, int buf) {
#pragma unroll
      for (int i = 0; i < Cfg::DMA_PER_WAVE; ++i) {
        const int ins = i * W + w;  // wave-uniform instruction index within the tile
        if (ins < Cfg::DMA_INSTS) {
          const int q = ins * 64 + lane;
          const int m = q / NCH, pc = q % NCH;
          int k = t * TK + m;
          k = k < K ? k : K - 1;
          const uint4* src = reinterpret_cast<const uint4*>(Cb + (int64_t)k * D) + (pc ^ (m & (NCH - 1)));
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&tile[buf][ins * 64], 16,
                                           0, 0);
        }
      }
      if (w == W - 1 && lane < TK / 4) {
        const float4* src = reinterpret_cast<const float4*>(hbb + (int64_t)t * TK) + lane;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&tb[buf][0], 16, 0, 0);
      }
      if constexpr (MODE == kGauss) {
        // the weights of the tile's centroids (zero-padded like the bias)
        if (w == W - 2 && lane < TK / 4) {
          const float4* src = reinterpret_cast<const float4*>(soft.wpad + (int64_t)b * kpad(K) + (int64_t)t * TK) + lane;
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&tw[buf][0], 16, 0, 0);
        }
      }
    };
    // all of this wave's LDS loads have landed (then a barrier publishes them)
    auto wait_tile = [] { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ };

    float best[PB];
    int bidx[PB];
    float sec[PB];   // kTop2: second-best score and index
    int sidx[PB];
    float lsum[PB];  // kSoft: sum of 2^(t_k - t_best) over the centroids seen
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      best[p] = -INFINITY;
      bidx[p] = 0;
      sec[p] = -INFINITY;
      sidx[p] = -1;
      lsum[p] = 0.f;
    }

    // point fragments: lane half h holds dims [h*D/2, (h+1)*D/2) of point col
    uint4 xf[PB][HV];
    if constexpr (RES) {
      // a new instance: every wave is done with the old tile, then load it
      const bool fresh = b != cur_b;
      if (fresh) {
        __syncthreads();
        issue_tile(0, 0);
        cur_b = b;
      }
      if constexpr (PB > 1) load_points(Xb, p0, xf);
      wait_tile();  // this wave's points (staged or loaded) and the tile it copied have landed
      if (fresh) __syncthreads();
      store_pending();
      if constexpr (PB == 1) {
        const int m = w * 32 + col;
#pragma unroll
        for (int v = 0; v < HV; ++v) {
          const int c = h * HV + v;
          xf[0][v] = tile[1][m * NCH + (c ^ (m & (NCH - 1)))];
        }
        // the reads above complete before the next job's rows overwrite the slice
        __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */
        if (job + 1 < jend) stage_points(job + 1);
      }
    } else {
      load_points(Xb, p0, xf);
      issue_tile(0, 0);
      wait_tile();
      __syncthreads();
    }

    // The centroid tile is consumed in groups of G sub-blocks of 32
    // centroids: the G x PB accumulation chains of a group are issued
    // interleaved step by step.  With kDelay the running max of the previous
    // group is reduced on the vector ALU after the current group's MFMAs are
    // issued, so it runs while they execute (`prev` starts at -inf, so the
    // first reduction changes nothing).  With kPrefetchA the centroid
    // fragments of the next group are read from LDS while the current group
    // computes.
    constexpr int G = Cfg::SBG;
    constexpr int NG = TK / (32 * G);
    auto read_frag = [&](int buf, int sb, uint4* af) {
      const int m = sb * 32 + col;
#pragma unroll
      for (int v = 0; v < HV; ++v) {
        const int c = h * HV + v;
        af[v] = tile[buf][m * NCH + (c ^ (m & (NCH - 1)))];
      }
    };
    auto read_bias = [&](int buf, int sb, f32x16& bias) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 bq = *reinterpret_cast<const float4*>(&tb[buf][sb * 32 + 8 * q + 4 * h]);
        bias[4 * q + 0] = bq.x;
        bias[4 * q + 1] = bq.y;
        bias[4 * q + 2] = bq.z;
        bias[4 * q + 3] = bq.w;
      }
    };
    auto read_weights = [&](int buf, int sb, f32x16& wv) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 wq = *reinterpret_cast<const float4*>(&tw[MODE == kGauss ? buf : 0][sb * 32 + 8 * q + 4 * h]);
        wv[4 * q + 0] = wq.x;
        wv[4 * q + 1] = wq.y;
        wv[4 * q + 2] = wq.z;
        wv[4 * q + 3] = wq.w;
      }
    };
    auto reduce_group = [&](const f32x16 (&a)[G][PB], int base, const f32x16 (&wv)[G]) {
      float tmax[G][PB];
      bool any = false;
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int p = 0; p < PB; ++p) {
          tmax[j][p] = max16(a[j][p]);
          any |= tmax[j][p] > (MODE == kTop2 ? sec[p] : best[p]);
        }
      if constexpr (MODE == kSoft || MODE == kGauss) {
        // rescale the running sum to the new maximum, then add this group's
        // terms (a group of padding rows, all -inf, changes nothing)
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int p = 0; p < PB; ++p) {
            if (tmax[j][p] == -INFINITY) continue;
            const float mb = tmax[j][p] > best[p] ? tmax[j][p] : best[p];
            const float m2 = mb * soft.scale2;
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(fmaf(a[j][p][r], soft.scale2, -m2));
              if constexpr (MODE == kGauss) sum = fmaf(wv[j][r], e, sum);
              else sum += e;
            }
            lsum[p] = lsum[p] * __builtin_amdgcn_exp2f(best[p] * soft.scale2 - m2) + sum;
          }
      }
      if (any) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int p = 0; p < PB; ++p) {
            if constexpr (MODE == kTop2) {
              insert_top2(a[j][p], best[p], bidx[p], sec[p], sidx[p], base + 32 * j);
            } else {
              improve(a[j][p], tmax[j][p], best[p], bidx[p], base + 32 * j);
            }
          }
      }
    };

    f32x16 prev[G][PB];
    f32x16 wprev[G];  // kGauss: the weights of the delayed group
    int prev_base = 0;
    if constexpr (DELAY) {
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int p = 0; p < PB; ++p)
#pragma unroll
          for (int r = 0; r < 16; ++r) prev[j][p][r] = -INFINITY;
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) wprev[j][r] = 0.f;
    }

    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
      uint4 afn[G][HV];
      if constexpr (Cfg::APF) {
#pragma unroll
        for (int j = 0; j < G; ++j) read_frag(buf, j, afn[j]);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (t * TK + g * G * 32 >= K) break;  // the rest of the tile is -inf padding
        uint4 af[G][HV];
        if constexpr (Cfg::APF) {
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int v = 0; v < HV; ++v) af[j][v] = afn[j][v];
          if (g + 1 < NG) {
#pragma unroll
            for (int j = 0; j < G; ++j) read_frag(buf, (g + 1) * G + j, afn[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < G; ++j) read_frag(buf, g * G + j, af[j]);
        }
        f32x16 acc[G][PB];
        f32x16 wv[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          f32x16 bias;
          read_bias(buf, g * G + j, bias);
#pragma unroll
          for (int p = 0; p < PB; ++p) acc[j][p] = bias;
          if constexpr (MODE == kGauss) read_weights(buf, g * G + j, wv[j]);
        }
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int p = 0; p < PB; ++p) acc[j][p] = Mfma<T>::step(af[j], xf[p], st, acc[j][p]);
        const int base = t * TK + g * G * 32 + 4 * h;
        if constexpr (DELAY) {
          reduce_group(prev, prev_base, wprev);
#pragma unroll
          for (int i = 0; i < STEPS * PB * G; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int p = 0; p < PB; ++p) prev[j][p] = acc[j][p];
          if constexpr (MODE == kGauss) {
#pragma unroll
            for (int j = 0; j < G; ++j) wprev[j] = wv[j];
          }
          prev_base = base;
        } else {
          reduce_group(acc, base, wv);
        }
      }
      if constexpr (!RES) {  // (RES: the single tile stays; the next job waits for its own points)
        wait_tile();
        __syncthreads();
      }
    }
    if constexpr (DELAY) reduce_group(prev, prev_base, wprev);

    // squared distance of point block p to centroid k, computed directly (no
    // cancellation): each lane half sums its dims, the halves then add.
    // With a single centroid tile every centroid is still in LDS buffer 0
    // (row k, chunks swizzled as the tile was written), so the row is read
    // there instead of from global memory.  A workgroup barrier after the
    // distances keeps the next job's tile load from overwriting the buffer
    // first (RES reloads the tile only for a new instance, behind a barrier
    // of its own); kTop2 reads global memory.  The chunks are all loaded
    // before the first is used, and each half adds its squared differences
    // with fused multiply-adds in dimension order.
    auto direct_d2 = [&](int p, int k) -> float {
      const uint4* cr = reinterpret_cast<const uint4*>(Cb + (int64_t)k * D) + h * HV;
      const bool in_lds = MODE != kTop2 && ntiles == 1;
      uint4 cw[HV];
#pragma unroll
      for (int v = 0; v < HV; ++v) {
        const int c = h * HV + v;
        cw[v] = in_lds ? tile[0][k * NCH + (c ^ (k & (NCH - 1)))] : cr[v];
      }
      float part_d = 0.f;
#pragma unroll
      for (int v = 0; v < HV; ++v) part_d = Vec<T>::sq_add(xf[p][v], cw[v], part_d);
      const float other = __shfl_xor(part_d, 32);
      return h == 0 ? part_d + other : other + part_d;
    };
    // larger score, then lower index
    auto better = [](float s1, int i1, float s2, int i2) { return s1 > s2 || (s1 == s2 && i1 < i2); };

    // merge the two lane halves of each point and write its results
    double wacc = 0.0;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const float ob = __shfl_xor(best[p], 32);
      const int oi = __shfl_xor(bidx[p], 32);
      const int64_t n = p0 + p * 32 + col;
      const bool writer = h == 0 && n < N;
      if constexpr (MODE == kTop2) {
        const float os = __shfl_xor(sec[p], 32);
        const int oj = __shfl_xor(sidx[p], 32);
        int k1, k2;
        if (better(best[p], bidx[p], ob, oi)) {
          k1 = bidx[p];
          k2 = better(sec[p], sidx[p], ob, oi) ? sidx[p] : oi;
        } else {
          k1 = oi;
          k2 = better(best[p], bidx[p], os, oj) ? bidx[p] : oj;
        }
        const float d1 = direct_d2(p, k1), d2 = direct_d2(p, k2);
        if (writer) {
          const int64_t o = 2 * ((int64_t)b * N + n);
          labels[o] = k1;
          labels[o + 1] = k2;
          if (min_d2) {
            min_d2[o] = d1;
            min_d2[o + 1] = d2;
          }
        }
      } else {
        float l = 0.f;
        if constexpr (MODE == kSoft || MODE == kGauss) {
          // combine the halves' sums at the larger maximum
          const float ol = __shfl_xor(lsum[p], 32);
          const float m2 = (ob > best[p] ? ob : best[p]) * soft.scale2;
          l = lsum[p] * __builtin_amdgcn_exp2f(best[p] * soft.scale2 - m2) +
              ol * __builtin_amdgcn_exp2f(ob * soft.scale2 - m2);
        }
        if (better(ob, oi, best[p], bidx[p])) {
          best[p] = ob;
          bidx[p] = oi;
        }
        const float d2 = direct_d2(p, bidx[p]);
        if constexpr (RES) {
          pend_o[p] = writer ? (int64_t)b * N + n : -1;
          pend_l[p] = bidx[p];
          pend_d[p] = d2;
          if (writer) wacc += (double)d2;
        } else if (writer) {
          labels[(int64_t)b * N + n] = bidx[p];
          if constexpr (MODE == kSoft) {
            // log sum_k w_k exp(-d_k / (2 sigma2)) = a_best + ln(sum_k 2^(t_k - t_best)),
            // anchored on the direct distance of the most responsible centroid
            const float lw = soft.log_w ? soft.log_w[(int64_t)b * K + bidx[p]] : 0.f;
            const float L = lw - d2 * soft.inv2s2 + __builtin_amdgcn_logf(l) * 0.693147180559945309f;
            min_d2[(int64_t)b * N + n] = L;
            wacc += (double)L;
          } else if constexpr (MODE == kGauss) {
            // sum_k w_k exp(-d_k / (2 sigma2)) = exp(-d_best / (2 sigma2)) * sum_k w_k 2^(t_k - t_best)
            const float Gs = l * __builtin_amdgcn_exp2f(-d2 * soft.inv2s2 * 1.44269504088896341f);
            min_d2[(int64_t)b * N + n] = Gs;
            wacc += (double)Gs;
          } else {
            if (min_d2) min_d2[(int64_t)b * N + n] = d2;
            wacc += (double)d2;
          }
        }
      }
    }
    if constexpr (MODE != kTop2) {
      // one partial per wave and job, in a fixed place (no atomics, no barrier)
      wacc = wave_sum_f64(wacc);
      const int64_t pi = ((int64_t)b * nblk + blk) * W + w;
      if constexpr (RES) {
        pend_pi = pi;
        pend_p = wacc;
      } else {
        if (lane == 0) part[pi] = wacc;
        // the next job reloads tile buffer 0, which direct_d2 read
        if (ntiles == 1) __syncthreads();
      }
    }
  }
  if constexpr (RES) store_pending();
}

// inertia[b] = fixed-order sum of part[b, :], one workgroup per instance
__global__ __launch_bounds__(256) void inertia_reduce_kernel(const double* __restrict__ part, int nwg,
                                                             double* __restrict__ inertia,
                                                             double* __restrict__ hist, int accumulate) {
  inertia_reduce_block(part, nwg, blockIdx.x, inertia, hist, accumulate != 0);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {

template <class T, int D>
hipError_t prep_t(const float* C, void* Chat, float* hb, int64_t B, int K, const float* log_w, float sigma2,
                  hipStream_t s) {
  const int64_t slots = B * kpad(K);
  const int64_t grid = (slots + 3) / 4;
  prep_kernel<T, D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(C, reinterpret_cast<typename T::raw*>(Chat), hb, B,
                                                                K, (int)kpad(K), log_w, sigma2);
  return hipGetLastError();
}

// Workgroup slots of the persistent grid on the current device: as many
// workgroups as fit at once (queried once per thread and device).
template <class T, int D, int PB, int W, int MODE, bool RES = false>
hipError_t assign_slots(int* slots) {
  using Cfg = AssignCfg<T, D, PB, W>;
  static thread_local int cached_dev = -1, cached_slots = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != cached_dev) {
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, assign_kernel<T, D, PB, W, MODE, RES>,
                                                          Cfg::THREADS, 0)) != hipSuccess)
      return e;
    cached_slots = cus * (per_cu > 0 ? per_cu : 1);
    cached_dev = dev;
  }
  *slots = cached_slots;
  return hipSuccess;
}

template <class T, int D, int PB, int W, int MODE, bool RES = false>
hipError_t assign_t(const void* X, const void* Chat, const float* hb, int64_t N, int K, int B, int32_t* labels,
                    float* min_d2, double* part, SoftArgs soft, hipStream_t s) {
  using Cfg = AssignCfg<T, D, PB, W>;
  const int64_t jobs = (N + Cfg::ROWS - 1) / Cfg::ROWS * (int64_t)B;
  int slots = 0;
  const hipError_t e = assign_slots<T, D, PB, W, MODE, RES>(&slots);
  if (e != hipSuccess) return e;
  const int64_t grid = jobs < slots ? jobs : slots;
  assign_kernel<T, D, PB, W, MODE, RES><<<dim3((unsigned)grid), dim3(Cfg::THREADS), 0, s>>>(
      reinterpret_cast<const typename T::raw*>(X), reinterpret_cast<const typename T::raw*>(Chat), hb, N, K, B,
      labels, min_d2, part, soft);
  return hipGetLastError();
}

// Compiled configurations.  The point fragments of PB blocks take
// PB * D * SZ / 8 VGPRs per lane, so deep blocking is limited to short rows.
// (8-wave workgroups run two waves per SIMD, i.e. 256 registers per wave.)
constexpr bool cfg_compiled(int elem_bytes, int row_bytes, int pb, int waves) {
  if (pb == 1 && waves == 4) return true;
  if (pb == 1 && waves == 8) return row_bytes <= 512;
  if (pb == 2 && waves == 4) return row_bytes <= 512;
  if (pb == 2 && waves == 8) return row_bytes <= 256;
  if (pb == 4 && waves == 4) return row_bytes <= 256;
  // (fp32 rows of 256 bytes spill inside the tile loop at three blocks)
  if (pb == 3 && waves == 8) return row_bytes <= (elem_bytes == 2 ? 256 : 128);
  return false;
}

// The top-2, soft and Gauss epilogues are compiled for one configuration per
// row size: two point blocks and 8 waves where the argmax kernel has that
// configuration (rows of at most 256 bytes), else one block and 8 waves
// when the row allows it.
constexpr int mode_pb(int row_bytes) { return row_bytes <= 256 ? 2 : 1; }
constexpr int mode_waves(int row_bytes) { return row_bytes <= 512 ? 8 : 4; }

template <class T, int D, int MODE>
hipError_t assign_cfg(AssignConfig c, const void* X, const void* Chat, const float* hb, int64_t N, int K, int B,
                      int32_t* labels, float* min_d2, double* part, SoftArgs soft, hipStream_t s) {
  constexpr int rb = D * T::SZ;
  if constexpr (MODE == kArgmax) {
    // one or two point blocks, 8 waves, all centroids in one 256-row tile:
    // the resident-tile form of that configuration
    if constexpr (rb <= 256 && AssignCfg<T, D, 1, 8>::TK == AssignCfg<T, D, 1, 8>::ROWS) {
      if (c.pb == 1 && c.waves == 8 && K <= AssignCfg<T, D, 1, 8>::TK)
        return assign_t<T, D, 1, 8, MODE, true>(X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
    }
    if constexpr (cfg_compiled(T::SZ, rb, 2, 8)) {
      if (c.pb == 2 && c.waves == 8 && K <= AssignCfg<T, D, 2, 8>::TK)
        return assign_t<T, D, 2, 8, MODE, true>(X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
    }
#define FKM_CASE(PB_, W_)                                                                      \
    if constexpr (cfg_compiled(T::SZ, rb, PB_, W_)) {                                          \
      if (c.pb == PB_ && c.waves == W_)                                                        \
        return assign_t<T, D, PB_, W_, MODE>(X, Chat, hb, N, K, B, labels, min_d2, part, soft, s); \
    }
    FKM_CASE(4, 4)
    FKM_CASE(3, 8)
    FKM_CASE(2, 8)
    FKM_CASE(2, 4)
    FKM_CASE(1, 8)
    FKM_CASE(1, 4)
#undef FKM_CASE
  } else {
    constexpr int MP = mode_pb(rb), MW = mode_waves(rb);
    if (c.pb == MP && c.waves == MW)
      return assign_t<T, D, MP, MW, MODE>(X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int D>
hipError_t assign_prime_cfg(AssignConfig c) {
  constexpr int rb = D * T::SZ;
  int slots = 0;
  // (1, 8) and (2, 8) may launch their resident-tile forms: query those too
  if constexpr (rb <= 256 && AssignCfg<T, D, 1, 8>::TK == AssignCfg<T, D, 1, 8>::ROWS) {
    if (c.pb == 1 && c.waves == 8) {
      const hipError_t e = assign_slots<T, D, 1, 8, kArgmax, true>(&slots);
      if (e != hipSuccess) return e;
    }
  }
  if constexpr (cfg_compiled(T::SZ, rb, 2, 8)) {
    if (c.pb == 2 && c.waves == 8) {
      const hipError_t e = assign_slots<T, D, 2, 8, kArgmax, true>(&slots);
      if (e != hipSuccess) return e;
    }
  }
#define FKM_CASE(PB_, W_)                                              \
  if constexpr (cfg_compiled(T::SZ, rb, PB_, W_)) {                    \
    if (c.pb == PB_ && c.waves == W_) return assign_slots<T, D, PB_, W_, kArgmax>(&slots); \
  }
  FKM_CASE(4, 4)
  FKM_CASE(3, 8)
  FKM_CASE(2, 8)
  FKM_CASE(2, 4)
  FKM_CASE(1, 8)
  FKM_CASE(1, 4)
#undef FKM_CASE
  return hipErrorInvalidValue;
}

template <template <class, int> class F, class... A>
hipError_t dispatch_dt_d(int dt, int D, A&&... a) {
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

template <class T, int D> struct PrepF {
  static hipError_t run(const float* C, void* Chat, float* hb, int64_t B, int K, const float* log_w, float sigma2,
                        hipStream_t s) {
    return prep_t<T, D>(C, Chat, hb, B, K, log_w, sigma2, s);
  }
};
template <class T, int D> struct PrimeF {
  static hipError_t run(AssignConfig c) { return assign_prime_cfg<T, D>(c); }
};
template <class T, int D> struct AssignF {
  static hipError_t run(int mode, AssignConfig c, const void* X, const void* Chat, const float* hb, int64_t N, int K,
                        int B, int32_t* labels, float* min_d2, double* part, SoftArgs soft, hipStream_t s) {
    switch (mode) {
      case kArgmax: return assign_cfg<T, D, kArgmax>(c, X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
      case kTop2: return assign_cfg<T, D, kTop2>(c, X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
      case kSoft: return assign_cfg<T, D, kSoft>(c, X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
      case kGauss: return assign_cfg<T, D, kGauss>(c, X, Chat, hb, N, K, B, labels, min_d2, part, soft, s);
      default: return hipErrorInvalidValue;
    }
  }
};

}  // namespace

namespace {
// FLASHKM_ASSIGN_CONFIG="pb,waves", parsed once; {0,0} when unset or malformed.
AssignConfig env_override() {
  static const AssignConfig c = [] {
    AssignConfig r{0, 0};
    if (const char* e = getenv("FLASHKM_ASSIGN_CONFIG")) {
      int pb = 0, w = 0;
      if (sscanf(e, "%d,%d", &pb, &w) == 2) r = AssignConfig{pb, w};
    }
    return r;
  }();
  return c;
}
}  // namespace

bool assign_config_compiled(int dt, int D, AssignConfig c) {
  return cfg_compiled(dtype_size(dt), D * dtype_size(dt), c.pb, c.waves);
}

int assign_configs(int dt, int D, AssignConfig* out, int cap) {
  const AssignConfig all[] = {{4, 4}, {3, 8}, {2, 8}, {2, 4}, {1, 8}, {1, 4}};
  int n = 0;
  for (const AssignConfig& c : all)
    if (n < cap && assign_config_compiled(dt, D, c)) out[n++] = c;
  return n;
}

AssignConfig assign_pick(int dt, int D, int64_t N, int B, int K) {
  const int rb = D * dtype_size(dt);
  const AssignConfig o = env_override();
  const int sz = dtype_size(dt);
  if (o.pb && cfg_compiled(sz, rb, o.pb, o.waves)) return o;
  AssignConfig tuned;
  if (tune_lookup(dt, D, N, B, K, &tuned) && cfg_compiled(sz, rb, tuned.pb, tuned.waves)) return tuned;
  // Two waves per SIMD (8-wave workgroups) so one wave's argmax epilogue
  // overlaps the other's MFMAs; the deepest register blocking that still
  // leaves >= 4 workgroups per CU.  Three point blocks (no delayed
  // reduction) reuse each centroid fragment 1.5x more and pay off when every
  // workgroup sweeps many tiles over many jobs (measured: 3.7% at N = 2^23,
  // K = 65,536); with few tiles per job or few jobs per workgroup the job
  // overheads and the uneven last round lose more.
  const bool long_sweep = K >= 8192 && (N + 767) / 768 * (int64_t)B >= 4096;
  if (long_sweep && cfg_compiled(sz, rb, 3, 8)) return AssignConfig{3, 8};
  // All centroids in one tile (rows of at most 256 bytes, K <= 256) and at
  // least 2048 jobs: the resident-tile forms keep each instance's tile in LDS
  // with no per-job barrier.  With 2048 jobs of 512 points, two point blocks
  // (half the centroid-fragment reads per MFMA) beat one block with staged
  // points (64 instances of 16,384 points, K = 256: 0.108-0.120 against
  // 0.114-0.130 ms); with fewer, one block with the next job's points staged
  // while the current one computes (5.6% more fit iterations than the plain
  // kernel at that shape; no change at 2^16 points, K = 64).
  if (rb <= 256 && K <= 256) {
    if ((N + 511) / 512 * (int64_t)B >= 2048 && cfg_compiled(sz, rb, 2, 8)) return AssignConfig{2, 8};
    if ((N + 255) / 256 * (int64_t)B >= 2048) return AssignConfig{1, 8};
  }
  const AssignConfig order[] = {{2, 8}, {1, 8}, {1, 4}};
  for (const AssignConfig& c : order) {
    if (!cfg_compiled(sz, rb, c.pb, c.waves)) continue;
    const int64_t wgs = (N + c.rows() - 1) / c.rows() * (int64_t)B;
    if (wgs >= 1024) return c;
  }
  return AssignConfig{1, 4};
}

hipError_t launch_prep(int dt, int D, const float* C, void* Chat, float* hb, int64_t B, int K, hipStream_t s,
                       const float* log_w, float sigma2) {
  return dispatch_dt_d<PrepF>(dt, D, C, Chat, hb, B, K, log_w, sigma2, s);
}

hipError_t launch_assign(int dt, int D, AssignConfig cfg, const void* X, const void* Chat, const float* hb, int64_t N,
                         int K, int B, int32_t* labels, float* min_d2, double* part, hipStream_t s) {
  return dispatch_dt_d<AssignF>(dt, D, (int)kArgmax, cfg, X, Chat, hb, N, K, B, labels, min_d2, part, SoftArgs{},
                                s);
}

AssignConfig mode_config(int dt, int D) {
  const int rb = D * dtype_size(dt);
  return AssignConfig{mode_pb(rb), mode_waves(rb)};
}

hipError_t launch_assign_top2(int dt, int D, const void* X, const void* Chat, const float* hb, int64_t N, int K, int B,
                              int32_t* labels2, float* d2, hipStream_t s) {
  return dispatch_dt_d<AssignF>(dt, D, (int)kTop2, mode_config(dt, D), X, Chat, hb, N, K, B, labels2, d2,
                                (double*)nullptr, SoftArgs{}, s);
}

hipError_t launch_assign_soft(int dt, int D, const void* X, const void* Chat, const float* hb, int64_t N, int K, int B,
                              int32_t* labels, float* logp, double* part, SoftArgs soft, hipStream_t s) {
  return dispatch_dt_d<AssignF>(dt, D, (int)kSoft, mode_config(dt, D), X, Chat, hb, N, K, B, labels, logp, part,
                                soft, s);
}

hipError_t launch_assign_gauss(int dt, int D, const void* X, const void* Chat, const float* hb, int64_t N, int K,
                               int B, int32_t* labels, float* gsum, double* part, SoftArgs soft, hipStream_t s) {
  return dispatch_dt_d<AssignF>(dt, D, (int)kGauss, mode_config(dt, D), X, Chat, hb, N, K, B, labels, gsum, part,
                                soft, s);
}

namespace {
__global__ __launch_bounds__(256) void pad_weights_kernel(const float* __restrict__ w, float* __restrict__ wpad,
                                                          int64_t B, int K, int Kp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= B * Kp) return;
  const int64_t b = i / Kp;
  const int k = (int)(i - b * Kp);
  wpad[i] = k < K ? w[b * K + k] : 0.f;
}
}  // namespace

hipError_t launch_pad_weights(const float* w, float* wpad, int64_t B, int K, hipStream_t s) {
  const int64_t n = B * kpad(K);
  pad_weights_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(w, wpad, B, K, (int)kpad(K));
  return hipGetLastError();
}

hipError_t assign_prime(int dt, int D, AssignConfig cfg) { return dispatch_dt_d<PrimeF>(dt, D, cfg); }

hipError_t launch_inertia_reduce(const double* part, int nwg, int B, double* inertia, double* hist, bool accumulate,
                                 hipStream_t s) {
  inertia_reduce_kernel<<<dim3((unsigned)B), dim3(256), 0, s>>>(part, nwg, inertia, hist, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fkm
