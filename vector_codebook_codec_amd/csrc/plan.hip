// Nearest-centroid search plan: for a fixed codebook, a grid over the plane
// whose every cell lists the centroids that can be the nearest one, under the
// encode kernels' fp32 scores, for some point of the cell.  The encode kernel
// then scores only a pair's cell list instead of all K centroids and returns
// the same index as the exhaustive search ("QAM-W: Joint 2D Codebook
// Quantization for LLM Weights via Hadamard Rotation and Activation-Aware
// Scaling"; Methodology: Joint 2D Quantization -- the nearest centroid in one
// 2D codebook).
//
// Why the lists are complete.  Let Q be a cell enlarged by eta, U(Q) =
// min_c max_{z in Q} |z - c|^2.  For z in Q the exact nearest centroid c*
// has |z - c*|^2 <= U(Q).  The kernels decide on fp32 scores S32(c) with
// |S32(c) - (|c|^2/2 - z.c)| <= e(c), e(c) <= 2^-24 (2.5 |c|^2 + 2 |z||c|)
// for the FMA sequence they use, so their choice c32 (and every centroid tied
// with it) satisfies |z - c32|^2 <= |z - c*|^2 + 2 (e(c32) + e(c*)), hence
// min_{z in Q} |z - c32|^2 <= U(Q) + delta whenever delta covers that slack.
// A list holds exactly the centroids passing that test, in ascending index
// order, so the first minimum met while scanning it is the lowest-index fp32
// minimum over the whole codebook.  delta is 1e-5 (Cmax + R sqrt 2)^2, about
// 10x the slack bound for points inside the grid; eta (1e-4) covers the fp32
// rounding of the cell index.  Points outside the grid, and cells whose list
// would exceed lmax entries, fall back to the exhaustive scan.
//
// Construction is two-level and gives the same lists as testing every
// centroid against every cell.  A supercell SQ (a square block of cells) first keeps
// the centroids with min_{z in SQ} |z - c|^2 <= U(SQ) + 2 delta.  Every
// centroid of a cell's list passes that test (SQ contains Q, so its minimum
// distances are smaller and U(SQ) >= U(Q)), and so does the centroid that
// attains U(Q); the cells then test only the supercell's survivors.
//
// Two grids: a fine one (G = 512 over [-5, 5)^2) where nearly all normalised
// pairs fall, and a coarse outer one (256 over [-40, 40)^2) for the few pairs
// beyond it -- rows dominated by one large weight put a whole Hadamard block
// there.  Each has its own delta (R = 5 or 40 in the formula above).  The
// outer cells that tile the fine grid's square are never consulted (points
// there take the fine grid) and hold overflow records.
//
// Layout (plan_bytes(K) bytes, 256-byte aligned):
//   [0, 256)     PlanHeader
//   [256, ...)   fine grid: uint16 lists [G*G][lmax], then the outer grid's
//                [G2*G2][lmax]; one 16- or 32-byte record per cell.
//                Entry i is 16 c_i | nibble_i: c_i the i-th listed centroid
//                (16 c_i is its byte offset in the encode kernel's LDS copy of
//                the codebook), nibble_0 = count - 1, nibble_1 = 1 when the
//                cell overflows (scan the whole codebook), other nibbles 0;
//                entries past the count repeat the last listed centroid.
// In a grid of G cells per axis over [-R, R)^2, cell (ix, iy) covers
// [-R + ix s, -R + (ix+1) s) x [-R + iy s, ...), s = 2R/G; its index is
// ix * G + iy.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

struct PlanHeader {
  float R;
  float cells_per_unit;   // G / (2 R)
  int G;
  int lmax;
  int K;
  float R2;               // outer grid
  float cells_per_unit2;
  int G2;
};
static_assert(offsetof(PlanHeader, K) == kPlanHeaderKOffset, "the encode kernel reads K at this offset");

constexpr double kPlanEta = 1e-4;
constexpr int kSuperMax = 2048;                    // survivors kept; more -> test all K
constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / kWave;

constexpr int kPerThread = kSuperMax / kPlanThreads;   // centroids one thread tests in the survivor pass

// Axis-aligned box [x0, x1] x [y0, y1] against centroid (cx, cy).
struct Box {
  double x0, x1, y0, y1;
  __device__ double dmax2(double cx, double cy) const {
    const double ax = fmax((cx - x0) * (cx - x0), (cx - x1) * (cx - x1));
    const double ay = fmax((cy - y0) * (cy - y0), (cy - y1) * (cy - y1));
    return ax + ay;
  }
  __device__ double dmin2(double cx, double cy) const {
    const double dx = fmax(fmax(x0 - cx, cx - x1), 0.0);
    const double dy = fmax(fmax(y0 - cy, cy - y1), 0.0);
    return dx * dx + dy * dy;
  }
};

// The same tests in fp32 on a box widened outward to the next floats: its
// distances bound the fp64 box's from the safe side (dmax2 larger, dmin2
// smaller) up to fp32 rounding (< 3 2^-24 relative), which the callers'
// 1e-6 margins cover.
struct BoxF {
  float x0, x1, y0, y1;
  __device__ float dmax2(float cx, float cy) const {
    const float ax = fmaxf(fabsf(cx - x0), fabsf(cx - x1));
    const float ay = fmaxf(fabsf(cy - y0), fabsf(cy - y1));
    return ax * ax + ay * ay;
  }
  __device__ float dmin2(float cx, float cy) const {
    const float dx = fmaxf(fmaxf(x0 - cx, cx - x1), 0.0f);
    const float dy = fmaxf(fmaxf(y0 - cy, cy - y1), 0.0f);
    return dx * dx + dy * dy;
  }
};

// the next float above a finite f, and the largest float <= / smallest >= v
__device__ __forceinline__ float float_next_up(float f) {
  const uint32_t u = __float_as_uint(f);
  return f > 0.0f ? __uint_as_float(u + 1u) : (f < 0.0f ? __uint_as_float(u - 1u) : __uint_as_float(1u));
}
__device__ __forceinline__ float f32_down(double v) {
  const float f = (float)v;
  return (double)f > v ? -float_next_up(-f) : f;
}
__device__ __forceinline__ float f32_up(double v) {
  const float f = (float)v;
  return (double)f < v ? float_next_up(f) : f;
}

__device__ __forceinline__ Box cell_box(double R, int G, int ix0, int iy0, int ncells) {
  const double s = 2.0 * R / G;
  return Box{-R + ix0 * s - kPlanEta, -R + (ix0 + ncells) * s + kPlanEta,
             -R + iy0 * s - kPlanEta, -R + (iy0 + ncells) * s + kPlanEta};
}

__device__ __forceinline__ double wave_min(double v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = fmin(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}

struct PlanShared {
  uint16_t surv[kSuperMax];
  float2 survc[kSuperMax];
  uint16_t cell_list[kPlanThreads][16];
  double red[kPlanWaves];
  double red2[kPlanWaves];
  int wsum[kPlanWaves];
};

// One workgroup per supercell (S x S cells) of a G x G grid over [-R, R)^2:
// the supercell's survivors (ascending, with coordinates) into LDS, then a
// group of LPC = 256 / S^2 lanes per cell scans them and writes the records.
template <int S>
__device__ void build_supercell(PlanShared& sh, const float* __restrict__ cb, int K, int lmax, double R, int G,
                                int sidx, uint16_t* __restrict__ lists) {
  constexpr int LPC = kPlanThreads / (S * S);
  static_assert(LPC >= 1 && LPC * S * S == kPlanThreads && kWave % LPC == 0, "cell groups tile the wavefronts");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nsuper = G / S;
  const int sx = sidx / nsuper, sy = sidx % nsuper;

  // ---- the codebook into registers once: thread t holds centroids
  // r kSuperMax + t P + u (round r < 2 since K <= 4096, u < P = kPerThread),
  // loaded as float4 pairs; past K a far-away dummy that never passes a test
  constexpr int kRounds = 4096 / kSuperMax;
  float2 v[kRounds][kPerThread];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int c0 = r * kSuperMax + tid * kPerThread;
    const float4* p4 = reinterpret_cast<const float4*>(cb + 2 * c0);
#pragma unroll
    for (int u = 0; u < kPerThread; u += 2) {
      float4 t = make_float4(1e30f, 1e30f, 1e30f, 1e30f);
      if (c0 + u + 1 < K) t = p4[u / 2];
      else if (c0 + u < K) t = make_float4(cb[2 * (c0 + u)], cb[2 * (c0 + u) + 1], 1e30f, 1e30f);
      v[r][u] = make_float2(t.x, t.y);
      v[r][u + 1] = make_float2(t.z, t.w);
    }
  }
  // ---- U(SQ) and the largest squared centroid radius, from the registers,
  // in fp32 on the outward-widened supercell box: U is raised by 1e-6 and the
  // survivor limit U + 2 delta by 1e-6 again, so the survivors can only be
  // more.  They stay a superset of every cell's candidates: the widened cell
  // boxes lie inside the widened supercell box, and the supercell limit's
  // second delta exceeds the cells' relative fp32 slop (~3e-6 U) at every
  // grid point.  delta (fp64) only needs to cover the scores' slack, which
  // it does ten times over.
  const Box sq64 = cell_box(R, G, sx * S, sy * S, S);
  const BoxF sq{f32_down(sq64.x0), f32_up(sq64.x1), f32_down(sq64.y0), f32_up(sq64.y1)};
  float U = INFINITY, cmax2 = 0.0f;
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
      if (r * kSuperMax + tid * kPerThread + u < K) {
        const float cx = v[r][u].x, cy = v[r][u].y;
        U = fminf(U, sq.dmax2(cx, cy));
        cmax2 = fmaxf(cmax2, cx * cx + cy * cy);
      }
  U = (float)wave_min((double)U);
  cmax2 = (float)wave_max((double)cmax2);
  if (lane == 0) { sh.red[wave] = U; sh.red2[wave] = cmax2; }
  __syncthreads();
  U = (float)sh.red[0];
  cmax2 = (float)sh.red2[0];
#pragma unroll
  for (int w = 1; w < kPlanWaves; ++w) { U = fminf(U, (float)sh.red[w]); cmax2 = fmaxf(cmax2, (float)sh.red2[w]); }
  const double reach = sqrt((double)cmax2 * 1.000001) + R * 1.4142135623730951;
  const double delta = 1e-5 * reach * reach;
  const float slim = (U * 1.000001f + f32_up(2.0 * delta)) * 1.000001f;

  // ---- supercell survivors in ascending order: per round, each thread's
  // passing centroids, placed by a block-wide exclusive scan of the counts
  int nsurv = 0;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (r * kSuperMax >= K) break;                 // uniform
    const int c0 = r * kSuperMax + tid * kPerThread;
    uint32_t mask = 0;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
      if (c0 + u < K && sq.dmin2(v[r][u].x, v[r][u].y) <= slim) mask |= 1u << u;
    const int mine = __popc(mask);
    int incl = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    __syncthreads();                        // the previous round's wsum reads are done
    if (lane == kWave - 1) sh.wsum[wave] = incl;
    __syncthreads();
    int before = nsurv + incl - mine, total = nsurv;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      before += (w < wave) ? sh.wsum[w] : 0;
      total += sh.wsum[w];
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
      if ((mask >> u) & 1u) {
        if (before < kSuperMax) { sh.surv[before] = (uint16_t)(c0 + u); sh.survc[before] = v[r][u]; }
        ++before;
      }
    nsurv = total;
  }
  __syncthreads();
  const bool all = nsurv > kSuperMax;       // too many survivors: test every centroid (from global memory)
  // pad the survivor list to whole unrolled rounds with a far-away dummy that
  // neither lowers any U nor passes any test
  constexpr int kRound = 4 * LPC;
  static_assert(kSuperMax % kRound == 0, "padding stays inside the survivor arrays");
  const int ns = all ? K : (nsurv + kRound - 1) / kRound * kRound;
  if (!all)
    for (int j = nsurv + tid; j < ns; j += kPlanThreads) {
      sh.survc[j] = make_float2(1e30f, 1e30f);
      sh.surv[j] = 0;
    }
  __syncthreads();

  // ---- LPC lanes per cell: survivors j = sub, sub + LPC, ...  The cell
  // tests run in fp32 with margins that can only lengthen a list (a list with
  // extra centroids still yields the exhaustive search's index, since it
  // keeps every centroid tied with the winner): U(Q) from the widened box,
  // raised by 1e-6, and the limit (U(Q) + delta) raised by 1e-6 again.
  const int qc = tid / LPC, sub = tid % LPC;
  const int ix = sx * S + qc / S, iy = sy * S + qc % S;
  const Box cq64 = cell_box(R, G, ix, iy, 1);
  const BoxF cq{f32_down(cq64.x0), f32_up(cq64.x1), f32_down(cq64.y0), f32_up(cq64.y1)};
  float Uc = INFINITY;
  if (all) {
    for (int j = sub; j < ns; j += LPC) Uc = fminf(Uc, cq.dmax2(cb[2 * j], cb[2 * j + 1]));
  } else {
    for (int j0 = 0; j0 < ns; j0 += kRound) {
      float2 v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v4[u] = sh.survc[j0 + u * LPC + sub];
#pragma unroll
      for (int u = 0; u < 4; ++u) Uc = fminf(Uc, cq.dmax2(v4[u].x, v4[u].y));
    }
  }
#pragma unroll
  for (int off = LPC / 2; off > 0; off >>= 1) Uc = fminf(Uc, __shfl_xor(Uc, off));   // within the group
  const float lim = (Uc * 1.000001f + f32_up(delta)) * 1.000001f;
  uint16_t* mine = sh.cell_list[qc];
  const int gshift = lane & ~(LPC - 1);
  const uint64_t gmask = (LPC == 64) ? ~0ull : ((1ull << LPC) - 1ull);
  int count = 0;
  // survivors in index order: chunk t = [t LPC, (t+1) LPC), one per lane of the group
  auto take = [&](bool pred, int c) {
    const uint64_t gm = (__ballot(pred) >> gshift) & gmask;
    const int pos = count + __popcll(gm & ((1ull << sub) - 1ull));
    if (pred && pos < lmax) mine[pos] = (uint16_t)(c * 16);
    count += __popcll(gm);
  };
  if (all) {
    for (int j0 = 0; j0 < ns; j0 += LPC) {  // same trip count in every lane (ballot)
      const int j = j0 + sub;
      take(j < ns && cq.dmin2(cb[2 * min(j, ns - 1)], cb[2 * min(j, ns - 1) + 1]) <= lim, j);
    }
  } else {
    for (int j0 = 0; j0 < ns; j0 += kRound) {
      float2 v4[4];
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4[u] = sh.survc[j0 + u * LPC + sub];
        c[u] = sh.surv[j0 + u * LPC + sub];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) take(cq.dmin2(v4[u].x, v4[u].y) <= lim, c[u]);
    }
  }
  __syncthreads();
  if (sub != 0) return;
  // ---- the record: tail repeats the last entry (rescoring it never wins a strict "<")
  const bool overflow = count > lmax || count == 0;   // (a cell always lists at least one centroid)
  uint32_t words[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t lo = 0, hi = 0;
    if (2 * q < lmax && !overflow) {
      lo = mine[min(2 * q, count - 1)];
      hi = mine[min(2 * q + 1, count - 1)];
    }
    words[q] = lo | (hi << 16);
  }
  words[0] |= overflow ? (1u << 16) : (uint32_t)(count - 1);
  uint4* out = reinterpret_cast<uint4*>(lists + ((size_t)ix * G + iy) * lmax);
  out[0] = make_uint4(words[0], words[1], words[2], words[3]);
  if (lmax == 16) out[1] = make_uint4(words[4], words[5], words[6], words[7]);
}

// One launch builds both grids: workgroups [0, nfine) are the fine grid's
// 16 x 16-cell supercells (one lane per cell), the rest the outer grid's
// 4 x 4-cell supercells (16 lanes per cell; its cells are larger, so a 16 x 16
// supercell would keep most of the codebook).  Every workgroup computes the
// largest centroid radius itself (with U of its supercell); workgroup 0 writes
// the header.
constexpr int kSuperFine = 16;
constexpr int kSuperOuter = 4;
constexpr int kFineSupercells = (kPlanG / kSuperFine) * (kPlanG / kSuperFine);
constexpr int kOuterSupercells = (kPlanG2 / kSuperOuter) * (kPlanG2 / kSuperOuter);
static_assert(kPlanG % kSuperFine == 0 && kPlanG2 % kSuperOuter == 0, "grids are whole supercells");

// Outer-grid cells [kOuterFineLo, kOuterFineHi) per axis cover exactly the fine
// grid's square [-R, R): a point there always takes the fine grid, so those
// cells are never consulted.  Their supercells write overflow records (scan
// the whole codebook, correct if ever read) instead of lists; near the centre
// they are also the most expensive ones (thousands of survivors).
constexpr int kOuterFineLo = (int)((kPlanR2 - kPlanR) * kPlanG2 / (2.0f * kPlanR2));
constexpr int kOuterFineHi = kPlanG2 - kOuterFineLo;
static_assert(kOuterFineLo * 2.0f * kPlanR2 == (kPlanR2 - kPlanR) * kPlanG2, "the fine square is whole outer cells");
static_assert(kOuterFineLo % kSuperOuter == 0, "and whole outer supercells");

__device__ __forceinline__ bool outer_supercell_unused(int sidx) {
  constexpr int nsuper = kPlanG2 / kSuperOuter;
  const int x0 = (sidx / nsuper) * kSuperOuter, y0 = (sidx % nsuper) * kSuperOuter;
  return x0 >= kOuterFineLo && x0 + kSuperOuter <= kOuterFineHi && y0 >= kOuterFineLo &&
         y0 + kSuperOuter <= kOuterFineHi;
}

__global__ __launch_bounds__(kPlanThreads) void build_plan_kernel(const float* __restrict__ cb, int K, int lmax,
                                                                  char* __restrict__ plan, size_t outer_offset) {
  __shared__ PlanShared sh;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    PlanHeader* hdr = reinterpret_cast<PlanHeader*>(plan);
    hdr->R = kPlanR;
    hdr->cells_per_unit = (float)kPlanG / (2.0f * kPlanR);
    hdr->G = kPlanG;
    hdr->lmax = lmax;
    hdr->K = K;
    hdr->R2 = kPlanR2;
    hdr->cells_per_unit2 = (float)kPlanG2 / (2.0f * kPlanR2);
    hdr->G2 = kPlanG2;
  }
  if (blockIdx.x < kFineSupercells)
    build_supercell<kSuperFine>(sh, cb, K, lmax, kPlanR, kPlanG, blockIdx.x,
                                reinterpret_cast<uint16_t*>(plan + kPlanHeaderBytes));
  else if (!outer_supercell_unused(blockIdx.x - kFineSupercells))
    build_supercell<kSuperOuter>(sh, cb, K, lmax, kPlanR2, kPlanG2, blockIdx.x - kFineSupercells,
                                 reinterpret_cast<uint16_t*>(plan + outer_offset));
  else if (threadIdx.x < kSuperOuter * kSuperOuter) {   // one overflow record per cell
    constexpr int nsuper = kPlanG2 / kSuperOuter;
    const int sidx = blockIdx.x - kFineSupercells;
    const int ix = (sidx / nsuper) * kSuperOuter + threadIdx.x / kSuperOuter;
    const int iy = (sidx % nsuper) * kSuperOuter + threadIdx.x % kSuperOuter;
    uint4* out = reinterpret_cast<uint4*>(plan + outer_offset + ((size_t)ix * kPlanG2 + iy) * lmax * sizeof(uint16_t));
    out[0] = make_uint4(1u << 16, 0u, 0u, 0u);
    if (lmax == 16) out[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}

int launch_build_plan(const float* cb, int K, void* plan, hipStream_t st) {
  hipLaunchKernelGGL(build_plan_kernel, dim3(kFineSupercells + kOuterSupercells), dim3(kPlanThreads), 0, st, cb, K,
                     plan_lmax(K), (char*)plan, plan_outer_offset(K));
  return check_launch("build_plan_kernel");
}

}  // namespace qamw
