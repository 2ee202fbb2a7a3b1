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
// there.  Each has its own delta (R = 5 or 40 in the formula above).
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

  // ---- U(SQ) and the largest centroid radius Cmax in one pass over the codebook
  const Box sq = cell_box(R, G, sx * S, sy * S, S);
  double U = INFINITY, cmax = 0.0;
  for (int c = tid; c < K; c += kPlanThreads) {
    const double cx = cb[2 * c], cy = cb[2 * c + 1];
    U = fmin(U, sq.dmax2(cx, cy));
    cmax = fmax(cmax, sqrt(cx * cx + cy * cy));
  }
  U = wave_min(U);
  cmax = wave_max(cmax);
  if (lane == 0) { sh.red[wave] = U; sh.red2[wave] = cmax; }
  __syncthreads();
  U = sh.red[0];
  cmax = sh.red2[0];
#pragma unroll
  for (int w = 1; w < kPlanWaves; ++w) { U = fmin(U, sh.red[w]); cmax = fmax(cmax, sh.red2[w]); }
  const double reach = cmax + R * 1.4142135623730951;
  const double delta = 1e-5 * reach * reach;
  const double slim = U + 2.0 * delta;

  // ---- supercell survivors: thread t tests centroids [t P, t P + P), P = kPerThread
  // (K <= 4096 = 2 kSuperMax, so two rounds at most), then one block-wide scan
  int nsurv = 0;
  for (int r0 = 0; r0 < K; r0 += kSuperMax) {
    const int c0 = r0 + tid * kPerThread;
    float2 v[kPerThread];
    uint32_t mask = 0;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int c = c0 + u;
      v[u] = c < K ? make_float2(cb[2 * c], cb[2 * c + 1]) : make_float2(0.0f, 0.0f);
      if (c < K && sq.dmin2(v[u].x, v[u].y) <= slim) mask |= 1u << u;
    }
    // exclusive prefix of the per-thread counts: wave scan, then across waves
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
        if (before < kSuperMax) { sh.surv[before] = (uint16_t)(c0 + u); sh.survc[before] = v[u]; }
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

  // ---- LPC lanes per cell: survivors j = sub, sub + LPC, ...
  const int qc = tid / LPC, sub = tid % LPC;
  const int ix = sx * S + qc / S, iy = sy * S + qc % S;
  const Box cq = cell_box(R, G, ix, iy, 1);
  double Uc = INFINITY;
  if (all) {
    for (int j = sub; j < ns; j += LPC) Uc = fmin(Uc, cq.dmax2(cb[2 * j], cb[2 * j + 1]));
  } else {
    for (int j0 = 0; j0 < ns; j0 += kRound) {
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = sh.survc[j0 + u * LPC + sub];
#pragma unroll
      for (int u = 0; u < 4; ++u) Uc = fmin(Uc, cq.dmax2(v[u].x, v[u].y));
    }
  }
#pragma unroll
  for (int off = LPC / 2; off > 0; off >>= 1) Uc = fmin(Uc, __shfl_xor(Uc, off));   // within the group
  const double lim = Uc + delta;
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
      float2 v[4];
      int c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = sh.survc[j0 + u * LPC + sub];
        c[u] = sh.surv[j0 + u * LPC + sub];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) take(cq.dmin2(v[u].x, v[u].y) <= lim, c[u]);
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
  else
    build_supercell<kSuperOuter>(sh, cb, K, lmax, kPlanR2, kPlanG2, blockIdx.x - kFineSupercells,
                                 reinterpret_cast<uint16_t*>(plan + outer_offset));
}

int launch_build_plan(const float* cb, int K, void* plan, hipStream_t st) {
  hipLaunchKernelGGL(build_plan_kernel, dim3(kFineSupercells + kOuterSupercells), dim3(kPlanThreads), 0, st, cb, K,
                     plan_lmax(K), (char*)plan, plan_outer_offset(K));
  return check_launch("build_plan_kernel");
}

}  // namespace qamw
