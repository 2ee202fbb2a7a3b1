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
  float cells_per_unit;   // G / (2 R) (uniform inner grid, K > kLdsMaxK)
  int G;
  int lmax;
  int K;
  float R2;               // outer grid
  float cells_per_unit2;
  int G2;
  int lds_G;              // LDS table (K <= kLdsMaxK; 0 otherwise): cells per axis
  int lds_bins;           // bins of the axis map over [-R, R)
  int lds_lists_cap;      // list records the image holds
  int lds_nlists;         // list records used (a cell over the capacity scans all)
  int lds_image_bytes;
  int lds_cells_off;      // byte offsets inside the image
  int lds_lists_off;
  int lds_image_off;      // byte offset of the image inside the plan
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

// The survivors of a supercell box SQ: every centroid with
// min_{z in SQ} |z - c|^2 <= U(SQ) + 2 delta, ascending, with coordinates, in
// sh.surv / sh.survc, padded with far-away dummies to whole rounds of `round`
// entries.  Returns their count (more than kSuperMax: `all` is set and the
// callers test every centroid from global memory); *cmax2 is the largest
// squared centroid radius and *delta the grid's score margin
// 1e-5 (Cmax + R sqrt 2)^2 (R: the grid's half-width).
__device__ int supercell_survivors(PlanShared& sh, const float* __restrict__ cb, int K, const Box& sq64, double R,
                                   int round, float* cmax2_out, double* delta_out, bool* all_out, int* ns_out) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
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
  // it does ten times over; a cell's own margin is never larger.
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
  // pad the survivor list to whole rounds with a far-away dummy that neither
  // lowers any U nor passes any test
  const int ns = all ? K : (nsurv + round - 1) / round * round;
  if (!all)
    for (int j = nsurv + tid; j < ns; j += kPlanThreads) {
      sh.survc[j] = make_float2(1e30f, 1e30f);
      sh.surv[j] = 0;
    }
  __syncthreads();
  *cmax2_out = cmax2;
  *delta_out = delta;
  *all_out = all;
  *ns_out = ns;
  return nsurv;
}

// One workgroup per supercell (S x S cells) of a G x G grid over [-R, R)^2:
// the supercell's survivors (ascending, with coordinates) into LDS, then a
// group of LPC = 256 / S^2 lanes per cell scans them and writes the records.
template <int S>
__device__ void build_supercell(PlanShared& sh, const float* __restrict__ cb, int K, int lmax, double R, int G,
                                int sidx, uint16_t* __restrict__ lists) {
  constexpr int LPC = kPlanThreads / (S * S);
  static_assert(LPC >= 1 && LPC * S * S == kPlanThreads && kWave % LPC == 0, "cell groups tile the wavefronts");
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int nsuper = G / S;
  const int sx = sidx / nsuper, sy = sidx % nsuper;
  constexpr int kRound = 4 * LPC;
  static_assert(kSuperMax % kRound == 0, "padding stays inside the survivor arrays");
  float cmax2;
  double delta;
  bool all;
  int ns;
  supercell_survivors(sh, cb, K, cell_box(R, G, sx * S, sy * S, S), R, kRound, &cmax2, &delta, &all, &ns);
  (void)cmax2;

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

// ===========================================================================
// LDS table (K <= kLdsMaxK): cell candidate sets decided exactly.
//
// A cell Q (its bins' box enlarged by eta) lists centroid c when some z in Q
// has |z - c|^2 <= |z - c'|^2 + delta_Q for every centroid c': the fp32
// winner c32 at z (and every centroid tied with it) qualifies, since
// |z - c32|^2 <= |z - c*|^2 + slack(z) <= |z - c'|^2 + slack(z) for all c'.
// slack(z) = 2 (e(c32) + e(c*)) <= 4 2^-24 (2.5 cm^2 + 2 zmax cm) with zmax
// the largest |z| over Q and cm >= |c32|, |c*|: both lie within
// sqrt(U(Q) + delta) of z (delta the grid's margin, >= slack everywhere), so
// cm = min(Cmax, zmax + sqrt(U(Q) + delta)); delta_Q is ten times that bound.
// The test for one c is the feasibility of a small 2D linear system (the box
// and one half-plane 2 z.(c' - c) <= |c'|^2 - |c|^2 + delta_Q per c'): if the
// feasible polygon is not empty, one of its vertices is the intersection of
// two of the lines, so every such intersection point is tried (in fp64, with
// a tolerance that errs towards listing).  Only the cell's loose candidates
// (min_{z in Q} |z - c|^2 <= U(Q) + delta_Q) need testing or acting as c': any
// other centroid is farther than the one attaining U(Q) everywhere in Q.
// ===========================================================================
constexpr int kLdsSuper = 8;           // LDS-table supercells: 8 x 8 cells, four lanes per cell
constexpr int kLdsLoose = 16;          // loose candidates a cell may keep (more: scan all)
constexpr int kLdsListMax = 8;         // exact candidates a cell may list (more: scan all)
constexpr int kHashSlots = 32768;      // list dedup table (>= 1.4 x the cells of any geometry)
static_assert(kHashSlots >= 2 * kLdsMaxG * kLdsMaxG / 4, "dedup table load factor");

struct LdsEdges {
  uint16_t e[kLdsMaxG + 1];
};

// dedup table entry: the list (4 x u16), the lowest cell holding it, its record id
struct HashSlot {
  unsigned long long key;
  unsigned int owner;
  unsigned int id;
};

struct LdsScratch {
  uint4* cellset;         // [G*G] exact candidate sets: 8 x u16 16c, low nibble of entry 0 = count - 1,
                          // of entry 1 = 1 when the cell must scan all
  int* slot;              // [G*G] dedup slot of a 2..4 list, -1 otherwise
  int* recid;             // [G*G] record id of a 5..8 list (two records), or of an owned 2..4 list
  int* total;             // records used
  int* blocksum;          // [kMaxScanBlocks] records needed per block of kScanBlock cells
  HashSlot* table;        // [kHashSlots]
};

constexpr int kScanBlock = 256;                  // cells per block of the record-id scan
constexpr int kMaxScanBlocks = kLdsMaxG * kLdsMaxG / kScanBlock;

__host__ __device__ inline size_t lds_scratch_bytes(int G) {
  const size_t cells = (size_t)G * G;
  return round_up(cells * 16, 256) + 2 * round_up(cells * 4, 256) + 256 + kMaxScanBlocks * sizeof(int) +
         (size_t)kHashSlots * sizeof(HashSlot);
}

__device__ __forceinline__ LdsScratch lds_scratch(char* base, int G) {
  const size_t cells = (size_t)G * G;
  LdsScratch s;
  s.cellset = reinterpret_cast<uint4*>(base);
  base += round_up(cells * 16, 256);
  s.slot = reinterpret_cast<int*>(base);
  base += round_up(cells * 4, 256);
  s.recid = reinterpret_cast<int*>(base);
  base += round_up(cells * 4, 256);
  s.total = reinterpret_cast<int*>(base);
  base += 256;
  s.blocksum = reinterpret_cast<int*>(base);
  base += kMaxScanBlocks * sizeof(int);
  s.table = reinterpret_cast<HashSlot*>(base);
  return s;
}

__device__ __forceinline__ Box lds_box(const LdsEdges& E, int x0, int x1, int y0, int y1) {
  // cells [x0, x1) x [y0, y1) of the LDS table: bins of width 2 R / kLdsBins
  const double h = 2.0 * kPlanR / kLdsBins;
  return Box{-kPlanR + E.e[x0] * h - kPlanEta, -kPlanR + E.e[x1] * h + kPlanEta,
             -kPlanR + E.e[y0] * h - kPlanEta, -kPlanR + E.e[y1] * h + kPlanEta};
}

// Candidate pruning inside one cell Q, for the loose candidates m[0..n) of
// the cell (survivor slots).  f(z) = |z - c_i|^2 - |z - c_k|^2 is linear in z,
// so its minimum over the box is at a corner: when it exceeds delta at all
// four corners, c_k beats c_i by more than delta everywhere in Q and c_i is
// never within delta of the minimum there ("k dominates i").  Such a c_i is
// dropped, and its constraint on the others can be dropped too: whatever
// satisfies |z - c_j|^2 <= |z - c_k|^2 + delta then satisfies it against c_i.
__device__ __forceinline__ double corner_min_diff(const Box& q, double ix, double iy, double kx, double ky) {
  // |z - c_i|^2 - |z - c_k|^2 = 2 z.(c_k - c_i) + |c_i|^2 - |c_k|^2, minimised over the corners
  const double ax = 2.0 * (kx - ix), ay = 2.0 * (ky - iy), c0 = (ix * ix + iy * iy) - (kx * kx + ky * ky);
  return fmin(ax * q.x0, ax * q.x1) + fmin(ay * q.y0, ay * q.y1) + c0;
}

// Is there a point z of q with |z - c_i|^2 <= |z - c_k|^2 + delta for every k
// in the set `keep` (a bitmask over m[0..n))?  If that polygon is not empty
// one of its vertices is the intersection of two of the lines (box edges and
// the constraints' boundaries), so every such point is tried, in fp64, with a
// tolerance that errs towards "feasible".
__device__ bool lds_feasible(const PlanShared& sh, const uint16_t* m, int n, uint32_t keep, int i, const Box& q,
                             double delta) {
  const float2 fi = sh.survc[m[i]];
  const double cix = fi.x, ciy = fi.y, ci2 = cix * cix + ciy * ciy;
  auto cons = [&](int k, double& ax, double& ay, double& b) {
    const float2 fk = sh.survc[m[k]];
    const double kx = fk.x, ky = fk.y;
    ax = 2.0 * (kx - cix);
    ay = 2.0 * (ky - ciy);
    b = (kx * kx + ky * ky) - ci2 + delta;
  };
  auto ok = [&](double px, double py) -> bool {
    const double tb = 1e-12 * (1.0 + fabs(px) + fabs(py));
    if (!(px >= q.x0 - tb && px <= q.x1 + tb && py >= q.y0 - tb && py <= q.y1 + tb)) return false;
    for (int k = 0; k < n; ++k) {
      if (k == i || !((keep >> k) & 1u)) continue;
      double ax, ay, b;
      cons(k, ax, ay, b);
      if (ax * px + ay * py > b + 1e-12 * (fabs(ax * px) + fabs(ay * py) + fabs(b)) + 1e-15) return false;
    }
    return true;
  };
  if (ok(q.x0, q.y0) || ok(q.x0, q.y1) || ok(q.x1, q.y0) || ok(q.x1, q.y1)) return true;
  for (int k = 0; k < n; ++k) {
    if (k == i || !((keep >> k) & 1u)) continue;
    double ax, ay, b;
    cons(k, ax, ay, b);
    if (ay != 0.0 && (ok(q.x0, (b - ax * q.x0) / ay) || ok(q.x1, (b - ax * q.x1) / ay))) return true;
    if (ax != 0.0 && (ok((b - ay * q.y0) / ax, q.y0) || ok((b - ay * q.y1) / ax, q.y1))) return true;
  }
  for (int k = 0; k < n; ++k) {
    if (k == i || !((keep >> k) & 1u)) continue;
    double axk, ayk, bk;
    cons(k, axk, ayk, bk);
    for (int j = k + 1; j < n; ++j) {
      if (j == i || !((keep >> j) & 1u)) continue;
      double axj, ayj, bj;
      cons(j, axj, ayj, bj);
      const double det = axk * ayj - ayk * axj;
      if (det == 0.0) continue;
      if (ok((bk * ayj - bj * ayk) / det, (axk * bj - axj * bk) / det)) return true;
    }
  }
  return false;
}

// One workgroup per 8 x 8-cell supercell of the LDS table: survivors, then
// four lanes per cell: U(Q), delta_Q, the loose candidates (ascending), the
// dominance pruning and the exact test of what is left, split over the lanes.
constexpr int kLdsLanes = 4;
__device__ void build_lds_supercell(PlanShared& sh, const float* __restrict__ cb, int K, const LdsEdges& E, int G,
                                    int sidx, LdsScratch scr) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int nsuper = (G + kLdsSuper - 1) / kLdsSuper;
  const int sx = sidx / nsuper, sy = sidx % nsuper;
  const int x0 = sx * kLdsSuper, y0 = sy * kLdsSuper;
  const int x1 = min(x0 + kLdsSuper, G), y1 = min(y0 + kLdsSuper, G);
  constexpr int kRound = 4 * kLdsLanes;
  float cmax2;
  double delta;
  bool all;
  int ns;
  supercell_survivors(sh, cb, K, lds_box(E, x0, x1, y0, y1), kPlanR, kRound, &cmax2, &delta, &all, &ns);
  // K <= kSuperMax here, so the survivors always fit (all == false)
  const int qc = tid / kLdsLanes, sub = tid % kLdsLanes;
  const int ix = x0 + qc / kLdsSuper, iy = y0 + qc % kLdsSuper;
  const bool real = ix < x1 && iy < y1;          // lanes of cells past the table's edge compute a copy of the last
  const int cx_ = min(ix, G - 1), cy_ = min(iy, G - 1);
  const Box cq64 = lds_box(E, cx_, cx_ + 1, cy_, cy_ + 1);
  const BoxF cq{f32_down(cq64.x0), f32_up(cq64.x1), f32_down(cq64.y0), f32_up(cq64.y1)};
  float Uc = INFINITY;
  for (int j0 = 0; j0 < ns; j0 += kRound) {
    float2 v4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v4[u] = sh.survc[j0 + u * kLdsLanes + sub];
#pragma unroll
    for (int u = 0; u < 4; ++u) Uc = fminf(Uc, cq.dmax2(v4[u].x, v4[u].y));
  }
#pragma unroll
  for (int off = kLdsLanes / 2; off > 0; off >>= 1) Uc = fminf(Uc, __shfl_xor(Uc, off));
  // the cell's margin: ten times the fp32 slack bound for its points
  const double zx = fmax(fabs(cq64.x0), fabs(cq64.x1)), zy = fmax(fabs(cq64.y0), fabs(cq64.y1));
  const double zmax = sqrt(zx * zx + zy * zy);
  const double cm = fmin(sqrt((double)cmax2 * 1.000001), zmax + sqrt((double)Uc * 1.000001 + delta));
  const double dq = 40.0 * 0x1p-24 * (2.5 * cm * cm + 2.0 * zmax * cm);
  const float lim = (Uc * 1.000001f + f32_up(dq)) * 1.000001f;
  // ---- loose candidates in ascending order: survivors j = sub, sub + 4, ...,
  // one chunk of four per ballot
  uint16_t* mine = sh.cell_list[qc];
  const int gshift = lane & ~(kLdsLanes - 1);
  int nl = 0;
  for (int j0 = 0; j0 < ns; j0 += kLdsLanes) {
    const float2 v = sh.survc[j0 + sub];
    const bool pred = cq.dmin2(v.x, v.y) <= lim;
    const uint64_t gm = (__ballot(pred) >> gshift) & ((1ull << kLdsLanes) - 1ull);
    const int pos = nl + __popcll(gm & ((1ull << sub) - 1ull));
    if (pred && pos < kLdsLoose) mine[pos] = (uint16_t)(j0 + sub);
    nl += __popcll(gm);
  }
  __syncthreads();
  // ---- dominance, then the exact test of the undominated candidates
  // (lane sub decides candidates sub, sub + 4, ...; the four masks are or-ed)
  const bool over_loose = nl > kLdsLoose || nl == 0;
  const int n = over_loose ? 0 : nl;
  uint32_t undom = 0;
  for (int i = sub; i < n; i += kLdsLanes) {
    const float2 fi = sh.survc[mine[i]];
    bool dominated = false;
    for (int k = 0; k < n && !dominated; ++k) {
      if (k == i) continue;
      const float2 fk = sh.survc[mine[k]];
      dominated = corner_min_diff(cq64, fi.x, fi.y, fk.x, fk.y) > dq * (1.0 + 1e-9) + 1e-15;
    }
    if (!dominated) undom |= 1u << i;
  }
#pragma unroll
  for (int off = kLdsLanes / 2; off > 0; off >>= 1) undom |= (uint32_t)__shfl_xor((int)undom, off);
  uint32_t keep = 0;
  for (int i = sub; i < n; i += kLdsLanes)
    if (((undom >> i) & 1u) && (__popc(undom) == 1 || lds_feasible(sh, mine, n, undom, i, cq64, dq))) keep |= 1u << i;
#pragma unroll
  for (int off = kLdsLanes / 2; off > 0; off >>= 1) keep |= (uint32_t)__shfl_xor((int)keep, off);
  if (sub != 0 || !real) return;
  // ---- the cell's exact set, ascending (mine[] ascends)
  const int count = __popc(keep);
  const bool over = over_loose || count > kLdsListMax || count == 0;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (!over) {
    uint32_t ent[kLdsListMax];
    int c = 0;
    uint32_t last = 0;
#pragma unroll
    for (int q = 0; q < kLdsListMax; ++q) ent[q] = 0;
    for (int i = 0; i < n; ++i)
      if ((keep >> i) & 1u) {
        last = 16u * sh.surv[mine[i]];
#pragma unroll
        for (int q = 0; q < kLdsListMax; ++q) ent[q] = (q == c) ? last : ent[q];
        ++c;
      }
#pragma unroll
    for (int q = 0; q < kLdsListMax; ++q) ent[q] = (q >= count) ? last : ent[q];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = ent[2 * q] | (ent[2 * q + 1] << 16);
  }
  w[0] |= over ? (1u << 16) : (uint32_t)(count - 1);
  scr.cellset[(size_t)ix * G + iy] = make_uint4(w[0], w[1], w[2], w[3]);
}

// Two launches build the grids: build_plan_kernel the inner grid's supercells
// (the LDS table's 8 x 8 cells with four lanes per cell for K <= kLdsMaxK,
// else the uniform 512 x 512 grid's 16 x 16 cells with one lane per cell),
// build_outer_kernel the outer grid's 4 x 4-cell supercells (16 lanes per
// cell; its cells are larger, so a 16 x 16 supercell would keep most of the
// codebook).  Every workgroup computes the largest centroid radius itself
// (with U of its supercell); workgroup 0 of the first writes the header, and
// with the LDS table every workgroup of the first clears a stripe of the
// dedup table.
constexpr int kSuperFine = 16;
constexpr int kSuperOuter = 4;
constexpr int kFineSupercells = (kPlanG / kSuperFine) * (kPlanG / kSuperFine);
constexpr int kOuterSupercells = (kPlanG2 / kSuperOuter) * (kPlanG2 / kSuperOuter);
static_assert(kPlanG % kSuperFine == 0 && kPlanG2 % kSuperOuter == 0, "grids are whole supercells");

// Outer-grid cells [kOuterFineLo, kOuterFineHi) per axis cover exactly the
// inner grid's square [-R, R): a point there always takes the inner grid, so
// those cells are never consulted.  Their supercells write overflow records
// (scan the whole codebook, correct if ever read) instead of lists; near the
// centre they are also the most expensive ones (thousands of survivors).
constexpr int kOuterFineLo = (int)((kPlanR2 - kPlanR) * kPlanG2 / (2.0f * kPlanR2));
constexpr int kOuterFineHi = kPlanG2 - kOuterFineLo;
static_assert(kOuterFineLo * 2.0f * kPlanR2 == (kPlanR2 - kPlanR) * kPlanG2, "the inner square is whole outer cells");
static_assert(kOuterFineLo % kSuperOuter == 0, "and whole outer supercells");

__device__ __forceinline__ bool outer_supercell_unused(int sidx) {
  constexpr int nsuper = kPlanG2 / kSuperOuter;
  const int x0 = (sidx / nsuper) * kSuperOuter, y0 = (sidx % nsuper) * kSuperOuter;
  return x0 >= kOuterFineLo && x0 + kSuperOuter <= kOuterFineHi && y0 >= kOuterFineLo &&
         y0 + kSuperOuter <= kOuterFineHi;
}

__global__ __launch_bounds__(kPlanThreads) void build_plan_kernel(const float* __restrict__ cb, int K, int lmax,
                                                                  char* __restrict__ plan, int lds_G, LdsEdges edges,
                                                                  size_t scratch_offset) {
  __shared__ PlanShared sh;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    PlanHeader* hdr = reinterpret_cast<PlanHeader*>(plan);
    hdr->R = kPlanR;
    hdr->cells_per_unit = lds_G ? 0.0f : (float)kPlanG / (2.0f * kPlanR);
    hdr->G = lds_G ? 0 : kPlanG;
    hdr->lmax = lmax;
    hdr->K = K;
    hdr->R2 = kPlanR2;
    hdr->cells_per_unit2 = (float)kPlanG2 / (2.0f * kPlanR2);
    hdr->G2 = kPlanG2;
    // the LDS table's fields: lds_image_kernel fills them when there is one
    hdr->lds_G = hdr->lds_bins = hdr->lds_lists_cap = hdr->lds_nlists = 0;
    hdr->lds_image_bytes = hdr->lds_cells_off = hdr->lds_lists_off = hdr->lds_image_off = 0;
  }
  if (lds_G) {
    LdsScratch scr = lds_scratch(plan + scratch_offset, lds_G);
    for (int i = blockIdx.x * kPlanThreads + threadIdx.x; i < kHashSlots; i += gridDim.x * kPlanThreads)
      scr.table[i] = HashSlot{0ull, 0xffffffffu, 0u};
    build_lds_supercell(sh, cb, K, edges, lds_G, blockIdx.x, scr);
  } else {
    build_supercell<kSuperFine>(sh, cb, K, lmax, kPlanR, kPlanG, blockIdx.x,
                                reinterpret_cast<uint16_t*>(plan + kPlanHeaderBytes));
  }
}

// The outer grid, one workgroup per 4 x 4-cell supercell.
__global__ __launch_bounds__(kPlanThreads) void build_outer_kernel(const float* __restrict__ cb, int K, int lmax,
                                                                   char* __restrict__ plan, size_t outer_offset) {
  __shared__ PlanShared sh;
  const int sidx = blockIdx.x;
  if (!outer_supercell_unused(sidx))
    build_supercell<kSuperOuter>(sh, cb, K, lmax, kPlanR2, kPlanG2, sidx,
                                 reinterpret_cast<uint16_t*>(plan + outer_offset));
  else if (threadIdx.x < kSuperOuter * kSuperOuter) {   // one overflow record per cell
    constexpr int nsuper = kPlanG2 / kSuperOuter;
    const int ix = (sidx / nsuper) * kSuperOuter + threadIdx.x / kSuperOuter;
    const int iy = (sidx % nsuper) * kSuperOuter + threadIdx.x % kSuperOuter;
    uint4* out = reinterpret_cast<uint4*>(plan + outer_offset + ((size_t)ix * kPlanG2 + iy) * lmax * sizeof(uint16_t));
    out[0] = make_uint4(1u << 16, 0u, 0u, 0u);
    if (lmax == 16) out[1] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// ---- list dedup.  A list of 2..4 candidates (4 x u16, tail repeated) is a
// 64-bit key; equal lists share one record.  The record belongs to the lowest
// cell holding the list, and records are numbered by a prefix sum over the
// cells in order, so the image does not depend on the order of the atomics.
__device__ __forceinline__ uint32_t cell_count(uint4 w) { return (w.x & 15u) + 1u; }
__device__ __forceinline__ bool cell_over(uint4 w) { return (w.x >> 16) & 1u; }
__device__ __forceinline__ unsigned long long list_key(uint4 w) {
  return (unsigned long long)(w.x & 0xfff0fff0u) | ((unsigned long long)w.y << 32);
}

__global__ __launch_bounds__(256) void lds_insert_kernel(char* __restrict__ plan, size_t scratch_offset, int G) {
  const int cell = blockIdx.x * 256 + threadIdx.x;
  if (cell >= G * G) return;
  LdsScratch scr = lds_scratch(plan + scratch_offset, G);
  const uint4 w = scr.cellset[cell];
  const uint32_t n = cell_count(w);
  int slot = -1;
  if (!cell_over(w) && n >= 2 && n <= 4) {
    const unsigned long long key = list_key(w);
    unsigned long long h = key * 0x9E3779B97F4A7C15ull;
    h ^= h >> 29;
    uint32_t at = (uint32_t)(h >> 17) & (kHashSlots - 1);
    for (int probe = 0; probe < kHashSlots; ++probe) {      // bounded: every slot at most once
      const unsigned long long prev = atomicCAS(&scr.table[at].key, 0ull, key);
      if (prev == 0ull || prev == key) {
        atomicMin(&scr.table[at].owner, (unsigned int)cell);
        slot = (int)at;
        break;
      }
      at = (at + 1) & (kHashSlots - 1);
    }
  }
  scr.slot[cell] = slot;
}

// Block-wide inclusive scan of one int per thread (kScanBlock threads).
__device__ __forceinline__ int block_scan(int v, int* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int off = 1; off < kScanBlock; off <<= 1) {
    const int t = threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
    __syncthreads();
    sh[threadIdx.x] += t;
    __syncthreads();
  }
  return sh[threadIdx.x];
}

// Records a cell needs: one for a 2..4 list it owns (it is the lowest cell
// holding that list), two for a 5..8 list, none otherwise; and each block's
// total.
__global__ __launch_bounds__(kScanBlock) void lds_need_kernel(char* __restrict__ plan, size_t scratch_offset, int G) {
  __shared__ int sh[kScanBlock];
  const int cell = blockIdx.x * kScanBlock + threadIdx.x;
  LdsScratch scr = lds_scratch(plan + scratch_offset, G);
  int need = 0;
  if (cell < G * G) {
    const uint4 w = scr.cellset[cell];
    if (!cell_over(w)) {
      const uint32_t n = cell_count(w);
      const int sl = scr.slot[cell];
      if (n >= 5) need = 2;
      else if (n >= 2 && sl >= 0 && scr.table[sl].owner == (unsigned int)cell) need = 1;
    }
    scr.recid[cell] = need;
  }
  const int incl = block_scan(need, sh);
  if (threadIdx.x == kScanBlock - 1) scr.blocksum[blockIdx.x] = incl;
}

// Record ids: an exclusive prefix sum of the needs over the cells in order
// (block offsets from the block totals, then a scan inside the block),
// published to the dedup table for the owned 2..4 lists.
__global__ __launch_bounds__(kScanBlock) void lds_ids_kernel(char* __restrict__ plan, size_t scratch_offset, int G) {
  __shared__ int sh[kScanBlock];
  LdsScratch scr = lds_scratch(plan + scratch_offset, G);
  const int nblk = (G * G + kScanBlock - 1) / kScanBlock;
  // this block's offset: the sum of the earlier blocks' totals
  const int before = (int)threadIdx.x < (int)blockIdx.x ? scr.blocksum[threadIdx.x] : 0;
  block_scan(before, sh);
  const int block_off = sh[kScanBlock - 1];              // the scan's last entry: the whole sum
  __syncthreads();
  const int cell = blockIdx.x * kScanBlock + threadIdx.x;
  const int need = cell < G * G ? scr.recid[cell] : 0;
  const int incl = block_scan(need, sh);
  if (cell < G * G) {
    const int id = block_off + incl - need;
    scr.recid[cell] = need ? id : -1;
    if (need == 1) scr.table[scr.slot[cell]].id = (unsigned int)id;
  }
  if ((int)blockIdx.x == nblk - 1 && threadIdx.x == kScanBlock - 1) *scr.total = block_off + incl;
}

// The image: bin -> cell map, one entry per cell, the list records; the
// header's table fields.  Records past the capacity are not written: their
// cells scan the whole codebook.
__global__ __launch_bounds__(256) void lds_image_kernel(char* __restrict__ plan, size_t scratch_offset,
                                                        size_t image_offset, int G, int cells_off, int lists_off,
                                                        int lists_cap, int image_bytes, LdsEdges E) {
  LdsScratch scr = lds_scratch(plan + scratch_offset, G);
  char* img = plan + image_offset;
  uint16_t* cells = reinterpret_cast<uint16_t*>(img + cells_off);
  uint2* lists = reinterpret_cast<uint2*>(img + lists_off);
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int used = min(*scr.total, lists_cap);
  if (t == 0) {
    PlanHeader* hdr = reinterpret_cast<PlanHeader*>(plan);
    hdr->lds_G = G;
    hdr->lds_bins = kLdsBins;
    hdr->lds_lists_cap = lists_cap;
    hdr->lds_nlists = used;
    hdr->lds_image_bytes = image_bytes;
    hdr->lds_cells_off = cells_off;
    hdr->lds_lists_off = lists_off;
    hdr->lds_image_off = (int)image_offset;
  }
  if (t < kLdsBins) {                                  // the bin -> cell map: the c with e[c] <= t < e[c + 1]
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (E.e[mid] <= t) lo = mid; else hi = mid;
    }
    reinterpret_cast<uint8_t*>(img)[t] = (uint8_t)lo;
  }
  // unused records and the cell padding are cleared, so the image is a pure
  // function of the codebook
  const int ncell = G * G;
  const int pad_end = (lists_off - cells_off) / 2;
  for (int i = ncell + t; i < pad_end; i += gridDim.x * 256) cells[i] = 0;
  for (int i = used + t; i < lists_cap; i += gridDim.x * 256) lists[i] = make_uint2(0u, 0u);
  if (t >= ncell) return;
  const uint4 w = scr.cellset[t];
  const uint32_t n = cell_count(w);
  uint16_t entry = kLdsScanAll;
  if (!cell_over(w)) {
    if (n == 1) {
      entry = (uint16_t)(w.x & 0xfff0u);
    } else if (n <= 4) {
      const int sl = scr.slot[t];
      if (sl >= 0) {
        const unsigned int id = scr.table[sl].id;
        if ((int)id < used) {
          entry = (uint16_t)(0x8000u | id);
          if (scr.table[sl].owner == (unsigned int)t) lists[id] = make_uint2(w.x & 0xfff0fff0u, w.y);
        }
      }
    } else {
      const int id = scr.recid[t];
      if (id >= 0 && id + 1 < used) {
        entry = (uint16_t)(0x8000u | (unsigned)id);
        lists[id] = make_uint2(w.x & 0xfff0fff0u, w.y | 0x80000000u);   // slot 3's top bit: continued
        lists[id + 1] = make_uint2(w.z, w.w);
      }
    }
  }
  cells[t] = entry;
}

// ===========================================================================
// host side
// ===========================================================================
bool lds_geometry(int K, LdsGeometry* g) {
  if (!plan_has_lds(K)) return false;
  // cell widths in bins grow as exp(t^2 / 8) away from the origin (centroid
  // spacing of a Lloyd-Max codebook for N(0, I_2) grows like p(z)^(-1/4)), from
  // 7 bins at the origin for K = 2048, scaled by sqrt(2048 / K)
  const double h = 2.0 * kPlanR / kLdsBins;
  const double w0 = 7.0 * sqrt(2048.0 / K);
  int pos[kLdsBins + 1];
  int np = 0;
  pos[np++] = kLdsBins / 2;
  while (pos[np - 1] < kLdsBins) {
    const double t = (pos[np - 1] - kLdsBins / 2) * h;
    const long w = lround(w0 * exp(t * t / 8.0));
    const int wi = (int)(w < 1 ? 1 : (w > 255 ? 255 : w));
    pos[np] = pos[np - 1] + wi > kLdsBins ? kLdsBins : pos[np - 1] + wi;
    ++np;
  }
  // mirror: edges kLdsBins - pos[np-1] .. kLdsBins - pos[1], then pos[0..np)
  if (2 * np - 1 > kLdsMaxG + 1) return false;
  int G = 0;
  for (int i = np - 1; i >= 1; --i) g->edges[G++] = (uint16_t)(kLdsBins - pos[i]);
  for (int i = 0; i < np; ++i) g->edges[G++] = (uint16_t)pos[i];
  G -= 1;
  g->G = G;
  const int B = qamw_index_bits(K);
  g->stage_bytes = (size_t)64 * B;
  g->cells_off = kLdsBins;
  g->lists_off = g->cells_off + round_up((size_t)2 * G * G, 16);
  const long avail = (long)kLdsBudget - 16L * K - (long)(kLdsWaves * g->stage_bytes) - (long)g->lists_off;
  long cap = avail / 8;
  cap = cap > 32767 ? 32767 : cap;
  cap &= ~1L;                                   // whole 16-byte rows
  if (cap < 2) return false;
  g->lists_cap = (int)cap;
  g->image_bytes = g->lists_off + (size_t)8 * cap;
  return true;
}

size_t plan_outer_offset(int K) {
  return plan_has_lds(K) ? kPlanHeaderBytes
                         : kPlanHeaderBytes + (size_t)kPlanG * kPlanG * plan_lmax(K) * sizeof(uint16_t);
}

size_t plan_image_offset(int K) {
  return plan_outer_offset(K) + (size_t)kPlanG2 * kPlanG2 * plan_lmax(K) * sizeof(uint16_t);
}

size_t plan_scratch_offset(int K) {
  LdsGeometry g;
  if (!lds_geometry(K, &g)) return plan_image_offset(K);
  return round_up(plan_image_offset(K) + g.image_bytes, 256);
}

size_t plan_bytes(int K) {
  LdsGeometry g;
  if (!lds_geometry(K, &g)) return plan_image_offset(K);
  return plan_scratch_offset(K) + lds_scratch_bytes(g.G);
}

int launch_build_plan(const float* cb, int K, void* plan, hipStream_t st) {
  LdsGeometry g;
  LdsEdges E{};
  int G = 0, ninner = kFineSupercells;
  if (lds_geometry(K, &g)) {
    G = g.G;
    for (int i = 0; i <= G; ++i) E.e[i] = g.edges[i];
    const int ns = (G + kLdsSuper - 1) / kLdsSuper;
    ninner = ns * ns;
  }
  char* p = (char*)plan;
  hipLaunchKernelGGL(build_plan_kernel, dim3(ninner), dim3(kPlanThreads), 0, st, cb, K, plan_lmax(K), p, G, E,
                     plan_scratch_offset(K));
  int rc = check_launch("build_plan_kernel");
  if (rc) return rc;
  hipLaunchKernelGGL(build_outer_kernel, dim3(kOuterSupercells), dim3(kPlanThreads), 0, st, cb, K, plan_lmax(K), p,
                     plan_outer_offset(K));
  if ((rc = check_launch("build_outer_kernel")) || !G) return rc;
  const size_t so = plan_scratch_offset(K);
  const int nblk = (G * G + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(lds_insert_kernel, dim3((G * G + 255) / 256), dim3(256), 0, st, p, so, G);
  if ((rc = check_launch("lds_insert_kernel"))) return rc;
  hipLaunchKernelGGL(lds_need_kernel, dim3(nblk), dim3(kScanBlock), 0, st, p, so, G);
  if ((rc = check_launch("lds_need_kernel"))) return rc;
  hipLaunchKernelGGL(lds_ids_kernel, dim3(nblk), dim3(kScanBlock), 0, st, p, so, G);
  if ((rc = check_launch("lds_ids_kernel"))) return rc;
  const int nthreads = G * G > kLdsBins ? G * G : kLdsBins;
  hipLaunchKernelGGL(lds_image_kernel, dim3((nthreads + 255) / 256), dim3(256), 0, st, p, so, plan_image_offset(K), G,
                     (int)g.cells_off, (int)g.lists_off, g.lists_cap, (int)g.image_bytes, E);
  return check_launch("lds_image_kernel");
}

}  // namespace qamw
