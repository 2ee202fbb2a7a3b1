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
// Two levels: an inner square [-5, 5)^2 where nearly all normalised pairs
// fall, and a coarse outer grid (128 cells per axis over [-20, 20)^2) for the
// few pairs beyond it -- rows dominated by one large weight put a whole
// Hadamard block there.  For K <= kLdsMaxK the inner square is the LDS table
// (non-uniform cells with exact candidate sets, below); for larger K it is a
// uniform 512 x 512 grid of supercell lists.  Each level has its own delta
// (R = 5 or 20 in the formula above).  The outer cells that tile the inner
// square are never consulted (points there take the inner level) and hold
// overflow records.
//
// Layout (plan_bytes(K) bytes, 256-byte aligned):
//   [0, 256)     PlanHeader
//   K > kLdsMaxK:  uniform inner grid, uint16 records [512*512][lmax], then
//                  the outer grid's [G2*G2][lmax]
//   K <= kLdsMaxK: the outer grid's records, then the LDS table image (bin
//                  map, cell entries, list records: qamw_internal.h), then the
//                  construction scratch of build_plan_kernel / lds_finish_kernel
// A uniform-grid record is 16 (lmax 8) or 32 (lmax 16) bytes: entry i is
// 16 c_i | nibble_i, c_i the i-th listed centroid (16 c_i is its byte offset in
// the encode kernel's LDS copy of the codebook), nibble_0 = count - 1,
// nibble_1 = 1 when the cell overflows (scan the whole codebook), other
// nibbles 0; entries past the count repeat the last listed centroid.
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
constexpr int kLdsLanes = 8;                           // LDS table: lanes per cell

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

// LDS of an inner-grid workgroup: the uniform grid (one lane per cell, 256
// cells) or the LDS table (eight lanes per cell, 32 cells).
template <bool kLdsTable>
struct PlanSharedT {
  static constexpr int kCells = kLdsTable ? kPlanThreads / kLdsLanes : kPlanThreads;
  uint16_t surv[kSuperMax];
  float2 survc[kSuperMax];
  uint16_t cell_list[kCells][16];
  float2 cand[kLdsTable ? kCells : 1][16];   // LDS table: a cell's loose candidates' coordinates
  unsigned long long ckey[kCells];           // LDS table: a cell's list (4 x 11-bit index) and class,
  int cneed[kCells];                         // records it needs, and its local record id
  float red[kPlanWaves];
  float red2[kPlanWaves];
  int wsum[kPlanWaves];
};

// The codebook in registers, once per workgroup: thread t holds centroids
// r kSuperMax + t P + u (round r < 2 since K <= 4096, u < P = kPerThread),
// loaded as float4 pairs; past K a far-away dummy that never passes a test.
constexpr int kRounds = 4096 / kSuperMax;
typedef float2 CbRegs[kRounds][kPerThread];
__device__ __forceinline__ void load_cb_regs(const float* __restrict__ cb, int K, CbRegs& v) {
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int c0 = r * kSuperMax + (int)threadIdx.x * kPerThread;
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
}

// The survivors of a supercell box SQ: every centroid with
// min_{z in SQ} |z - c|^2 <= U(SQ) + 2 delta, ascending, with coordinates, in
// sh.surv / sh.survc, padded with far-away dummies to whole rounds of `round`
// entries.  Returns their count (more than sh holds: `all` is set and the
// callers test every centroid from global memory); *cmax2 is the largest
// squared centroid radius and *delta the grid's score margin
// 1e-5 (Cmax + R sqrt 2)^2 (R: the grid's half-width).
template <typename SH>
__device__ int supercell_survivors(SH& sh, const CbRegs& v, int K, const Box& sq64, double R,
                                   int round, float* cmax2_out, double* delta_out, bool* all_out, int* ns_out) {
  constexpr int kCap = sizeof(sh.surv) / sizeof(sh.surv[0]);   // survivors the LDS holds
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
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
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {     // the two reductions side by side
    U = fminf(U, __shfl_xor(U, off));
    cmax2 = fmaxf(cmax2, __shfl_xor(cmax2, off));
  }
  if (lane == 0) { sh.red[wave] = U; sh.red2[wave] = cmax2; }
  __syncthreads();
  U = sh.red[0];
  cmax2 = sh.red2[0];
#pragma unroll
  for (int w = 1; w < kPlanWaves; ++w) { U = fminf(U, sh.red[w]); cmax2 = fmaxf(cmax2, sh.red2[w]); }
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
    // survivors in lower lanes of the wave, and in the wave: one ballot per slot u
    const uint64_t below = (1ull << lane) - 1ull;
    int in_wave_before = 0, in_wave = 0;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const uint64_t b = __ballot((mask >> u) & 1u);
      in_wave_before += __popcll(b & below);
      in_wave += __popcll(b);
    }
    __syncthreads();                        // the previous round's wsum reads are done
    if (lane == 0) sh.wsum[wave] = in_wave;
    __syncthreads();
    int before = nsurv + in_wave_before, total = nsurv;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      before += (w < wave) ? sh.wsum[w] : 0;
      total += sh.wsum[w];
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
      if ((mask >> u) & 1u) {
        if (before < kCap) { sh.surv[before] = (uint16_t)(c0 + u); sh.survc[before] = v[r][u]; }
        ++before;
      }
    nsurv = total;
  }
  __syncthreads();
  const bool all = nsurv > kCap;            // too many survivors: test every centroid (from global memory)
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
template <int S, typename SH>
__device__ void build_supercell(SH& sh, const float* __restrict__ cb, const CbRegs& v, int K, int lmax,
                                double R, int G, int sidx, uint16_t* __restrict__ lists) {
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
  supercell_survivors(sh, v, K, cell_box(R, G, sx * S, sy * S, S), R, kRound, &cmax2, &delta, &all, &ns);
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
// and one half-plane 2 z.(c' - c) <= |c'|^2 - |c|^2 + delta_Q per c'),
// decided by eliminating y (in fp64, with bounds that err towards listing).
// Only the cell's loose candidates
// (min_{z in Q} |z - c|^2 <= U(Q) + delta_Q) need testing or acting as c': any
// other centroid is farther than the one attaining U(Q) everywhere in Q.
// ===========================================================================
constexpr int kLdsSuperX = 8;          // LDS-table supercells: 8 x 4 cells, eight lanes per cell
constexpr int kLdsSuperY = 4;
constexpr int kLdsLoose = 16;          // loose candidates a cell may keep (more: scan all)
constexpr int kLdsListMax = 8;         // exact candidates a cell may list (more: scan all)
struct LdsEdges {
  uint16_t e[kLdsMaxG + 1];
};

// Global scratch of the build, per supercell of the LDS table (8 x 4 cells):
// its cells' entries before numbering (u32 per cell: the final 16-bit entry,
// or 1 << 16 | local record id, with 1 << 17 for a two-record list), its
// count of records, and the records themselves (at most two per cell).  Equal
// lists inside one supercell share a record; the table's record ids are the
// local ones offset by the records of the supercells before it.
constexpr int kLdsSuperCells = kLdsSuperX * kLdsSuperY;
static_assert(kLdsSuperCells * kLdsLanes == kPlanThreads, "one workgroup per supercell");
constexpr int kRecsPerSuper = 2 * kLdsSuperCells;
struct LdsScratch {
  uint32_t* desc;         // [G*G]
  int* nrec;              // [nsuper^2]
  uint2* recs;            // [supercells][kRecsPerSuper]
};
__host__ __device__ inline int lds_nsuper_x(int G) { return (G + kLdsSuperX - 1) / kLdsSuperX; }
__host__ __device__ inline int lds_nsuper_y(int G) { return (G + kLdsSuperY - 1) / kLdsSuperY; }
__host__ __device__ inline int lds_nsupercells(int G) { return lds_nsuper_x(G) * lds_nsuper_y(G); }
__host__ __device__ inline size_t lds_scratch_bytes(int G) {
  const size_t ns2 = (size_t)lds_nsupercells(G);
  return round_up((size_t)G * G * 4, 256) + round_up(ns2 * 4, 256) + ns2 * kRecsPerSuper * 8;
}
__device__ __forceinline__ LdsScratch lds_scratch(char* base, int G) {
  const size_t ns2 = (size_t)lds_nsupercells(G);
  LdsScratch s;
  s.desc = reinterpret_cast<uint32_t*>(base);
  base += round_up((size_t)G * G * 4, 256);
  s.nrec = reinterpret_cast<int*>(base);
  base += round_up(ns2 * 4, 256);
  s.recs = reinterpret_cast<uint2*>(base);
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
// in the set `keep` (a bitmask over the cell's candidates cand[0..n))?  Each
// such condition is the half-plane a_k . z <= b_k, a_k = 2 (c_k - c_i),
// b_k = |c_k|^2 - |c_i|^2 + delta, and q adds y <= y1, -y <= -y0 and the
// x-range [x0, x1].  Fourier-Motzkin elimination of y decides it exactly:
// every pair of an upper row (a_y > 0) and a lower row (a_y < 0) implies
// alpha x <= beta with alpha = ay_p ax_q - ay_q ax_p and beta = ay_p b_q -
// ay_q b_p, rows with a_y = 0 bound x directly, and the system has a
// solution iff the x-interval those bounds leave is not empty.  The a's are
// differences of fp32 values, exact in fp64, so the sign of alpha is exact;
// the b's and betas carry rounding, which every bound absorbs by moving
// outward (by 1e-12 of the magnitudes involved), so the test errs towards
// "feasible" (listing a centroid too many is harmless).  Bounds are kept as
// fractions and compared by cross-multiplication (no division per pair).
// The lanes of a cell share one test: lane sub takes the rows p = sub,
// sub + kLdsLanes, ... and the lanes' intervals are intersected.
__device__ bool lds_feasible(const float2* cand, int n, uint32_t keep, int i, const Box& q, double delta,
                             int sub) {
  const double cix = cand[i].x, ciy = cand[i].y, ci2 = cix * cix + ciy * ciy;
  // row r < n: candidate r (when kept and not i); r == n: y <= y1; r == n + 1: -y <= -y0.
  // s is the magnitude of b's terms, for its rounding bound.
  auto row = [&](int r, double& ax, double& ay, double& b, double& s) -> bool {
    if (r == n) { ax = 0.0; ay = 1.0; b = q.y1; s = fabs(q.y1); return true; }
    if (r == n + 1) { ax = 0.0; ay = -1.0; b = -q.y0; s = fabs(q.y0); return true; }
    if (r == i || !((keep >> r) & 1u)) return false;
    const double kx = cand[r].x, ky = cand[r].y, k2 = kx * kx + ky * ky;
    ax = 2.0 * (kx - cix);
    ay = 2.0 * (ky - ciy);
    b = k2 - ci2 + delta;
    s = k2 + ci2 + delta;
    return true;
  };
  // the x-interval [lo_n / lo_d, hi_n / hi_d] (denominators > 0): a bound
  // num / den replaces the current one when it is tighter, by cross-multiplying
  double lo_n = q.x0, lo_d = 1.0, hi_n = q.x1, hi_d = 1.0;
  bool bad = false;
  auto upper = [&](double num, double den) {
    if (num * hi_d < hi_n * den) { hi_n = num; hi_d = den; }
  };
  auto lower = [&](double num, double den) {
    if (num * lo_d > lo_n * den) { lo_n = num; lo_d = den; }
  };
  auto bound = [&](double al, double be) {      // al x <= be
    if (al > 0.0) upper(be, al);
    else if (al < 0.0) lower(-be, -al);          // x >= be / al = -be / -al
    else bad = bad || be < 0.0;
  };
  for (int p = sub; p < n + 2; p += kLdsLanes) {
    double axp, ayp, bp, sp;
    if (!row(p, axp, ayp, bp, sp)) continue;
    if (ayp == 0.0) {
      bound(axp, bp + 1e-12 * (fabs(bp) + sp));
      continue;
    }
    if (ayp < 0.0) continue;
    for (int r = 0; r < n + 2; ++r) {
      double axq, ayq, bq, sq;
      if (!row(r, axq, ayq, bq, sq) || !(ayq < 0.0)) continue;
      const double al = ayp * axq - ayq * axp;
      const double be = ayp * bq - ayq * bp;
      bound(al, be + 1e-12 * (ayp * (fabs(bq) + sq) - ayq * (fabs(bp) + sp)));
    }
  }
  // intersect the lanes' intervals
#pragma unroll
  for (int off = kLdsLanes / 2; off > 0; off >>= 1) {
    const double ln = __shfl_xor(lo_n, off), ld = __shfl_xor(lo_d, off);
    const double hn = __shfl_xor(hi_n, off), hd = __shfl_xor(hi_d, off);
    bad = __shfl_xor((int)bad, off) != 0 || bad;
    lower(ln, ld);
    upper(hn, hd);
  }
  // lo <= hi, with a relative tolerance
  const double lo = lo_n / lo_d, hi = hi_n / hi_d;
  return !bad && lo <= hi + 1e-12 * (1.0 + fabs(lo) + fabs(hi));
}

// One workgroup per 8 x 4-cell supercell of the LDS table: survivors, then
// eight lanes per cell: U(Q), delta_Q, the loose candidates (ascending), the
// dominance pruning and the exact test of what is left, split over the lanes.
static_assert(sizeof(PlanSharedT<true>::cand) / sizeof(PlanSharedT<true>::cand[0]) == kPlanThreads / kLdsLanes &&
              sizeof(PlanSharedT<true>::cand[0]) / sizeof(float2) >= kLdsLoose, "one candidate row per cell");
__device__ void build_lds_supercell(PlanSharedT<true>& sh, const CbRegs& v, int K, const LdsEdges& E, int G, int sidx,
                                    LdsScratch scr) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int nsy = lds_nsuper_y(G);
  const int sx = sidx / nsy, sy = sidx % nsy;
  const int x0 = sx * kLdsSuperX, y0 = sy * kLdsSuperY;
  const int x1 = min(x0 + kLdsSuperX, G), y1 = min(y0 + kLdsSuperY, G);
  constexpr int kRound = 4 * kLdsLanes;
  float cmax2;
  double delta;
  bool all;
  int ns;
  supercell_survivors(sh, v, K, lds_box(E, x0, x1, y0, y1), kPlanR, kRound, &cmax2, &delta, &all, &ns);
  // K <= kSuperMax here, so the survivors always fit (all == false)
  const int qc = tid / kLdsLanes, sub = tid % kLdsLanes;
  const int ix = x0 + qc / kLdsSuperY, iy = y0 + qc % kLdsSuperY;
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
  // ---- loose candidates in ascending order: survivors j = sub, sub + 8, ...,
  // one chunk of eight per ballot
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
  // (lane sub decides candidates sub, sub + 8, ...; the eight masks are or-ed)
  const bool over_loose = nl > kLdsLoose || nl == 0;
  const int n = over_loose ? 0 : nl;
  float2* cand = sh.cand[qc];
  for (int k = sub; k < n; k += kLdsLanes) cand[k] = sh.survc[mine[k]];
  __syncthreads();
  uint32_t undom = 0;
  for (int i = sub; i < n; i += kLdsLanes) {
    const float2 fi = cand[i];
    bool dominated = false;
    for (int k = 0; k < n && !dominated; ++k) {
      if (k == i) continue;
      const float2 fk = cand[k];
      dominated = corner_min_diff(cq64, fi.x, fi.y, fk.x, fk.y) > dq * (1.0 + 1e-9) + 1e-15;
    }
    if (!dominated) undom |= 1u << i;
  }
#pragma unroll
  for (int off = kLdsLanes / 2; off > 0; off >>= 1) undom |= (uint32_t)__shfl_xor((int)undom, off);
  // ---- a cheap sufficient test first: a candidate within dq of the minimum
  // at one of 16 points of the cell (a 4 x 4 grid including the corners;
  // lane sub takes column sub % 4 and two of its rows) qualifies.  fp32 here
  // can only keep a candidate too many, which is harmless.
  static_assert(kLdsLanes == 8, "two of the 16 points per lane");
  uint32_t keep = 0;
  if (__popc(undom) > 1) {
    const float px = cq.x0 + (cq.x1 - cq.x0) * (float)(sub & 3) * (1.0f / 3.0f);
    float py[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) py[t] = cq.y0 + (cq.y1 - cq.y0) * (float)(2 * (sub >> 2) + t) * (1.0f / 3.0f);
    const float dqf = (float)dq;
    float dmin[2] = {INFINITY, INFINITY};
    for (int k = 0; k < n; ++k) {
      if (!((undom >> k) & 1u)) continue;
      const float2 c = cand[k];
      const float dx = px - c.x;
#pragma unroll
      for (int t = 0; t < 2; ++t) dmin[t] = fminf(dmin[t], dx * dx + (py[t] - c.y) * (py[t] - c.y));
    }
    for (int k = 0; k < n; ++k) {
      if (!((undom >> k) & 1u)) continue;
      const float2 c = cand[k];
      const float dx = px - c.x;
      bool near = false;
#pragma unroll
      for (int t = 0; t < 2; ++t) near = near || dx * dx + (py[t] - c.y) * (py[t] - c.y) <= dmin[t] + dqf;
      if (near) keep |= 1u << k;
    }
  } else {
    keep = undom;
  }
#pragma unroll
  for (int off = kLdsLanes / 2; off > 0; off >>= 1) keep |= (uint32_t)__shfl_xor((int)keep, off);
  // ---- the exact test for the rest, each shared by the cell's lanes (the
  // same trip count in them: `rest` is the same in them)
  for (uint32_t rest = undom & ~keep; rest != 0u; rest &= rest - 1u) {
    const int i = __ffs(rest) - 1;
    if (lds_feasible(cand, n, undom, i, cq64, dq, sub)) keep |= 1u << i;
  }
  // ---- the cell's exact set, ascending (mine[] ascends): its class (0 scan
  // all, 1 one centroid, 2 a 2..4 list, 3 a 5..8 list) and entries
  const int count = __popc(keep);
  const bool over = over_loose || count > kLdsListMax || count == 0 || !real;
  uint32_t ent[kLdsListMax];
#pragma unroll
  for (int q = 0; q < kLdsListMax; ++q) ent[q] = 0;
  if (!over) {
    int c = 0;
    uint32_t last = 0;
    for (int i = 0; i < n; ++i)
      if ((keep >> i) & 1u) {
        last = 16u * sh.surv[mine[i]];
#pragma unroll
        for (int q = 0; q < kLdsListMax; ++q) ent[q] = (q == c) ? last : ent[q];
        ++c;
      }
#pragma unroll
    for (int q = 0; q < kLdsListMax; ++q) ent[q] = (q >= count) ? last : ent[q];
  }
  const int cls = over ? 0 : (count == 1 ? 1 : (count <= 4 ? 2 : 3));
  // ---- equal 2..4 lists share the record of the first cell holding them
  if (sub == 0) {
    const unsigned long long key = (unsigned long long)(ent[0] >> 4) | ((unsigned long long)(ent[1] >> 4) << 11) |
                                   ((unsigned long long)(ent[2] >> 4) << 22) |
                                   ((unsigned long long)(ent[3] >> 4) << 33);
    sh.ckey[qc] = key | ((unsigned long long)cls << 60);
  }
  __syncthreads();
  int owner = qc;
  if (cls == 2)
    for (int c = 0; c < qc; ++c)
      if (sh.ckey[c] == sh.ckey[qc]) { owner = c; break; }
  if (sub == 0) sh.cneed[qc] = cls == 3 ? 2 : (cls == 2 && owner == qc ? 1 : 0);
  __syncthreads();
  if (sub == 0 && real) {
    int lid = 0;                                 // the owner's local record id
    for (int c = 0; c < owner; ++c) lid += sh.cneed[c];
    uint32_t desc = kLdsScanAll;
    if (cls == 1) desc = ent[0];
    else if (cls >= 2) desc = (1u << 16) | (cls == 3 ? 1u << 17 : 0u) | (uint32_t)lid;
    scr.desc[(size_t)ix * G + iy] = desc;
    uint2* recs = scr.recs + (size_t)sidx * kRecsPerSuper;
    if (cls == 2 && owner == qc) recs[lid] = make_uint2(ent[0] | (ent[1] << 16), ent[2] | (ent[3] << 16));
    if (cls == 3) {
      recs[lid] = make_uint2(ent[0] | (ent[1] << 16), ent[2] | (ent[3] << 16) | 0x80000000u);   // continued
      recs[lid + 1] = make_uint2(ent[4] | (ent[5] << 16), ent[6] | (ent[7] << 16));
    }
  }
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int c = 0; c < kLdsSuperCells; ++c) tot += sh.cneed[c];
    scr.nrec[sidx] = tot;
  }
}

// One launch builds both grids: the inner grid's supercells (the LDS table's
// 8 x 4 cells with eight lanes per cell for K <= kLdsMaxK, else the uniform
// 512 x 512 grid's 16 x 16 cells with one lane per cell), then the outer
// grid's 4 x 4-cell supercells (16 lanes per cell; its cells are larger, so a
// 16 x 16 supercell would keep most of the codebook), several per workgroup.  Every workgroup
// computes the largest centroid radius itself (with U of its supercell);
// workgroup 0 writes the header.
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

// The outer grid: each workgroup builds a 2 x 2 block of 4 x 4-cell
// supercells, one per wavefront.  The block's survivors (the supercell test
// on the block's box, all 256 lanes) are a superset of each supercell's
// (a larger box has smaller distances and a larger U), and contain the
// centroid attaining each supercell's U; each wavefront then takes its
// supercell's survivors from them by ballot, and its 16 cells' lists with
// four lanes per cell, with no barrier.  The lists are the ones the
// supercell test on the whole codebook gives.
constexpr int kOuterPerWG = kPlanThreads / kWave;   // supercells per workgroup, 2 x 2
// a supercell's survivors kept (more: its cells use the block's list); the
// block's: up to K (more would mean the whole codebook from global memory)
constexpr int kOuterLPC = kWave / (kSuperOuter * kSuperOuter);
static_assert(kOuterPerWG == 4 && kOuterLPC == 4, "2 x 2 supercells per workgroup, four lanes per outer cell");
template <int kBlockCap, int kOuterSurvMax>
struct OuterShared {
  uint16_t surv[kBlockCap];                       // the block's survivors (supercell_survivors)
  float2 survc[kBlockCap];
  float red[kPlanWaves];
  float red2[kPlanWaves];
  int wsum[kPlanWaves];
  float2 wsurvc[kOuterPerWG][kOuterSurvMax];      // each supercell's
  uint16_t wsurv[kOuterPerWG][kOuterSurvMax];
  uint16_t list[kOuterPerWG][kSuperOuter * kSuperOuter][16];
};

template <typename OS>
__device__ void build_outer_block(OS& os, const float* __restrict__ cb, const CbRegs& v, int K, int lmax,
                                  uint16_t* __restrict__ lists, int blk) {
  constexpr int kOuterSurvMax = sizeof(os.wsurv[0]) / sizeof(os.wsurv[0][0]);
  constexpr int nsuper = kPlanG2 / kSuperOuter, nblk = nsuper / 2;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int bx = blk / nblk, by = blk % nblk;
  // ---- the block's survivors (and the grid's delta), all lanes
  float cmax2;
  double delta;
  bool ball;
  int nb;
  supercell_survivors(os, v, K, cell_box(kPlanR2, kPlanG2, bx * 2 * kSuperOuter, by * 2 * kSuperOuter, 2 * kSuperOuter),
                      kPlanR2, kWave, &cmax2, &delta, &ball, &nb);
  const int sx = 2 * bx + (w >> 1), sy = 2 * by + (w & 1), sidx = sx * nsuper + sy;
  if (outer_supercell_unused(sidx)) {          // never consulted: one overflow record per cell
    if (lane < kSuperOuter * kSuperOuter) {
      const int ix = sx * kSuperOuter + lane / kSuperOuter, iy = sy * kSuperOuter + lane % kSuperOuter;
      uint4* out = reinterpret_cast<uint4*>(lists + ((size_t)ix * kPlanG2 + iy) * lmax);
      out[0] = make_uint4(1u << 16, 0u, 0u, 0u);
      if (lmax == 16) out[1] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  // the block's list (padded to whole wavefronts), or the whole codebook
  auto bsurv = [&](int j, float2* c, int* idx) {
    if (ball) { *c = make_float2(cb[2 * j], cb[2 * j + 1]); *idx = j; }
    else { *c = os.survc[j]; *idx = os.surv[j]; }
  };
  const Box sq64 = cell_box(kPlanR2, kPlanG2, sx * kSuperOuter, sy * kSuperOuter, kSuperOuter);
  const BoxF sq{f32_down(sq64.x0), f32_up(sq64.x1), f32_down(sq64.y0), f32_up(sq64.y1)};
  // ---- U(SQ) (margins as in supercell_survivors): the block's list holds its minimiser
  float U = INFINITY;
  for (int j = lane; j < nb; j += kWave) {
    float2 c;
    int idx;
    bsurv(j, &c, &idx);
    U = fminf(U, sq.dmax2(c.x, c.y));
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) U = fminf(U, __shfl_xor(U, off));
  const float slim = (U * 1.000001f + f32_up(2.0 * delta)) * 1.000001f;
  // ---- the supercell's survivors, ascending, compacted by ballot
  float2* survc = os.wsurvc[w];
  uint16_t* surv = os.wsurv[w];
  const uint64_t below = (1ull << lane) - 1ull;
  int ns = 0;
  for (int j0 = 0; j0 < nb; j0 += kWave) {      // nb is a whole number of wavefronts (or K)
    const int j = j0 + lane;
    float2 c = make_float2(1e30f, 1e30f);
    int idx = 0;
    if (j < nb) bsurv(j, &c, &idx);
    const bool pred = j < nb && sq.dmin2(c.x, c.y) <= slim;
    const uint64_t b = __ballot(pred);
    const int pos = ns + __popcll(b & below);
    if (pred && pos < kOuterSurvMax) { survc[pos] = c; surv[pos] = (uint16_t)idx; }
    ns += __popcll(b);
  }
  const bool wall = ns > kOuterSurvMax;          // too many: the cells test the block's list
  const int nsp = wall ? nb : (ns + kOuterLPC - 1) / kOuterLPC * kOuterLPC;
  if (!wall && ns + lane < nsp) { survc[ns + lane] = make_float2(1e30f, 1e30f); surv[ns + lane] = 0; }
  wave_lds_fence();
  auto src = [&](int j, float2* c, int* idx) {
    if (wall) bsurv(j, c, idx);
    else { *c = survc[j]; *idx = surv[j]; }
  };
  // ---- four lanes per cell: U(Q), then the loose list in index order
  const int qc = lane / kOuterLPC, sub = lane % kOuterLPC;
  const int ix = sx * kSuperOuter + qc / kSuperOuter, iy = sy * kSuperOuter + qc % kSuperOuter;
  const Box cq64 = cell_box(kPlanR2, kPlanG2, ix, iy, 1);
  const BoxF cq{f32_down(cq64.x0), f32_up(cq64.x1), f32_down(cq64.y0), f32_up(cq64.y1)};
  float Uc = INFINITY;
  for (int j = sub; j < nsp; j += kOuterLPC) {
    float2 c;
    int idx;
    src(j, &c, &idx);
    Uc = fminf(Uc, cq.dmax2(c.x, c.y));
  }
#pragma unroll
  for (int off = kOuterLPC / 2; off > 0; off >>= 1) Uc = fminf(Uc, __shfl_xor(Uc, off));
  const float lim = (Uc * 1.000001f + f32_up(delta)) * 1.000001f;
  uint16_t* mine = os.list[w][qc];
  const int gshift = lane & ~(kOuterLPC - 1);
  int count = 0;
  for (int j0 = 0; j0 < nsp; j0 += kOuterLPC) {   // the same trip count in every lane
    const int j = j0 + sub;
    float2 c;
    int idx;
    src(min(j, nsp - 1), &c, &idx);
    const bool pred = j < nsp && cq.dmin2(c.x, c.y) <= lim;
    const uint64_t gm = (__ballot(pred) >> gshift) & ((1ull << kOuterLPC) - 1ull);
    const int pos = count + __popcll(gm & ((1ull << sub) - 1ull));
    if (pred && pos < lmax) mine[pos] = (uint16_t)(16 * idx);
    count += __popcll(gm);
  }
  wave_lds_fence();
  if (sub != 0) return;
  // ---- the record: tail repeats the last entry (rescoring it never wins a strict "<")
  const bool overflow = count > lmax || count == 0;
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
  uint4* out = reinterpret_cast<uint4*>(lists + ((size_t)ix * kPlanG2 + iy) * lmax);
  out[0] = make_uint4(words[0], words[1], words[2], words[3]);
  if (lmax == 16) out[1] = make_uint4(words[4], words[5], words[6], words[7]);
}

// Both grids in one launch: workgroups [0, ninner) build the inner grid's
// supercells (dispatched first: near the origin they hold the most work),
// the rest the outer grid's.
template <bool kLdsTable>
__global__ __launch_bounds__(kPlanThreads) void build_plan_kernel(const float* __restrict__ cb, int K, int lmax,
                                                                  char* __restrict__ plan, int lds_G, LdsEdges edges,
                                                                  size_t scratch_offset, int ninner,
                                                                  size_t outer_offset) {
  __shared__ union {
    PlanSharedT<kLdsTable> inner;
    OuterShared<kLdsTable ? kLdsMaxK : 4096, kLdsTable ? 128 : 256> outer;
  } lds;
  CbRegs v;
  load_cb_regs(cb, K, v);
  if ((int)blockIdx.x >= ninner) {
    build_outer_block(lds.outer, cb, v, K, lmax, reinterpret_cast<uint16_t*>(plan + outer_offset),
                      (int)blockIdx.x - ninner);
    return;
  }
  auto& sh = lds.inner;
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
    // the LDS table's fields: lds_finish_kernel fills them when there is one
    hdr->lds_G = hdr->lds_bins = hdr->lds_lists_cap = hdr->lds_nlists = 0;
    hdr->lds_image_bytes = hdr->lds_cells_off = hdr->lds_lists_off = hdr->lds_image_off = 0;
  }
  if constexpr (kLdsTable)
    build_lds_supercell(sh, v, K, edges, lds_G, blockIdx.x, lds_scratch(plan + scratch_offset, lds_G));
  else
    build_supercell<kSuperFine>(sh, cb, v, K, lmax, kPlanR, kPlanG, blockIdx.x,
                                reinterpret_cast<uint16_t*>(plan + kPlanHeaderBytes));
}

// ---- the table image, one workgroup per supercell (at least eight): its record ids start
// after the records of the supercells before it (in index order), so the
// image is a pure function of the cells' sets.  Records past the capacity
// are not written; their cells scan the whole codebook.  The first eight
// workgroups also write the bin -> cell map, workgroup 0 the cell padding and
// the header's table fields; every workgroup clears a stripe of the unused
// records.
constexpr int kFinishThreads = 256;
__global__ __launch_bounds__(kFinishThreads) void lds_finish_kernel(char* __restrict__ plan, size_t scratch_offset,
                                                                    size_t image_offset, int G, int cells_off,
                                                                    int lists_off, int lists_cap, int image_bytes,
                                                                    LdsEdges E) {
  __shared__ int red[2][kFinishThreads / kWave];
  __shared__ uint16_t edges[kLdsMaxG + 1];
  static_assert(kLdsBins % kFinishThreads == 0, "whole workgroups of bins");
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t >> 6;
  const int sidx = blockIdx.x, nsy = lds_nsuper_y(G), ns2 = lds_nsupercells(G);
  LdsScratch scr = lds_scratch(plan + scratch_offset, G);
  char* img = plan + image_offset;
  uint16_t* cells = reinterpret_cast<uint16_t*>(img + cells_off);
  uint2* lists = reinterpret_cast<uint2*>(img + lists_off);
  // this supercell's cell entries and records (workgroups past the last
  // supercell have none), loaded before the wait for the counts
  const bool real = sidx < ns2;
  const int mine = real ? scr.nrec[sidx] : 0;
  const int ix = (sidx / nsy) * kLdsSuperX + t / kLdsSuperY, iy = (sidx % nsy) * kLdsSuperY + t % kLdsSuperY;
  const bool has_cell = real && t < kLdsSuperCells && ix < G && iy < G;
  const uint32_t d = has_cell ? scr.desc[(size_t)ix * G + iy] : 0u;
  static_assert(kRecsPerSuper <= kFinishThreads, "one record per thread");
  const uint2 rec = t < mine ? scr.recs[(size_t)sidx * kRecsPerSuper + t] : make_uint2(0u, 0u);
  // records before this supercell, and in all
  int before = 0, total = 0;
  for (int i = t; i < ns2; i += kFinishThreads) {
    const int v = scr.nrec[i];
    before += i < sidx ? v : 0;
    total += v;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    before += __shfl_xor(before, off);
    total += __shfl_xor(total, off);
  }
  if (lane == 0) { red[0][wave] = before; red[1][wave] = total; }
  __syncthreads();
  before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kFinishThreads / kWave; ++w) { before += red[0][w]; total += red[1][w]; }
  const int used = min(total, lists_cap);
  if (t < mine && before + t < used) lists[before + t] = rec;
  if (has_cell) {
    uint16_t entry = (uint16_t)d;
    if (d >> 16) {
      const int id = before + (int)(d & 0xffffu);
      entry = (id + ((d >> 17) & 1) < used) ? (uint16_t)(0x8000u | (unsigned)id) : kLdsScanAll;
    }
    cells[(size_t)ix * G + iy] = entry;
  }
  for (int i = used + sidx * kFinishThreads + t; i < lists_cap; i += (int)gridDim.x * kFinishThreads)
    lists[i] = make_uint2(0u, 0u);
  // the bin -> cell map, one bin per thread over the first workgroups: the c
  // with e[c] <= bin < e[c + 1], by binary search over the edges (in LDS)
  const int bin = sidx * kFinishThreads + t;
  if (sidx < kLdsBins / kFinishThreads) {
    for (int c = t; c <= G; c += kFinishThreads) edges[c] = E.e[c];
    __syncthreads();
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (edges[mid] <= bin) lo = mid; else hi = mid;
    }
    reinterpret_cast<uint8_t*>(img)[bin] = (uint8_t)lo;
  }
  if (sidx != 0) return;
  const int pad_end = (lists_off - cells_off) / 2;
  for (int i = G * G + t; i < pad_end; i += kFinishThreads) cells[i] = 0;
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
  // the encode kernel holds the map and cells in its own layout (guard bins,
  // a guard row and column): the records get what is left of its LDS
  const long avail = (long)kLdsBudget - 8L * K - (long)(kLdsWaves * g->stage_bytes) - (long)kLdsMapBytes -
                     (long)lds_cell_bytes(G);
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
    ninner = lds_nsupercells(G);
  }
  char* p = (char*)plan;
  const dim3 grid(ninner + kOuterSupercells / kOuterPerWG);
  if (G)
    hipLaunchKernelGGL(build_plan_kernel<true>, grid, dim3(kPlanThreads), 0, st, cb, K, plan_lmax(K), p, G, E,
                       plan_scratch_offset(K), ninner, plan_outer_offset(K));
  else
    hipLaunchKernelGGL(build_plan_kernel<false>, grid, dim3(kPlanThreads), 0, st, cb, K, plan_lmax(K), p, G, E,
                       plan_scratch_offset(K), ninner, plan_outer_offset(K));
  int rc = check_launch("build_plan_kernel");
  if (rc || !G) return rc;
  const int nfin = lds_nsupercells(G) > kLdsBins / kFinishThreads ? lds_nsupercells(G) : kLdsBins / kFinishThreads;
  hipLaunchKernelGGL(lds_finish_kernel, dim3(nfin), dim3(kFinishThreads), 0, st, p,
                     plan_scratch_offset(K),
                     plan_image_offset(K), G, (int)g.cells_off, (int)g.lists_off, g.lists_cap, (int)g.image_bytes, E);
  return check_launch("lds_finish_kernel");
}

}  // namespace qamw
