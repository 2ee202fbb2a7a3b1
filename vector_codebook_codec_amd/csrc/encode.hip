// Encode kernels: rotation, normalisation, nearest centroid and bit packing
// ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Separation of Scale and
// Direction, Deterministic Rotation, Pairing and Calibration, Joint 2D
// Quantization).
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"
#include "encode_window.h"

namespace qamw {

// ---------------------------------------------------------------------------
// Encode.  One wavefront per (row, window): 512 pairs; eight wavefronts per
// workgroup share one copy of the codebook in LDS.
//
// Nearest centroid on the expanded score S_c = |c|^2/2 - z.c, which orders
// centroids exactly as |z - c|^2 does.  The scores of 32 centroids x 32 pairs
// are one v_mfma_f32_32x32x2_f32:  A[i][k] = (-cx_i, -cy_i),  B[k][j] =
// (zx_j, zy_j),  C[i][j] = |c_i|^2 / 2.  That instruction computes
// fma(A[i][1], B[1][j], fma(A[i][0], B[0][j], C[i][j])) in fp32 -- exactly
// the VALU sequence fma(zy, -cy, fma(zx, -cx, h)) -- so every score is
// reproducible on the VALU bit for bit.
//
// Accumulator layout (32x32 fp32 MFMA): lane l, register r holds row
// (r & 3) + 8 (r >> 2) + 4 (l >> 5), column l & 31.  Each lane therefore sees
// 16 of a tile's 32 centroids for one pair, folds them into a running minimum
// with v_min3, and records the tile whenever that minimum drops strictly.
// Afterwards the two half-waves' minima are combined, and the recorded tile is
// rescanned on the VALU for the smallest index whose score equals the
// minimum: exact ties go to the lowest index.
// ---------------------------------------------------------------------------
constexpr int kTile = 32;                              // centroids per MFMA tile
constexpr int kPairSets = kWinPairs / 32;              // 16 MFMA columns blocks per window

typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Shared by both encode kernels.
// ---------------------------------------------------------------------------
// Encode, phase 1, in one launch: workgroups [0, row_blocks) compute the row
// norms (one wavefront per row); the rest compute the per-matrix factors of
// the transform: f_j = eps_j s_j (sign mask times channel scale, exact) and
// 1 / sigma_k (fp64 division rounded to fp32; 0 where sigma_k <= 0, which
// codes z~ = 0).
template <typename Tin>
__global__ __launch_bounds__(kBlockThreads) void encode_prepare_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ s,
    const float* __restrict__ sigma, uint64_t seed, int row_blocks, double sqrt_b, double* __restrict__ rho,
    uint16_t* __restrict__ rho_f16, float* __restrict__ f, float* __restrict__ isig) {
  if ((int)blockIdx.x < row_blocks) {
    const int n = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (n < N) row_norm_wave(W, ldw, n, d, s, sqrt_b, rho, rho_f16);
    return;
  }
  const int j = (blockIdx.x - row_blocks) * kBlockThreads + threadIdx.x;
  if (j < d) f[j] = s[j] * sign_eps(seed, (uint32_t)j);
  if (j < d / 2) {
    const float sg = sigma[j];
    isig[j] = sg > 0.0f ? (float)(1.0 / (double)sg) : 0.0f;
  }
}

template <int L, typename Tin>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(4))) void encode_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ f,
    const float* __restrict__ isig, const float* __restrict__ codebook, int K, int Kpad,
    int B, int row_words, const double* __restrict__ rho, uint32_t* __restrict__ packed) {
  extern __shared__ float4 lds4[];
  float* cbx = reinterpret_cast<float*>(lds4);   // -cx
  float* cby = cbx + Kpad;                       // -cy
  float* cbh = cby + Kpad;                       // |c|^2 / 2
  float2* zall = reinterpret_cast<float2*>(cbh + Kpad);

  for (int c = threadIdx.x; c < Kpad; c += kEncThreads) {
    if (c < K) {
      const float cx = codebook[2 * c], cy = codebook[2 * c + 1];
      cbx[c] = -cx;
      cby[c] = -cy;
      cbh[c] = 0.5f * __builtin_fmaf(cx, cx, cy * cy);
    } else {
      cbx[c] = 0.0f;
      cby[c] = 0.0f;
      cbh[c] = INFINITY;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  float2* zbuf = zall + wave * kWinPairs;         // the window's normalised pairs, window order
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int gw = blockIdx.x * kEncWaves + wave;
  if ((int64_t)gw >= (int64_t)N * nwin) return;   // no barriers follow
  const int n = gw / nwin;
  const int win = gw % nwin;
  {
    float zx[8], zy[8];
    const bool active = win * kWinChunks + lane < nchunks;   // whole Hadamard blocks are active or not
    WinLoads<Tin> wl;
    load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
    const int co_local = window_transform<L>(wl, active, lane, zx, zy);
#pragma unroll
    for (int p = 0; p < 8; ++p) zbuf[co_local * kPairsPerLane + p] = make_float2(zx[p], zy[p]);
  }
  wave_lds_fence();

  // ---- MFMA operands: B column block ps = window pairs [32 ps, 32 ps + 32)
  const int half = lane >> 5;                      // 0: k = 0 (x), 1: k = 1 (y)
  const int jcol = lane & 31;
  float bop[kPairSets];
#pragma unroll
  for (int ps = 0; ps < kPairSets; ++ps) {
    const float2 z = zbuf[ps * 32 + jcol];
    bop[ps] = half ? z.y : z.x;
  }
  const float* abase = (half ? cby : cbx) + jcol;  // A[i][k]: row i = jcol of the tile
  const float* hbase = cbh + 4 * half;             // C rows of this half-wave

  float best[kPairSets];
  int tile_of_best[kPairSets];
#pragma unroll
  for (int ps = 0; ps < kPairSets; ++ps) { best[ps] = INFINITY; tile_of_best[ps] = 0; }

  // Each column block's scores are folded right after its MFMA (on this chip
  // the fp32 MFMAs and the VALU do not overlap, so deferring the fold under
  // the next MFMA gains nothing and costs an accumulator set).  Tiles go in
  // pairs with their own A and C operand registers: each register set is
  // reloaded for the tile after next as soon as its tile's MFMAs are issued,
  // so no operand is copied and every load has a whole tile to land.
  auto fold = [&](const f32x16& dsc, int ps, int c0) {
    float m = best[ps];
#pragma unroll
    for (int r = 0; r < 16; r += 2) m = fminf(fminf(m, dsc[r]), dsc[r + 1]);   // v_min3
    tile_of_best[ps] = (m < best[ps]) ? c0 : tile_of_best[ps];
    best[ps] = m;
  };
  auto load_c = [&](int c0, f32x16& cop) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 h4 = *reinterpret_cast<const float4*>(hbase + c0 + 8 * g);
      cop[4 * g + 0] = h4.x; cop[4 * g + 1] = h4.y; cop[4 * g + 2] = h4.z; cop[4 * g + 3] = h4.w;
    }
  };
  auto tile = [&](float aop, const f32x16& cop, int c0) {
#pragma unroll
    for (int ps = 0; ps < kPairSets; ++ps)
      fold(__builtin_amdgcn_mfma_f32_32x32x2f32(aop, bop[ps], cop, 0, 0, 0), ps, c0);
  };
  // tiles in pairs, then an odd last tile; padded centroids score +inf
  float a0 = abase[0], a1 = abase[min(kTile, Kpad - kTile)];
  f32x16 c0v, c1v;
  load_c(0, c0v);
  load_c(min(kTile, Kpad - kTile), c1v);
  int c0 = 0;
  for (; c0 + 2 * kTile <= Kpad; c0 += 2 * kTile) {
    const int cn0 = c0 + 2 * kTile < Kpad ? c0 + 2 * kTile : 0;   // past the end: any valid tile
    const int cn1 = c0 + 3 * kTile < Kpad ? c0 + 3 * kTile : 0;
    tile(a0, c0v, c0);
    a0 = abase[cn0];
    load_c(cn0, c0v);
    tile(a1, c1v, c0 + kTile);
    a1 = abase[cn1];
    load_c(cn1, c1v);
  }
  if (c0 < Kpad) tile(a0, c0v, c0);

  // ---- combine the half-waves: smaller minimum, then earlier tile.  A
  // half-wave holds rows 8 g + 4 half + k (g, k < 4) of every tile, so the
  // rescan below needs only the 16 rows of the half that holds the minimum
  // in the recorded tile -- both halves when they tie in the same tile.
  uint32_t from_other = 0, both_halves = 0;
#pragma unroll
  for (int ps = 0; ps < kPairSets; ++ps) {
    const float ob = __shfl_xor(best[ps], 32);
    const int ot = __shfl_xor(tile_of_best[ps], 32);
    const bool take = ob < best[ps] || (ob == best[ps] && ot < tile_of_best[ps]);
    both_halves |= (ob == best[ps] && ot == tile_of_best[ps]) ? 1u << ps : 0u;
    from_other |= take ? 1u << ps : 0u;
    if (take) { best[ps] = ob; tile_of_best[ps] = ot; }
  }

  // ---- lowest index: rescan the tile; lane handles column blocks 2m + half
  uint32_t idxv[kPairSets / 2];
#pragma unroll
  for (int m2 = 0; m2 < kPairSets / 2; ++m2) {
    const int ps = 2 * m2 + half;
    const float bb = half ? best[2 * m2 + 1] : best[2 * m2];
    const int t0 = half ? tile_of_best[2 * m2 + 1] : tile_of_best[2 * m2];
    const float2 z = zbuf[ps * 32 + jcol];
    const int src = ((from_other >> ps) & 1u) ? (half ^ 1) : half;
    const bool both = (both_halves >> ps) & 1u;
    // lane-rotated order keeps the lanes on different LDS banks (tiles start
    // on multiples of 32 entries); the smallest matching index wins
    int id = INT_MAX;
    const int span = both ? kTile : kTile / 2;
    for (int cc = 0; cc < span; ++cc) {
      const int q = (cc + lane) & (span - 1);
      const int ci = t0 + (both ? q : 8 * (q >> 2) + 4 * src + (q & 3));
      const float sc = __builtin_fmaf(z.y, cby[ci], __builtin_fmaf(z.x, cbx[ci], cbh[ci]));
      id = (sc == bb) ? min(id, ci) : id;
    }
    // no score of the tile equals the minimum (a NaN pair has no finite
    // score): the whole codebook on the VALU, first strict minimum, as the
    // planned search's scan does -- index 0 when no score is below +inf
    if (__any(id == INT_MAX)) {
      float fb = INFINITY;
      int fo = 0;
      for (int cc = 0; cc < K; ++cc) {                 // same address in every lane: broadcast
        const float sc = __builtin_fmaf(z.y, cby[cc], __builtin_fmaf(z.x, cbx[cc], cbh[cc]));
        if (sc < fb) { fb = sc; fo = cc; }
      }
      if (id == INT_MAX) id = fo;
    }
    idxv[m2] = (uint32_t)id;
  }

  // ---- pack: stage the window's 512 indices (reusing the pair buffer), then
  // build whole words; the window owns words [16*B*win, 16*B*(win+1))
  uint16_t* stage = reinterpret_cast<uint16_t*>(zbuf);
  wave_lds_fence();
#pragma unroll
  for (int m2 = 0; m2 < kPairSets / 2; ++m2) stage[(2 * m2 + half) * 32 + jcol] = (uint16_t)idxv[m2];
  wave_lds_fence();
  pack_window(stage, lane, win, nwin, d >> 1, B, row_words, packed + (int64_t)n * row_words);
}

// ---------------------------------------------------------------------------
// Encode with a search plan (plan.hip).  Same transform and packing as the
// exhaustive kernel; each pair scores only the centroids listed for its grid
// cell, in ascending index order, with the same fp32 FMA sequence and a strict
// "<", which returns the exhaustive search's index (the plan's lists contain
// every centroid that can be the fp32 minimum in the cell).  Pairs outside the
// grids or in overflowing cells scan the whole codebook.
//
// The codebook sits in LDS as (-cx, -cy) per centroid, one 8-byte gather per
// candidate at half the byte offset 16 c the list stores.  A lane's
// pairs are scored in groups of PG with all their record loads issued
// together; list slot i is scored for the whole group while any lane of the
// wavefront has a pair with more than i candidates (a list's unused tail
// repeats its last entry, which cannot win a strict "<" again).
// ---------------------------------------------------------------------------
constexpr int kPlanWgPerCu = 2;   // 4 wavefronts per SIMD

template <int L, typename Tin, int KMAX, int LMAX, int PG>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(4))) void encode_plan_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ f,
    const float* __restrict__ isig, const float* __restrict__ codebook, int K, int B, int row_words,
    const double* __restrict__ rho, const int* __restrict__ plan_K, const uint16_t* __restrict__ lists,
    const uint16_t* __restrict__ lists2, uint32_t* __restrict__ packed) {
  static_assert(LMAX % 8 == 0 && LMAX <= 16 && kPairsPerLane % PG == 0, "list and group sizes");
  __shared__ float2 cb2[KMAX];                                      // (-cx, -cy)
  __shared__ uint16_t stage_all[kEncWaves * kWinPairs];             // 8 waves x 512 indices
  const char* cbytes = reinterpret_cast<const char*>(cb2);

  for (int c = threadIdx.x; c < K; c += kEncThreads) {
    const float cx = codebook[2 * c], cy = codebook[2 * c + 1];
    cb2[c] = make_float2(-cx, -cy);
  }
  __syncthreads();
  // Twice the score of centroid c from (x2, y2) = 2 z~: fma(y2, -cy, fma(x2,
  // -cx, |c|^2)), |c|^2 = fma(cx, cx, cy cy) -- every step exactly twice the
  // exhaustive search's fma(y, -cy, fma(x, -cx, |c|^2 / 2)), so the order and
  // the ties are the same; 8-byte gathers meet far fewer bank conflicts.
  auto score2 = [](float x2, float y2, float2 c) -> float {
    return __builtin_fmaf(y2, c.y, __builtin_fmaf(x2, c.x, __builtin_fmaf(c.x, c.x, c.y * c.y)));
  };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: window bookkeeping stays scalar
  uint16_t* stage = stage_all + wave * kWinPairs;
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int total = N * nwin;                      // fits in int (checked on the host)
  const int stride = gridDim.x * kEncWaves;
  int gw = blockIdx.x * kEncWaves + wave;
  if (gw >= total) return;                         // no barriers follow

  // persistent wavefront: windows gw, gw + stride, ...; the next window's
  // weights are loaded while the current one is searched
  int n = gw / nwin, win = gw - (gw / nwin) * nwin;
  WinLoads<Tin> wl;
  load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);

  // the lanes hold 2 z~: the cell factors are halved (exactly)
  const float cells_per_unit = 0.5f * ((float)kPlanG / (2.0f * kPlanR));
  const float cells_per_unit2 = 0.5f * ((float)kPlanG2 / (2.0f * kPlanR2));
  const float tmax = __uint_as_float(__float_as_uint((float)kPlanG) - 1u);     // largest float below G
  const float tmax2 = __uint_as_float(__float_as_uint((float)kPlanG2) - 1u);
  const bool plan_ok = *plan_K == K;   // a plan built for another K: scan the whole codebook

  for (;;) {
    const bool active = win * kWinChunks + lane < nchunks;   // whole Hadamard blocks are active or not
    float zx[8], zy[8];                            // 2 z~ (see score2)
    const int co_local = window_transform<L, Tin, 2>(wl, active, lane, zx, zy);
    const int n_cur = n, win_cur = win;
    const int gnext = gw + stride;
    {
      // the next window's loads stay in flight during the search; past the
      // end the last window is loaded again (unused), keeping them unconditional
      const int gl = min(gnext, total - 1);
      n = gl / nwin;
      win = gl - n * nwin;
      load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
    }

#pragma unroll
    for (int g = 0; g < kPairsPerLane; g += PG) {
      uint32_t words[PG][LMAX / 2];
      bool inside[PG];
      const uint4* recp[PG];
      // ---- every record load of the group first.  Cell coordinate t = x G/(2R) + G/2:
      // its rounding error (< 1e-5 cell) is far inside the plan's eta margin;
      // the clamp changes nothing inside the grid, so "unchanged" is the range test
#pragma unroll
      for (int p = 0; p < PG; ++p) {
        const float x = zx[g + p], y = zy[g + p];
        const float tx = __builtin_fmaf(x, cells_per_unit, 0.5f * kPlanG);
        const float ty = __builtin_fmaf(y, cells_per_unit, 0.5f * kPlanG);
        const float cx = __builtin_amdgcn_fmed3f(tx, 0.0f, tmax);
        const float cy = __builtin_amdgcn_fmed3f(ty, 0.0f, tmax);
        const bool fine = cx == tx && cy == ty;      // false for NaN
        const uint16_t* rec = lists + (size_t)((int)cx * kPlanG + (int)cy) * LMAX;
        inside[p] = plan_ok;
        if (!fine) {                                 // rare: the outer grid, else a full scan
          const float ux = __builtin_fmaf(x, cells_per_unit2, 0.5f * kPlanG2);
          const float uy = __builtin_fmaf(y, cells_per_unit2, 0.5f * kPlanG2);
          const float vx = __builtin_amdgcn_fmed3f(ux, 0.0f, tmax2);
          const float vy = __builtin_amdgcn_fmed3f(uy, 0.0f, tmax2);
          inside[p] = plan_ok && vx == ux && vy == uy;
          rec = lists2 + (size_t)(inside[p] ? (int)vx * kPlanG2 + (int)vy : 0) * LMAX;
        }
        // the record's first 16 bytes (entries 0..7); the rest only for
        // lists of more than 8, below
        recp[p] = reinterpret_cast<const uint4*>(rec);
        const uint4 t = recp[p][0];
        words[p][0] = t.x; words[p][1] = t.y; words[p][2] = t.z; words[p][3] = t.w;
      }
      // ---- record flags: nibble 0 = count - 1, nibble 1 = overflow
      bool full[PG];
      int maxc = 1, cnt[PG];
#pragma unroll
      for (int p = 0; p < PG; ++p) {
        const uint32_t w0 = words[p][0];
        full[p] = !inside[p] || ((w0 >> 16) & 1u);
        cnt[p] = full[p] ? 1 : (int)(w0 & 15u) + 1;
        maxc = max(maxc, cnt[p]);
        words[p][0] = w0 & 0xfff0fff0u;
      }
      if constexpr (LMAX > 8) {
        // entries 8..15 for the lanes whose list is longer than 8 (rare);
        // the others repeat their entry 7, which cannot win a strict "<" again
        bool longer[PG];
        bool any_longer = false;
#pragma unroll
        for (int p = 0; p < PG; ++p) {
          longer[p] = cnt[p] > 8;
          any_longer |= longer[p];
        }
        if (__any(any_longer)) {
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            const uint32_t rep = (words[p][3] >> 16) * 0x10001u;
            uint4 t = make_uint4(rep, rep, rep, rep);
            if (longer[p]) t = recp[p][1];
            words[p][4] = t.x; words[p][5] = t.y; words[p][6] = t.z; words[p][7] = t.w;
          }
        }
      }
      // ---- list slots, two per word
      float best[PG];
      uint32_t boff[PG];
#pragma unroll
      for (int p = 0; p < PG; ++p) { best[p] = INFINITY; boff[p] = 0; }
#pragma unroll
      for (int w = 0; w < LMAX / 2; ++w) {
        if (w > 0 && !__any(2 * w < maxc)) continue;     // wave-uniform; later words are skipped too
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t off[PG];                    // 8 c: the entry's 16 c halved
          float2 e[PG];
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            off[p] = h ? (words[p][w] >> 17) : ((words[p][w] & 0xffffu) >> 1);
            e[p] = *reinterpret_cast<const float2*>(__builtin_assume_aligned(cbytes + off[p], 8));
          }
          __builtin_amdgcn_sched_barrier(0);   // keep the group's LDS reads in flight together
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            const float sc = score2(zx[g + p], zy[g + p], e[p]);
            if (sc < best[p]) { best[p] = sc; boff[p] = off[p]; }
          }
        }
      }
      // ---- pairs outside the grids or in overflowing cells: the whole codebook
#pragma unroll
      for (int p = 0; p < PG; ++p) {
        if (__any(full[p])) {
          float fb = INFINITY;
          uint32_t fo = 0;
          for (int cc = 0; cc < K; ++cc) {
            const float sc = score2(zx[g + p], zy[g + p], cb2[cc]);   // same address in every lane: broadcast
            if (sc < fb) { fb = sc; fo = (uint32_t)cc * 8u; }
          }
          if (full[p]) boff[p] = fo;
        }
        stage[co_local * kPairsPerLane + g + p] = (uint16_t)(boff[p] >> 3);
      }
    }
    wave_lds_fence();
    pack_window(stage, lane, win_cur, nwin, d >> 1, B, row_words, packed + (int64_t)n_cur * row_words);
    gw = gnext;
    if (gw >= total) break;
    wave_lds_fence();                              // the stage is rewritten next round
  }
}

// ---------------------------------------------------------------------------
// Encode with the LDS search table (plan.hip, K <= kLdsMaxK).  One workgroup
// of 16 wavefronts per CU keeps the codebook (-cx, -cy) and the plan's table
// in LDS: the bin -> cell map shared by both axes, one 16-bit
// entry per cell (16 c: the cell's only candidate; 0x8000 | r: list record r;
// 0xFFFF: scan the whole codebook) and the list records (4 x 16 c, ascending,
// the tail repeating the last; the top bit of the fourth entry continues the
// list in record r + 1).  A pair looks its cell up, scores its list with the
// same fp32 FMA sequence and strict "<" as the exhaustive search, and so
// returns its index.  Pairs outside [-R, R)^2 take the outer grid's record
// (global memory), or scan the whole codebook beyond it.  Indices are packed
// from registers through a byte stage per wavefront.
//
// LDS layout (the kernel's own, staged from the plan's image): the map with a
// guard bin at each end, kLdsMapBytes; the codebook at kLdsMapBytes, 8 bytes
// per centroid (a 64-lane gather of 8-byte entries meets far fewer bank
// conflicts than one of 16-byte entries, whose starting banks are a quarter
// as many); the cells as a (G + 1) x (G + 1) array whose last row and column ("cell G",
// where the guard bins point) say "scan all"; the records; the stages.  A bin
// outside [-R, R), an infinite or a NaN coordinate (the clamp and the
// conversion send NaN to bin 0) lands in a guard bin, so the lookup needs no
// range test.  A plan built for another K points every bin at the guard.
// ---------------------------------------------------------------------------
template <int L, typename Tin>
__global__ __launch_bounds__(kLdsThreads) __attribute__((amdgpu_waves_per_eu(4))) void encode_lds_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ f,
    const float* __restrict__ isig, const float* __restrict__ codebook, int K, int B, int row_words,
    const double* __restrict__ rho, const int* __restrict__ plan_K, const uint4* __restrict__ image, int image_bytes,
    int G, int lists_off, const uint16_t* __restrict__ outer, uint32_t* __restrict__ packed) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBudget];
  const uint8_t* map = reinterpret_cast<const uint8_t*>(lds);
  const char* cbase = lds + kLdsMapBytes;          // codebook: centroid c at byte 8 c
  const int cb_bytes = 8 * K;
  const int cells_lds = kLdsMapBytes + cb_bytes;
  const int lists_lds = cells_lds + (int)lds_cell_bytes(G);
  const int rec_bytes = image_bytes - lists_off;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: window bookkeeping stays scalar
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int total = N * nwin;                      // fits in int (checked on the host)
  const int stride = gridDim.x * kLdsWaves;
  int gw = blockIdx.x * kLdsWaves + wave;
  // the first window's weights are in flight while the tables are staged
  int n = min(gw, total - 1) / nwin, win = min(gw, total - 1) - (min(gw, total - 1) / nwin) * nwin;
  WinLoads<Tin> wl;
  load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
  const bool plan_ok = *plan_K == K;               // a plan built for another K: scan the whole codebook
  {
    // records: verbatim 16-byte chunks of the image
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(image) + lists_off);
    uint4* dst = reinterpret_cast<uint4*>(lds + lists_lds);
    const int nv = rec_bytes / 16;
    constexpr int kU = 8;                          // loads in flight per thread (clamped, always valid)
    for (int i0 = threadIdx.x; i0 < nv; i0 += kU * kLdsThreads) {
      uint4 t[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) t[u] = src[min(i0 + u * kLdsThreads, nv - 1)];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (i0 + u * kLdsThreads < nv) dst[i0 + u * kLdsThreads] = t[u];
    }
    // the cells, 16-byte chunks of the image's G x G array re-strided to
    // G + 1 (element i of the image goes to i + i / G), then the guard row
    // and column; the map one chunk per thread, shifted by the low guard bin
    const uint4* gcells = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(image) + kLdsBins);
    uint16_t* lcells = reinterpret_cast<uint16_t*>(lds + cells_lds);
    const int ncv = (G * G + 7) / 8;
    constexpr int kC = 4;
    for (int i0 = threadIdx.x; i0 < ncv; i0 += kC * kLdsThreads) {
      uint4 t[kC];
#pragma unroll
      for (int u = 0; u < kC; ++u) t[u] = gcells[min(i0 + u * kLdsThreads, ncv - 1)];
#pragma unroll
      for (int u = 0; u < kC; ++u) {
        const int v = i0 + u * kLdsThreads;
        const uint32_t w[4] = {t[u].x, t[u].y, t[u].z, t[u].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = 8 * v + k;
          if (v < ncv && i < G * G) lcells[i + i / G] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
        }
      }
    }
    for (int i = threadIdx.x; i < 2 * G + 1; i += kLdsThreads)
      lcells[i < G + 1 ? i * (G + 1) + G : G * (G + 1) + (i - (G + 1))] = kLdsScanAll;
    uint8_t* lmap = reinterpret_cast<uint8_t*>(lds);
    if (threadIdx.x < kLdsBins / 16) {
      const uint4 m = reinterpret_cast<const uint4*>(image)[threadIdx.x];
      const uint32_t w[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
      for (int k = 0; k < 16; ++k)
        lmap[1 + 16 * threadIdx.x + k] = plan_ok ? (uint8_t)(w[k >> 2] >> (8 * (k & 3))) : (uint8_t)G;
    }
    if (threadIdx.x < 2) lmap[threadIdx.x ? kLdsBins + 1 : 0] = (uint8_t)G;
  }
  for (int c = threadIdx.x; c < K; c += kLdsThreads) {
    const float cx = codebook[2 * c], cy = codebook[2 * c + 1];
    reinterpret_cast<float2*>(lds + kLdsMapBytes)[c] = make_float2(-cx, -cy);
  }
  __syncthreads();
  if (gw >= total) return;                         // no barriers follow
  uint8_t* stage = reinterpret_cast<uint8_t*>(lds + lists_lds + rec_bytes + wave * 64 * B);
  // Twice the score of centroid c at byte h8 = 8 c, from (x2, y2) = 2 z~:
  // fma(y2, -cy, fma(x2, -cx, |c|^2)) with |c|^2 = fma(cx, cx, cy cy).  Every
  // step is exactly twice that of fma(y, -cy, fma(x, -cx, |c|^2 / 2)) (a
  // power-of-two scaling commutes with the rounding), so the scores order
  // and tie exactly as the exhaustive search's.  The codebook holds only
  // (-cx, -cy): 8-byte gathers, half the LDS bytes of (-cx, -cy, |c|^2 / 2).
  auto cand = [&](uint32_t h8) -> float2 {
    return *reinterpret_cast<const float2*>(__builtin_assume_aligned(cbase + h8, 8));
  };
  auto score2c = [](float x2, float y2, float2 c) -> float {
    return __builtin_fmaf(y2, c.y, __builtin_fmaf(x2, c.x, __builtin_fmaf(c.x, c.x, c.y * c.y)));
  };
  auto score2 = [&](float x2, float y2, uint32_t h8) -> float { return score2c(x2, y2, cand(h8)); };
  // record r of an entry 0x8000 | r sits at lists_lds + 8 r = 8 e + (lists_lds - 0x40000)
  const uint32_t rec_bias = (uint32_t)lists_lds - 0x40000u;
  auto record = [&](uint32_t e) -> uint2 {
    return *reinterpret_cast<const uint2*>(__builtin_assume_aligned(lds + ((e << 3) + rec_bias), 8));
  };

  // bin t = x kLdsBins / (2R) + kLdsBins / 2 + 1 (its rounding, < 1e-3 bin,
  // is inside the table's eta margin); bins 0 and kLdsBins + 1 are the guards.
  // The lanes hold 2 z~: the factors below are halved (exactly), so every
  // product is that of z~ with the full factor.
  const float bins_per_unit = 0.5f * ((float)kLdsBins / (2.0f * kPlanR));
  const float bmax = __uint_as_float(__float_as_uint((float)(kLdsBins + 2)) - 1u);   // largest float below kLdsBins + 2
  const float cells_per_unit2 = 0.5f * ((float)kPlanG2 / (2.0f * kPlanR2));
  const float tmax2 = __uint_as_float(__float_as_uint((float)kPlanG2) - 1u);
  const uint32_t gstride = (uint32_t)(G + 1);

  for (;;) {
    const bool active = win * kWinChunks + lane < nchunks;   // whole Hadamard blocks are active or not
    float zx[8], zy[8];                            // 2 z~ (see score2c)
    const int co_local = window_transform<L, Tin, 2>(wl, active, lane, zx, zy);
    const int n_cur = n, win_cur = win;
    const int gnext = gw + stride;
    {
      const int gl = min(gnext, total - 1);
      n = gl / nwin;
      win = gl - n * nwin;
      load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
    }

    uint32_t idx[8];
#pragma unroll
    for (int g = 0; g < 8; g += 4) {
      uint32_t e[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float tx = __builtin_fmaf(zx[g + p], bins_per_unit, 0.5f * kLdsBins + 1.0f);
        const float ty = __builtin_fmaf(zy[g + p], bins_per_unit, 0.5f * kLdsBins + 1.0f);
        const uint32_t ix = map[(int)__builtin_amdgcn_fmed3f(tx, 0.0f, bmax)];
        const uint32_t iy = map[(int)__builtin_amdgcn_fmed3f(ty, 0.0f, bmax)];
        const uint32_t cell = __umul24(ix, gstride) + iy;
        e[p] = *reinterpret_cast<const uint16_t*>(lds + cells_lds + 2u * cell);
      }
      // ---- lists: scan the record's distinct slots in ascending order with a
      // strict "<" (the first of equal scores wins, as in the exhaustive
      // search).  The four pairs' records are read together (other lanes read
      // record 0, unused); a list's repeated tail slots skip the gather (fewer
      // bank conflicts) and the comparison.
      uint32_t boff[4];
      bool wide = false, lst[4], more[4];          // more: the list continues in the next record
      uint2 rr[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        lst[p] = e[p] >= 0x8000u && e[p] != kLdsScanAll;
        wide |= e[p] == kLdsScanAll;
        rr[p] = record(lst[p] ? e[p] : 0x8000u);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        boff[p] = e[p];
        more[p] = lst[p] && (rr[p].y >> 31) != 0u;
        if (lst[p]) {
          // slots as byte offsets 8 c (the record holds 16 c)
          const uint32_t o0 = (rr[p].x & 0xffffu) >> 1, o1 = rr[p].x >> 17, o2 = (rr[p].y & 0xffffu) >> 1,
                         o3 = (rr[p].y >> 17) & 0x3fffu;
          const bool n2 = o2 != o1, n3 = o3 != o2;
          const float x2 = zx[g + p], y2 = zy[g + p];
          // lists of 5..8 (rare per pair, but a group of 256 pairs holds one
          // often): the continuation record is read with the first gathers
          uint2 rc;
          if (more[p]) rc = record(e[p] + 1u);
          const float2 c0 = cand(o0), c1 = cand(o1);
          float2 c2, c3;                           // gathered only where the slot is new
          if (n2) c2 = cand(o2);
          if (n3) c3 = cand(o3);
          const float s0 = score2c(x2, y2, c0), s1 = score2c(x2, y2, c1);
          const float s2 = score2c(x2, y2, c2), s3 = score2c(x2, y2, c3);
          float best = s0;
          uint32_t o = o0;
          if (s1 < best) { best = s1; o = o1; }
          if (n2 && s2 < best) { best = s2; o = o2; }
          if (n3 && s3 < best) { best = s3; o = o3; }
          // its entries all follow the first record's; a list of 5 has one
          // (the others repeat it), longer lists take the other three slots
          if (__any(more[p])) {
            if (more[p]) {
              const uint32_t oc[4] = {(rc.x & 0xffffu) >> 1, rc.x >> 17, (rc.y & 0xffffu) >> 1,
                                      (rc.y >> 17) & 0x3fffu};
              const float sc0 = score2c(x2, y2, cand(oc[0]));
              if (sc0 < best) { best = sc0; o = oc[0]; }
              if (__any(oc[1] != oc[0])) {
                float2 c[3];
#pragma unroll
                for (int i = 0; i < 3; ++i) c[i] = cand(oc[i + 1]);
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                  const float sc = score2c(x2, y2, c[i]);
                  if (sc < best) { best = sc; o = oc[i + 1]; }
                }
              }
            }
          }
          boff[p] = 2u * o;
        }
      }
      // ---- outside the table or a cell without a list: the outer grid's
      // record, else the whole codebook (rare)
      if (__any(wide)) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (!__any(e[p] == kLdsScanAll)) continue;
          const float x2 = zx[g + p], y2 = zy[g + p];
          const float ux = __builtin_fmaf(x2, cells_per_unit2, 0.5f * kPlanG2);
          const float uy = __builtin_fmaf(y2, cells_per_unit2, 0.5f * kPlanG2);
          const float vx = __builtin_amdgcn_fmed3f(ux, 0.0f, tmax2);
          const float vy = __builtin_amdgcn_fmed3f(uy, 0.0f, tmax2);
          // the outer grid is consulted only outside [-R, R)^2, where its
          // records are lists (its cells inside the square say "scan all")
          const bool full = e[p] == kLdsScanAll;
          uint4 rec = make_uint4(1u << 16, 0u, 0u, 0u);
          if (full && plan_ok && vx == ux && vy == uy)
            rec = *reinterpret_cast<const uint4*>(outer + ((int)vx * kPlanG2 + (int)vy) * 8);
          const uint32_t words[4] = {rec.x, rec.y, rec.z, rec.w};
          const bool over = !full || ((words[0] >> 16) & 1u);
          if (full && !over) {
            const int cnt = (int)(words[0] & 15u) + 1;
            float fb = INFINITY;
            uint32_t fo = 0;
            for (int i = 0; i < cnt; ++i) {
              const uint32_t w = words[i >> 1];
              const uint32_t off = ((i & 1) ? (w >> 16) : w) & 0xfff0u;
              const float sc = score2(x2, y2, off >> 1);
              if (sc < fb) { fb = sc; fo = off; }
            }
            boff[p] = fo;
          }
          if (__any(full && over)) {
            float fb = INFINITY;
            uint32_t fo = 0;
            for (int cc = 0; cc < K; ++cc) {
              const float sc = score2(x2, y2, (uint32_t)cc * 8u);   // same address in every lane: broadcast
              if (sc < fb) { fb = sc; fo = (uint32_t)cc * 16u; }
            }
            if (full && over) boff[p] = fo;
          }
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) idx[g + p] = active ? boff[p] >> 4 : 0u;
    }
    stage_lane_bytes(stage, co_local, idx, B);
    wave_lds_fence();
    store_stage(stage, lane, win_cur, B, row_words, packed + (int64_t)n_cur * row_words);
    gw = gnext;
    if (gw >= total) break;
    wave_lds_fence();                              // the stage is rewritten next round
  }
}

// ===========================================================================
// launcher
// ===========================================================================
template <int L>
struct LaunchEncode {
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const float* isig,
                 const float* cb, int K, int B, int row_words, const double* rho, const void* plan, uint32_t* packed,
                 hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    const int64_t waves = (int64_t)N * nwin;
    const dim3 grid((unsigned)((waves + kEncWaves - 1) / kEncWaves)), blk(kEncThreads);
    if (plan) {
      // persistent: as many workgroups as fit at once
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return fail(QAMW_EHIP, "cannot query the device's compute units");
      LdsGeometry g;
      if (lds_geometry(K, &g)) {                 // one 16-wavefront workgroup per CU
        const char* base = (const char*)plan;
        const int* plan_K = (const int*)(base + kPlanHeaderKOffset);
        const uint4* image = (const uint4*)(base + plan_image_offset(K));
        const uint16_t* outer = (const uint16_t*)(base + plan_outer_offset(K));
        const int64_t wgs = (waves + kLdsWaves - 1) / kLdsWaves;
        const dim3 lgrid((unsigned)std::min<int64_t>(wgs, (int64_t)cus)), lblk(kLdsThreads);
        const size_t lds = kLdsMapBytes + (size_t)8 * K + lds_cell_bytes(g.G) + (g.image_bytes - g.lists_off) +
                           (size_t)kLdsWaves * g.stage_bytes;
        if (lds > kLdsBudget) return fail(QAMW_EUNSUPPORTED, "LDS table too large");
        if (wdt == QAMW_F32)
          hipLaunchKernelGGL((encode_lds_kernel<L, float>), lgrid, lblk, 0, st, (const float*)W, ldw, N, d, f, isig,
                             cb, K, B, row_words, rho, plan_K, image, (int)g.image_bytes, g.G, (int)g.lists_off, outer,
                             packed);
        else
          hipLaunchKernelGGL((encode_lds_kernel<L, uint16_t>), lgrid, lblk, 0, st, (const uint16_t*)W, ldw, N, d, f,
                             isig, cb, K, B, row_words, rho, plan_K, image, (int)g.image_bytes, g.G, (int)g.lists_off,
                             outer, packed);
        return check_launch("encode_lds_kernel");
      }
      const dim3 pgrid((unsigned)std::min<int64_t>(grid.x, (int64_t)cus * kPlanWgPerCu));
      const char* base = (const char*)plan;
      const int* plan_K = (const int*)(base + kPlanHeaderKOffset);
      const uint16_t* lists = (const uint16_t*)(base + kPlanHeaderBytes);
      const uint16_t* lists2 = (const uint16_t*)(base + plan_outer_offset(K));
#define QAMW_PLAN_LAUNCH(TIN, KM, LM, PG)                                                                      \
  hipLaunchKernelGGL((encode_plan_kernel<L, TIN, KM, LM, PG>), pgrid, blk, 0, st, (const TIN*)W, ldw, N, d, f, \
                     isig, cb, K, B, row_words, rho, plan_K, lists, lists2, packed)
      if (plan_lmax(K) == 8) {
        if (wdt == QAMW_F32) QAMW_PLAN_LAUNCH(float, 2048, 8, 2); else QAMW_PLAN_LAUNCH(uint16_t, 2048, 8, 2);
      } else {
        if (wdt == QAMW_F32) QAMW_PLAN_LAUNCH(float, 4096, 16, 2); else QAMW_PLAN_LAUNCH(uint16_t, 4096, 16, 2);
      }
#undef QAMW_PLAN_LAUNCH
      return check_launch("encode_plan_kernel");
    }
    const int Kpad = (int)round_up((size_t)K, kTile);
    const size_t lds = (size_t)Kpad * 3 * sizeof(float) + (size_t)kEncWaves * kWinPairs * sizeof(float2);
    if (wdt == QAMW_F32)
      hipLaunchKernelGGL((encode_kernel<L, float>), grid, blk, lds, st, (const float*)W, ldw, N, d, f, isig, cb, K,
                         Kpad, B, row_words, rho, packed);
    else
      hipLaunchKernelGGL((encode_kernel<L, uint16_t>), grid, blk, lds, st, (const uint16_t*)W, ldw, N, d, f, isig,
                         cb, K, Kpad, B, row_words, rho, packed);
    return check_launch("encode_kernel");
  }
};

int launch_encode_prepare(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s,
                          const float* sigma, uint64_t seed, double* rho, uint16_t* rho_f16, float* f, float* isig,
                          hipStream_t st) {
  const int row_blocks = grid_for_waves(N);
  const dim3 grid((unsigned)(row_blocks + (d + kBlockThreads - 1) / kBlockThreads)), blk(kBlockThreads);
  const double sqrt_b = sqrt((double)(1 << L));
  if (wdt == QAMW_F32)
    hipLaunchKernelGGL(encode_prepare_kernel<float>, grid, blk, 0, st, (const float*)W, ldw, N, d, s, sigma, seed,
                       row_blocks, sqrt_b, rho, rho_f16, f, isig);
  else
    hipLaunchKernelGGL(encode_prepare_kernel<uint16_t>, grid, blk, 0, st, (const uint16_t*)W, ldw, N, d, s, sigma,
                       seed, row_blocks, sqrt_b, rho, rho_f16, f, isig);
  return check_launch("encode_prepare_kernel");
}

int launch_encode(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const float* isig,
                  const float* cb, int K, int B, int row_words, const double* rho, const void* plan, uint32_t* packed,
                  hipStream_t st) {
  return dispatch_L<LaunchEncode>(L, W, wdt, N, d, ldw, f, isig, cb, K, B, row_words, rho, plan, packed, st);
}


}  // namespace qamw
