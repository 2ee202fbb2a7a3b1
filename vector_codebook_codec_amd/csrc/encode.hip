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
    const float* __restrict__ sigma, uint64_t seed, int row_blocks, double* __restrict__ rho,
    uint16_t* __restrict__ rho_f16, float* __restrict__ f, float* __restrict__ isig) {
  if ((int)blockIdx.x < row_blocks) {
    const int n = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (n < N) row_norm_wave(W, ldw, n, d, s, rho, rho_f16);
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

  // Software pipeline: the MFMA of column block ps runs while the VALU folds
  // the scores of block ps - 1 (two accumulator sets); the next tile's A and C
  // operands are loaded during the current tile.
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
  float aop = abase[0];
  f32x16 cop;
  load_c(0, cop);
  for (int c0 = 0; c0 < Kpad; c0 += kTile) {
    const int cn = (c0 + kTile < Kpad) ? c0 + kTile : c0;
    const float anext = abase[cn];
    f32x16 cnext;
    load_c(cn, cnext);
    f32x16 dprev = __builtin_amdgcn_mfma_f32_32x32x2f32(aop, bop[0], cop, 0, 0, 0);
#pragma unroll
    for (int ps = 1; ps < kPairSets; ++ps) {
      const f32x16 dcur = __builtin_amdgcn_mfma_f32_32x32x2f32(aop, bop[ps], cop, 0, 0, 0);
      fold(dprev, ps - 1, c0);
      dprev = dcur;
    }
    fold(dprev, kPairSets - 1, c0);
    aop = anext;
    cop = cnext;
  }

  // ---- combine the half-waves: smaller minimum, then earlier tile
#pragma unroll
  for (int ps = 0; ps < kPairSets; ++ps) {
    const float ob = __shfl_xor(best[ps], 32);
    const int ot = __shfl_xor(tile_of_best[ps], 32);
    if (ob < best[ps] || (ob == best[ps] && ot < tile_of_best[ps])) { best[ps] = ob; tile_of_best[ps] = ot; }
  }

  // ---- lowest index: rescan the tile; lane handles column blocks 2m + half
  uint32_t idxv[kPairSets / 2];
#pragma unroll
  for (int m2 = 0; m2 < kPairSets / 2; ++m2) {
    const float bb = half ? best[2 * m2 + 1] : best[2 * m2];
    const int t0 = half ? tile_of_best[2 * m2 + 1] : tile_of_best[2 * m2];
    const float2 z = zbuf[(2 * m2 + half) * 32 + jcol];
    // lane-rotated order keeps the lanes on different LDS banks (tiles start
    // on multiples of 32 entries); the smallest matching index wins
    int id = INT_MAX;
    for (int cc = 0; cc < kTile; ++cc) {
      const int ci = t0 + ((cc + lane) & (kTile - 1));
      const float sc = __builtin_fmaf(z.y, cby[ci], __builtin_fmaf(z.x, cbx[ci], cbh[ci]));
      id = (sc == bb) ? min(id, ci) : id;
    }
    idxv[m2] = (uint32_t)min(id, K - 1);
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
// The codebook sits in LDS as (-cx, -cy, |c|^2/2, 0) per centroid, one
// ds_read_b128 per candidate at the byte offset the list stores.  A lane's
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
  __shared__ float4 cb4[KMAX];                                      // (-cx, -cy, |c|^2/2, 0)
  __shared__ uint16_t stage_all[kEncWaves * kWinPairs];             // 8 waves x 512 indices
  const char* cbytes = reinterpret_cast<const char*>(cb4);

  for (int c = threadIdx.x; c < K; c += kEncThreads) {
    const float cx = codebook[2 * c], cy = codebook[2 * c + 1];
    cb4[c] = make_float4(-cx, -cy, 0.5f * __builtin_fmaf(cx, cx, cy * cy), 0.0f);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
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

  const float cells_per_unit = (float)kPlanG / (2.0f * kPlanR);
  const float cells_per_unit2 = (float)kPlanG2 / (2.0f * kPlanR2);
  const float tmax = __uint_as_float(__float_as_uint((float)kPlanG) - 1u);     // largest float below G
  const float tmax2 = __uint_as_float(__float_as_uint((float)kPlanG2) - 1u);
  const bool plan_ok = *plan_K == K;   // a plan built for another K: scan the whole codebook

  for (;;) {
    const bool active = win * kWinChunks + lane < nchunks;   // whole Hadamard blocks are active or not
    float zx[8], zy[8];
    const int co_local = window_transform<L>(wl, active, lane, zx, zy);
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
        const uint4* lp = reinterpret_cast<const uint4*>(rec);
#pragma unroll
        for (int q = 0; q < LMAX / 8; ++q) {
          const uint4 t = lp[q];
          words[p][4 * q + 0] = t.x; words[p][4 * q + 1] = t.y; words[p][4 * q + 2] = t.z; words[p][4 * q + 3] = t.w;
        }
      }
      // ---- record flags: nibble 0 = count - 1, nibble 1 = overflow
      bool full[PG];
      int maxc = 1;
#pragma unroll
      for (int p = 0; p < PG; ++p) {
        const uint32_t w0 = words[p][0];
        full[p] = !inside[p] || ((w0 >> 16) & 1u);
        maxc = max(maxc, full[p] ? 1 : (int)(w0 & 15u) + 1);
        words[p][0] = w0 & 0xfff0fff0u;
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
          uint32_t off[PG];
          float3 e[PG];
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            off[p] = h ? (words[p][w] >> 16) : (words[p][w] & 0xffffu);
            const float4 t = *reinterpret_cast<const float4*>(cbytes + off[p]);
            e[p] = make_float3(t.x, t.y, t.z);
          }
          __builtin_amdgcn_sched_barrier(0);   // keep the group's LDS reads in flight together
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            const float sc = __builtin_fmaf(zy[g + p], e[p].y, __builtin_fmaf(zx[g + p], e[p].x, e[p].z));
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
            const float4 e = cb4[cc];                // same address in every lane: broadcast
            const float sc = __builtin_fmaf(zy[g + p], e.y, __builtin_fmaf(zx[g + p], e.x, e.z));
            if (sc < fb) { fb = sc; fo = (uint32_t)cc * 16u; }
          }
          if (full[p]) boff[p] = fo;
        }
        stage[co_local * kPairsPerLane + g + p] = (uint16_t)(boff[p] >> 4);
      }
    }
    wave_lds_fence();
    pack_window(stage, lane, win_cur, nwin, d >> 1, B, row_words, packed + (int64_t)n_cur * row_words);
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
      // persistent: as many workgroups as fit at once (2 of 8 wavefronts per CU)
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return fail(QAMW_EHIP, "cannot query the device's compute units");
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

int launch_encode_prepare(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, const float* sigma,
                          uint64_t seed, double* rho, uint16_t* rho_f16, float* f, float* isig, hipStream_t st) {
  const int row_blocks = grid_for_waves(N);
  const dim3 grid((unsigned)(row_blocks + (d + kBlockThreads - 1) / kBlockThreads)), blk(kBlockThreads);
  if (wdt == QAMW_F32)
    hipLaunchKernelGGL(encode_prepare_kernel<float>, grid, blk, 0, st, (const float*)W, ldw, N, d, s, sigma, seed,
                       row_blocks, rho, rho_f16, f, isig);
  else
    hipLaunchKernelGGL(encode_prepare_kernel<uint16_t>, grid, blk, 0, st, (const uint16_t*)W, ldw, N, d, s, sigma,
                       seed, row_blocks, rho, rho_f16, f, isig);
  return check_launch("encode_prepare_kernel");
}

int launch_encode(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const float* isig,
                  const float* cb, int K, int B, int row_words, const double* rho, const void* plan, uint32_t* packed,
                  hipStream_t st) {
  return dispatch_L<LaunchEncode>(L, W, wdt, N, d, ldw, f, isig, cb, K, B, row_words, rho, plan, packed, st);
}


}  // namespace qamw
