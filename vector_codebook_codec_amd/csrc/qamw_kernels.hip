// QAM-W codec kernels for gfx950 and the C ABI declared in include/qamw.h.
//
// Method: "QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling" (cited as "QAM-W, <section>").
//
// Kernels (one wavefront = one 1024-column window of one or more rows):
//   scale_kernel        s_j = r_j ^ alpha                       (Activation-Aware Scaling)
//   rownorm_kernel      rho_n = ||W_n diag(s)||_2 in fp64        (Separation of Scale and Direction)
//   amplitude_kernel    per row tile: sum_n |z_{n,k}| over the   (Pairing and Calibration)
//                       tile's rows, z from the rotated unit row
//   sigma_kernel        sigma_k = sum over tiles / (N sqrt(pi/2)), fixed order, fp64
//   encode_kernel       rotate, normalise by rho sigma, nearest  (Joint 2D Quantization)
//                       centroid with the codebook in LDS, pack
//   decode_kernel       unpack, centroid * sigma, inverse        (Decoding)
//                       rotation, * rho_hat / s, convert, store
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <string.h>

#include <cstdio>
#include <string>

#include "qamw.h"
#include "qamw_device.h"

namespace qamw {

constexpr int kBlockThreads = 256;                   // 4 wavefronts per workgroup
constexpr int kWavesPerBlock = kBlockThreads / kWave;
constexpr int kCalibRowsPerTile = 16;                // rows per amplitude partial sum

// Decode tunables: rows whose packed words are loaded ahead, and wavefronts
// of work per CU the launch aims for (each wave then walks several rows).
#ifndef QAMW_DECODE_PREFETCH
#define QAMW_DECODE_PREFETCH 4
#endif
#ifndef QAMW_DECODE_WAVES_PER_CU
#define QAMW_DECODE_WAVES_PER_CU 16
#endif
constexpr int kDecodePrefetch = QAMW_DECODE_PREFETCH;

// ---------------------------------------------------------------------------
// s_j = r_j ^ alpha.  alpha = 0 gives exactly 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlockThreads) void scale_kernel(const float* __restrict__ r, float alpha,
                                                              int d, float* __restrict__ s) {
  const int j = blockIdx.x * kBlockThreads + threadIdx.x;
  if (j < d) s[j] = (alpha == 0.0f) ? 1.0f : powf(r[j], alpha);
}

// ---------------------------------------------------------------------------
// rho_n = sqrt(sum_j (W_nj s_j)^2), one wavefront per row.  W_nj s_j is exact
// in fp64 (24-bit x 24-bit significands); squares and sums are fp64, reduced
// in a fixed order, so rho is deterministic and accurate to ~1e-16.
// Optionally writes the binary16 (RNE) row norm.
// ---------------------------------------------------------------------------
template <typename Tin>
__global__ __launch_bounds__(kBlockThreads) void rownorm_kernel(const Tin* __restrict__ W, int64_t ldw,
                                                                int N, int d, const float* __restrict__ s,
                                                                double* __restrict__ rho,
                                                                uint16_t* __restrict__ rho_f16) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (n >= N) return;
  const int nchunks = d >> 4;
  const Tin* row = W + (int64_t)n * ldw;
  double acc = 0.0;
  for (int c = lane; c < nchunks; c += kWave) {
    float x[16];
    load_chunk(row + c * kChunk, x);
    const float4* sp = reinterpret_cast<const float4*>(s + c * kChunk);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 sv = sp[v];
      const float sc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double w = (double)x[4 * v + i] * (double)sc[i];
        acc = fma(w, w, acc);
      }
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    const double r = sqrt(acc);
    rho[n] = r;
    if (rho_f16) rho_f16[n] = f64_to_f16_bits(r);
  }
}

// Per-lane column factors f_j = s_j * eps_j for the lane's 16 columns.
__device__ __forceinline__ void column_scale(const float* __restrict__ s, uint64_t seed, int col0,
                                             float f[16]) {
  const float4* sp = reinterpret_cast<const float4*>(s + col0);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float4 sv = sp[v];
    f[4 * v + 0] = sv.x * sign_eps(seed, col0 + 4 * v + 0);
    f[4 * v + 1] = sv.y * sign_eps(seed, col0 + 4 * v + 1);
    f[4 * v + 2] = sv.z * sign_eps(seed, col0 + 4 * v + 2);
    f[4 * v + 3] = sv.w * sign_eps(seed, col0 + 4 * v + 3);
  }
}

// 1 / (sqrt(b) rho sigma) in fp64, rounded once to fp32; 0 when rho sigma == 0.
__device__ __forceinline__ float pair_normaliser(double rho, float sigma, double sqrt_b) {
  const double den = rho * (double)sigma * sqrt_b;
  return den > 0.0 ? (float)(1.0 / den) : 0.0f;
}

// ---------------------------------------------------------------------------
// Calibration, pass 2: per (window, row tile) wavefront, accumulate the pair
// amplitudes |z_{n,k}| of the normalised rotated rows over the tile.
// partial[t][k] = sum_{n in tile t} hypot(y_{n,2k}, y_{n,2k+1}) / (sqrt(b) rho_n)
// ---------------------------------------------------------------------------
template <int L, typename Tin>
__global__ __launch_bounds__(kBlockThreads) void amplitude_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ s, uint64_t seed,
    const double* __restrict__ rho, float* __restrict__ partial) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int ntiles = (N + kCalibRowsPerTile - 1) / kCalibRowsPerTile;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= nwin * ntiles) return;
  const int win = gw % nwin;
  const int tile = gw / nwin;
  const int c = win * kWinChunks + lane;
  const bool active = c < nchunks;   // whole Hadamard blocks are active or not
  const int co = win * kWinChunks + BlockOut<L>::chunk(lane);
  const double sqrt_b = sqrt((double)(1 << L));

  float f[16];
  if (active) column_scale(s, seed, c * kChunk, f);
  float acc[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) acc[p] = 0.0f;

  const int n0 = tile * kCalibRowsPerTile;
  const int n1 = min(N, n0 + kCalibRowsPerTile);
  // 1 / (sqrt(b) rho_n) of the tile's rows, one per lane
  float inv_lane = 0.0f;
  if (lane < n1 - n0) {
    const double r = rho[n0 + lane];
    inv_lane = r > 0.0 ? (float)(1.0 / (sqrt_b * r)) : 0.0f;
  }
  float nxt[16];
  if (active) load_chunk(W + (int64_t)n0 * ldw + c * kChunk, nxt);
  for (int n = n0; n < n1; ++n) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = active ? nxt[i] * f[i] : 0.0f;
    if (active && n + 1 < n1) load_chunk(W + (int64_t)(n + 1) * ldw + c * kChunk, nxt);
    fwht_block<L>(x, lane);
    const float inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv_lane), n - n0));
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float a = x[2 * p], b = x[2 * p + 1];
      acc[p] += sqrtf(__builtin_fmaf(a, a, b * b)) * inv;
    }
  }
  if (active) {
    float4* out = reinterpret_cast<float4*>(partial + (int64_t)tile * (d >> 1) + co * kPairsPerLane);
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// sigma_k = (sum over tiles, fp64, fixed order) / (N sqrt(pi/2)).  A
// workgroup owns 16 columns; thread (column, slice) sums tiles slice,
// slice + 16, ... and the 16 slice sums are then added in slice order.
constexpr int kSigmaSlices = 16;
__global__ __launch_bounds__(kBlockThreads) void sigma_kernel(const float* __restrict__ partial, int ntiles,
                                                              int half_d, int N, float* __restrict__ sigma) {
  __shared__ double part[kSigmaSlices][kBlockThreads / kSigmaSlices];
  const int col_in = threadIdx.x % (kBlockThreads / kSigmaSlices);
  const int slice = threadIdx.x / (kBlockThreads / kSigmaSlices);
  const int k = blockIdx.x * (kBlockThreads / kSigmaSlices) + col_in;
  double acc = 0.0;
  if (k < half_d)
    for (int t = slice; t < ntiles; t += kSigmaSlices) acc += (double)partial[(int64_t)t * half_d + k];
  part[slice][col_in] = acc;
  __syncthreads();
  if (slice == 0 && k < half_d) {
    double tot = 0.0;
#pragma unroll
    for (int q = 0; q < kSigmaSlices; ++q) tot += part[q][col_in];
    sigma[k] = (float)(tot / ((double)N * 1.2533141373155002512078826));  // sqrt(pi/2)
  }
}

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
// rescanned on the VALU to find the first centroid whose score equals the
// minimum: exact ties go to the lowest index.
// ---------------------------------------------------------------------------
constexpr int kEncThreads = 512;                       // 8 wavefronts per workgroup
constexpr int kEncWaves = kEncThreads / kWave;
constexpr int kTile = 32;                              // centroids per MFMA tile
constexpr int kPairSets = kWinPairs / 32;              // 16 MFMA columns blocks per window

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int L, typename Tin>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ s,
    const float* __restrict__ sigma, uint64_t seed, const float* __restrict__ codebook, int K, int Kpad,
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
  const int c = win * kWinChunks + lane;
  const bool active = c < nchunks;

  // ---- rotate the lane's 16 columns: x = H_b (eps . s . w) (unnormalised)
  float x[16];
  if (active) {
    float f[16];
    column_scale(s, seed, c * kChunk, f);
    load_chunk(W + (int64_t)n * ldw + c * kChunk, x);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] *= f[i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.0f;
  }
  fwht_block<L>(x, lane);
  const int co_local = BlockOut<L>::chunk(lane);   // the lane now holds (sign *) chunk co_local
  const int co = win * kWinChunks + co_local;

  // ---- z~ = y / sigma_k with y = x / (sqrt(b) rho), into the wave's LDS buffer
  {
    const double r = rho[n];
    const double sqrt_b = sqrt((double)(1 << L));
    const float osign = BlockOut<L>::sign(lane);
    float sg[8];
    if (active) {
      const float4* sp = reinterpret_cast<const float4*>(sigma + co * kPairsPerLane);
      const float4 s0 = sp[0], s1 = sp[1];
      sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
      sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) sg[p] = 0.0f;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float inv = pair_normaliser(r, sg[p], sqrt_b) * osign;
      zbuf[co_local * kPairsPerLane + p] = make_float2(x[2 * p] * inv, x[2 * p + 1] * inv);
    }
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
    int id = t0;
    for (int cc = kTile - 1; cc >= 0; --cc) {
      const int ci = t0 + cc;
      const float sc = __builtin_fmaf(z.y, cby[ci], __builtin_fmaf(z.x, cbx[ci], cbh[ci]));
      id = (sc == bb) ? ci : id;
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
  const int half_d = d >> 1;
  const int npairs = min(kWinPairs, half_d - win * kWinPairs);
  const int word0 = win * 16 * B;
  const int nwords = (win == nwin - 1) ? row_words - word0 : 16 * B;
  uint32_t* out = packed + (int64_t)n * row_words + word0;
  for (int q = lane; q < nwords; q += kWave) {
    const int bit0 = q * 32;
    const int k0 = bit0 / B;
    const int k1 = min((bit0 + 31) / B, npairs - 1);
    uint32_t word = 0;
    for (int k = k0; k <= k1; ++k) {
      const int off = k * B - bit0;
      const uint32_t v = stage[k];
      word |= (off >= 0) ? (v << off) : (v >> (-off));
    }
    out[q] = word;
  }
}

// ---------------------------------------------------------------------------
// Decode.  Each workgroup keeps one 1024-column window and walks rows with a
// stride (row n goes to workgroup (n / 4) mod blocks_per_window of its
// window, wave n mod 4), so the codebook (K x float2) and the window's column
// factors g_j = eps_j / (sqrt(b) s_j) are staged in LDS once per workgroup,
// with all prologue loads in flight together.  Each lane keeps its 8 sigma_k
// and 16 factors in registers, holds the row norms of 64 rows at a time (one
// per lane), and prefetches the packed words of the next rows while it
// decodes the current one.  BT > 0 fixes the index width at compile time
// (BT = 0: width B from the argument).
// ---------------------------------------------------------------------------
template <int BT>
__device__ __forceinline__ void unpack8(const uint32_t w[4], uint32_t sh, int Bdyn, uint32_t idx[8]) {
  const int B = BT ? BT : Bdyn;
  const uint32_t mask = (1u << B) - 1u;
  // the lane's 8*B bits, starting at bit 0 of a[0]
  const uint32_t a[3] = {__builtin_amdgcn_alignbit(w[1], w[0], sh), __builtin_amdgcn_alignbit(w[2], w[1], sh),
                         __builtin_amdgcn_alignbit(w[3], w[2], sh)};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int o = p * B;
    const int q = o >> 5;
    const uint32_t lo = (q == 0) ? a[0] : ((q == 1) ? a[1] : a[2]);
    const uint32_t hi = (q == 0) ? a[1] : ((q == 1) ? a[2] : 0u);
    idx[p] = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(o & 31)) & mask;
  }
}

template <int L, int BT, typename Out>
__global__ __launch_bounds__(kBlockThreads) void decode_kernel(
    const uint32_t* __restrict__ packed, const uint16_t* __restrict__ rho_f16, int N, int d,
    const float* __restrict__ s, const float* __restrict__ sigma, uint64_t seed,
    const float* __restrict__ codebook, int K, int Bdyn, int row_words, int blocks_per_window,
    typename Out::T* __restrict__ out, int64_t ldo) {
  extern __shared__ float4 lds4[];
  uint4* stage_all = reinterpret_cast<uint4*>(lds4);    // 4 waves x 256 x 16 bytes
  float* gwin = reinterpret_cast<float*>(stage_all + kWavesPerBlock * 256);  // kWinChunks * kChunk factors
  float2* cb = reinterpret_cast<float2*>(gwin + kWinChunks * kChunk);

  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int win = blockIdx.x % nwin;
  const int rblk = blockIdx.x / nwin;               // 0 .. blocks_per_window-1
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int c = win * kWinChunks + lane;
  // Lanes past the row end hold zeros but stay: the window store reads back
  // columns for every lane of the wave.
  const bool active = c < nchunks;
  // rows of this wave: n = first + k * stride, k = 0 .. nrows-1
  const int first = rblk * kWavesPerBlock + wave;
  const int stride = blocks_per_window * kWavesPerBlock;
  const int nrows = first < N ? (N - first + stride - 1) / stride : 0;

  // ---- the first rows' loads go out before the LDS prologue, so their
  // latency overlaps it
  const int B = BT ? BT : Bdyn;
  const int64_t bitstart = (int64_t)c * kPairsPerLane * B;
  const int wstart = (int)(bitstart >> 5);
  const uint32_t sh = (uint32_t)(bitstart & 31);
  int widx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) widx[i] = min(wstart + i, row_words - 1);
  uint32_t ring[kDecodePrefetch][4];   // packed words of the next rows, in flight
#pragma unroll
  for (int q = 0; q < kDecodePrefetch; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ring[q][i] = 0u;
    if (active && q < nrows) {
      const uint32_t* rw = packed + (int64_t)(first + q * stride) * row_words;
#pragma unroll
      for (int i = 0; i < 4; ++i) ring[q][i] = rw[widx[i]];
    }
  }
  float rh_lane = (lane < nrows) ? f16_bits_to_f32(rho_f16[first + lane * stride]) : 0.0f;  // 64 rows at a time
  float sg[8];
  if (active) {
    const float4* sp = reinterpret_cast<const float4*>(sigma + c * kPairsPerLane);
    const float4 s0 = sp[0], s1 = sp[1];
    sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
    sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
  } else {
#pragma unroll
    for (int p = 0; p < 8; ++p) sg[p] = 0.0f;
  }

  // ---- LDS prologue: codebook and the window's column factors
  {
    const float4* cb4 = reinterpret_cast<const float4*>(codebook);   // two centroids per float4
    float4* cbl = reinterpret_cast<float4*>(cb);
    const int npairs4 = K >> 1;
#pragma unroll 8
    for (int cc = threadIdx.x; cc < npairs4; cc += kBlockThreads) cbl[cc] = cb4[cc];
    if ((K & 1) && threadIdx.x == 0) cb[K - 1] = make_float2(codebook[2 * (K - 1)], codebook[2 * (K - 1) + 1]);
    const float inv_sqrt_b = (float)(1.0 / sqrt((double)(1 << L)));
    constexpr int kPer = kWinChunks * kChunk / kBlockThreads;   // 4
    float sv[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int j = win * kWinChunks * kChunk + q * kBlockThreads + threadIdx.x;
      sv[q] = (j < d) ? (s ? s[j] : 1.0f) : 1.0f;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int t = q * kBlockThreads + threadIdx.x;
      const int j = win * kWinChunks * kChunk + t;
      gwin[t] = (j < d) ? sign_eps(seed, j) * (inv_sqrt_b / sv[q]) : 0.0f;
    }
  }
  __syncthreads();
  if (nrows == 0) return;                          // no barriers follow

  uint4* stage = stage_all + wave * 256;
  const int valid_cols = d - win * kWinChunks * kChunk;
  const int co_local = BlockOut<L>::chunk(lane);
  float g[16];
  {
    const float osign = BlockOut<L>::sign(lane);
    const float4* gp = reinterpret_cast<const float4*>(gwin + co_local * kChunk);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 t = gp[v];
      g[4 * v + 0] = t.x * osign; g[4 * v + 1] = t.y * osign;
      g[4 * v + 2] = t.z * osign; g[4 * v + 3] = t.w * osign;
    }
  }

  for (int k = 0; k < nrows; ++k) {
    if (k > 0 && (k & (kWave - 1)) == 0) {
      const int kk = k + lane;
      rh_lane = (kk < nrows) ? f16_bits_to_f32(rho_f16[first + kk * stride]) : 0.0f;
    }
    const int n = first + k * stride;
    uint32_t w[4] = {ring[0][0], ring[0][1], ring[0][2], ring[0][3]};
#pragma unroll
    for (int q = 0; q + 1 < kDecodePrefetch; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) ring[q][i] = ring[q + 1][i];
    if (active && k + kDecodePrefetch < nrows) {
      const uint32_t* rw = packed + (int64_t)(n + kDecodePrefetch * stride) * row_words;
#pragma unroll
      for (int i = 0; i < 4; ++i) ring[kDecodePrefetch - 1][i] = rw[widx[i]];
    }
    uint32_t idx[8];
    unpack8<BT>(w, sh, Bdyn, idx);
    float x[16];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float2 cc = cb[min((int)idx[p], K - 1)];
      x[2 * p] = cc.x * sg[p];
      x[2 * p + 1] = cc.y * sg[p];
    }
    fwht_block<L>(x, lane);
    const float rh =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rh_lane), k & (kWave - 1)));
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (x[i] * rh) * g[i];
    Out::store(stage, lane, co_local, x, out + (int64_t)n * ldo + win * kWinChunks * kChunk, valid_cols);
  }
}

// ===========================================================================
// host side
// ===========================================================================
thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QAMW_EHIP, "%s: %s", what, hipGetErrorString(e));
  return QAMW_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int log2_exact(int64_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

int check_matrix(int64_t N, int64_t d, int32_t block, int* L) {
  if (N <= 0 || d <= 0) return fail(QAMW_EINVAL, "N and d must be positive (N=%lld d=%lld)", (long long)N, (long long)d);
  // every wavefront index (rows x 1024-column windows) must fit in an int
  if (N > kMaxDim || d > kMaxDim || N * ((d + 1023) / 1024) > (int64_t(1) << 30))
    return fail(QAMW_EUNSUPPORTED, "matrix too large");
  *L = log2_exact(block);
  if (*L < 4 || *L > 10) return fail(QAMW_EUNSUPPORTED, "block must be a power of two in [16, 1024] (got %d)", block);
  if (d % block) return fail(QAMW_EINVAL, "d=%lld is not a multiple of block=%d", (long long)d, block);
  return QAMW_OK;
}

int elem_size(int32_t dt) { return dt == QAMW_F32 ? 4 : (dt == QAMW_BF16 || dt == QAMW_F16) ? 2 : 0; }

size_t calib_tiles(int64_t N) { return (size_t)((N + kCalibRowsPerTile - 1) / kCalibRowsPerTile); }

template <template <int> class Launch, typename... A>
int dispatch_L(int L, A&&... args) {
  switch (L) {
    case 4: return Launch<4>::run(args...);
    case 5: return Launch<5>::run(args...);
    case 6: return Launch<6>::run(args...);
    case 7: return Launch<7>::run(args...);
    case 8: return Launch<8>::run(args...);
    case 9: return Launch<9>::run(args...);
    case 10: return Launch<10>::run(args...);
    default: return fail(QAMW_EUNSUPPORTED, "block size");
  }
}

unsigned grid_for_waves(int64_t waves) { return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

template <int L>
struct LaunchAmplitude {
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, uint64_t seed,
                 const double* rho, float* partial, hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    const int64_t waves = (int64_t)nwin * (int64_t)calib_tiles(N);
    if (wdt == QAMW_F32)
      hipLaunchKernelGGL((amplitude_kernel<L, float>), dim3(grid_for_waves(waves)), dim3(kBlockThreads), 0, st,
                         (const float*)W, ldw, N, d, s, seed, rho, partial);
    else
      hipLaunchKernelGGL((amplitude_kernel<L, uint16_t>), dim3(grid_for_waves(waves)), dim3(kBlockThreads), 0,
                         st, (const uint16_t*)W, ldw, N, d, s, seed, rho, partial);
    return check_launch("amplitude_kernel");
  }
};

template <int L>
struct LaunchEncode {
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, const float* sigma,
                 uint64_t seed, const float* cb, int K, int B, int row_words, const double* rho,
                 uint32_t* packed, hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    const int64_t waves = (int64_t)N * nwin;
    const int Kpad = (int)round_up((size_t)K, kTile);
    const size_t lds = (size_t)Kpad * 3 * sizeof(float) + (size_t)kEncWaves * kWinPairs * sizeof(float2);
    const dim3 grid((unsigned)((waves + kEncWaves - 1) / kEncWaves)), blk(kEncThreads);
    if (wdt == QAMW_F32)
      hipLaunchKernelGGL((encode_kernel<L, float>), grid, blk, lds, st, (const float*)W, ldw, N, d, s, sigma, seed,
                         cb, K, Kpad, B, row_words, rho, packed);
    else
      hipLaunchKernelGGL((encode_kernel<L, uint16_t>), grid, blk, lds, st, (const uint16_t*)W, ldw, N, d, s, sigma,
                         seed, cb, K, Kpad, B, row_words, rho, packed);
    return check_launch("encode_kernel");
  }
};

template <int L, int BT>
int launch_decode_bt(const uint32_t* packed, const uint16_t* rho_f16, int N, int d, const float* s,
                     const float* sigma, uint64_t seed, const float* cb, int K, int B, int row_words, void* out,
                     int32_t odt, int64_t ldo, hipStream_t st) {
  const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
  // Persistent-style grid: every workgroup keeps one window (codebook and
  // column factors loaded once) and walks rows with a stride; about
  // QAMW_DECODE_WAVES_PER_CU / 4 workgroups per CU in total.
  const int64_t target_blocks = 256 * QAMW_DECODE_WAVES_PER_CU / kWavesPerBlock;
  int64_t bpw = target_blocks / nwin;
  const int64_t need = (N + kWavesPerBlock - 1) / kWavesPerBlock;   // one row per wave at most
  bpw = bpw < 1 ? 1 : (bpw > need ? need : bpw);
  const int blocks_per_window = (int)bpw;
  const int64_t blocks = (int64_t)nwin * blocks_per_window;
  const size_t lds = (size_t)kWavesPerBlock * 256 * 16 + (size_t)kWinChunks * kChunk * sizeof(float) +
                     (size_t)K * sizeof(float2);
  const dim3 grid((unsigned)blocks), blk(kBlockThreads);
  if (odt == QAMW_F32)
    hipLaunchKernelGGL((decode_kernel<L, BT, StageF32>), grid, blk, lds, st, packed, rho_f16, N, d, s, sigma, seed,
                       cb, K, B, row_words, blocks_per_window, (float*)out, ldo);
  else if (odt == QAMW_BF16)
    hipLaunchKernelGGL((decode_kernel<L, BT, StageBF16>), grid, blk, lds, st, packed, rho_f16, N, d, s, sigma,
                       seed, cb, K, B, row_words, blocks_per_window, (uint16_t*)out, ldo);
  else
    hipLaunchKernelGGL((decode_kernel<L, BT, StageF16>), grid, blk, lds, st, packed, rho_f16, N, d, s, sigma, seed,
                       cb, K, B, row_words, blocks_per_window, (uint16_t*)out, ldo);
  return check_launch("decode_kernel");
}

template <int L>
struct LaunchDecode {
  static int run(const uint32_t* packed, const uint16_t* rho_f16, int N, int d, const float* s, const float* sigma,
                 uint64_t seed, const float* cb, int K, int B, int row_words, void* out, int32_t odt, int64_t ldo,
                 hipStream_t st) {
    // compile-time index widths for the common rates (K = 256, 1024, 2048, 4096)
    if constexpr (L == 7 || L == 8) {
      switch (B) {
        case 8: return launch_decode_bt<L, 8>(packed, rho_f16, N, d, s, sigma, seed, cb, K, B, row_words, out, odt, ldo, st);
        case 10: return launch_decode_bt<L, 10>(packed, rho_f16, N, d, s, sigma, seed, cb, K, B, row_words, out, odt, ldo, st);
        case 11: return launch_decode_bt<L, 11>(packed, rho_f16, N, d, s, sigma, seed, cb, K, B, row_words, out, odt, ldo, st);
        case 12: return launch_decode_bt<L, 12>(packed, rho_f16, N, d, s, sigma, seed, cb, K, B, row_words, out, odt, ldo, st);
        default: break;
      }
    }
    return launch_decode_bt<L, 0>(packed, rho_f16, N, d, s, sigma, seed, cb, K, B, row_words, out, odt, ldo, st);
  }
};

int launch_rownorm(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, double* rho,
                   uint16_t* rho_f16, hipStream_t st) {
  const dim3 grid(grid_for_waves(N)), blk(kBlockThreads);
  if (wdt == QAMW_F32)
    hipLaunchKernelGGL(rownorm_kernel<float>, grid, blk, 0, st, (const float*)W, ldw, N, d, s, rho, rho_f16);
  else
    hipLaunchKernelGGL(rownorm_kernel<uint16_t>, grid, blk, 0, st, (const uint16_t*)W, ldw, N, d, s, rho, rho_f16);
  return check_launch("rownorm_kernel");
}

int check_weights(const void* W, int32_t wdt, int64_t d, int64_t ldw) {
  if (!W) return fail(QAMW_EINVAL, "W is NULL");
  if (wdt != QAMW_F32 && wdt != QAMW_BF16) return fail(QAMW_EUNSUPPORTED, "weight dtype %d not supported", wdt);
  if (ldw < d) return fail(QAMW_EINVAL, "ldw=%lld < d=%lld", (long long)ldw, (long long)d);
  if (!aligned16(W) || (ldw * elem_size(wdt)) % 16)
    return fail(QAMW_EINVAL, "W must be 16-byte aligned with 16-byte aligned rows");
  return QAMW_OK;
}

int check_codebook(const float* cb, int32_t K) {
  if (!cb) return fail(QAMW_EINVAL, "codebook is NULL");
  if (!aligned16(cb)) return fail(QAMW_EINVAL, "codebook must be 16-byte aligned");
  if (K < 2 || K > 4096) return fail(QAMW_EUNSUPPORTED, "K=%d outside [2, 4096]", K);
  return QAMW_OK;
}

}  // namespace qamw

// ===========================================================================
// C ABI
// ===========================================================================
using namespace qamw;

extern "C" {

int32_t qamw_index_bits(int32_t K) {
  if (K < 2 || K > 4096) return -1;
  int32_t b = 0;
  while ((1 << b) < K) ++b;
  return b;
}

int64_t qamw_packed_row_words(int64_t d, int32_t K) {
  const int32_t B = qamw_index_bits(K);
  if (B < 0 || d <= 0 || (d & 1) || d > kMaxDim) return -1;
  const int64_t words = ((d / 2) * B + 31) / 32;
  return (words + 3) / 4 * 4;
}

size_t qamw_calibrate_workspace_bytes(int64_t N, int64_t d, int32_t block) {
  (void)block;
  if (N <= 0 || d <= 0 || N > kMaxDim || d > kMaxDim) return 0;
  return round_up((size_t)N * sizeof(double), 256) + calib_tiles(N) * (size_t)(d / 2) * sizeof(float);
}

size_t qamw_encode_workspace_bytes(int64_t N) {
  if (N <= 0 || N > kMaxDim) return 0;
  return round_up((size_t)N * sizeof(double), 256);
}

const char* qamw_status_string(int32_t status) {
  switch (status) {
    case QAMW_OK: return "ok";
    case QAMW_EINVAL: return "invalid argument";
    case QAMW_EUNSUPPORTED: return "unsupported argument";
    case QAMW_EHIP: return "HIP runtime error";
    case QAMW_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* qamw_last_error(void) { return g_last_error.c_str(); }

const char* qamw_version(void) { return "qamw 0.1 gfx950"; }

int32_t qamw_calibrate(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* chan_rms,
                       float alpha, int32_t block, uint64_t sign_seed, float* s_out, float* sigma_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if (!chan_rms || !s_out || !sigma_out) return fail(QAMW_EINVAL, "chan_rms, s_out and sigma_out must be non-NULL");
  if (!aligned16(s_out) || !aligned16(sigma_out)) return fail(QAMW_EINVAL, "s_out and sigma_out must be 16-byte aligned");
  if (!isfinite(alpha)) return fail(QAMW_EINVAL, "alpha must be finite");
  const size_t need = qamw_calibrate_workspace_bytes(N, d, block);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "calibrate needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  double* rho = (double*)workspace;
  float* partial = (float*)((char*)workspace + round_up((size_t)N * sizeof(double), 256));
  const int n = (int)N, dd = (int)d;

  hipLaunchKernelGGL(scale_kernel, dim3((dd + kBlockThreads - 1) / kBlockThreads), dim3(kBlockThreads), 0, st,
                     chan_rms, alpha, dd, s_out);
  if ((rc = check_launch("scale_kernel"))) return rc;
  if ((rc = launch_rownorm(W, wdtype, n, dd, ldw, s_out, rho, nullptr, st))) return rc;
  if ((rc = dispatch_L<LaunchAmplitude>(L, W, wdtype, n, dd, ldw, (const float*)s_out, sign_seed, (const double*)rho,
                                         partial, st)))
    return rc;
  const int half_d = dd / 2;
  const int sigma_cols = kBlockThreads / kSigmaSlices;
  hipLaunchKernelGGL(sigma_kernel, dim3((half_d + sigma_cols - 1) / sigma_cols), dim3(kBlockThreads), 0, st,
                     (const float*)partial, (int)calib_tiles(N), half_d, n, sigma_out);
  return check_launch("sigma_kernel");
}

int32_t qamw_encode(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* s,
                    const float* sigma, int32_t block, uint64_t sign_seed, const float* codebook, int32_t K,
                    uint32_t* packed, uint16_t* rownorm_f16, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!s || !sigma || !packed || !rownorm_f16) return fail(QAMW_EINVAL, "s, sigma, packed and rownorm_f16 must be non-NULL");
  if (!aligned16(s) || !aligned16(sigma) || !aligned16(packed))
    return fail(QAMW_EINVAL, "s, sigma and packed must be 16-byte aligned");
  const size_t need = qamw_encode_workspace_bytes(N);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "encode needs %zu bytes of 256-byte aligned workspace (got %zu)", need, workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  double* rho = (double*)workspace;
  const int n = (int)N, dd = (int)d;
  const int B = qamw_index_bits(K);
  const int row_words = (int)qamw_packed_row_words(d, K);
  if ((rc = launch_rownorm(W, wdtype, n, dd, ldw, s, rho, rownorm_f16, st))) return rc;
  return dispatch_L<LaunchEncode>(L, W, wdtype, n, dd, ldw, s, sigma, sign_seed, codebook, (int)K, B, row_words,
                                  (const double*)rho, packed, st);
}

int32_t qamw_decode(const uint32_t* packed, const uint16_t* rownorm_f16, int64_t N, int64_t d, const float* s,
                    const float* sigma, int32_t block, uint64_t sign_seed, const float* codebook, int32_t K,
                    void* W_out, int32_t out_dtype, int64_t ldo, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!packed || !rownorm_f16 || !sigma || !W_out)
    return fail(QAMW_EINVAL, "packed, rownorm_f16, sigma and W_out must be non-NULL");
  if (out_dtype != QAMW_F32 && out_dtype != QAMW_BF16 && out_dtype != QAMW_F16)
    return fail(QAMW_EUNSUPPORTED, "output dtype %d not supported", out_dtype);
  if (ldo < d) return fail(QAMW_EINVAL, "ldo=%lld < d=%lld", (long long)ldo, (long long)d);
  if (!aligned16(packed) || !aligned16(W_out) || (ldo * elem_size(out_dtype)) % 16 || !aligned16(sigma))
    return fail(QAMW_EINVAL, "packed, sigma and W_out must be 16-byte aligned with 16-byte aligned rows");
  hipStream_t st = (hipStream_t)stream;
  const int B = qamw_index_bits(K);
  const int row_words = (int)qamw_packed_row_words(d, K);
  return dispatch_L<LaunchDecode>(L, packed, rownorm_f16, (int)N, (int)d, s, sigma, sign_seed, codebook, (int)K, B,
                                  row_words, W_out, out_dtype, ldo, st);
}

}  // extern "C"
