// Calibration kernels: channel scales, row norms, per-pair amplitude sums and
// sigma ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Activation-Aware
// Scaling, Separation of Scale and Direction, Pairing and Calibration).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

// ---------------------------------------------------------------------------
// s_j = r_j ^ alpha.  alpha = 0 gives exactly 1.
// ---------------------------------------------------------------------------
// Also f_j = eps_j s_j, the column factor the rotation pass applies.
__global__ __launch_bounds__(kBlockThreads) void scale_kernel(const float* __restrict__ r, float alpha,
                                                              uint64_t seed, int d, float* __restrict__ s,
                                                              float* __restrict__ f) {
  const int j = blockIdx.x * kBlockThreads + threadIdx.x;
  if (j < d) {
    const float sj = (alpha == 0.0f) ? 1.0f : powf(r[j], alpha);
    s[j] = sj;
    f[j] = sj * sign_eps(seed, (uint32_t)j);
  }
}

// rho_n = ||W_n diag(s)||, one wavefront per row (row_norm_wave): its
// binary16 bits and the row factor 1 / (sqrt(b) rho_n).
template <typename Tin>
__global__ __launch_bounds__(kBlockThreads) void rownorm_kernel(const Tin* __restrict__ W, int64_t ldw,
                                                                int N, int d, const float* __restrict__ s,
                                                                double sqrt_b, double* __restrict__ rowf,
                                                                uint16_t* __restrict__ rho_f16) {
  const int n = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (n < N) row_norm_wave(W, ldw, n, d, s, sqrt_b, rowf, rho_f16);
}

// ---------------------------------------------------------------------------
// Calibration, pass 2: per (window, row tile) wavefront, accumulate the pair
// amplitudes |z_{n,k}| of the normalised rotated rows over the tile.
// partial[t][k] = sum_{n in tile t} hypot(y_{n,2k}, y_{n,2k+1}) / (sqrt(b) rho_n),
// the divisor read as the row factor rownorm_kernel wrote.
// ---------------------------------------------------------------------------
template <int L, typename Tin>
__global__ __launch_bounds__(kBlockThreads) void amplitude_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ fcol,
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
  if (active) load_chunk(fcol + c * kChunk, f);
  float acc[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) acc[p] = 0.0f;

  const int n0 = tile * kCalibRowsPerTile;
  const int n1 = min(N, n0 + kCalibRowsPerTile);
  // 1 / (sqrt(b) rho_n) of the tile's rows (the row factors), one per lane
  float inv_lane = 0.0f;
  if (lane < n1 - n0) inv_lane = (float)rho[n0 + lane];
  // a ring of kAmpDepth rows in flight: row n + kAmpDepth is loaded while row n is processed
  constexpr int kAmpDepth = 4;
  RawChunk<Tin> ring[kAmpDepth];
  const Tin* base = W + c * kChunk;
#pragma unroll
  for (int u = 0; u < kAmpDepth; ++u)
    if (active && n0 + u < n1) ring[u].load(base + (int64_t)(n0 + u) * ldw);
  for (int n = n0; n < n1; n += kAmpDepth) {
#pragma unroll
    for (int u = 0; u < kAmpDepth; ++u) {
      if (n + u >= n1) break;
      float x[16];
      ring[u].unpack(x);
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = active ? x[i] * f[i] : 0.0f;
      if (active && n + u + kAmpDepth < n1) ring[u].load(base + (int64_t)(n + u + kAmpDepth) * ldw);
      fwht_block<L>(x, lane);
      const float inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv_lane), n + u - n0));
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float a = x[2 * p], b = x[2 * p + 1];
        // v_sqrt_f32 (1 ulp) rather than the correctly rounded sqrtf expansion
        acc[p] += __builtin_amdgcn_sqrtf(__builtin_fmaf(a, a, b * b)) * inv;
      }
    }
  }
  if (active) {
    float4* out = reinterpret_cast<float4*>(partial + (int64_t)tile * (d >> 1) + co * kPairsPerLane);
    out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// ---------------------------------------------------------------------------
// Passes 1 and 2 with one read of W (rows of up to kFuseMaxWin windows).  A
// workgroup owns a tile of rows_per_tile rows across the whole width,
// wavefront w = window w.  For each row every wavefront forms its window's
// share of rho_n^2 (chunk_sumsq + window_sum, as row_norm_wave does) and the
// pair amplitudes; the shares meet in LDS, every wavefront adds them in window
// order (the same fp64 sum as row_norm_wave, so rho is identical; one lane
// per row of a batch, which also writes the row factor 1 / (sqrt(b) rho_n)),
// and the amplitudes are scaled and accumulated exactly as amplitude_kernel
// does.  A barrier per batch of rows; the share buffer
// alternates between batches.
// ---------------------------------------------------------------------------
constexpr int kFuseMaxWin = 16;   // 1024 threads
constexpr int kFuseMidWin = 12;   // up to 768 threads: registers for more rows per barrier

template <int L, typename Tin, int kMaxWin>
__global__ __launch_bounds__(kMaxWin * kWave) void norm_amplitude_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ fcol,
    double* __restrict__ rho, uint16_t* __restrict__ rho_f16, float* __restrict__ partial, int rows_per_tile) {
  // rows per barrier (and loads in flight); blocks below 32 or above 256
  // columns need more registers for their lane stages, and take two
  constexpr bool kWide = sizeof(Tin) == 2 && kMaxWin <= kFuseMidWin && L >= 5 && L <= 8;
  constexpr int kBatch = kWide ? 4 : (sizeof(Tin) == 2 || kMaxWin <= kFuseMidWin ? 2 : 1);
  __shared__ double share[2][kBatch][kMaxWin];
  const int lane = threadIdx.x & (kWave - 1);
  const int win = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wavefront
  const int nwin = blockDim.x >> 6;
  const int nchunks = d >> 4;
  const int tile = blockIdx.x;
  const int c = win * kWinChunks + lane;
  const bool active = c < nchunks;   // whole Hadamard blocks are active or not
  const int co = win * kWinChunks + BlockOut<L>::chunk(lane);
  const double sqrt_b = sqrt((double)(1 << L));

  float f[16];
  if (active) {
    load_chunk(fcol + c * kChunk, f);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = 0.0f;
  }
  float acc[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) acc[p] = 0.0f;

  const int n0 = tile * rows_per_tile;
  const int n1 = min(N, n0 + rows_per_tile);
  RawChunk<Tin> ring[kBatch];   // the batch's rows; each slot reloads the row kBatch ahead
  const Tin* base = W + c * kChunk;
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
    if (active && n0 + u < n1) ring[u].load(base + (int64_t)(n0 + u) * ldw);
    else ring[u].zero();                         // lanes past the row end keep zeros: no per-row select
  int buf = 0;
  for (int nb = n0; nb < n1; nb += kBatch) {     // uniform over the workgroup
    float amp[kBatch][8];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int n = nb + u;
      if (n >= n1) break;
      float x[16];
      ring[u].unpack(x);                        // zeros in lanes past the row end
      if (active && n + kBatch < n1) ring[u].load(base + (int64_t)(n + kBatch) * ldw);
      // an empty asm "redefines" f each row, so its fp64 conversions are redone
      // here instead of being hoisted and held (32 registers) for the loop
      asm volatile("" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]), "+v"(f[6]),
                   "+v"(f[7]), "+v"(f[8]), "+v"(f[9]), "+v"(f[10]), "+v"(f[11]), "+v"(f[12]), "+v"(f[13]),
                   "+v"(f[14]), "+v"(f[15]));
      const double sh = window_sum(chunk_sumsq(x, f));   // f = eps s: the same squares as s
      if (lane == 0) share[buf][u][win] = sh;
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] *= f[i];
      fwht_block<L>(x, lane);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float a = x[2 * p], b = x[2 * p + 1];
        // v_sqrt_f32 (1 ulp) rather than the correctly rounded sqrtf expansion
        amp[u][p] = __builtin_amdgcn_sqrtf(__builtin_fmaf(a, a, b * b));
      }
    }
    __syncthreads();
    // lane u sums row nb + u over the windows, in window order
    double t = 0.0;
    if (lane < kBatch)
      for (int w = 0; w < nwin; ++w) t += share[buf][lane][w];
    const double rn = sqrt(t);
    const double rowf = row_factor(rn, sqrt_b);
    const float inv_l = (float)rowf;
    if (win == 0 && lane < kBatch && nb + lane < n1) {
      rho[nb + lane] = rowf;
      if (rho_f16) rho_f16[nb + lane] = f64_to_f16_bits(rn);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (nb + u >= n1) break;
      const float inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv_l), u));
#pragma unroll
      for (int p = 0; p < 8; ++p) acc[p] += amp[u][p] * inv;
    }
    // the next batch writes the other buffer; the one after it has passed
    // the next barrier, so every wavefront has read this one by then
    buf ^= 1;
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
// With isig non-NULL it also writes 1 / sigma_k (fp64 division of the stored
// fp32 sigma, rounded once; 0 where sigma_k <= 0), the encode's pair factor.
__global__ __launch_bounds__(kBlockThreads) void sigma_kernel(const float* __restrict__ partial, int ntiles,
                                                              int half_d, int N, float* __restrict__ sigma,
                                                              float* __restrict__ isig) {
  __shared__ double part[kSigmaSlices][kBlockThreads / kSigmaSlices];
  const int col_in = threadIdx.x % (kBlockThreads / kSigmaSlices);
  const int slice = threadIdx.x / (kBlockThreads / kSigmaSlices);
  const int k = blockIdx.x * (kBlockThreads / kSigmaSlices) + col_in;
  double acc = 0.0;
  if (k < half_d) {
    // four loads in flight, added in tile order
    int t = slice;
    for (; t + 3 * kSigmaSlices < ntiles; t += 4 * kSigmaSlices) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = partial[(int64_t)(t + u * kSigmaSlices) * half_d + k];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += (double)v[u];
    }
    for (; t < ntiles; t += kSigmaSlices) acc += (double)partial[(int64_t)t * half_d + k];
  }
  part[slice][col_in] = acc;
  __syncthreads();
  if (slice == 0 && k < half_d) {
    double tot = 0.0;
#pragma unroll
    for (int q = 0; q < kSigmaSlices; ++q) tot += part[q][col_in];
    const float sg = (float)(tot / ((double)N * 1.2533141373155002512078826));  // sqrt(pi/2)
    sigma[k] = sg;
    if (isig) isig[k] = sg > 0.0f ? (float)(1.0 / (double)sg) : 0.0f;
  }
}

// ===========================================================================
// launchers
// ===========================================================================
int launch_scale(const float* r, float alpha, uint64_t seed, int d, float* s, float* f, hipStream_t st) {
  hipLaunchKernelGGL(scale_kernel, dim3((d + kBlockThreads - 1) / kBlockThreads), dim3(kBlockThreads), 0, st, r,
                     alpha, seed, d, s, f);
  return check_launch("scale_kernel");
}

int launch_rownorm(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, double* rho,
                   uint16_t* rho_f16, hipStream_t st) {
  const dim3 grid(grid_for_waves(N)), blk(kBlockThreads);
  const double sqrt_b = sqrt((double)(1 << L));
  if (wdt == QAMW_F32)
    hipLaunchKernelGGL(rownorm_kernel<float>, grid, blk, 0, st, (const float*)W, ldw, N, d, s, sqrt_b, rho,
                       rho_f16);
  else
    hipLaunchKernelGGL(rownorm_kernel<uint16_t>, grid, blk, 0, st, (const uint16_t*)W, ldw, N, d, s, sqrt_b, rho,
                       rho_f16);
  return check_launch("rownorm_kernel");
}

template <int L>
struct LaunchAmplitude {
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const double* rho,
                 float* partial, hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    const int64_t waves = (int64_t)nwin * (int64_t)calib_tiles(N, d);
    if (wdt == QAMW_F32)
      hipLaunchKernelGGL((amplitude_kernel<L, float>), dim3(grid_for_waves(waves)), dim3(kBlockThreads), 0, st,
                         (const float*)W, ldw, N, d, f, rho, partial);
    else
      hipLaunchKernelGGL((amplitude_kernel<L, uint16_t>), dim3(grid_for_waves(waves)), dim3(kBlockThreads), 0,
                         st, (const uint16_t*)W, ldw, N, d, f, rho, partial);
    return check_launch("amplitude_kernel");
  }
};

int launch_amplitude(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const double* rho,
                     float* partial, hipStream_t st) {
  return dispatch_L<LaunchAmplitude>(L, W, wdt, N, d, ldw, f, rho, partial, st);
}

template <int L>
struct LaunchNormAmplitude {
  template <typename Tin, int kMaxWin>
  static void go(dim3 grid, dim3 blk, const void* W, int64_t ldw, int N, int d, const float* f, double* rho,
                 uint16_t* rho_f16, float* partial, hipStream_t st) {
    hipLaunchKernelGGL((norm_amplitude_kernel<L, Tin, kMaxWin>), grid, blk, 0, st, (const Tin*)W, ldw, N, d, f, rho,
                       rho_f16, partial, calib_rows_per_tile(N, d));
  }
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, double* rho,
                 uint16_t* rho_f16, float* partial, hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    const dim3 grid((unsigned)calib_tiles(N, d)), blk((unsigned)(nwin * kWave));
    const bool mid = nwin <= kFuseMidWin;
    if (wdt == QAMW_F32) {
      if (mid) go<float, kFuseMidWin>(grid, blk, W, ldw, N, d, f, rho, rho_f16, partial, st);
      else go<float, kFuseMaxWin>(grid, blk, W, ldw, N, d, f, rho, rho_f16, partial, st);
    } else {
      if (mid) go<uint16_t, kFuseMidWin>(grid, blk, W, ldw, N, d, f, rho, rho_f16, partial, st);
      else go<uint16_t, kFuseMaxWin>(grid, blk, W, ldw, N, d, f, rho, rho_f16, partial, st);
    }
    return check_launch("norm_amplitude_kernel");
  }
};

int launch_norm_amplitude(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s,
                          const float* f, double* rho, uint16_t* rho_f16, float* partial, hipStream_t st) {
  const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
  if (nwin <= kFuseMaxWin) return dispatch_L<LaunchNormAmplitude>(L, W, wdt, N, d, ldw, f, rho, rho_f16, partial, st);
  int rc;
  if ((rc = launch_rownorm(L, W, wdt, N, d, ldw, s, rho, rho_f16, st))) return rc;
  return launch_amplitude(L, W, wdt, N, d, ldw, f, rho, partial, st);
}

int launch_sigma(const float* partial, int ntiles, int half_d, int N, float* sigma, float* isig, hipStream_t st) {
  const int cols = kBlockThreads / kSigmaSlices;
  hipLaunchKernelGGL(sigma_kernel, dim3((half_d + cols - 1) / cols), dim3(kBlockThreads), 0, st, partial, ntiles,
                     half_d, N, sigma, isig);
  return check_launch("sigma_kernel");
}

}  // namespace qamw
