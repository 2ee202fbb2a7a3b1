// Codebook refinement on a matrix's own normalised pairs (Lloyd rounds;
// "QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Significance and Claims, on a
// learned codebook).
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
// Codebook refinement on the matrix's own pairs (the pages suggest a learned
// codebook; Lloyd rounds on the normalised pairs z~).  One round = the encode
// (assignment, any kernel above) followed by these two kernels:
//   lloyd_accum_kernel   re-derives z~ with the encode's own transform, reads
//                        each pair's index from the packed rows and adds z~
//                        into its centroid's sums -- fixed point, 2^-28 units,
//                        in 64-bit integers (LDS atomics per workgroup, then
//                        global atomics), so the sums do not depend on the
//                        order of the additions; |z~ - C[idx]|^2 is summed in
//                        fp64 per lane, per wavefront and per workgroup in a
//                        fixed order
//   lloyd_update_kernel  C'[c] = sum / count rounded to fp32 (a centroid with no
//                        pair keeps its place), and the mean squared distance.
// Deterministic.
// ---------------------------------------------------------------------------
constexpr double kLloydScale = 268435456.0;      // 2^28
constexpr int kLloydWgPerCu = 2;

template <int L, typename Tin>
__global__ __launch_bounds__(kEncThreads) void lloyd_accum_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ f,
    const float* __restrict__ isig, const double* __restrict__ rho, const uint32_t* __restrict__ packed,
    int row_words, int B, const float* __restrict__ codebook, int K, unsigned long long* __restrict__ gacc,
    double* __restrict__ partial) {
  extern __shared__ unsigned long long lacc[];     // K x (sum x, sum y, count)
  __shared__ double red[kEncWaves];
  for (int i = threadIdx.x; i < 3 * K; i += kEncThreads) lacc[i] = 0ull;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: window bookkeeping stays scalar
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int total = N * nwin;
  const int stride = gridDim.x * kEncWaves;
  double dsum = 0.0;
  for (int gw = blockIdx.x * kEncWaves + wave; gw < total; gw += stride) {
    const int n = gw / nwin, win = gw - (gw / nwin) * nwin;
    WinLoads<Tin> wl;
    load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
    const bool active = win * kWinChunks + lane < nchunks;
    float zx[8], zy[8];
    const int co_local = window_transform<L>(wl, active, lane, zx, zy);
    // the 8 indices of window pairs 8 co_local .. + 7: 8 B bits from bit
    // (512 win + 8 co_local) B of the row (words past the row end only feed
    // unused bits, so their loads are clamped into the row)
    const int64_t bit0 = (int64_t)(win * kWinPairs + co_local * kPairsPerLane) * B;
    const int w0 = (int)(bit0 >> 5);
    const uint32_t* prow = packed + (int64_t)n * row_words;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = prow[min(w0 + i, row_words - 1)];
    uint32_t idx[8];
    unpack8<0>(w, (uint32_t)(bit0 & 31), B, idx);
    if (active) {
#pragma unroll
      for (int p = 0; p < kPairsPerLane; ++p) {
        const int c = min((int)idx[p], K - 1);
        const double cx = (double)codebook[2 * c], cy = (double)codebook[2 * c + 1];
        const double dx = (double)zx[p] - cx, dy = (double)zy[p] - cy;
        dsum += dx * dx + dy * dy;
        atomicAdd(&lacc[3 * c + 0], (unsigned long long)__double2ll_rn((double)zx[p] * kLloydScale));
        atomicAdd(&lacc[3 * c + 1], (unsigned long long)__double2ll_rn((double)zy[p] * kLloydScale));
        atomicAdd(&lacc[3 * c + 2], 1ull);
      }
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) dsum += __shfl_xor(dsum, off);
  if (lane == 0) red[wave] = dsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kEncWaves; ++i) t += red[i];
    partial[blockIdx.x] = t;
  }
  for (int i = threadIdx.x; i < 3 * K; i += kEncThreads)
    if (lacc[i]) atomicAdd(&gacc[i], lacc[i]);
}

__global__ __launch_bounds__(256) void lloyd_zero_kernel(unsigned long long* __restrict__ gacc, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) gacc[i] = 0ull;
}

__global__ __launch_bounds__(256) void lloyd_update_kernel(const unsigned long long* __restrict__ gacc,
                                                           const float* __restrict__ codebook, int K,
                                                           const double* __restrict__ partial, int nparts,
                                                           double npairs, float* __restrict__ out,
                                                           double* __restrict__ distortion) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < K) {
    const long long cnt = (long long)gacc[3 * c + 2];
    if (cnt > 0) {
      const double sx = (double)(long long)gacc[3 * c] / kLloydScale;
      const double sy = (double)(long long)gacc[3 * c + 1] / kLloydScale;
      out[2 * c] = (float)(sx / (double)cnt);
      out[2 * c + 1] = (float)(sy / (double)cnt);
    } else {
      out[2 * c] = codebook[2 * c];
      out[2 * c + 1] = codebook[2 * c + 1];
    }
  }
  if (blockIdx.x == 0) {                       // partial sums: strided per thread, then a fixed tree
    __shared__ double sh[256];
    double t = 0.0;
    for (int i = threadIdx.x; i < nparts; i += 256) t += partial[i];
    sh[threadIdx.x] = t;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if ((int)threadIdx.x < h) sh[threadIdx.x] += sh[threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x == 0) *distortion = sh[0] / npairs;
  }
}

// ===========================================================================
// launchers
// ===========================================================================
template <int L>
struct LaunchLloyd {
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const float* isig,
                 const double* rho, const uint32_t* packed, int row_words, int B, const float* cb, int K,
                 unsigned long long* gacc, double* partial, int nparts, hipStream_t st) {
    const size_t lds = (size_t)3 * K * sizeof(unsigned long long);
    if (wdt == QAMW_F32)
      hipLaunchKernelGGL((lloyd_accum_kernel<L, float>), dim3(nparts), dim3(kEncThreads), lds, st, (const float*)W,
                         ldw, N, d, f, isig, rho, packed, row_words, B, cb, K, gacc, partial);
    else
      hipLaunchKernelGGL((lloyd_accum_kernel<L, uint16_t>), dim3(nparts), dim3(kEncThreads), lds, st,
                         (const uint16_t*)W, ldw, N, d, f, isig, rho, packed, row_words, B, cb, K, gacc, partial);
    return check_launch("lloyd_accum_kernel");
  }
};

int lloyd_parts(int N, int d) {
  const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
  const int64_t wgs = ((int64_t)N * nwin + kEncWaves - 1) / kEncWaves;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return (int)std::min<int64_t>(std::min<int64_t>(wgs, (int64_t)cus * kLloydWgPerCu), kLloydMaxParts);
}

int launch_lloyd_update(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f,
                        const float* isig, const double* rho, const uint32_t* packed, int row_words, int B,
                        const float* cb, int K, float* cb_out, double* distortion, unsigned long long* gacc,
                        double* partial, hipStream_t st) {
  hipLaunchKernelGGL(lloyd_zero_kernel, dim3((3 * K + 255) / 256), dim3(256), 0, st, gacc, 3 * K);
  int rc = check_launch("lloyd_zero_kernel");
  if (rc) return rc;
  const int nparts = lloyd_parts(N, d);
  if ((rc = dispatch_L<LaunchLloyd>(L, W, wdt, N, d, ldw, f, isig, rho, packed, row_words, B, cb, K, gacc, partial,
                                    nparts, st)))
    return rc;
  const int64_t npairs = (int64_t)N * (d / 2);
  hipLaunchKernelGGL(lloyd_update_kernel, dim3((K + 255) / 256), dim3(256), 0, st, gacc, cb, K, partial, nparts,
                     (double)npairs, cb_out, distortion);
  return check_launch("lloyd_update_kernel");
}

}  // namespace qamw
