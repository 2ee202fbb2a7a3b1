// Calibration statistics of the activations and the layer-output error
// ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Activation-Aware
// Scaling, for the channel RMS r_j; the composite bound chain's trace
// identity || X dW^T ||_F^2 = Tr(dW M dW^T), M = X^T X, for the error).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

// ---------------------------------------------------------------------------
// r_j = sqrt(sum_t X[t][j]^2 / T).  Pass 1: thread (8 columns, row tile)
// sums the squares of its tile's rows in row order (fp32); pass 2 adds the
// tiles in tile order in fp64.  Deterministic.
// ---------------------------------------------------------------------------
template <typename Tin>
__device__ __forceinline__ void load8(const Tin* p, float x[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float x[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float x[8]) {
  const uint4 t = reinterpret_cast<const uint4*>(p)[0];
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

template <typename Tin>
__global__ __launch_bounds__(kBlockThreads) void sumsq_kernel(const Tin* __restrict__ X, int64_t ldx, int T, int d,
                                                              float* __restrict__ partial) {
  const int g = blockIdx.x * kBlockThreads + threadIdx.x;     // column group: columns 8 g .. 8 g + 7
  if (8 * g >= d) return;
  const int t0 = blockIdx.y * kRmsRowsPerTile;
  const int t1 = min(T, t0 + kRmsRowsPerTile);
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  const Tin* p = X + (int64_t)t0 * ldx + 8 * g;
#pragma unroll 8
  for (int t = t0; t < t1; ++t, p += ldx) {
    float x[8];
    load8<Tin>(p, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += x[i] * x[i];
  }
  float4* out = reinterpret_cast<float4*>(partial + (int64_t)blockIdx.y * d + 8 * g);
  out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

__global__ __launch_bounds__(kBlockThreads) void rms_finish_kernel(const float* __restrict__ partial, int ntiles,
                                                                   int T, int d, float* __restrict__ r) {
  const int j = blockIdx.x * kBlockThreads + threadIdx.x;
  if (j >= d) return;
  double s = 0.0;
  for (int t = 0; t < ntiles; ++t) s += (double)partial[(int64_t)t * d + j];
  r[j] = (float)sqrt(s / (double)T);
}

// ---------------------------------------------------------------------------
// E = sum_{t < T, n < N} D[t][n]^2,  D = X dW^T,  dW = W - W^ (fp32
// difference rounded to bf16; X rounded to bf16 unless it is bf16).
//
// A workgroup of four wavefronts owns a 128 (tokens) x 128 (rows) block of D
// and walks the columns in steps of 32: the step's X and dW tiles are
// written to LDS as bf16, and each wavefront multiplies a 64 x 64 quarter as
// 4 x 4 v_mfma_f32_16x16x32_bf16 tiles.  MFMA layout: lane l holds
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16]; result register r
// of lane l is C[4 (l / 16) + r][l % 16].  Rows and tokens past N, T reload
// the last one and are left out of the sum; columns past d are zero.  Each
// workgroup sums its squares in fp64 in a fixed order; a second kernel adds
// the workgroups' sums in a fixed order.  Deterministic.
// ---------------------------------------------------------------------------
constexpr int kOeTile = kOutputErrorTile;
constexpr int kOeK = 32;
constexpr int kOeRow = kOeK + 8;        // LDS row stride in bf16 elements (80 bytes: spreads the banks)

// 16 consecutive values of row `row` from column c (zeros past d)
template <typename Tin>
__device__ __forceinline__ void load16(const Tin* base, int64_t ld, int row, int c, int d, float x[16]) {
  if (c < d) {
    const Tin* p = base + (int64_t)row * ld + c;
    load8<Tin>(p, x);
    load8<Tin>(p + 8, x + 8);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.0f;
  }
}

template <typename TX, typename TW, typename TH>
__global__ __launch_bounds__(256) void output_error_kernel(const TX* __restrict__ X, int64_t ldx, int T, int d,
                                                           const TW* __restrict__ W, int64_t ldw,
                                                           const TH* __restrict__ Wh, int64_t ldh, int N,
                                                           double* __restrict__ partial) {
  __shared__ __align__(16) uint16_t As[kOeTile * kOeRow];
  __shared__ __align__(16) uint16_t Bs[kOeTile * kOeRow];
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wt = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.y * kOeTile, n0 = blockIdx.x * kOeTile;
  // loader: thread -> tile row tid / 2, 16 columns at 16 (tid % 2)
  const int lrow = tid >> 1, lcol = 16 * (tid & 1);
  const int xt = min(t0 + lrow, T - 1), wr = min(n0 + lrow, N - 1);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int k0 = 0; k0 < d; k0 += kOeK) {
    {
      float xv[16], wv[16], hv[16];
      load16<TX>(X, ldx, xt, k0 + lcol, d, xv);
      load16<TW>(W, ldw, wr, k0 + lcol, d, wv);
      load16<TH>(Wh, ldh, wr, k0 + lcol, d, hv);
      uint32_t ab[8], bb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ab[i] = f32_to_bf16_bits(xv[2 * i]) | (f32_to_bf16_bits(xv[2 * i + 1]) << 16);
        bb[i] = f32_to_bf16_bits(wv[2 * i] - hv[2 * i]) | (f32_to_bf16_bits(wv[2 * i + 1] - hv[2 * i + 1]) << 16);
      }
      uint4* ad = reinterpret_cast<uint4*>(As + lrow * kOeRow + lcol);
      uint4* bd = reinterpret_cast<uint4*>(Bs + lrow * kOeRow + lcol);
      ad[0] = make_uint4(ab[0], ab[1], ab[2], ab[3]);
      ad[1] = make_uint4(ab[4], ab[5], ab[6], ab[7]);
      bd[0] = make_uint4(bb[0], bb[1], bb[2], bb[3]);
      bd[1] = make_uint4(bb[4], bb[5], bb[6], bb[7]);
    }
    __syncthreads();
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const bf16x8*>(As + (64 * wt + 16 * i + l16) * kOeRow + 8 * g);
      b[i] = *reinterpret_cast<const bf16x8*>(Bs + (64 * wn + 16 * i + l16) * kOeRow + 8 * g);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  // ---- squares of the valid entries, fp64, fixed order
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 64 * wt + 16 * i + 4 * g + r;
        const int n = n0 + 64 * wn + 16 * j + l16;
        const double v = (double)acc[i][j][r];
        s += (t < T && n < N) ? v * v : 0.0;
      }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

// thread i adds partials i, i + 256, ... in order; the 256 sums are then
// added pairwise in a fixed tree: the same order on every call
__global__ __launch_bounds__(256) void sum_partials_kernel(const double* __restrict__ partial, int n,
                                                           double* __restrict__ out) {
  __shared__ double sh[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += partial[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) sh[threadIdx.x] += sh[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = sh[0];
}

// ===========================================================================
// launchers
// ===========================================================================
int launch_channel_rms(const void* X, int32_t xdt, int T, int d, int64_t ldx, float* r, float* partial,
                       hipStream_t st) {
  const int ntiles = (T + kRmsRowsPerTile - 1) / kRmsRowsPerTile;
  const dim3 grid((unsigned)((d / 8 + kBlockThreads - 1) / kBlockThreads), (unsigned)ntiles), blk(kBlockThreads);
  if (xdt == QAMW_F32)
    hipLaunchKernelGGL(sumsq_kernel<float>, grid, blk, 0, st, (const float*)X, ldx, T, d, partial);
  else
    hipLaunchKernelGGL(sumsq_kernel<uint16_t>, grid, blk, 0, st, (const uint16_t*)X, ldx, T, d, partial);
  int rc = check_launch("sumsq_kernel");
  if (rc) return rc;
  hipLaunchKernelGGL(rms_finish_kernel, dim3((d + kBlockThreads - 1) / kBlockThreads), dim3(kBlockThreads), 0, st,
                     partial, ntiles, T, d, r);
  return check_launch("rms_finish_kernel");
}

template <typename TX, typename TW, typename TH>
static void launch_oe(const void* X, int64_t ldx, int T, int d, const void* W, int64_t ldw, const void* Wh,
                      int64_t ldh, int N, double* partial, hipStream_t st) {
  const dim3 grid((unsigned)((N + kOeTile - 1) / kOeTile), (unsigned)((T + kOeTile - 1) / kOeTile)), blk(256);
  hipLaunchKernelGGL((output_error_kernel<TX, TW, TH>), grid, blk, 0, st, (const TX*)X, ldx, T, d, (const TW*)W,
                     ldw, (const TH*)Wh, ldh, N, partial);
}

template <typename TX, typename TW>
static void launch_oe_h(int32_t hdt, const void* X, int64_t ldx, int T, int d, const void* W, int64_t ldw,
                        const void* Wh, int64_t ldh, int N, double* partial, hipStream_t st) {
  if (hdt == QAMW_F32) launch_oe<TX, TW, float>(X, ldx, T, d, W, ldw, Wh, ldh, N, partial, st);
  else launch_oe<TX, TW, uint16_t>(X, ldx, T, d, W, ldw, Wh, ldh, N, partial, st);
}

int launch_output_error(const void* X, int32_t xdt, int T, int d, int64_t ldx, const void* W, int32_t wdt, int N,
                        int64_t ldw, const void* Wh, int32_t hdt, int64_t ldh, double* out, double* partial,
                        hipStream_t st) {
  if (xdt == QAMW_F32) {
    if (wdt == QAMW_F32) launch_oe_h<float, float>(hdt, X, ldx, T, d, W, ldw, Wh, ldh, N, partial, st);
    else launch_oe_h<float, uint16_t>(hdt, X, ldx, T, d, W, ldw, Wh, ldh, N, partial, st);
  } else {
    if (wdt == QAMW_F32) launch_oe_h<uint16_t, float>(hdt, X, ldx, T, d, W, ldw, Wh, ldh, N, partial, st);
    else launch_oe_h<uint16_t, uint16_t>(hdt, X, ldx, T, d, W, ldw, Wh, ldh, N, partial, st);
  }
  int rc = check_launch("output_error_kernel");
  if (rc) return rc;
  const int nparts = ((N + kOeTile - 1) / kOeTile) * ((T + kOeTile - 1) / kOeTile);
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, st, partial, nparts, out);
  return check_launch("sum_partials_kernel");
}

}  // namespace qamw
