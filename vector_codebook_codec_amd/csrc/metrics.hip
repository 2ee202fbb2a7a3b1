// Calibration statistics of the activations and the layer-output error
// ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Activation-Aware
// Scaling, for the channel RMS r_j; the composite bound chain's trace
// identity || X dW^T ||_F^2 = Tr(dW M dW^T), M = X^T X, for the error).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

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
// Pass 1 (oe_prep_kernel) writes dW, and X when it is fp32, as bf16 rows to
// the workspace.  Pass 2 (output_error_kernel), a GEMM with a sum of squares
// instead of a store: a workgroup of four wavefronts owns a 128 (tokens) x
// 128 (rows) block of D and walks the columns in steps of 64.  Each step's A
// (X) and B (dW) tiles are loaded from memory once per workgroup -- coalesced,
// 16 bytes per thread and instruction, two steps ahead into registers, from
// clamped addresses (rows past T, N reload the last one and are left out of
// the sum; 8-column pieces past d are zeroed) -- and written to one of two
// LDS buffers (rows padded to 144 bytes), one barrier per step.  Wavefront w
// multiplies tokens 64 (w / 2) .. + 64 by rows 64 (w % 2) .. + 64 as 4 x 4
// v_mfma_f32_16x16x32_bf16 tiles, reading its fragments from LDS in the MFMA
// layout -- lane l holds A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e]
// [l % 16] -- with the step's 64 columns permuted identically for A and B
// (lane group g takes columns 16 g + 8 h .. + 8 for MFMA h).  Result register
// r of lane l is C[4 (l / 16) + r][l % 16].  Squares are summed in fp64 per
// lane, wavefront and workgroup in a fixed order, the workgroups' sums in a
// fixed tree.  A single TA pass per operand per workgroup is the point: the
// earlier direct-to-register version spent ~83% of its time in address
// processing.
// ---------------------------------------------------------------------------
constexpr int kOeT = kOutputErrorTokens;
constexpr int kOeN = kOutputErrorRows;
constexpr int kOeK = 64;                // columns per step
constexpr int kOeRowE = kOeK + 8;       // LDS row stride in bf16 elements (144 bytes)

template <typename TX, typename TW, typename TH>
__global__ __launch_bounds__(256) void oe_prep_kernel(const TX* __restrict__ X, int64_t ldx, int T,
                                                      const TW* __restrict__ W, int64_t ldw,
                                                      const TH* __restrict__ Wh, int64_t ldh, int N, int d,
                                                      uint16_t* __restrict__ dWb, uint16_t* __restrict__ Xb) {
  const int cpr = d >> 4;                                  // 16-column chunks per row
  const int64_t nW = (int64_t)N * cpr;
  const int64_t nX = Xb ? (int64_t)T * cpr : 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nW + nX; i += (int64_t)gridDim.x * 256) {
    float v[16];
    int64_t row, c;
    uint16_t* dst;
    if (i < nW) {
      row = i / cpr;
      c = (i - row * cpr) * 16;
      float w[16], h[16];
      load8<TW>(W + row * ldw + c, w);
      load8<TW>(W + row * ldw + c + 8, w + 8);
      load8<TH>(Wh + row * ldh + c, h);
      load8<TH>(Wh + row * ldh + c + 8, h + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = w[e] - h[e];
      dst = dWb + row * d + c;
    } else {
      const int64_t k = i - nW;
      row = k / cpr;
      c = (k - row * cpr) * 16;
      load8<TX>(X + row * ldx + c, v);
      load8<TX>(X + row * ldx + c + 8, v + 8);
      dst = Xb + row * d + c;
    }
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    uint4* q = reinterpret_cast<uint4*>(dst);
    q[0] = make_uint4(o[0], o[1], o[2], o[3]);
    q[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// Workgroups are dealt to the 8 XCDs round-robin by index (each XCD has its
// own L2), so index L runs on XCD L % 8; the mapping below gives every XCD
// whole row blocks -- row block 8 q + (L % 8) with all its token blocks in a
// row -- so a row block's dW tile is fetched into one L2 while every token
// block uses it.  Indices past the last row block only write a zero partial.
constexpr int kXcds = 8;

__global__ __launch_bounds__(256) void output_error_kernel(const uint16_t* __restrict__ A, int64_t lda, int T,
                                                           const uint16_t* __restrict__ Bm, int N, int d,
                                                           int tblocks, double* __restrict__ partial) {
  __shared__ __align__(16) uint16_t As[2][kOeT * kOeRowE];
  __shared__ __align__(16) uint16_t Bs[2][kOeN * kOeRowE];
  __shared__ double red[4];
  const int L = blockIdx.x;
  const int kk = L / kXcds;
  const int nb = (L % kXcds) + kXcds * (kk / tblocks);
  const int tb = kk % tblocks;
  if (nb * kOeN >= N) {                          // padding: uniform per workgroup
    if (threadIdx.x == 0) partial[L] = 0.0;
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wt = wave >> 1, wn = wave & 1;
  const int t0 = tb * kOeT, n0 = nb * kOeN;
  const int nsteps = (d + kOeK - 1) / kOeK;

  // loader: piece p = tid + 256 u (u < 4) of a 128 x 64 tile is row p / 8,
  // columns 8 (p % 8) .. + 8
  const uint16_t* ap[4];
  const uint16_t* bp[4];
  int lrow[4], lcol[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pc = tid + 256 * u;
    lrow[u] = pc >> 3;
    lcol[u] = 8 * (pc & 7);
    ap[u] = A + (int64_t)min(t0 + lrow[u], T - 1) * lda;
    bp[u] = Bm + (int64_t)min(n0 + lrow[u], N - 1) * d;
  }
  u32x4 ra[4], rb[4];                            // one step's pieces in flight
  auto gload = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = min(st * kOeK + lcol[u], d - 8);
      ra[u] = *reinterpret_cast<const u32x4*>(ap[u] + c);
      rb[u] = *reinterpret_cast<const u32x4*>(bp[u] + c);
    }
  };
  auto lstore = [&](int st, int buf) __attribute__((always_inline)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = st * kOeK + lcol[u] < d;
      *reinterpret_cast<u32x4*>(&As[buf][lrow[u] * kOeRowE + lcol[u]]) = in ? ra[u] : z;
      *reinterpret_cast<u32x4*>(&Bs[buf][lrow[u] * kOeRowE + lcol[u]]) = in ? rb[u] : z;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  gload(0);
  lstore(0, 0);
  gload(1);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(64 * wt + 16 * i + l16) * kOeRowE + 16 * g + 8 * h]);
        b[i] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(64 * wn + 16 * i + l16) * kOeRowE + 16 * g + 8 * h]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    // the next step's tile into the other buffer (its readers passed the
    // previous barrier), then the loads of the step after it
    lstore(st + 1, buf ^ 1);
    gload(st + 2);
    __syncthreads();
  }

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
  if (threadIdx.x == 0) partial[L] = ((red[0] + red[1]) + red[2]) + red[3];
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
static void launch_prep(const void* X, int64_t ldx, int T, const void* W, int64_t ldw, const void* Wh, int64_t ldh,
                        int N, int d, uint16_t* dWb, uint16_t* Xb, hipStream_t st) {
  const int64_t work = ((int64_t)N + (Xb ? T : 0)) * (d / 16);
  const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 8192);
  hipLaunchKernelGGL((oe_prep_kernel<TX, TW, TH>), dim3(blocks), dim3(256), 0, st, (const TX*)X, ldx, T, (const TW*)W,
                     ldw, (const TH*)Wh, ldh, N, d, dWb, Xb);
}

template <typename TX, typename TW>
static void launch_prep_h(int32_t hdt, const void* X, int64_t ldx, int T, const void* W, int64_t ldw, const void* Wh,
                          int64_t ldh, int N, int d, uint16_t* dWb, uint16_t* Xb, hipStream_t st) {
  if (hdt == QAMW_F32) launch_prep<TX, TW, float>(X, ldx, T, W, ldw, Wh, ldh, N, d, dWb, Xb, st);
  else launch_prep<TX, TW, uint16_t>(X, ldx, T, W, ldw, Wh, ldh, N, d, dWb, Xb, st);
}

int launch_output_error(const void* X, int32_t xdt, int T, int d, int64_t ldx, const void* W, int32_t wdt, int N,
                        int64_t ldw, const void* Wh, int32_t hdt, int64_t ldh, double* out, double* partial,
                        uint16_t* dWb, uint16_t* Xb, hipStream_t st) {
  uint16_t* xb = (xdt == QAMW_F32) ? Xb : nullptr;        // bf16 activations are used in place
  if (xdt == QAMW_F32) {
    if (wdt == QAMW_F32) launch_prep_h<float, float>(hdt, X, ldx, T, W, ldw, Wh, ldh, N, d, dWb, xb, st);
    else launch_prep_h<float, uint16_t>(hdt, X, ldx, T, W, ldw, Wh, ldh, N, d, dWb, xb, st);
  } else {
    if (wdt == QAMW_F32) launch_prep_h<uint16_t, float>(hdt, X, ldx, T, W, ldw, Wh, ldh, N, d, dWb, xb, st);
    else launch_prep_h<uint16_t, uint16_t>(hdt, X, ldx, T, W, ldw, Wh, ldh, N, d, dWb, xb, st);
  }
  int rc = check_launch("oe_prep_kernel");
  if (rc) return rc;
  const uint16_t* A = xb ? xb : (const uint16_t*)X;
  const int64_t lda = xb ? d : ldx;
  const int nblocks = (N + kOeN - 1) / kOeN, tblocks = (T + kOeT - 1) / kOeT;
  const int nwg = kXcds * ((nblocks + kXcds - 1) / kXcds) * tblocks;
  hipLaunchKernelGGL(output_error_kernel, dim3((unsigned)nwg), dim3(256), 0, st, A, lda, T, (const uint16_t*)dWb, N,
                     d, tblocks, partial);
  if ((rc = check_launch("output_error_kernel"))) return rc;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, st, partial, nwg, out);
  return check_launch("sum_partials_kernel");
}

}  // namespace qamw
