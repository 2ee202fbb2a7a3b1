// Decoded-weight matmul without materialising the decoded matrix:
// Y = X W^^T for activations X [T][d] and a packed QAM-W matrix [N][d]
// ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Decoding, and the
// dequantise-then-matmul inference path whose fused form the pages leave
// open).
//
// A decoded row is W^_n = rho^_n (R_fwd^T y^_n) / s with the looked-up pairs
// y^_{n,2k:2k+2} = sigma_k C[idx_{n,k}].  R_fwd is orthogonal, so
//     Y[t][n] = <X_t, W^_n> = rho^_n <Xr_t, y^_n>,   Xr_t = R_fwd (X_t / s).
// The activations are rotated once (rotate_act_kernel, bf16 out); the matmul
// then needs per weight only an index unpack, a codebook lookup and a scale
// by sigma_k -- no inverse rotation -- and runs on bf16 MFMA.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Xr_t = R_fwd (X_t / s), rounded to bf16 (RNE).  One wavefront per window of
// 1024 columns, walking rows t = first, first + stride, ...; the window's
// column factors eps_j / (sqrt(b) s_j) are formed once per wavefront.
// ---------------------------------------------------------------------------
template <int L, typename Tin>
__global__ __launch_bounds__(kBlockThreads) void rotate_act_kernel(const Tin* __restrict__ X, int64_t ldx, int T,
                                                                   int d, const float* __restrict__ s,
                                                                   uint64_t seed, int row_groups,
                                                                   uint16_t* __restrict__ Xr, int64_t ldr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= nwin * row_groups) return;
  const int win = gw % nwin;
  const int first = gw / nwin;
  const int c = win * kWinChunks + lane;
  const bool active = c < nchunks;   // whole Hadamard blocks are active or not
  const float inv_sqrt_b = (float)(1.0 / sqrt((double)(1 << L)));
  float g[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = c * kChunk + i;
    g[i] = active ? sign_eps(seed, (uint32_t)j) * (inv_sqrt_b / (s ? s[j] : 1.0f)) : 0.0f;
  }
  const int co = win * kWinChunks + BlockOut<L>::chunk(lane);
  const float osign = BlockOut<L>::sign(lane);
  for (int t = first; t < T; t += row_groups) {
    float x[16];
    if (active) {
      RawChunk<Tin> raw;
      raw.load(X + (int64_t)t * ldx + c * kChunk);
      raw.unpack(x);
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] *= g[i];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.0f;
    }
    fwht_block<L>(x, lane);
    if (active) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = f32_to_bf16_bits(x[2 * i] * osign) | (f32_to_bf16_bits(x[2 * i + 1] * osign) << 16);
      uint4* out = reinterpret_cast<uint4*>(Xr + (int64_t)t * ldr + co * kChunk);
      out[0] = make_uint4(w[0], w[1], w[2], w[3]);
      out[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

// ---------------------------------------------------------------------------
// Y[t][n] = rho^_n sum_k Xr[t][k] y^[n][k] on v_mfma_f32_16x16x32_bf16.
//
// A workgroup (8 wavefronts) owns 16 output channels n0..n0+15 and 16 TT
// tokens; its wavefronts split the columns in super-steps of 64 columns (32
// pairs).  In a super-step lane l (g = l / 16) decodes the 8 pairs
// [32 ss + 8 g, +8) of row n0 + l % 16 -- one byte-aligned run of 8 B bits --
// into two bf16x8 B operands, and loads the matching 16 activation columns
// as two bf16x8 A operands per 16-token tile.  The MFMA's k slots are thereby
// a permutation of the columns, applied identically to A and B.  MFMA
// layout (16x16x32 bf16): lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16]; the result register r of lane l is
// C[4 (l / 16) + r][l % 16].  Partial sums of the 8 wavefronts are added in
// a fixed order through LDS, so results are deterministic.
// ---------------------------------------------------------------------------
// output element types
struct OutF32 {
  typedef float T;
  static __device__ void put(float* p, float v) { *p = v; }
};
struct OutBF16 {
  typedef uint16_t T;
  static __device__ void put(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }
};

constexpr int kMmThreads = 512;
constexpr int kMmWaves = kMmThreads / kWave;

template <int BT, int TT, typename Out>
__global__ __launch_bounds__(kMmThreads) void decode_matmul_kernel(
    const uint16_t* __restrict__ Xr, int T, int d, int64_t ldr, const uint32_t* __restrict__ packed,
    int row_words, const uint16_t* __restrict__ rho_f16, int N, const float* __restrict__ sigma,
    const float* __restrict__ codebook, int K, int Bdyn, typename Out::T* __restrict__ Y, int64_t ldy) {
  extern __shared__ float4 lds4[];
  float2* cb = reinterpret_cast<float2*>(lds4);                    // K centroids
  float* red = reinterpret_cast<float*>(cb + ((K + 1) & ~1));       // kMmWaves x TT x 256 partial sums

  for (int c = threadIdx.x; c < K; c += kMmThreads) cb[c] = make_float2(codebook[2 * c], codebook[2 * c + 1]);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;                 // k-slot group
  const int nl = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int t0 = blockIdx.y * 16 * TT;
  const int n = n0 + nl;
  const int B = BT ? BT : Bdyn;
  const int half_d = d >> 1;
  const int nsteps = (half_d + 31) / 32;
  const uint32_t* prow = packed + (int64_t)min(n, N - 1) * row_words;

  f32x4 acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int ss = wave; ss < nsteps; ss += kMmWaves) {
    const int p0 = ss * 32 + 8 * g;        // first of the lane's 8 pairs
    // ---- B: 8 looked-up pairs of row n (zeros past the row end or past N)
    float v[16];
    if (p0 < half_d && n < N) {
      const int bitstart = p0 * B;
      const int wstart = bitstart >> 5;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = prow[min(wstart + i, row_words - 1)];
      uint32_t idx[8];
      unpack8<BT>(w, (uint32_t)(bitstart & 31), Bdyn, idx);
      const float4* sp = reinterpret_cast<const float4*>(sigma + p0);   // p0 % 8 == 0, half_d % 8 == 0
      const float4 s0 = sp[0], s1 = sp[1];
      const float sg[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float2 cc = cb[min((int)idx[p], K - 1)];
        v[2 * p] = cc.x * sg[p];
        v[2 * p + 1] = cc.y * sg[p];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    bf16x8 b0, b1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b0[e] = (__bf16)v[e];
      b1[e] = (__bf16)v[8 + e];
    }
    // ---- A: columns [2 p0, 2 p0 + 16) of token t0 + 16 tt + nl, for each tile
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + 16 * tt + nl;
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
      if (t < T && p0 < half_d) {
        const uint4* ap = reinterpret_cast<const uint4*>(Xr + (int64_t)t * ldr + 2 * p0);
        a0 = ap[0];
        a1 = ap[1];
      }
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), b0, acc[tt], 0, 0, 0);
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), b1, acc[tt], 0, 0, 0);
    }
  }

  // ---- fixed-order sum over the wavefronts, scale by rho^_n, store
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * TT + tt) * 256 + (4 * g + r) * 16 + nl] = acc[tt][r];
  __syncthreads();
  for (int o = threadIdx.x; o < TT * 256; o += kMmThreads) {
    const int tt = o >> 8, tl = (o >> 4) & 15, nn = o & 15;
    const int t = t0 + 16 * tt + tl, col = n0 + nn;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kMmWaves; ++w) sum += red[(w * TT + tt) * 256 + tl * 16 + nn];
    if (t < T && col < N) Out::put(Y + (int64_t)t * ldy + col, sum * f16_bits_to_f32(rho_f16[col]));
  }
}

// ===========================================================================
// launchers
// ===========================================================================
template <int L>
struct LaunchRotateAct {
  static int run(const void* X, int32_t xdt, int T, int d, int64_t ldx, const float* s, uint64_t seed, uint16_t* Xr,
                 int64_t ldr, hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    // about 2048 wavefronts: each walks T / row_groups rows of one window
    int row_groups = (2048 + nwin - 1) / nwin;
    row_groups = row_groups < 1 ? 1 : (row_groups > T ? T : row_groups);
    const dim3 grid(grid_for_waves((int64_t)nwin * row_groups)), blk(kBlockThreads);
    if (xdt == QAMW_F32)
      hipLaunchKernelGGL((rotate_act_kernel<L, float>), grid, blk, 0, st, (const float*)X, ldx, T, d, s, seed,
                         row_groups, Xr, ldr);
    else
      hipLaunchKernelGGL((rotate_act_kernel<L, uint16_t>), grid, blk, 0, st, (const uint16_t*)X, ldx, T, d, s, seed,
                         row_groups, Xr, ldr);
    return check_launch("rotate_act_kernel");
  }
};

int launch_rotate_act(int L, const void* X, int32_t xdt, int T, int d, int64_t ldx, const float* s, uint64_t seed,
                      uint16_t* Xr, int64_t ldr, hipStream_t st) {
  return dispatch_L<LaunchRotateAct>(L, X, xdt, T, d, ldx, s, seed, Xr, ldr, st);
}

template <int BT, int TT>
static int launch_mm(const uint16_t* Xr, int T, int d, int64_t ldr, const uint32_t* packed, int row_words,
                     const uint16_t* rn, int N, const float* sigma, const float* cb, int K, int B, void* Y,
                     int32_t ydt, int64_t ldy, hipStream_t st) {
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((T + 16 * TT - 1) / (16 * TT))), blk(kMmThreads);
  const size_t lds = (size_t)((K + 1) & ~1) * sizeof(float2) + (size_t)kMmWaves * TT * 256 * sizeof(float);
  if (ydt == QAMW_F32)
    hipLaunchKernelGGL((decode_matmul_kernel<BT, TT, OutF32>), grid, blk, lds, st, Xr, T, d, ldr, packed, row_words,
                       rn, N, sigma, cb, K, B, (float*)Y, ldy);
  else
    hipLaunchKernelGGL((decode_matmul_kernel<BT, TT, OutBF16>), grid, blk, lds, st, Xr, T, d, ldr, packed,
                       row_words, rn, N, sigma, cb, K, B, (uint16_t*)Y, ldy);
  return check_launch("decode_matmul_kernel");
}

template <int BT>
static int launch_mm_tt(const uint16_t* Xr, int T, int d, int64_t ldr, const uint32_t* packed, int row_words,
                        const uint16_t* rn, int N, const float* sigma, const float* cb, int K, int B, void* Y,
                        int32_t ydt, int64_t ldy, hipStream_t st) {
  // token tiles per workgroup: one for T <= 16, up to four (64 tokens) sharing each decoded operand
  if (T <= 16) return launch_mm<BT, 1>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
  if (T <= 32) return launch_mm<BT, 2>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
  return launch_mm<BT, 4>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
}

int launch_decode_matmul(const uint16_t* Xr, int T, int d, int64_t ldr, const uint32_t* packed, int row_words,
                         const uint16_t* rn, int N, const float* sigma, const float* cb, int K, int B, void* Y,
                         int32_t ydt, int64_t ldy, hipStream_t st) {
  switch (B) {
    case 8: return launch_mm_tt<8>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
    case 10: return launch_mm_tt<10>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
    case 11: return launch_mm_tt<11>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
    case 12: return launch_mm_tt<12>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
    default: return launch_mm_tt<0>(Xr, T, d, ldr, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, ldy, st);
  }
}

}  // namespace qamw
