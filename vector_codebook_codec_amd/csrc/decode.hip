// Decode kernel: unpack, centroid lookup, inverse rotation, rescale, store
// ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Decoding).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

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
// launchers
// ===========================================================================
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

int launch_decode(int L, const uint32_t* packed, const uint16_t* rho_f16, int N, int d, const float* s,
                  const float* sigma, uint64_t seed, const float* cb, int K, int B, int row_words, void* out,
                  int32_t odt, int64_t ldo, hipStream_t st) {
  return dispatch_L<LaunchDecode>(L, packed, rho_f16, N, d, s, sigma, seed, cb, K, B, row_words, out, odt, ldo, st);
}

}  // namespace qamw
