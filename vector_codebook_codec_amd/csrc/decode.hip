// Decode kernel: unpack, centroid lookup, inverse rotation, rescale, store
// ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
// Rotation and Activation-Aware Scaling"; Methodology: Decoding).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

// Decode tunables: rows whose packed words are loaded ahead, and wavefronts
// of work per CU the launch aims for (each wave then walks several rows).
constexpr int kDecodePrefetch = 3;
constexpr int kDecodeWavesPerCu = 20;
constexpr int kDecodeMaxRows = 16;   // rows per wavefront, at most

// ---------------------------------------------------------------------------
// Decode.  Each workgroup keeps one 1024-column window and walks rows with a
// stride (row n goes to workgroup (n / 4) mod blocks_per_window of its
// window, wave n mod 4), so the codebook and the window's column factors
// g_j = eps_j / (sqrt(b) s_j) are staged in LDS once per workgroup, with all
// prologue loads in flight together.  Each lane keeps its 8 sigma_k and 16
// factors in registers; the packed words (and fp16 norm) of the next
// kDecodePrefetch rows stay in flight in a ring of named register slots.  A
// wavefront has at most kDecodeMaxRows rows and walks them as straight-line
// code (see the walk below).
//
// The LDS codebook holds each centroid as (c_x + c_y, c_x - c_y): the first
// in-register butterfly of the inverse rotation acts on exactly the pair
// (y_2k, y_2k+1), so it is folded into the table and the transform starts
// at its second stage.  The row norm is folded into the pair scales.
// BT > 0 fixes the index width at compile time and pads the table to 2^BT
// entries, those past K repeating centroid K - 1, so any B-bit index reads
// inside it and indices >= K decode as K - 1 without a clamp instruction;
// BT = 0 takes the width B from the argument and clamps indices to K - 1.
// ---------------------------------------------------------------------------
// Five waves per SIMD (at most 102 VGPRs) with three rows in flight per wave
// measured a little faster than four waves with four rows in flight (blocks up
// to 256; the larger ones need more registers for their LDS-staged stores).
template <int L, int BT, typename Out>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(L <= 8 ? 5 : 1))) void decode_kernel(
    const uint32_t* packed, const uint16_t* rho_f16, int N, int d,
    const float* __restrict__ s, const float* __restrict__ sigma, uint64_t seed,
    const float* __restrict__ codebook, int K, int Bdyn, int row_words, int blocks_per_window,
    typename Out::T* __restrict__ out, int64_t ldo) {
  // packed and rho_f16 are deliberately not __restrict__: the output stores
  // then keep each ring-slot prefetch in the row that issues it (the compiler
  // may not move a load past a store that could alias it), instead of letting
  // it sink into the row that consumes it.
  // Blocks of up to 256 columns store straight from registers; larger ones
  // go through a 4 KB LDS buffer per wave.
  constexpr bool kDirect = L <= 8;
  extern __shared__ float4 lds4[];
  uint4* stage_all = reinterpret_cast<uint4*>(lds4);    // 4 waves x 256 x 16 bytes (LDS-staged stores only)
  u32x4* pk_all = reinterpret_cast<u32x4*>(stage_all + (kDirect ? 0 : kWavesPerBlock * 256));   // 4 waves x 64 x 16 bytes
  float* gwin = reinterpret_cast<float*>(pk_all + kWavesPerBlock * kWave);  // kWinChunks * kChunk factors
  float2* cb = reinterpret_cast<float2*>(gwin + kWinChunks * kChunk);

  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int win = blockIdx.x % nwin;
  const int rblk = blockIdx.x / nwin;               // 0 .. blocks_per_window-1
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = win * kWinChunks + lane;
  // Lanes past the row end hold zeros but stay: the window store reads back
  // columns for every lane of the wave.
  const bool active = c < nchunks;
  // rows of this wave: n = first + k * stride, k = 0 .. nrows-1
  const int first = rblk * kWavesPerBlock + wave;
  const int stride = blocks_per_window * kWavesPerBlock;
  const int nrows = first < N ? (N - first + stride - 1) / stride : 0;
  const int last = nrows > 0 ? nrows - 1 : 0;

  // ---- the first rows' loads go out before the LDS prologue, so their
  // latency overlaps it.  The window's packed bits are 16 B words
  // (512 pairs x B bits) starting at word win * 16 B of the row, 64-byte
  // aligned (rows are padded to 16 bytes): lane l loads the 16 bytes at word
  // win * 16 B + 4 l with one aligned load (lanes past the window's words or
  // the row's end reload its last 16 bytes), and at its turn the slot goes through the wave's
  // LDS slice so that each lane reads the 4 words holding its 8 indices.
  // Row loads are unconditional: rows past the wave's last reload its last
  // row.  Each ring slot also carries its row's fp16 norm (a uniform load),
  // so the row walk has no other global loads.
  const int B = BT ? BT : Bdyn;
  const int pbase = win * 16 * B;                   // first word of the window's bits
  const int64_t bitstart = (int64_t)c * kPairsPerLane * B;
  const uint32_t sh = (uint32_t)(bitstart & 31);
  // this lane's first word, relative to the window; lanes past the row end
  // read somewhere inside the slice (their results are never stored)
  const int wl0 = min((int)(bitstart >> 5) - pbase, 4 * kWave - 4);
  // this lane's 16-byte load; lanes past the window's 4 B words repeat the
  // last one (same address: no extra traffic)
  const int u4 = min(pbase / 4 + min(lane, 4 * B - 1), row_words / 4 - 1);
  u32x4 ring[kDecodePrefetch];         // packed words of the next rows, in flight
  uint16_t ring_rh[kDecodePrefetch];   // their row norms
  if (nrows > 0) {
#pragma unroll
    for (int q = 0; q < kDecodePrefetch; ++q) {
      const int n = first + min(q, last) * stride;
      ring[q] = reinterpret_cast<const u32x4*>(packed + (int64_t)n * row_words)[u4];
      ring_rh[q] = rho_f16[n];
    }
  }
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

  // ---- LDS prologue: codebook (sum/difference form, padded) and the
  // window's column factors
  {
    const float4* cb4 = reinterpret_cast<const float4*>(codebook);   // two centroids per float4
    float4* cbl = reinterpret_cast<float4*>(cb);
    const int npairs4 = K >> 1;
#pragma unroll 8
    for (int cc = threadIdx.x; cc < npairs4; cc += kBlockThreads) {
      const float4 t = cb4[cc];
      cbl[cc] = make_float4(t.x + t.y, t.x - t.y, t.z + t.w, t.z - t.w);
    }
    if ((K & 1) && threadIdx.x == 0) {
      const float cx = codebook[2 * (K - 1)], cy = codebook[2 * (K - 1) + 1];
      cb[K - 1] = make_float2(cx + cy, cx - cy);
    }
    if constexpr (BT > 0) {   // entries past K repeat centroid K - 1: the clamp, without an instruction
      const float cx = codebook[2 * (K - 1)], cy = codebook[2 * (K - 1) + 1];
      for (int cc = K + (int)threadIdx.x; cc < (1 << BT); cc += kBlockThreads) cb[cc] = make_float2(cx + cy, cx - cy);
    }
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
      gwin[t] = (j < d) ? sign_eps(seed, j) * col_scale(inv_sqrt_b, sv[q]) : 0.0f;
    }
  }
  __syncthreads();
  if (nrows == 0) return;                          // no barriers follow

  uint4* stage = stage_all + wave * 256;
  const int valid_cols = d - win * kWinChunks * kChunk;
  const int co_local = BlockOut<L>::chunk(lane);
  // first output column of this lane's direct stores
  const int e0 = 16 * BlockOut<L>::chunk(lane & (Out::kGroup - 1)) + (lane / Out::kGroup) * Out::kPiece;
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

  typename Out::T* out_win = out + win * kWinChunks * kChunk;
  // One copy of the row walk for full windows (stores without a per-lane
  // test) and one for the ragged last window, chosen once per workgroup.
  // A wave has at most kDecodeMaxRows rows (the launcher picks the stride),
  // and the walk is straight-line code: row k runs inside the test for row
  // k - 1, so every row has one path to it and the compiler's memory-counter
  // waits wait only for the ring slot being consumed, never for the stores
  // and prefetches issued after it.
  auto rows = [&](auto full) {
    constexpr bool kFull = decltype(full)::value;
    u32x4* pk = pk_all + wave * kWave;
    const uint32_t* pkw = reinterpret_cast<const uint32_t*>(pk) + wl0;
    auto row = [&](int q, int k) {
      const int n = first + k * stride;
      wave_lds_fence();
      pk[lane] = ring[q];
      wave_lds_fence();
      const uint32_t w[4] = {pkw[0], pkw[1], pkw[2], pkw[3]};
      uint32_t idx[8];
      unpack8<BT>(w, sh, Bdyn, idx);
      const float rh = f16_bits_to_f32(ring_rh[q]);
      {   // this slot now takes row k + kDecodePrefetch (or the last row again)
        const int nn = first + min(k + kDecodePrefetch, last) * stride;
        ring[q] = reinterpret_cast<const u32x4*>(packed + (int64_t)nn * row_words)[u4];
        ring_rh[q] = rho_f16[nn];
      }
      float x[16];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float2 cc = cb[BT ? (int)idx[p] : min((int)idx[p], K - 1)];
        const float f = sg[p] * rh;
        x[2 * p] = cc.x * f;
        x[2 * p + 1] = cc.y * f;
      }
      fwht_block<L, 2>(x, lane);
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] *= g[i];
      if constexpr (kDirect)
        Out::template direct<kFull>(x, e0, out_win + (int64_t)n * ldo, valid_cols);
      else
        Out::template store<kFull>(stage, lane, co_local, x, out_win + (int64_t)n * ldo, valid_cols);
    };
    auto walk = [&](auto self, auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < kDecodeMaxRows) {
        if (k < nrows) {
          row(k % kDecodePrefetch, k);
          self(self, std::integral_constant<int, k + 1>());
        }
      }
    };
    walk(walk, std::integral_constant<int, 0>());
  };
  if (valid_cols >= kWinChunks * kChunk)
    rows(std::integral_constant<bool, true>());
  else
    rows(std::integral_constant<bool, false>());
}

// ===========================================================================
// launchers
// ===========================================================================
template <int L, int BT>
int launch_decode_bt(const uint32_t* packed, const uint16_t* rho_f16, int N, int d, const float* s,
                     const float* sigma, uint64_t seed, const float* cb, int K, int B, int row_words, void* out,
                     int32_t odt, int64_t ldo, hipStream_t st) {
  const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
  const size_t lds = (size_t)kWavesPerBlock * ((L <= 8 ? 0 : 256) + kWave) * 16 + (size_t)kWinChunks * kChunk * sizeof(float) +
                     (size_t)(BT ? (1 << BT) : K) * sizeof(float2);
  // Persistent-style grid: every workgroup keeps one window (codebook and
  // column factors loaded once) and walks rows with a stride.  Aim for the
  // workgroups that fit on the chip at once (LDS-limited, at most
  // kDecodeWavesPerCu / 4 per CU), unless that would give a wave more
  // than kDecodeMaxRows rows: then the stride grows and the grid runs in
  // several rounds.
  int64_t per_cu = (int64_t)(160 * 1024 / lds);
  const int64_t cap = kDecodeWavesPerCu / kWavesPerBlock;
  per_cu = per_cu < 1 ? 1 : (per_cu > cap ? cap : per_cu);
  int64_t bpw = 256 * per_cu / nwin;
  const int64_t need = (N + kWavesPerBlock - 1) / kWavesPerBlock;   // one row per wave at most
  const int64_t min_bpw = (N + kWavesPerBlock * kDecodeMaxRows - 1) / (kWavesPerBlock * kDecodeMaxRows);
  bpw = bpw < min_bpw ? min_bpw : bpw;
  bpw = bpw < 1 ? 1 : (bpw > need ? need : bpw);
  if ((N + bpw * kWavesPerBlock - 1) / (bpw * kWavesPerBlock) > kDecodeMaxRows)
    return fail(QAMW_EUNSUPPORTED, "decode: %d rows need more than %d rows per wavefront", N, kDecodeMaxRows);
  const int blocks_per_window = (int)bpw;
  const int64_t blocks = (int64_t)nwin * blocks_per_window;
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
