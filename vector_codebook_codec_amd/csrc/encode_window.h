// Per-window building blocks shared by the encode kernels (joint, polar) and
// the codebook refinement: a wavefront owns a 1024-column window of one row,
// a lane 16 columns (8 pairs) ("QAM-W: Joint 2D Codebook Quantization for
// LLM Weights via Hadamard Rotation and Activation-Aware Scaling";
// Methodology: Separation of Scale and Direction, Deterministic Rotation,
// Pairing and Calibration).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qamw_device.h"
#include "qamw_internal.h"

namespace qamw {

constexpr int kEncThreads = 512;                       // 8 wavefronts per workgroup
constexpr int kEncWaves = kEncThreads / kWave;

// Everything one lane reads for one (row, window): its 16 weights, their
// column factors eps_j s_j, 1 / sigma of the 8 pairs it holds after the
// rotation, and the row norm.  load_window issues every load unconditionally
// from clamped, valid addresses (lanes past the row's last chunk reload the
// last chunk and are zeroed by the transform), so a wavefront can keep the
// next window's loads in flight with exact wait counts.
template <typename Tin>
struct WinLoads {
  RawChunk<Tin> raw;
  float4 fc[4];
  float4 is[2];
  double rho;   // the row factor 1 / (sqrt(b) rho_n) (0 for rho_n = 0)
};

template <int L, typename Tin>
__device__ __forceinline__ void load_window(WinLoads<Tin>& w, const Tin* __restrict__ W, int64_t ldw,
                                            const float* __restrict__ f, const float* __restrict__ isig,
                                            const double* __restrict__ rho, int n, int win, int lane, int nchunks) {
  const int c = min(win * kWinChunks + lane, nchunks - 1);
  const int co = min(win * kWinChunks + BlockOut<L>::chunk(lane), nchunks - 1);
  w.raw.load(W + (int64_t)n * ldw + c * kChunk);
  const float4* fp = reinterpret_cast<const float4*>(f + c * kChunk);
#pragma unroll
  for (int v = 0; v < 4; ++v) w.fc[v] = fp[v];
  const float4* ip = reinterpret_cast<const float4*>(isig + co * kPairsPerLane);
  w.is[0] = ip[0];
  w.is[1] = ip[1];
  w.rho = rho[n];
}

// Rotate the lane's 16 columns and normalise: on return the lane holds the
// normalised pairs z~ of window chunk co_local (8 pairs), z~ = y / sigma_k
// with y = H_b (f . w) / (sqrt(b) rho_n); each pair's factor
// (1 / (sqrt(b) rho_n)) * (1 / sigma_k) is formed in fp64 and rounded once to
// fp32 (0 for rho_n = 0).  Inactive lanes (past the row's last chunk) give 0
// (NaN where the chunk they copied holds a non-finite weight).  With
// kScale = 2 the lane gets 2 z~ instead, exactly (the factor is doubled in
// fp64 before its one rounding; doubling commutes with every rounding).
template <int L, typename Tin, int kScale = 1>
__device__ __forceinline__ int window_transform(const WinLoads<Tin>& w, bool active, int lane, float zx[8],
                                                float zy[8]) {
  float x[16];
  w.raw.unpack(x);
  const float fc[16] = {w.fc[0].x, w.fc[0].y, w.fc[0].z, w.fc[0].w, w.fc[1].x, w.fc[1].y, w.fc[1].z, w.fc[1].w,
                        w.fc[2].x, w.fc[2].y, w.fc[2].z, w.fc[2].w, w.fc[3].x, w.fc[3].y, w.fc[3].z, w.fc[3].w};
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] *= fc[i];   // lanes past the row end: a copy of the last chunk, zeroed below
  fwht_block<L>(x, lane);
  const int co_local = BlockOut<L>::chunk(lane);   // the lane now holds (sign *) chunk co_local
  const float osign = BlockOut<L>::sign(lane);
  // the lane's sign and activity folded into the row factor once: a sign
  // flip commutes with the rounding, and inactive lanes get 0 (their pairs
  // are 0, or NaN where the copied chunk holds Inf or NaN; whole Hadamard
  // blocks are active or not, so they never mix with active lanes, and every
  // caller discards their indices)
  const double inv_row = active ? w.rho * (double)osign : 0.0;
  const float is[8] = {w.is[0].x, w.is[0].y, w.is[0].z, w.is[0].w, w.is[1].x, w.is[1].y, w.is[1].z, w.is[1].w};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const float inv = (float)(inv_row * (double)is[p] * (double)kScale);
    zx[p] = x[2 * p] * inv;
    zy[p] = x[2 * p + 1] * inv;
  }
  return co_local;
}

// Pack the window's 512 indices (stage[k] = index of window pair k) into
// whole words: a window owns words [16 B win, 16 B (win + 1)) of its row
// because 512 B is a multiple of 32; the last window also writes the row's
// zero padding.
__device__ __forceinline__ void pack_window(const uint16_t* stage, int lane, int win, int nwin, int half_d, int B,
                                            int row_words, uint32_t* __restrict__ row_out) {
  const int npairs = min(kWinPairs, half_d - win * kWinPairs);
  const int word0 = win * 16 * B;
  const int nwords = (win == nwin - 1) ? row_words - word0 : 16 * B;
  uint32_t* out = row_out + word0;
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
// Packing from registers.  A lane's 8 indices are those of the 8 consecutive
// pairs of window chunk co, i.e. bits [8 B co, 8 B co + 8 B) of the window's
// stream: exactly bytes [B co, B co + B).  stage_lane_bytes writes them into
// the wavefront's 64 B-byte stage (dword writes for B = 8..11, bytes below); store_stage then writes the window's
// 16 B words from it with 16-byte stores (the last window of a row stops at
// row_words; lanes past the row end must have staged zero indices, which are
// the row's zero padding bits).
// ---------------------------------------------------------------------------
template <int BT>
__device__ __forceinline__ void stage_lane_bytes_t(uint8_t* __restrict__ stage, int co, const uint32_t idx[8]) {
  constexpr int B = BT;
  static_assert(B >= 8 && B <= 11, "8 B bits span at most four dwords");
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int pos = p * B, wd = pos >> 5, sh = pos & 31;
    w[wd] |= idx[p] << sh;
    if (sh + B > 32) w[wd + 1] |= idx[p] >> (32 - sh);
  }
  // The lane's bits start at byte B co: byte t of dword j0.  Shifted into
  // place they are d0..d3 (v_perm selects the bytes of (w_k : w_(k-1)) >>
  // (32 - 8 t)).  A dword shared with the previous lane (t > 0: that lane
  // wrote its low bytes, zeros above) is OR-ed in after every lane's plain
  // writes; every other dword the lane touches it owns alone.
  const uint32_t bc = (uint32_t)(B * co), t = bc & 3u, j0 = bc >> 2;
  const uint32_t sel = 0x07060504u - t * 0x01010101u;
  const uint32_t d0 = __builtin_amdgcn_perm(w[0], 0u, sel), d1 = __builtin_amdgcn_perm(w[1], w[0], sel),
                 d2 = __builtin_amdgcn_perm(w[2], w[1], sel), d3 = __builtin_amdgcn_perm(0u, w[2], sel);
  const uint32_t last = (8u * t + 8u * B - 1u) >> 5;   // the last dword touched, relative to j0 (1..3)
  uint32_t* s32 = reinterpret_cast<uint32_t*>(stage) + j0;
  s32[1] = d1;
  if (last >= 2u) s32[2] = d2;
  if (last == 3u) s32[3] = d3;
  if (t == 0u) s32[0] = d0;
  wave_lds_fence();                                  // the plain writes of every lane first
  if (t != 0u) __hip_atomic_fetch_or(s32, d0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

__device__ __forceinline__ void stage_lane_bytes(uint8_t* __restrict__ stage, int co, const uint32_t idx[8], int B) {
  switch (B) {
    case 11: stage_lane_bytes_t<11>(stage, co, idx); return;
    case 10: stage_lane_bytes_t<10>(stage, co, idx); return;
    case 9: stage_lane_bytes_t<9>(stage, co, idx); return;
    case 8: stage_lane_bytes_t<8>(stage, co, idx); return;
    default: break;
  }
  // other widths (B <= 7): 8 B <= 56 bits fit one 64-bit word
  uint64_t v = 0;
  for (int p = 0; p < 8; ++p) v |= (uint64_t)idx[p] << (p * B);
  uint8_t* dst = stage + B * co;
  for (int b = 0; b < B; ++b) dst[b] = (uint8_t)(v >> (8 * b));
}

__device__ __forceinline__ void store_stage(const uint8_t* __restrict__ stage, int lane, int win, int B, int row_words,
                                            uint32_t* __restrict__ row_out) {
  const int word0 = win * 16 * B;                      // a multiple of 16 B: 16-byte aligned
  const int nvec = min(4 * B, (row_words - word0) >> 2);
  if (lane < nvec)
    reinterpret_cast<uint4*>(row_out + word0)[lane] = reinterpret_cast<const uint4*>(stage)[lane];
}

}  // namespace qamw
