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

__device__ __forceinline__ double row_normaliser(double rho, int L) {
  const double den = rho * sqrt((double)(1 << L));
  return den > 0.0 ? 1.0 / den : 0.0;
}

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
  double rho;
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
// fp32 (0 for rho_n = 0).  Inactive lanes (past the row's last chunk) give 0.
template <int L, typename Tin>
__device__ __forceinline__ int window_transform(const WinLoads<Tin>& w, bool active, int lane, float zx[8],
                                                float zy[8]) {
  float x[16];
  w.raw.unpack(x);
  const float fc[16] = {w.fc[0].x, w.fc[0].y, w.fc[0].z, w.fc[0].w, w.fc[1].x, w.fc[1].y, w.fc[1].z, w.fc[1].w,
                        w.fc[2].x, w.fc[2].y, w.fc[2].z, w.fc[2].w, w.fc[3].x, w.fc[3].y, w.fc[3].z, w.fc[3].w};
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = active ? x[i] * fc[i] : 0.0f;
  fwht_block<L>(x, lane);
  const int co_local = BlockOut<L>::chunk(lane);   // the lane now holds (sign *) chunk co_local
  const float osign = BlockOut<L>::sign(lane);
  const double inv_row = row_normaliser(w.rho, L);
  const float is[8] = {w.is[0].x, w.is[0].y, w.is[0].z, w.is[0].w, w.is[1].x, w.is[1].y, w.is[1].z, w.is[1].w};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const float inv = (float)(inv_row * (double)(active ? is[p] : 0.0f)) * osign;
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

}  // namespace qamw
