// Device-side building blocks of the QAM-W kernels for gfx950 (CDNA4).
//
// Work decomposition shared by every kernel: a row of d columns is cut into
// 16-column "chunks"; one lane of a 64-wide wavefront owns one chunk (16
// consecutive elements = 8 consecutive pairs), and one wavefront owns a
// "window" of 64 consecutive chunks (1024 columns, 512 pairs) of one row.  A
// Hadamard block of b = 2^L columns therefore spans b/16 adjacent lanes, which
// always sit inside one wavefront (16 <= b <= 1024), so the whole rotation is
// done in registers: 4 butterfly stages inside each lane, then L-4 stages
// across lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qamw {

constexpr int kWave = 64;          // wavefront width on CDNA
constexpr int kChunk = 16;         // elements per lane
constexpr int kPairsPerLane = 8;
constexpr int kWinChunks = 64;     // chunks per window (one per lane)
constexpr int kWinPairs = kWinChunks * kPairsPerLane;  // 512

// ---------------------------------------------------------------------------
// Sign mask.  eps_j = -1 exactly when bit 63 of the j-th SplitMix64 output
// (0-based) is set.  Counter form of the generator (Steele, Lea & Flood 2014):
// the j-th output mixes seed + (j + 1) * gamma with the variant-13 finaliser;
// its last xor-shift by 31 leaves bit 63 unchanged, so it is skipped.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sign_eps(uint64_t seed, uint32_t j) {
  uint64_t z = seed + (uint64_t)(j + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (z >> 63) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// Loads / stores of one 16-element chunk (16-byte aligned).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ void load_chunk(const float* __restrict__ p, float x[16]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float4 t = q[v];
    x[4 * v + 0] = t.x; x[4 * v + 1] = t.y; x[4 * v + 2] = t.z; x[4 * v + 3] = t.w;
  }
}

__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ p, float x[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    uint4 t = q[v];
    uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * v + 2 * i + 0] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[8 * v + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

struct OutF32 {
  using T = float;
  static __device__ __forceinline__ void store(float* __restrict__ p, const float x[16]) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int v = 0; v < 4; ++v) q[v] = make_float4(x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]);
  }
};

struct OutBF16 {
  using T = uint16_t;
  static __device__ __forceinline__ void store(uint16_t* __restrict__ p, const float x[16]) {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = f32_to_bf16_bits(x[8 * v + 2 * i]) | (f32_to_bf16_bits(x[8 * v + 2 * i + 1]) << 16);
      q[v] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
};

struct OutF16 {
  using T = uint16_t;
  static __device__ __forceinline__ void store(uint16_t* __restrict__ p, const float x[16]) {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = f32_to_f16_bits(x[8 * v + 2 * i]) | (f32_to_f16_bits(x[8 * v + 2 * i + 1]) << 16);
      q[v] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
};

// ---------------------------------------------------------------------------
// Unnormalised Walsh-Hadamard transform (Sylvester order) of every block of
// 2^L elements held by the wavefront, block = b/16 adjacent lanes x 16
// registers.  Element i of a block lives in lane (i >> 4) of its lane group,
// register (i & 15); the result keeps that placement.  Requires 4 <= L <= 10.
//
// In-lane stages pair registers r and r ^ h.  Cross-lane stages pair lanes a
// and a ^ m; the lane whose bit m is set takes (partner - own), the other
// (own + partner), both as one fma with a +-1 factor.
// ---------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ void fwht_block(float x[16], int lane) {
  static_assert(L >= 4 && L <= 10, "block size must be 16..1024");
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < L - 4; ++t) {
    const int m = 1 << t;
    const float sgn = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __shfl_xor(x[i], m);
      x[i] = __builtin_fmaf(x[i], sgn, p);
    }
  }
}

// fp64 -> IEEE binary16 bits with one round-to-nearest-even step.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull) return (uint16_t)(sign | (a > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u));
  const int e = (int)(a >> 52) - 1023;
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  if (e < -25) return (uint16_t)sign;                       // below half the smallest subnormal
  const uint64_t m = (a & ((1ull << 52) - 1)) | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);         // bits dropped from the 53-bit significand
  uint64_t keep = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1ull))) ++keep;
  if (e >= -14) {
    uint32_t he = (uint32_t)(e + 15);
    if (keep == (1ull << 11)) { keep >>= 1; ++he; }
    if (he >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (he << 10) | (uint32_t)(keep & 0x3ffu));
  }
  return (uint16_t)(sign | (uint32_t)keep);                  // subnormal (0x400 carries into the exponent)
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

}  // namespace qamw
