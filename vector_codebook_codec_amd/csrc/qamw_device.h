// Device-side building blocks of the QAM-W kernels for gfx950 (CDNA4).
//
// Work decomposition shared by every kernel: a row of d columns is cut into
// 16-column "chunks"; one lane of a 64-wide wavefront owns one chunk (16
// consecutive elements = 8 consecutive pairs), and one wavefront owns a
// "window" of 64 consecutive chunks (1024 columns, 512 pairs) of one row.  A
// Hadamard block of b = 2^L >= 16 columns therefore spans b/16 adjacent lanes,
// which always sit inside one wavefront (b <= 1024), so the whole rotation is
// done in registers: 4 butterfly stages inside each lane, then L-4 stages
// across lanes; blocks of 2, 4 or 8 columns need only L in-lane stages (the
// row length is then still a multiple of 16).
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

// The same signs for the 16 consecutive columns j0 .. j0 + 15.  The counter
// advances by gamma per column, so only the first needs a multiply; of the
// last product only bit 63 is needed, the top bit of the high word of its low
// 64 bits: hi(xl cl) + xl ch + xh cl (mod 2^32) for x = (xh, xl), c = (ch, cl).
__device__ __forceinline__ void sign_eps16(uint64_t seed, uint32_t j0, float out[16]) {
  constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
  constexpr uint32_t kC2lo = 0x133111EBu, kC2hi = 0x94D049BBu;
  uint64_t ctr = seed + (uint64_t)(j0 + 1u) * kGamma;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint64_t z = (ctr ^ (ctr >> 30)) * 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    const uint32_t xl = (uint32_t)z, xh = (uint32_t)(z >> 32);
    const uint32_t hi = __umulhi(xl, kC2lo) + xl * kC2hi + xh * kC2lo;
    out[i] = (hi >> 31) ? -1.0f : 1.0f;
    ctr += kGamma;
  }
}

// 1 / (sqrt(b) s_j), the per-column factor of the decode side (decoded weight
// = rho^ (R_fwd^T y^) / s_j; rotated activations = R_fwd (x / s)).  A column
// with s_j = 0 (an input channel whose activations are all zero, so its
// weights never reach the output) gets 0: it decodes as 0 and its activations
// are dropped, instead of dividing by zero.
__device__ __forceinline__ float col_scale(float inv_sqrt_b, float s) { return s != 0.0f ? inv_sqrt_b / s : 0.0f; }

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

// A chunk as loaded, before conversion: lets a kernel issue the next chunk's
// load early and convert it later.
template <typename Tin> struct RawChunk;
template <> struct RawChunk<float> {
  float4 v[4];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  __device__ void load(const float* __restrict__ p) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = q[i];
  }
  __device__ void unpack(float x[16]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[4 * i + 0] = v[i].x; x[4 * i + 1] = v[i].y; x[4 * i + 2] = v[i].z; x[4 * i + 3] = v[i].w;
    }
  }
};
template <> struct RawChunk<uint16_t> {
  uint4 v[2];
  __device__ void zero() { v[0] = v[1] = make_uint4(0u, 0u, 0u, 0u); }
  __device__ void load(const uint16_t* __restrict__ p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    v[0] = q[0];
    v[1] = q[1];
  }
  __device__ void unpack(float x[16]) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * h + 2 * i + 0] = bf16_bits_to_f32(w[i] & 0xffffu);
        x[8 * h + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  }
};

// MFMA operand and accumulator vectors (v_mfma_f32_16x16x32_bf16)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even: one v_cvt_pk_bf16_f32 per two
// values (NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------------------
// Window-contiguous stores.  After the rotation lane l holds the 16 outputs
// of chunk co_l of its window.  Storing them straight from registers makes
// every store instruction scatter 16-byte pieces over the window; instead the
// wave writes its window (64 chunks) to an LDS buffer and reads it back so
// that store instruction v writes the window's v-th contiguous 64 x 16 bytes.
// 16-byte slots are XOR-swizzled so that both LDS passes spread over all bank
// groups.  The buffer is private to the wave; LDS operations of one wave
// complete in order, and the fences keep the compiler from reordering the
// cross-lane accesses.
// ---------------------------------------------------------------------------
// Output stores stream through L2: non-temporal.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16(void* dst, uint4 t) {
  const u32x4 v = {t.x, t.y, t.z, t.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
}

__device__ __forceinline__ int stage_slot(int chunk, int q) {  // q: 16-byte piece of the chunk (0..3)
  return chunk * 4 + (q ^ ((chunk >> 2) & 3));
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stage 16 fp32 outputs of chunk `co_local`, store the window contiguously.
// buf: 256 x 16 bytes of LDS private to the wave.  Columns at or beyond
// `valid_cols` (relative to the window start) are not written.
// kFull: the window is known to be whole (valid_cols >= 1024), no test.
template <bool kFull = false>
__device__ __forceinline__ void store_window_f32(uint4* buf, int lane, int co_local, const float x[16],
                                                float* __restrict__ dst, int valid_cols) {
  wave_lds_fence();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    buf[stage_slot(co_local, q)] = make_uint4(__float_as_uint(x[4 * q]), __float_as_uint(x[4 * q + 1]),
                                              __float_as_uint(x[4 * q + 2]), __float_as_uint(x[4 * q + 3]));
  wave_lds_fence();
  uint4 t[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {                 // all reads first: one LDS wait
    const int e = v * 256 + lane * 4;          // first column of this lane's piece
    t[v] = buf[stage_slot(e >> 4, (e >> 2) & 3)];
  }
  if (kFull || valid_cols >= kWinChunks * kChunk) {      // a full window: no per-lane test
#pragma unroll
    for (int v = 0; v < 4; ++v) store16(dst + v * 256 + lane * 4, t[v]);
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = v * 256 + lane * 4;
      if (e < valid_cols) store16(dst + e, t[v]);
    }
  }
}

// Same for 16-bit outputs (already packed two per word): 32 bytes per lane.
template <bool kFull = false>
__device__ __forceinline__ void store_window_b16(uint4* buf, int lane, int co_local, const uint32_t w[8],
                                                 uint16_t* __restrict__ dst, int valid_cols) {
  wave_lds_fence();
  buf[stage_slot(co_local, 0)] = make_uint4(w[0], w[1], w[2], w[3]);
  buf[stage_slot(co_local, 1)] = make_uint4(w[4], w[5], w[6], w[7]);
  wave_lds_fence();
  uint4 t[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int e = v * 512 + lane * 8;          // first column of this lane's piece
    t[v] = buf[stage_slot(e >> 4, (e >> 3) & 1)];
  }
  if (kFull || valid_cols >= kWinChunks * kChunk) {
#pragma unroll
    for (int v = 0; v < 2; ++v) store16(dst + v * 512 + lane * 8, t[v]);
  } else {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int e = v * 512 + lane * 8;
      if (e < valid_cols) store16(dst + e, t[v]);
    }
  }
}

// Stores straight from registers, for blocks of at most 256 columns (the
// lane network then stays inside lane bits 0..3).  Lane a holds columns
// 16 co(a) + r, r = 0..15, co(a) its output chunk.  v_permlane16_swap and
// v_permlane32_swap exchange halves of a register pair across lane bit 4 or
// 5, i.e. transpose one lane bit with one register bit.  For fp32, swapping
// lane bits 4, 5 with register bits 2, 3 leaves lane a holding, in registers
// 4v .. 4v+3, the four columns from 256 v + 16 co(a & 15) + 4 (a >> 4): each
// 16-byte store instruction writes 1 KB of the window contiguously.  For
// 16-bit outputs (word i = columns 2i, 2i+1) one swap of lane bit 5 with word
// bit 2 leaves words 4v .. 4v+3 holding the eight columns from
// 512 v + 16 co(a & 31) + 8 (a >> 5).  `e0` is that first column for v = 0.
//
// swap_halves32(a, b): lanes 32..63 of a and lanes 0..31 of b trade places
// (a[l + 32] <-> b[l], l < 32); swap_halves16 does the same between the odd
// 16-lane rows of a and the even rows of b (a[l + 16] <-> b[l], bit 4 of l clear).
__device__ __forceinline__ void swap_halves32(uint32_t& a, uint32_t& b) {
  const auto t = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = t[0];
  b = t[1];
}
__device__ __forceinline__ void swap_halves16(uint32_t& a, uint32_t& b) {
  const auto t = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = t[0];
  b = t[1];
}

template <bool kFull>
__device__ __forceinline__ void store_direct_f32(const float x[16], int e0, float* __restrict__ dst, int valid_cols) {
  uint32_t u[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) u[r] = __float_as_uint(x[r]);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if ((r & 4) == 0) swap_halves16(u[r], u[r + 4]);   // lane bit 4 <-> register bit 2
#pragma unroll
  for (int r = 0; r < 8; ++r) swap_halves32(u[r], u[r + 8]);   // lane bit 5 <-> register bit 3
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = v * 256 + e0;
    if (kFull || e < valid_cols) store16(dst + e, make_uint4(u[4 * v], u[4 * v + 1], u[4 * v + 2], u[4 * v + 3]));
  }
}

template <bool kFull>
__device__ __forceinline__ void store_direct_b16(uint32_t w[8], int e0, uint16_t* __restrict__ dst, int valid_cols) {
#pragma unroll
  for (int i = 0; i < 4; ++i) swap_halves32(w[i], w[i + 4]);   // lane bit 5 <-> word bit 2
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int e = v * 512 + e0;
    if (kFull || e < valid_cols) store16(dst + e, make_uint4(w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]));
  }
}

// Output types of the decode: `store` goes through the wave's LDS buffer
// (any block size), `direct` stores from registers (blocks up to 256).
// kGroup / kPiece give e0 = 16 co(lane & (kGroup - 1)) + (lane / kGroup) kPiece.
struct StageF32 {
  using T = float;
  static constexpr int kGroup = 16, kPiece = 4;
  template <bool kFull = false>
  static __device__ __forceinline__ void direct(const float x[16], int e0, float* dst, int valid_cols) {
    store_direct_f32<kFull>(x, e0, dst, valid_cols);
  }
  template <bool kFull = false>
  static __device__ __forceinline__ void store(uint4* buf, int lane, int co_local, const float x[16], float* dst,
                                               int valid_cols) {
    store_window_f32<kFull>(buf, lane, co_local, x, dst, valid_cols);
  }
};

struct StageBF16 {
  using T = uint16_t;
  static constexpr int kGroup = 32, kPiece = 8;
  template <bool kFull = false>
  static __device__ __forceinline__ void direct(const float x[16], int e0, uint16_t* dst, int valid_cols) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    store_direct_b16<kFull>(w, e0, dst, valid_cols);
  }
  template <bool kFull = false>
  static __device__ __forceinline__ void store(uint4* buf, int lane, int co_local, const float x[16], uint16_t* dst,
                                               int valid_cols) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    store_window_b16<kFull>(buf, lane, co_local, w, dst, valid_cols);
  }
};

struct StageF16 {
  using T = uint16_t;
  static constexpr int kGroup = 32, kPiece = 8;
  template <bool kFull = false>
  static __device__ __forceinline__ void direct(const float x[16], int e0, uint16_t* dst, int valid_cols) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = f32_to_f16_bits(x[2 * i]) | (f32_to_f16_bits(x[2 * i + 1]) << 16);
    store_direct_b16<kFull>(w, e0, dst, valid_cols);
  }
  template <bool kFull = false>
  static __device__ __forceinline__ void store(uint4* buf, int lane, int co_local, const float x[16], uint16_t* dst,
                                               int valid_cols) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = f32_to_f16_bits(x[2 * i]) | (f32_to_f16_bits(x[2 * i + 1]) << 16);
    store_window_b16<kFull>(buf, lane, co_local, w, dst, valid_cols);
  }
};

// ---------------------------------------------------------------------------
// Unnormalised Walsh-Hadamard transform (Sylvester order) of every block of
// b = 2^L elements held by the wavefront: a block is 2^(L-4) adjacent lanes
// x 16 registers, element i in lane (i >> 4) of the group, register i & 15.
//
// Register bits: four in-lane butterfly stages (registers r and r ^ h).
// Lane bits: one butterfly stage per lane bit, each a single DPP-fed FMA.
// DPP on gfx9 has no xor-4 / xor-8 lane pattern, so the lane stages pair
// lanes a and a ^ m for m in {1, 2, 7, 15} (quad_perm, quad_perm,
// row_half_mirror, row_mirror), then 16 and 32 (ds_bpermute) for b >= 512.
// These masks form a basis of the lane-index space; with "lower/upper"
// decided by the dual functionals lambda_i (parity(a & D_i), where
// parity(D_i & m_j) = [i == j]) each stage is an exact Walsh-Hadamard
// butterfly along one coordinate, so the network computes the Sylvester
// transform up to a known relabelling of lanes and a per-lane sign:
//
//   lane a ends up holding  sign(a) * out[16 * G(a) + r],  r = 0..15,
//   G(a) = XOR of D_i over the i with parity(a & D_i) = 1,
//   sign(a) = (-1)^parity(a & (D_0 ^ D_1 ^ ...)).
//
// Stage i computes own + c_a * partner with c_a = (-1)^lambda_i(a); the
// lanes with lambda_i(a) = 1 then hold the negated difference, which the
// per-lane sign above accounts for.
// ---------------------------------------------------------------------------
constexpr int kLaneMasks[6] = {1, 2, 7, 15, 16, 32};

constexpr int parity(int v) {
  int p = 0;
  while (v) { p ^= v & 1; v >>= 1; }
  return p;
}

// D_i for a network over NB lane bits (brute force over the 2^NB functionals).
constexpr int lane_dual(int NB, int i) {
  for (int D = 0; D < (1 << NB); ++D) {
    bool ok = true;
    for (int j = 0; j < NB; ++j) ok = ok && (parity(D & kLaneMasks[j]) == (i == j ? 1 : 0));
    if (ok) return D;
  }
  return -1;
}

constexpr int lane_sign_mask(int NB) {
  int m = 0;
  for (int i = 0; i < NB; ++i) m ^= lane_dual(NB, i);
  return m;
}

// G(a): index (in 16-element chunks, within the block) of the outputs lane a holds.
template <int NB, int I = 0>
__device__ __forceinline__ int lane_out_chunk(int a) {
  if constexpr (I < NB) {
    constexpr int D = lane_dual(NB, I);
    static_assert(D >= 0, "lane masks must form a basis");
    return ((__builtin_popcount(a & D) & 1) ? D : 0) ^ lane_out_chunk<NB, I + 1>(a);
  } else {
    return 0;
  }
}

template <int NB>
__device__ __forceinline__ float lane_out_sign(int a) {
  constexpr int M = lane_sign_mask(NB);
  return (__builtin_popcount(a & M) & 1) ? -1.0f : 1.0f;
}

// Partner value across lane bit 4 or 5 (b >= 512): ds_bpermute.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(M == 16 || M == 32, "DPP covers the other masks");
  return __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, v), M));
}

// x[r] += c * x[r] of the partner lane, for all 16 registers, as single
// v_fmac_f32 instructions with a DPP-routed src0.  The compiler does not fuse
// a DPP move into v_fmac, hence the inline assembly (ALU only).  A VALU write
// followed by a DPP read of the same VGPR needs two wait states: the leading
// s_nop covers the previous stage; inside the block each instruction reads a
// register last written 16 instructions earlier.
#define QAMW_DPP_FMAC16(CTRL, x, c)                                                                      \
  asm("s_nop 1\n"                                                                                         \
      "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"  \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),  \
        "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]),         \
        "+v"(x[15])                                                                                       \
      : "v"(c))

template <int I, int NB>
__device__ __forceinline__ void lane_stage(float x[16], int a) {
  if constexpr (I < NB) {
    constexpr int D = lane_dual(NB, I);
    constexpr int M = kLaneMasks[I];
    const float c = (__builtin_popcount(a & D) & 1) ? -1.0f : 1.0f;
    if constexpr (M == 1) {
      QAMW_DPP_FMAC16("quad_perm:[1,0,3,2]", x, c);
    } else if constexpr (M == 2) {
      QAMW_DPP_FMAC16("quad_perm:[2,3,0,1]", x, c);
    } else if constexpr (M == 7) {
      QAMW_DPP_FMAC16("row_half_mirror", x, c);
    } else if constexpr (M == 15) {
      QAMW_DPP_FMAC16("row_mirror", x, c);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(lane_xor<M>(x[r]), c, x[r]);
    }
    lane_stage<I + 1, NB>(x, a);
  }
}

// In-register stages plus the lane network; BlockOut says where each lane's
// outputs land.  `lane` is the lane index in the wavefront.  The stages
// commute, so a caller whose input already went through the in-register
// stages below H0 (pairs (x[2p], x[2p+1]) already replaced by their sum and
// difference, for H0 = 2) starts at H0.  Blocks of 2, 4 or 8 columns lie
// inside one lane's 16 registers: only the in-register stages below b run,
// and every lane keeps its own chunk.
template <int L, int H0 = 1>
__device__ __forceinline__ void fwht_block(float x[16], int lane) {
  static_assert(L >= 1 && L <= 10, "block size must be 2..1024");
  static_assert(H0 == 1 || H0 == 2, "first in-register stage");
  constexpr int kRegLimit = L < 4 ? (1 << L) : 16;   // in-register stages h < min(b, 16)
#pragma unroll
  for (int h = H0; h < kRegLimit; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  if constexpr (L > 4) lane_stage<0, L - 4>(x, lane & ((1 << (L - 4)) - 1));
}

// Block-relative placement of a lane's outputs after fwht_block<L>.
template <int L>
struct BlockOut {
  static constexpr int NB = L > 4 ? L - 4 : 0;
  // chunk index (within the wavefront window) holding this lane's outputs
  static __device__ __forceinline__ int chunk(int lane) {
    const int a = lane & ((1 << NB) - 1);
    return (lane - a) + lane_out_chunk<NB>(a);
  }
  static __device__ __forceinline__ float sign(int lane) { return lane_out_sign<NB>(lane & ((1 << NB) - 1)); }
};

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


// ---------------------------------------------------------------------------
// rho_n = sqrt(sum_j (W_nj s_j)^2) for one row, by one wavefront.  W_nj s_j
// is exact in fp64 (24-bit x 24-bit significands); squares and sums are fp64
// in a fixed order, so rho is deterministic and accurate to ~1e-16.  The
// order is by window (64 chunks, 1024 columns): lane l's share of window w is
// the FMA chain over the 16 squares of chunk 64 w + l, the window's share is
// their butterfly sum over the lanes (window_sum), and rho^2 adds the
// windows' shares in window order.  The fused calibration kernel, which has
// one wavefront per window, forms the same sum.
// Lane 0 writes the row factor (row_factor, below) and, when rho_f16 is
// given, rho_n's binary16 (RNE) bits.
// ---------------------------------------------------------------------------
// Sum over the wavefront, every lane getting the same bits, in VALU
// instructions only: inside each 16-lane row, DPP pairs lane i with i ^ 1,
// i ^ 2, then 7 - i within 8 lanes (half-row mirror) and 15 - i within 16
// (row mirror) -- each time two lanes whose partial sums are already equal
// across their groups, so a + b and b + a agree; then lane-half swaps
// (v_permlane16_swap, v_permlane32_swap) bring in the partner across lane
// bit 4 and 5.
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  // every lane reads a lane of its own row (quad permutes and mirrors), so
  // bound_ctrl never applies and the old value is not needed: no init move
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, 0xf, 0xf, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, 0xf, 0xf, true);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// v of lane l ^ 16 (kBit = 4) or l ^ 32 (kBit = 5)
template <int kBit>
__device__ __forceinline__ double partner_f64(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t lo2 = lo, hi2 = hi;
  // swap(x, x): the first result holds the partner in the upper half of each
  // pair of lane groups, the second in the lower half
  if constexpr (kBit == 4) {
    swap_halves16(lo, lo2);
    swap_halves16(hi, hi2);
  } else {
    swap_halves32(lo, lo2);
    swap_halves32(hi, hi2);
  }
  const bool upper = (lane >> kBit) & 1;
  const uint64_t r = upper ? (((uint64_t)hi << 32) | lo) : (((uint64_t)hi2 << 32) | lo2);
  return __longlong_as_double((long long)r);
}

__device__ __forceinline__ double window_sum(double v) {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  v += dpp_f64<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f64<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f64<0x141>(v);   // row_half_mirror
  v += dpp_f64<0x140>(v);   // row_mirror
  v += partner_f64<4>(v, lane);
  v += partner_f64<5>(v, lane);
  return v;
}

// The factor every pair of row n is scaled by before its nearest-centroid
// search: 1 / (sqrt(b) rho_n) in fp64 (0 for rho_n = 0), formed once per row
// by the kernel that computes rho_n.
__device__ __forceinline__ double row_factor(double rho, double sqrt_b) {
  const double den = rho * sqrt_b;
  return den > 0.0 ? 1.0 / den : 0.0;
}

// One chunk's share: sum of (x_i s_i)^2, i = 0..15, as an FMA chain from 0.
// The sign of s does not matter (the square of an exact product).
__device__ __forceinline__ double chunk_sumsq(const float x[16], const float sc[16]) {
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const double w = (double)x[i] * (double)sc[i];   // exact: a bf16/fp32 times an fp32
    acc = fma(w, w, acc);
  }
  return acc;
}

// Lane 0 writes the row factor 1 / (sqrt(b) rho_n) (fp64; 0 for rho_n = 0)
// that the transform scales the row's pairs by, and rho_n's binary16 bits.
template <typename Tin>
__device__ __forceinline__ void row_norm_wave(const Tin* __restrict__ W, int64_t ldw, int n, int d,
                                              const float* __restrict__ s, double sqrt_b,
                                              double* __restrict__ rowf, uint16_t* __restrict__ rho_f16) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const Tin* row = W + (int64_t)n * ldw;
  // one window is summed while the next one's loads are in flight; lanes
  // past the row end load nothing and add zero
  RawChunk<Tin> rw[2];
  RawChunk<float> rs[2];
  auto load = [&](int slot, int w) {
    const int c = w * kWinChunks + lane;
    if (w < nwin && c < nchunks) {
      rw[slot].load(row + c * kChunk);
      rs[slot].load(s + c * kChunk);
    } else {
      rw[slot].zero();
      rs[slot].zero();
    }
  };
  auto add = [&](int slot, double& total) {
    float x[16], sc[16];
    rw[slot].unpack(x);
    rs[slot].unpack(sc);
    total += window_sum(chunk_sumsq(x, sc));
  };
  double total = 0.0;
  load(0, 0);
  for (int w = 0; w < nwin; w += 2) {
    load(1, w + 1);
    add(0, total);
    if (w + 1 >= nwin) break;
    load(0, w + 2);
    add(1, total);
  }
  if (lane == 0) {
    const double r = sqrt(total);
    rowf[n] = row_factor(r, sqrt_b);
    if (rho_f16) rho_f16[n] = f64_to_f16_bits(r);
  }
}

// ---------------------------------------------------------------------------
// Eight B-bit indices from a lane's packed words: w[0..3] hold the bits from
// word floor(bitstart / 32) on, sh = bitstart mod 32; index p is bits
// [p B, p B + B) of the stream that starts at bit sh of w[0] (sh + 8 B <= 127
// bits, gathered into three words by alignbit).  BT > 0 fixes B at compile time.
// ---------------------------------------------------------------------------
template <int BT>
__device__ __forceinline__ void unpack8(const uint32_t w[4], uint32_t sh, int Bdyn, uint32_t idx[8]) {
  const int B = BT ? BT : Bdyn;
  const uint32_t mask = (1u << B) - 1u;
  // the lane's 8*B bits, starting at bit 0 of a[0]
  const uint32_t a[3] = {__builtin_amdgcn_alignbit(w[1], w[0], sh), __builtin_amdgcn_alignbit(w[2], w[1], sh),
                         __builtin_amdgcn_alignbit(w[3], w[2], sh)};
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int o = p * B;
    const int q = o >> 5;
    const uint32_t lo = (q == 0) ? a[0] : ((q == 1) ? a[1] : a[2]);
    const uint32_t hi = (q == 0) ? a[1] : ((q == 1) ? a[2] : 0u);
    idx[p] = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(o & 31)) & mask;
  }
}

}  // namespace qamw
