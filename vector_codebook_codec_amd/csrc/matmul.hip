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

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
  sign_eps16(seed, (uint32_t)(c * kChunk), g);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = c * kChunk + i;
    g[i] = active ? g[i] * col_scale(inv_sqrt_b, s ? s[j] : 1.0f) : 0.0f;
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
        w[i] = pack_bf16x2(x[2 * i] * osign, x[2 * i + 1] * osign);
      uint4* out = reinterpret_cast<uint4*>(Xr + (int64_t)t * ldr + co * kChunk);
      out[0] = make_uint4(w[0], w[1], w[2], w[3]);
      out[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

// ---------------------------------------------------------------------------
// Y[t][n] = rho^_n sum_k Xr[t][k] y^[n][k] on v_mfma_f32_16x16x32_bf16.
//
// A workgroup (16 wavefronts; 8 for more than one token tile) owns 16 output channels n0..n0+15 and 16 TT
// tokens; its wavefronts split the columns in super-steps of 64 columns (32
// pairs), each loading the next super-step's operands while it works on the
// current one.  In a super-step lane l (g = l / 16) decodes the 8 pairs
// [32 ss + 8 g, +8) of row n0 + l % 16 -- one byte-aligned run of 8 B bits --
// into two bf16x8 B operands, and loads the matching 16 activation columns
// as two bf16x8 A operands per 16-token tile.  The MFMA's k slots are thereby
// a permutation of the columns, applied identically to A and B.  MFMA
// layout (16x16x32 bf16): lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16]; the result register r of lane l is
// C[4 (l / 16) + r][l % 16].  Partial sums of the wavefronts are added in
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

// wavefronts per workgroup: 16 for one token tile, 8 when more tiles need registers
template <int TT> constexpr int mm_waves() { return TT == 1 ? 16 : 8; }

// Global loads are coalesced: per super-step a wavefront loads the 16 rows'
// packed bits (the 16-byte-aligned 64 bytes covering each row's 4 B bytes),
// the 16 TT activation rows' 64 columns (128 bytes each) and the 32 sigma
// values, into a ring of D super-steps in registers.  When a super-step is
// consumed the wavefront moves it through a private LDS stage into the MFMA
// lane layout.  All loads of a super-step are issued together, in the order
// they are consumed, from clamped valid addresses (vector memory counters
// complete in order; a conditional load would make them unknown).
template <int TT>
struct MmLoads {       // plain vector members so the slots stay in registers
  u32x4 pk;            // packed row l / 4, 16-byte chunk l % 4 of the super-step's span
  u32x4 a[TT][2];      // activation row l / 4 (of tile tt), columns 16 (l % 4) .. + 16
  u32x4 sg;            // sigma of pairs 4 (l % 8) .. + 4
};
template <int TT> constexpr int mm_depth() { return TT == 1 ? 4 : 2; }
// stage rows are padded (packed rows 72 bytes, activation rows 144) so that the
// MFMA-layout reads of 16 rows fall in different LDS banks
constexpr int kStPkRow = 18;      // dwords
constexpr int kStARow = 144;      // bytes
template <int TT> constexpr int mm_stage_bytes() { return 16 * kStPkRow * 4 + 16 * TT * kStARow + 128; }

template <int BT, int TT, typename Out>
__global__ __launch_bounds__(mm_waves<TT>() * kWave) void decode_matmul_kernel(
    const uint16_t* __restrict__ Xr, int T, int d, int64_t ldr, const uint32_t* __restrict__ packed,
    int row_words, const uint16_t* __restrict__ rho_f16, int N, const float* __restrict__ sigma,
    const float* __restrict__ codebook, int K, int Bdyn, typename Out::T* __restrict__ Y, int64_t ldy) {
  constexpr int kMmWaves = mm_waves<TT>();
  constexpr int kMmThreads = kMmWaves * kWave;
  constexpr int D = mm_depth<TT>();
  extern __shared__ float4 lds4[];
  float2* cb = reinterpret_cast<float2*>(lds4);                    // K centroids
  float* red = reinterpret_cast<float*>(cb + ((K + 1) & ~1));       // kMmWaves x TT x 256 partial sums
  char* stage_all = reinterpret_cast<char*>(red + kMmWaves * TT * 256);

  for (int c = threadIdx.x; c < K; c += kMmThreads) cb[c] = make_float2(codebook[2 * c], codebook[2 * c + 1]);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: step bookkeeping stays scalar
  const int g = lane >> 4;                 // k-slot group (MFMA layout)
  const int nl = lane & 15;
  const int lr = lane >> 2, lq = lane & 3; // row and 16/32-byte chunk (load layout)
  const int n0 = blockIdx.x * 16;
  const int t0 = blockIdx.y * 16 * TT;
  const int B = BT ? BT : Bdyn;
  const int half_d = d >> 1;
  const int nsteps = (half_d + 31) / 32;
  char* stage = stage_all + wave * mm_stage_bytes<TT>();
  uint32_t* st_pk = reinterpret_cast<uint32_t*>(stage);                         // [16 rows][kStPkRow dwords]
  char* st_a = stage + 16 * kStPkRow * 4;                                       // [16 TT rows][kStARow bytes]
  float* st_sg = reinterpret_cast<float*>(st_a + 16 * TT * kStARow);           // [32]
  const u32x4* prow16 = reinterpret_cast<const u32x4*>(packed + (int64_t)min(n0 + lr, N - 1) * row_words);
  const int row_chunks = row_words >> 2;   // row_words % 4 == 0

  auto load = [&](int ss) __attribute__((always_inline)) {
    MmLoads<TT> m;
    const int abase16 = (ss * 4 * B) >> 4;                // first 16-byte chunk of the super-step's span
    m.pk = prow16[min(abase16 + lq, row_chunks - 1)];
#pragma clang loop unroll(full)
    for (int tt = 0; tt < TT; ++tt) {
      const int t = min(t0 + 16 * tt + lr, T - 1);
      const int col = min(64 * ss + 16 * lq, d - 16);
      const u32x4* ap = reinterpret_cast<const u32x4*>(Xr + (int64_t)t * ldr + col);
      m.a[tt][0] = ap[0];
      m.a[tt][1] = ap[1];
    }
    const int sp = min(32 * ss + 4 * (lane & 7), half_d - 4);
    m.sg = *reinterpret_cast<const u32x4*>(sigma + sp);
    return m;
  };

  f32x4 acc[TT];
#pragma clang loop unroll(full)
  for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // one sub-step: stage super-step ss (held in `slot`), reload the slot for
  // ss + D W, decode and multiply
  auto step = [&](MmLoads<TT>& slot, int ss) __attribute__((always_inline)) {
    // ---- through the stage into the MFMA layout
    {
      u32x2* pd = reinterpret_cast<u32x2*>(st_pk + lr * kStPkRow + 4 * lq);
      pd[0] = u32x2{slot.pk.x, slot.pk.y};
      pd[1] = u32x2{slot.pk.z, slot.pk.w};
    }
#pragma clang loop unroll(full)
    for (int tt = 0; tt < TT; ++tt) {
      u32x4* ad = reinterpret_cast<u32x4*>(st_a + (16 * tt + lr) * kStARow + 32 * lq);
      ad[0] = slot.a[tt][0];
      ad[1] = slot.a[tt][1];
    }
    if (lane < 8) reinterpret_cast<u32x4*>(st_sg)[lane] = slot.sg;
    wave_lds_fence();
    slot = load(ss + D * kMmWaves);

    const int p0 = ss * 32 + 8 * g;
    const int n = n0 + nl;
    float v[16];
    if (p0 < half_d && n < N) {
      const int bit = p0 * B - ((ss * 4 * B) >> 4) * 128;   // bit offset inside the row's staged 64 bytes
      const int w0 = bit >> 5;                               // <= 12 for B <= 12: w0 + 3 < 16
      uint32_t w[4];
#pragma clang loop unroll(full)
      for (int i = 0; i < 4; ++i) w[i] = st_pk[nl * kStPkRow + w0 + i];
      uint32_t idx[8];
      unpack8<BT>(w, (uint32_t)(bit & 31), Bdyn, idx);
      const float4 s0 = reinterpret_cast<const float4*>(st_sg)[2 * g];
      const float4 s1 = reinterpret_cast<const float4*>(st_sg)[2 * g + 1];
      const float sg[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma clang loop unroll(full)
      for (int p = 0; p < 8; ++p) {
        const float2 cc = cb[min((int)idx[p], K - 1)];
        v[2 * p] = cc.x * sg[p];
        v[2 * p + 1] = cc.y * sg[p];
      }
    } else {
#pragma clang loop unroll(full)
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    bf16x8 b0, b1;
#pragma clang loop unroll(full)
    for (int e = 0; e < 8; ++e) {
      b0[e] = (__bf16)v[e];
      b1[e] = (__bf16)v[8 + e];
    }
#pragma clang loop unroll(full)
    for (int tt = 0; tt < TT; ++tt) {
      // activation rows past T contribute zeros (their loads read row T - 1)
      const bool tin = t0 + 16 * tt + nl < T;
      const u32x4* as = reinterpret_cast<const u32x4*>(st_a + (16 * tt + nl) * kStARow + 32 * g);
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 a0 = tin ? as[0] : z, a1 = tin ? as[1] : z;
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), b0, acc[tt], 0, 0, 0);
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), b1, acc[tt], 0, 0, 0);
    }
    wave_lds_fence();                        // the stage is rewritten by the next sub-step
  };

  // D named ring slots: slot u holds super-step ss0 + u W.  Named variables
  // keep each slot in its own registers (moving in-flight loads between
  // registers would wait for them), and every path runs all D sub-steps (a
  // super-step past the end multiplies zeros) so the counters agree on every
  // path.
  static_assert(D >= 2 && D <= 4, "ring depth");
  // The prologue issues the slots' loads strictly in slot order (scheduling
  // barriers), so that at the loop head the oldest loads are slot 0's.
  MmLoads<TT> r0 = load(wave), r1, r2, r3;
  __builtin_amdgcn_sched_barrier(0);
  r1 = load(wave + kMmWaves);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (D > 2) r2 = load(wave + 2 * kMmWaves);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (D > 3) r3 = load(wave + 3 * kMmWaves);
  __builtin_amdgcn_sched_barrier(0);
  for (int ss0 = wave; ss0 < nsteps; ss0 += D * kMmWaves) {
    step(r0, ss0);
    step(r1, ss0 + kMmWaves);
    if constexpr (D > 2) step(r2, ss0 + 2 * kMmWaves);
    if constexpr (D > 3) step(r3, ss0 + 3 * kMmWaves);
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

// ---------------------------------------------------------------------------
// One token (T = 1): the same product as a GEMV, without MFMA.  y[n] =
// rho^_n sum_k (u_k.x C[idx_nk].x + u_k.y C[idx_nk].y) with u_k = sigma_k
// (xr_2k, xr_2k+1), all fp32.  Wavefront w of a workgroup owns the column
// slices w, w + W, ... of 512 pairs (lane l: pairs 8 l .. 8 l + 7 of the
// slice, one byte-aligned run of 8 B bits) for the workgroup's 8 rows.
//
// Memory: a slice's packed bits are 16 B words starting at word 16 B sl of
// the row, 64-byte aligned (rows are padded to 16 bytes), so each row's slice
// is fetched by one aligned 16-byte load per lane (lanes past the slice's
// 4 B loads, or past the row end, repeat the last one), and handed to the
// lanes through the wave's 1 KB LDS slice.  The first slice's packed loads
// are issued before the codebook is staged in LDS, so the two latencies
// overlap (rows longer than 16 slices load their later slices in turn); the
// slice's activations and sigma, shared by all workgroups and cache-resident,
// are loaded after the barrier, which keeps two workgroups per CU.  With
// the index width fixed at compile time the table is padded to 2^B entries
// repeating centroid K - 1, so indices >= K act as K - 1 without a clamp.
//
// Sums: each lane keeps its 8 rows' fp32 partials over all its slices; a
// reduce-scatter across the wavefront (halving the set of rows at each of
// the first three exchange steps) leaves row r's total in lanes 8 r .. 8 r + 7
// after 10 exchanges instead of 8 x 6; the wavefronts' totals are added in
// wavefront order through LDS.  Deterministic.
// ---------------------------------------------------------------------------
constexpr int kGvRows = 8;
constexpr int kGvSlice = 512;
constexpr int kGvMaxWaves = 16;

// Sum R per-lane values (one per row, R = 8 or 16) across the wavefront: a
// reduce-scatter that halves the set of rows at each exchange at distances
// 32, 16, ... until one row is left, then a butterfly over the lanes that
// share it.  Returns row `row`'s total, which lanes (64 / R) row .. + 64 / R
// - 1 hold (row = the lane's top log2(R) bits, taken in that order).  R - 1
// + log2(64 / R) exchanges instead of 6 R; fixed order, deterministic.
template <int R>
__device__ __forceinline__ float reduce_rows(const float acc[R], int lane, int& row) {
  static_assert(R == 8 || R == 16, "rows per reduction");
  float v[R];
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = acc[i];
  row = 0;
#pragma unroll
  for (int half = R / 2, dist = 32; half >= 1; half >>= 1, dist >>= 1) {
    const bool hi = (lane & dist) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = hi ? v[i] : v[i + half];
      const float keep = hi ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, dist);
    }
    row = 2 * row + (hi ? 1 : 0);
  }
  float t = v[0];
#pragma unroll
  for (int dist = 32 / R; dist >= 1; dist >>= 1) t += __shfl_xor(t, dist);
  return t;
}

struct GvLoads {
  uint4 xa, xb;            // 16 bf16 rotated activations
  float4 s0, s1;           // 8 sigma_k
  u32x4 rw[kGvRows];       // the rows' 16-byte pieces of the slice
};

template <int BT, typename Out>
__global__ __launch_bounds__(kGvMaxWaves * kWave) void decode_gemv_kernel(
    const uint16_t* __restrict__ Xr, int d, const uint32_t* __restrict__ packed, int row_words,
    const uint16_t* __restrict__ rho_f16, int N, const float* __restrict__ sigma,
    const float* __restrict__ codebook, int K, int Bdyn, typename Out::T* __restrict__ Y) {
  extern __shared__ float4 lds4[];
  const int kp = BT ? (1 << BT) : K;                                 // table entries
  float2* cb = reinterpret_cast<float2*>(lds4);
  u32x4* pk_all = reinterpret_cast<u32x4*>(cb + ((kp + 1) & ~1));   // [waves][64] 16-byte slots
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  float* part = reinterpret_cast<float*>(pk_all + nw * kWave);       // [waves][kGvRows]
  const int B = BT ? BT : Bdyn;
  const int half_d = d >> 1;
  const int nslices = (half_d + kGvSlice - 1) / kGvSlice;
  const int n0 = blockIdx.x * kGvRows;
  const int lane_u4 = min(lane, 4 * B - 1);
  const int last_u4 = row_words / 4 - 1;

  // unconditional loads from clamped addresses: the rows' packed pieces
  // (from HBM) and the slice's activations and sigma (small, cache-resident)
  auto load_packed = [&](int sl, GvLoads& g) {
    const int u4 = min(sl * 4 * B + lane_u4, last_u4);
#pragma unroll
    for (int r = 0; r < kGvRows; ++r)
      g.rw[r] = reinterpret_cast<const u32x4*>(packed + (int64_t)min(n0 + r, N - 1) * row_words)[u4];
  };
  auto load_x = [&](int sl, GvLoads& g) {
    const int p0 = min(sl * kGvSlice + 8 * lane, half_d - 8);
    g.xa = *reinterpret_cast<const uint4*>(Xr + 2 * p0);
    g.xb = *reinterpret_cast<const uint4*>(Xr + 2 * p0 + 8);
    g.s0 = *reinterpret_cast<const float4*>(sigma + p0);
    g.s1 = *reinterpret_cast<const float4*>(sigma + p0 + 4);
  };

  GvLoads cur;
  load_packed(wave, cur);                // wave < nw <= nslices

  {   // the codebook, padded: 2 centroids per float4
    const float4* cb4 = reinterpret_cast<const float4*>(codebook);
    float4* cbl = reinterpret_cast<float4*>(cb);
    for (int c = threadIdx.x; c < (K >> 1); c += blockDim.x) cbl[c] = cb4[c];
    if ((K & 1) && threadIdx.x == 0) cb[K - 1] = make_float2(codebook[2 * (K - 1)], codebook[2 * (K - 1) + 1]);
    if constexpr (BT > 0) {   // entries past K repeat centroid K - 1 (the clamp)
      const float2 last = make_float2(codebook[2 * (K - 1)], codebook[2 * (K - 1) + 1]);
      for (int c = K + (int)threadIdx.x; c < kp; c += blockDim.x) cb[c] = last;
    }
  }
  __syncthreads();

  u32x4* pk = pk_all + wave * kWave;
  const uint32_t lbit = (uint32_t)(8 * lane * B);        // the lane's first bit within the slice
  const uint32_t sh = lbit & 31u;
  const uint32_t* pkw = reinterpret_cast<const uint32_t*>(pk) + min((int)(lbit >> 5), 4 * kWave - 4);
  float rowacc[kGvRows];
#pragma unroll
  for (int r = 0; r < kGvRows; ++r) rowacc[r] = 0.0f;

  for (int sl = wave; sl < nslices; sl += nw) {
    if (sl != wave) load_packed(sl, cur);   // later slices (d > 16384 only): loaded in turn
    load_x(sl, cur);
    const bool act = sl * kGvSlice + 8 * lane < half_d;   // half_d % 8 == 0: all 8 pairs in or out
    float ux[8], uy[8];
    {
      const uint32_t xw[8] = {cur.xa.x, cur.xa.y, cur.xa.z, cur.xa.w, cur.xb.x, cur.xb.y, cur.xb.z, cur.xb.w};
      const float sg[8] = {cur.s0.x, cur.s0.y, cur.s0.z, cur.s0.w, cur.s1.x, cur.s1.y, cur.s1.z, cur.s1.w};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        ux[p] = act ? sg[p] * bf16_bits_to_f32(xw[p] & 0xffffu) : 0.0f;
        uy[p] = act ? sg[p] * bf16_bits_to_f32(xw[p] >> 16) : 0.0f;
      }
    }
#pragma unroll
    for (int r = 0; r < kGvRows; ++r) {
      wave_lds_fence();
      pk[lane] = cur.rw[r];
      wave_lds_fence();
      const uint32_t w[4] = {pkw[0], pkw[1], pkw[2], pkw[3]};
      uint32_t idx[8];
      unpack8<BT>(w, sh, Bdyn, idx);
      float acc = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float2 cc = cb[BT ? (int)idx[p] : min((int)idx[p], K - 1)];
        acc = __builtin_fmaf(ux[p], cc.x, acc);
        acc = __builtin_fmaf(uy[p], cc.y, acc);
      }
      rowacc[r] += acc;
    }
  }

  int myrow;
  const float v1 = reduce_rows<kGvRows>(rowacc, lane, myrow);
  if ((lane & (kWave / kGvRows - 1)) == 0) part[wave * kGvRows + myrow] = v1;
  __syncthreads();
  if ((int)threadIdx.x < kGvRows) {
    const int n = n0 + threadIdx.x;
    if (n < N) {
      float sum = 0.0f;
      for (int ww = 0; ww < nw; ++ww) sum += part[ww * kGvRows + threadIdx.x];
      Out::put(Y + n, sum * f16_bits_to_f32(rho_f16[n]));
    }
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
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((T + 16 * TT - 1) / (16 * TT))), blk(mm_waves<TT>() * kWave);
  const size_t lds = (size_t)((K + 1) & ~1) * sizeof(float2) + (size_t)mm_waves<TT>() * TT * 256 * sizeof(float) +
                     (size_t)mm_waves<TT>() * mm_stage_bytes<TT>();
  if (ydt == QAMW_F32)
    hipLaunchKernelGGL((decode_matmul_kernel<BT, TT, OutF32>), grid, blk, lds, st, Xr, T, d, ldr, packed, row_words,
                       rn, N, sigma, cb, K, B, (float*)Y, ldy);
  else
    hipLaunchKernelGGL((decode_matmul_kernel<BT, TT, OutBF16>), grid, blk, lds, st, Xr, T, d, ldr, packed,
                       row_words, rn, N, sigma, cb, K, B, (uint16_t*)Y, ldy);
  return check_launch("decode_matmul_kernel");
}

template <int BT>
static int launch_gemv(const uint16_t* Xr, int d, const uint32_t* packed, int row_words, const uint16_t* rn, int N,
                       const float* sigma, const float* cb, int K, int B, void* Y, int32_t ydt, hipStream_t st) {
  const int nslices = (d / 2 + kGvSlice - 1) / kGvSlice;
  const int nw = nslices < kGvMaxWaves ? nslices : kGvMaxWaves;
  const dim3 grid((unsigned)((N + kGvRows - 1) / kGvRows)), blk((unsigned)(nw * kWave));
  const int kp = BT ? (1 << BT) : K;
  const size_t lds = (size_t)((kp + 1) & ~1) * sizeof(float2) + (size_t)nw * kWave * 16 +
                     (size_t)nw * kGvRows * sizeof(float);
  if (ydt == QAMW_F32)
    hipLaunchKernelGGL((decode_gemv_kernel<BT, OutF32>), grid, blk, lds, st, Xr, d, packed, row_words, rn, N, sigma,
                       cb, K, B, (float*)Y);
  else
    hipLaunchKernelGGL((decode_gemv_kernel<BT, OutBF16>), grid, blk, lds, st, Xr, d, packed, row_words, rn, N, sigma,
                       cb, K, B, (uint16_t*)Y);
  return check_launch("decode_gemv_kernel");
}

template <int BT>
static int launch_mm_tt(const uint16_t* Xr, int T, int d, int64_t ldr, const uint32_t* packed, int row_words,
                        const uint16_t* rn, int N, const float* sigma, const float* cb, int K, int B, void* Y,
                        int32_t ydt, int64_t ldy, hipStream_t st) {
  // one token: the GEMV kernel
  if (T == 1) return launch_gemv<BT>(Xr, d, packed, row_words, rn, N, sigma, cb, K, B, Y, ydt, st);
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
