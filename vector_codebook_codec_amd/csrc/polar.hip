// Polar-code baseline encode: the joint encode's transform with amplitude and
// phase of each normalised pair quantised independently ("QAM-W: Joint 2D
// Codebook Quantization for LLM Weights via Hadamard Rotation and
// Activation-Aware Scaling"; Methodology: Joint 2D Quantization, and the
// Experiments' joint-versus-polar ablation).
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "qamw.h"
#include "qamw_device.h"
#include "qamw_internal.h"
#include "encode_window.h"

namespace qamw {

// ---------------------------------------------------------------------------
// Polar code (the pages' joint-versus-polar ablation): amplitude and phase of
// each normalised pair quantised independently.  Same transform and packing
// as the joint encode; index = ia * Kp + ip with
//   r  = sqrt(x*x + y*y) in fp32, each operation rounded (sqrt correctly rounded)
//   ia = the first i minimising |r - a_i| over the ascending fp32 levels
//   ip = the first j maximising x c_j + y s_j over the fp32 unit directions.
// ia: with both levels' fp32 rule folded into squared thresholds (one per
// adjacent pair, computed by each workgroup), ia is the number of thresholds
// below x*x + y*y -- no square root per pair.  That equals the first-minimum
// rule while rounded differences to non-adjacent levels cannot tie, which
// holds for r below 2^21 times the smallest level gap; larger r (never seen
// from a normalised matrix) take the definition itself.  ip: an approximate
// atan2 (error < 1.2e-5 rad, far below half a sector for Kp <= 4096) gives
// q = phi Kp / 2 pi; the first maximum is sector j0 = round(q) or its
// neighbour on the side of q - j0 (directions farther away score lower by
// ~r (2 pi / Kp)^2, far above fp32 rounding).  Points with |z~|^2 < 1e-20,
// where scores could underflow, scan every direction.
// ---------------------------------------------------------------------------
// Squared decision threshold between adjacent levels lo < hi (both >= 0):
// the largest fp32 s such that r = sqrt(s) (correctly rounded) still picks
// lo under the fp32 rule fl(r - lo) <= fl(hi - r).  That rule is monotone in
// r, and sqrt is monotone in s, so for s = x^2 + y^2 the level index is the
// number of thresholds below s.  Found by stepping one ulp at a time from
// the midpoint and from its square (a few steps).
__device__ __forceinline__ float ulp_up(float t) { return __uint_as_float(__float_as_uint(t) + 1u); }
__device__ __forceinline__ float ulp_down(float t) { return t > 0.0f ? __uint_as_float(__float_as_uint(t) - 1u) : 0.0f; }
__device__ float polar_threshold_sq(float lo, float hi) {
  float t = (lo + hi) * 0.5f;
  for (int it = 0; it < 64 && ulp_up(t) - lo <= hi - ulp_up(t); ++it) t = ulp_up(t);
  for (int it = 0; it < 64 && !(t - lo <= hi - t); ++it) t = ulp_down(t);
  float sv = t * t;
  for (int it = 0; it < 64 && sqrtf(ulp_up(sv)) <= t; ++it) sv = ulp_up(sv);
  for (int it = 0; it < 64 && sqrtf(sv) > t; ++it) sv = ulp_down(sv);
  return sv;
}

constexpr int kPolarLinearLevels = 17;   // up to 16 thresholds are counted one by one

// atan2(y, x) to within 1.2e-5 rad: octant reduction to a = min/max in [0, 1]
// and the odd degree-9 polynomial of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 4.4.47 (|error| <= 1e-5 on [-1, 1]).  It
// only places a point among the phase sectors; the decision itself is made
// on exact fp32 inner products.
__device__ __forceinline__ float approx_atan2(float y, float x) {
  const float ax = fabsf(x), ay = fabsf(y);
  const float mx = fmaxf(ax, ay), mn = fminf(ax, ay);
  const float a = mx > 0.0f ? mn * __builtin_amdgcn_rcpf(mx) : 0.0f;
  const float a2 = a * a;
  float t = 0.0208351f;
  t = t * a2 - 0.0851330f;
  t = t * a2 + 0.1801410f;
  t = t * a2 - 0.3302995f;
  t = t * a2 + 0.9998660f;
  t *= a;
  t = (ay > ax) ? 1.5707963267948966f - t : t;
  t = (x < 0.0f) ? 3.1415926535897932f - t : t;
  return (y < 0.0f) ? -t : t;
}

constexpr int kPolarWgPerCu = 2;   // 4 wavefronts per SIMD

template <int L, typename Tin>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(4))) void encode_polar_kernel(
    const Tin* __restrict__ W, int64_t ldw, int N, int d, const float* __restrict__ f,
    const float* __restrict__ isig, const float* __restrict__ levels, int Ka, const float* __restrict__ dirs,
    int Kp, int B, int row_words, const double* __restrict__ rho, uint32_t* __restrict__ packed) {
  extern __shared__ float4 lds4[];
  float2* dv = reinterpret_cast<float2*>(lds4);                       // Kp directions
  float* lv = reinterpret_cast<float*>(dv + Kp);                       // Ka levels
  float* sq = lv + Ka;                                                 // Ka - 1 squared thresholds
  uint16_t* stage_all = reinterpret_cast<uint16_t*>(sq + Ka);
  __shared__ uint32_t gap_bits;                                        // smallest level gap (>= 0)
  if (threadIdx.x == 0) gap_bits = 0x7f800000u;                        // +inf
  for (int j = threadIdx.x; j < Kp; j += kEncThreads) dv[j] = make_float2(dirs[2 * j], dirs[2 * j + 1]);
  for (int i = threadIdx.x; i < Ka; i += kEncThreads) lv[i] = levels[i];
  __syncthreads();
  for (int i = threadIdx.x + 1; i < Ka; i += kEncThreads) {
    sq[i - 1] = polar_threshold_sq(lv[i - 1], lv[i]);
    atomicMin(&gap_bits, __float_as_uint(fmaxf(lv[i] - lv[i - 1], 0.0f)));
  }
  __syncthreads();
  // below r_safe = gap 2^21 the rounded differences r - a_j of non-adjacent
  // levels cannot tie, so counting thresholds is the first-minimum rule
  const float r_safe = __uint_as_float(gap_bits) * 2097152.0f;
  const float s_safe = r_safe * r_safe;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: window bookkeeping stays scalar
  uint16_t* stage = stage_all + wave * kWinPairs;
  const int nchunks = d >> 4;
  const int nwin = (nchunks + kWinChunks - 1) / kWinChunks;
  const int total = N * nwin;                      // fits in int (checked on the host)
  const int stride = gridDim.x * kEncWaves;
  int gw = blockIdx.x * kEncWaves + wave;
  if (gw >= total) return;                         // no barriers follow

  int n = gw / nwin, win = gw - (gw / nwin) * nwin;
  WinLoads<Tin> wl;
  load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
  const float sectors_per_radian = (float)Kp * 0.15915494309189535f;   // Kp / (2 pi)
  int ka_top = 1;                                  // largest power of two <= Ka - 1 thresholds
  while (2 * ka_top <= Ka - 1) ka_top *= 2;

  for (;;) {
    const bool active = win * kWinChunks + lane < nchunks;   // whole Hadamard blocks are active or not
    float zx[8], zy[8];
    const int co_local = window_transform<L>(wl, active, lane, zx, zy);
    const int n_cur = n, win_cur = win;
    const int gnext = gw + stride;
    {
      // the next window's loads stay in flight during the search; past the
      // end the last window is loaded again (unused), keeping them unconditional
      const int gl = min(gnext, total - 1);
      n = gl / nwin;
      win = gl - n * nwin;
      load_window<L>(wl, W, ldw, f, isig, rho, n, win, lane, nchunks);
    }
    // Each step below runs for all of the lane's pairs at once, LDS reads
    // first, without branches; the rare cases are wave-uniform fallbacks.
    float s2[kPairsPerLane];
    int ia[kPairsPerLane];
    bool big = false;
#pragma unroll
    for (int p = 0; p < kPairsPerLane; ++p) {
      s2[p] = zx[p] * zx[p] + zy[p] * zy[p];
      ia[p] = 0;
      big |= !(s2[p] <= s_safe);
    }
    // ---- amplitude: ia = number of squared thresholds below x^2 + y^2
    if (Ka <= kPolarLinearLevels) {
      for (int t = 0; t < Ka - 1; ++t) {
        const float th = sq[t];                    // same address in every lane: broadcast
#pragma unroll
        for (int p = 0; p < kPairsPerLane; ++p) ia[p] += (s2[p] > th) ? 1 : 0;
      }
    } else {
      for (int h = ka_top; h > 0; h >>= 1) {       // thresholds ascend; same trip count in every lane
        float th[kPairsPerLane];
#pragma unroll
        for (int p = 0; p < kPairsPerLane; ++p) th[p] = sq[min(ia[p] + h, Ka - 1) - 1];
#pragma unroll
        for (int p = 0; p < kPairsPerLane; ++p) {
          const int t = ia[p] + h;
          ia[p] = ((t <= Ka - 1) & (s2[p] > th[p])) ? t : ia[p];
        }
      }
    }
    if (__any(big)) {                              // |z~| dwarfs the level spacing: the definition itself
#pragma unroll
      for (int p = 0; p < kPairsPerLane; ++p) {
        if (!(s2[p] <= s_safe)) {
          const float r = sqrtf(s2[p]);
          float best = INFINITY;
          int bi = 0;
          for (int i2 = 0; i2 < Ka; ++i2) {
            const float dd = fabsf(r - lv[i2]);
            if (dd < best) { best = dd; bi = i2; }
          }
          ia[p] = bi;
        }
      }
    }
    // ---- phase: the sector estimate j0 and its neighbour on the side the
    // point leans to; the larger score wins, the lower index on a tie
    int ip[kPairsPerLane];
    bool tiny = false;
    {
      int ja[kPairsPerLane], jb[kPairsPerLane];
      float2 ua[kPairsPerLane], ub[kPairsPerLane];
#pragma unroll
      for (int p = 0; p < kPairsPerLane; ++p) {
        const float qv = approx_atan2(zy[p], zx[p]) * sectors_per_radian;   // in [-Kp/2, Kp/2]
        const float qr = rintf(qv);
        int j0 = (int)qr;
        j0 += (j0 < 0) ? Kp : 0;
        j0 = (j0 >= Kp) ? j0 - Kp : j0;
        const int jup = (j0 == Kp - 1) ? 0 : j0 + 1;
        const int jdn = (j0 == 0) ? Kp - 1 : j0 - 1;
        ja[p] = j0;
        jb[p] = (qv > qr) ? jup : jdn;
        ua[p] = dv[ja[p]];
        ub[p] = dv[jb[p]];
      }
#pragma unroll
      for (int p = 0; p < kPairsPerLane; ++p) {
        const float x = zx[p], y = zy[p];
        const float sa = x * ua[p].x + y * ua[p].y;
        const float sb = x * ub[p].x + y * ub[p].y;
        const bool take = (sb > sa) | ((sb == sa) & (jb[p] < ja[p]));
        ip[p] = take ? jb[p] : ja[p];
        tiny |= !(s2[p] >= 1e-20f);
      }
    }
    if (__any(tiny)) {                             // scores could underflow: every direction
#pragma unroll
      for (int p = 0; p < kPairsPerLane; ++p) {
        if (!(s2[p] >= 1e-20f)) {
          const float x = zx[p], y = zy[p];
          float best = -INFINITY;
          int bj = 0;
          for (int j2 = 0; j2 < Kp; ++j2) {
            const float2 uu = dv[j2];
            const float sc = x * uu.x + y * uu.y;
            if (sc > best) { best = sc; bj = j2; }
          }
          ip[p] = bj;
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kPairsPerLane; ++p) stage[co_local * kPairsPerLane + p] = (uint16_t)(ia[p] * Kp + ip[p]);
    wave_lds_fence();
    pack_window(stage, lane, win_cur, nwin, d >> 1, B, row_words, packed + (int64_t)n_cur * row_words);
    gw = gnext;
    if (gw >= total) break;
    wave_lds_fence();                              // the stage is rewritten next round
  }
}

// ===========================================================================
// launcher
// ===========================================================================
template <int L>
struct LaunchEncodePolar {
  static int run(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const float* isig,
                 const float* levels, int Ka, const float* dirs, int Kp, int B, int row_words, const double* rho,
                 uint32_t* packed, hipStream_t st) {
    const int nwin = (d / 16 + kWinChunks - 1) / kWinChunks;
    const int64_t waves = (int64_t)N * nwin;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return fail(QAMW_EHIP, "cannot query the device's compute units");
    const dim3 grid((unsigned)std::min<int64_t>((waves + kEncWaves - 1) / kEncWaves, (int64_t)cus * kPolarWgPerCu)),
        blk(kEncThreads);
    const size_t lds = (size_t)Kp * sizeof(float2) + (size_t)2 * Ka * sizeof(float) +
                       (size_t)kEncWaves * kWinPairs * sizeof(uint16_t);
    if (wdt == QAMW_F32)
      hipLaunchKernelGGL((encode_polar_kernel<L, float>), grid, blk, lds, st, (const float*)W, ldw, N, d, f, isig,
                         levels, Ka, dirs, Kp, B, row_words, rho, packed);
    else
      hipLaunchKernelGGL((encode_polar_kernel<L, uint16_t>), grid, blk, lds, st, (const uint16_t*)W, ldw, N, d, f,
                         isig, levels, Ka, dirs, Kp, B, row_words, rho, packed);
    return check_launch("encode_polar_kernel");
  }
};

int launch_encode_polar(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f,
                        const float* isig, const float* levels, int Ka, const float* dirs, int Kp, int B,
                        int row_words, const double* rho, uint32_t* packed, hipStream_t st) {
  return dispatch_L<LaunchEncodePolar>(L, W, wdt, N, d, ldw, f, isig, levels, Ka, dirs, Kp, B, row_words, rho,
                                       packed, st);
}


}  // namespace qamw
