// Host-side interfaces shared by the translation units of libqamw.so:
// launch helpers of each stage, argument checks and error reporting.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qamw.h"

namespace qamw {

constexpr int kBlockThreads = 256;                   // 4 wavefronts per workgroup (most kernels)
constexpr int kWavesPerBlock = kBlockThreads / 64;
constexpr int kCalibRowsPerTile = 16;                // rows per amplitude partial sum
constexpr int kRmsRowsPerTile = 64;                  // activation rows per channel-RMS partial sum
constexpr int kOutputErrorTokens = 128;              // tokens per output-error workgroup
constexpr int kOutputErrorRows = 128;                // weight rows per output-error workgroup
constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;   // per-GPU workspace of qamw_encode_noalloc

// ---- errors (the message of the calling thread's last failure)
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* what);

// ---- small helpers
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
__host__ __device__ inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int elem_size(int32_t dt) { return dt == QAMW_F32 ? 4 : (dt == QAMW_BF16 || dt == QAMW_F16) ? 2 : 0; }
// Rows per calibration tile (one amplitude partial sum each).  Rows of 5 to
// 16 windows of 1024 columns are calibrated by one workgroup per CU (one
// wavefront per window), so more than kCalibTileTarget tiles would run in a
// second, mostly idle round of workgroups: there a tile grows to
// ceil(N / kCalibTileTarget) rows, a multiple of 4.  Every entry point takes
// its tiles from this one rule, so the fp32 partial sums, and sigma, agree
// bit for bit between them.
constexpr int64_t kCalibTileTarget = 256;
inline int calib_rows_per_tile(int64_t N, int64_t d) {
  const int64_t nwin = (d / 16 + 63) / 64;
  if (nwin <= 4 || nwin > 16) return kCalibRowsPerTile;
  const int64_t t = (N + kCalibTileTarget - 1) / kCalibTileTarget;
  return t <= kCalibRowsPerTile ? kCalibRowsPerTile : (int)((t + 3) / 4 * 4);
}
inline size_t calib_tiles(int64_t N, int64_t d) {
  const int64_t r = calib_rows_per_tile(N, d);
  return (size_t)((N + r - 1) / r);
}
inline unsigned grid_for_waves(int64_t waves) { return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

// Call Launch<L>::run(args...) for the Hadamard block size 2^L, 2 <= b <= 1024.
template <template <int> class Launch, typename... A>
int dispatch_L(int L, A&&... args) {
  switch (L) {
    case 1: return Launch<1>::run(args...);
    case 2: return Launch<2>::run(args...);
    case 3: return Launch<3>::run(args...);
    case 4: return Launch<4>::run(args...);
    case 5: return Launch<5>::run(args...);
    case 6: return Launch<6>::run(args...);
    case 7: return Launch<7>::run(args...);
    case 8: return Launch<8>::run(args...);
    case 9: return Launch<9>::run(args...);
    case 10: return Launch<10>::run(args...);
    default: return fail(QAMW_EUNSUPPORTED, "block size");
  }
}

// ---- nearest-centroid search plan (see plan.hip): a grid over [-kPlanR, kPlanR)^2
// and a coarse outer grid over [-kPlanR2, kPlanR2)^2, both centred on the origin.
// For K <= kLdsMaxK the inner grid is a table the encode kernel keeps in LDS
// (non-uniform cells, one 16-bit entry per cell, shared candidate lists); for
// larger K it is a uniform grid of per-cell records read from global memory.
constexpr int kPlanG = 512;                  // global inner grid (K > kLdsMaxK): cells per axis
constexpr float kPlanR = 5.0f;
constexpr int kPlanG2 = 128;                 // outer grid: cells per axis over [-kPlanR2, kPlanR2)
constexpr float kPlanR2 = 20.0f;
constexpr size_t kPlanHeaderBytes = 256;
constexpr size_t kPlanHeaderKOffset = 16;    // int32 K inside the header (plan.hip)
__host__ __device__ inline int plan_lmax(int K) { return K <= 2048 ? 8 : 16; }

// LDS table geometry.  Both axes share one map from kLdsBins equal bins over
// [-kPlanR, kPlanR) to cell coordinates; cells are whole runs of bins, widest
// far from the origin where centroids are sparse.  The plan's image is
// [bin -> cell map, u8 x kLdsBins][cell entries, u16 x G x G, padded to 16
// bytes][candidate lists, 4 x u16 each, lists_cap of them]; the encode kernel
// stages it into LDS in a layout of its own (below), and lists_cap is what
// fits there.
constexpr int kLdsMaxK = 2048;
constexpr int kLdsBins = 2048;
constexpr int kLdsMaxG = 255;                // the guard cell index G fits the u8 map
constexpr int kLdsThreads = 1024;            // one 16-wavefront workgroup per CU
constexpr int kLdsWaves = kLdsThreads / 64;
constexpr size_t kLdsBudget = 160 * 1024 - 1024;   // LDS bytes one encode workgroup may take
constexpr uint16_t kLdsScanAll = 0xFFFFu;    // cell entry: search the whole codebook
// The encode kernel's own LDS copy of the table: the map with one guard bin
// at each end (padded to 16 bytes), then the codebook (-cx, -cy) at 8 bytes
// per centroid, then the cells as a (G + 1) x (G + 1) array with a "scan all"
// guard row and column, then the records, then 16 packing stages.
constexpr size_t kLdsMapBytes = (kLdsBins + 2 + 15) / 16 * 16;
__host__ __device__ inline size_t lds_cell_bytes(int G) { return ((size_t)2 * (G + 1) * (G + 1) + 15) / 16 * 16; }
struct LdsGeometry {
  int G;                         // cells per axis (<= kLdsMaxG)
  int lists_cap;                 // list records the image holds
  size_t cells_off, lists_off;   // byte offsets inside the image
  size_t image_bytes;            // multiple of 16
  size_t stage_bytes;            // per-wavefront packing stage (64 B bytes)
  uint16_t edges[kLdsMaxG + 1];  // cell c covers bins [edges[c], edges[c + 1])
};
bool lds_geometry(int K, LdsGeometry* g);    // false when K > kLdsMaxK
inline bool plan_has_lds(int K) { return K >= 2 && K <= kLdsMaxK; }
size_t plan_outer_offset(int K);             // outer grid records
size_t plan_image_offset(int K);             // LDS image (K <= kLdsMaxK)
size_t plan_scratch_offset(int K);           // construction scratch (K <= kLdsMaxK)
size_t plan_bytes(int K);

// ---- stage launchers (enqueue on `st`, return a qamw_status)
int launch_scale(const float* r, float alpha, uint64_t seed, int d, float* s, float* f, hipStream_t st);
int launch_rownorm(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, double* rho,
                   uint16_t* rho_f16, hipStream_t st);
int launch_amplitude(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const double* rho,
                     float* partial, hipStream_t st);
int launch_norm_amplitude(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s,
                          const float* f, double* rho, uint16_t* rho_f16, float* partial, hipStream_t st);
int launch_sigma(const float* partial, int ntiles, int half_d, int N, float* sigma, float* isig, hipStream_t st);
int launch_encode_prepare(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, const float* sigma,
                          uint64_t seed, double* rho, uint16_t* rho_f16, float* f, float* isig, hipStream_t st);
int launch_encode(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const float* isig,
                  const float* cb, int K, int B, int row_words, const double* rho, const void* plan, uint32_t* packed,
                  hipStream_t st);
int launch_encode_polar(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f,
                        const float* isig, const float* levels, int Ka, const float* dirs, int Kp, int B,
                        int row_words, const double* rho, uint32_t* packed, hipStream_t st);
int launch_build_plan(const float* cb, int K, void* plan, hipStream_t st);
constexpr int kLloydMaxParts = 4096;                 // workgroups (fp64 partial sums) of one refinement round
int launch_lloyd_update(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f,
                        const float* isig, const double* rho, const uint32_t* packed, int row_words, int B,
                        const float* cb, int K, float* cb_out, double* distortion, unsigned long long* gacc,
                        double* partial, hipStream_t st);
int launch_channel_rms(const void* X, int32_t xdt, int T, int d, int64_t ldx, float* r, float* partial,
                       hipStream_t st);
int launch_output_error(const void* X, int32_t xdt, int T, int d, int64_t ldx, const void* W, int32_t wdt, int N,
                        int64_t ldw, const void* Wh, int32_t hdt, int64_t ldh, double* out, double* partial,
                        uint16_t* dWb, uint16_t* Xb, hipStream_t st);
int launch_rotate_act(int L, const void* X, int32_t xdt, int T, int d, int64_t ldx, const float* s, uint64_t seed,
                      uint16_t* Xr, int64_t ldr, hipStream_t st);
int launch_decode_matmul(const uint16_t* Xr, int T, int d, int64_t ldr, const uint32_t* packed, int row_words,
                         const uint16_t* rn, int N, const float* sigma, const float* cb, int K, int B, void* Y,
                         int32_t ydt, int64_t ldy, hipStream_t st);
int launch_decode(int L, const uint32_t* packed, const uint16_t* rho_f16, int N, int d, const float* s,
                  const float* sigma, uint64_t seed, const float* cb, int K, int B, int row_words, void* out,
                  int32_t odt, int64_t ldo, hipStream_t st);

}  // namespace qamw
