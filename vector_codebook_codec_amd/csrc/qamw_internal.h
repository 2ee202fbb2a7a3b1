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

// ---- errors (the message of the calling thread's last failure)
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* what);

// ---- small helpers
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int elem_size(int32_t dt) { return dt == QAMW_F32 ? 4 : (dt == QAMW_BF16 || dt == QAMW_F16) ? 2 : 0; }
inline size_t calib_tiles(int64_t N) { return (size_t)((N + kCalibRowsPerTile - 1) / kCalibRowsPerTile); }
inline unsigned grid_for_waves(int64_t waves) { return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

// Call Launch<L>::run(args...) for the Hadamard block size 2^L, 16 <= b <= 1024.
template <template <int> class Launch, typename... A>
int dispatch_L(int L, A&&... args) {
  switch (L) {
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

// ---- nearest-centroid search plan (see plan.hip): a fine grid and a coarse
// outer grid, both square and centred on the origin
constexpr int kPlanG = 512;                  // fine grid: cells per axis over [-kPlanR, kPlanR)
constexpr float kPlanR = 5.0f;
constexpr int kPlanG2 = 256;                 // outer grid: cells per axis over [-kPlanR2, kPlanR2)
constexpr float kPlanR2 = 40.0f;
constexpr size_t kPlanHeaderBytes = 256;
constexpr size_t kPlanHeaderKOffset = 16;    // int32 K inside the header (plan.hip)
__host__ __device__ inline int plan_lmax(int K) { return K <= 2048 ? 8 : 16; }
inline size_t plan_outer_offset(int K) {
  return kPlanHeaderBytes + (size_t)kPlanG * kPlanG * plan_lmax(K) * sizeof(uint16_t);
}
inline size_t plan_bytes(int K) {
  return plan_outer_offset(K) + (size_t)kPlanG2 * kPlanG2 * plan_lmax(K) * sizeof(uint16_t);
}

// ---- stage launchers (enqueue on `st`, return a qamw_status)
int launch_scale(const float* r, float alpha, uint64_t seed, int d, float* s, float* f, hipStream_t st);
int launch_rownorm(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, double* rho,
                   uint16_t* rho_f16, hipStream_t st);
int launch_amplitude(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* f, const double* rho,
                     float* partial, hipStream_t st);
int launch_norm_amplitude(int L, const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s,
                          const float* f, double* rho, uint16_t* rho_f16, float* partial, hipStream_t st);
int launch_sigma(const float* partial, int ntiles, int half_d, int N, float* sigma, float* isig, hipStream_t st);
int launch_encode_prepare(const void* W, int32_t wdt, int N, int d, int64_t ldw, const float* s, const float* sigma,
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
int launch_decode_matvec(int L, const void* X, int32_t xdt, int d, const float* s, uint64_t seed,
                         const uint32_t* packed, int row_words, const uint16_t* rn, int N, const float* sigma,
                         const float* cb, int K, int B, void* Y, int32_t ydt, hipStream_t st);
int launch_decode(int L, const uint32_t* packed, const uint16_t* rho_f16, int N, int d, const float* s,
                  const float* sigma, uint64_t seed, const float* cb, int K, int B, int row_words, void* out,
                  int32_t odt, int64_t ldo, hipStream_t st);

}  // namespace qamw
