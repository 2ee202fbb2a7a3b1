// C ABI of libqamw.so (declared in include/qamw.h): argument validation on
// the host, then the stage launchers of calibrate.hip, encode.hip, plan.hip
// and decode.hip on the caller's stream.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>

#include <cstdio>
#include <mutex>
#include <string>

#include "qamw.h"
#include "qamw_internal.h"

namespace qamw {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QAMW_EHIP, "%s: %s", what, hipGetErrorString(e));
  return QAMW_OK;
}

int log2_exact(int64_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

int check_matrix(int64_t N, int64_t d, int32_t block, int* L) {
  if (N <= 0 || d <= 0) return fail(QAMW_EINVAL, "N and d must be positive (N=%lld d=%lld)", (long long)N, (long long)d);
  // every wavefront index (rows x 1024-column windows) must fit in an int
  if (N > kMaxDim || d > kMaxDim || N * ((d + 1023) / 1024) > (int64_t(1) << 30))
    return fail(QAMW_EUNSUPPORTED, "matrix too large");
  *L = log2_exact(block);
  if (*L < 1 || *L > 10) return fail(QAMW_EUNSUPPORTED, "block must be a power of two in [2, 1024] (got %d)", block);
  if (d % block) return fail(QAMW_EINVAL, "d=%lld is not a multiple of block=%d", (long long)d, block);
  // a lane owns 16 columns: with blocks under 16 the row must still be whole 16-column chunks
  if (d % 16) return fail(QAMW_EUNSUPPORTED, "d=%lld is not a multiple of 16", (long long)d);
  return QAMW_OK;
}

int check_weights(const void* W, int32_t wdt, int64_t d, int64_t ldw) {
  if (!W) return fail(QAMW_EINVAL, "W is NULL");
  if (wdt != QAMW_F32 && wdt != QAMW_BF16) return fail(QAMW_EUNSUPPORTED, "weight dtype %d not supported", wdt);
  if (ldw < d) return fail(QAMW_EINVAL, "ldw=%lld < d=%lld", (long long)ldw, (long long)d);
  if (!aligned16(W) || (ldw * elem_size(wdt)) % 16)
    return fail(QAMW_EINVAL, "W must be 16-byte aligned with 16-byte aligned rows");
  return QAMW_OK;
}

int check_codebook(const float* cb, int32_t K) {
  if (!cb) return fail(QAMW_EINVAL, "codebook is NULL");
  if (!aligned16(cb)) return fail(QAMW_EINVAL, "codebook must be 16-byte aligned");
  if (K < 2 || K > 4096) return fail(QAMW_EUNSUPPORTED, "K=%d outside [2, 4096]", K);
  return QAMW_OK;
}

// A search plan passed to an encode: NULL, or 256-byte aligned with at least
// plan_bytes(K) bytes (the kernels read that much of it).
int check_plan(const void* plan, size_t plan_size, int32_t K) {
  if (!plan) return QAMW_OK;
  if ((uintptr_t)plan & 255u) return fail(QAMW_EINVAL, "plan must be 256-byte aligned");
  if (plan_size < plan_bytes(K))
    return fail(QAMW_EWORKSPACE, "a plan for K=%d needs %zu bytes (got %zu)", (int)K, plan_bytes(K), plan_size);
  return QAMW_OK;
}

}  // namespace qamw

// ===========================================================================
// C ABI
// ===========================================================================
using namespace qamw;

extern "C" {

int32_t qamw_index_bits(int32_t K) {
  if (K < 2 || K > 4096) return -1;
  int32_t b = 0;
  while ((1 << b) < K) ++b;
  return b;
}

int64_t qamw_packed_row_words(int64_t d, int32_t K) {
  const int32_t B = qamw_index_bits(K);
  if (B < 0 || d <= 0 || (d & 1) || d > kMaxDim) return -1;
  const int64_t words = ((d / 2) * B + 31) / 32;
  return (words + 3) / 4 * 4;
}

size_t qamw_calibrate_workspace_bytes(int64_t N, int64_t d, int32_t block) {
  (void)block;
  if (N <= 0 || d <= 0 || N > kMaxDim || d > kMaxDim) return 0;
  return round_up((size_t)N * sizeof(double), 256) + round_up((size_t)d * sizeof(float), 256) +
         calib_tiles(N, d) * (size_t)(d / 2) * sizeof(float);
}

size_t qamw_encode_workspace_bytes(int64_t N, int64_t d) {
  if (N <= 0 || N > kMaxDim || d <= 0 || d > kMaxDim) return 0;
  return round_up((size_t)N * sizeof(double), 256) + round_up((size_t)d * sizeof(float), 256) +
         round_up((size_t)(d / 2) * sizeof(float), 256);
}

const char* qamw_status_string(int32_t status) {
  switch (status) {
    case QAMW_OK: return "ok";
    case QAMW_EINVAL: return "invalid argument";
    case QAMW_EUNSUPPORTED: return "unsupported argument";
    case QAMW_EHIP: return "HIP runtime error";
    case QAMW_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* qamw_last_error(void) { return g_last_error.c_str(); }

const char* qamw_version(void) { return "qamw 0.1 gfx950"; }

int32_t qamw_calibrate(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* chan_rms,
                       float alpha, int32_t block, uint64_t sign_seed, float* s_out, float* sigma_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if (!chan_rms || !s_out || !sigma_out) return fail(QAMW_EINVAL, "chan_rms, s_out and sigma_out must be non-NULL");
  if (!aligned16(s_out) || !aligned16(sigma_out)) return fail(QAMW_EINVAL, "s_out and sigma_out must be 16-byte aligned");
  if (!isfinite(alpha)) return fail(QAMW_EINVAL, "alpha must be finite");
  const size_t need = qamw_calibrate_workspace_bytes(N, d, block);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "calibrate needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  double* rho = (double*)workspace;
  float* fcol = (float*)((char*)workspace + round_up((size_t)N * sizeof(double), 256));
  float* partial = (float*)((char*)fcol + round_up((size_t)d * sizeof(float), 256));
  const int n = (int)N, dd = (int)d;
  if ((rc = launch_scale(chan_rms, alpha, sign_seed, dd, s_out, fcol, st))) return rc;
  if ((rc = launch_norm_amplitude(L, W, wdtype, n, dd, ldw, s_out, fcol, rho, nullptr, partial, st))) return rc;
  return launch_sigma(partial, (int)calib_tiles(N, d), dd / 2, n, sigma_out, nullptr, st);
}

size_t qamw_plan_bytes(int32_t K) {
  if (K < 2 || K > 4096) return 0;
  return plan_bytes(K);
}

int32_t qamw_build_plan(const float* codebook, int32_t K, void* plan, size_t plan_size, void* stream) {
  int rc = check_codebook(codebook, K);
  if (rc) return rc;
  if (!plan || ((uintptr_t)plan & 255u)) return fail(QAMW_EINVAL, "plan must be non-NULL and 256-byte aligned");
  if (plan_size < plan_bytes(K))
    return fail(QAMW_EWORKSPACE, "plan needs %zu bytes (got %zu)", plan_bytes(K), plan_size);
  return launch_build_plan(codebook, K, plan, (hipStream_t)stream);
}

struct EncodeWorkspace {
  double* rho;    // [N] fp64 row factors 1 / (sqrt(b) rho_n) (0 for rho_n = 0)
  float* f;       // [d] eps_j s_j
  float* isig;    // [d/2] 1 / sigma_k
};

static EncodeWorkspace encode_workspace(void* workspace, int64_t N, int64_t d) {
  char* ws = (char*)workspace;
  EncodeWorkspace e;
  e.rho = (double*)ws;
  ws += round_up((size_t)N * sizeof(double), 256);
  e.f = (float*)ws;
  ws += round_up((size_t)d * sizeof(float), 256);
  e.isig = (float*)ws;
  return e;
}

static int check_encode_workspace(const void* workspace, size_t workspace_bytes, int64_t N, int64_t d) {
  const size_t need = qamw_encode_workspace_bytes(N, d);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "encode needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  return QAMW_OK;
}

int32_t qamw_encode_prepare(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* s,
                            const float* sigma, int32_t block, uint64_t sign_seed, uint16_t* rownorm_f16,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if (!s || !sigma || !rownorm_f16) return fail(QAMW_EINVAL, "s, sigma and rownorm_f16 must be non-NULL");
  if (!aligned16(s) || !aligned16(sigma)) return fail(QAMW_EINVAL, "s and sigma must be 16-byte aligned");
  if ((rc = check_encode_workspace(workspace, workspace_bytes, N, d))) return rc;
  hipStream_t st = (hipStream_t)stream;
  const EncodeWorkspace e = encode_workspace(workspace, N, d);
  return launch_encode_prepare(L, W, wdtype, (int)N, (int)d, ldw, s, sigma, sign_seed, e.rho, rownorm_f16, e.f, e.isig,
                               st);
}

int32_t qamw_encode_indices(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, int32_t block,
                            const float* codebook, int32_t K, const void* plan, size_t plan_size, uint32_t* packed,
                            const void* workspace, size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!packed) return fail(QAMW_EINVAL, "packed must be non-NULL");
  if (!aligned16(packed)) return fail(QAMW_EINVAL, "packed must be 16-byte aligned");
  if ((rc = check_plan(plan, plan_size, K))) return rc;
  if ((rc = check_encode_workspace(workspace, workspace_bytes, N, d))) return rc;
  const EncodeWorkspace e = encode_workspace(const_cast<void*>(workspace), N, d);
  return launch_encode(L, W, wdtype, (int)N, (int)d, ldw, e.f, e.isig, codebook, (int)K, qamw_index_bits(K),
                       (int)qamw_packed_row_words(d, K), e.rho, plan, packed, (hipStream_t)stream);
}

int32_t qamw_encode(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* s,
                    const float* sigma, int32_t block, uint64_t sign_seed, const float* codebook, int32_t K,
                    const void* plan, size_t plan_size, uint32_t* packed, uint16_t* rownorm_f16, void* workspace,
                    size_t workspace_bytes, void* stream) {
  // validate everything before the first launch
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!s || !sigma || !packed || !rownorm_f16) return fail(QAMW_EINVAL, "s, sigma, packed and rownorm_f16 must be non-NULL");
  if (!aligned16(s) || !aligned16(sigma) || !aligned16(packed))
    return fail(QAMW_EINVAL, "s, sigma and packed must be 16-byte aligned");
  if ((rc = check_plan(plan, plan_size, K))) return rc;
  if ((rc = check_encode_workspace(workspace, workspace_bytes, N, d))) return rc;
  if ((rc = qamw_encode_prepare(W, wdtype, N, d, ldw, s, sigma, block, sign_seed, rownorm_f16, workspace,
                                workspace_bytes, stream)))
    return rc;
  return qamw_encode_indices(W, wdtype, N, d, ldw, block, codebook, K, plan, plan_size, packed, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The no-allocation encode keeps qamw_encode's workspace (row norms, column
// factors, 1 / sigma) in this file-scope device array instead of a caller
// buffer.  Each GPU holds its own copy until the process ends; its device
// address is looked up once per device (hipGetSymbolAddress, with the device
// current) and every later call on that device uses that address.  All calls
// on one GPU share the array: calls that overlap on one GPU (different
// streams, or host threads) race and must be ordered by the caller.  Nothing
// in it has to start at zero: the encode writes every byte it reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QAMW_EHIP, "cannot query the current device for the no-allocation scratch");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(QAMW_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QAMW_OK;
}
}  // namespace

extern "C" {

size_t qamw_encode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int32_t qamw_encode_noalloc(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* s,
                            const float* sigma, int32_t block, uint64_t sign_seed, const float* codebook, int32_t K,
                            const void* plan, size_t plan_size, uint32_t* packed, uint16_t* rownorm_f16,
                            void* stream) {
  // the size limit first (host only), then everything qamw_encode checks
  const size_t need = qamw_encode_workspace_bytes(N, d);
  if (need > kNoAllocScratchBytes)
    return fail(QAMW_EUNSUPPORTED,
                "the no-allocation encode holds %zu bytes of workspace per GPU; N=%lld d=%lld needs %zu "
                "(use qamw_encode with a workspace)",
                kNoAllocScratchBytes, (long long)N, (long long)d, need);
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!s || !sigma || !packed || !rownorm_f16) return fail(QAMW_EINVAL, "s, sigma, packed and rownorm_f16 must be non-NULL");
  if (!aligned16(s) || !aligned16(sigma) || !aligned16(packed))
    return fail(QAMW_EINVAL, "s, sigma and packed must be 16-byte aligned");
  if ((rc = check_plan(plan, plan_size, K))) return rc;
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return qamw_encode(W, wdtype, N, d, ldw, s, sigma, block, sign_seed, codebook, K, plan, plan_size, packed,
                     rownorm_f16, ws, kNoAllocScratchBytes, stream);
}

size_t qamw_calibrate_encode_workspace_bytes(int64_t N, int64_t d) {
  const size_t e = qamw_encode_workspace_bytes(N, d);
  if (!e) return 0;
  return e + calib_tiles(N, d) * (size_t)(d / 2) * sizeof(float);
}

int32_t qamw_calibrate_prepare(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                               const float* chan_rms, float alpha, int32_t block, uint64_t sign_seed, float* s_out,
                               float* sigma_out, uint16_t* rownorm_f16, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if (!chan_rms || !s_out || !sigma_out || !rownorm_f16)
    return fail(QAMW_EINVAL, "chan_rms, s_out, sigma_out and rownorm_f16 must be non-NULL");
  if (!aligned16(s_out) || !aligned16(sigma_out)) return fail(QAMW_EINVAL, "s_out and sigma_out must be 16-byte aligned");
  if (!isfinite(alpha)) return fail(QAMW_EINVAL, "alpha must be finite");
  const size_t need = qamw_calibrate_encode_workspace_bytes(N, d);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "calibrate_prepare needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  const EncodeWorkspace e = encode_workspace(workspace, N, d);
  float* partial = (float*)((char*)workspace + qamw_encode_workspace_bytes(N, d));
  const int n = (int)N, dd = (int)d;
  // the calibration pass leaves exactly what qamw_encode_prepare would compute:
  // column factors (scale_kernel), row norms with their fp16 bits
  // (norm_amplitude_kernel) and 1 / sigma (sigma_kernel)
  if ((rc = launch_scale(chan_rms, alpha, sign_seed, dd, s_out, e.f, st))) return rc;
  if ((rc = launch_norm_amplitude(L, W, wdtype, n, dd, ldw, s_out, e.f, e.rho, rownorm_f16, partial, st))) return rc;
  return launch_sigma(partial, (int)calib_tiles(N, d), dd / 2, n, sigma_out, e.isig, st);
}

int32_t qamw_calibrate_encode(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                              const float* chan_rms, float alpha, int32_t block, uint64_t sign_seed,
                              const float* codebook, int32_t K, const void* plan, size_t plan_size, float* s_out,
                              float* sigma_out, uint32_t* packed, uint16_t* rownorm_f16, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!chan_rms || !s_out || !sigma_out || !packed || !rownorm_f16)
    return fail(QAMW_EINVAL, "chan_rms, s_out, sigma_out, packed and rownorm_f16 must be non-NULL");
  if (!aligned16(s_out) || !aligned16(sigma_out) || !aligned16(packed))
    return fail(QAMW_EINVAL, "s_out, sigma_out and packed must be 16-byte aligned");
  if (!isfinite(alpha)) return fail(QAMW_EINVAL, "alpha must be finite");
  if ((rc = check_plan(plan, plan_size, K))) return rc;
  const size_t need = qamw_calibrate_encode_workspace_bytes(N, d);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "calibrate_encode needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  if ((rc = qamw_calibrate_prepare(W, wdtype, N, d, ldw, chan_rms, alpha, block, sign_seed, s_out, sigma_out,
                                   rownorm_f16, workspace, workspace_bytes, stream)))
    return rc;
  const EncodeWorkspace e = encode_workspace(workspace, N, d);
  return launch_encode(L, W, wdtype, (int)N, (int)d, ldw, e.f, e.isig, codebook, (int)K, qamw_index_bits(K),
                       (int)qamw_packed_row_words(d, K), e.rho, plan, packed, (hipStream_t)stream);
}

size_t qamw_lloyd_workspace_bytes(int32_t K) {
  if (K < 2 || K > 4096) return 0;
  return round_up((size_t)3 * K * sizeof(unsigned long long), 256) + round_up((size_t)kLloydMaxParts * sizeof(double), 256) +
         round_up((size_t)2 * K * sizeof(float), 256);
}

int32_t qamw_lloyd_update(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, int32_t block,
                          const uint32_t* packed, const float* codebook, int32_t K, const void* enc_workspace,
                          size_t enc_workspace_bytes, float* codebook_out, double* distortion_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!packed || !aligned16(packed)) return fail(QAMW_EINVAL, "packed must be non-NULL and 16-byte aligned");
  if (!codebook_out || !aligned16(codebook_out)) return fail(QAMW_EINVAL, "codebook_out must be non-NULL and 16-byte aligned");
  if (codebook_out == codebook) return fail(QAMW_EINVAL, "codebook_out must not be the input codebook");
  if (!distortion_out || ((uintptr_t)distortion_out & 7u)) return fail(QAMW_EINVAL, "distortion_out must be non-NULL and 8-byte aligned");
  if ((rc = check_encode_workspace(enc_workspace, enc_workspace_bytes, N, d))) return rc;
  const size_t need = qamw_lloyd_workspace_bytes(K);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "lloyd update needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  const EncodeWorkspace e = encode_workspace(const_cast<void*>(enc_workspace), N, d);
  unsigned long long* gacc = (unsigned long long*)workspace;
  double* partial = (double*)((char*)workspace + round_up((size_t)3 * K * sizeof(unsigned long long), 256));
  return launch_lloyd_update(L, W, wdtype, (int)N, (int)d, ldw, e.f, e.isig, e.rho, packed,
                             (int)qamw_packed_row_words(d, K), qamw_index_bits(K), codebook, (int)K, codebook_out,
                             distortion_out, gacc, partial, (hipStream_t)stream);
}

int32_t qamw_learn_codebook(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, int32_t block,
                            const void* enc_workspace, size_t enc_workspace_bytes, const float* codebook_init,
                            int32_t K, int32_t iters, float* codebook_out, double* distortion_out, void* plan,
                            size_t plan_size, uint32_t* packed, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if ((rc = check_codebook(codebook_init, K))) return rc;
  if (iters < 1) return fail(QAMW_EINVAL, "iters must be >= 1 (got %d)", (int)iters);
  if (!codebook_out || !aligned16(codebook_out) || codebook_out == codebook_init)
    return fail(QAMW_EINVAL, "codebook_out must be non-NULL, 16-byte aligned and not the initial codebook");
  if (!distortion_out || ((uintptr_t)distortion_out & 7u)) return fail(QAMW_EINVAL, "distortion_out must be non-NULL and 8-byte aligned");
  if (!packed || !aligned16(packed)) return fail(QAMW_EINVAL, "packed must be non-NULL and 16-byte aligned");
  if (!plan || ((uintptr_t)plan & 255u) || plan_size < plan_bytes(K))
    return fail(QAMW_EWORKSPACE, "plan must be 256-byte aligned with %zu bytes", plan_bytes(K));
  if ((rc = check_encode_workspace(enc_workspace, enc_workspace_bytes, N, d))) return rc;
  const size_t need = qamw_lloyd_workspace_bytes(K);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "learn_codebook needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  hipStream_t st = (hipStream_t)stream;
  const EncodeWorkspace e = encode_workspace(const_cast<void*>(enc_workspace), N, d);
  unsigned long long* gacc = (unsigned long long*)workspace;
  double* partial = (double*)((char*)workspace + round_up((size_t)3 * K * sizeof(unsigned long long), 256));
  float* spare = (float*)((char*)partial + round_up((size_t)kLloydMaxParts * sizeof(double), 256));
  const int B = qamw_index_bits(K), rw = (int)qamw_packed_row_words(d, K);
  // round t reads cur and writes dst; the last round writes codebook_out
  const float* cur = codebook_init;
  for (int t = 0; t < iters; ++t) {
    float* dst = ((iters - 1 - t) % 2 == 0) ? codebook_out : spare;
    if ((rc = launch_build_plan(cur, (int)K, plan, st))) return rc;
    if ((rc = launch_encode(L, W, wdtype, (int)N, (int)d, ldw, e.f, e.isig, cur, (int)K, B, rw, e.rho, plan, packed,
                            st)))
      return rc;
    if ((rc = launch_lloyd_update(L, W, wdtype, (int)N, (int)d, ldw, e.f, e.isig, e.rho, packed, rw, B, cur, (int)K,
                                  dst, distortion_out + t, gacc, partial, st)))
      return rc;
    cur = dst;
  }
  return QAMW_OK;
}

int32_t qamw_encode_polar(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, const float* s,
                          const float* sigma, int32_t block, uint64_t sign_seed, const float* levels, int32_t Ka,
                          const float* dirs, int32_t Kp, uint32_t* packed, uint16_t* rownorm_f16, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_weights(W, wdtype, d, ldw))) return rc;
  if (!levels || !dirs) return fail(QAMW_EINVAL, "levels and dirs must be non-NULL");
  if (Ka < 1 || Kp < 1 || (int64_t)Ka * Kp < 2 || (int64_t)Ka * Kp > 4096)
    return fail(QAMW_EUNSUPPORTED, "polar code needs Ka, Kp >= 1 and 2 <= Ka * Kp <= 4096 (got %d x %d)", (int)Ka,
                (int)Kp);
  if (!s || !sigma || !packed || !rownorm_f16) return fail(QAMW_EINVAL, "s, sigma, packed and rownorm_f16 must be non-NULL");
  if (!aligned16(s) || !aligned16(sigma) || !aligned16(packed))
    return fail(QAMW_EINVAL, "s, sigma and packed must be 16-byte aligned");
  if ((rc = check_encode_workspace(workspace, workspace_bytes, N, d))) return rc;
  if ((rc = qamw_encode_prepare(W, wdtype, N, d, ldw, s, sigma, block, sign_seed, rownorm_f16, workspace,
                                workspace_bytes, stream)))
    return rc;
  const int K = Ka * Kp;
  const EncodeWorkspace e = encode_workspace(workspace, N, d);
  return launch_encode_polar(L, W, wdtype, (int)N, (int)d, ldw, e.f, e.isig, levels, (int)Ka, dirs, (int)Kp,
                             qamw_index_bits(K), (int)qamw_packed_row_words(d, K), e.rho, packed,
                             (hipStream_t)stream);
}

size_t qamw_channel_rms_workspace_bytes(int64_t T, int64_t d) {
  if (T <= 0 || T > kMaxDim || d <= 0 || d > kMaxDim) return 0;
  return round_up((size_t)((T + kRmsRowsPerTile - 1) / kRmsRowsPerTile) * (size_t)d * sizeof(float), 256);
}

static size_t oe_partials_bytes(int64_t T, int64_t N) {
  // one per workgroup: row blocks rounded up to whole groups of 8 (one per XCD) x token blocks
  const int64_t nb = (N + kOutputErrorRows - 1) / kOutputErrorRows;
  return round_up((size_t)((nb + 7) / 8 * 8) * (size_t)((T + kOutputErrorTokens - 1) / kOutputErrorTokens) *
                      sizeof(double), 256);
}

size_t qamw_output_error_workspace_bytes(int64_t T, int64_t N, int64_t d) {
  if (T <= 0 || T > kMaxDim || N <= 0 || N > kMaxDim || d <= 0 || d > kMaxDim) return 0;
  return oe_partials_bytes(T, N) + round_up((size_t)N * (size_t)d * 2, 256) + round_up((size_t)T * (size_t)d * 2, 256);
}

static int check_rows16(const void* p, int32_t dt, int64_t d, int64_t ld, const char* name, bool allow_f16) {
  if (!p) return fail(QAMW_EINVAL, "%s is NULL", name);
  if (dt != QAMW_F32 && dt != QAMW_BF16 && !(allow_f16 && dt == QAMW_F16))
    return fail(QAMW_EUNSUPPORTED, "%s dtype %d not supported", name, dt);
  if (ld < d) return fail(QAMW_EINVAL, "%s: leading dimension %lld < d=%lld", name, (long long)ld, (long long)d);
  if (!aligned16(p) || (ld * elem_size(dt)) % 16)
    return fail(QAMW_EINVAL, "%s must be 16-byte aligned with 16-byte aligned rows", name);
  return QAMW_OK;
}

int32_t qamw_channel_rms(const void* X, int32_t xdtype, int64_t T, int64_t d, int64_t ldx, float* r_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (T <= 0 || d <= 0) return fail(QAMW_EINVAL, "T and d must be positive (T=%lld d=%lld)", (long long)T, (long long)d);
  if (T > kMaxDim || d > kMaxDim) return fail(QAMW_EUNSUPPORTED, "activations too large");
  if (d % 8) return fail(QAMW_EINVAL, "d=%lld is not a multiple of 8", (long long)d);
  int rc = check_rows16(X, xdtype, d, ldx, "X", false);
  if (rc) return rc;
  if (!r_out || !aligned16(r_out)) return fail(QAMW_EINVAL, "r_out must be non-NULL and 16-byte aligned");
  const size_t need = qamw_channel_rms_workspace_bytes(T, d);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "channel RMS needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  return launch_channel_rms(X, xdtype, (int)T, (int)d, ldx, r_out, (float*)workspace, (hipStream_t)stream);
}

int32_t qamw_output_error(const void* X, int32_t xdtype, int64_t T, int64_t d, int64_t ldx, const void* W,
                          int32_t wdtype, int64_t N, int64_t ldw, const void* W_hat, int32_t hdtype, int64_t ldh,
                          double* err_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (T <= 0 || d <= 0 || N <= 0)
    return fail(QAMW_EINVAL, "T, N and d must be positive (T=%lld N=%lld d=%lld)", (long long)T, (long long)N,
                (long long)d);
  if (T > kMaxDim || d > kMaxDim || N > kMaxDim) return fail(QAMW_EUNSUPPORTED, "operands too large");
  if (d % 16) return fail(QAMW_EINVAL, "d=%lld is not a multiple of 16", (long long)d);
  int rc;
  if ((rc = check_rows16(X, xdtype, d, ldx, "X", false))) return rc;
  if ((rc = check_rows16(W, wdtype, d, ldw, "W", false))) return rc;
  if ((rc = check_rows16(W_hat, hdtype, d, ldh, "W_hat", false))) return rc;
  if (!err_out || ((uintptr_t)err_out & 7u)) return fail(QAMW_EINVAL, "err_out must be non-NULL and 8-byte aligned");
  const size_t need = qamw_output_error_workspace_bytes(T, N, d);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(QAMW_EWORKSPACE, "output error needs %zu bytes of 256-byte aligned workspace (got %zu)", need,
                workspace_bytes);
  char* ws = (char*)workspace;
  double* partial = (double*)ws;
  uint16_t* dWb = (uint16_t*)(ws + oe_partials_bytes(T, N));
  uint16_t* Xb = (uint16_t*)((char*)dWb + round_up((size_t)N * (size_t)d * 2, 256));
  return launch_output_error(X, xdtype, (int)T, (int)d, ldx, W, wdtype, (int)N, ldw, W_hat, hdtype, ldh, err_out,
                             partial, dWb, Xb, (hipStream_t)stream);
}

int32_t qamw_decode(const uint32_t* packed, const uint16_t* rownorm_f16, int64_t N, int64_t d, const float* s,
                    const float* sigma, int32_t block, uint64_t sign_seed, const float* codebook, int32_t K,
                    void* W_out, int32_t out_dtype, int64_t ldo, void* stream) {
  int L = 0;
  int rc = check_matrix(N, d, block, &L);
  if (rc) return rc;
  if ((rc = check_codebook(codebook, K))) return rc;
  if (!packed || !rownorm_f16 || !sigma || !W_out)
    return fail(QAMW_EINVAL, "packed, rownorm_f16, sigma and W_out must be non-NULL");
  if (out_dtype != QAMW_F32 && out_dtype != QAMW_BF16 && out_dtype != QAMW_F16)
    return fail(QAMW_EUNSUPPORTED, "output dtype %d not supported", out_dtype);
  if (ldo < d) return fail(QAMW_EINVAL, "ldo=%lld < d=%lld", (long long)ldo, (long long)d);
  if (!aligned16(packed) || !aligned16(W_out) || (ldo * elem_size(out_dtype)) % 16 || !aligned16(sigma) ||
      (s && !aligned16(s)))
    return fail(QAMW_EINVAL, "packed, s, sigma and W_out must be 16-byte aligned with 16-byte aligned rows");
  const int B = qamw_index_bits(K);
  const int row_words = (int)qamw_packed_row_words(d, K);
  return launch_decode(L, packed, rownorm_f16, (int)N, (int)d, s, sigma, sign_seed, codebook, (int)K, B, row_words,
                       W_out, out_dtype, ldo, (hipStream_t)stream);
}

int32_t qamw_rotate_activations(const void* X, int32_t xdtype, int64_t T, int64_t d, int64_t ldx, const float* s,
                                int32_t block, uint64_t sign_seed, uint16_t* Xr_bf16, int64_t ldr, void* stream) {
  int L = 0;
  int rc = check_matrix(T, d, block, &L);
  if (rc) return rc;
  if (!X) return fail(QAMW_EINVAL, "X is NULL");
  if (xdtype != QAMW_F32 && xdtype != QAMW_BF16) return fail(QAMW_EUNSUPPORTED, "activation dtype %d not supported", xdtype);
  if (ldx < d || ldr < d) return fail(QAMW_EINVAL, "ldx and ldr must be >= d");
  if (!Xr_bf16) return fail(QAMW_EINVAL, "Xr_bf16 is NULL");
  if (!aligned16(X) || (ldx * elem_size(xdtype)) % 16 || !aligned16(Xr_bf16) || (ldr * 2) % 16 || (s && !aligned16(s)))
    return fail(QAMW_EINVAL, "X, Xr_bf16 and s must be 16-byte aligned with 16-byte aligned rows");
  return launch_rotate_act(L, X, xdtype, (int)T, (int)d, ldx, s, sign_seed, Xr_bf16, ldr, (hipStream_t)stream);
}

int32_t qamw_decode_matmul(const uint16_t* Xr_bf16, int64_t T, int64_t d, int64_t ldr, const uint32_t* packed,
                           const uint16_t* rownorm_f16, int64_t N, const float* sigma, const float* codebook,
                           int32_t K, void* Y, int32_t ydtype, int64_t ldy, void* stream) {
  if (T <= 0 || N <= 0 || d <= 0) return fail(QAMW_EINVAL, "T, N and d must be positive");
  if (T > kMaxDim || N > kMaxDim || d > kMaxDim) return fail(QAMW_EUNSUPPORTED, "matrix too large");
  if (d % 16) return fail(QAMW_EINVAL, "d=%lld is not a multiple of 16", (long long)d);
  int rc = check_codebook(codebook, K);
  if (rc) return rc;
  if (!Xr_bf16 || !packed || !rownorm_f16 || !sigma || !Y)
    return fail(QAMW_EINVAL, "Xr_bf16, packed, rownorm_f16, sigma and Y must be non-NULL");
  if (ydtype != QAMW_F32 && ydtype != QAMW_BF16) return fail(QAMW_EUNSUPPORTED, "output dtype %d not supported", ydtype);
  if (ldr < d || ldy < N) return fail(QAMW_EINVAL, "ldr must be >= d and ldy >= N");
  if (!aligned16(Xr_bf16) || (ldr * 2) % 16 || !aligned16(packed) || !aligned16(sigma))
    return fail(QAMW_EINVAL, "Xr_bf16, packed and sigma must be 16-byte aligned, Xr rows too");
  const int B = qamw_index_bits(K);
  const int row_words = (int)qamw_packed_row_words(d, K);
  return launch_decode_matmul(Xr_bf16, (int)T, (int)d, ldr, packed, row_words, rownorm_f16, (int)N, sigma, codebook,
                              K, B, Y, ydtype, ldy, (hipStream_t)stream);
}

}  // extern "C"
