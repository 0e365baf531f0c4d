// The GEMM entry point that allocates nothing: loop_op_gemm with the split-K
// partials in a fixed device array of the library instead of a caller
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a
// host-side stand-in, never a device address: the device address is taken
// once per device with hipGetSymbolAddress (that device current) and kept in
// `g_scratch`; only that pointer is handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "host.h"

namespace {

constexpr size_t SCRATCH_BYTES = LOOP_GEMM_STATIC_SCRATCH_BYTES;
static_assert(SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) float scratch[SCRATCH_BYTES / sizeof(float)];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// The device address of this device's scratch array (looked up on the first
// call on the device, with the device current).
int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return loop_hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return loop_fail(LOOP_EDEVICE, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return loop_hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return loop_fail(LOOP_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return 0;
}

}  // namespace

extern "C" int loop_op_gemm_static(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                                   const float* R, int32_t M, int32_t N, int32_t K, int32_t epi, void* stream) {
  if (!A || !B || !C) return loop_fail(LOOP_EINVAL, "gemm_static: null operand");
  if (epi < 0 || epi > 3) return loop_fail(LOOP_EINVAL, "gemm_static: bad epilogue %d", epi);
  if (epi == LOOP_EPI_F32_RES && !R) return loop_fail(LOOP_EINVAL, "gemm_static: residual epilogue needs R");
  if (M < 0 || N <= 0 || K <= 0 || K % 64) return loop_fail(LOOP_ESHAPE, "gemm_static: need N > 0, K > 0, K %% 64 == 0");
  if (lda % 8 || ldb % 8 || lda < K || ldb < K || ldc < N)
    return loop_fail(LOOP_ESHAPE, "gemm_static: lda, ldb must be multiples of 8 and cover K; ldc >= N");
  if (((uintptr_t)A | (uintptr_t)B) % 16) return loop_fail(LOOP_EINVAL, "gemm_static: A and B must be 16-byte aligned");
  if (M > LOOP_GEMM_STATIC_MAX_ROWS)
    return loop_fail(LOOP_ECAPACITY, "gemm_static: %d rows above the %d this entry point takes", M,
                     LOOP_GEMM_STATIC_MAX_ROWS);
  if (M == 0) return 0;
  const size_t need = gemm_small_m_partial_bytes(M, N, K, epi, lda, ldb);
  if (need > SCRATCH_BYTES)
    return loop_fail(LOOP_ECAPACITY, "gemm_static: the split-K partials need %zu bytes, the static scratch holds %zu",
                     need, SCRATCH_BYTES);
  void* ptr = nullptr;
  if (int r = scratch_of_current_device(&ptr)) return r;
  // every partial the split kernels read is written by them first in the
  // same call: nothing needs clearing
  hipError_t e = launch_gemm(A, lda, B, ldb, C, ldc, R, M, N, K, epi, (hipStream_t)stream, (float*)ptr, SCRATCH_BYTES);
  return e == hipSuccess ? 0 : loop_hip_fail(e, "gemm_static launch");
}
