// awq_act_stats_noalloc: awq_act_stats with its scratch in a static device array, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The statistics' workspace (fp64 chunk partials and, for bf16 / fp32 X, one exponent byte per
// chunk and column) lives in `scratch`, a file-scope __device__ array of AWQ_NOALLOC_SCRATCH_BYTES
// that every GPU the library runs on holds until the process ends. In host code the name
// `scratch` is only a stand-in for the symbol; its device address is looked up once per device
// with hipGetSymbolAddress (on the first call made while that device is current) and that
// address is what the kernels receive. Pass 1 writes every partial and exponent byte that pass 2
// reads, so nothing has to start at zero; calls that overlap on one GPU share the array and race.
#include <mutex>

#include "../../include/awq.h"
#include "kernels.h"

static __device__ __align__(256) unsigned char scratch[AWQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up once per device).
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" awq_status awq_act_stats_noalloc(const void* X, awq_dtype xdt, int64_t M, int64_t K,
                                            int64_t ldx, float* sx, uint32_t* flags,
                                            hipStream_t stream) {
  if (!X || !sx || !flags) return AWQ_ERR_NULL;
  if (xdt != AWQ_F32 && xdt != AWQ_F16 && xdt != AWQ_BF16) return AWQ_ERR_DTYPE;
  constexpr int64_t kMaxDim = int64_t(1) << 24;
  if (M < 1 || K < 8 || K % 8 || ldx < K || ldx % 8 || M > kMaxDim || K > kMaxDim ||
      ldx > kMaxDim || (reinterpret_cast<uintptr_t>(X) & 15u) || awq::stats_chunks(M) > 65535)
    return AWQ_ERR_SHAPE;
  if (awq::stats_workspace_bytes(M, K) > (size_t)AWQ_NOALLOC_SCRATCH_BYTES)
    return AWQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return AWQ_ERR_HIP;
  return awq::launch_stats(X, (int)xdt, M, K, ldx, sx, flags, ws, stream) == hipSuccess
             ? AWQ_OK
             : AWQ_ERR_HIP;
}
