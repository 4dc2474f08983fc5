// Folding s^-1 into the previous operator: the AWQ notes (bg51717.github.io/14592, section 方法)
// list, among the method's further optimisations, fusing the input's down-scaling into the
// operator that produces that input, so the quantized layer takes its input unscaled. Every
// parameter of the previous operator that lands on input channel c of the layer is divided by
// s[c]: along the columns of a norm weight [1, K] (axis 1) or the rows (output channels) of a
// previous linear layer [K, *] (axis 0). Each value is fp32(fp32(p) / s), rounded once to the
// parameter's dtype. A small elementwise pass (norm weights and one projection at most), one
// element per lane in a grid-stride loop.
#include "device_common.h"
#include "kernels.h"

namespace awq {

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
  if (DT == kF32) return reinterpret_cast<const float*>(base)[i];
  const uint16_t b = reinterpret_cast<const uint16_t*>(base)[i];
  return DT == kF16 ? h2f(b) : bf2f(b);
}

template <int DT>
__device__ __forceinline__ bool store1(void* base, int64_t i, float v) {   // true: now non-finite
  if (DT == kF32) {
    reinterpret_cast<float*>(base)[i] = v;
    return !isfinite(v);
  }
  const uint16_t b = (DT == kF16) ? f2h(v) : f2bf(v);
  reinterpret_cast<uint16_t*>(base)[i] = b;
  return (DT == kF16) ? ((b & 0x7C00u) == 0x7C00u) : ((b & 0x7F80u) == 0x7F80u);
}

template <int DT>
__global__ __launch_bounds__(256) void fold_kernel(void* __restrict__ prev, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   const float* __restrict__ s, int axis,
                                                   uint32_t* __restrict__ flags) {
  bool over = false;
  const int64_t total = rows * cols;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / cols, c = idx % cols;
    const int64_t e = r * ld + c;
    const float p = load1<DT>(prev, e);
    const float q = p / (axis ? s[c] : s[r]);   // IEEE fp32 division
    over |= store1<DT>(prev, e, q) && isfinite(p);
  }
  wave_flag(flags, over, kFlagFoldRange);
}

hipError_t launch_fold(void* prev, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       const float* s, int axis, uint32_t* flags, hipStream_t stream) {
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  switch (dtype) {
    case kF16:
      fold_kernel<kF16><<<(unsigned)blocks, 256, 0, stream>>>(prev, rows, cols, ld, s, axis, flags);
      break;
    case kBF16:
      fold_kernel<kBF16><<<(unsigned)blocks, 256, 0, stream>>>(prev, rows, cols, ld, s, axis, flags);
      break;
    default:
      fold_kernel<kF32><<<(unsigned)blocks, 256, 0, stream>>>(prev, rows, cols, ld, s, axis, flags);
      break;
  }
  return hipGetLastError();
}

}  // namespace awq
