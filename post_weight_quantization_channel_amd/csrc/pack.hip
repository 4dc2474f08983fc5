// Packing of the chosen quantization: the stored result of "AWQ 量化方案..." (qwbw.cn/news/39982),
// section 三 (QuantLinear(q_weight, scales_per_group, awq_scale): "INT4 packed" codes, per-group
// fp16 steps and the per-channel scale).
//   qweight[n, j] = sum_t (q[n, 8j+t] & 0xF) << 4t      (element 8j+t in bits 4t..4t+3)
//   scales16[n, g] = fp16(Delta[n, g]),  s16[k] = fp16(s[k])   (round to nearest even)
// The codes come from quant8(), the same device function as the search, so they are
// bit-identical to the codes the search scored. With clip ratios (one per row and group, from
// the clipping search) the codes come from quant8_clip(), as in that search.
#include "device_common.h"
#include "kernels.h"

namespace awq {

template <int DT, bool CLIP>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                   const float* __restrict__ s,
                                                   const float* __restrict__ clip, float qmin,
                                                   float qmax, uint32_t* __restrict__ qweight,
                                                   uint16_t* __restrict__ scales16,
                                                   uint16_t* __restrict__ s16,
                                                   int8_t* __restrict__ codes,
                                                   uint32_t* __restrict__ flags) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  const int64_t chunks = K / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = id / chunks;
  const int64_t c8 = id % chunks;
  bool of = false, sub = false, uf_any = false, bad_clip = false;
  if (n < N) {  // uniform over each 16-lane group (chunks % 16 == 0)
    float w[8], sv[8], ws[8], q[8];
    load8_f32<DT>(reinterpret_cast<const char*>(W) + (n * K + c8 * 8) * ES, w);
    load8_f32<kF32>(s + c8 * 8, sv);
#pragma unroll
    for (int t = 0; t < 8; ++t) ws[t] = w[t] * sv[t];
    bool uf;
    float delta;
    if (CLIP) {
      float r = clip[n * (K / 128) + c8 / 16];
      if (!(r > 0.0f && r <= 1.0f)) {   // outside (0, 1]: flagged, packed unclipped
        bad_clip = true;
        r = 1.0f;
      }
      delta = quant8_clip(ws, r, qmin, qmax, q, uf);
    } else {
      delta = quant8(ws, qmin, qmax, q, uf);
    }
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) word |= ((uint32_t)((int)q[t]) & 0xFu) << (4 * t);
    qweight[n * chunks + c8] = word;
    if (codes) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo |= ((uint32_t)((int)q[t]) & 0xFFu) << (8 * t);
        hi |= ((uint32_t)((int)q[t + 4]) & 0xFFu) << (8 * t);
      }
      *reinterpret_cast<uint2*>(codes + n * K + c8 * 8) = make_uint2(lo, hi);
    }
    if ((c8 & 15) == 0) {
      const uint16_t h = f2h(delta);
      scales16[n * (K / 128) + c8 / 16] = h;
      of |= (h & 0x7C00u) == 0x7C00u;
      sub |= (delta > 0.0f) && ((h & 0x7C00u) == 0u);
      uf_any |= uf;
    }
    if (n == 0) {
      uint32_t p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t lo = f2h(sv[2 * t]), hi = f2h(sv[2 * t + 1]);
        of |= ((lo & 0x7C00u) == 0x7C00u) || ((hi & 0x7C00u) == 0x7C00u);
        sub |= (sv[2 * t] != 0.0f && (lo & 0x7C00u) == 0u) ||
               (sv[2 * t + 1] != 0.0f && (hi & 0x7C00u) == 0u);
        p[t] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      *reinterpret_cast<uint4*>(s16 + c8 * 8) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
  wave_flag(flags, of, kFlagScale16Overflow);
  wave_flag(flags, sub, kFlagScale16Subnormal);
  wave_flag(flags, uf_any, kFlagStepUnderflow);
  if (CLIP) wave_flag(flags, bad_clip, kFlagClipRange);
}

hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                       const float* clip, int bits, uint32_t* qweight, uint16_t* scales16,
                       uint16_t* s16, int8_t* codes, uint32_t* flags, hipStream_t stream) {
  const float qmax = (float)((1 << (bits - 1)) - 1);
  const float qmin = -(float)(1 << (bits - 1));
  const int64_t threads = N * (K / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
#define AWQ_PACK(DT_, CLIP_)                                                                  \
  pack_kernel<DT_, CLIP_><<<blocks, 256, 0, stream>>>(W, N, K, s, clip, qmin, qmax, qweight,   \
                                                      scales16, s16, codes, flags)
  if (dtype == kF32) {
    if (clip) AWQ_PACK(kF32, true); else AWQ_PACK(kF32, false);
  } else {
    if (clip) AWQ_PACK(kF16, true); else AWQ_PACK(kF16, false);
  }
#undef AWQ_PACK
  return hipGetLastError();
}

}  // namespace awq
