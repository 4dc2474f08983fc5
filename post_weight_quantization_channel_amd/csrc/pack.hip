// Packing of the chosen quantization: the stored result of "AWQ 量化方案..." (qwbw.cn/news/39982),
// section 三 (QuantLinear(q_weight, scales_per_group, awq_scale): "INT4 packed" codes, per-group
// fp16 steps and the per-channel scale).
//   qweight[n, j] = sum_t (q[n, 8j+t] & 0xF) << 4t      (element 8j+t in bits 4t..4t+3)
//   scales16[n, g] = fp16(Delta[n, g]),  s16[k] = fp16(s[k])   (round to nearest even)
//   zeros[n, g] = z[n, g]  (zero-point form only)
// The codes come from quant8_g(), the quantizer of the search (groups of 128 or 64, symmetric or
// zero point), so they are bit-identical to the codes the search scored; with clip ratios (one
// per row and group, from the clipping search) the scaled weights are clipped first, as in that
// search. Zero-point codes are unsigned (0 .. 2^b - 1) in the same nibble layout, and
// zeros[n, g] holds z.
#include "device_common.h"
#include "kernels.h"

namespace awq {

template <int DT, bool CLIP, int GL, bool ZP>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                   const float* __restrict__ s,
                                                   const float* __restrict__ clip, float qmin,
                                                   float qmax, uint32_t* __restrict__ qweight,
                                                   uint16_t* __restrict__ scales16,
                                                   uint8_t* __restrict__ zeros,
                                                   uint16_t* __restrict__ s16,
                                                   int8_t* __restrict__ codes,
                                                   uint32_t* __restrict__ flags) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  const int64_t chunks = K / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = id / chunks;
  const int64_t c8 = id % chunks;
  bool of = false, sub = false, uf_any = false, bad_clip = false;
  constexpr int G = 8 * GL;   // channels per group
  const int64_t groups = K / G;
  if (n < N) {  // uniform over each GL-lane group (chunks % GL == 0)
    float w[8], sv[8], ws[8], q[8];
    load8_f32<DT>(reinterpret_cast<const char*>(W) + (n * K + c8 * 8) * ES, w);
    load8_f32<kF32>(s + c8 * 8, sv);
#pragma unroll
    for (int t = 0; t < 8; ++t) ws[t] = w[t] * sv[t];
    bool uf;
    float r = 1.0f, z;
    if (CLIP) {
      r = clip[n * groups + c8 / GL];
      if (!(r > 0.0f && r <= 1.0f)) {   // outside (0, 1]: flagged, packed unclipped
        bad_clip = true;
        r = 1.0f;
      }
    }
    const float delta = quant8_g<GL, ZP, CLIP>(ws, r, qmin, qmax, q, z, uf);
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
    if ((c8 & (GL - 1)) == 0) {
      const uint16_t h = f2h(delta);
      scales16[n * groups + c8 / GL] = h;
      if (ZP) zeros[n * groups + c8 / GL] = (uint8_t)(int)z;
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

template <int DT, bool CLIP>
static void pack_dispatch(int group, bool zp, unsigned blocks, hipStream_t stream, const void* W,
                          int64_t N, int64_t K, const float* s, const float* clip, float qmin,
                          float qmax, uint32_t* qweight, uint16_t* scales16, uint8_t* zeros,
                          uint16_t* s16, int8_t* codes, uint32_t* flags) {
#define AWQ_PACK(GL_, ZP_)                                                                       \
  pack_kernel<DT, CLIP, GL_, ZP_><<<blocks, 256, 0, stream>>>(W, N, K, s, clip, qmin, qmax,       \
                                                              qweight, scales16, zeros, s16,     \
                                                              codes, flags)
  if (group == 64) {
    if (zp) AWQ_PACK(8, true); else AWQ_PACK(8, false);
  } else {
    if (zp) AWQ_PACK(16, true); else AWQ_PACK(16, false);
  }
#undef AWQ_PACK
}

hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                       const float* clip, int bits, int group, uint32_t* qweight,
                       uint16_t* scales16, uint8_t* zeros, uint16_t* s16, int8_t* codes,
                       uint32_t* flags, hipStream_t stream) {
  const bool zp = zeros != nullptr;
  const float qmax = zp ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float qmin = zp ? 0.0f : -(float)(1 << (bits - 1));
  const int64_t threads = N * (K / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (dtype == kF32) {
    if (clip)
      pack_dispatch<kF32, true>(group, zp, blocks, stream, W, N, K, s, clip, qmin, qmax, qweight,
                                scales16, zeros, s16, codes, flags);
    else
      pack_dispatch<kF32, false>(group, zp, blocks, stream, W, N, K, s, clip, qmin, qmax,
                                 qweight, scales16, zeros, s16, codes, flags);
  } else {
    if (clip)
      pack_dispatch<kF16, true>(group, zp, blocks, stream, W, N, K, s, clip, qmin, qmax, qweight,
                                scales16, zeros, s16, codes, flags);
    else
      pack_dispatch<kF16, false>(group, zp, blocks, stream, W, N, K, s, clip, qmin, qmax,
                                 qweight, scales16, zeros, s16, codes, flags);
  }
  return hipGetLastError();
}

}  // namespace awq
