// Device helpers shared by the AWQ kernels (gfx950, wave64).
//
// The integer-deciding arithmetic (scaled weight, group step, rounded quotient) follows the
// quantizer of the AWQ notes (bg51717.github.io/14592, section 方法: Q(w) = Delta*Round(w/Delta))
// with the step denominator and clamp of "AWQ 量化方案：激活感知的权重量化与工程实现全解析"
// (qwbw.cn/news/39982, section 三, awq_quantize): Delta = max|w s| / (2^(b-1)-1), codes clamped to
// [-2^(b-1), 2^(b-1)-1], torch.round semantics (half to even). Every step is one IEEE fp32
// operation with round-to-nearest-even; the library is built with -ffp-contract=off so no step is
// fused, and fp32 division is the correctly rounded sequence.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };

enum : uint32_t {
  kFlagNonfiniteX = 1u << 0,
  kFlagNonfiniteW = 1u << 1,
  kFlagStatsInexact = 1u << 2,
  kFlagXF16Range = 1u << 3,
  kFlagScale16Overflow = 1u << 4,
  kFlagScale16Subnormal = 1u << 5,
  kFlagNonfiniteLoss = 1u << 6,
  kFlagStepUnderflow = 1u << 7,
  kFlagClipRange = 1u << 8,
  kFlagFoldRange = 1u << 9,
  kFlagNoGram = 1u << 10,
};

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Two values rounded to nearest even fp16, a in the low half: one packed conversion on gfx950.
__device__ __forceinline__ uint32_t f2h2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Load 8 consecutive elements starting at p (16-byte aligned for 16-bit types, 32-byte for f32)
// and widen them to fp32 (exact for every input type).
template <int DT>
__device__ __forceinline__ void load8_f32(const void* p, float (&v)[8]) {
  if constexpr (DT == kF32) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint16_t lo = (uint16_t)(w[t] & 0xFFFFu), hi = (uint16_t)(w[t] >> 16);
      if constexpr (DT == kF16) {
        v[2 * t] = h2f(lo);
        v[2 * t + 1] = h2f(hi);
      } else {
        v[2 * t] = bf2f(lo);
        v[2 * t + 1] = bf2f(hi);
      }
    }
  }
}

// DPP row (16-lane) permutations.
#define AWQ_DPP_QUAD_1032 0xB1   // quad_perm [1,0,3,2]
#define AWQ_DPP_QUAD_2301 0x4E   // quad_perm [2,3,0,1]
#define AWQ_DPP_ROW_MIRROR 0x140
#define AWQ_DPP_ROW_HALF_MIRROR 0x141

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane gets the result.
// Used for the per-group maximum: one group of 128 input channels = 16 lanes x 8 elements.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<AWQ_DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f32<AWQ_DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f32<AWQ_DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f32<AWQ_DPP_ROW_MIRROR>(v));
  return v;
}

// Maximum over the GL lanes (16: a DPP row; 8: half a row) that hold one quantization group of
// 8 GL channels; every lane of the group gets the result.
template <int GL>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f32<AWQ_DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f32<AWQ_DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f32<AWQ_DPP_ROW_HALF_MIRROR>(v));
  if (GL == 16) v = fmaxf(v, dpp_f32<AWQ_DPP_ROW_MIRROR>(v));
  return v;
}

// Maximum of non-negative values (a group's max |x|) over its GL lanes. For x >= 0 the fp32
// order is the order of the bit patterns as unsigned integers, so the steps run on integer max,
// which takes the DPP operand directly (fp32 max first quiets its inputs, one extra instruction
// per step).
template <int GL>
__device__ __forceinline__ float group_absmax(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, AWQ_DPP_QUAD_1032, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, AWQ_DPP_QUAD_2301, 0xF, 0xF, false));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, AWQ_DPP_ROW_HALF_MIRROR, 0xF, 0xF,
                                                   false));
  if (GL == 16)
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, AWQ_DPP_ROW_MIRROR, 0xF, 0xF, false));
  return __uint_as_float(u);
}

// Sum over the 16 lanes of a DPP row, as a butterfly (adjacent pairs, pairs of pairs, the two
// quads of each half, the two halves): addition is commutative, so every lane of the row ends
// with the bit-identical sum.
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f32<AWQ_DPP_QUAD_1032>(v);
  v = v + dpp_f32<AWQ_DPP_QUAD_2301>(v);
  v = v + dpp_f32<AWQ_DPP_ROW_HALF_MIRROR>(v);
  v = v + dpp_f32<AWQ_DPP_ROW_MIRROR>(v);
  return v;
}

// Quantize 8 scaled weights ws[] held by this lane; the 16 lanes of the lane's DPP row hold the
// rest of the 128-channel group. On return q[] holds the codes (as exact small floats) and the
// group step Delta is returned (0 for an all-zero group, or when max/qmax underflows to 0, in
// which case *underflow is set when the group was not all zero).
//
//   Delta = fp32(m / qmax),  q = clamp(rint(fp32(ws / Delta)), qmin, qmax)
//
// The quotient is formed as t' = fp32(ws * r) first, r = v_rcp_f32(Delta) (within 1 ulp of
// 1/Delta, so |r Delta - 1| <= 2^-23). Every code decision that can survive the clamp has
// |t| <= 16 (|ws| <= m in the symmetric form; in the zero-point form quotients beyond the clamp
// range give the clamped code on both sides), where |t' - fp32(ws/Delta)| <= 16 (2^-23 + 2^-24) +
// 2^-20 < 3.9e-6 < 2^-17. So rint(t') equals the specified rint(fp32(ws/Delta)) unless t' lies
// within 2^-17 of a half-integer; in that case (probability ~1.5e-5 per element), and whenever
// Delta lies outside [2^-126, 2^125] (r then not a normal number), the exact quotient is computed
// by IEEE division.
// Power-of-two exponent e for storing values bounded by m in fp16 as v * 2^e: 2^e m lies in
// [2^14, 2^15), so the values stay finite and keep normal fp16 precision (e = 0 for m = 0 or a
// non-finite m; e clamped to [-100, 100]).
__device__ __forceinline__ int escale_for_max(float m) {
  if (!(m > 0.0f) || !isfinite(m)) return 0;
  const uint32_t bits = __float_as_uint(m);
  const int e2 = (int)((bits >> 23) & 0xFFu);  // biased exponent; 0 for subnormal
  const int fl = (e2 == 0) ? -127 : e2 - 127;  // floor(log2 m) (subnormals clamped)
  int e = 14 - fl;
  if (e > 100) e = 100;
  if (e < -100) e = -100;
  return e;
}

struct QuantStep {
  float delta;      // Delta = fp32(m / qmax); 0 for m = 0 or when the quotient underflows
  float rcp;        // 1/Delta within 1 ulp; 0 when Delta is 0 (every code is then 0)
  bool exact_only;  // Delta or 1/Delta is not a normal number: always divide
};

// Delta = fp32(m / qmax) by one corrected product (Markstein's correction step): y = fp32(1/qmax),
// d0 = fp32(m y), r = m - qmax d0 (exact, one fma), Delta = fp32(d0 + r y). It equals the IEEE
// quotient for every fp32 significand of m with qmax in {3, 7, 15} (checked exhaustively against
// IEEE division), and all three steps scale exactly by powers of two while m lies in
// [2^-90, 2^100]; outside that range (and for 0, Inf, NaN) the IEEE division is taken.
__device__ __forceinline__ QuantStep quant_step(float m, float qmax) {
  QuantStep st;
  const float y = 1.0f / qmax;   // loop-invariant: hoisted by the compiler
  const float d0 = m * y;
  st.delta = __builtin_fmaf(__builtin_fmaf(-qmax, d0, m), y, d0);
  if (!(m >= 0x1p-90f && m <= 0x1p100f)) {
    // a real branch: without the empty volatile asm the compiler computes the division for
    // every group and selects
    float mm = m;
    asm volatile("" : "+v"(mm));
    st.delta = mm / qmax;
  }
  if (st.delta > 0.0f) {
    st.rcp = __builtin_amdgcn_rcpf(st.delta);
    st.exact_only = !(st.delta >= 0x1p-126f) || !(st.delta <= 0x1p+125f);
  } else {
    st.delta = 0.0f;
    st.rcp = 0.0f;
    st.exact_only = false;
  }
  return st;
}

// Codes of v[] (every |v| <= m) for the step of quant_step(m, qmax). The fast quotient is formed
// for every element; a lane that holds a quotient near a half-integer (or has exact_only set)
// redoes just those by IEEE division in one block that is rarely entered, so the common path has
// no branches.
template <int NV>
__device__ __forceinline__ void quant_codes(const float (&v)[NV], const QuantStep& st, float qmin,
                                            float qmax, float (&q)[NV]) {
  bool slow = st.exact_only;
#pragma unroll
  for (int t = 0; t < NV; ++t) {
    const float tq = v[t] * st.rcp;
    q[t] = rintf(tq);
    slow |= fabsf(tq - q[t]) > 0.5f - 0x1p-17f;
  }
  if (slow) {
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const float tq = v[t] * st.rcp;
      if (st.exact_only || fabsf(tq - rintf(tq)) > 0.5f - 0x1p-17f) q[t] = rintf(v[t] / st.delta);
    }
  }
#pragma unroll
  for (int t = 0; t < NV; ++t) q[t] = fminf(fmaxf(q[t], qmin), qmax);
}

// The codes of 8 values for one step: q = med3(rint(fp32(ws / Delta)) [+ z], qmin, qmax). The fast
// quotients are formed first and their largest distance from an integer is kept; only when
// that distance is within 2^-17 of one half (or the step needs exact division) does the lane
// enter the block that redoes the near-half elements by IEEE division. med3 equals the clamp for
// every finite value.
// The symmetric codes of the fast path need no clamp: there Delta = fp32(m / qmax) is a normal
// number (exact_only false), so Delta >= (m / qmax)(1 - 2^-24), v_rcp_f32 is within one ulp of
// 1 / Delta, and every |ws| <= m gives |fp32(ws rcp)| <= qmax (1 + 2^-21) < qmax + 1/2, i.e.
// |q| <= qmax. A step of 0 has rcp = 0 and gives codes 0 on the fast path. Zero-point codes add z
// and are clamped on both paths (q + z can pass either end by one).
template <bool ZP>
__device__ __forceinline__ void codes8(const float (&ws)[8], const QuantStep& st, float z,
                                       float qmin, float qmax, float (&q)[8]) {
  float dev = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float tq = ws[t] * st.rcp;
    q[t] = rintf(tq);
    dev = fmaxf(dev, fabsf(tq - q[t]));
  }
  if (st.exact_only || dev > 0.5f - 0x1p-17f) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float tq = ws[t] * st.rcp;
      if (st.exact_only || fabsf(tq - rintf(tq)) > 0.5f - 0x1p-17f) q[t] = rintf(ws[t] / st.delta);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = __builtin_amdgcn_fmed3f(ZP ? q[t] + z : q[t], qmin, qmax);
  } else if (ZP) {
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = __builtin_amdgcn_fmed3f(q[t] + z, qmin, qmax);
  }
}

// Codes of ws[] for the group maximum m (every |ws| <= m); returns Delta. A zero step (m = 0, or
// m / qmax below the smallest subnormal) gives codes 0 without a branch: quant_step returns
// rcp = 0 and exact_only false for it.
__device__ __forceinline__ float quant8_core(const float (&ws)[8], float m, float qmin,
                                             float qmax, float (&q)[8], bool& underflow) {
  const QuantStep st = quant_step(m, qmax);
  underflow = (m > 0.0f) && !(st.delta > 0.0f);
  codes8<false>(ws, st, 0.0f, qmin, qmax, q);
  return st.delta;
}

__device__ __forceinline__ float quant8(const float (&ws)[8], float qmin, float qmax,
                                        float (&q)[8], bool& underflow) {
  float m = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(ws[t]));
  m = row16_max(m);
  return quant8_core(ws, m, qmin, qmax, q, underflow);
}

// The quantizer of the search and of the packing, for a group of 8 GL channels held as 8
// values by each of GL consecutive lanes, optionally clipped (ratio r in (0, 1]: ws[] first moved
// into [-c, c], c = fp32(r m), m the group's max |ws|) and optionally with a zero point:
//   symmetric:  Delta = fp32(m' / qmax), q = clamp(rint(fp32(ws / Delta)), qmin, qmax)
//   zero point: Delta = fp32(fp32(max - min) / qmax_u), z = clamp(rint(fp32(-min / Delta)), 0,
//               qmax_u), q = clamp(rint(fp32(ws / Delta)) + z, 0, qmax_u)
// (qmax_u = 2^b - 1 is passed as qmax and 0 as qmin for the zero-point form). Returns Delta and
// sets z (0 for the symmetric form). Quotients as in quant8_core: |ws / Delta| <= 2^b - 1, so the
// fast product quotient is within 3e-6 of the specified one and the near-half-integer test
// decides when to divide exactly.
template <int GL, bool ZP, bool CLIP>
__device__ __forceinline__ float quant8_g(float (&ws)[8], float ratio, float qmin, float qmax,
                                          float (&q)[8], float& z, bool& underflow) {
  if (CLIP) {
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(ws[t]));
    m = group_absmax<GL>(m);
    const float c = ratio * m;
#pragma unroll
    for (int t = 0; t < 8; ++t) ws[t] = fminf(fmaxf(ws[t], -c), c);
  }
  if (!ZP) {
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(ws[t]));
    m = group_absmax<GL>(m);
    z = 0.0f;
    return quant8_core(ws, m, qmin, qmax, q, underflow);
  }
  float mx = ws[0], nmn = -ws[0];
#pragma unroll
  for (int t = 1; t < 8; ++t) {
    mx = fmaxf(mx, ws[t]);
    nmn = fmaxf(nmn, -ws[t]);
  }
  mx = group_max<GL>(mx);
  const float mn = -group_max<GL>(nmn);
  const float range = mx - mn;
  const QuantStep st = quant_step(range, qmax);
  underflow = (range > 0.0f) && !(st.delta > 0.0f);
  if (!(st.delta > 0.0f)) {
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = 0.0f;
    z = 0.0f;
    return 0.0f;
  }
  // z = clamp(rint(fp32(-min / Delta)), 0, qmax) by the fast quotient and the near-half test of
  // the codes (only |t| <= 16 can decide the clamped value); the IEEE division in a real branch
  float nm = -mn;
  const float tz = nm * st.rcp;
  float zq = rintf(tz);
  if (st.exact_only || fabsf(tz - zq) > 0.5f - 0x1p-17f) {
    asm volatile("" : "+v"(nm));
    zq = rintf(nm / st.delta);
  }
  z = __builtin_amdgcn_fmed3f(zq, 0.0f, qmax);
  codes8<true>(ws, st, z, 0.0f, qmax, q);
  return st.delta;
}

// Clipped quantization (the clipping search's ratio r in (0, 1]): ws[] is first moved into
// [-c, c], c = fp32(r * m) with m the group maximum; since c <= m, the clipped group's maximum
// is c, and the codes follow as in quant8.
__device__ __forceinline__ float quant8_clip(float (&ws)[8], float ratio, float qmin, float qmax,
                                             float (&q)[8], bool& underflow) {
  float m = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(ws[t]));
  m = row16_max(m);
  const float c = ratio * m;
#pragma unroll
  for (int t = 0; t < 8; ++t) ws[t] = fminf(fmaxf(ws[t], -c), c);
  return quant8_core(ws, c, qmin, qmax, q, underflow);
}

// The eight codes of one packed word as four exact fp16 pairs p[j] = (c_j, c_{j+4}), where
// c = q for two's-complement nibbles and c = q - z for unsigned zero-point nibbles (z the
// group's zero point). Each pair costs one mask-and-xor (a single v_bitop3_b32) and one packed
// fp16 operation, plus one shift per word:
//   * the xor constant both flips bit 3 of each nibble (u = q + 8 for signed codes; zero-point
//     codes are unsigned already, u = q) and places the exponent 0x6400 around it;
//   * nibbles j, j + 4 of pairs 0 and 2 sit at mantissa bits 0..3: the fp16 value is 1024 + u,
//     and subtracting 1024 + zc (zc = 8 or z) gives c;
//   * nibbles of pairs 1 and 3 stay at bits 4..7 (no shift): the value is 1024 + 16 u, and
//     fma(v, 1/16, -(64 + zc)) gives c;
// every intermediate is an integer below 2^11, so all of it is exact.
// sub_lo = 1024 + zc, sub_hi = -(64 + zc), both as fp16 pairs.
template <bool ZP>
__device__ __forceinline__ void unpack_word8(uint32_t w, half2_t sub_lo, half2_t sub_hi,
                                             half2_t (&p)[4]) {
  constexpr uint32_t kLo = ZP ? 0x64006400u : 0x64086408u;   // exponent + flip of bit 3
  constexpr uint32_t kHi = ZP ? 0x64006400u : 0x64806480u;   // the same for bits 4..7
  const half2_t sixteenth = half2_t{(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t y = w >> 8;
  p[0] = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) ^ kLo) - sub_lo;
  p[1] = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, (w & 0x00F000F0u) ^ kHi),
                                   sixteenth, sub_hi);
  p[2] = __builtin_bit_cast(half2_t, (y & 0x000F000Fu) ^ kLo) - sub_lo;
  p[3] = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, (y & 0x00F000F0u) ^ kHi),
                                   sixteenth, sub_hi);
}

// Buffer resource over [base, base + num_bytes): loads at offsets >= num_bytes return zero,
// which handles ragged tiles without branches. Word 1 holds the top 16 address bits with
// stride 0 (raw buffer); word 3 = 0x00020000 is the raw 32-bit data format used for untyped
// buffer access on gfx9-family (CDNA) parts. The descriptor must be wave-uniform (SGPRs).
typedef int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  rsrc_t r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)((uint32_t)(b >> 32) & 0xFFFFu);
  r[2] = (int)num_bytes;
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a __shared__ object (for M0 below).
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ uint32_t lds_addr(const void* shared_obj) {
  return (uint32_t)(uintptr_t)(const lds_char_t*)shared_obj;
}

// 16 bytes per lane from global memory (buffer offset `voff`) straight into LDS: lane l writes
// bytes [16 l, 16 l + 16) of the 1 KiB block at LDS address `lds` (wave-uniform).
//
// Written as inline asm on purpose: the compiler cannot tell which LDS bytes such a load writes,
// so with the builtin it would wait for every load in flight before each LDS read of the K loop,
// which serialises the multi-stage pipeline. The asm block has no register outputs (the data goes
// to LDS); it keeps the one wait state the hardware needs between writing M0 and the load that
// reads it, restores M0 before it ends, and the callers order LDS accesses against these loads
// with explicit vmcnt waits and barriers.
__device__ __forceinline__ void buffer_load16_lds(rsrc_t r, uint32_t lds, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"                      // one wait state between an M0 write and its LDS-DMA use
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(r)
      : "memory");
}

// The same load with a wave-uniform byte offset `soff` added in the scalar offset field, so a
// run of loads can share one per-lane offset register. The range check covers the whole offset
// (voff + soff; measured on gfx950: bytes at or past the buffer's size read as zeros whether the
// excess is in voff or in soff).
__device__ __forceinline__ void buffer_load16_lds_so(rsrc_t r, uint32_t lds, uint32_t voff,
                                                     uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(r), "s"(so)
      : "memory");
}

// s_waitcnt immediate: at most n vector-memory loads outstanding (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ void flag_or(uint32_t* flags, uint32_t bits) {
  if (bits) atomicOr(flags, bits);
}

// OR `bits` into *flags once per wave for the lanes where `cond` holds.
__device__ __forceinline__ void wave_flag(uint32_t* flags, bool cond, uint32_t bits) {
  const unsigned long long b = __ballot(cond);
  if (b != 0ull && __lane_id() == (unsigned)(__ffsll((long long)b) - 1)) atomicOr(flags, bits);
}

}  // namespace awq
