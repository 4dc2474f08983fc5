// Clipping search: the AWQ notes (bg51717.github.io/14592, section 方法) list clipping the
// scaled-up weights among the method's further optimisations. Per (output row n, group g of 128
// input channels), every ratio r_j of the grid 1 .. clip_min is tried on W s: the scaled weights
// are clipped to [-c, c], c = fp32(r_j max|w s|), quantized as in the search (quant_step /
// quant_codes), and scored by the output error the group causes on its own,
//   err_j[n, g] = sum_m ( sum_{k in g} X[m,k] E[n,k] )^2 = E_g H_gg E_g^T,  E = Q(W s)/s - W;
// the smallest wins, the lowest index on ties.
//
// The quadratic form uses the Gram form's conditioning (gram.hip): with E' = 2^e E d (d_k =
// sqrt(H_kk), e a power of two per row and group so that |E'| < 2^15) and C the correlation
// block, E_g H_gg E_g^T = 2^(1-2e) sum_l E'_l P_l, P_l = sum_{k<l} E'_k C_kl + E'_l / 2, where the
// operand B_gg (strict lower correlations, 1/2 diagonal) is the diagonal block of the
// block-diagonal correlation operand.
//
// Precision: each error is compared across ratios that differ little, so the contraction is
// carried to ~2^-22 rather than fp16's 2^-11: E' = E'_hi + E'_lo and B = B_hi + B_lo (each part
// fp16; B_lo from the operand's preparation), and P = E'_lo B_hi + E'_hi B_lo + E'_hi B_hi in
// fp32 accumulation (E'_lo B_lo, below 2^-22 relative, is left out); the epilogue takes E' in
// fp32.
//
// gfx950 layout: a workgroup of 4 waves takes 64 rows of one group of GS channels (128 or 64).
// Lane (i = lane % 16, q = lane / 16) of a wave owns row 16 w + i and the channels 32 kb + 8 q + t
// (kb < GS / 32, t < 8) of the group: exactly the A operand of v_mfma_f32_16x16x32_f16 for the
// group's 32-channel K blocks, so the quantized E' goes from registers straight into the MFMA.
// B_gg sits in LDS and the lower-triangular 32 x 16 fragments of its two parts in registers (20
// each for 128 channels, 6 for 64); P for 16 rows costs three times that many MFMAs. The
// epilogue needs E' in the accumulator layout (lane holds rows 4 q .. 4 q + 3 of column
// 16 cb + i), which it reads back from a per-wave fp32 LDS tile. With zero points (ZP) the
// clipped range is [max(min, -c), min(max, c)] of the unclipped group extremes, so the ratios
// need no further cross-lane reductions.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {
constexpr int kClipWaves = 4;
constexpr int kClipRows = 16 * kClipWaves;   // rows per workgroup

// Offset of the fragments of column block cb in the register array: column block c holds the
// K blocks kb <= c / 2, so the offset is sum_{c < cb} (c / 2 + 1) (and frag_base(CB) the count).
__host__ __device__ constexpr int frag_base(int cb) {
  return (cb % 2 == 0) ? (cb / 2) * (cb / 2 + 1) : (cb / 2 + 1) * (cb / 2 + 1);
}
static_assert(frag_base(8) == 20 && frag_base(4) == 6 && frag_base(7) == 16, "fragment count");

__device__ __forceinline__ float clip_ratio(int j, int n_clip, float clip_min) {
  return (float)(1.0 - (1.0 - (double)clip_min) * j / (n_clip - 1));
}
}  // namespace

template <int DT, int GS, bool ZP>
__global__ __launch_bounds__(256) void clip_search_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ d32, const uint16_t* __restrict__ Bd, int64_t bd_block,
    int64_t bd_kstride, const uint16_t* __restrict__ Bdl, const SearchCtrl* __restrict__ ctrl,
    int n_grid, int n_clip, float clip_min,
    float qmin, float qmax, float* __restrict__ clip, float* __restrict__ clip_err,
    uint32_t* __restrict__ flags) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  constexpr int KB = GS / 32;               // 32-channel K blocks per group
  constexpr int CB = GS / 16;               // 16-channel column blocks per group
  constexpr int NF = frag_base(CB);         // lower-triangular B fragments
  constexpr int kPitch = GS + 8;            // LDS row pitch in halves (no bank conflicts)
  constexpr int kPitchF = GS + 4;           // fp32 E' tile pitch in floats (no bank conflicts)
  constexpr int NV = 8 * KB;                // channels per lane
  __shared__ __attribute__((aligned(16))) uint16_t Bg[GS * kPitch];
  __shared__ __attribute__((aligned(16))) float Et[kClipWaves][16 * kPitchF];
  const int64_t G = K / GS;
  const int g = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * kClipRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, q = lane >> 4;

  // with the operand of a preceding Gram-form search: that search must have been the last to
  // write it, for this K and this grid size (the operand's offsets follow from both; uniform
  // over the grid: every workgroup leaves, one raises the flag)
  if (ctrl && (ctrl->gram_k != (uint32_t)K || ctrl->n_grid != (uint32_t)n_grid)) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(flags, kFlagNoGram);
    return;
  }
  // B_gg: rows l, columns k of the group, from the diagonal 256 x 256 block holding it. The
  // operand is K-blocked: element (l, k) of block a (l, k < 256 within it) at Bd + a * bd_block +
  // (k / 32) * bd_kstride + 32 l + k % 32
  {
    const int64_t c0 = (int64_t)g * GS;
    const int o = (int)(c0 % 256);
    const uint16_t* blk = Bd + (c0 / 256) * bd_block;
    for (int idx = tid; idx < GS * (GS / 8); idx += 256) {
      const int l = idx / (GS / 8), ch = idx % (GS / 8);
      const int kk = o + 8 * ch, ll = o + l;
      *reinterpret_cast<uint4*>(&Bg[l * kPitch + ch * 8]) = *reinterpret_cast<const uint4*>(
          blk + (int64_t)(kk >> 5) * bd_kstride + ll * 32 + (kk & 31));
    }
  }

  // this lane's row and channels
  const int64_t n = n0 + wave * 16 + i;
  const bool live = n < N;
  const int64_t kb0 = (int64_t)g * GS + 8 * q;
  float ws[KB][8], ca[KB][8], cb_[KB][8];   // w s;  E' = fma((q - z) Delta, ca, -cb_)
  float m = 0.0f, md = 0.0f, mx = -INFINITY, nmn = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float w[8], sv[8], dv[8];
    if (live) {
      load8_f32<DT>(reinterpret_cast<const char*>(W) + (n * K + kb0 + 32 * kb) * ES, w);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) w[t] = 0.0f;
    }
    load8_f32<kF32>(s + kb0 + 32 * kb, sv);
    load8_f32<kF32>(d32 + kb0 + 32 * kb, dv);   // d / s below: correctly rounded
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bad |= !isfinite(w[t]);
      ws[kb][t] = w[t] * sv[t];
      m = fmaxf(m, fabsf(ws[kb][t]));
      mx = fmaxf(mx, ws[kb][t]);
      nmn = fmaxf(nmn, -ws[kb][t]);
      md = fmaxf(md, fabsf(w[t]) * dv[t]);
      ca[kb][t] = dv[t] / sv[t];
      cb_[kb][t] = w[t] * dv[t];
    }
  }
  // the four lanes q = 0..3 of row i hold its channels
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  md = fmaxf(md, __shfl_xor(md, 16));
  md = fmaxf(md, __shfl_xor(md, 32));
  if (ZP) {
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    nmn = fmaxf(nmn, __shfl_xor(nmn, 16));
    nmn = fmaxf(nmn, __shfl_xor(nmn, 32));
  }
  const float mn = -nmn;
  const int e = escale_for_max(md);   // |E| <= |w|, so |E'| < 2^15
  const float esc = ldexpf(1.0f, e);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      ca[kb][t] *= esc;
      cb_[kb][t] *= esc;
    }
  __syncthreads();

  half8_t bf[NF], bfl[NF];
  {
    // B_lo fragments straight from memory: the diagonal block holding the group, [256][256]
    const int64_t c0 = (int64_t)g * GS;
    const int o = (int)(c0 % 256);
    const uint16_t* srcl = Bdl + (c0 / 256) * (int64_t)(kLossBM * kLossBN) + (int64_t)o * kLossBN + o;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int kb = 0; kb <= cb / 2; ++kb) {
        bf[frag_base(cb) + kb] =
            *reinterpret_cast<const half8_t*>(&Bg[(16 * cb + i) * kPitch + 32 * kb + 8 * q]);
        bfl[frag_base(cb) + kb] = *reinterpret_cast<const half8_t*>(
            srcl + (int64_t)(16 * cb + i) * kLossBN + 32 * kb + 8 * q);
      }
  }

  // lanes i < 4 of each 16-lane quarter track row R = 4 q + i of the accumulator layout
  const int R = 4 * q + (i & 3);
  const int eR = __shfl(e, R);           // lane R (< 16) owns row R
  const int64_t nR = n0 + wave * 16 + R;
  float best = 0.0f;
  int best_j = 0;
  bool uf_any = false;
  float* et = Et[wave];

  for (int j = 0; j < n_clip; ++j) {
    const float c = clip_ratio(j, n_clip, clip_min) * m;
    float v[NV], qv[NV];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < 8; ++t) v[8 * kb + t] = fminf(fmaxf(ws[kb][t], -c), c);
    QuantStep st;
    float z = 0.0f;
    if (ZP) {
      const float range = fminf(mx, c) - fmaxf(mn, -c);
      st = quant_step(range, qmax);
      uf_any |= (range > 0.0f) && !(st.delta > 0.0f);
      if (st.delta > 0.0f) z = fminf(fmaxf(rintf(-fmaxf(mn, -c) / st.delta), 0.0f), qmax);
      quant_codes(v, st, -INFINITY, INFINITY, qv);
#pragma unroll
      for (int t = 0; t < NV; ++t) qv[t] = fminf(fmaxf(qv[t] + z, 0.0f), qmax) - z;
    } else {
      st = quant_step(c, qmax);
      uf_any |= (c > 0.0f) && !(st.delta > 0.0f);
      quant_codes(v, st, qmin, qmax, qv);
    }
    half8_t af[KB], al[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float evs[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float ev = __builtin_fmaf(qv[8 * kb + t] * st.delta, ca[kb][t], -cb_[kb][t]);
        const uint16_t h = f2h(ev);
        af[kb][t] = __builtin_bit_cast(_Float16, h);
        al[kb][t] = __builtin_bit_cast(_Float16, f2h(ev - h2f(h)));   // exact difference
        evs[t] = ev;
      }
      float* dst = &et[i * kPitchF + 32 * kb + 8 * q];
      *reinterpret_cast<float4*>(dst) = make_float4(evs[0], evs[1], evs[2], evs[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(evs[4], evs[5], evs[6], evs[7]);
    }
    floatx4 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      acc[cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      // the two small cross terms first, then the leading one
#pragma unroll
      for (int kb = 0; kb <= cb / 2; ++kb) {
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[kb], bf[frag_base(cb) + kb], acc[cb],
                                                        0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[kb], bfl[frag_base(cb) + kb], acc[cb],
                                                        0, 0, 0);
      }
#pragma unroll
      for (int kb = 0; kb <= cb / 2; ++kb)
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[kb], bf[frag_base(cb) + kb], acc[cb],
                                                        0, 0, 0);
    }
    // the tile written above is read back by other lanes of this wave: LDS accesses of one
    // wave complete in order; keep the compiler from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float part[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      part[rr] = 0.0f;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        part[rr] = __builtin_fmaf(et[(4 * q + rr) * kPitchF + 16 * cb + i], acc[cb][rr], part[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) part[rr] = row16_sum(part[rr]);   // the 16 columns i
    const int sel = i & 3;
    const float val = (sel == 0) ? part[0] : (sel == 1) ? part[1] : (sel == 2) ? part[2] : part[3];
    if (j == 0 || val < best) {          // strict: the lowest index wins ties
      best = val;
      best_j = j;
    }
    if (clip_err && i < 4 && nR < N)
      clip_err[((int64_t)j * N + nR) * G + g] = ldexpf(2.0f * val, -2 * eR);
    // all reads of the tile are done before the next ratio overwrites it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (i < 4 && nR < N) clip[nR * G + g] = clip_ratio(best_j, n_clip, clip_min);
  wave_flag(flags, bad, kFlagNonfiniteW);
  wave_flag(flags, uf_any, kFlagStepUnderflow);
}

hipError_t launch_clip_search(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                              const float* d32, const uint16_t* Bd, int64_t bd_block,
                              int64_t bd_kstride, const uint16_t* Bdl, const SearchCtrl* ctrl,
                              int n_grid, int n_clip, float clip_min, int bits, int group,
                              bool zero_point, float* clip, float* clip_err, uint32_t* flags,
                              hipStream_t stream) {
  const float qmax = zero_point ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float qmin = zero_point ? 0.0f : -(float)(1 << (bits - 1));
  dim3 grid((unsigned)((N + kClipRows - 1) / kClipRows), (unsigned)(K / group));
#define AWQ_CLIP(DT_, GS_, ZP_)                                                                  \
  clip_search_kernel<DT_, GS_, ZP_><<<grid, 256, 0, stream>>>(                                    \
      W, N, K, s, d32, Bd, bd_block, bd_kstride, Bdl, ctrl, n_grid, n_clip, clip_min, qmin, qmax,   \
      clip,                                                                                      \
      clip_err, flags)
  if (dtype == kF32) {
    if (group == 64) {
      if (zero_point) AWQ_CLIP(kF32, 64, true); else AWQ_CLIP(kF32, 64, false);
    } else {
      if (zero_point) AWQ_CLIP(kF32, 128, true); else AWQ_CLIP(kF32, 128, false);
    }
  } else {
    if (group == 64) {
      if (zero_point) AWQ_CLIP(kF16, 64, true); else AWQ_CLIP(kF16, 64, false);
    } else {
      if (zero_point) AWQ_CLIP(kF16, 128, true); else AWQ_CLIP(kF16, 128, false);
    }
  }
#undef AWQ_CLIP
  return hipGetLastError();
}

}  // namespace awq
