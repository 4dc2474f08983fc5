// The alpha grid search of the AWQ notes (bg51717.github.io/14592, section 方法):
//   s = s_X^alpha, alpha in [0, 1];  alpha* = argmin_alpha L(s_X^alpha),
//   L(s) = || Q(W s)(s^-1 X) - W X ||.
// This file holds every stage except the contractions (lossgemm.hip, gram.hip):
//   search_prep      s_i[k] = fp32(pow(max(s_X[k], s_floor), i/(n-1))) in fp64, and the reset
//                    of the control block;
//   absmax           max |W|, or max |W[n,k]| d_k in the Gram form (integer atomicMax on the
//                    fp32 bit patterns: order-free);
//   x_to_f16         fp16 copy of an fp32/bf16 X for the fp16 contraction;
//   quantize_stack   for all alpha at once: Q(W s_i) group-wise (the fp32 specification of
//                    device_common.h; symmetric or zero-point, groups of 128 or 64) and the error
//                    E_i = Q(W s_i)/s_i - W, stored in fp16 as
//                    E_i * 2^escale (Gram form: E_i[n,k] d_k 2^escale). By linearity
//                    X E_i^T = Q(W s_i)(s_i^-1 X) - W X.
//   finalize         fixed-order fp64 sum of the per-tile partial losses, L_i / (M N),
//                    argmin with the lowest index on ties, s_best = s_{i*}.
#include "device_common.h"
#include "kernels.h"

namespace awq {

// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void search_prep_kernel(const float* __restrict__ sx, int K,
                                                          int n_grid, float s_floor,
                                                          float* __restrict__ S,
                                                          SearchCtrl* __restrict__ ctrl) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx == 0) {
    ctrl->absmax_bits = 0u;
    ctrl->done = 0u;
    ctrl->gram_k = 0u;   // set again by the Gram form's finish pass
    ctrl->n_grid = (uint32_t)n_grid;
  }
  if (idx >= (int64_t)n_grid * K) return;
  const int i = (int)(idx / K);
  const int k = (int)(idx % K);
  const float b = fmaxf(sx[k], s_floor);          // floor compared in fp32
  const double alpha = (double)i / (double)(n_grid - 1);
  S[idx] = (float)pow((double)b, alpha);          // fp64 power, one rounding to fp32
}

hipError_t launch_search_prep(const float* sx, int K, int n_grid, float s_floor, float* S,
                              SearchCtrl* ctrl, hipStream_t stream) {
  const int64_t total = (int64_t)n_grid * K;
  search_prep_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(sx, K, n_grid, s_floor,
                                                                           S, ctrl);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// With COL, every |W[n,k]| is weighted by dcol[k] (the Gram form's column scaling). K is a
// multiple of 8, so the 8 elements of a chunk share one row and consecutive columns.
template <int DT, bool COL>
__global__ __launch_bounds__(256) void absmax_kernel(const void* __restrict__ W, int64_t count8,
                                                     int64_t K, const float* __restrict__ dcol,
                                                     SearchCtrl* __restrict__ ctrl,
                                                     uint32_t* __restrict__ flags) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  float m = 0.0f;
  bool bad = false;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  auto fold = [&](int64_t cc, const float (&v)[8]) {
    float d[8];
    if (COL) {
      load8_f32<kF32>(dcol + (cc * 8) % K, d);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bad |= !isfinite(v[t]);
      m = fmaxf(m, COL ? fabsf(v[t]) * d[t] : fabsf(v[t]));
    }
  };
  for (; c + 3 * stride < count8; c += 4 * stride) {     // four loads in flight per thread
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      load8_f32<DT>(reinterpret_cast<const char*>(W) + (c + u * stride) * 8 * ES, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) fold(c + u * stride, v[u]);
  }
  for (; c < count8; c += stride) {
    float v[8];
    load8_f32<DT>(reinterpret_cast<const char*>(W) + c * 8 * ES, v);
    fold(c, v);
  }
  // wave maximum, then workgroup maximum, then at most one atomic per workgroup (max is
  // order-free)
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[4];
  if (__lane_id() == 0) wmax[threadIdx.x >> 6] = m;
  wave_flag(flags, bad, kFlagNonfiniteW);
  __syncthreads();
  if (threadIdx.x == 0) {
    const float bm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    // Atomics on one address serialise; the maximum only grows, so a workgroup whose value
    // does not exceed one the maximum already held (a device-scope read, parallel across
    // workgroups) has nothing to add.
    const uint32_t seen =
        __hip_atomic_load(&ctrl->absmax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(bm) > seen) atomicMax(&ctrl->absmax_bits, __float_as_uint(bm));
  }
}

hipError_t launch_absmax(const void* W, int dtype, int64_t N, int64_t K, const float* dcol,
                         SearchCtrl* ctrl, uint32_t* flags, hipStream_t stream) {
  const int64_t count8 = N * K / 8;
  int64_t blocks = (count8 + 1023) / 1024;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  const unsigned g = (unsigned)blocks;
  if (dtype == kF32) {
    if (dcol)
      absmax_kernel<kF32, true><<<g, 256, 0, stream>>>(W, count8, K, dcol, ctrl, flags);
    else
      absmax_kernel<kF32, false><<<g, 256, 0, stream>>>(W, count8, K, dcol, ctrl, flags);
  } else {
    if (dcol)
      absmax_kernel<kF16, true><<<g, 256, 0, stream>>>(W, count8, K, dcol, ctrl, flags);
    else
      absmax_kernel<kF16, false><<<g, 256, 0, stream>>>(W, count8, K, dcol, ctrl, flags);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void x_to_f16_kernel(const void* __restrict__ X, int64_t count8,
                                                       uint16_t* __restrict__ X16,
                                                       uint32_t* __restrict__ flags) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  bool over = false;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < count8;
       c += (int64_t)gridDim.x * 256) {
    float v[8];
    load8_f32<DT>(reinterpret_cast<const char*>(X) + c * 8 * ES, v);
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint16_t lo = f2h(v[2 * t]), hi = f2h(v[2 * t + 1]);
      over |= ((lo & 0x7C00u) == 0x7C00u) || ((hi & 0x7C00u) == 0x7C00u);
      w[t] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *reinterpret_cast<uint4*>(X16 + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  wave_flag(flags, over, kFlagXF16Range);
}

hipError_t launch_x_to_f16(const void* X, int dtype, int64_t count, uint16_t* X16,
                           uint32_t* flags, hipStream_t stream) {
  const int64_t count8 = count / 8;
  int64_t blocks = (count8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (dtype == kBF16)
    x_to_f16_kernel<kBF16><<<(unsigned)blocks, 256, 0, stream>>>(X, count8, X16, flags);
  else
    x_to_f16_kernel<kF32><<<(unsigned)blocks, 256, 0, stream>>>(X, count8, X16, flags);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The error stack is stored as E * 2^escale with 2^escale * max|W| in [2^14, 2^15): every |E|
// is at most ~|w| (a code of 0 gives E = -w; a non-zero code means |w s| >= Delta/2 and the
// rounding error is at most Delta/2), so the fp16 values stay finite, and small errors keep
// fp16 normal precision instead of falling into the fp16 subnormal range. In the Gram form the
// same bound holds for E d_k against max |W d| (d_k >= 0).
__device__ __forceinline__ int escale_from_absmax(uint32_t bits) {
  return escale_for_max(__uint_as_float(bits));
}

constexpr int kQuantRows = 4;  // rows per thread in quantize_stack

// Thread layout: one thread owns 8 consecutive input channels (one 16-byte fp16 load) of
// kQuantRows rows; GL = group / 8 consecutive lanes cover one group (16 lanes, a DPP row, for
// 128 channels; 8 for 64), so the group maximum (and minimum) is four (three) DPP steps. The
// scale row s_i for the thread's 8 channels is loaded once per alpha and reused for all its rows.
// Stores: 16 bytes per lane, 1 KiB per wave, contiguous (the K-blocked stack of the Gram form
// takes its own thread layout, below). ZP: zero-point codes, E = (q - z) Delta
// / s - w. F32: the stack is fp32 (the vector-ALU contraction of small layers) and E is formed as
// fp32(fp32(fp32(q Delta) / s) - w) with an IEEE quotient, times the power of two.
template <int DT, bool COL, int GL, bool ZP, bool F32>
__global__ __launch_bounds__(256) void quantize_stack_kernel(
    const void* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ S, int n_grid,
    float qmin, float qmax, const float* __restrict__ dcol, const SearchCtrl* __restrict__ ctrl,
    void* __restrict__ Estack_, int64_t ld_rows, uint32_t* __restrict__ flags) {
  static_assert(!(F32 && COL), "the fp32 stack holds E itself");
  constexpr int ES = (DT == kF32) ? 4 : 2;
  const int64_t chunks = K / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // rows of this thread: rbase + r * rstep, r < kQuantRows
  int64_t c8, rbase, rstep;
  if constexpr (COL) {
    // K-blocked stack: a wave takes 16 rows x 128 channels; DPP row q (16 lanes, one or two
    // groups) holds rows 4 r + q, so one store instruction writes four runs of 4 rows x 64 bytes
    // and the thread's four rows complete 1 KiB runs of each 32-channel block. Consecutive waves
    // take consecutive row blocks of one 128-channel column, so a workgroup's stores fill four
    // 4 KiB runs and consecutive workgroups continue them (column-block-first order spread each
    // workgroup's stores over sixteen blocks 256 KiB apart)
    const int64_t wid = id >> 6, rblocks = (N + 15) / 16;
    const int lane = threadIdx.x & 63;
    c8 = (wid / rblocks) * 16 + (lane & 15);
    rbase = (wid % rblocks) * 16 + (lane >> 4);
    rstep = 4;
    if (c8 >= chunks) return;   // K is a multiple of the group: whole groups exit
  } else {
    c8 = id % chunks;
    rbase = (id / chunks) * kQuantRows;
    rstep = 1;
  }
  if (rbase >= N) return;  // whole GL-lane groups share their rows: no partial group exits here
  const int e = escale_from_absmax(ctrl->absmax_bits);
  const float esc = ldexpf(1.0f, e);
  float cs[8];   // per-column factor: 2^escale, times dcol[k] in the Gram form
  if (COL) {
    load8_f32<kF32>(dcol + c8 * 8, cs);
#pragma unroll
    for (int t = 0; t < 8; ++t) cs[t] *= esc;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) cs[t] = esc;
  }

  float w[kQuantRows][8];
  bool live[kQuantRows];
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r) {
    live[r] = (rbase + r * rstep) < N;
    if (live[r]) {
      load8_f32<DT>(reinterpret_cast<const char*>(W) + ((rbase + r * rstep) * K + c8 * 8) * ES,
                    w[r]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) w[r][t] = 0.0f;
    }
  }
  const size_t stride_alpha = (size_t)ld_rows * (size_t)K;
  for (int i = 0; i < n_grid; ++i) {
    float s[8], ics[8];   // ics: cs / s (v_rcp_f32, one rounding more)
    load8_f32<kF32>(S + (size_t)i * K + c8 * 8, s);
#pragma unroll
    for (int t = 0; t < 8; ++t) ics[t] = __builtin_amdgcn_rcpf(s[t]) * cs[t];
#pragma unroll
    for (int r = 0; r < kQuantRows; ++r) {
      if (!live[r]) continue;  // uniform over the GL-lane group
      float ws[8], q[8], z;
#pragma unroll
      for (int t = 0; t < 8; ++t) ws[t] = w[r][t] * s[t];
      bool uf;
      const float delta = quant8_g<GL, ZP, false>(ws, 1.0f, qmin, qmax, q, z, uf);
      if (ZP) {
#pragma unroll
        for (int t = 0; t < 8; ++t) q[t] -= z;   // exact: small integers
      }
      if constexpr (F32) {
        float ev[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) ev[t] = ((q[t] * delta) / s[t] - w[r][t]) * cs[t];
        float* dst = static_cast<float*>(Estack_) + i * stride_alpha + (rbase + r) * K + c8 * 8;
        *reinterpret_cast<float4*>(dst) = make_float4(ev[0], ev[1], ev[2], ev[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(ev[4], ev[5], ev[6], ev[7]);
        continue;
      }
      uint16_t* __restrict__ Estack = static_cast<uint16_t*>(Estack_);
      uint32_t packed[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // E = (q Delta)/s - w (q already centred by z), scaled (by the exact power of two, or by
        // d_k 2^escale) and rounded to fp16, as (q Delta - ws) (cs / s): q Delta - ws is exact in
        // one fma for every unclamped code (|q Delta - ws| <= Delta / 2 is a multiple of half an
        // ulp of Delta or of ws); what remains are the roundings of ws = w s (at most
        // 2^-24 |ws| <= 2^-24 qmax Delta) and of cs / s (2^-23 relative), small against error
        // terms of size ~Delta / 2 and against their fp16 rounding
        const float e0 = __builtin_fmaf(q[2 * t], delta, -ws[2 * t]) * ics[2 * t];
        const float e1 = __builtin_fmaf(q[2 * t + 1], delta, -ws[2 * t + 1]) * ics[2 * t + 1];
        packed[t] = f2h2(e0, e1);
      }
      // the Gram form's operand is K-blocked ([K / 32][ld_rows][32] per grid point): the 8
      // channels stay inside one 32-channel block
      const int64_t off = COL ? (c8 >> 2) * (ld_rows * 32) + (rbase + r * rstep) * 32 + (c8 & 3) * 8
                              : (rbase + r) * K + c8 * 8;
      *reinterpret_cast<uint4*>(Estack + i * stride_alpha + off) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
  }
}

template <int DT, bool COL, bool F32>
static void qs_dispatch(int group, bool zp, unsigned blocks, hipStream_t stream, const void* W,
                        int64_t N, int64_t K, const float* S, int n_grid, float qmin, float qmax,
                        const float* dcol, const SearchCtrl* ctrl, void* Estack,
                        int64_t ld_rows, uint32_t* flags) {
#define AWQ_QS(GL_, ZP_)                                                                         \
  quantize_stack_kernel<DT, COL, GL_, ZP_, F32><<<blocks, 256, 0, stream>>>(                     \
      W, N, K, S, n_grid, qmin, qmax, dcol, ctrl, Estack, ld_rows, flags)
  if (group == 64) {
    if (zp) AWQ_QS(8, true); else AWQ_QS(8, false);
  } else {
    if (zp) AWQ_QS(16, true); else AWQ_QS(16, false);
  }
#undef AWQ_QS
}

hipError_t launch_quantize_stack(const void* W, int dtype, int64_t N, int64_t K, const float* S,
                                 int n_grid, int bits, int group, bool zero_point,
                                 const float* dcol, const SearchCtrl* ctrl, void* Estack,
                                 bool f32_stack, int64_t ld_rows, uint32_t* flags,
                                 hipStream_t stream) {
  const float qmax = zero_point ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
  const float qmin = zero_point ? 0.0f : -(float)(1 << (bits - 1));
  // the K-blocked stack (dcol, fp16): waves of 16 rows x 128 channels
  const int64_t threads = (dcol && !f32_stack)
                              ? ((N + 15) / 16) * ((K / 8 + 15) / 16) * 64
                              : ((N + kQuantRows - 1) / kQuantRows) * (K / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
#define AWQ_QSD(DT_, COL_, F32_)                                                                 \
  qs_dispatch<DT_, COL_, F32_>(group, zero_point, blocks, stream, W, N, K, S, n_grid, qmin, qmax, \
                               dcol, ctrl, Estack, ld_rows, flags)
  if (f32_stack) {
    if (dcol) return hipErrorInvalidValue;   // the fp32 stack holds E itself
    if (dtype == kF32) AWQ_QSD(kF32, false, true); else AWQ_QSD(kF16, false, true);
  } else if (dtype == kF32) {
    if (dcol) AWQ_QSD(kF32, true, false); else AWQ_QSD(kF32, false, false);
  } else {
    if (dcol) AWQ_QSD(kF16, true, false); else AWQ_QSD(kF16, false, false);
  }
#undef AWQ_QSD
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// One workgroup per grid point sums that point's tile partials (thread t takes tiles t, t+256,
// ... into four independent accumulators, combined and tree-reduced in a fixed order). The last
// workgroup to finish -- found with an atomic counter -- picks the argmin and copies s_best.
__global__ __launch_bounds__(256) void finalize_kernel(
    const double* __restrict__ partials, int64_t tiles, int n_grid, int64_t M, int64_t N,
    int64_t K, const float* __restrict__ S, SearchCtrl* __restrict__ ctrl,
    double* __restrict__ losses, int32_t* __restrict__ best, float* __restrict__ s_best,
    uint32_t* __restrict__ flags) {
  __shared__ double red[256];
  __shared__ int is_last;
  __shared__ int sbest;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const double* p = partials + (int64_t)i * tiles;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int64_t t = tid;
  for (; t + 768 < tiles; t += 1024) {
    a0 += p[t];
    a1 += p[t + 256];
    a2 += p[t + 512];
    a3 += p[t + 768];
  }
  for (; t < tiles; t += 256) a0 += p[t];
  red[tid] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const int e = escale_from_absmax(ctrl->absmax_bits);
    losses[i] = ldexp(red[0], -2 * e) / ((double)M * (double)N);
    __threadfence();
    is_last = (atomicAdd(&ctrl->done, 1u) == (unsigned)(n_grid - 1));
  }
  __syncthreads();
  if (!is_last) return;
  if (tid == 0) __threadfence();
  __syncthreads();
  // every grid point's loss at once (device-scope loads, one per thread: a serial scan of
  // n_grid dependent reads from memory took most of this kernel's ~20 us), then the scan
  for (int j = tid; j < n_grid; j += 256)
    red[j] = __hip_atomic_load(losses + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid == 0) {
    int b = 0;
    bool bad = false;
    for (int j = 0; j < n_grid; ++j) {
      const double v = red[j];
      bad |= !isfinite(v);
      if (v < red[b]) b = j;
    }
    *best = b;
    sbest = b;
    if (bad) atomicOr(flags, kFlagNonfiniteLoss);
  }
  __syncthreads();
  const float* src = S + (int64_t)sbest * K;
  for (int64_t k = tid; k < K; k += 256) s_best[k] = src[k];
}

hipError_t launch_finalize(const double* partials, int64_t tiles_per_alpha, int n_grid,
                           int64_t M, int64_t N, int64_t K, const float* S,
                           SearchCtrl* ctrl, double* losses, int32_t* best,
                           float* s_best, uint32_t* flags, hipStream_t stream) {
  finalize_kernel<<<n_grid, 256, 0, stream>>>(partials, tiles_per_alpha, n_grid, M, N, K, S, ctrl,
                                              losses, best, s_best, flags);
  return hipGetLastError();
}

}  // namespace awq
