// Activation statistics: s_X[k] = mean_m |X[m,k]|.
//
// AWQ notes (bg51717.github.io/14592), section 方法: the scale is a power of s_X, a statistic of
// the layer input; "AWQ 量化方案..." (qwbw.cn/news/39982), section 三 Step 1: act_norm =
// calib_data.abs().mean(dim=0).
//
// HBM-bound column reduction. Pass 1: each thread owns 8 consecutive columns (one 16-byte load
// per row for 16-bit inputs) and sums |x| over a chunk of 256 rows in fp64; a 64-lane wave reads
// 1 KiB of a row contiguously. Pass 2 adds the chunk partials of each column in a fixed order
// (eight interleaved slices per column, combined in slice order) and divides by M in fp64 before
// the single rounding to fp32, so a run is reproducible bit for bit. For fp16 inputs every
// partial sum is exact (all |x| are multiples of 2^-24 and the sums stay below 2^29, which is
// checked), so the result does not depend on the reduction order at all. The Gram-form search
// can take the same chunk partials in its transpose pass (gram.hip) and reduce them with the
// final pass here, which then gives the same s_X bit for bit.
#include "device_common.h"
#include "kernels.h"

namespace awq {

template <int DT>
__global__ __launch_bounds__(256) void stats_partial_kernel(const void* __restrict__ X, int64_t M,
                                                            int64_t K, int64_t ldx,
                                                            double* __restrict__ partials) {
  const int64_t c8 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // column chunk of 8
  if (c8 * 8 >= K) return;
  const int64_t chunk = blockIdx.y;
  const int64_t r0 = chunk * kStatsRowsPerChunk;
  const int64_t r1 = (r0 + kStatsRowsPerChunk < M) ? r0 + kStatsRowsPerChunk : M;
  constexpr int ES = (DT == kF32) ? 4 : 2;
  const char* base = reinterpret_cast<const char*>(X) + (c8 * 8) * ES;
  double acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.0;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8_f32<DT>(base + (r + u) * ldx * ES, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] += (double)fabsf(v[u][t]);
  }
  for (; r < r1; ++r) {
    float v[8];
    load8_f32<DT>(base + r * ldx * ES, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] += (double)fabsf(v[t]);
  }
  double* out = partials + chunk * K + c8 * 8;
#pragma unroll
  for (int t = 0; t < 8; ++t) out[t] = acc[t];
}

// Pass 2: a workgroup owns 32 columns; its 256 threads are (column c = t % 32, slice
// j = t / 32): slice j adds the chunks j, j + 8, j + 16, ... of its column with four independent
// accumulators (fixed assignment), then the 8 slices are added in slice order through LDS.
__global__ __launch_bounds__(256) void stats_final_kernel(const double* __restrict__ partials,
                                                          int64_t chunks, int64_t M, int64_t K,
                                                          int dtype, float* __restrict__ sx,
                                                          uint32_t* __restrict__ flags) {
  __shared__ double part[8][32];
  const int c = threadIdx.x & 31, j = threadIdx.x >> 5;
  const int64_t k = (int64_t)blockIdx.x * 32 + c;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  if (k < K) {
    int64_t ch = j;
    for (; ch + 24 < chunks; ch += 32) {
      a0 += partials[ch * K + k];
      a1 += partials[(ch + 8) * K + k];
      a2 += partials[(ch + 16) * K + k];
      a3 += partials[(ch + 24) * K + k];
    }
    for (; ch < chunks; ch += 8) a0 += partials[ch * K + k];
  }
  part[j][c] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  bool bad = false, inexact = false;
  if (j == 0 && k < K) {
    double S = part[0][c];
#pragma unroll
    for (int q = 1; q < 8; ++q) S += part[q][c];
    bad = !isfinite(S);
    inexact = (dtype == kF16) && (S >= 0x1p29);
    sx[k] = (float)(S / (double)M);
  }
  wave_flag(flags, bad, kFlagNonfiniteX);
  wave_flag(flags, inexact, kFlagStatsInexact);
}

int64_t stats_chunks(int64_t M) { return (M + kStatsRowsPerChunk - 1) / kStatsRowsPerChunk; }

hipError_t launch_stats(const void* X, int dtype, int64_t M, int64_t K, int64_t ldx, float* sx,
                        uint32_t* flags, double* partials, hipStream_t stream) {
  const int64_t chunks = stats_chunks(M);
  dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)chunks);
  switch (dtype) {
    case kF16:
      stats_partial_kernel<kF16><<<grid, 256, 0, stream>>>(X, M, K, ldx, partials);
      break;
    case kBF16:
      stats_partial_kernel<kBF16><<<grid, 256, 0, stream>>>(X, M, K, ldx, partials);
      break;
    default:
      stats_partial_kernel<kF32><<<grid, 256, 0, stream>>>(X, M, K, ldx, partials);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_stats_final(partials, chunks, M, K, dtype, sx, flags, stream);
}

hipError_t launch_stats_final(const double* partials, int64_t chunks, int64_t M, int64_t K,
                              int dtype, float* sx, uint32_t* flags, hipStream_t stream) {
  stats_final_kernel<<<(unsigned)((K + 31) / 32), 256, 0, stream>>>(partials, chunks, M, K,
                                                                     dtype, sx, flags);
  return hipGetLastError();
}

}  // namespace awq
