// Loss contraction of the AWQ grid search for layers with few weight rows or few tokens:
//   partial[i][tile] = sum over the tile's tokens m and rows n of ( sum_k X[m,k] E_i[n,k] )^2,
// the objective of the AWQ notes (bg51717.github.io/14592, section 方法) with E_i = Q(W s_i)/s_i
// - W, on the vector ALUs with fp32 operands: X is read in its own dtype (fp16, bf16 and fp32
// values are all exact in fp32) and E_i comes from an fp32 error stack. The fp16 contractions
// (lossgemm.hip, gram.hip) round every E entry to 11 bits; over many rows those errors average
// out, but with a handful of rows one output's error is systematic (~5e-4 of the loss for a
// single row). Here every product is an fp32 product of exact operands, sums of 256 channels are
// fp32, and everything beyond is fp64: the loss is within ~1e-6 of the exact one.
//
// Work split: a workgroup of 256 threads takes 256 tokens (one per thread), kRows weight rows and
// one grid point. Each thread walks its token's row of X in 128-byte steps (all loads of a step
// issued together, so each line is fetched once), and the error rows, which are the same for the
// whole wave, are read with uniform addresses -- scalar loads feeding the FMAs' scalar operand.
// Workgroups are ordered grid point fastest and dealt to the XCDs in contiguous ranges, so the
// grid points of one token block run together on one XCD and share its lines of X in L2.
// The partial of each (token block, row chunk) is reduced in a fixed order: deterministic.
#include "device_common.h"
#include "kernels.h"
#include "mfma_kloop.h"

namespace awq {

namespace {
constexpr int kVRows = 16;       // weight rows per workgroup
constexpr int kVFold = 256;      // channels summed in fp32 before the fp64 accumulator
}  // namespace

template <int DT>
__global__ __launch_bounds__(256) void loss_valu_kernel(const void* __restrict__ X, int64_t M,
                                                        int64_t K, const float* __restrict__ Est,
                                                        int64_t N, int64_t ld_rows, int n_grid,
                                                        int tiles_tok, int chunks,
                                                        double* __restrict__ partials) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  constexpr int CK = 128 / ES;     // channels per 128-byte step of a token's row
  const int logical = kloop::xcd_logical(blockIdx.x, gridDim.x);
  const int alpha = logical % n_grid;
  const int rest = logical / n_grid;
  const int rc = rest % chunks;
  const int tb = rest / chunks;
  const int tid = threadIdx.x;
  const int64_t m = (int64_t)tb * 256 + tid;
  const bool live = m < M;
  const char* xrow = reinterpret_cast<const char*>(X) + (live ? m : M - 1) * K * ES;
  const int64_t r0 = (int64_t)rc * kVRows;
  const int nr = (int)((N - r0 < kVRows) ? N - r0 : kVRows);   // uniform
  const float* __restrict__ E = Est + ((int64_t)alpha * ld_rows + r0) * K;

  double acc64[kVRows];
  float acc[kVRows];
#pragma unroll
  for (int r = 0; r < kVRows; ++r) {
    acc64[r] = 0.0;
    acc[r] = 0.0f;
  }
  for (int64_t k0 = 0; k0 < K; k0 += CK) {
    uint4 raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = *reinterpret_cast<const uint4*>(xrow + k0 * ES + 16 * u);
    float x[CK];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (DT == kF32) {
        x[4 * u] = __uint_as_float(raw[u].x);
        x[4 * u + 1] = __uint_as_float(raw[u].y);
        x[4 * u + 2] = __uint_as_float(raw[u].z);
        x[4 * u + 3] = __uint_as_float(raw[u].w);
      } else {
        const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint16_t lo = (uint16_t)(w[t] & 0xFFFFu), hi = (uint16_t)(w[t] >> 16);
          x[8 * u + 2 * t] = (DT == kF16) ? h2f(lo) : bf2f(lo);
          x[8 * u + 2 * t + 1] = (DT == kF16) ? h2f(hi) : bf2f(hi);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kVRows; ++r) {
      if (r < nr) {   // uniform
        const float* er = E + (int64_t)r * K + k0;
#pragma unroll
        for (int t = 0; t < CK; ++t) acc[r] = __builtin_fmaf(x[t], er[t], acc[r]);
      }
    }
    if (((k0 + CK) % kVFold) == 0 || k0 + CK >= K) {
#pragma unroll
      for (int r = 0; r < kVRows; ++r) {
        acc64[r] += (double)acc[r];
        acc[r] = 0.0f;
      }
    }
  }
  double tot = 0.0;
  if (live) {
#pragma unroll
    for (int r = 0; r < kVRows; ++r) tot += acc64[r] * acc64[r];   // rows >= nr hold 0
  }
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  __shared__ double wsum[4];
  if ((tid & 63) == 0) wsum[tid >> 6] = tot;
  __syncthreads();
  if (tid == 0) {
    const double t = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    partials[(int64_t)alpha * ((int64_t)tiles_tok * chunks) + (int64_t)tb * chunks + rc] = t;
  }
}

int64_t loss_valu_tiles(int64_t M, int64_t N) {
  return ((M + 255) / 256) * ((N + kVRows - 1) / kVRows);
}

hipError_t launch_loss_valu(const void* X, int xdt, int64_t M, int64_t K, const float* Estack,
                            int64_t N, int n_grid, double* partials, hipStream_t stream) {
  const int tiles_tok = (int)((M + 255) / 256);
  const int chunks = (int)((N + kVRows - 1) / kVRows);
  const int64_t blocks = (int64_t)tiles_tok * chunks * n_grid;
#define AWQ_LV(DT_)                                                                              \
  loss_valu_kernel<DT_><<<(unsigned)blocks, 256, 0, stream>>>(X, M, K, Estack, N, N, n_grid,    \
                                                               tiles_tok, chunks, partials)
  if (xdt == kF16)
    AWQ_LV(kF16);
  else if (xdt == kBF16)
    AWQ_LV(kBF16);
  else
    AWQ_LV(kF32);
#undef AWQ_LV
  return hipGetLastError();
}

}  // namespace awq
