// Loss contraction of the AWQ grid search:
//   partial[i][tile] = sum over the tile's (m, n) of ( sum_k X[m,k] * E_i[n,k] )^2
// for all grid points i at once, as one GEMM X [M,K] x [E_0; ...; E_{n-1}]^T whose M x (n N)
// output is never stored: the epilogue squares and reduces each 256x256 tile in registers.
// With E_i = Q(W s_i)/s_i - W this is ||Q(W s_i)(s_i^-1 X) - W X||_F^2 restricted to the tile,
// the objective of the AWQ notes (bg51717.github.io/14592, section 方法).
//
// gfx950 design:
//   * 256 threads = 4 waves (2 x 2), workgroup tile 256 x 256, wave tile 128 x 128, BK = 64;
//   * v_mfma_f32_32x32x16_f16: 4 x 4 MFMA blocks per wave, 256 fp32 accumulators per lane
//     (held in AGPRs; one wave per SIMD);
//   * both operands are K-contiguous rows; global -> register -> LDS staging, double-buffered
//     (2 x 64 KiB), one barrier per K step; the 16-byte chunks of each 128-byte LDS row are
//     XOR-swizzled by (row & 7) so the 128-bit fragment reads of 8 consecutive rows hit
//     distinct banks;
//   * tile order: blocks are dealt round-robin to the 8 XCDs, so block b is remapped to give
//     each XCD a contiguous range of tiles, and tiles are walked in groups of 8 M-tiles so the
//     32 workgroups resident on one XCD share X and E panels in that XCD's L2;
//   * epilogue: per lane, squares summed in fp32 per 32x32 block, blocks summed in fp64, wave
//     and workgroup reductions in fp64 in a fixed order: the partial is deterministic.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {

constexpr int BM = kLossBM, BN = kLossBN, BK = kLossBK;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kRowsPerPass = kThreads / (BK / 8);           // 32 rows per load pass
constexpr int kLoadsPerOp = BM / kRowsPerPass;              // 8 x 16-byte loads per operand
constexpr int kStageHalves = (BM + BN) * BK;                // halves per LDS stage

__device__ __forceinline__ int swz(int row, int chunk) {   // half offset inside a stage operand
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void lossgemm_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Est,
    int64_t N, int tilesM, int tilesN, int n_grid, double* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * kStageHalves];

  // ---- tile assignment -------------------------------------------------------------------
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int per = G / 8, rem = G % 8, xcd = b % 8, loc = b / 8;
  const int logical = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int tilesNp = n_grid * tilesN;
  const int group_size = kGroupM * tilesNp;
  const int gid = logical / group_size;
  const int first_m = gid * kGroupM;
  const int gm = (tilesM - first_m < kGroupM) ? tilesM - first_m : kGroupM;
  const int in_group = logical % group_size;
  const int mt = first_m + in_group % gm;
  const int ntp = in_group / gm;
  const int alpha = ntp / tilesN;
  const int nt = ntp % tilesN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global load mapping: row = tid/8 + 32*j, 16-byte chunk = tid%8 ---------------------
  const int lchunk = tid & 7;
  const int lrow = tid >> 3;
  // row j of this thread's load set is lrow + 32 j; one base pointer per operand plus the
  // uniform stride 32 K keeps the addresses in a few registers.
  const int64_t arow0 = (int64_t)mt * BM + lrow;
  const int64_t brow0 = (int64_t)nt * BN + lrow;
  const int64_t a_left = M - arow0;   // rows of this thread's set that exist: 32 j < a_left
  const int64_t b_left = N - brow0;
  const uint16_t* abase = X + arow0 * K + lchunk * 8;
  const uint16_t* bbase = Est + ((int64_t)alpha * N + brow0) * K + lchunk * 8;
  const int64_t jstride = (int64_t)kRowsPerPass * K;

  uint4 ra[kLoadsPerOp], rb[kLoadsPerOp];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < kLoadsPerOp; ++j) {
      ra[j] = (kRowsPerPass * j < a_left)
                  ? *reinterpret_cast<const uint4*>(abase + j * jstride + k0)
                  : make_uint4(0, 0, 0, 0);
      rb[j] = (kRowsPerPass * j < b_left)
                  ? *reinterpret_cast<const uint4*>(bbase + j * jstride + k0)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    _Float16* sa = smem + stage * kStageHalves;
    _Float16* sb = sa + BM * BK;
#pragma unroll
    for (int j = 0; j < kLoadsPerOp; ++j) {
      const int r = lrow + kRowsPerPass * j;
      *reinterpret_cast<uint4*>(sa + swz(r, lchunk)) = ra[j];
      *reinterpret_cast<uint4*>(sb + swz(r, lchunk)) = rb[j];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int frow = lane & 31;   // fragment row within a 32-row block
  const int fhalf = lane >> 5;  // which 8-element half of the 16-wide k slice
  const int nk = (int)(K / BK);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
    const _Float16* sa = smem + stage * kStageHalves;
    const _Float16* sb = sa + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = kk * 2 + fhalf;
      half8_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + frow;
        af[i] = *reinterpret_cast<const half8_t*>(sa + swz(r, chunk));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + frow;
        bf[j] = *reinterpret_cast<const half8_t*>(sb + swz(r, chunk));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: sum of squares, fixed order ---------------------------------------------
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s = __builtin_fmaf(acc[i][j][e], acc[i][j][e], s);
      tot += (double)s;
    }
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  __shared__ double wsum[4];
  if (lane == 0) wsum[wave] = tot;
  __syncthreads();
  if (tid == 0) {
    const double t = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    partials[(int64_t)alpha * ((int64_t)tilesM * tilesN) + (int64_t)mt * tilesN + nt] = t;
  }
}

hipError_t launch_lossgemm(const uint16_t* X16, int64_t M, int64_t K, const uint16_t* Estack,
                           int64_t N, int n_grid, double* partials, hipStream_t stream) {
  const int tilesM = (int)((M + BM - 1) / BM);
  const int tilesN = (int)((N + BN - 1) / BN);
  const int64_t blocks = (int64_t)tilesM * tilesN * n_grid;
  lossgemm_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(X16, M, K, Estack, N, tilesM,
                                                             tilesN, n_grid, partials);
  return hipGetLastError();
}

}  // namespace awq
