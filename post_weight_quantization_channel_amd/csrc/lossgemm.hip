// Loss contraction of the AWQ grid search (direct form):
//   partial[i][tile] = sum over the tile's (m, n) of ( sum_k X[m,k] * E_i[n,k] )^2
// for all grid points i at once, as one GEMM X [M,K] x [E_0; ...; E_{n-1}]^T whose M x (n N)
// output is never stored: the epilogue squares and reduces each 256x256 tile in registers.
// With E_i = Q(W s_i)/s_i - W this is ||Q(W s_i)(s_i^-1 X) - W X||_F^2 restricted to the tile,
// the objective of the AWQ notes (bg51717.github.io/14592, section 方法).
//
// The K loop (LDS pipeline, MFMA blocks) is the one of mfma_kloop.h. Here:
//   * tile order: blocks are dealt round-robin to the 8 XCDs, so block b is remapped to give
//     each XCD a contiguous range of tiles, and tiles are walked in groups of 8 M-tiles so the
//     32 workgroups resident on one XCD share X and E panels in that XCD's L2;
//   * epilogue: per lane, squares summed in fp32 per 32x32 block, blocks summed in fp64, wave
//     and workgroup reductions in fp64 in a fixed order: the partial is deterministic.
#include "mfma_kloop.h"

namespace awq {

namespace {
constexpr int kGroupM = 8;   // M-tiles walked together (they share E panels in L2)
}  // namespace

__global__ __launch_bounds__(kloop::kThreads, 1) void lossgemm_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Est,
    int64_t N, int tilesM, int tilesN, int n_grid, double* __restrict__ partials) {
  using namespace kloop;
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];

  // ---- tile assignment -------------------------------------------------------------------
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
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

  // ---- operand panels as buffer ranges ---------------------------------------------------
  const int64_t a_rows = (M - (int64_t)mt * BM < BM) ? M - (int64_t)mt * BM : BM;
  const int64_t b_rows = (N - (int64_t)nt * BN < BN) ? N - (int64_t)nt * BN : BN;
  Tile T;
  T.ra = make_rsrc(X + (int64_t)mt * BM * K, (uint32_t)(a_rows * K * 2));
  T.rb = make_rsrc(Est + ((int64_t)alpha * N + (int64_t)nt * BN) * K, (uint32_t)(b_rows * K * 2));
  tile_setup(T, smem, (uint32_t)(K * 2));

  floatx16 acc[4][4];
  acc_zero(acc);
  kl_run(smem, T, (int)(K / BK), acc);

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
  if (lane == 0) wsum[T.wave] = tot;
  __syncthreads();
  if (tid == 0) {
    const double t = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    partials[(int64_t)alpha * ((int64_t)tilesM * tilesN) + (int64_t)mt * tilesN + nt] = t;
  }
}

hipError_t launch_lossgemm(const uint16_t* X16, int64_t M, int64_t K, const uint16_t* Estack,
                           int64_t N, int n_grid, double* partials, hipStream_t stream) {
  const int tilesM = (int)((M + kloop::BM - 1) / kloop::BM);
  const int tilesN = (int)((N + kloop::BN - 1) / kloop::BN);
  const int64_t blocks = (int64_t)tilesM * tilesN * n_grid;
  lossgemm_kernel<<<(unsigned)blocks, kloop::kThreads, 0, stream>>>(X16, M, K, Estack, N, tilesM,
                                                                    tilesN, n_grid, partials);
  return hipGetLastError();
}

}  // namespace awq
