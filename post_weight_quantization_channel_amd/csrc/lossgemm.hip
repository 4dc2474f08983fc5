// Loss contraction of the AWQ grid search:
//   partial[i][tile] = sum over the tile's (m, n) of ( sum_k X[m,k] * E_i[n,k] )^2
// for all grid points i at once, as one GEMM X [M,K] x [E_0; ...; E_{n-1}]^T whose M x (n N)
// output is never stored: the epilogue squares and reduces each 256x256 tile in registers.
// With E_i = Q(W s_i)/s_i - W this is ||Q(W s_i)(s_i^-1 X) - W X||_F^2 restricted to the tile,
// the objective of the AWQ notes (bg51717.github.io/14592, section 方法).
//
// gfx950 design:
//   * 256 threads = 4 waves (2 x 2), workgroup tile 256 x 256, wave tile 128 x 128, BK = 32;
//   * v_mfma_f32_32x32x16_f16: 4 x 4 MFMA blocks per wave, 256 fp32 accumulators per lane
//     (held in AGPRs; one wave per SIMD);
//   * operands go from HBM straight into LDS (buffer_load_dwordx4 ... lds): no staging
//     registers and no ds_write; each wave instruction fills 1 KiB = 16 rows x 64 bytes. The
//     buffer range of each operand panel ends at its last valid row, so rows of a ragged tile
//     read as zeros without branches;
//   * four LDS stages of 32 KiB: the loads of steps k+1..k+4 are in flight while step k
//     computes (one stage ahead left the waves waiting ~40% of the time on loads whose lines
//     missed L2; LDS bank conflicts: none). Fragment reads of the next step overlap the second
//     half of the current step's MFMAs;
//   * LDS layout: row r holds its 4 chunks of 16 bytes at positions c ^ f(r),
//     f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1), so the 128-bit fragment reads of 8 (and of 16)
//     consecutive rows at one chunk touch distinct banks whether the LDS has 32 or 64 banks;
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
constexpr int kStages = 4;
constexpr int kRowBytes = BK * 2;                           // 64 bytes of a row per K step
constexpr int kStageBytes = (BM + BN) * kRowBytes;          // 32 KiB per stage
constexpr int kRowsPerWave = BM / 4;                        // rows each wave loads per operand
constexpr int kRowsPerInst = 1024 / kRowBytes;              // 16 rows per 1 KiB wave load
constexpr int kInstPerOp = kRowsPerWave / kRowsPerInst;     // 4 loads per operand per step

__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding (gfx9
// encoding: vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

}  // namespace

// The K loop over four LDS stages (addresses base + j * kStageBytes).
//
// Per step kt (stage kt % 4): read the second half (k 16..31) of the stage's fragments, issue the
// 16 MFMAs of the first half, wait until step kt+1 has landed (steps kt+2, kt+3 may still be in
// flight) and until this wave's LDS reads are done, barrier, refill stage kt with step kt+4,
// read the first half of step kt+1's fragments, issue the 16 MFMAs of the second half of step kt.
struct LossTile {
  rsrc_t ra, rb;        // operand panels
  uint32_t voff;        // this lane's byte offset for load j = 0, step 0
  uint32_t row_stride;  // bytes between rows (K * 2)
  int wave, wm, wn, frow, fhalf;
};

__device__ __forceinline__ void loss_kloop(const char* smem, const LossTile& T, int nk,
                                           floatx16 (&acc)[4][4]) {
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int stage, int kt) {
    const uint32_t la = lds0 + (uint32_t)(stage * kStageBytes);
    const uint32_t lb = la + (uint32_t)(BM * kRowBytes);
    const uint32_t kofs = (uint32_t)kt * (uint32_t)kRowBytes;
#pragma unroll
    for (int j = 0; j < kInstPerOp; ++j) {
      const uint32_t o = T.voff + (uint32_t)(kRowsPerInst * j) * T.row_stride + kofs;
      const uint32_t row_ofs = (uint32_t)((T.wave * kRowsPerWave + kRowsPerInst * j) * kRowBytes);
      buffer_load16_lds(T.ra, la + row_ofs, o);
      buffer_load16_lds(T.rb, lb + row_ofs, o);
    }
  };
  auto read_frags = [&](int stage, int kk, half8_t (&af)[4], half8_t (&bf)[4]) {
    const char* sa = smem + stage * kStageBytes;
    const char* sb = sa + BM * kRowBytes;
    const int chunk = kk * 2 + T.fhalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = T.wm * 128 + i * 32 + T.frow;
      af[i] = *reinterpret_cast<const half8_t*>(sa + r * kRowBytes + ((chunk ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = T.wn * 128 + j * 32 + T.frow;
      bf[j] = *reinterpret_cast<const half8_t*>(sb + r * kRowBytes + ((chunk ^ swz(r)) << 4));
    }
  };
  auto mfma16 = [&](const half8_t (&af)[4], const half8_t (&bf)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
  };

  half8_t a0[4], b0[4], a1[4], b1[4];
  auto step = [&](int stage, int kt) {
    read_frags(stage, 1, a1, b1);
    mfma16(a0, b0);
    // wait: step kt+1 landed (this wave's loads) and this wave's LDS reads returned
    if (kt + 3 < nk) __builtin_amdgcn_s_waitcnt(vmcnt(16) & ~0x0F00);
    else if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(vmcnt(8) & ~0x0F00);
    else __builtin_amdgcn_s_waitcnt(vmcnt(0) & ~0x0F00);
    __syncthreads();
    if (kt + 4 < nk) issue(stage, kt + 4);
    if (kt + 1 < nk) read_frags((stage + 1) & 3, 0, a0, b0);
    mfma16(a1, b1);
  };

#pragma unroll
  for (int p = 0; p < kStages; ++p) issue(p, p);   // nk >= 4 (K is a multiple of 128)
  __builtin_amdgcn_s_waitcnt(vmcnt(24));           // step 0 has landed
  __syncthreads();
  read_frags(0, 0, a0, b0);
  for (int q = 0; q < nk; q += 4) {
    step(0, q);
    step(1, q + 1);
    step(2, q + 2);
    step(3, q + 3);
  }
}

__global__ __launch_bounds__(kThreads, 1) void lossgemm_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Est,
    int64_t N, int tilesM, int tilesN, int n_grid, double* __restrict__ partials) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];

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

  // ---- operand panels as buffer ranges ---------------------------------------------------
  const int64_t a_rows = (M - (int64_t)mt * BM < BM) ? M - (int64_t)mt * BM : BM;
  const int64_t b_rows = (N - (int64_t)nt * BN < BN) ? N - (int64_t)nt * BN : BN;
  LossTile T;
  T.ra = make_rsrc(X + (int64_t)mt * BM * K, (uint32_t)(a_rows * K * 2));
  T.rb = make_rsrc(Est + ((int64_t)alpha * N + (int64_t)nt * BN) * K, (uint32_t)(b_rows * K * 2));
  T.wave = tid >> 6;
  T.wm = T.wave >> 1;
  T.wn = T.wave & 1;
  T.frow = lane & 31;   // fragment row within a 32-row block
  T.fhalf = lane >> 5;  // which 8-element half of a 16-wide k slice
  // lane l of load instruction j fills LDS row wave*64 + 16j + l/4, physical chunk l%4, i.e.
  // the logical chunk (l%4) ^ swz(row); swz depends on row % 16 = l/4 only.
  const int lrow = lane >> 2;
  T.row_stride = (uint32_t)(K * 2);
  T.voff = (uint32_t)(T.wave * kRowsPerWave + lrow) * T.row_stride +
           (uint32_t)(((lane & 3) ^ swz(lrow)) * 16);

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  loss_kloop(smem, T, (int)(K / BK), acc);

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
  const int tilesM = (int)((M + BM - 1) / BM);
  const int tilesN = (int)((N + BN - 1) / BN);
  const int64_t blocks = (int64_t)tilesM * tilesN * n_grid;
  lossgemm_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(X16, M, K, Estack, N, tilesM,
                                                             tilesN, n_grid, partials);
  return hipGetLastError();
}

}  // namespace awq
