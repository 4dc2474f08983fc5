// Gram form of the AWQ loss: the objective of the AWQ notes (bg51717.github.io/14592, section
// 方法), L(s) = ||Q(W s)(s^-1 X) - W X||_F^2 / (M N), written with E = Q(W s)/s - W as
//   L = sum_n E_n H E_n^T / (M N),   H = X^T X,
// the quadratic form in H = X^T X that the GPTQ section of "量化方案详解"
// (luoboask.github.io/fde-learning/04-inference-optimization/quantization-schemes/) writes its
// layer objective as. H is computed once per layer; each grid point then costs a K x K
// contraction instead of an M x K one.
//
// Conditioning for fp16 operands. With d_k = sqrt(H_kk) (d_k = 0 for a channel that is zero in
// every token) the correlation matrix C = D^-1 H D^-1 has a unit diagonal and entries in
// [-1, 1], and E' = 2^e E D carries the loss: E_n H E_n^T = 2^-2e E'_n C E'_n^T. By symmetry,
//   E'_n C E'_n^T = 2 sum_l E'_nl P_nl,   P_nl = sum_{k<l} E'_nk C_kl + E'_nl / 2,
// so the contraction only needs B[l][k] = C_kl for k < l, 1/2 for k = l and 0 for k > l: a
// lower-triangular operand that halves the work and keeps the dominant diagonal exact.
//
// Kernels, in launch order:
//   gram_gemm_x      partials of H over chunks of tokens, upper-triangle 256 x 256 tiles only,
//                    read straight from fp16 X (the K loop of mfma_kloop.h on LDS transpose
//                    reads), fp32 accumulation, stored in fragment order;
//   gram_transpose   (bf16/fp32 X, or chunks past a 4 GiB buffer range) X [M, K] -> Xt [K, Mp]
//                    fp16, zero for m >= M, so that the token index is the contiguous
//                    reduction index; then gram_gemm, the same partials from Xt;
//   gram_diag        d_k = sqrt(sum over chunks of the H_kk partials) in fp64;
//   gram_finish      B from the fp64 sums of the partials (fixed chunk order);
//   gram_loss        per (grid point, row tile, column tile): P on the MFMA K loop, epilogue
//                    2 sum E'_nl P_nl against E' read back from the error stack.
#include "mfma_kloop.h"

namespace awq {

// ------------------------------------------------------------------------------------------
// Work split of X^T X over token chunks: every (tile, chunk) is one workgroup; the chunk count
// is picked so that the workgroups fill whole waves of the 256 compute units.
GramPlan gram_plan(int64_t M, int64_t K, bool diag) {
  GramPlan p{};
  p.t = (int)((K + kLossBN - 1) / kLossBN);
  p.diag = diag;
  p.T = diag ? (int64_t)p.t : (int64_t)p.t * (p.t + 1) / 2;
  p.Mp = (M + kGramMAlign - 1) / kGramMAlign * kGramMAlign;
  // at most kGramMaxChunks chunks, at least kGramMAlign tokens each, and no more than
  // kGramMaxBlocks workgroups once one chunk per tile is there (bounds the partials' memory)
  int64_t max_s = p.Mp / kGramMAlign < kGramMaxChunks ? p.Mp / kGramMAlign : kGramMaxChunks;
  if (max_s > kGramMaxBlocks / p.T) max_s = kGramMaxBlocks / p.T;
  if (max_s < 1) max_s = 1;
  int64_t best_cost = -1;
  for (int64_t s = 1; s <= max_s; ++s) {
    const int64_t per = (p.Mp + s - 1) / s;
    const int64_t chunk = (per + kGramMAlign - 1) / kGramMAlign * kGramMAlign;
    const int64_t se = (p.Mp + chunk - 1) / chunk;
    const int64_t waves = (p.T * se + 255) / 256;
    const int64_t cost = waves * chunk;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      p.chunk = chunk;
      p.S = (int)se;
    }
  }
  return p;
}

// ------------------------------------------------------------------------------------------
// One lane moves an 8 x 8 block: 8 rows of 16 bytes in, transposed in registers with byte
// permutes, 8 rows of 16 bytes out. Lane l of a wave takes channel block l % 8 and token block
// l / 8, so a load instruction reads 8 runs of 128 contiguous bytes (one per token row) and a
// store instruction writes 8 runs of 128 contiguous bytes (one per channel row of Xt).
template <int DT>
__global__ __launch_bounds__(256) void gram_transpose_kernel(const void* __restrict__ X,
                                                             int64_t M, int64_t K, int64_t Mp,
                                                             uint16_t* __restrict__ Xt,
                                                             uint32_t* __restrict__ flags) {
  constexpr int ES = (DT == kF32) ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t k0 = (int64_t)blockIdx.x * 64 + (lane & 7) * 8;
  const int64_t m0 = (int64_t)blockIdx.y * 256 + wave * 64 + (lane >> 3) * 8;
  // Mp is a multiple of 64: whole waves are past it together
  if (m0 >= Mp) return;
  bool over = false;
  uint32_t v[8][4];       // v[r][w]: channels 2w, 2w+1 of token row m0 + r
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t m = m0 + r;
    if (m < M) {
      if (DT == kF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(
            reinterpret_cast<const char*>(X) + (m * K + k0) * ES);
        v[r][0] = u.x; v[r][1] = u.y; v[r][2] = u.z; v[r][3] = u.w;
      } else {
        float f[8];
        load8_f32<DT>(reinterpret_cast<const char*>(X) + (m * K + k0) * ES, f);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint16_t lo = f2h(f[2 * w]), hi = f2h(f[2 * w + 1]);
          over |= ((lo & 0x7C00u) == 0x7C00u) || ((hi & 0x7C00u) == 0x7C00u);
          v[r][w] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) v[r][w] = 0u;
    }
  }
  // output row c (channel k0 + c) holds tokens m0..m0+7: word w = (token 2w, token 2w+1)
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(v[2 * w + 1][c >> 1], v[2 * w][c >> 1], sel);
    *reinterpret_cast<uint4*>(Xt + (k0 + c) * Mp + m0) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (DT != kF16) wave_flag(flags, over, kFlagXF16Range);
}

// ------------------------------------------------------------------------------------------
// Upper-triangle tile index -> (a, b), a <= b, row-major over a.
__device__ __forceinline__ void tri_tile(int64_t idx, int t, int& a, int& b) {
  int aa = 0;
  while (idx >= t - aa) {
    idx -= t - aa;
    ++aa;
  }
  a = aa;
  b = aa + (int)idx;
}

// Offset (in floats) of acc[i][j][e] of `lane` in `wave` inside a tile stored in fragment order:
// [wave][i][j][e / 4][lane][e % 4] -- each float4 store of a wave writes 1 KiB contiguously.
__device__ __forceinline__ int64_t frag_off(int wave, int i, int j, int e, int lane) {
  return ((((int64_t)(wave * 4 + i) * 4 + j) * 4 + (e >> 2)) * 64 + lane) * 4 + (e & 3);
}

__global__ __launch_bounds__(kloop::kThreads, 1) void gram_gemm_kernel(
    const uint16_t* __restrict__ Xt, int64_t K, int64_t Mp, int t, int64_t T, int64_t chunk,
    int diag, float* __restrict__ Hpart) {
  using namespace kloop;
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int64_t logical = xcd_logical(blockIdx.x, gridDim.x);
  const int64_t c = logical / T, tile = logical % T;    // chunk-major: neighbours share tokens
  int a, b;
  if (diag) {
    a = b = (int)tile;
  } else {
    tri_tile(tile, t, a, b);
  }
  const int64_t m0 = c * chunk;
  const int64_t clen = (Mp - m0 < chunk) ? Mp - m0 : chunk;   // multiple of 128
  const int64_t rows_a = (K - (int64_t)a * BM < BM) ? K - (int64_t)a * BM : BM;
  const int64_t rows_b = (K - (int64_t)b * BN < BN) ? K - (int64_t)b * BN : BN;
  Tile T_;
  T_.ra = make_rsrc(Xt + (int64_t)a * BM * Mp + m0, (uint32_t)(((rows_a - 1) * Mp + clen) * 2));
  T_.rb = make_rsrc(Xt + (int64_t)b * BN * Mp + m0, (uint32_t)(((rows_b - 1) * Mp + clen) * 2));
  tile_setup(T_, smem, (uint32_t)(Mp * 2));
  floatx16 acc[4][4];
  acc_zero(acc);
  kl_run(smem, T_, (int)(clen / BK), acc);

  // the partials are read once, by the finish pass: non-temporal stores keep these 256 KiB per
  // tile from displacing the X^T operand lines that the other workgroups are reading (-2%)
  const int lane = threadIdx.x & 63;
  float* out = Hpart + (c * T + tile) * (int64_t)(BM * BN);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        __builtin_nontemporal_store(
            floatx4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                    acc[i][j][4 * e4 + 3]},
            reinterpret_cast<floatx4*>(out + frag_off(T_.wave, i, j, 4 * e4, lane)));
}

// The same partials read straight from fp16 X [M, K] (no transposed copy): the tile's two
// channel panels of the chunk's tokens, gathered into MFMA fragments by LDS transpose reads
// (mfma_kloop.h, kl_run_x). Tokens past M read as zeros; channels past K read neighbouring
// values that only reach partial-tile entries no later pass uses.
__global__ __launch_bounds__(kloop::kThreads, 1) void gram_gemm_x_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t Mp, int t, int64_t T,
    int64_t chunk, int diag, float* __restrict__ Hpart) {
  using namespace kloop;
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const int64_t logical = xcd_logical(blockIdx.x, gridDim.x);
  const int64_t c = logical / T, tile = logical % T;
  int a, b;
  if (diag) {
    a = b = (int)tile;
  } else {
    tri_tile(tile, t, a, b);
  }
  const int64_t m0 = c * chunk;
  const int64_t clen = (Mp - m0 < chunk) ? Mp - m0 : chunk;   // multiple of 128
  const int64_t valid = (M - m0 < clen) ? M - m0 : clen;      // >= 1: m0 <= Mp - 128 < M
  TileX T_;
  T_.ra = make_rsrc(X + m0 * K + (int64_t)a * BM, (uint32_t)(valid * K * 2));
  T_.rb = make_rsrc(X + m0 * K + (int64_t)b * BN, (uint32_t)(valid * K * 2));
  tile_setup_x(T_, smem, (uint32_t)(K * 2));
  floatx16 acc[4][4];
  acc_zero(acc);
  kl_run_x(smem, T_, (int)(clen / BK), acc);

  const int lane = threadIdx.x & 63;
  float* out = Hpart + (c * T + tile) * (int64_t)(BM * BN);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        __builtin_nontemporal_store(
            floatx4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                    acc[i][j][4 * e4 + 3]},
            reinterpret_cast<floatx4*>(out + frag_off(T_.wave, i, j, 4 * e4, lane)));
}

// ------------------------------------------------------------------------------------------
// d_k = sqrt(H_kk): H_kk is element (k', k') of diagonal tile (a, a), k = 256 a + k'. In the
// fragment order that element sits in wave 3 (k' / 128), block (i, i) with i = (k' % 128) / 32,
// lane r + 32 ((r / 4) % 2) and register 4 (r / 8) + r % 4, r = k' % 32.
__global__ __launch_bounds__(256) void gram_diag_kernel(const float* __restrict__ Hpart,
                                                        int64_t K, int t, int64_t T, int S,
                                                        int diag, double* __restrict__ d64,
                                                        float* __restrict__ d32) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int a = (int)(k / kLossBN), kp = (int)(k % kLossBN);
  const int64_t tile = diag ? (int64_t)a : (int64_t)a * t - (int64_t)a * (a - 1) / 2;
  const int wm = kp >> 7, i = (kp & 127) >> 5, r = kp & 31;
  const int lane = r + 32 * ((r >> 2) & 1);
  const int e = 4 * (r >> 3) + (r & 3);
  const int64_t off = frag_off(3 * wm, i, i, e, lane);
  // the chunks' values are loaded eight at a time (past the last chunk: the last one again, not
  // added), then added in chunk order
  double h = 0.0;
  const float* src = Hpart + tile * (kLossBM * kLossBN) + off;
  const int64_t cs = T * (kLossBM * kLossBN);
  for (int c0 = 0; c0 < S; c0 += 8) {
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = src[(int64_t)(c0 + u < S ? c0 + u : S - 1) * cs];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < S) h += (double)p[u];
  }
  const double d = sqrt(h);
  d64[k] = d;
  d32[k] = (float)d;
}

// One thread per float4 of the fragment order: tokens-chunk sums in fp64 (chunk order fixed),
// then B[l][k..k+3] for the four channels k..k+3 (consecutive A rows) of output row l. With
// `diag`, B is stored as the diagonal blocks only: block a at B + 65536 a, row l - 256 a. With
// Blo, the diagonal blocks' low-order parts fp16(b - fp16(b)) go to Blo in that same layout
// (b the correlation in fp64): the clipping search carries the operand to ~2^-22 with them.
__global__ __launch_bounds__(256) void gram_finish_kernel(const float* __restrict__ Hpart,
                                                          int64_t K, int t, int64_t T, int S,
                                                          int diag,
                                                          const double* __restrict__ d64,
                                                          uint16_t* __restrict__ B,
                                                          uint16_t* __restrict__ Blo,
                                                          uint32_t* __restrict__ gram_k) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index
  constexpr int64_t kPerTile = kLossBM * kLossBN / 4;
  if (g == 0 && gram_k) *gram_k = (uint32_t)K;   // read by later launches only
  if (g >= T * kPerTile) return;
  const int64_t tile = g / kPerTile;
  const int rem = (int)(g % kPerTile);
  const int lane = rem & 63, e4 = (rem >> 6) & 3, j = (rem >> 8) & 3, i = (rem >> 10) & 3,
            wave = rem >> 12;
  int a, b;
  if (diag) {
    a = b = (int)tile;
  } else {
    tri_tile(tile, t, a, b);
  }
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t l = (int64_t)b * kLossBN + wn * 128 + 32 * j + (lane & 31);
  const int64_t k = (int64_t)a * kLossBM + wm * 128 + 32 * i + 8 * e4 + 4 * (lane >> 5);
  if (l >= K || k >= K) return;   // k is a multiple of 4 and K of 128: k..k+3 all valid
  // the chunks' partials are loaded eight at a time (independent loads in flight), then added in
  // chunk order
  double h[4] = {0.0, 0.0, 0.0, 0.0};
  const float* src = Hpart + tile * (4 * kPerTile) + (int64_t)rem * 4;
  const int64_t cs = T * (4 * kPerTile);
  for (int c0 = 0; c0 < S; c0 += 8) {
    float4 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)   // past the last chunk: the last chunk again, not added
      p[u] = *reinterpret_cast<const float4*>(src + (int64_t)(c0 + u < S ? c0 + u : S - 1) * cs);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c0 + u < S) {
        h[0] += (double)p[u].x;
        h[1] += (double)p[u].y;
        h[2] += (double)p[u].z;
        h[3] += (double)p[u].w;
      }
    }
  }
  const double dl = d64[l];
  uint16_t o[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t kq = k + q;
    double vd = 0.0;
    if (kq == l) {
      vd = 0.5;
    } else if (kq < l) {
      const double dk = d64[kq];
      vd = (dk > 0.0 && dl > 0.0) ? h[q] / (dk * dl) : 0.0;
    }
    o[q] = f2h((float)vd);
    lo[q] = f2h((float)(vd - (double)h2f(o[q])));
  }
  const int64_t doff = (int64_t)a * (kLossBM * kLossBN) + (l - (int64_t)a * kLossBN) * kLossBN +
                       (k - (int64_t)a * kLossBM);
  // B is K-blocked, [K / 32][K][32] (with diag: per block, [8][256][32]): the 256 x 32 piece of
  // one K step of the loss contraction is contiguous
  const int64_t kl = k - (int64_t)a * kLossBM, ll = l - (int64_t)a * kLossBN;
  const int64_t off = diag ? (int64_t)a * (kLossBM * kLossBN) + (kl >> 5) * (kLossBN * 32) +
                                 ll * 32 + (kl & 31)
                           : (k >> 5) * (K * 32) + l * 32 + (k & 31);
  *reinterpret_cast<uint2*>(B + off) =
      make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
  if (Blo && a == b)
    *reinterpret_cast<uint2*>(Blo + doff) = make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16),
                                                       (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
}

// ------------------------------------------------------------------------------------------
// Workgroup (grid point, row tile nt, column tile lt): column tile lt needs the K steps of
// channels below 256 (lt + 1) only. Row panels (grid point, nt) go in groups of kLossPanelGroup;
// inside a group the logical order runs over the column tiles longest first and, for each, over
// the group's panels. The 32 workgroups resident on an XCD then hold the longest tiles of a few
// panels at once: each B column panel is read by up to kLossPanelGroup of them and each E'
// panel by several, so both operands are shared in the XCD's L2 (panel-major order shared only
// the E' panel and streamed B once per panel: 9% slower; groups of 16 or more panels stream
// the E' panels instead). The short tiles fill in behind the long ones. (Pairing tiles lt and
// t-1-lt in one workgroup balances the work exactly but was slower: the second tile of a pair
// runs out of phase with its neighbours and loses the L2 sharing.)
constexpr int kLossPanelGroup = 8;

__global__ __launch_bounds__(kloop::kThreads, 1) void gram_loss_kernel(
    const uint16_t* __restrict__ Est, int64_t N, int64_t K, const uint16_t* __restrict__ B,
    int tilesN, int t, double* __restrict__ partials) {
  using namespace kloop;
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  __shared__ double wsum[4];
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int n_panels = (int)(gridDim.x / t);
  const int grp = logical / (kLossPanelGroup * t), q = logical % (kLossPanelGroup * t);
  const int gp = (n_panels - grp * kLossPanelGroup < kLossPanelGroup)
                     ? n_panels - grp * kLossPanelGroup : kLossPanelGroup;   // panels in group
  const int lt = t - 1 - q / gp;
  const int panel = grp * kLossPanelGroup + q % gp;
  const int alpha = panel / tilesN, nt = panel % tilesN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t rows = (N - (int64_t)nt * BM < BM) ? N - (int64_t)nt * BM : BM;
  const int nk_all = (int)(K / BK);

  // both operands K-blocked: E' [n_grid][K / 32][N][32], B [K / 32][K][32]
  TileK T_;
  T_.pa = reinterpret_cast<const char*>(Est + (int64_t)alpha * N * K + (int64_t)nt * BM * BK);
  T_.ka = (uint64_t)N * kRowBytes;
  T_.na = (uint32_t)(rows * kRowBytes);
  const int64_t brows = (K - (int64_t)lt * BN < BN) ? K - (int64_t)lt * BN : BN;
  T_.pb = reinterpret_cast<const char*>(B + (int64_t)lt * BN * BK);
  T_.kb = (uint64_t)K * kRowBytes;
  T_.nb = (uint32_t)(brows * kRowBytes);
  T_.nkb = nk_all;
  tile_setup_k(T_, smem);   // columns interleaved: block j of column half wn is c = 2 j + wn
  const int wn = T_.wave & 1;   // the wave's column half of the tile
  {
    const int nk = (8 * (lt + 1) < nk_all) ? 8 * (lt + 1) : nk_all;
    floatx16 acc[4][4];
    acc_zero(acc);
    // The epilogue needs the E' tile [256 n][256 l]: operand A of steps 8 lt .. 8 lt + 7. A full
    // tile (the last eight steps are exactly these) keeps them in LDS: steps 8 lt + 4 + s stay in
    // the A half of stage s, and steps 8 lt + s are loaded again into the free B half of stage s
    // during the last four steps. The ragged last tile (K % 256 != 0) loads all eight after the
    // loop; its columns past K read as zeros (K blocks past the last) and are masked below
    // anyway.
    if (nk == 8 * (lt + 1)) {
      kl_run_t<true, true, TileK>(smem, T_, nk, acc);
    } else {
      kl_run(smem, T_, nk, acc);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kl_issue_a_to_b(T_, s4, 8 * lt + s4, j);
          kl_issue(T_, s4, 8 * lt + 4 + s4, 2 * j);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt(0));
    __syncthreads();

    // epilogue: sum over the tile of E'_nl P_nl (P = acc). Columns l of block (wn, j) are
    // c = 2 j + wn, those of step 8 lt + c. Two MFMAs against the identity put the E' block into
    // the layout of the accumulators exactly (one product by 1 per element, fp16 -> fp32 is exact):
    // D = A_0 I_0 + A_1 I_1 with I_h[k][c] = (c == 16 h + k) over the block's 32 columns.
    const int l32 = lane & 31, lh = lane >> 5;
    half8_t id0, id1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      id0[q] = (_Float16)((l32 == 8 * lh + q) ? 1.0f : 0.0f);
      id1[q] = (_Float16)((l32 == 16 + 8 * lh + q) ? 1.0f : 0.0f);
    }
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 2 * j + wn;
        const char* src = smem + (c & 3) * kStageBytes + (c >= 4 ? 0 : BM * kRowBytes);
        const half8_t f0 = *reinterpret_cast<const half8_t*>(src + T_.rd[0][0] + i * 32 * kRowBytes);
        const half8_t f1 = *reinterpret_cast<const half8_t*>(src + T_.rd[0][1] + i * 32 * kRowBytes);
        floatx16 ev = {};
        ev = __builtin_amdgcn_mfma_f32_32x32x16_f16(f0, id0, ev, 0, 0, 0);
        ev = __builtin_amdgcn_mfma_f32_32x32x16_f16(f1, id1, ev, 0, 0, 0);
        const int lcol = 32 * c + l32;
        const bool lok = (int64_t)lt * BN + lcol < K;
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) s = __builtin_fmaf(ev[e], acc[i][j][e], s);
        tot += lok ? (double)s : 0.0;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    if (lane == 0) wsum[T_.wave] = tot;
    __syncthreads();
    if (tid == 0) {
      const double v = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
      partials[(int64_t)alpha * ((int64_t)tilesN * t) + (int64_t)nt * t + lt] = 2.0 * v;
    }
  }
}

// ------------------------------------------------------------------------------------------
bool gram_direct_x(const GramPlan& p, int64_t K) {
  // a chunk's rows must stay within one buffer range (32-bit offsets)
  return p.chunk * K * 2 < (int64_t(1) << 32);
}

hipError_t launch_gram_transpose(const void* X, int xdt, int64_t M, int64_t K, int64_t Mp,
                                 uint16_t* Xt, uint32_t* flags, hipStream_t stream) {
  dim3 grid((unsigned)(K / 64), (unsigned)((Mp + 255) / 256));
  switch (xdt) {
    case kF16:
      gram_transpose_kernel<kF16><<<grid, 256, 0, stream>>>(X, M, K, Mp, Xt, flags);
      break;
    case kBF16:
      gram_transpose_kernel<kBF16><<<grid, 256, 0, stream>>>(X, M, K, Mp, Xt, flags);
      break;
    default:
      gram_transpose_kernel<kF32><<<grid, 256, 0, stream>>>(X, M, K, Mp, Xt, flags);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gram_hmat(const uint16_t* Xt, int64_t K, const GramPlan& p, float* Hpart,
                            double* d64, float* d32, uint16_t* B, uint16_t* Blo,
                            uint32_t* gram_k, hipStream_t stream, hipEvent_t ev, hipEvent_t ev2,
                            const uint16_t* X, int64_t M) {
  if (X)
    gram_gemm_x_kernel<<<(unsigned)(p.T * p.S), kloop::kThreads, 0, stream>>>(
        X, M, K, p.Mp, p.t, p.T, p.chunk, (int)p.diag, Hpart);
  else
    gram_gemm_kernel<<<(unsigned)(p.T * p.S), kloop::kThreads, 0, stream>>>(
        Xt, K, p.Mp, p.t, p.T, p.chunk, (int)p.diag, Hpart);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev, stream);
  if (e == hipSuccess && ev2) e = hipEventRecord(ev2, stream);
  if (e == hipSuccess) {
    gram_diag_kernel<<<(unsigned)((K + 255) / 256), 256, 0, stream>>>(Hpart, K, p.t, p.T, p.S,
                                                                      (int)p.diag, d64, d32);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    const int64_t threads = p.T * (kLossBM * kLossBN / 4);
    gram_finish_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(Hpart, K, p.t, p.T,
                                                                              p.S, (int)p.diag,
                                                                              d64, B, Blo, gram_k);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_gram_prepare(const void* X, int xdt, int64_t M, int64_t K, const GramPlan& p,
                               uint16_t* Xt, float* Hpart, double* d64, float* d32, uint16_t* B,
                               uint16_t* Blo, uint32_t* gram_k, uint32_t* flags,
                               hipStream_t stream, hipEvent_t* ev) {
  const bool direct = xdt == kF16 && gram_direct_x(p, K);
  hipError_t e = direct ? hipSuccess
                        : launch_gram_transpose(X, xdt, M, K, p.Mp, Xt, flags, stream);
  if (e == hipSuccess && ev) e = hipEventRecord(ev[0], stream);
  if (e == hipSuccess)
    e = launch_gram_hmat(Xt, K, p, Hpart, d64, d32, B, Blo, gram_k, stream, ev ? ev[1] : nullptr,
                         nullptr, direct ? static_cast<const uint16_t*>(X) : nullptr, M);
  return e;
}

hipError_t launch_gram_loss(const uint16_t* Estack, int64_t N, int64_t K, const uint16_t* B,
                            int n_grid, double* partials, hipStream_t stream) {
  const int tilesN = (int)((N + kLossBM - 1) / kLossBM);
  const int t = (int)((K + kLossBN - 1) / kLossBN);
  const int64_t blocks = (int64_t)n_grid * tilesN * t;
  gram_loss_kernel<<<(unsigned)blocks, kloop::kThreads, 0, stream>>>(Estack, N, K, B, tilesN, t,
                                                                     partials);
  return hipGetLastError();
}

}  // namespace awq
