// W4A16 GEMM on the packed AWQ artefacts: QuantLinear.forward of "AWQ 量化方案..."
// (qwbw.cn/news/39982), section 三 -- scale the input per channel, dequantize the packed codes
// with the per-group steps, then a linear layer:
//   Y[m, n] = sum_k (A[m,k] / s[k]) * c(q[n,k]) * step[n, k/G],
// c(q) = q for symmetric codes, q - z[n, k/G] for zero-point codes. The activation is divided by
// s because the weight was multiplied by s (AWQ notes, bg51717.github.io/14592, section 方法).
//
// Kernels by batch size M:
//   M = 1        w4a16_gemv.hip: fp16 dot products against a block-scaled A / s table;
//   2 <= M <= 64 w4a16_skinny.hip: MFMA with the activations read straight from memory; with a
//                workspace, where it pays, w4a16_splitk.hip: K split over workgroups of 64
//                weight rows;
//   M > 64       the tiled kernel below (and from 49 rows on for weights of 8192 rows or more);
//                with a workspace, while the tiles leave CUs idle, on K slices whose fp32
//                partials w4a16_sum_slices_kernel adds in slice order.
// All of them apply 1/s without an fp16 value that a tiny s could overflow: either A / s is kept
// in fp32 and stored scaled by a power of two per 128-channel block, or the weight operand is
// fp16(q r_k) with r_k = fp16(2^b / s_k), 2^b chosen per block so that the block's largest r_k lies
// in [2^10, 2^11), and 2^-b rides on the fp32 group step.
#include "device_common.h"
#include "kernels.h"

namespace awq {

// ---------------------------------------------------------------------------------------------
// Larger batches: a tiled MFMA GEMM. Workgroup tile 128 (batch rows m) x 64 (weight rows n), one
// 128-channel block of K per step, 4 waves of 64 x 32 (2 x 2), each a grid of 4 (m) x 2 (n)
// v_mfma_f32_16x16x32_f16 blocks (weights as the A operand, activations as B); for groups of 64
// or zero points 4 waves of 128 x 16; on small grids tiles of 64 batch rows (waves of 32 x 32 or
// 64 x 16).
//
// The activation tile of a step (128 rows x 256 B, 8 loads of 1 KiB per wave) is moved into LDS
// by the buffer unit (buffer_load ... lds), so that no load's result goes through a register and
// the compiler places no wait on it: the kernel orders LDS against these loads itself, with
// vmcnt waits and barriers. It lands in the swizzled layout the fragment reads expect: lane i of
// a load fills physical chunk i % 16 of its row, so it fetches the logical chunk
// (i % 16) ^ (row & 15). Each wave loads the packed codes of its 32 weight rows into registers
// and turns them into the MFMA operand itself: there is no unpacked weight tile in LDS, and one
// barrier per step. The two waves of an n-half both unpack its rows. The steps (and zero points)
// of the 64 rows for all K, r_k for all K and 2^-b per block are tables in LDS filled once.
// Step g: wait for step g's loads; barrier (everyone's have landed, and the other stage's last
// reader, step g - 1, is done); issue step g + 1's loads into the other stage; the MFMAs of step
// g into a fresh fp32 partial per group, added to the accumulators times step 2^-b of each row.
// (A third stage, two steps ahead, was no faster; with the codes staged in LDS too, one workgroup
// per CU fit instead of two, and 11008 rows at M = 512 took 106 instead of 89 us.)
// Rows past M read as zeros (the buffer range ends at the last valid row), rows past N read row
// N - 1, and neither's outputs are stored.
namespace {
constexpr int TBN = 64, TBK = 128;
__device__ __forceinline__ int tswz(int row, int chunk) {   // byte offset inside a 256-byte row
  return row * (TBK * 2) + ((chunk ^ (row & 15)) << 4);
}
constexpr int kRwSmem = 2 * 128 * TBK * 2;            // two stages of 128 rows: 64 KiB
}  // namespace

// bytes of the dynamic tables: fp16 r [K], fp32 2^-b [K/128], fp16 steps [K/GS][64], (ZP) uint8
// zeros [K/GS][64]
__host__ __device__ constexpr int64_t w4a16_tiled_tables(int64_t K, int GS, bool ZP) {
  return K * 2 + (K / 128) * 4 + (int64_t)TBN * (K / GS) * 2 + (ZP ? (int64_t)TBN * (K / GS) : 0);
}

// Which channels a lane holds: with G = 128 lane group lg takes words 4 lg .. 4 lg + 3 of a row's
// 16 words per step and MFMA kk its word 4 lg + kk, i.e. channels 32 lg + 8 kk ..; with G = 64
// MFMA kk takes word 4 kk + lg (channels 32 kk + 8 lg ..), so MFMAs 0, 1 cover the step's first
// group and 2, 3 the second. The activation fragment of a lane holds the same 8 channels, in
// natural order: a code word is decoded in pairs (2j, 2j + 1), byte j of the word spread to bytes
// 0 and 2 (v_perm), then (t & 0x00F0000F) | 0x64006400 is the fp16 pair (1024 + u_2j,
// 1024 + 16 u_2j+1) and one packed fma with (1, 1/16) and -(1032, 72) (or -(1024 + z, 64 + z))
// gives (c(q_2j), c(q_2j+1)) exactly; times the r pair, rounded once (without s the exact pair is
// the operand).

template <int GS, bool ZP, bool HAS_S, int NBW, int BMT>
__global__ __launch_bounds__(256) void w4a16_tiled_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t N, int64_t K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales16,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ s16,
    uint16_t* __restrict__ Y, int64_t tiles, int KB, float* __restrict__ partials,
    int64_t slice_stride) {
  // BMT batch rows per tile (128, or 64 where two workgroups per CU beat one)
  constexpr int kStage = BMT * TBK * 2;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  // tables of this workgroup's K slice (KB blocks from kb0)
  const int64_t ngr = K / GS;
  const int64_t kc = (int64_t)KB * 128;                                    // slice channels
  constexpr int kGpb = 128 / GS;
  uint16_t* rtab = reinterpret_cast<uint16_t*>(dyn);                       // [kc]
  float* bfac = reinterpret_cast<float*>(dyn + kc * 2);                    // [KB]
  uint16_t* st_lds = reinterpret_cast<uint16_t*>(dyn + kc * 2 + (int64_t)KB * 4);  // [KB kGpb][64]
  uint8_t* z_lds = reinterpret_cast<uint8_t*>(st_lds + TBN * KB * kGpb);   // [KB kGpb][64] (ZP)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int MBW = BMT / (16 * NBW);      // 16-row blocks of m per wave
  constexpr int WAVES_N = 4 / NBW;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t tilesN = (N + TBN - 1) / TBN;
  int64_t bl = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bl = (int64_t)(blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int split = (int)(bl / tiles);     // K slice (slice-major: one XCD shares slices)
  const int64_t tile = bl % tiles;
  const int64_t m0 = (tile / tilesN) * BMT;
  const int64_t n0 = (tile % tilesN) * TBN;
  const int64_t kb0 = (int64_t)split * KB;
  const int64_t groups = (K / 128 - kb0 < KB) ? K / 128 - kb0 : KB;   // this slice's steps

  // ---- tables: r_k = fp16(2^b / s_k) in natural order, 2^-b per block (with s), steps, zero
  // points ------------------------------------------------------------------------------------
  for (int64_t k8 = tid; HAS_S && k8 < groups * 16; k8 += 256) {
    float inv[8];
    float mx = 0.0f;
    if (HAS_S) {
      float sv[8];
      load8_f32<kF16>(s16 + kb0 * 128 + k8 * 8, sv);
#pragma unroll
      for (int t = 0; t < 8; ++t) inv[t] = __builtin_amdgcn_rcpf(sv[t]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) inv[t] = 1.0f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) mx = fmaxf(mx, inv[t]);
    mx = group_absmax<16>(mx);
    const int b = escale_for_max(mx) - 4;      // 2^b mx in [2^10, 2^11)
    const float sc = ldexpf(1.0f, b);
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = (uint32_t)f2h(inv[2 * p] * sc) | ((uint32_t)f2h(inv[2 * p + 1] * sc) << 16);
    *reinterpret_cast<uint4*>(rtab + k8 * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    if ((k8 & 15) == 0) bfac[k8 >> 4] = ldexpf(1.0f, -b);
  }
  for (int64_t e = tid; e < TBN * groups * kGpb; e += 256) {
    const int64_t r = e % TBN, gq = kb0 * kGpb + e / TBN;
    const int64_t row = (n0 + r < N) ? n0 + r : N - 1;
    st_lds[e] = (n0 + r < N) ? scales16[row * ngr + gq] : (uint16_t)0;
    if (ZP) z_lds[e] = zeros[row * ngr + gq];
  }

  // ---- activation stages ---------------------------------------------------------------------
  const int64_t arows = (M - m0 < BMT) ? M - m0 : BMT;
  const rsrc_t ra = make_rsrc(A + m0 * K, (uint32_t)(arows * K * 2));
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  uint32_t avoff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int rl = 4 * jj + (lane >> 4);
    avoff[jj] = (uint32_t)((lane >> 4) * K * 2) + (uint32_t)((((lane & 15) ^ (rl & 15))) << 4);
  }
  auto issue = [&](int64_t g, int st) {
#pragma unroll
    for (int j = 0; j < BMT / 16; ++j) {   // BMT / 4 rows per wave, 4 per load
      const int r0 = (BMT / 4) * wave + 4 * j;
      const uint32_t lds = lds0 + (uint32_t)(st * kStage) + (uint32_t)(r0 * 256);
      const uint32_t so = (uint32_t)(r0 * K * 2) + (uint32_t)((kb0 + g) * 256);
      buffer_load16_lds_so(ra, lds, avoff[j & 3], so);
    }
  };
  // this wave's code rows
  const uint32_t* wr[2];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int64_t n = n0 + 16 * NBW * wn + 16 * nb + li;
    wr[nb] = qweight + (n < N ? n : N - 1) * (K / 8) + kb0 * 16;
  }
  struct Codes {
    uint32_t w[NBW][4];   // [nb][kk]: the word MFMA kk of the step takes
  };
  auto load_codes = [&](int64_t g, Codes& c) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (GS == 128) {
        const uint4 v = *reinterpret_cast<const uint4*>(wr[nb] + g * 16 + 4 * lg);
        c.w[nb][0] = v.x; c.w[nb][1] = v.y; c.w[nb][2] = v.z; c.w[nb][3] = v.w;
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c.w[nb][kk] = wr[nb][g * 16 + 4 * kk + lg];
      }
    }
  };

  floatx4 acc[NBW][MBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int kKKPerGroup = (GS == 64) ? 2 : 4;
  // the fp16 exponent bits of the decode, held in a register so that the mask-and-insert is one
  // v_and_or_b32 (a VALU instruction reads one scalar or literal operand)
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  auto compute = [&](int64_t g, int st, const Codes& c) {
    const char* sa = smem + st * kStage;
    // without s the weight operand is c(q) itself (exact) and no block scale applies
    const float bs = HAS_S ? bfac[g] : 1.0f;
#pragma unroll
    for (int h = 0; h < 4 / kKKPerGroup; ++h) {
      const int64_t gq = (GS == 64) ? 2 * g + h : g;
      half2_t sub2[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        // subtrahends of the decoded pair (1024 + u, 64 + u'): 1032 and 72 for signed codes
        // (biased by the xor), 1024 + z and 64 + z with zero points
        const float z = ZP ? (float)z_lds[gq * TBN + 16 * NBW * wn + 16 * nb + li] : 8.0f;
        sub2[nb] = half2_t{(_Float16)(1024.0f + z), (_Float16)(64.0f + z)};
      }
      floatx4 part[NBW][MBW];
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < MBW; ++j) part[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = h * kKKPerGroup; kk < (h + 1) * kKKPerGroup; ++kk) {
        const int ch = (GS == 128) ? 4 * lg + kk : 4 * kk + lg;   // the lane's 8-channel chunk
        const uint4 rv = HAS_S ? *reinterpret_cast<const uint4*>(rtab + g * 128 + ch * 8)
                               : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t rp[4] = {rv.x, rv.y, rv.z, rv.w};
        half8_t wf[NBW], af[MBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const uint32_t x = ZP ? c.w[nb][kk] : (c.w[nb][kk] ^ 0x88888888u);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // byte j (channels 2j, 2j + 1) to bytes 0 and 2
            const uint32_t t =
                __builtin_amdgcn_perm(x, x, 0x0C000C00u | (uint32_t)j | ((uint32_t)j << 16));
            const uint32_t bits = (t & 0x00F0000Fu) | magic;
            const half2_t q = __builtin_elementwise_fma(
                __builtin_bit_cast(half2_t, bits), half2_t{(_Float16)1.0f, (_Float16)0.0625f},
                -sub2[nb]);
            const half2_t wv = HAS_S ? q * __builtin_bit_cast(half2_t, rp[j]) : q;
            wf[nb][2 * j] = wv[0];
            wf[nb][2 * j + 1] = wv[1];
          }
        }
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
          af[mb] = *reinterpret_cast<const half8_t*>(sa + tswz(wm * 16 * MBW + mb * 16 + li, ch));
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int mb = 0; mb < MBW; ++mb)
            part[nb][mb] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[nb], af[mb], part[nb][mb], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const uint2 sr = *reinterpret_cast<const uint2*>(st_lds + gq * TBN + wn * 16 * NBW + nb * 16 +
                                                         4 * lg);
        const float sc[4] = {h2f((uint16_t)(sr.x & 0xFFFFu)) * bs, h2f((uint16_t)(sr.x >> 16)) * bs,
                             h2f((uint16_t)(sr.y & 0xFFFFu)) * bs, h2f((uint16_t)(sr.y >> 16)) * bs};
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[nb][mb][r] = __builtin_fmaf(part[nb][mb][r], sc[r], acc[nb][mb][r]);
      }
    }
  };

  // ---- main loop: step g + 1 in flight while step g computes; two sets of code registers take
  // turns (the loop unrolled by two, so that their indices are static) ------------------------
  Codes cb[2];
  issue(0, 0);
  load_codes(0, cb[0]);
  auto step = [&](int64_t g, int st, const Codes& cur, Codes& nxt) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));    // this wave's loads of step g have landed
    __syncthreads();                              // everyone's; and stage st ^ 1 is read
    if (g + 1 < groups) {
      issue(g + 1, st ^ 1);
      load_codes(g + 1, nxt);
    }
    compute(g, st, cur);
  };
  for (int64_t g = 0; g < groups; g += 2) {
    step(g, 0, cb[0], cb[1]);
    if (g + 1 < groups) step(g + 1, 1, cb[1], cb[0]);
  }

  if (partials) {   // one of several K slices: fp32 partial [m][n] of slice `split`
    float* P = partials + split * slice_stride;
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int j = 0; j < MBW; ++j) {
        const int64_t m = m0 + wm * 16 * MBW + j * 16 + li;
        const int64_t nb = n0 + wn * 16 * NBW + i * 16 + 4 * lg;
        if (m < M) {
          if (nb + 3 < N && ((N & 3) == 0)) {
            *reinterpret_cast<floatx4*>(P + m * N + nb) = acc[i][j];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (nb + r < N) P[m * N + nb + r] = acc[i][j][r];
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
      const int64_t m = m0 + wm * 16 * MBW + j * 16 + li;
      const int64_t nb = n0 + wn * 16 * NBW + i * 16 + 4 * lg;
      if (m < M) {
        if (nb + 3 < N && ((N & 3) == 0)) {
          const uint32_t lo = (uint32_t)f2h(acc[i][j][0]) | ((uint32_t)f2h(acc[i][j][1]) << 16);
          const uint32_t hi = (uint32_t)f2h(acc[i][j][2]) | ((uint32_t)f2h(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2*>(Y + m * N + nb) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) Y[m * N + nb + r] = f2h(acc[i][j][r]);
        }
      }
    }
}

// Y = fp16(sum of the S slices' fp32 partials [S][M][N], slice stride `stride` floats, a multiple
// of 4), added in slice order 0 .. S-1; four elements per thread, eight slices' loads in flight.
__global__ __launch_bounds__(256) void w4a16_sum_slices_kernel(const float* __restrict__ P, int S,
                                                               int64_t stride, int64_t MN,
                                                               uint16_t* __restrict__ Y) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= MN) return;
  constexpr int kC = 8;
  floatx4 t = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < S; j0 += kC) {
    floatx4 v[kC];
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const int j = (j0 + u < S) ? j0 + u : 0;
      v[u] = *reinterpret_cast<const floatx4*>(P + j * stride + e);   // within the padded slice
    }
#pragma unroll
    for (int u = 0; u < kC; ++u)
      if (j0 + u < S) t = (j0 + u == 0) ? v[u] : t + v[u];
  }
  if (e + 3 < MN && (((uintptr_t)(Y + e)) & 7u) == 0) {
    const uint32_t lo = (uint32_t)f2h(t[0]) | ((uint32_t)f2h(t[1]) << 16);
    const uint32_t hi = (uint32_t)f2h(t[2]) | ((uint32_t)f2h(t[3]) << 16);
    *reinterpret_cast<uint2*>(Y + e) = make_uint2(lo, hi);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e + r < MN) Y[e + r] = f2h(t[r]);
  }
}

W4a16TiledPlan w4a16_tiled_plan(int64_t M, int64_t N, int64_t K, bool split) {
  W4a16TiledPlan p{};
  // Tiles of 128 batch rows; without slices and with at most 128 such tiles (half the CUs or
  // fewer busy), tiles of 64 rows, two or more workgroups per CU (graph replay: 4096 x 4096 at
  // M = 128 30.4 vs 36.6 us, M = 256 31.2 vs 36.0, 4096 x 11008 at M = 128 74.4 vs 91.8; at 172
  // tiles, 11008 x 4096 at M = 128, 41.2 vs 38.5, and with slices 64 rows lose everywhere)
  const int64_t tiles128 = ((M + 127) / 128) * ((N + TBN - 1) / TBN);
  p.tbm = (!split && tiles128 <= 128) ? 64 : 128;
  p.tiles = ((M + p.tbm - 1) / p.tbm) * ((N + TBN - 1) / TBN);
  const int64_t nblk = K / 128;
  int64_t S = 1;
  if (split && p.tiles < 256) {
    // slices while fewer tiles than CUs, the grid within two workgroups per CU, at least 8 steps
    // each (measured, graph replay: 4096 x 4096 at 128 rows 19.7 us vs 36.5 in one slice,
    // 4096 x 11008 33.6 vs 92.0, 8192 x 8192 40.8 vs 70.0; at 256 tiles two slices are no faster
    // at 4096 x 4096 x 512 rows and slower at 4096 x 11008: 113 vs 95 us)
    S = kW4a16SplitTarget / p.tiles;
    const int64_t smax = nblk / 8;
    S = S > smax ? smax : S;
    S = S < 1 ? 1 : S;
  }
  p.KB = (nblk + S - 1) / S;
  p.S = (nblk + p.KB - 1) / p.KB;
  p.stride = (M * N + 3) / 4 * 4;
  p.ws_bytes = p.S > 1 ? (size_t)(p.S * p.stride * 4) : 0;
  return p;
}

template <int GS, bool ZP>
static hipError_t w4a16_tiled(const uint16_t* A, int64_t M, int64_t N, int64_t K,
                              const uint32_t* qweight, const uint16_t* scales16,
                              const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                              const W4a16TiledPlan& p, float* partials, hipStream_t stream) {
  const size_t dyn = (size_t)w4a16_tiled_tables(p.KB * 128, GS, ZP);
  const unsigned grid = (unsigned)(p.tiles * p.S);
  float* P = p.S > 1 ? partials : nullptr;
  // waves of 64 x 32 (two 16-row weight blocks each) for symmetric groups of 128; with groups of
  // 64 or zero points, whose per-group work doubles the unpacking cost, waves of 128 x 16 (each
  // wave unpacks only its own 16 rows; 4096 x 4096 at M = 512: 45.7 vs 57.3 us, while symmetric
  // groups of 128 run 38.8 vs 37.6 us that way)
  constexpr int NBW = (GS == 64 || ZP) ? 1 : 2;
#define AWQ_TT(HS_, BM_)                                                                         \
  w4a16_tiled_kernel<GS, ZP, HS_, NBW, BM_><<<grid, 256, dyn, stream>>>(                         \
      A, M, N, K, qweight, scales16, zeros, s16, Y, p.tiles, (int)p.KB, P, p.stride)
  if (s16) {
    if (p.tbm == 64) AWQ_TT(true, 64); else AWQ_TT(true, 128);
  } else {
    if (p.tbm == 64) AWQ_TT(false, 64); else AWQ_TT(false, 128);
  }
#undef AWQ_TT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const int64_t MN = M * N;
  w4a16_sum_slices_kernel<<<(unsigned)((MN / 4 + 255) / 256 + 1), 256, 0, stream>>>(
      partials, (int)p.S, p.stride, MN, Y);
  return hipGetLastError();
}

hipError_t launch_w4a16_tiled_split(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                                    const uint32_t* qweight, const uint16_t* scales16,
                                    const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  const W4a16TiledPlan p = w4a16_tiled_plan(M, N, K, true);
  if (p.S > 1 && (ws == nullptr || ws_bytes < p.ws_bytes)) return hipErrorInvalidValue;
  const bool zp = zeros != nullptr;
  float* P = static_cast<float*>(ws);
  if (group == 64)
    return zp ? w4a16_tiled<64, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, P, stream)
              : w4a16_tiled<64, false>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, P, stream);
  return zp ? w4a16_tiled<128, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, P, stream)
            : w4a16_tiled<128, false>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, P, stream);
}

hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                        const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                        const uint16_t* s16, uint16_t* Y, hipStream_t stream) {
  if (w4a16_gemv_fits(M, K))
    return launch_w4a16_gemv(A, M, N, K, group, qweight, scales16, zeros, s16, Y, stream);
  // the tiled kernel above 64 batch rows, and from 49 on for tall weights (each skinny
  // workgroup reads all of A, which at 8192+ weight rows costs more than the tiles' unpacking),
  // while its tables fit next to the 64 KiB of stages; otherwise the skinny kernel in passes
  // of 64 rows
  const bool zp = zeros != nullptr;
  const bool tiled = (M > 64 || (M > 48 && N >= 8192)) &&
                     kRwSmem + w4a16_tiled_tables(K, group, zp) <= 160 * 1024;
  if (!tiled)
    return launch_w4a16_skinny(A, M, N, K, group, qweight, scales16, zeros, s16, Y, stream);
  const W4a16TiledPlan p = w4a16_tiled_plan(M, N, K, false);
  if (group == 64)
    return zp ? w4a16_tiled<64, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, nullptr,
                                      stream)
              : w4a16_tiled<64, false>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, nullptr,
                                       stream);
  return zp ? w4a16_tiled<128, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, nullptr,
                                     stream)
            : w4a16_tiled<128, false>(A, M, N, K, qweight, scales16, zeros, s16, Y, p, nullptr,
                                      stream);
}

}  // namespace awq
