// W4A16 GEMM on the packed AWQ artefacts: QuantLinear.forward of "AWQ 量化方案..."
// (qwbw.cn/news/39982), section 三 -- scale the input per channel, dequantize the packed codes
// with the per-group steps, then a linear layer:
//   Y[m, n] = sum_k (A[m,k] / s[k]) * c(q[n,k]) * step[n, k/G],
// c(q) = q for symmetric codes, q - z[n, k/G] for zero-point codes. The activation is divided by
// s because the weight was multiplied by s (AWQ notes, bg51717.github.io/14592, section 方法).
//
// Three kernels by batch size M:
//   M = 1        w4a16_gemv.hip: fp16 dot products against a block-scaled A / s table;
//   2 <= M <= 64 w4a16_skinny.hip: MFMA with the activations read straight from memory;
//   M > 64       the tiled kernel below (and from 49 rows on for weights of 8192 rows or more).
// All of them apply 1/s without an fp16 value that a tiny s could overflow: either A / s is kept
// in fp32 and stored scaled by a power of two per 128-channel block, or the weight operand is
// fp16(q r_k) with r_k = fp16(2^b / s_k), 2^b chosen per block so that the block's largest r_k lies
// in [2^10, 2^11), and 2^-b rides on the fp32 group step.
#include "device_common.h"
#include "kernels.h"

namespace awq {

// ---------------------------------------------------------------------------------------------
// Larger batches: a tiled MFMA GEMM. Workgroup tile 128 (batch rows m) x 64 (weight rows n), one
// 128-channel block of K per step, 4 waves of 64 x 32 (2 x 2), each a 4 x 2 grid of
// v_mfma_f32_16x16x32_f16 blocks (weights as the A operand, activations as B).
//
// Every main-loop load is moved into LDS by the buffer unit (buffer_load ... lds), so that no
// load's result goes through a register and the compiler places no wait on them: the kernel
// orders LDS against these loads itself, with vmcnt waits and barriers. Per K step the workgroup
// moves the activation tile (128 rows x 256 B, 8 loads of 1 KiB per wave, written in the swizzled
// layout the fragment reads expect: lane i of a load fills physical chunk i % 16 of its row, so it
// fetches the logical chunk (i % 16) ^ (row & 15)) and the raw codes of its 64 weight rows
// (64 x 64 B, one load per wave). The steps (and zero points) of the 64 rows for all K, r_k for
// all K and 2^-b per block are tables in LDS filled once. Step g:
//   wait for step g's loads; barrier; issue step g + 1's loads into the other stage (its last
//   reader, step g - 1, is behind the barrier); unpack step g's codes into fp16(c(q) r_k) in the
//   swizzled layout; barrier; the MFMAs of step g into a fresh fp32 partial per group, added to
//   the accumulators times step 2^-b of each row.
// Rows past M or N read as zeros (the buffer ranges end at the last valid row) and their outputs
// are not stored.
namespace {
constexpr int TBM = 128, TBN = 64, TBK = 128;
__device__ __forceinline__ int tswz(int row, int chunk) {   // byte offset inside a 256-byte row
  return row * (TBK * 2) + ((chunk ^ (row & 15)) << 4);
}
constexpr int kRawStage = TBN * 64;                   // 4 KiB of packed codes per step
constexpr int kAStage = TBM * TBK * 2;                // 32 KiB of activations per step
constexpr int kWStage = TBN * TBK * 2;                // 16 KiB of unpacked weights per step
// two stages each of activations, codes and unpacked weights: 104 KiB
constexpr int kDmaSmem = 2 * (kAStage + kRawStage + kWStage);
// s_waitcnt immediate: at most n vector-memory loads outstanding (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
}  // namespace

// bytes of the dynamic tables: fp16 r [K], fp32 2^-b [K/128], fp16 steps [K/GS][64], (ZP) uint8
// zeros [K/GS][64]
__host__ __device__ constexpr int64_t w4a16_dma_tables(int64_t K, int GS, bool ZP) {
  return K * 2 + (K / 128) * 4 + (int64_t)TBN * (K / GS) * 2 + (ZP ? (int64_t)TBN * (K / GS) : 0);
}

template <int GS, bool ZP, bool HAS_S>
__global__ __launch_bounds__(256) void w4a16_tiled_dma_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t N, int64_t K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales16,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ s16,
    uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(1024))) char smem[kDmaSmem];
  // LDS: activation stages [2][32 KiB], unpacked weight stages [2][16 KiB], code stages [2][4 KiB]
  constexpr int kWBase = 2 * kAStage, kRawBase = 2 * kAStage + 2 * kWStage;
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int64_t ngr = K / GS;
  uint16_t* rtab = reinterpret_cast<uint16_t*>(dyn);                      // [K]
  float* bfac = reinterpret_cast<float*>(dyn + K * 2);                    // [K/128]
  uint16_t* st_lds = reinterpret_cast<uint16_t*>(dyn + K * 2 + (K / 128) * 4);   // [ngr][64]
  uint8_t* z_lds = reinterpret_cast<uint8_t*>(st_lds + TBN * ngr);        // [ngr][64] (ZP)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tilesN = (N + TBN - 1) / TBN;
  // Workgroup b runs on XCD b % 8: when the grid divides by 8, XCD x takes the x-th contiguous
  // eighth of the row-major tile order, so the tiles in one XCD's L2 share activation rows.
  int64_t bl = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bl = (int64_t)(blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t m0 = (bl / tilesN) * TBM;
  const int64_t n0 = (bl % tilesN) * TBN;
  const int64_t groups = K / 128;

  // ---- tables (plain loads: the compiler's waits here cost nothing). r_k = fp16(2^b / s_k):
  // the 16 chunks of a 128-channel block are 16 consecutive threads (one DPP row; K / 8 is a
  // multiple of 16, so a row is all inside or all past the loop) ---------------------------
  for (int64_t k8 = tid; k8 < K / 8; k8 += 256) {
    float inv[8];
    float mx = 0.0f;
    if (HAS_S) {
      float sv[8];
      load8_f32<kF16>(s16 + k8 * 8, sv);
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
  for (int64_t e = tid; e < TBN * ngr; e += 256) {
    const int64_t r = e % TBN, gq = e / TBN;
    const int64_t row = (n0 + r < N) ? n0 + r : N - 1;
    st_lds[e] = (n0 + r < N) ? scales16[row * ngr + gq] : (uint16_t)0;
    if (ZP) z_lds[e] = zeros[row * ngr + gq];
  }

  // ---- buffer loads into LDS ----------------------------------------------------------------
  const int64_t arows = (M - m0 < TBM) ? M - m0 : TBM;
  const int64_t wrows = (N - n0 < TBN) ? N - n0 : TBN;
  const rsrc_t ra = make_rsrc(A + m0 * K, (uint32_t)(arows * K * 2));
  const rsrc_t rw = make_rsrc(qweight + n0 * (K / 8), (uint32_t)(wrows * (K / 2)));
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  // activation load j of this wave: tile rows 32 wave + 4 j + lane / 16; the lane's logical
  // chunk depends on the row mod 16, i.e. on j mod 4 -- four per-lane offsets
  uint32_t avoff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int rl = 4 * jj + (lane >> 4);
    avoff[jj] = (uint32_t)((lane >> 4) * K * 2) + (uint32_t)((((lane & 15) ^ (rl & 15))) << 4);
  }
  // raw codes: this wave's load covers weight rows 16 wave + lane / 4, bytes 16 (lane % 4) of the
  // step's 64
  const uint32_t wvoff = (uint32_t)((lane >> 2) * (K / 2)) + (uint32_t)((lane & 3) * 16);
  auto issue = [&](int64_t g, int st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lds = lds0 + (uint32_t)(st * kAStage) + (uint32_t)((32 * wave + 4 * j) * 256);
      const uint32_t so = (uint32_t)((32 * wave + 4 * j) * K * 2) + (uint32_t)(g * 256);
      buffer_load16_lds_so(ra, lds, avoff[j & 3], so);
    }
    const uint32_t lds = lds0 + (uint32_t)(kRawBase + st * kRawStage) + (uint32_t)(wave * 1024);
    const uint32_t so = (uint32_t)(16 * wave * (K / 2)) + (uint32_t)(g * 64);
    buffer_load16_lds_so(rw, lds, wvoff, so);
  };

  // ---- unpack: thread t owns weight row t / 4, channels 32 (t % 4) .. + 31 of the step -------
  const int wrow_l = tid >> 2, wq = tid & 3;
  auto unpack = [&](int64_t g, int st) {
    const char* raw = smem + kRawBase + st * kRawStage;
    char* sw = smem + kWBase + (int)(g & 1) * kWStage;
    const uint4 wv = *reinterpret_cast<const uint4*>(raw + wrow_l * 64 + wq * 16);
    const int64_t gq = (GS == 64) ? 2 * g + (wq >> 1) : g;
    const _Float16 subh = ZP ? (_Float16)(1024.0f + (float)z_lds[gq * TBN + wrow_l])
                             : (_Float16)1032.0f;
    const half2_t sub2 = half2_t{subh, subh};
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 iv = *reinterpret_cast<const uint4*>(rtab + g * 128 + wq * 32 + v * 8);
      // r pairs (j, j + 4) to match the unpack order
      const uint32_t i04 = __builtin_amdgcn_perm(iv.z, iv.x, 0x05040100u);
      const uint32_t i15 = __builtin_amdgcn_perm(iv.z, iv.x, 0x07060302u);
      const uint32_t i26 = __builtin_amdgcn_perm(iv.w, iv.y, 0x05040100u);
      const uint32_t i37 = __builtin_amdgcn_perm(iv.w, iv.y, 0x07060302u);
      const uint32_t rp[4] = {i04, i15, i26, i37};
      const uint32_t x = ZP ? words[v] : (words[v] ^ 0x88888888u);
      uint32_t pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t bits = ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const half2_t q = __builtin_bit_cast(half2_t, bits) - sub2;
        pr[j] = __builtin_bit_cast(uint32_t, q * __builtin_bit_cast(half2_t, rp[j]));
      }
      const uint32_t n01 = __builtin_amdgcn_perm(pr[1], pr[0], 0x05040100u);
      const uint32_t n23 = __builtin_amdgcn_perm(pr[3], pr[2], 0x05040100u);
      const uint32_t n45 = __builtin_amdgcn_perm(pr[1], pr[0], 0x07060302u);
      const uint32_t n67 = __builtin_amdgcn_perm(pr[3], pr[2], 0x07060302u);
      *reinterpret_cast<uint4*>(sw + tswz(wrow_l, wq * 4 + v)) = make_uint4(n01, n23, n45, n67);
    }
  };

  floatx4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int li = lane & 15, lg = lane >> 4;
  // per group: MFMAs into a fresh partial, then acc += partial * step 2^-b of each weight row
  // (rows wn 32 + 16 i + 4 lg + r of this lane: four consecutive entries of the step table)
  constexpr int kKKPerGroup = (GS == 64) ? 2 : 4;
  auto compute = [&](int64_t g, int st) {
    const char* sa = smem + st * kAStage;
    const char* sw = smem + kWBase + (int)(g & 1) * kWStage;
    const float bs = bfac[g];
#pragma unroll
    for (int h = 0; h < 4 / kKKPerGroup; ++h) {
      floatx4 part[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = h * kKKPerGroup; kk < (h + 1) * kKKPerGroup; ++kk) {
        const int chunk = kk * 4 + lg;         // this lane's 8 channels of the 32-wide slice
        half8_t wf[2], af[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          wf[i] = *reinterpret_cast<const half8_t*>(sw + tswz(wn * 32 + i * 16 + li, chunk));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          af[j] = *reinterpret_cast<const half8_t*>(sa + tswz(wm * 64 + j * 16 + li, chunk));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[i], af[j], part[i][j], 0, 0, 0);
      }
      const int64_t gq = (GS == 64) ? 2 * g + h : g;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint2 sr = *reinterpret_cast<const uint2*>(st_lds + gq * TBN + wn * 32 + i * 16 +
                                                         4 * lg);
        const float sc[4] = {h2f((uint16_t)(sr.x & 0xFFFFu)) * bs, h2f((uint16_t)(sr.x >> 16)) * bs,
                             h2f((uint16_t)(sr.y & 0xFFFFu)) * bs, h2f((uint16_t)(sr.y >> 16)) * bs};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[i][j][r], sc[r], acc[i][j][r]);
      }
    }
  };

  // ---- main loop: 9 loads per wave per step, issued one step ahead -------------------------
  issue(0, 0);
  for (int64_t g = 0; g < groups; ++g) {
    const int st = (int)(g & 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));    // this wave's loads of step g have landed
    __syncthreads();                              // everyone's; and step g - 1 is read
    if (g + 1 < groups) issue(g + 1, st ^ 1);
    unpack(g, st);
    __syncthreads();
    compute(g, st);
  }

  // D layout of the 16x16 MFMA: lane holds D[4 (lane / 16) + r][lane % 16] -> weight rows
  // 4 lg + r of block i, batch row li of block j.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + wm * 64 + j * 16 + li;
      const int64_t nb = n0 + wn * 32 + i * 16 + 4 * lg;
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

template <int GS, bool ZP>
static hipError_t w4a16_tiled(const uint16_t* A, int64_t M, int64_t N, int64_t K,
                              const uint32_t* qweight, const uint16_t* scales16,
                              const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                              hipStream_t stream) {
  const int64_t tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
  const size_t dyn = (size_t)w4a16_dma_tables(K, GS, ZP);
  if (s16)
    w4a16_tiled_dma_kernel<GS, ZP, true><<<(unsigned)tiles, 256, dyn, stream>>>(
        A, M, N, K, qweight, scales16, zeros, s16, Y);
  else
    w4a16_tiled_dma_kernel<GS, ZP, false><<<(unsigned)tiles, 256, dyn, stream>>>(
        A, M, N, K, qweight, scales16, zeros, s16, Y);
  return hipGetLastError();
}

hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                        const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                        const uint16_t* s16, uint16_t* Y, hipStream_t stream) {
  if (M == 1 && K <= kW4a16GemvMaxK)
    return launch_w4a16_gemv(A, M, N, K, group, qweight, scales16, zeros, s16, Y, stream);
  // the tiled kernel above 64 batch rows, and from 49 on for tall weights (each skinny
  // workgroup reads all of A, which at 8192+ weight rows costs more than the tiles' unpacking),
  // while its tables fit next to the 104 KiB of stages; otherwise the skinny kernel in passes
  // of 64 rows
  const bool zp = zeros != nullptr;
  const bool tiled = (M > 64 || (M > 48 && N >= 8192)) &&
                     kDmaSmem + w4a16_dma_tables(K, group, zp) <= 160 * 1024;
  if (!tiled)
    return launch_w4a16_skinny(A, M, N, K, group, qweight, scales16, zeros, s16, Y, stream);
  if (group == 64)
    return zp ? w4a16_tiled<64, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream)
              : w4a16_tiled<64, false>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream);
  return zp ? w4a16_tiled<128, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream)
            : w4a16_tiled<128, false>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream);
}

}  // namespace awq
