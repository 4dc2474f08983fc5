// W4A16 for small batches (2 to 64 activation rows) with K split over workgroups:
// QuantLinear.forward of "AWQ 量化方案..." (qwbw.cn/news/39982), section 三 -- scale the input per
// channel, dequantize, linear:
//   Y[m, n] = sum_k (A[m,k] / s[k]) * c(q[n,k]) * step[n, k/G],
// c(q) = q (symmetric codes) or q - z[n, k/G] (zero-point codes); A is divided by s because the
// weight was multiplied by s (AWQ notes, bg51717.github.io/14592, section 方法).
//
// Why split K: with few activation rows the packed weight is the traffic, and a grid that fills
// 256 CUs with one all-K workgroup per 16 weight rows reads all of A once per workgroup (at 64
// rows and 4096 weight rows: 256 x 512 KiB from L2). Here a workgroup owns 64 weight rows and a
// slice of K, so A is read once per 64 rows, and the slices give the grid its width; the partial
// sums of the slices are added through a workspace in a fixed order.
//
// Workgroup: 4 waves; wave w owns weight rows 16 w .. 16 w + 15 of the tile and all MB blocks of
// 16 activation rows, i.e. MB v_mfma_f32_16x16x32_f16 per 32 channels (weights as the A operand,
// activations as B). Per 128-channel block the activation tile (16 MB rows x 256 B) and the
// packed codes (64 rows x 64 B) are moved into LDS by the buffer unit (buffer_load ... lds), in
// 8, 6 or 3 stages for MB = 1, 2, 4 (as many blocks in flight from the start) with explicit vmcnt
// waits; rows past M or N read as zeros. Codes are decoded in registers in natural channel pairs as in the tiled kernel
// (w4a16.hip): v_perm, v_and_or_b32, one packed fma, times the r pair. Per group the fp32 partial
// is added to the accumulators times step 2^-b of each row.
//
// Slices and the reduction: slice j covers blocks [j KB, (j + 1) KB). Every workgroup stores its
// fp32 partial [4 waves][MB][64 lanes] (floatx4 per lane) in the workspace, and a second kernel
// adds the S partials of each tile in slice order 0 .. S-1 and rounds once to fp16, so the result
// does not depend on scheduling. (Adding them in the same kernel, by the last workgroup of a tile
// to bump a counter, costs three dependent trips to memory at the end -- the partial's store,
// the count, the other partials' loads -- and took 12 us at 16 x 4096 x 4096.) With one slice the
// main kernel stores Y itself.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {
constexpr int kSkTileN = 64;                // weight rows per workgroup
// LDS stages by activation blocks: 8 KiB, 12 KiB or 20 KiB each, two workgroups per CU
__host__ __device__ constexpr int sk_stages(int MB) { return MB == 1 ? 8 : (MB == 2 ? 6 : 3); }
// s_waitcnt for "at most n later blocks' loads outstanding" (n = 0 .. NMAX), L loads a block
template <int L, int NMAX>
__device__ __forceinline__ void sk_wait_ahead(int n) {
  if constexpr (NMAX == 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    if (n >= NMAX)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NMAX * L));
    else
      sk_wait_ahead<L, NMAX - 1>(n);
  }
}
constexpr int kSkCodeStage = kSkTileN * 64; // packed codes of 64 rows x 128 channels: 4 KiB
constexpr int64_t kSkMaxKB = 64;            // blocks per slice: the tables stay within 41 KiB
__device__ __forceinline__ int sk_swz(int row, int chunk) {   // byte offset in a 256-byte row
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}
}  // namespace

// Tables in dynamic LDS for a slice of KB blocks: fp16 r [KB 128], fp16 steps [KB 128/GS][64],
// (ZP) uint8 zeros [KB 128/GS][64], fp32 2^-b [KB]
__host__ __device__ constexpr int64_t sk_tables_bytes(int64_t KB, int GS, bool ZP) {
  return KB * 256 + KB * (128 / GS) * kSkTileN * 2 + (ZP ? KB * (128 / GS) * kSkTileN : 0) +
         KB * 4;
}

// Where the split pays (measured against the skinny kernel, graph replay, rotated weights):
// always above 32 rows (4096 x 4096 at 64 rows 16.7 us vs 18.9, 8192 x 8192 29.5 vs 69.1,
// 4096 x 11008 23.9 vs 46.3); from 17 rows on tall weights (11008 x 4096 at 32 rows 22.7 vs
// 28.2); from 16 rows on long K (8192 x 8192 20.4 vs 24.2, 1024 x 8192 9.1 vs 12.1). Below, the
// second launch and the slices' shorter pipelines cost more than re-reading A (4096 x 4096 at 16
// rows 10.2 vs 7.8 us).
bool w4a16_prefer_split(int64_t M, int64_t N, int64_t K) {
  if (M < 2 || M > 64) return false;
  return M > 32 || (M > 16 && N >= 8192) || (M >= 16 && K >= 8192);
}

W4a16SplitPlan w4a16_splitk_plan(int64_t M, int64_t N, int64_t K) {
  W4a16SplitPlan p{};
  p.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.tiles = (N + kSkTileN - 1) / kSkTileN;
  const int64_t nblk = K / 128;
  // at most two workgroups per CU (one round: every instance fits twice in a CU's LDS), slices
  // of at least 4 blocks (and at most kSkMaxKB)
  int64_t S = kW4a16SplitTarget / p.tiles;
  const int64_t smax = nblk / 4 > 1 ? nblk / 4 : 1;
  const int64_t smin = (nblk + kSkMaxKB - 1) / kSkMaxKB;
  S = S < 1 ? 1 : (S > smax ? smax : S);
  S = S < smin ? smin : S;
  p.KB = (nblk + S - 1) / S;
  p.S = (nblk + p.KB - 1) / p.KB;
  p.ws_bytes = p.S > 1 ? (size_t)(p.S * p.tiles * 4 * p.MB * 64 * 16) : 0;
  return p;
}

template <int MB, int GS, bool ZP, bool HAS_S>
__global__ __launch_bounds__(256) void w4a16_splitk_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t N, int64_t K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales16,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ s16,
    uint16_t* __restrict__ Y, int64_t tiles, int S, int KB, floatx4* __restrict__ partials) {
  constexpr int kAStageB = MB * 16 * 256;
  constexpr int kStageB = kAStageB + kSkCodeStage;
  constexpr int L = MB + 1;                       // loads per wave and block
  constexpr int kSkStages = sk_stages(MB);
  __shared__ __attribute__((aligned(1024))) char smem[kSkStages * kStageB];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  constexpr int kGpb = 128 / GS;                  // groups per block
  uint16_t* rtab = reinterpret_cast<uint16_t*>(dyn);                         // [KB 128]
  uint16_t* st_lds = reinterpret_cast<uint16_t*>(dyn + (int64_t)KB * 256);   // [KB kGpb][64]
  uint8_t* z_lds = reinterpret_cast<uint8_t*>(st_lds + (int64_t)KB * kGpb * kSkTileN);
  float* bfac = reinterpret_cast<float*>(dyn + (int64_t)KB * 256 +
                                         (int64_t)KB * kGpb * kSkTileN * (ZP ? 3 : 2));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // Workgroup b runs on XCD b % 8: when the grid divides by 8, XCD x takes the x-th contiguous
  // eighth of the slice-major order, so the workgroups in one XCD's L2 share activation slices.
  int64_t bl = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bl = (int64_t)(blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int split = (int)(bl / tiles);
  const int64_t tile = bl % tiles;
  const int64_t n0 = tile * kSkTileN;
  const int64_t nblk = K / 128;
  const int64_t kb0 = (int64_t)split * KB;
  const int nkb = (int)((nblk - kb0 < KB) ? nblk - kb0 : KB);

  // ---- the first T blocks' loads, before the tables (their latencies overlap) --------------
  const int64_t arows = M < 16 * MB ? M : 16 * MB;
  const int64_t wrows = (N - n0 < kSkTileN) ? N - n0 : kSkTileN;
  const rsrc_t ra = make_rsrc(A, (uint32_t)(arows * K * 2));
  const rsrc_t rw = make_rsrc(qweight + n0 * (K / 8), (uint32_t)(wrows * (K / 2)));
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  // activation rows: load j of wave w fills rows 4 (w MB + j) .. + 3, lane i row 4 (..) + i / 16,
  // physical chunk i % 16 holding the logical chunk (i % 16) ^ (row & 15)
  uint32_t avoff[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j)
    avoff[j] = (uint32_t)((lane >> 4) * K * 2) +
               (uint32_t)(((lane & 15) ^ ((4 * (wave * MB + j) + (lane >> 4)) & 15)) << 4);
  // codes: wave w's load covers rows 16 w + i / 4, bytes 16 (i % 4) of the block's 64
  const uint32_t wvoff = (uint32_t)((lane >> 2) * (K / 2)) + (uint32_t)((lane & 3) * 16);
  auto issue = [&](int b) {
    const int st = b % kSkStages;
    const int64_t g = kb0 + b;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int rb = wave * MB + j;      // rows 4 rb .. 4 rb + 3
      const uint32_t lds = lds0 + (uint32_t)(st * kStageB) + (uint32_t)(rb * 1024);
      const uint32_t so = (uint32_t)(4 * rb * K * 2) + (uint32_t)(g * 256);
      buffer_load16_lds_so(ra, lds, avoff[j], so);
    }
    const uint32_t lds = lds0 + (uint32_t)(st * kStageB + kAStageB) + (uint32_t)(wave * 1024);
    const uint32_t so = (uint32_t)(16 * wave * (K / 2)) + (uint32_t)(g * 64);
    buffer_load16_lds_so(rw, lds, wvoff, so);
  };
  for (int b = 0; b < kSkStages && b < nkb; ++b) issue(b);

  // ---- tables: r_k = fp16(2^b / s_k) in natural order, 2^-b per block, steps, zero points ----
  for (int k8 = tid; HAS_S && k8 < nkb * 16; k8 += 256) {
    float inv[8];
    float mx = 0.0f;
    if (HAS_S) {
      float sv[8];
      load8_f32<kF16>(s16 + kb0 * 128 + (int64_t)k8 * 8, sv);
#pragma unroll
      for (int t = 0; t < 8; ++t) inv[t] = __builtin_amdgcn_rcpf(sv[t]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) inv[t] = 1.0f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) mx = fmaxf(mx, inv[t]);
    mx = group_absmax<16>(mx);                  // a block's 16 chunks: one DPP row
    const int eb = escale_for_max(mx) - 4;      // 2^eb mx in [2^10, 2^11)
    const float sc = ldexpf(1.0f, eb);
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = (uint32_t)f2h(inv[2 * p] * sc) | ((uint32_t)f2h(inv[2 * p + 1] * sc) << 16);
    *reinterpret_cast<uint4*>(rtab + k8 * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    if ((k8 & 15) == 0) bfac[k8 >> 4] = ldexpf(1.0f, -eb);
  }
  const int64_t ngr = K / GS;
  for (int e = tid; e < nkb * kGpb * kSkTileN; e += 256) {
    const int r = e % kSkTileN, gq = e / kSkTileN;
    const int64_t row = (n0 + r < N) ? n0 + r : N - 1;
    const int64_t gg = kb0 * kGpb + gq;
    st_lds[e] = (n0 + r < N) ? scales16[row * ngr + gg] : (uint16_t)0;
    if (ZP) z_lds[e] = zeros[row * ngr + gg];
  }

  floatx4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  constexpr int kKKPerGroup = (GS == 64) ? 2 : 4;
  // the fp16 exponent bits of the decode, in a register so that mask-and-insert is one
  // v_and_or_b32
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));

  auto compute = [&](int b) {
    const char* sa = smem + (b % kSkStages) * kStageB;
    const char* rowp = sa + kAStageB + (16 * wave + li) * 64;   // this lane's code row
    // without s the weight operand is c(q) itself (exact) and no block scale applies
    const float bs = HAS_S ? bfac[b] : 1.0f;
    // Which channels a lane holds: G = 128: MFMA kk takes word 4 lg + kk (channels
    // 32 lg + 8 kk ..); G = 64: word 4 kk + lg, so MFMAs 0, 1 cover the block's first group
    uint32_t cw[4];
    if (GS == 128) {
      const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * lg);
      cw[0] = v.x; cw[1] = v.y; cw[2] = v.z; cw[3] = v.w;
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) cw[kk] = *reinterpret_cast<const uint32_t*>(rowp + 16 * kk + 4 * lg);
    }
#pragma unroll
    for (int h = 0; h < 4 / kKKPerGroup; ++h) {
      const int gq = b * kGpb + h;
      // subtrahends of the decoded pair (1024 + u, 64 + u'): 1032 and 72 for signed codes
      // (biased by the xor), 1024 + z and 64 + z with zero points
      const float z = ZP ? (float)z_lds[gq * kSkTileN + 16 * wave + li] : 8.0f;
      const half2_t sub2 = half2_t{(_Float16)(1024.0f + z), (_Float16)(64.0f + z)};
      floatx4 part[MB];
#pragma unroll
      for (int kk = h * kKKPerGroup; kk < (h + 1) * kKKPerGroup; ++kk) {
        const int ch = (GS == 128) ? 4 * lg + kk : 4 * kk + lg;   // the lane's 8-channel chunk
        const uint4 rv = HAS_S ? *reinterpret_cast<const uint4*>(rtab + b * 128 + ch * 8)
                               : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t rp[4] = {rv.x, rv.y, rv.z, rv.w};
        const uint32_t x = ZP ? cw[kk] : (cw[kk] ^ 0x88888888u);
        half8_t wf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // byte j (channels 2j, 2j + 1) to bytes 0 and 2; (t & 0x00F0000F) | magic is the fp16
          // pair (1024 + u_2j, 1024 + 16 u_2j+1); the fma gives (c(q_2j), c(q_2j+1)) exactly
          const uint32_t t =
              __builtin_amdgcn_perm(x, x, 0x0C000C00u | (uint32_t)j | ((uint32_t)j << 16));
          const uint32_t bits = (t & 0x00F0000Fu) | magic;
          const half2_t q = __builtin_elementwise_fma(
              __builtin_bit_cast(half2_t, bits), half2_t{(_Float16)1.0f, (_Float16)0.0625f},
              -sub2);
          const half2_t wv = HAS_S ? q * __builtin_bit_cast(half2_t, rp[j]) : q;
          wf[2 * j] = wv[0];
          wf[2 * j + 1] = wv[1];
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const half8_t af = *reinterpret_cast<const half8_t*>(sa + sk_swz(mb * 16 + li, ch));
          const floatx4 c0 = (kk == h * kKKPerGroup) ? floatx4{0.f, 0.f, 0.f, 0.f} : part[mb];
          part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af, c0, 0, 0, 0);
        }
      }
      // steps of this lane's output rows 4 lg .. 4 lg + 3 (times the block's 2^-b)
      const uint2 sr =
          *reinterpret_cast<const uint2*>(st_lds + gq * kSkTileN + 16 * wave + 4 * lg);
      const float sc[4] = {h2f((uint16_t)(sr.x & 0xFFFFu)) * bs, h2f((uint16_t)(sr.x >> 16)) * bs,
                           h2f((uint16_t)(sr.y & 0xFFFFu)) * bs, h2f((uint16_t)(sr.y >> 16)) * bs};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mb][r] = __builtin_fmaf(part[mb][r], sc[r], acc[mb][r]);
    }
  };

  // ---- main loop: block b waits for its own loads only (later blocks stay in flight); the
  // barrier makes everyone's visible and retires block b - 1, the last reader of the stage that
  // block b + T - 1 then takes (T stages). Blocks 0 .. T - 1 were issued before the loop, block
  // b + T - 1 (b >= 1) at b.
  for (int b = 0; b < nkb; ++b) {
    const int last_issued = (b + kSkStages - 2 > kSkStages - 1 ? b + kSkStages - 2 : kSkStages - 1);
    const int ahead = (last_issued < nkb - 1 ? last_issued : nkb - 1) - b;
    sk_wait_ahead<L, kSkStages - 1>(ahead);
    __syncthreads();   // (the first pass also publishes the tables)
    if (b >= 1 && b + kSkStages - 1 < nkb) issue(b + kSkStages - 1);
    compute(b);
  }

  // ---- several slices: the fp32 partial to the workspace; w4a16_splitk_reduce_kernel adds them
  if (S > 1) {
    floatx4* mine = partials + (((int64_t)split * tiles + tile) * 4 + wave) * MB * 64;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) mine[mb * 64 + lane] = acc[mb];
    return;
  }

  // D layout of the 16x16 MFMA: lane holds D[4 lg + r][li], r = 0..3: weight rows
  // n0 + 16 wave + 4 lg + r, activation row 16 mb + li
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = mb * 16 + li;
    const int64_t nb = n0 + 16 * wave + 4 * lg;
    if (m < M) {
      if (nb + 3 < N && ((N & 3) == 0)) {
        const uint32_t lo = (uint32_t)f2h(acc[mb][0]) | ((uint32_t)f2h(acc[mb][1]) << 16);
        const uint32_t hi = (uint32_t)f2h(acc[mb][2]) | ((uint32_t)f2h(acc[mb][3]) << 16);
        *reinterpret_cast<uint2*>(Y + m * N + nb) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) Y[m * N + nb + r] = f2h(acc[mb][r]);
      }
    }
  }
}

// The slices' partials of one 64-row tile per workgroup, added in slice order 0 .. S-1 (eight
// slices' loads in flight at a time), rounded once to fp16. Same lane layout as the main kernel.
template <int MB>
__global__ __launch_bounds__(256) void w4a16_splitk_reduce_kernel(
    const floatx4* __restrict__ partials, int64_t tiles, int S, int64_t M, int64_t N,
    uint16_t* __restrict__ Y) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t tile = blockIdx.x;
  const floatx4* src = partials + (tile * 4 + wave) * MB * 64 + lane;
  const int64_t slice_stride = tiles * 4 * MB * 64;
  floatx4 acc[MB];
  constexpr int kC = 8;
  for (int j0 = 0; j0 < S; j0 += kC) {
    floatx4 v[kC][MB];
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const int j = (j0 + u < S) ? j0 + u : 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) v[u][mb] = src[j * slice_stride + mb * 64];
    }
#pragma unroll
    for (int u = 0; u < kC; ++u)
      if (j0 + u < S)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = (j0 + u == 0) ? v[u][mb] : acc[mb] + v[u][mb];
  }
  const int64_t n0 = tile * kSkTileN;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = mb * 16 + li;
    const int64_t nb = n0 + 16 * wave + 4 * lg;
    if (m < M) {
      if (nb + 3 < N && ((N & 3) == 0)) {
        const uint32_t lo = (uint32_t)f2h(acc[mb][0]) | ((uint32_t)f2h(acc[mb][1]) << 16);
        const uint32_t hi = (uint32_t)f2h(acc[mb][2]) | ((uint32_t)f2h(acc[mb][3]) << 16);
        *reinterpret_cast<uint2*>(Y + m * N + nb) = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) Y[m * N + nb + r] = f2h(acc[mb][r]);
      }
    }
  }
}

hipError_t launch_w4a16_splitk(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                               const uint32_t* qweight, const uint16_t* scales16,
                               const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 1 || M > 64 || K % 128) return hipErrorInvalidValue;
  const W4a16SplitPlan p = w4a16_splitk_plan(M, N, K);
  if (p.S > 1 && (ws == nullptr || ws_bytes < p.ws_bytes)) return hipErrorInvalidValue;
  const bool zp = zeros != nullptr;
  const size_t lds = (size_t)sk_tables_bytes(p.KB, group, zp);
  floatx4* partials = p.S > 1 ? static_cast<floatx4*>(ws) : nullptr;
  const unsigned grid = (unsigned)(p.tiles * p.S);
#define AWQ_SPK(MB_, GS_, ZP_, HS_)                                                              \
  w4a16_splitk_kernel<MB_, GS_, ZP_, HS_><<<grid, 256, lds, stream>>>(                          \
      A, M, N, K, qweight, scales16, zeros, s16, Y, p.tiles, p.S, p.KB, partials)
#define AWQ_SPK_S(MB_, GS_, ZP_) \
  do { if (s16) AWQ_SPK(MB_, GS_, ZP_, true); else AWQ_SPK(MB_, GS_, ZP_, false); } while (0)
#define AWQ_SPK_Z(MB_, GS_) \
  do { if (zp) AWQ_SPK_S(MB_, GS_, true); else AWQ_SPK_S(MB_, GS_, false); } while (0)
#define AWQ_SPK_G(MB_) \
  do { if (group == 64) AWQ_SPK_Z(MB_, 64); else AWQ_SPK_Z(MB_, 128); } while (0)
  if (p.MB == 1)
    AWQ_SPK_G(1);
  else if (p.MB == 2)
    AWQ_SPK_G(2);
  else
    AWQ_SPK_G(4);
#undef AWQ_SPK_G
#undef AWQ_SPK_Z
#undef AWQ_SPK_S
#undef AWQ_SPK
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const unsigned rgrid = (unsigned)p.tiles;
  if (p.MB == 1)
    w4a16_splitk_reduce_kernel<1><<<rgrid, 256, 0, stream>>>(partials, p.tiles, (int)p.S, M, N, Y);
  else if (p.MB == 2)
    w4a16_splitk_reduce_kernel<2><<<rgrid, 256, 0, stream>>>(partials, p.tiles, (int)p.S, M, N, Y);
  else
    w4a16_splitk_reduce_kernel<4><<<rgrid, 256, 0, stream>>>(partials, p.tiles, (int)p.S, M, N, Y);
  return hipGetLastError();
}

}  // namespace awq
