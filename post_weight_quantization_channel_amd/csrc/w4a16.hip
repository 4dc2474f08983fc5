// W4A16 GEMM on the packed AWQ artefacts: QuantLinear.forward of "AWQ 量化方案..."
// (qwbw.cn/news/39982), section 三 -- scale the input per channel, dequantize the packed codes
// with the per-group steps, then a linear layer:
//   Y[m, n] = sum_k (A[m,k] / s[k]) * q[n,k] * step[n, k/128]
// The activation is divided by s because the weight was multiplied by s (AWQ notes,
// bg51717.github.io/14592, section 方法: Q(w s) x / s).
//
// gfx950 design (batch M <= 64 per pass; the bytes of the packed weight dominate, so the kernel
// is built to stream them at HBM speed):
//   * v_mfma_f32_16x16x32_f16 with the weights as the 16-row A operand (rows n) and the
//     activations as the B operand (columns m, zero beyond M);
//   * a workgroup owns 16 weight rows and all of K; its 8 waves take the 128-channel groups
//     round-robin, and every lane issues the 16-byte loads of its groups (up to 4 at a time,
//     double-buffered) before unpacking any of them;
//   * unpacking: one 32-bit word holds the codes of 8 consecutive channels. x = w ^ 0x88888888
//     turns each two's-complement nibble into q + 8; (x >> 4j) & 0x000F000F | 0x64006400 is the
//     fp16 pair (1024 + q_j + 8, 1024 + q_{j+4} + 8) and one packed subtract of 1032 gives
//     (q_j, q_{j+4}) exactly. The MFMA k slots therefore hold channels in the order
//     0,4,1,5,2,6,3,7 of each 8; the activations are permuted the same way, which leaves the
//     dot products unchanged;
//   * 1/s is folded into the weight pairs (one packed multiply per pair) from a table of
//     fp16(1/s) that each workgroup builds in LDS, stored in the same permuted order; the
//     per-group step multiplies the fp32 partial of each group's 4 MFMAs;
//   * the eight waves' partial outputs are added in a fixed order through LDS.
// Rounding: 1/s and q/s are each rounded once to fp16, the accumulation is fp32 and Y is rounded
// once to fp16.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {
constexpr int kRows = 16;       // weight rows per workgroup
constexpr int kWaves = 8;       // waves per workgroup; wave w takes groups w, w + 8, ...
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 4;       // groups whose weight words a lane keeps in flight at once
constexpr int kTableIters = 4;  // table chunks per thread: 4 * 512 * 16 B = 32 KiB
constexpr int kMaxK = 12288;    // LDS tables + reduction buffer stay below 64 KiB
constexpr size_t kActLdsBytes = 32768;   // largest M * K * 2 staged as fp16(A / s) in LDS
}  // namespace

// s = 1 for every channel (fp16 1.0): read instead of s16 when s^-1 has been folded into the
// producer of A (the kernels' HAS_S = false instances). Selecting the pointer at compile time
// keeps the HAS_S = true code unchanged: a run-time select measured ~10% slower on the
// latency-bound decode path. (The table is only referenced from device code: as a namespace-scope
// const object it has internal linkage, so the runtime cannot look up its address by name.)
struct OnesTable {
  uint16_t v[kMaxK];
  constexpr OnesTable() : v() {
    for (int i = 0; i < kMaxK; ++i) v[i] = 0x3C00;
  }
};
__device__ const OnesTable kOnes16;

// permuted position of channel t (0..7) inside its block of 8: order 0,4,1,5,2,6,3,7
__device__ __forceinline__ int perm8(int t) { return ((t & 3) << 1) | (t >> 2); }

// ACT_LDS (small batches, M * K * 2 bytes <= kActLdsBytes): the workgroup first writes
// fp16(A / s) for all M rows into LDS in the permuted order, and the weights are used as exact
// integers. Otherwise 1/s is folded into the weight pairs and the activations are read from
// global memory.
//
// Latency structure: a workgroup's critical path is table loads -> table -> weight loads ->
// unpack/MFMA -> cross-wave sum. The table loads (at most 2 per thread, into registers) are
// issued first and the weight loads right after them, so both are in flight together (loads
// complete in order: consuming the table waits only for the table loads); 8 waves split the
// groups so each unpacks only K/1024 of them.
// Bytes of the skinny kernel's LDS regions (the launcher sizes the dynamic LDS with the same).
__host__ __device__ constexpr int64_t w4a16_red_bytes(int MB) { return (int64_t)kWaves * MB * 64 * 16; }

// SR > 0: a row has at most kThreads 16-byte chunks of channels (K <= 4096), so thread t loads
// chunk t of 1/s and, when A is staged, chunk t of each of the (at most SR) staged rows: the
// prologue holds 1 + SR table loads per thread instead of up to 2 kTableIters, and 1 (groups of
// 128) or 2 (groups of 64) step loads instead of up to 6, and a wave's groups (at most 4) are
// one chunk of weight loads, so the second chunk buffer goes too. These instances fit in 80
// VGPRs without spilling. The staged ones are held to that: three 512-thread workgroups fit on
// a CU, and a GEMV with more than 512 workgroups (N > 8192) runs in one round instead of two.
// (Held to it too, the unstaged ones (batches of 5 to 16) ran 2% slower at 11008 x 4096:
// they are bound by reading A once per workgroup, not by residency.)
template <int MB, bool ACT_LDS, int GS, bool ZP, bool HAS_S, int SR>
__global__ __launch_bounds__(kThreads, (MB == 1 && SR > 0 && ACT_LDS) ? 6 : 1)
void w4a16_kernel(const uint16_t* __restrict__ A, int64_t M,
                                                         int64_t N, int64_t K,
                                                         const uint32_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales16,
                                                         const uint8_t* __restrict__ zeros,
                                                         const uint16_t* __restrict__ s16_in,
                                                         uint16_t* __restrict__ Y, int64_t m0) {
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const uint16_t* __restrict__ s16 = HAS_S ? s16_in : kOnes16.v;
  // LDS: [K] fp16 1/s (permuted) or [mrows][K] fp16 A / s (permuted; ACT_LDS) -- the same
  // region holds the cross-wave reduction buffer after the main loop -- then the 16 rows' fp32
  // steps [K / GS][16], then (ZP) their zero points as fp16 (1024 + z) [K / GS][16].
  const int64_t mrows = ACT_LDS ? (M - m0 < 16 ? M - m0 : 16) : 0;
  const int64_t table_bytes = ACT_LDS ? mrows * K * 2 : K * 2;
  const int64_t region0 = table_bytes > w4a16_red_bytes(MB) ? table_bytes : w4a16_red_bytes(MB);
  const int64_t ngr = K / GS;                                   // quantization groups
  uint16_t* table = reinterpret_cast<uint16_t*>(dyn);
  floatx4* red = reinterpret_cast<floatx4*>(dyn);
  float* step_lds = reinterpret_cast<float*>(dyn + region0);
  uint16_t* zero_lds = reinterpret_cast<uint16_t*>(dyn + region0 + ngr * kRows * 4);
  uint4* trash = reinterpret_cast<uint4*>(dyn + region0 + ngr * kRows * (ZP ? 6 : 4));  // 16 B

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;   // weight row of the A operand / activation column of the B operand
  const int lg = lane >> 4;   // which 32-channel quarter of a 128-channel group
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t groups = K / 128;                               // 128-channel blocks
  const int64_t words_per_row = K / 8;

  // All prologue loads are unconditional (out-of-range indices are clamped and their values
  // discarded): a load inside a divergent branch makes the compiler wait for it -- and, as loads
  // complete in order, for every earlier load -- at the branch's join.
  const int kc = (int)(K / 8);                                  // 16-byte chunks per row
  const int gr = (int)groups;
  // ---- 1. table loads into registers (at most kTableIters per thread) ------------------------
  const int tchunks = ACT_LDS ? (int)mrows * kc : kc;           // 16-byte chunks of the table
  constexpr int kTI = SR ? 1 : kTableIters;                      // 1/s loads per thread
  constexpr int kTA = !ACT_LDS ? 1 : (SR ? SR : kTableIters);    // A loads per thread
  uint4 ta[kTA], ts[kTI];
  if constexpr (SR > 0) {
    const int k8 = tid < kc ? tid : 0;
    ts[0] = *reinterpret_cast<const uint4*>(s16 + (int64_t)k8 * 8);
    if (ACT_LDS) {
#pragma unroll
      for (int r = 0; r < kTA; ++r) {
        const int64_t rr = r < mrows ? r : mrows - 1;
        ta[r] = *reinterpret_cast<const uint4*>(A + (m0 + rr) * K + (int64_t)k8 * 8);
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < kTI; ++it) {
      const int e = tid + it * kThreads;
      const int ec = e < tchunks ? e : 0;
      const int k8 = ACT_LDS ? ec % kc : ec;
      ts[it] = *reinterpret_cast<const uint4*>(s16 + (int64_t)k8 * 8);
      if (ACT_LDS) ta[it] = *reinterpret_cast<const uint4*>(A + (m0 + ec / kc) * K + (int64_t)k8 * 8);
    }
  }
  // steps: with SR > 0, K <= 4096 holds at most (4096 / GS) * kRows of them (1 or 2 per thread)
  constexpr int kStepIters = SR ? (4096 / GS * kRows + kThreads - 1) / kThreads
                                : (kMaxK / GS * kRows + kThreads - 1) / kThreads;
  const int ng = (int)ngr;
  uint16_t sraw[kStepIters];
  uint8_t zraw[kStepIters];
#pragma unroll
  for (int it = 0; it < kStepIters; ++it) {
    const int e = tid + it * kThreads;
    const int ec = e < ng * kRows ? e : 0;
    const int64_t row = (n0 + (ec & (kRows - 1)) < N) ? n0 + (ec & (kRows - 1)) : N - 1;
    sraw[it] = scales16[row * ngr + (ec >> 4)];
    if (ZP) zraw[it] = zeros[row * ngr + (ec >> 4)];
  }

  __builtin_amdgcn_sched_barrier(0);   // keep the issue order: tables, steps, then weights
  // ---- 2. this wave's weight words (first chunk) --------------------------------------------
  const int64_t n = n0 + li;
  const bool nok = n < N;
  const uint4* wrow = reinterpret_cast<const uint4*>(qweight + (nok ? n : N - 1) * words_per_row) + lg;
  const int my_groups = (gr - wave + kWaves - 1) / kWaves;     // g = wave + kWaves i
  uint4 wbuf[2][kChunk];
  auto load_chunk = [&](int c, uint4 (&dst)[kChunk]) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = c * kChunk + u;
      const int gi = (i < my_groups) ? wave + kWaves * i : wave;
      dst[u] = wrow[(int64_t)gi * 4];      // rows >= N: a valid row whose results are dropped
    }
  };
  load_chunk(0, wbuf[0]);
  // an empty asm that may read or write the weight rows: no weight load above may be moved
  // below it (sinking them to their first use, after the barrier, would serialise them behind
  // the table). It names only the row pointer, not the loaded values, so it adds no wait.
  asm volatile("" : : "v"(wrow) : "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. tables into LDS (straight-line: out-of-range entries go to a trash slot, so no
  // load above is sunk into a conditional block and waited for there) ------------------------
  // table entry: fp16(a / s) (a = 1 without staging) of 8 channels, in the permuted order
  auto table_chunk = [&](const uint4& sv4, const uint4& av4, uint4* dst) {
    const uint32_t sw[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
    const uint32_t aw[4] = {av4.x, av4.y, av4.z, av4.w};
    uint16_t h[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float sv = h2f((uint16_t)(sw[t >> 1] >> (16 * (t & 1))));
      const float num = ACT_LDS ? h2f((uint16_t)(aw[t >> 1] >> (16 * (t & 1)))) : 1.0f;
      h[perm8(t)] = f2h(num / sv);
    }
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) w[p] = (uint32_t)h[2 * p] | ((uint32_t)h[2 * p + 1] << 16);
    *dst = make_uint4(w[0], w[1], w[2], w[3]);
  };
  if constexpr (SR > 0) {
#pragma unroll
    for (int r = 0; r < (ACT_LDS ? kTA : 1); ++r) {
      const bool ok = tid < kc && (!ACT_LDS || r < mrows);
      table_chunk(ts[0], ACT_LDS ? ta[r] : make_uint4(0, 0, 0, 0),
                  ok ? reinterpret_cast<uint4*>(table + (int64_t)r * K + tid * 8) : trash);
    }
  } else {
#pragma unroll
    for (int it = 0; it < kTI; ++it) {
      const int e = tid + it * kThreads;
      table_chunk(ts[it], ACT_LDS ? ta[it] : make_uint4(0, 0, 0, 0),
                  (e < tchunks) ? reinterpret_cast<uint4*>(table + e * 8) : trash);
    }
  }
#pragma unroll
  for (int it = 0; it < kStepIters; ++it) {
    const int e = tid + it * kThreads;
    const float stv = (n0 + (e & (kRows - 1)) < N) ? h2f(sraw[it]) : 0.0f;
    float* sdst = (e < ng * kRows) ? step_lds + e : reinterpret_cast<float*>(trash);
    *sdst = stv;
    if (ZP) {
      uint16_t* zdst = (e < ng * kRows) ? zero_lds + e : reinterpret_cast<uint16_t*>(trash);
      *zdst = f2h(1024.0f + (float)zraw[it]);   // exact: the subtrahend of the unpack
    }
  }
  __syncthreads();

  floatx4 acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const uint4 (&cur)[kChunk], int c) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = c * kChunk + u;
      if (i >= my_groups) break;                            // uniform over the wave
      const int64_t g = wave + kWaves * i;                  // 128-channel block
      const int64_t kbase = g * 128 + lg * 32;              // this lane's 32 channels
      const uint32_t words[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
      // fp16 subtrahend of the unpack: 1032 (signed codes, biased by the xor) or 1024 + z of
      // this lane's row and group (the lane's 32 channels lie in one group for GS = 64 too)
      half2_t sub2 = half2_t{(_Float16)1032.0f, (_Float16)1032.0f};
      if (ZP) {
        const int64_t gz = (GS == 64) ? 2 * g + (lg >> 1) : g;
        const _Float16 zh = __builtin_bit_cast(_Float16, zero_lds[gz * kRows + li]);
        sub2 = half2_t{zh, zh};
      }
      half8_t wf[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {                          // word v: channels kbase + 8v ..
        const uint32_t x = ZP ? words[v] : (words[v] ^ 0x88888888u);
        uint32_t invw[4] = {0u, 0u, 0u, 0u};
        if (!ACT_LDS) {
          const uint4 inv = *reinterpret_cast<const uint4*>(table + kbase + 8 * v);
          invw[0] = inv.x; invw[1] = inv.y; invw[2] = inv.z; invw[3] = inv.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t bits = ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
          half2_t q = __builtin_bit_cast(half2_t, bits) - sub2;
          if (!ACT_LDS) q = q * __builtin_bit_cast(half2_t, invw[j]);
          wf[v][2 * j] = q[0];
          wf[v][2 * j + 1] = q[1];
        }
      }
      // per-group fp32 steps of this lane's 4 output rows (rows 4 lg + r); with GS = 64 the two
      // halves of the block have their own steps, so each MFMA is done twice with the A operand
      // of the other half's lanes (lg < 2 hold channels 0..63, lg >= 2 channels 64..127) zeroed
      const int64_t gs0 = (GS == 64) ? 2 * g : g;
      const floatx4 st0 = *reinterpret_cast<const floatx4*>(step_lds + gs0 * kRows + 4 * lg);
      floatx4 st1 = st0;
      if (GS == 64) st1 = *reinterpret_cast<const floatx4*>(step_lds + (gs0 + 1) * kRows + 4 * lg);
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int64_t m = m0 + b * 16 + li;
        floatx4 part = {0.f, 0.f, 0.f, 0.f}, part1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // Batch rows past M read row M - 1 (a valid row): column m of the MFMA result depends
          // on activation row m only, and columns m >= M are never stored. Zeroing instead
          // would put each load under a divergent branch that waits for it at once.
          const int64_t mc = (m < M) ? m : M - 1;
          half8_t af;
          if (ACT_LDS) {
            af = *reinterpret_cast<const half8_t*>(table + (mc - m0) * K + kbase + 8 * v);
          } else {
            const uint4 a = *reinterpret_cast<const uint4*>(A + mc * K + kbase + 8 * v);
            // permute channels 0..7 to the order 0,4,1,5,2,6,3,7 of the weight operand
            const uint32_t p0 = __builtin_amdgcn_perm(a.z, a.x, 0x05040100u);  // (a0, a4)
            const uint32_t p1 = __builtin_amdgcn_perm(a.z, a.x, 0x07060302u);  // (a1, a5)
            const uint32_t p2 = __builtin_amdgcn_perm(a.w, a.y, 0x05040100u);  // (a2, a6)
            const uint32_t p3 = __builtin_amdgcn_perm(a.w, a.y, 0x07060302u);  // (a3, a7)
            af = __builtin_bit_cast(half8_t, make_uint4(p0, p1, p2, p3));
          }
          if (GS == 64) {
            const half8_t w0 = (lg < 2) ? wf[v] : half8_t{};
            const half8_t w1 = (lg < 2) ? half8_t{} : wf[v];
            part = __builtin_amdgcn_mfma_f32_16x16x32_f16(w0, af, part, 0, 0, 0);
            part1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(w1, af, part1, 0, 0, 0);
          } else {
            part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[v], af, part, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[b][r] = __builtin_fmaf(part[r], st0[r], acc[b][r]);
          if (GS == 64) acc[b][r] = __builtin_fmaf(part1[r], st1[r], acc[b][r]);
        }
      }
    }
  };

  if constexpr (SR > 0) {
    // K <= 4096: at most 32 groups, so a wave's groups (at most 4) are the one chunk in flight
    process(wbuf[0], 0);
  } else {
    // chunks alternate between the two register buffers (static indices: no scratch)
    const int nchunks = (my_groups + kChunk - 1) / kChunk;
    for (int c = 0; c < nchunks; c += 2) {
      if (c + 1 < nchunks) load_chunk(c + 1, wbuf[1]);
      process(wbuf[0], c);
      if (c + 1 < nchunks) {
        if (c + 2 < nchunks) load_chunk(c + 2, wbuf[0]);
        process(wbuf[1], c + 1);
      }
    }
  }

  __syncthreads();   // the reduction buffer reuses the table's LDS: every wave is done with it
#pragma unroll
  for (int b = 0; b < MB; ++b) red[(wave * MB + b) * 64 + lane] = acc[b];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      floatx4 t = red[b * 64 + lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const floatx4 o = red[(w * MB + b) * 64 + lane];
        t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
      }
      // D layout of the 16x16 MFMA: lane holds D[4*(lane/16) + r][lane % 16], r = 0..3,
      // i.e. weight rows 4*lg + r and activation column li.
      const int64_t m = m0 + b * 16 + li;
      const int64_t nb = n0 + 4 * lg;
      if (m < M) {
        if (nb + 3 < N && ((N & 3) == 0)) {
          const uint32_t lo = (uint32_t)f2h(t[0]) | ((uint32_t)f2h(t[1]) << 16);
          const uint32_t hi = (uint32_t)f2h(t[2]) | ((uint32_t)f2h(t[3]) << 16);
          *reinterpret_cast<uint2*>(Y + m * N + nb) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) Y[m * N + nb + r] = f2h(t[r]);
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------------------------
// Larger batches (M > 64): a tiled MFMA GEMM. Workgroup tile 128 (batch rows m) x 64 (weight
// rows n), BK = 128 = one quantization group per K step, 4 waves of 64 x 32 (2 x 2), each a
// 4 x 2 grid of v_mfma_f32_16x16x32_f16 blocks (weights as the A operand, activations as B).
// The workgroup first builds a table of fp16(1/s) for all K in LDS. Per K step every thread
// loads 128 bytes of the activation tile, one 16-byte word group of the packed weight tile and
// its row's step into registers (the next step is prefetched while the current one computes),
// unpacks its 32 codes into fp16 q * (fp16(step) * fp16(1/s)) in natural channel order (two
// packed multiplies per channel pair) and writes both tiles to LDS (double-buffered). The weight
// tile is unpacked once per 128-row batch tile, not once per batch row. LDS rows are 256 bytes; 16-byte chunks are XOR-swizzled by (row & 15) so the
// fragment reads of 16 consecutive rows touch distinct banks.
namespace {
constexpr int TBM = 128, TBN = 64, TBK = 128;
constexpr int kTileStage = (TBM + TBN) * TBK * 2;   // 48 KiB
__device__ __forceinline__ int tswz(int row, int chunk) {   // byte offset inside a 256-byte row
  return row * (TBK * 2) + ((chunk ^ (row & 15)) << 4);
}
}  // namespace

template <int GS, bool ZP, bool HAS_S>
__global__ __launch_bounds__(256) void w4a16_tiled_kernel(const uint16_t* __restrict__ A,
                                                          int64_t M, int64_t N, int64_t K,
                                                          const uint32_t* __restrict__ qweight,
                                                          const uint16_t* __restrict__ scales16,
                                                          const uint8_t* __restrict__ zeros,
                                                          const uint16_t* __restrict__ s16_in,
                                                          uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileStage];
  const uint16_t* __restrict__ s16 = HAS_S ? s16_in : kOnes16.v;
  __shared__ __attribute__((aligned(16))) uint16_t inv_s[kMaxK];   // fp16(1/s), natural order
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;     // wave tile: batch rows 64 wm.., weight rows 32 wn..
  const int64_t tilesN = (N + TBN - 1) / TBN;
  const int64_t m0 = (int64_t)(blockIdx.x / tilesN) * TBM;
  const int64_t n0 = (int64_t)(blockIdx.x % tilesN) * TBN;
  const int64_t groups = K / 128;      // 128-channel K steps
  const int64_t ngr = K / GS;          // quantization groups

  // activation tile: thread t loads rows (t / 16) + 16 j (j = 0..7), 16-byte chunk t % 16
  const int arow = tid >> 4, achunk = tid & 15;
  // weight tile: thread t loads row t / 4, words 4 (t % 4) .. 4 (t % 4) + 3 of the group
  const int wrow_l = tid >> 2, wq = tid & 3;
  const int64_t wn_row = n0 + wrow_l;
  const bool wok = wn_row < N;
  const uint4* wsrc = reinterpret_cast<const uint4*>(qweight + (wok ? wn_row : 0) * (K / 8)) + wq;

  constexpr int kARows = TBM / 16;   // activation rows per thread per step
  for (int64_t k8 = tid; k8 < K / 8; k8 += 256) {
    float sv[8];
    load8_f32<kF16>(s16 + k8 * 8, sv);
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = (uint32_t)f2h(1.0f / sv[2 * p]) | ((uint32_t)f2h(1.0f / sv[2 * p + 1]) << 16);
    *reinterpret_cast<uint4*>(inv_s + k8 * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __syncthreads();

  // step and zero are 32 bits wide: two 16-bit fields would share a register, and merging a
  // load into half of it waits for the load at once, which undoes the two-step prefetch
  struct Regs {
    uint4 a[kARows];
    uint4 w;
    uint32_t step;   // fp16 bits
    uint32_t zero;   // ZP: z of the thread's row and group
  };
  auto gload = [&](int64_t g, Regs& R) {
#pragma unroll
    for (int j = 0; j < kARows; ++j) {
      const int64_t m = m0 + arow + 16 * j;
      R.a[j] = (m < M) ? *reinterpret_cast<const uint4*>(A + m * K + g * 128 + achunk * 8)
                       : make_uint4(0, 0, 0, 0);
    }
    R.w = wok ? wsrc[g * 4] : make_uint4(0, 0, 0, 0);
    // the thread's 32 channels 128 g + 32 wq .. lie in one group for GS = 64 too
    const int64_t gq = (GS == 64) ? 2 * g + (wq >> 1) : g;
    R.step = wok ? (uint32_t)scales16[wn_row * ngr + gq] : 0u;
    R.zero = (ZP && wok) ? (uint32_t)zeros[wn_row * ngr + gq] : 0u;
  };
  auto lstore = [&](int stage, int64_t g, const Regs& R) {
    char* sa = smem + stage * kTileStage;
    char* sw = sa + TBM * TBK * 2;
#pragma unroll
    for (int j = 0; j < kARows; ++j)
      *reinterpret_cast<uint4*>(sa + tswz(arow + 16 * j, achunk)) = R.a[j];
    // unpack 4 words = 32 channels k = 128 g + 32 wq + 8 v + t into q * (step * 1/s) in fp16
    const _Float16 sth = __builtin_bit_cast(_Float16, (uint16_t)R.step);
    const half2_t st2 = half2_t{sth, sth};
    const _Float16 subh = ZP ? (_Float16)(1024.0f + (float)R.zero) : (_Float16)1032.0f;
    const half2_t sub2 = half2_t{subh, subh};
    const uint32_t words[4] = {R.w.x, R.w.y, R.w.z, R.w.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 iv = *reinterpret_cast<const uint4*>(inv_s + g * 128 + wq * 32 + v * 8);
      // (1/s) pairs (j, j + 4) to match the unpack order
      const uint32_t i04 = __builtin_amdgcn_perm(iv.z, iv.x, 0x05040100u);
      const uint32_t i15 = __builtin_amdgcn_perm(iv.z, iv.x, 0x07060302u);
      const uint32_t i26 = __builtin_amdgcn_perm(iv.w, iv.y, 0x05040100u);
      const uint32_t i37 = __builtin_amdgcn_perm(iv.w, iv.y, 0x07060302u);
      const uint32_t invp[4] = {i04, i15, i26, i37};
      const uint32_t x = ZP ? words[v] : (words[v] ^ 0x88888888u);
      uint32_t pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t bits = ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const half2_t q = __builtin_bit_cast(half2_t, bits) - sub2;
        const half2_t c = st2 * __builtin_bit_cast(half2_t, invp[j]);
        pr[j] = __builtin_bit_cast(uint32_t, q * c);              // channels (j, j + 4)
      }
      // back to natural order: (0,1) (2,3) (4,5) (6,7)
      const uint32_t n01 = __builtin_amdgcn_perm(pr[1], pr[0], 0x05040100u);
      const uint32_t n23 = __builtin_amdgcn_perm(pr[3], pr[2], 0x05040100u);
      const uint32_t n45 = __builtin_amdgcn_perm(pr[1], pr[0], 0x07060302u);
      const uint32_t n67 = __builtin_amdgcn_perm(pr[3], pr[2], 0x07060302u);
      *reinterpret_cast<uint4*>(sw + tswz(wrow_l, wq * 4 + v)) = make_uint4(n01, n23, n45, n67);
    }
  };

  floatx4 acc[2][4];   // [weight block i][batch block j]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int li = lane & 15, lg = lane >> 4;
  auto compute = [&](int stage) {
    const char* sa = smem + stage * kTileStage;
    const char* sw = sa + TBM * TBK * 2;
#pragma unroll
    for (int kk = 0; kk < TBK / 32; ++kk) {
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
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  };

  // Two register sets: the loads of step g + 2 are issued while step g computes, so each load
  // has two steps of MFMA work to land before its tile is written to LDS.
  Regs R0, R1;
  gload(0, R0);
  if (groups > 1) gload(1, R1);
  lstore(0, 0, R0);
  __syncthreads();
  for (int64_t g = 0; g < groups; g += 2) {
    if (g + 2 < groups) gload(g + 2, R0);
    compute(0);
    if (g + 1 < groups) lstore(1, g + 1, R1);
    __syncthreads();
    if (g + 1 >= groups) break;
    if (g + 3 < groups) gload(g + 3, R1);
    compute(1);
    if (g + 2 < groups) lstore(0, g + 2, R0);
    __syncthreads();
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

// ---------------------------------------------------------------------------------------------
// The same tiling with every main-loop load moved into LDS by the buffer unit (buffer_load ...
// lds), so that no load's result goes through a register and the compiler places no wait on them:
// the kernel orders LDS against these loads itself, with vmcnt waits and barriers. Per K step
// (128 channels) the workgroup moves the activation tile (128 rows x 256 B, 8 loads of 1 KiB per
// wave, written in the swizzled layout the fragment reads expect: lane i of a load fills physical
// chunk i % 16 of its row, so it fetches the logical chunk (i % 16) ^ (row & 15)) and the raw
// codes of its 64 weight rows (64 x 64 B, one load per wave). The steps (and zero points) of the
// 64 rows for all K, and fp16(1/s) for all K, are tables in LDS filled once. Step g:
//   wait for step g's loads; barrier; issue step g + 1's loads into the other stage (its last
//   reader, step g - 1, is behind the barrier); unpack step g's codes into q * (step / s) fp16 in
//   the swizzled layout; barrier; the MFMAs of step g.
// Rows past M or N read as zeros (the buffer ranges end at the last valid row) and their outputs
// are not stored. Against the register-staged kernel above (whose loads sat under per-row
// conditions, so the compiler drained them at every loop head) this is 6-10% faster at M = 512;
// what bounds it now is LDS traffic: ~170 KiB per step and CU (activation and weight tiles in,
// each fragment read by two waves, the codes and 1/s), against 32 MFMAs per wave.
namespace {
constexpr int kRawStage = TBN * 64;                   // 4 KiB of packed codes per step
constexpr int kAStage = TBM * TBK * 2;                // 32 KiB of activations per step
constexpr int kWStage = TBN * TBK * 2;                // 16 KiB of unpacked weights per step
// two stages each of activations, codes and unpacked weights: 104 KiB
constexpr int kDmaSmem = 2 * (kAStage + kRawStage + kWStage);
// s_waitcnt immediate: at most n vector-memory loads outstanding (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
}  // namespace

// bytes of the dynamic tables: fp16 1/s [K], fp16 steps [64][K / GS], (ZP) uint8 zeros [64][K / GS]
__host__ __device__ constexpr int64_t w4a16_dma_tables(int64_t K, int GS, bool ZP) {
  return K * 2 + (int64_t)TBN * (K / GS) * 2 + (ZP ? (int64_t)TBN * (K / GS) : 0);
}

template <int GS, bool ZP, bool HAS_S>
__global__ __launch_bounds__(256) void w4a16_tiled_dma_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t N, int64_t K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales16,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ s16_in,
    uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(1024))) char smem[kDmaSmem];
  // LDS: activation stages [2][32 KiB], unpacked weight stages [2][16 KiB], code stages [2][4 KiB]
  constexpr int kWBase = 2 * kAStage, kRawBase = 2 * kAStage + 2 * kWStage;
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const uint16_t* __restrict__ s16 = HAS_S ? s16_in : kOnes16.v;
  const int64_t ngr = K / GS;
  uint16_t* inv_s = reinterpret_cast<uint16_t*>(dyn);                 // [K]
  uint16_t* st_lds = inv_s + K;                                       // [64][ngr] fp16 steps
  uint8_t* z_lds = reinterpret_cast<uint8_t*>(st_lds + TBN * ngr);    // [64][ngr] (ZP)

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

  // ---- tables (plain loads: the compiler's waits here cost nothing) -------------------------
  for (int64_t k8 = tid; k8 < K / 8; k8 += 256) {
    float sv[8];
    load8_f32<kF16>(s16 + k8 * 8, sv);
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = (uint32_t)f2h(1.0f / sv[2 * p]) | ((uint32_t)f2h(1.0f / sv[2 * p + 1]) << 16);
    *reinterpret_cast<uint4*>(inv_s + k8 * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int64_t e = tid; e < TBN * ngr; e += 256) {
    const int64_t r = e / ngr, gq = e % ngr;
    const int64_t row = (n0 + r < N) ? n0 + r : N - 1;
    st_lds[e] = scales16[row * ngr + gq];
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
    const _Float16 sth = __builtin_bit_cast(_Float16, st_lds[wrow_l * ngr + gq]);
    const half2_t st2 = half2_t{sth, sth};
    const _Float16 subh = ZP ? (_Float16)(1024.0f + (float)z_lds[wrow_l * ngr + gq])
                             : (_Float16)1032.0f;
    const half2_t sub2 = half2_t{subh, subh};
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 iv = *reinterpret_cast<const uint4*>(inv_s + g * 128 + wq * 32 + v * 8);
      const uint32_t i04 = __builtin_amdgcn_perm(iv.z, iv.x, 0x05040100u);
      const uint32_t i15 = __builtin_amdgcn_perm(iv.z, iv.x, 0x07060302u);
      const uint32_t i26 = __builtin_amdgcn_perm(iv.w, iv.y, 0x05040100u);
      const uint32_t i37 = __builtin_amdgcn_perm(iv.w, iv.y, 0x07060302u);
      const uint32_t invp[4] = {i04, i15, i26, i37};
      const uint32_t x = ZP ? words[v] : (words[v] ^ 0x88888888u);
      uint32_t pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t bits = ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const half2_t q = __builtin_bit_cast(half2_t, bits) - sub2;
        const half2_t c = st2 * __builtin_bit_cast(half2_t, invp[j]);
        pr[j] = __builtin_bit_cast(uint32_t, q * c);
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
  auto compute = [&](int64_t g, int st) {
    const char* sa = smem + st * kAStage;
    const char* sw = smem + kWBase + (int)(g & 1) * kWStage;
#pragma unroll
    for (int kk = 0; kk < TBK / 32; ++kk) {
      const int chunk = kk * 4 + lg;
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
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[i], af[j], acc[i][j], 0, 0, 0);
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

template <int GS, bool ZP, bool HAS_S>
static hipError_t w4a16_dispatch(const uint16_t* A, int64_t M, int64_t N, int64_t K,
                                 const uint32_t* qweight, const uint16_t* scales16,
                                 const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                                 hipStream_t stream) {
  const unsigned blocks = (unsigned)((N + kRows - 1) / kRows);
  const size_t tables = (size_t)(K / GS) * kRows * (ZP ? 6 : 4) + 16;   // steps, zeros, trash
  // The tiled kernel above 64 batch rows, and from 49 on for tall weights: each skinny
  // workgroup reads all of A, which at N = 11008 costs more than the tiles' unpacking (measured
  // at M = 64: 49.5 against 39.8 us; equal near M = 48; at N = 4096 the skinny kernel wins
  // throughout, 19.7 against ~36 us at M = 64).
  if (M > 64 || (M > 48 && N >= 8192)) {
    const int64_t tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
    const int64_t dyn = w4a16_dma_tables(K, GS, ZP);
    // (three stages, loads two steps ahead, measured slower: the loop is bound by LDS traffic,
    // not by load latency)
    if (kDmaSmem + dyn <= 160 * 1024) {
      w4a16_tiled_dma_kernel<GS, ZP, HAS_S><<<(unsigned)tiles, 256, (size_t)dyn, stream>>>(
          A, M, N, K, qweight, scales16, zeros, s16, Y);
    } else {   // groups of 64 with zero points and K > 8192: the tables would not fit
      w4a16_tiled_kernel<GS, ZP, HAS_S><<<(unsigned)tiles, 256, 0, stream>>>(
          A, M, N, K, qweight, scales16, zeros, s16, Y);
    }
    return hipGetLastError();
  }
  auto region0 = [&](size_t table, int MB) {
    const size_t red = (size_t)w4a16_red_bytes(MB);
    return table > red ? table : red;
  };
  hipError_t e = hipSuccess;
  for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += 64) {
    const int64_t rest = M - m0;
    // one chunk of channels and one step entry per thread at most: the SR > 0 instances
    const bool small = K / 8 <= kThreads;   // then the steps take at most 2 loads per thread
    if (rest <= 16 && (size_t)rest * K * 2 <= kActLdsBytes) {
      const size_t lds = region0((size_t)rest * K * 2, 1) + tables;
      if (small && rest == 1)
        w4a16_kernel<1, true, GS, ZP, HAS_S, 1><<<blocks, kThreads, lds, stream>>>(
            A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
      else if (small && rest <= 4)
        w4a16_kernel<1, true, GS, ZP, HAS_S, 4><<<blocks, kThreads, lds, stream>>>(
            A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
      else
        w4a16_kernel<1, true, GS, ZP, HAS_S, 0><<<blocks, kThreads, lds, stream>>>(
            A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
    } else if (rest <= 16) {
      const size_t lds = region0((size_t)K * 2, 1) + tables;
      if (small)
        w4a16_kernel<1, false, GS, ZP, HAS_S, 1><<<blocks, kThreads, lds, stream>>>(
            A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
      else
        w4a16_kernel<1, false, GS, ZP, HAS_S, 0><<<blocks, kThreads, lds, stream>>>(
            A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
    } else if (rest <= 32) {
      w4a16_kernel<2, false, GS, ZP, HAS_S, 0><<<blocks, kThreads,
                                                  region0((size_t)K * 2, 2) + tables, stream>>>(
          A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
    } else {
      w4a16_kernel<4, false, GS, ZP, HAS_S, 0><<<blocks, kThreads,
                                                  region0((size_t)K * 2, 4) + tables, stream>>>(
          A, M, N, K, qweight, scales16, zeros, s16, Y, m0);
    }
    e = hipGetLastError();
  }
  return e;
}

template <int GS, bool ZP>
static hipError_t w4a16_dispatch_s(const uint16_t* A, int64_t M, int64_t N, int64_t K,
                                   const uint32_t* qweight, const uint16_t* scales16,
                                   const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                                   hipStream_t stream) {
  return s16 ? w4a16_dispatch<GS, ZP, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream)
             : w4a16_dispatch<GS, ZP, false>(A, M, N, K, qweight, scales16, zeros, s16, Y,
                                             stream);
}

hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                        const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                        const uint16_t* s16, uint16_t* Y, hipStream_t stream) {
  if (K > kMaxK) return hipErrorInvalidValue;
  if (group == 64)
    return zeros ? w4a16_dispatch_s<64, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream)
                 : w4a16_dispatch_s<64, false>(A, M, N, K, qweight, scales16, zeros, s16, Y,
                                               stream);
  return zeros ? w4a16_dispatch_s<128, true>(A, M, N, K, qweight, scales16, zeros, s16, Y, stream)
               : w4a16_dispatch_s<128, false>(A, M, N, K, qweight, scales16, zeros, s16, Y,
                                              stream);
}

}  // namespace awq
