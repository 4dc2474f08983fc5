// W4A16 for small batches (2 to 64 activation rows per pass): QuantLinear.forward of "AWQ
// 量化方案..." (qwbw.cn/news/39982), section 三 -- scale the input per channel, dequantize,
// linear:
//   Y[m, n] = sum_k (A[m,k] / s[k]) * c(q[n,k]) * step[n, k/G],
// c(q) = q (symmetric codes) or q - z[n, k/G] (zero-point codes). The activation is divided by s
// because the weight was multiplied by s (AWQ notes, bg51717.github.io/14592, section 方法).
//
// gfx950 design (the packed weight's bytes dominate; the kernel streams them):
//   * v_mfma_f32_16x16x32_f16 with the weights as the 16-row A operand (rows n) and the
//     activations, read straight from memory, as the B operand (columns m, up to 4 blocks of 16);
//   * a workgroup owns 16 weight rows and all of K; its 8 waves take the 128-channel blocks
//     round-robin, every lane issuing the 16-byte loads of its blocks (up to 4 at a time,
//     double-buffered) before unpacking any of them;
//   * unpacking: one 32-bit word holds the codes of 8 consecutive channels; one shift, four
//     mask-and-xor and four packed fp16 operations turn it into the exact fp16 pairs (q_j,
//     q_{j+4}), j = 0..3 (zero-point codes: q - z), as unpack_word8 describes. The MFMA k slots
//     therefore hold channels in the order 0,4,1,5,2,6,3,7 of each 8, and the activations are
//     permuted the same way;
//   * 1/s enters the weight operand as fp16(q * r_k), r_k = fp16(2^b / s_k) with one power of
//     two 2^b per 128-channel block chosen so that the block's largest r_k lies in [2^10, 2^11):
//     |q r_k| < 2^15, so no s -- not even a dead channel's s_floor -- can overflow fp16 (an
//     fp16 1/s or A/s can). The block's 2^-b and the group step scale the fp32 partial of each
//     group's MFMAs;
//   * the eight waves' partial outputs are added in a fixed order through LDS.
// Rounding: r_k and q r_k are each rounded once to fp16, accumulation is fp32, Y is rounded once
// to fp16.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {
constexpr int kRows = 16;       // weight rows per workgroup
constexpr int kWaves = 8;       // waves per workgroup; wave w takes 128-channel blocks w, w + 8..
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 4;       // blocks whose weight words a lane keeps in flight at once

// permuted position of channel t (0..7) inside its block of 8: order 0,4,1,5,2,6,3,7
__device__ __forceinline__ int perm8(int t) { return ((t & 3) << 1) | (t >> 2); }
}  // namespace

// Bytes of the reduction buffer and of the whole dynamic LDS.
__host__ __device__ constexpr int64_t skinny_red_bytes(int MB) {
  return (int64_t)kWaves * MB * 64 * 16;
}
size_t w4a16_skinny_lds_bytes(int MB, int64_t K, int GS, bool ZP) {
  const int64_t r0 = (K * 2 > skinny_red_bytes(MB)) ? K * 2 : skinny_red_bytes(MB);
  return (size_t)(r0 + (K / 128) * 4 + (K / GS) * kRows * (ZP ? 6 : 4) + 16);
}

// TI: 16-byte chunks of s per thread in the prologue (K <= 4096 TI). Every prologue load is
// unconditional (indices clamped), issued before the weight loads: a load inside a conditional
// block is issued there, and since loads complete in order, waiting for it would mean waiting
// for all the weight loads in flight.
// TI = 1 (K <= 4096): a wave's blocks (at most 4) are one chunk of loads, so there is one load
// buffer and no loop; with MB = 1 these instances fit in 80 VGPRs (6 waves per SIMD), so three
// workgroups fit on a CU and a weight of up to 768 row blocks (12288 rows) runs in one round.
template <int MB, int GS, bool ZP, bool HAS_S, int TI>
__global__ __launch_bounds__(kThreads, (MB == 1 && TI == 1) ? 6 : 1) void w4a16_skinny_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t N, int64_t K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales16,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ s16,
    uint16_t* __restrict__ Y, int64_t m0) {
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  // LDS: r = fp16(2^b / s) [K] (permuted pairs; the reduction buffer reuses it after the main
  // loop) | 2^-b fp32 [K/128] | steps fp32 [K/GS][16] | (ZP) fp16(1024 + z) [K/GS][16] | 16 B
  // trash slot for the stores of clamped entries
  const int64_t region0 = (K * 2 > skinny_red_bytes(MB)) ? K * 2 : skinny_red_bytes(MB);
  const int64_t nblk = K / 128;
  const int64_t ngr = K / GS;
  uint16_t* rtab = reinterpret_cast<uint16_t*>(dyn);
  floatx4* red = reinterpret_cast<floatx4*>(dyn);
  float* bfac = reinterpret_cast<float*>(dyn + region0);
  float* step_lds = reinterpret_cast<float*>(dyn + region0 + nblk * 4);
  uint16_t* zero_lds = reinterpret_cast<uint16_t*>(dyn + region0 + nblk * 4 + ngr * kRows * 4);
  char* trash = dyn + region0 + nblk * 4 + ngr * kRows * (ZP ? 6 : 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;   // weight row of the A operand / activation column of the B operand
  const int lg = lane >> 4;   // which 32-channel quarter of a 128-channel block
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int gr = (int)nblk;
  const int kc = (int)(K / 8);                                  // 16-byte chunks of a row
  const int64_t words_per_row = K / 8;

  // ---- 1. s loads (TI per thread) and step / zero-point loads ---------------------------------
  uint4 ts[TI];
#pragma unroll
  for (int it = 0; it < TI; ++it) {
    const int e = tid + it * kThreads;
    const int ec = e < kc ? e : 0;
    ts[it] = HAS_S ? *reinterpret_cast<const uint4*>(s16 + (int64_t)ec * 8)
                   : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  }
  constexpr int kStepIters = (TI * kThreads * 8 / GS * kRows + kThreads - 1) / kThreads;
  const int ng = (int)ngr;
  uint32_t sraw[kStepIters], zraw[kStepIters];   // 32-bit registers: no merged 16-bit halves
#pragma unroll
  for (int it = 0; it < kStepIters; ++it) {
    const int e = tid + it * kThreads;
    const int ec = e < ng * kRows ? e : 0;
    const int64_t row = (n0 + (ec & (kRows - 1)) < N) ? n0 + (ec & (kRows - 1)) : N - 1;
    sraw[it] = scales16[row * ngr + (ec >> 4)];
    zraw[it] = ZP ? zeros[row * ngr + (ec >> 4)] : 0u;
  }
  __builtin_amdgcn_sched_barrier(0);   // keep the issue order: tables, steps, then weights

  // ---- 2. this wave's weight words (first chunk) ----------------------------------------------
  const int64_t n = n0 + li;
  const bool nok = n < N;
  const uint4* wrow = reinterpret_cast<const uint4*>(qweight + (nok ? n : N - 1) * words_per_row) + lg;
  const int my_blocks = (gr - wave + kWaves - 1) / kWaves;     // g = wave + kWaves i
  uint4 wbuf[TI == 1 ? 1 : 2][kChunk];
  auto load_chunk = [&](int c, uint4 (&dst)[kChunk]) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = c * kChunk + u;
      const int gi = (i < my_blocks) ? wave + kWaves * i : wave;
      dst[u] = wrow[(int64_t)gi * 4];      // rows >= N: a valid row whose results are dropped
    }
  };
  load_chunk(0, wbuf[0]);
  // an empty asm that may read or write the weight rows: no weight load above may be moved
  // below it. It names only the row pointer, not the loaded values, so it adds no wait.
  asm volatile("" : : "v"(wrow) : "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. tables: r = fp16(2^b / s) per channel, 2^-b per 128-channel block (its 16 chunks
  // are 16 consecutive threads: one DPP row), steps and zero points --------------------------
#pragma unroll
  for (int it = 0; it < TI; ++it) {
    const int e = tid + it * kThreads;
    const uint32_t sw[4] = {ts[it].x, ts[it].y, ts[it].z, ts[it].w};
    float inv[8];
    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      inv[t] = __builtin_amdgcn_rcpf(h2f((uint16_t)(sw[t >> 1] >> (16 * (t & 1)))));
      mx = fmaxf(mx, inv[t]);
    }
    mx = group_absmax<16>(mx);
    const int b = escale_for_max(mx) - 4;      // 2^b mx in [2^10, 2^11)
    const float sc = ldexpf(1.0f, b);
    uint16_t h[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) h[perm8(t)] = f2h(inv[t] * sc);
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) w[p] = (uint32_t)h[2 * p] | ((uint32_t)h[2 * p + 1] << 16);
    const bool ok = e < kc;
    *reinterpret_cast<uint4*>(ok ? reinterpret_cast<char*>(rtab + e * 8) : trash) =
        make_uint4(w[0], w[1], w[2], w[3]);
    if ((e & 15) == 0) *reinterpret_cast<float*>(ok ? reinterpret_cast<char*>(bfac + (e >> 4)) : trash) =
        ldexpf(1.0f, -b);
  }
#pragma unroll
  for (int it = 0; it < kStepIters; ++it) {
    const int e = tid + it * kThreads;
    const bool ok = e < ng * kRows;
    const float stv = (n0 + (e & (kRows - 1)) < N) ? h2f((uint16_t)sraw[it]) : 0.0f;
    *reinterpret_cast<float*>(ok ? reinterpret_cast<char*>(step_lds + e) : trash) = stv;
    if (ZP)
      *reinterpret_cast<uint16_t*>(ok ? reinterpret_cast<char*>(zero_lds + e) : trash) =
          f2h(1024.0f + (float)zraw[it]);   // exact: the subtrahend of the unpack
  }
  __syncthreads();

  floatx4 acc[MB];
#pragma unroll
  for (int bb = 0; bb < MB; ++bb) acc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const uint4 (&cur)[kChunk], int c) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = c * kChunk + u;
      if (i >= my_blocks) break;                            // uniform over the wave
      const int64_t g = wave + kWaves * i;                  // 128-channel block
      const int64_t kbase = g * 128 + lg * 32;              // this lane's 32 channels
      const uint32_t words[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
      // fp16 subtrahends of the unpack: zc = 8 (signed codes, biased by the flip) or z of this
      // lane's row and group (the lane's 32 channels lie in one group for GS = 64 too)
      _Float16 slo = (_Float16)1032.0f, shi = (_Float16)-72.0f;
      if (ZP) {
        const int64_t gz = (GS == 64) ? 2 * g + (lg >> 1) : g;
        slo = __builtin_bit_cast(_Float16, zero_lds[gz * kRows + li]);
        shi = (_Float16)960.0f - slo;   // -(64 + z), exact
      }
      const half2_t sub_lo = half2_t{slo, slo}, sub_hi = half2_t{shi, shi};
      half8_t wf[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {                          // word v: channels kbase + 8v ..
        const uint4 rv = HAS_S ? *reinterpret_cast<const uint4*>(rtab + kbase + 8 * v)
                               : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
        half2_t d[4];
        unpack_word8<ZP>(words[v], sub_lo, sub_hi, d);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // without s the operand is c(q) itself (exact) and no block scale applies
          const half2_t q = HAS_S ? d[j] * __builtin_bit_cast(half2_t, rw[j]) : d[j];
          wf[v][2 * j] = q[0];
          wf[v][2 * j + 1] = q[1];
        }
      }
      // per-group fp32 steps of this lane's 4 output rows (rows 4 lg + r) times the block's
      // 2^-b; with GS = 64 the two halves of the block have their own steps, so each MFMA is
      // done twice with the A operand of the other half's lanes (lg < 2 hold channels 0..63,
      // lg >= 2 channels 64..127) zeroed
      const float bs = HAS_S ? bfac[g] : 1.0f;
      const int64_t gs0 = (GS == 64) ? 2 * g : g;
      floatx4 st0 = *reinterpret_cast<const floatx4*>(step_lds + gs0 * kRows + 4 * lg);
      floatx4 st1 = st0;
      if (GS == 64) st1 = *reinterpret_cast<const floatx4*>(step_lds + (gs0 + 1) * kRows + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st0[r] *= bs;
        st1[r] *= bs;
      }
#pragma unroll
      for (int bb = 0; bb < MB; ++bb) {
        const int64_t m = m0 + bb * 16 + li;
        floatx4 part = {0.f, 0.f, 0.f, 0.f}, part1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // Batch rows past M read row M - 1 (a valid row): column m of the MFMA result depends
          // on activation row m only, and columns m >= M are never stored.
          const int64_t mc = (m < M) ? m : M - 1;
          const uint4 a = *reinterpret_cast<const uint4*>(A + mc * K + kbase + 8 * v);
          // permute channels 0..7 to the order 0,4,1,5,2,6,3,7 of the weight operand
          const uint32_t p0 = __builtin_amdgcn_perm(a.z, a.x, 0x05040100u);  // (a0, a4)
          const uint32_t p1 = __builtin_amdgcn_perm(a.z, a.x, 0x07060302u);  // (a1, a5)
          const uint32_t p2 = __builtin_amdgcn_perm(a.w, a.y, 0x05040100u);  // (a2, a6)
          const uint32_t p3 = __builtin_amdgcn_perm(a.w, a.y, 0x07060302u);  // (a3, a7)
          const half8_t af = __builtin_bit_cast(half8_t, make_uint4(p0, p1, p2, p3));
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
          acc[bb][r] = __builtin_fmaf(part[r], st0[r], acc[bb][r]);
          if (GS == 64) acc[bb][r] = __builtin_fmaf(part1[r], st1[r], acc[bb][r]);
        }
      }
    }
  };

  if constexpr (TI == 1) {
    process(wbuf[0], 0);
  } else {
    // chunks alternate between the two register buffers (static indices: no scratch)
    const int nchunks = (my_blocks + kChunk - 1) / kChunk;
    for (int c = 0; c < nchunks; c += 2) {
      if (c + 1 < nchunks) load_chunk(c + 1, wbuf[TI == 1 ? 0 : 1]);
      process(wbuf[0], c);
      if (c + 1 < nchunks) {
        if (c + 2 < nchunks) load_chunk(c + 2, wbuf[0]);
        process(wbuf[TI == 1 ? 0 : 1], c + 1);
      }
    }
  }

  __syncthreads();   // the reduction buffer reuses the table's LDS: every wave is done with it
#pragma unroll
  for (int bb = 0; bb < MB; ++bb) red[(wave * MB + bb) * 64 + lane] = acc[bb];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int bb = 0; bb < MB; ++bb) {
      floatx4 t = red[bb * 64 + lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const floatx4 o = red[(w * MB + bb) * 64 + lane];
        t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
      }
      // D layout of the 16x16 MFMA: lane holds D[4*(lane/16) + r][lane % 16], r = 0..3,
      // i.e. weight rows 4*lg + r and activation column li.
      const int64_t m = m0 + bb * 16 + li;
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

hipError_t launch_w4a16_skinny(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                               const uint32_t* qweight, const uint16_t* scales16,
                               const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                               hipStream_t stream) {
  if (K > kW4a16SkinnyMaxK) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((N + kRows - 1) / kRows);
  const bool zp = zeros != nullptr;
  hipError_t e = hipSuccess;
  for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += 64) {
    const int64_t rest = M - m0;
    const int MB = rest <= 16 ? 1 : (rest <= 32 ? 2 : 4);
    const size_t lds = w4a16_skinny_lds_bytes(MB, K, group, zp);
#define AWQ_SK(MB_, GS_, ZP_, HS_, TI_)                                                          \
  w4a16_skinny_kernel<MB_, GS_, ZP_, HS_, TI_><<<blocks, kThreads, lds, stream>>>(              \
      A, M, N, K, qweight, scales16, zeros, s16, Y, m0)
#define AWQ_SK_TI(MB_, GS_, ZP_, HS_)                                                            \
  do {                                                                                           \
    if (K <= 4096) AWQ_SK(MB_, GS_, ZP_, HS_, 1);                                               \
    else if (K <= 8192) AWQ_SK(MB_, GS_, ZP_, HS_, 2);                                          \
    else if (K <= 16384) AWQ_SK(MB_, GS_, ZP_, HS_, 4);                                         \
    else AWQ_SK(MB_, GS_, ZP_, HS_, 8);                                                         \
  } while (0)
#define AWQ_SK_S(MB_, GS_, ZP_) \
  do { if (s16) AWQ_SK_TI(MB_, GS_, ZP_, true); else AWQ_SK_TI(MB_, GS_, ZP_, false); } while (0)
#define AWQ_SK_Z(MB_, GS_) \
  do { if (zp) AWQ_SK_S(MB_, GS_, true); else AWQ_SK_S(MB_, GS_, false); } while (0)
#define AWQ_SK_G(MB_) \
  do { if (group == 64) AWQ_SK_Z(MB_, 64); else AWQ_SK_Z(MB_, 128); } while (0)
    if (MB == 1)
      AWQ_SK_G(1);
    else if (MB == 2)
      AWQ_SK_G(2);
    else
      AWQ_SK_G(4);
#undef AWQ_SK_G
#undef AWQ_SK_Z
#undef AWQ_SK_S
#undef AWQ_SK_TI
#undef AWQ_SK
    e = hipGetLastError();
  }
  return e;
}

}  // namespace awq
