// W4A16 for one or two activation rows (decode): QuantLinear.forward of "AWQ 量化方案..."
// (qwbw.cn/news/39982), section 三 -- scale the input per channel, dequantize, linear:
//   Y[m, n] = sum_k (A[m, k] / s[k]) * c(q[n,k]) * step[n, k/G],
// c(q) = q for symmetric codes, q - z[n, k/G] for zero-point ones. The activation is divided by
// s because the weight was multiplied by s (AWQ notes, bg51717.github.io/14592, section 方法).
//
// The bytes of the packed weight are all that matters at this size, so the kernel is a streaming
// read with as little arithmetic per code as possible:
//   * a' = A / s is formed once per workgroup in fp32 and stored in LDS as fp16 scaled by a power
//     of two per 128-channel block, a'' = fp16(a' 2^-e), with 2^-e max|a'| in [2^14, 2^15): no
//     value of A or s can overflow it (a dead channel's s_floor gives a huge 1/s, which fp16 1/s
//     or fp16 A/s cannot hold);
//   * the activation and s loads are issued first, the code loads right after them, so the
//     table is built while the codes stream in;
//   * a workgroup of 8 waves owns 16 weight rows, a wave 2 rows and all of K (more waves per CU
//     to hide the latency of their loads: 4 waves of 4 rows were 12-15% slower, 16 waves of one
//     row slower still); lane l takes the 32-channel chunks l, l + 64, ... of each row (16 bytes
//     of codes per row and chunk); a chunk of a'' read from LDS serves both rows;
//   * decoding: each word of 8 codes gives the exact fp16 pairs (c(q_j), c(q_{j+4})) in one
//     shift, four mask-and-xor and four packed fp16 operations (unpack_word8); v_dot2_f32_f16
//     against the a'' pair (j, j + 4) adds both exact products in fp32. (Summing (1024 + u) a''
//     and subtracting the offset times the chunk's sum afterwards would save the packed
//     operation but lose everything else in the block to the rounding of one huge term: a dead
//     channel's a'' next to q = 0.) The chunk's sum times step 2^e goes into the row's partial;
//   * with two activation rows each has its own a'' table and the decoded code pairs serve both;
//   * the two rows' partials are summed over the wave's 64 lanes by a transposing butterfly
//     (the first exchange halves the values a lane holds), in a fixed order.
// Rounding: a'' one fp16 rounding (of the fp32 a' = A rcp(s)); products exact, sums fp32; Y
// rounded once to fp16.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {
constexpr int kGvPos = 2;      // chunk positions per lane whose loads are in flight together
constexpr int kChunkBytes = 80;   // LDS bytes per 32-channel chunk: 64 of a'', 16 of padding
}  // namespace

// LDS bytes of one activation row's table: K/32 chunks, then the K/128 block factors 2^-e
// (fp32), rounded up to 16 bytes; MB rows' tables follow one another.
__host__ __device__ static inline size_t gemv_table_bytes(int64_t K) {
  return ((size_t)(K / 32) * kChunkBytes + (size_t)(K / 128) * sizeof(float) + 15) & ~(size_t)15;
}
size_t w4a16_gemv_lds_bytes(int MB, int64_t K) { return (size_t)MB * gemv_table_bytes(K); }

// ONE: every chunk position of a lane fits one load batch (K <= 64 * 32 * kGvPos = 4096), so
// there is one set of load registers and no loop. TI: table entries of 8 channels per thread
// (K <= 4096 TI); all their loads are unconditional, issued before the code loads, and only the
// LDS stores are conditional -- a load inside a conditional block would be issued there, after
// the code loads, and waiting for it would wait for all of them.
// RW weight rows per wave, NW waves per workgroup, MB activation rows (M <= MB; rows past M
// read row M - 1 and are not stored): one a'' table per activation row, the codes decoded once
// for all of them.
template <int GS, bool ZP, bool HAS_S, bool ONE, int TI, int RW, int NW, int MB>
__global__ __launch_bounds__(64 * NW) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t N, int64_t K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales16,
    const uint8_t* __restrict__ zeros, const uint16_t* __restrict__ s16,
    uint16_t* __restrict__ Y) {
  constexpr int kGvRows = RW, kGvWaves = NW, kGvThreads = 64 * NW;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const size_t tbytes = gemv_table_bytes(K);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = ((int64_t)blockIdx.x * kGvWaves + wave) * kGvRows;
  const int nch = (int)(K / 32);                 // 32-channel chunks of a row
  const int64_t ngr = K / GS;                    // quantization groups of a row
  const int64_t wpr = K / 8;                     // uint32 words of a row
  const int npos = (nch + 63) / 64;              // chunk positions of a lane (the last partial)
  // table of activation row m: lds + m tbytes; its block factors [K/128] 2^-e after the chunks
  auto bfac = [&](int m) {
    return reinterpret_cast<float*>(lds + m * tbytes + (size_t)nch * kChunkBytes);
  };

  // ---- 1. activation and s loads of this thread's table entries (8 channels each) ----------
  uint4 araw[MB][TI], sraw[TI];
  const int nq8 = (int)(K / 8);
#pragma unroll
  for (int it = 0; it < TI; ++it) {
    const int q8 = tid + kGvThreads * it;
    const int qc = q8 < nq8 ? q8 : 0;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int64_t mr = (m < M) ? m : M - 1;
      araw[m][it] = *reinterpret_cast<const uint4*>(A + mr * K + (int64_t)qc * 8);
    }
    sraw[it] = HAS_S ? *reinterpret_cast<const uint4*>(s16 + (int64_t)qc * 8)
                     : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  }

  // ---- 2. this wave's code loads (rows past N read row N - 1, never stored) ----------------
  const uint32_t* wrow[kGvRows];
  int64_t srow[kGvRows];
#pragma unroll
  for (int r = 0; r < kGvRows; ++r) {
    const int64_t n = (n0 + r < N) ? n0 + r : N - 1;
    wrow[r] = qweight + n * wpr;
    srow[r] = n * ngr;
  }
  // codes, steps and zero points of positions p0 .. p0 + kGvPos - 1 (a chunk past the row reads
  // chunk 0: its step is zeroed at use, so it adds nothing)
  struct Buf {
    uint4 w[kGvPos][kGvRows];
    uint32_t st[kGvPos][kGvRows];   // fp16 step bits (32-bit registers: no merged halves)
    uint32_t z[kGvPos][kGvRows];    // zero points (ZP)
  };
  auto load = [&](int p0, Buf& buf) {
#pragma unroll
    for (int j = 0; j < kGvPos; ++j) {
      const int c = lane + 64 * (p0 + j);
      const int cc = c < nch ? c : 0;
      const int64_t g = ((int64_t)cc * 32) / GS;
#pragma unroll
      for (int r = 0; r < kGvRows; ++r) {
        buf.w[j][r] = *reinterpret_cast<const uint4*>(wrow[r] + 4 * cc);
        buf.st[j][r] = scales16[srow[r] + g];
        if (ZP) buf.z[j][r] = zeros[srow[r] + g];
      }
    }
  };
  Buf wb[ONE ? 1 : 2];
  load(0, wb[0]);
  asm volatile("" : : "v"(wrow[0]) : "memory");   // the code loads stay ahead of the table
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. the a'' tables: 16 consecutive threads hold one 128-channel block ----------------
#pragma unroll
  for (int it = 0; it < TI; ++it) {
    const int q8 = tid + kGvThreads * it;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const uint32_t aw[4] = {araw[m][it].x, araw[m][it].y, araw[m][it].z, araw[m][it].w};
      const uint32_t sw[4] = {sraw[it].x, sraw[it].y, sraw[it].z, sraw[it].w};
      float v[8];
      float mx = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float a = h2f((uint16_t)(aw[t >> 1] >> (16 * (t & 1))));
        const float sv = h2f((uint16_t)(sw[t >> 1] >> (16 * (t & 1))));
        v[t] = a * __builtin_amdgcn_rcpf(sv);
        mx = fmaxf(mx, fabsf(v[t]));
      }
      mx = group_absmax<16>(mx);                  // the 128-channel block of this thread
      const int e = escale_for_max(mx);           // 2^e mx in [2^14, 2^15); 0 for 0 or Inf/NaN
      const float sc = ldexpf(1.0f, e);
      uint16_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) h[t] = f2h(v[t] * sc);
      // pairs in the decode order (t, t + 4)
      const uint32_t p0 = (uint32_t)h[0] | ((uint32_t)h[4] << 16);
      const uint32_t p1 = (uint32_t)h[1] | ((uint32_t)h[5] << 16);
      const uint32_t p2 = (uint32_t)h[2] | ((uint32_t)h[6] << 16);
      const uint32_t p3 = (uint32_t)h[3] | ((uint32_t)h[7] << 16);
      if (q8 < nq8) {
        char* d = lds + m * tbytes + (size_t)(q8 >> 2) * kChunkBytes + (q8 & 3) * 16;
        *reinterpret_cast<uint4*>(d) = make_uint4(p0, p1, p2, p3);
        if ((q8 & 15) == 0) bfac(m)[q8 >> 4] = ldexpf(1.0f, -e);
      }
    }
  }
  __syncthreads();

  float part[kGvRows][MB];
#pragma unroll
  for (int r = 0; r < kGvRows; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) part[r][m] = 0.0f;

  auto process = [&](int p0, const Buf& buf) {
#pragma unroll
    for (int j = 0; j < kGvPos; ++j) {
      const int c = lane + 64 * (p0 + j);
      const bool ok = c < nch;
      const int cc = ok ? c : 0;
      float f[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) f[m] = ok ? bfac(m)[cc >> 2] : 0.0f;   // 2^-e of the block
      half2_t sub_lo[kGvRows], sub_hi[kGvRows];
#pragma unroll
      for (int r = 0; r < kGvRows; ++r) {
        // fp16 subtrahends of the unpack: zc = 8 (signed codes, biased by the flip) or z
        const float zc = ZP ? (float)buf.z[j][r] : 8.0f;
        const _Float16 slo = (_Float16)(1024.0f + zc), shi = (_Float16)(-64.0f - zc);
        sub_lo[r] = half2_t{slo, slo};
        sub_hi[r] = half2_t{shi, shi};
      }
      float acc0[kGvRows][MB], acc1[kGvRows][MB];
#pragma unroll
      for (int r = 0; r < kGvRows; ++r)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc0[r][m] = acc1[r][m] = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {               // word v: channels 8v .. 8v + 7 of the chunk
        uint4 a4[MB];                             // the a'' pairs (t, t + 4) of those channels
#pragma unroll
        for (int m = 0; m < MB; ++m)
          a4[m] = *reinterpret_cast<const uint4*>(lds + m * tbytes + (size_t)cc * kChunkBytes +
                                                  16 * v);
#pragma unroll
        for (int r = 0; r < kGvRows; ++r) {
          const uint32_t wv = v == 0 ? buf.w[j][r].x : v == 1 ? buf.w[j][r].y
                            : v == 2 ? buf.w[j][r].z : buf.w[j][r].w;
          half2_t qp[4];
          unpack_word8<ZP>(wv, sub_lo[r], sub_hi[r], qp);
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const uint32_t ap[4] = {a4[m].x, a4[m].y, a4[m].z, a4[m].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const half2_t apair = __builtin_bit_cast(half2_t, ap[jj]);
              if (jj & 1)
                acc1[r][m] = __builtin_amdgcn_fdot2(qp[jj], apair, acc1[r][m], false);
              else
                acc0[r][m] = __builtin_amdgcn_fdot2(qp[jj], apair, acc0[r][m], false);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kGvRows; ++r) {
        const float st = h2f((uint16_t)buf.st[j][r]);
#pragma unroll
        for (int m = 0; m < MB; ++m)
          part[r][m] = __builtin_fmaf(st * f[m], acc0[r][m] + acc1[r][m], part[r][m]);
      }
    }
  };

  if constexpr (ONE) {
    process(0, wb[0]);
  } else {
    // positions in pairs, the loads of the next pair in flight while one pair is processed
    for (int p = 0; p < npos; p += 2 * kGvPos) {
      if (p + kGvPos < npos) load(p + kGvPos, wb[ONE ? 0 : 1]);
      process(p, wb[0]);
      if (p + kGvPos < npos) {
        if (p + 2 * kGvPos < npos) load(p + 2 * kGvPos, wb[0]);
        process(p + kGvPos, wb[ONE ? 0 : 1]);
      }
    }
  }

  // ---- sums over the 64 lanes: log2(RW) transposing exchanges (lanes with the exchange's lane
  // bit set keep the upper half of their rows and send the lower half, the others the reverse),
  // then the plain butterfly over the lanes below the last exchanged bit; a fixed order ---------
  static_assert(kGvRows == 1 || kGvRows == 2 || kGvRows == 4, "one, two or four rows per wave");
  constexpr int kLastMask = (kGvRows == 4) ? 16 : (kGvRows == 2) ? 32 : 64;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    float v[kGvRows];
#pragma unroll
    for (int r = 0; r < kGvRows; ++r) v[r] = part[r][m];
    int row = 0;
#pragma unroll
    for (int n = kGvRows, mask = 32; n > 1; n >>= 1, mask >>= 1) {
      const bool hi = (lane & mask) != 0;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float keep = hi ? v[n / 2 + i] : v[i];
        const float give = hi ? v[i] : v[n / 2 + i];
        v[i] = keep + __shfl_xor(give, mask);
      }
      if (hi) row += n / 2;
    }
    float kk = v[0];
#pragma unroll
    for (int mk = kLastMask / 2; mk >= 1; mk >>= 1) kk += __shfl_xor(kk, mk);
    if ((lane & (kLastMask - 1)) == 0 && n0 + row < N && m < M) Y[m * N + n0 + row] = f2h(kk);
  }
}

// Two activation rows share the decoded codes with K <= 28672, where their two tables (145 KiB)
// still fit the LDS (4096 x 4096: 5.7 against 5.9 us in the small-batch MFMA kernel, 11008 x
// 4096: 10.2 against 11.3, 8192 x 8192: 13.1 against 15.8, 4096 x 11008: 11.0 against 14.1,
// 1024 x 16384: 11.0 against 16.0, 8192 x 28672: 43 against 50); four rows took 185 VGPRs and
// were slower than that kernel (4096 x 4096: 7.0 against 5.9 us).
bool w4a16_gemv_fits(int64_t M, int64_t K) {
  return (M == 1 && K <= kW4a16GemvMaxK) || (M == 2 && K <= 28672);
}

hipError_t launch_w4a16_gemv(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                             const uint32_t* qweight, const uint16_t* scales16,
                             const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                             hipStream_t stream) {
  if (!w4a16_gemv_fits(M, K)) return hipErrorInvalidValue;
  constexpr int RW = 2, NW = 8;
  constexpr int kGvThreads = 64 * NW;
  static_assert(kW4a16GemvMaxK <= 64 * kGvThreads, "table entries per thread: at most 8");
  const int mb = (int)M;
  const unsigned blocks = (unsigned)((N + RW * NW - 1) / (RW * NW));
  const size_t lds = w4a16_gemv_lds_bytes(mb, K);
  const bool one = K <= 64 * 32 * kGvPos;   // K <= 4096: one table entry per thread, one batch
#define AWQ_GV1(GS_, ZP_, HS_, ONE_, TI_, MB_)                                                   \
  w4a16_gemv_kernel<GS_, ZP_, HS_, ONE_, TI_, RW, NW, MB_><<<blocks, kGvThreads, lds, stream>>>( \
      A, M, N, K, qweight, scales16, zeros, s16, Y)
#define AWQ_GV(GS_, ZP_, HS_)                                                                    \
  do {                                                                                           \
    if (mb == 2 && one) AWQ_GV1(GS_, ZP_, HS_, true, 1, 2);                                      \
    else if (mb == 2 && K <= 8192) AWQ_GV1(GS_, ZP_, HS_, false, 2, 2);                          \
    else if (mb == 2 && K <= 16384) AWQ_GV1(GS_, ZP_, HS_, false, 4, 2);                         \
    else if (mb == 2) AWQ_GV1(GS_, ZP_, HS_, false, 8, 2);                                       \
    else if (one) AWQ_GV1(GS_, ZP_, HS_, true, (4096 / 8 + kGvThreads - 1) / kGvThreads, 1);    \
    else if (K <= 8 * kGvThreads) AWQ_GV1(GS_, ZP_, HS_, false, 1, 1);                          \
    else if (K <= 16 * kGvThreads) AWQ_GV1(GS_, ZP_, HS_, false, 2, 1);                         \
    else if (K <= 32 * kGvThreads) AWQ_GV1(GS_, ZP_, HS_, false, 4, 1);                         \
    else AWQ_GV1(GS_, ZP_, HS_, false, 8, 1);                                                   \
  } while (0)
#define AWQ_GV_S(GS_, ZP_) \
  do { if (s16) AWQ_GV(GS_, ZP_, true); else AWQ_GV(GS_, ZP_, false); } while (0)
#define AWQ_GV_Z(GS_) \
  do { if (zeros) AWQ_GV_S(GS_, true); else AWQ_GV_S(GS_, false); } while (0)
  if (group == 64)
    AWQ_GV_Z(64);
  else
    AWQ_GV_Z(128);
#undef AWQ_GV_Z
#undef AWQ_GV_S
#undef AWQ_GV
#undef AWQ_GV1
  return hipGetLastError();
}

}  // namespace awq
