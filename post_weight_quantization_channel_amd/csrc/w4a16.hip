// W4A16 GEMM on the packed AWQ artefacts: QuantLinear.forward of "AWQ 量化方案..."
// (qwbw.cn/news/39982), section 三 -- scale the input per channel, dequantize the packed codes
// with the per-group steps, then a linear layer:
//   Y[m, n] = sum_k (A[m,k] / s[k]) * q[n,k] * step[n, k/128]
// The activation is divided by s because the weight was multiplied by s (AWQ notes,
// bg51717.github.io/14592, section 方法: Q(w s) x / s).
//
// gfx950 design: v_mfma_f32_16x16x32_f16 with the weights as the 16-row A operand (rows n) and
// the activations as the B operand (columns m). A workgroup owns 16 weight rows and all of K;
// its 4 waves take the 128-channel groups round-robin (split K), so each lane issues one
// 16-byte load per group (4 words = 32 codes of one row; 16 lanes x 4 cover 16 rows), the
// nibbles are unpacked in registers (never materialised in memory), and the four waves' partial
// outputs are added in a fixed order through LDS. Per group and row the step is one fp16
// value; code * step and activation / s are each rounded once to fp16 for the MFMA; the
// accumulation is fp32 and Y is rounded once to fp16.
#include "device_common.h"
#include "kernels.h"

namespace awq {

namespace {
constexpr int kRows = 16;       // weight rows per workgroup
constexpr int kMB = 4;          // 16-column activation blocks per pass (M <= 64 per pass)
}  // namespace

__global__ __launch_bounds__(256) void w4a16_kernel(const uint16_t* __restrict__ A, int64_t M,
                                                    int64_t N, int64_t K,
                                                    const uint32_t* __restrict__ qweight,
                                                    const uint16_t* __restrict__ scales16,
                                                    const uint16_t* __restrict__ s16,
                                                    uint16_t* __restrict__ Y, int64_t m0) {
  __shared__ floatx4 red[4][kMB][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;   // weight row within the 16 (A operand) / activation column (B)
  const int lg = lane >> 4;   // which 32-channel quarter of the 128-channel group
  const int64_t n = (int64_t)blockIdx.x * kRows + li;
  const bool nok = n < N;
  const int64_t groups = K / 128;
  const int64_t words_per_row = K / 8;

  floatx4 acc[kMB];
#pragma unroll
  for (int b = 0; b < kMB; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int64_t g = wave; g < groups; g += 4) {
    // weights: 4 words = codes of k = 128 g + 32 lg + [0, 32)
    uint4 wq = make_uint4(0, 0, 0, 0);
    float sc = 0.0f;
    if (nok) {
      wq = *reinterpret_cast<const uint4*>(qweight + n * words_per_row + g * 16 + lg * 4);
      sc = h2f(scales16[n * groups + g]);
    }
    const uint32_t words[4] = {wq.x, wq.y, wq.z, wq.w};
    half8_t wf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int code = ((int)(words[u] << (28 - 4 * t))) >> 28;
        wf[u][t] = (_Float16)((float)code * sc);
      }
    // 1/s for k = 128 g + 32 lg + 8u + t
    float inv[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float sv[8];
      load8_f32<kF16>(s16 + g * 128 + lg * 32 + u * 8, sv);
#pragma unroll
      for (int t = 0; t < 8; ++t) inv[u][t] = __builtin_amdgcn_rcpf(sv[t]);
    }
#pragma unroll
    for (int b = 0; b < kMB; ++b) {
      const int64_t m = m0 + b * 16 + li;
      if (m0 + b * 16 >= M) break;   // uniform: whole block beyond M
      const bool mok = m < M;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        half8_t af;
        if (mok) {
          float av[8];
          load8_f32<kF16>(A + m * K + g * 128 + lg * 32 + u * 8, av);
#pragma unroll
          for (int t = 0; t < 8; ++t) af[t] = (_Float16)(av[t] * inv[u][t]);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) af[t] = (_Float16)0.0f;
        }
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[u], af, acc[b], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < kMB; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < kMB; ++b) {
      if (m0 + b * 16 >= M) break;
      floatx4 t = red[0][b][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const floatx4 o = red[w][b][lane];
        t[0] += o[0]; t[1] += o[1]; t[2] += o[2]; t[3] += o[3];
      }
      // D layout of the 16x16 MFMA: lane holds D[4*(lane/16) + r][lane % 16], r = 0..3,
      // i.e. weight rows 4*lg + r and activation column li.
      const int64_t m = m0 + b * 16 + li;
      const int64_t nb = (int64_t)blockIdx.x * kRows + 4 * lg;
      if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) Y[m * N + nb + r] = f2h(t[r]);
      }
    }
  }
}

hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K,
                        const uint32_t* qweight, const uint16_t* scales16, const uint16_t* s16,
                        uint16_t* Y, hipStream_t stream) {
  const unsigned blocks = (unsigned)((N + kRows - 1) / kRows);
  for (int64_t m0 = 0; m0 < M; m0 += 16 * kMB) {
    w4a16_kernel<<<blocks, 256, 0, stream>>>(A, M, N, K, qweight, scales16, s16, Y, m0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace awq
