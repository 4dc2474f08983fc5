// Internal launchers of the AWQ kernels (C++ linkage, not part of the public ABI).
// Every launcher only enqueues work on `stream`; argument checking happens in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

// ---- activation statistics ----
constexpr int kStatsRowsPerChunk = 256;
int64_t stats_chunks(int64_t M);
hipError_t launch_stats(const void* X, int dtype, int64_t M, int64_t K, int64_t ldx, float* sx,
                        uint32_t* flags, double* partials, hipStream_t stream);

// ---- search ----
constexpr int kLossBM = 256;
constexpr int kLossBN = 256;
constexpr int kLossBK = 32;

struct SearchCtrl {        // lives at the start of the search workspace
  uint32_t absmax_bits;    // max |W| as fp32 bits (atomicMax on non-negative floats)
  uint32_t done;           // grid points whose loss is final (finalize's completion count)
};

hipError_t launch_search_prep(const float* sx, int K, int n_grid, float s_floor, float* S,
                              SearchCtrl* ctrl, hipStream_t stream);
hipError_t launch_absmax(const void* W, int dtype, int64_t count, SearchCtrl* ctrl,
                         uint32_t* flags, hipStream_t stream);
hipError_t launch_x_to_f16(const void* X, int dtype, int64_t count, uint16_t* X16,
                           uint32_t* flags, hipStream_t stream);
hipError_t launch_quantize_stack(const void* W, int dtype, int64_t N, int64_t K, const float* S,
                                 int n_grid, int bits, const SearchCtrl* ctrl, uint16_t* Estack,
                                 uint32_t* flags, hipStream_t stream);
hipError_t launch_lossgemm(const uint16_t* X16, int64_t M, int64_t K, const uint16_t* Estack,
                           int64_t N, int n_grid, double* partials, hipStream_t stream);
hipError_t launch_finalize(const double* partials, int64_t tiles_per_alpha, int n_grid,
                           int64_t M, int64_t N, int64_t K, const float* S,
                           SearchCtrl* ctrl, double* losses, int32_t* best,
                           float* s_best, uint32_t* flags, hipStream_t stream);

// ---- pack ----
hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s, int bits,
                       uint32_t* qweight, uint16_t* scales16, uint16_t* s16, int8_t* codes,
                       uint32_t* flags, hipStream_t stream);

// ---- W4A16 ----
hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K,
                        const uint32_t* qweight, const uint16_t* scales16, const uint16_t* s16,
                        uint16_t* Y, hipStream_t stream);

}  // namespace awq
