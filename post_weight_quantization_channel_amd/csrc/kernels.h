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
// the second pass of launch_stats on chunk partials [chunks][K] (256 rows per chunk)
hipError_t launch_stats_final(const double* partials, int64_t chunks, int64_t M, int64_t K,
                              int dtype, float* sx, uint32_t* flags, hipStream_t stream);
hipError_t launch_stats(const void* X, int dtype, int64_t M, int64_t K, int64_t ldx, float* sx,
                        uint32_t* flags, double* partials, hipStream_t stream);

// ---- search ----
constexpr int kLossBM = 256;
constexpr int kLossBN = 256;
constexpr int kLossBK = 32;

struct SearchCtrl {        // lives at the start of the search workspace
  uint32_t absmax_bits;    // max |W| as fp32 bits (atomicMax on non-negative floats)
  uint32_t done;           // grid points whose loss is final (finalize's completion count)
  uint32_t gram_k;         // K of the Gram-form operand B in this workspace (0: none)
};

// Gram form (gram.hip): H = X^T X over token chunks, then the lower-triangular operand B.
constexpr int64_t kGramMAlign = 128;     // tokens are padded to this multiple (>= 4 K steps)
constexpr int64_t kGramMaxChunks = 32;
constexpr int64_t kGramMaxBlocks = 4096;
struct GramPlan {
  int t;          // 256-channel blocks, ceil(K / 256)
  int S;          // token chunks
  bool diag;      // only the t diagonal 256 x 256 blocks of X^T X (the clipping search)
  int64_t T;      // tiles: t (t + 1) / 2 upper-triangle tiles, or t diagonal ones
  int64_t Mp;     // padded token count
  int64_t chunk;  // tokens per chunk (multiple of kGramMAlign; the last chunk may be shorter)
};
GramPlan gram_plan(int64_t M, int64_t K, bool diag = false);
// transpose -> ev[0] -> X^T X partials -> ev[1] -> d and B. B is [K, K] (row l, column k), or
// with plan.diag the t diagonal blocks [t][256][256] (block a: rows and columns 256 a ..).
// gram_k: nullptr, or where the finish pass records K (the operand is then complete once the
// stream has passed this call).
// The two halves of launch_gram_prepare. stats: nullptr, or (fp16 X only) [ceil(M/256)][K] fp64
// column sums of |x| per 256 tokens, the chunk partials that launch_stats_final reduces.
hipError_t launch_gram_transpose(const void* X, int xdt, int64_t M, int64_t K, int64_t Mp,
                                 uint16_t* Xt, double* stats, uint32_t* flags,
                                 hipStream_t stream);
// X^T X partials -> ev, ev2 (each if not null) -> d and B
hipError_t launch_gram_hmat(const uint16_t* Xt, int64_t K, const GramPlan& p, float* Hpart,
                            double* d64, float* d32, uint16_t* B, uint32_t* gram_k,
                            hipStream_t stream, hipEvent_t ev, hipEvent_t ev2);
hipError_t launch_gram_prepare(const void* X, int xdt, int64_t M, int64_t K, const GramPlan& p,
                               uint16_t* Xt, float* Hpart, double* d64, float* d32, uint16_t* B,
                               uint32_t* gram_k, uint32_t* flags, hipStream_t stream,
                               hipEvent_t* ev);
hipError_t launch_gram_loss(const uint16_t* Estack, int64_t N, int64_t K, const uint16_t* B,
                            int n_grid, double* partials, hipStream_t stream);

hipError_t launch_search_prep(const float* sx, int K, int n_grid, float s_floor, float* S,
                              SearchCtrl* ctrl, hipStream_t stream);
// max |W| (dcol == nullptr) or max |W[n,k]| * dcol[k] over W [N, K]
hipError_t launch_absmax(const void* W, int dtype, int64_t N, int64_t K, const float* dcol,
                         SearchCtrl* ctrl, uint32_t* flags, hipStream_t stream);
hipError_t launch_x_to_f16(const void* X, int dtype, int64_t count, uint16_t* X16,
                           uint32_t* flags, hipStream_t stream);
// E_i * 2^escale (dcol == nullptr) or E_i[n,k] * dcol[k] * 2^escale, for the N rows of W, written
// to rows 0..N-1 of Estack whose grid-point slices are ld_rows rows apart (ld_rows >= N: several
// weights fill one stack)
hipError_t launch_quantize_stack(const void* W, int dtype, int64_t N, int64_t K, const float* S,
                                 int n_grid, int bits, int group, bool zero_point,
                                 const float* dcol, const SearchCtrl* ctrl, uint16_t* Estack,
                                 int64_t ld_rows, uint32_t* flags, hipStream_t stream);
hipError_t launch_lossgemm(const uint16_t* X16, int64_t M, int64_t K, const uint16_t* Estack,
                           int64_t N, int n_grid, double* partials, hipStream_t stream);
hipError_t launch_finalize(const double* partials, int64_t tiles_per_alpha, int n_grid,
                           int64_t M, int64_t N, int64_t K, const float* S,
                           SearchCtrl* ctrl, double* losses, int32_t* best,
                           float* s_best, uint32_t* flags, hipStream_t stream);

// ---- pack ----
// clip: ratios [N, K/group] in (0, 1] or nullptr; zeros: [N, K/group] (zero-point form) or
// nullptr (symmetric)
hipError_t launch_pack(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                       const float* clip, int bits, int group, uint32_t* qweight,
                       uint16_t* scales16, uint8_t* zeros, uint16_t* s16, int8_t* codes,
                       uint32_t* flags, hipStream_t stream);

// ---- folding s^-1 into the previous operator (fold.hip) ----
hipError_t launch_fold(void* prev, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       const float* s, int axis, uint32_t* flags, hipStream_t stream);

// ---- clipping search (clip.hip) ----
// Per (row, group of 128): the ratio of the grid 1 .. clip_min whose clipped quantization of
// W * s gives the smallest group error E_g H_gg E_g^T, with H_gg taken from the diagonal blocks
// of the correlation operand and d = sqrt(diag H). The diagonal block a of the operand starts
// at Bd + a * bd_block with rows bd_pitch elements apart ([t][256][256] from the diagonal-only
// preparation: 65536 and 256; the full [K][K] operand of a Gram-form search: 256 K + 256 and K).
// gram_k: nullptr, or the workspace's record of the K its operand was formed for; when it differs
// from K nothing is written and AWQ_FLAG_NO_GRAM is raised.
hipError_t launch_clip_search(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                              const float* d32, const uint16_t* Bd, int64_t bd_block,
                              int64_t bd_pitch, const uint32_t* gram_k, int n_clip,
                              float clip_min, int bits, int group, bool zero_point, float* clip,
                              float* clip_err, uint32_t* flags, hipStream_t stream);

// ---- W4A16 ----
// group 128 or 64; zeros [N, K/group] (zero-point codes) or nullptr; s16 nullptr: s folded
hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                        const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                        const uint16_t* s16, uint16_t* Y, hipStream_t stream);

}  // namespace awq
