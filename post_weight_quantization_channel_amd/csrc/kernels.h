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
// workspace of launch_stats: fp64 chunk partials [chunks][K], then (bf16 / fp32 X) the smallest
// exponent field per chunk and column, uint8 [chunks][K]
size_t stats_workspace_bytes(int64_t M, int64_t K);
// the second pass of launch_stats on fp16 chunk partials [chunks][K] (256 rows per chunk)
hipError_t launch_stats_final(const double* partials, int64_t chunks, int64_t M, int64_t K,
                              float* sx, uint32_t* flags, hipStream_t stream);
hipError_t launch_stats(const void* X, int dtype, int64_t M, int64_t K, int64_t ldx, float* sx,
                        uint32_t* flags, void* ws, hipStream_t stream);

// ---- search ----
constexpr int kLossBM = 256;
constexpr int kLossBN = 256;
constexpr int kLossBK = 32;

struct SearchCtrl {        // lives at the start of the search workspace
  uint32_t absmax_bits;    // max |W| as fp32 bits (atomicMax on non-negative floats)
  uint32_t done;           // grid points whose loss is final (finalize's completion count)
  uint32_t gram_k;         // K of the Gram-form operand B in this workspace (0: none)
  uint32_t n_grid;         // grid points of the search that last wrote this workspace (the
                           // offsets of its Gram operand depend on it)
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
// transpose (unless X^T X reads fp16 X directly) -> ev[0] -> X^T X partials -> ev[1] -> d and
// B. B (row l, column k) is K-blocked: [K / 32][K][32], element (l, k) at (k / 32) 32 K + 32 l +
// k % 32; with plan.diag only the t diagonal blocks, [t][8][256][32] (block a: rows and columns
// 256 a ..).
// gram_k: nullptr, or where the finish pass records K (the operand is then complete once the
// stream has passed this call).
// The two halves of launch_gram_prepare.
hipError_t launch_gram_transpose(const void* X, int xdt, int64_t M, int64_t K, int64_t Mp,
                                 uint16_t* Xt, uint32_t* flags, hipStream_t stream);
// X^T X partials -> ev, ev2 (each if not null) -> d and B. Blo: nullptr, or [t][256][256] fp16,
// the low-order parts fp16(b - fp16(b)) of the operand's diagonal blocks (block a: rows and
// columns 256 a ..), for the clipping search.
// X: nullptr (read the transposed copy Xt [K, Mp]), or fp16 X [M, K] read directly (Xt unused).
hipError_t launch_gram_hmat(const uint16_t* Xt, int64_t K, const GramPlan& p, float* Hpart,
                            double* d64, float* d32, uint16_t* B, uint16_t* Blo,
                            uint32_t* gram_k, hipStream_t stream, hipEvent_t ev, hipEvent_t ev2,
                            const uint16_t* X = nullptr, int64_t M = 0);
// whether fp16 X is read directly by X^T X (no transposed copy) under plan p
bool gram_direct_x(const GramPlan& p, int64_t K);
hipError_t launch_gram_prepare(const void* X, int xdt, int64_t M, int64_t K, const GramPlan& p,
                               uint16_t* Xt, float* Hpart, double* d64, float* d32, uint16_t* B,
                               uint16_t* Blo, uint32_t* gram_k, uint32_t* flags,
                               hipStream_t stream, hipEvent_t* ev);
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
// weights fill one stack); fp16, or fp32 with f32_stack (then dcol must be nullptr). Row-major
// ([n_grid][ld_rows][K]), except with dcol (the Gram form's operand): K-blocked,
// [n_grid][K / 32][ld_rows][32], element (n, k) of slice i at i ld_rows K + (k / 32) 32 ld_rows +
// 32 n + k % 32 (Estack then points at row 0 of the weight in K block 0).
hipError_t launch_quantize_stack(const void* W, int dtype, int64_t N, int64_t K, const float* S,
                                 int n_grid, int bits, int group, bool zero_point,
                                 const float* dcol, const SearchCtrl* ctrl, void* Estack,
                                 bool f32_stack, int64_t ld_rows, uint32_t* flags,
                                 hipStream_t stream);
// Layers with fewer rows or tokens than this take the fp32 vector-ALU contraction.
constexpr int64_t kPreciseRows = 256;
constexpr int64_t kPreciseTokens = 256;
// per-grid-point partials of launch_loss_valu: 256-token blocks x 16-row chunks
int64_t loss_valu_tiles(int64_t M, int64_t N);
// the loss of every grid point on an fp32 error stack [n_grid][N][K] (times 2^escale), X [M, K]
// read in its own dtype
hipError_t launch_loss_valu(const void* X, int xdt, int64_t M, int64_t K, const float* Estack,
                            int64_t N, int n_grid, double* partials, hipStream_t stream);
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
// at Bd + a * bd_block, K-blocked: element (l, k) of it (l, k < 256) at (k / 32) bd_kstride +
// 32 l + k % 32 (the diagonal-only preparation: 65536 and 8192; the full operand of a Gram-form
// search: 256 K + 8192 and 32 K).
// Bdl: the low-order parts of the diagonal blocks, [t][256][256] (launch_gram_hmat's Blo).
// ctrl: nullptr, or the control block of the Gram-form search whose operand is read; when its
// record of K or of the grid size differs from K and n_grid nothing is written and
// AWQ_FLAG_NO_GRAM is raised.
hipError_t launch_clip_search(const void* W, int dtype, int64_t N, int64_t K, const float* s,
                              const float* d32, const uint16_t* Bd, int64_t bd_block,
                              int64_t bd_kstride, const uint16_t* Bdl, const SearchCtrl* ctrl,
                              int n_grid, int n_clip,
                              float clip_min, int bits, int group, bool zero_point, float* clip,
                              float* clip_err, uint32_t* flags, hipStream_t stream);

// ---- W4A16 ----
// one or two activation rows: fp16 dot products against the block-scaled A / s tables (one per
// row), the codes decoded once for both rows; M = 1 with K up to kW4a16GemvMaxK, M = 2 with
// K <= 28672 (w4a16_gemv_fits); dynamic LDS of w4a16_gemv_lds_bytes(M, K) bytes (the launcher
// passes it)
constexpr int64_t kW4a16GemvMaxK = 32768;
size_t w4a16_gemv_lds_bytes(int MB, int64_t K);
bool w4a16_gemv_fits(int64_t M, int64_t K);
hipError_t launch_w4a16_gemv(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                             const uint32_t* qweight, const uint16_t* scales16,
                             const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                             hipStream_t stream);
// any M (passes of 64 rows), K up to kW4a16SkinnyMaxK, dynamic LDS of w4a16_skinny_lds_bytes
constexpr int64_t kW4a16SkinnyMaxK = 32768;
size_t w4a16_skinny_lds_bytes(int MB, int64_t K, int GS, bool ZP);
hipError_t launch_w4a16_skinny(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                               const uint32_t* qweight, const uint16_t* scales16,
                               const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                               hipStream_t stream);
// 1 <= M <= 64 with K split over workgroups (w4a16_splitk.hip): 64 weight rows per workgroup,
// S slices of KB 128-channel blocks; with S > 1 the fp32 partials go through a workspace of
// ws_bytes and a second kernel adds them
constexpr int64_t kW4a16SplitTarget = 512;   // workgroups the slices aim at
struct W4a16SplitPlan {
  int MB;            // 16-row blocks of activations
  int64_t tiles;     // 64-row weight tiles
  int64_t S;         // K slices
  int64_t KB;        // blocks per slice
  size_t ws_bytes;   // 0 when S == 1
};
W4a16SplitPlan w4a16_splitk_plan(int64_t M, int64_t N, int64_t K);
bool w4a16_prefer_split(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16_splitk(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                               const uint32_t* qweight, const uint16_t* scales16,
                               const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                               void* ws, size_t ws_bytes, hipStream_t stream);
// M > 64 (the tiled kernel, w4a16.hip) with K split over workgroups while the tiles leave CUs
// idle: S slices of KB steps, fp32 partials [S][M][N] (slice stride `stride` floats) in a
// workspace of ws_bytes, added by a second kernel
struct W4a16TiledPlan {
  int tbm;           // batch rows per tile (128 or 64)
  int64_t tiles;     // tbm x 64 output tiles
  int64_t S;         // K slices
  int64_t KB;        // 128-channel steps per slice
  int64_t stride;    // M N rounded up to a multiple of 4
  size_t ws_bytes;   // 0 when S == 1
};
W4a16TiledPlan w4a16_tiled_plan(int64_t M, int64_t N, int64_t K, bool split);
hipError_t launch_w4a16_tiled_split(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                                    const uint32_t* qweight, const uint16_t* scales16,
                                    const uint8_t* zeros, const uint16_t* s16, uint16_t* Y,
                                    void* ws, size_t ws_bytes, hipStream_t stream);
// group 128 or 64; zeros [N, K/group] (zero-point codes) or nullptr; s16 nullptr: s folded
hipError_t launch_w4a16(const uint16_t* A, int64_t M, int64_t N, int64_t K, int group,
                        const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                        const uint16_t* s16, uint16_t* Y, hipStream_t stream);

}  // namespace awq
