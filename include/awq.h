/*
 * awq.h -- C ABI of the AWQ (activation-aware weight quantization) engine for AMD gfx950.
 *
 * The engine computes, for one linear layer y = W x with W [N, K] (rows = output channels,
 * columns = input channels) and calibration activations X [M, K] (tokens x input channels):
 *   1. awq_act_stats     s_X[k] = mean_m |X[m,k]|
 *   2. awq_search_layer  for alpha_i = i/(n_grid-1): s_i = max(s_X, s_floor)^alpha_i,
 *                        group-wise symmetric round-to-nearest quantization of W*s_i, and the
 *                        output loss L_i = ||Q(W s_i)(s_i^-1 X) - W X||_F^2 / (M N);
 *                        alpha* = argmin_i L_i (lowest index on ties), s* = s_{i*}
 *   3. awq_clip_search   (optional) per row and group, the clip ratio r of W s* that minimises
 *                        the group's own output error
 *   4. awq_pack_int4     codes of Q(W s*) (clipped by r if given) packed 8 per uint32, fp16
 *                        group steps, fp16 s*
 *   5. w4a16_gemm        Y = (A / s) (q * step)^T with fp16 A and Y
 * and, for weights that read the same input (q/k/v, gate/up), awq_search_layers (one s for all
 * of them) with awq_fold_scale (s^-1 folded into the operator that produces the input, after
 * which w4a16_gemm runs without s).
 *
 * Pages defining the operations (cited by title and section):
 *   [notes]  bg51717.github.io/14592, notes on "AWQ: Activation-aware Weight Quantization for
 *            LLM Compression and Acceleration", section 方法: Q(w) = Delta * Round(w / Delta),
 *            the objective L(s) = ||Q(W s)(s^-1 X) - W X||, and s = s_X^alpha, alpha in [0,1].
 *   [eng]    qwbw.cn/news/39982, "AWQ 量化方案：激活感知的权重量化与工程实现全解析", section 三:
 *            awq_quantize (per-channel activation norm, group 128, step max/(2^(b-1)-1), round,
 *            clamp to [-2^(b-1), 2^(b-1)-1]) and QuantLinear (packed codes, per-group fp16
 *            steps, per-channel scale; forward = scale the input, dequantize, linear).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library never allocates,
 *     frees or synchronises; it launches kernels on `stream` and returns. Outputs are valid once
 *     the stream has reached that point.
 *   - Matrices are dense row-major. fp16/bf16 values are passed as their 16-bit patterns.
 *   - Host-checkable problems return a non-zero awq_status BEFORE any HIP call; no output is
 *     touched then. Problems only the device can see set bits (AWQ_FLAG_*) in the caller's
 *     uint32 `flags` word with atomic OR; the library never clears it, so the caller zeroes it.
 *   - Every device-side reduction has a fixed order: results are bitwise reproducible.
 *   - No global state; calls are thread-safe. Calls that share a workspace must be ordered.
 *   - The awq_cfg struct is read during the call only.
 */
#ifndef AWQ_H_
#define AWQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AWQ_OK = 0,
  AWQ_ERR_NULL = 1,       /* a required pointer is NULL                                   */
  AWQ_ERR_SHAPE = 2,      /* M, N or K out of range, K % group != 0, ldx < K, misalignment */
  AWQ_ERR_DTYPE = 3,      /* dtype not accepted by this call                               */
  AWQ_ERR_CONFIG = 4,     /* bits not in {3,4}, group not 64 or 128, n_grid not in [2,64], */
                          /* s_floor not a positive finite number, unknown form,           */
                          /* zero_point not 0 or 1                                         */
  AWQ_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than the *_workspace_bytes query    */
  AWQ_ERR_HIP = 6         /* a kernel launch reported an error                             */
} awq_status;

typedef enum { AWQ_F32 = 0, AWQ_F16 = 1, AWQ_BF16 = 2 } awq_dtype;

/* Device-side conditions, OR-ed into *flags. */
enum {
  AWQ_FLAG_NONFINITE_X = 1u << 0,      /* X holds an Inf or NaN                                */
  AWQ_FLAG_NONFINITE_W = 1u << 1,      /* W holds an Inf or NaN                                */
  AWQ_FLAG_STATS_INEXACT = 1u << 2,    /* a column sum of |X| may have been rounded in fp64, so */
                                       /* it is no longer order-free: fp16 X with a sum of 2^29 */
                                       /* or more; bf16 / fp32 X with S >= 2^(53 + e - p), e the */
                                       /* exponent of the column's smallest non-zero |x|, p = 7  */
                                       /* (bf16) or 23 (fp32)                                    */
  AWQ_FLAG_X_F16_RANGE = 1u << 3,      /* fp32/bf16 X has a value beyond fp16 range where X is  */
                                       /* converted to fp16: the fp16 contractions and the Gram  */
                                       /* form's operand (not the fp32 contraction)              */
  AWQ_FLAG_SCALE16_OVERFLOW = 1u << 4, /* a group step or s exceeds the fp16 range at packing   */
  AWQ_FLAG_SCALE16_SUBNORMAL = 1u << 5,/* a non-zero group step or s is fp16-subnormal or 0     */
  AWQ_FLAG_NONFINITE_LOSS = 1u << 6,   /* some L_i is not finite                                */
  AWQ_FLAG_STEP_UNDERFLOW = 1u << 7,   /* a group with max|w s| > 0 got step 0 (codes set to 0)*/
  AWQ_FLAG_CLIP_RANGE = 1u << 8,       /* a clip ratio given to awq_pack_int4 is outside (0, 1]; */
                                       /* that group was packed unclipped                       */
  AWQ_FLAG_FOLD_RANGE = 1u << 9,       /* awq_fold_scale turned a finite parameter into Inf      */
  AWQ_FLAG_NO_GRAM = 1u << 10          /* awq_clip_search_gram: the workspace holds no operand of */
                                       /* a Gram-form search with this K and n_grid; nothing was */
                                       /* written                                                */
};

/* How awq_search_layer evaluates the loss (same value, different contraction):
 *   AWQ_FORM_DIRECT  ||X E_i^T||_F^2 as one fp16 GEMM of X [M,K] with the n_grid error matrices
 *                    (2 M N K n_grid flops);
 *   AWQ_FORM_GRAM    H = X^T X once (about M K^2 flops), then sum_n E_i,n H E_i,n^T for each
 *                    grid point (about N K^2 flops each): the quadratic form in H = X^T X that
 *                    the GPTQ section of "量化方案详解"
 *                    (luoboask.github.io/fde-learning/04-inference-optimization/
 *                    quantization-schemes/) writes its layer objective as. Needs K <= 32768 and
 *                    M <= 2^23 - 128.
 * Layers with N < 256 weight rows or M < 256 tokens take, in either form, an fp32 contraction
 * on the vector ALUs instead (X read in its own dtype, fp32 error matrices, fp64 sums): with few
 * rows or tokens the fp16 rounding of E does not average out below 1e-4 of the loss. The Gram form still forms its operand
 * there, for awq_clip_search_gram. */
enum { AWQ_FORM_DIRECT = 0, AWQ_FORM_GRAM = 1 };

typedef struct {
  int32_t bits;    /* 4 (codes [-8,7]) or 3 (codes [-4,3]); the step is max|w s|/(2^(bits-1)-1) */
  int32_t group;   /* input channels per step: 128 or 64 (K a multiple of it and at least 128)  */
  int32_t n_grid;  /* number of alpha points, alpha_i = i/(n_grid-1), 2 <= n_grid <= 64         */
  float s_floor;   /* s = max(s_X, s_floor)^alpha, typically 1e-5f                              */
  int32_t form;    /* AWQ_FORM_DIRECT or AWQ_FORM_GRAM                                          */
  int32_t n_clip;  /* clipping search: ratios r_j = fp32(1 - (1 - clip_min) j / (n_clip - 1)),   */
  float clip_min;  /* j = 0 .. n_clip-1 in fp64; 2 <= n_clip <= 64, 0 < clip_min < 1 (read by    */
                   /* awq_clip_search only; typically 11 and 0.5)                                 */
  int32_t zero_point; /* 0: symmetric codes as above. 1: zero-point (asymmetric) codes: per     */
                   /* (row, group) Delta = fp32(fp32(max - min) / (2^bits - 1)), z =            */
                   /* clamp(rint(fp32(-min / Delta)), 0, 2^bits - 1), unsigned codes             */
                   /* clamp(rint(fp32(w s / Delta)) + z, 0, 2^bits - 1), Q(w s) = (q - z) Delta  */
                   /* ("AWQ 量化方案..." 三 Step 4 names a scale and a zero point per group; the   */
                   /* worked example of "量化方案详解", section AWQ, uses this 16-level range)     */
} awq_cfg;

/* Human-readable name of a status code (static storage). */
const char* awq_status_string(awq_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t awq_version(void);

/* ------------------------------------------------------------------------------------------
 * awq_act_stats -- per-input-channel activation magnitude.
 *   [notes] 方法 (s_X is computed from the layer input); [eng] 三 Step 1 (act_norm = mean|X|
 *   over calibration samples).
 * X      [M, K] with row stride ldx elements (ldx >= K, ldx % 8 == 0, K % 8 == 0), dtype xdt
 *        (AWQ_F16, AWQ_BF16 or AWQ_F32); 16-byte aligned.
 * sx     out, fp32 [K]: sx[k] = fp32( (sum_m |X[m,k]|) / M ), the sum accumulated in fp64 and
 *        the division done in fp64 before the single rounding to fp32. The sum is exact, hence
 *        independent of the order of the additions, unless AWQ_FLAG_STATS_INEXACT is raised:
 *        for fp16 X while it stays below 2^29 (every |x| is a multiple of 2^-24); for bf16 and
 *        fp32 X while it stays below 2^(53 + e - p) (every |x| of the column is a multiple of
 *        2^(e - p), e the exponent of its smallest non-zero |x|, p = 7 or 23), which wide
 *        dynamic ranges can break.
 * flags  in/out, uint32 [1]: NONFINITE_X, STATS_INEXACT.
 * ws     device workspace of at least awq_act_stats_workspace_bytes(M, K) bytes.
 * Errors: NULL pointers -> AWQ_ERR_NULL; M < 1, K < 8, shape/stride rules -> AWQ_ERR_SHAPE;
 *         unknown xdt -> AWQ_ERR_DTYPE; small workspace -> AWQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------------------------- */
size_t awq_act_stats_workspace_bytes(int64_t M, int64_t K);
awq_status awq_act_stats(const void* X, awq_dtype xdt, int64_t M, int64_t K, int64_t ldx,
                         float* sx, uint32_t* flags, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_search_layer -- the alpha grid search of [notes] 方法.
 * W      [N, K] row-major, dtype wdt (AWQ_F16 or AWQ_F32), 16-byte aligned; N >= 1.
 * X      [M, K] row-major (row stride K), dtype xdt (AWQ_F16, AWQ_BF16 or AWQ_F32).
 * sx     fp32 [K], typically the output of awq_act_stats on the same X.
 * cfg    host pointer, see awq_cfg. K must be a multiple of cfg->group, at least 128 and at
 *        most 2^22. With cfg->zero_point the codes below are the zero-point codes of awq_cfg.
 * For each i: s_i[k] = fp32(pow_f64(max(sx[k], s_floor), i/(n_grid-1))),
 *   codes q = clamp(rint(fp32(fp32(w s_i) / Delta)), -2^(b-1), 2^(b-1)-1) with
 *   Delta = fp32(max_group |fp32(w s_i)| / (2^(b-1)-1)) per (row, group of 128), all in IEEE
 *   fp32 with round-to-nearest-even (bit-identical to the specification);
 *   L_i = ||X E_i^T||_F^2 / (M N), E_i = q Delta / s_i - W, contracted on fp16 operands with
 *   fp32 accumulation and fp64 reduction (relative error ~1e-5). In the Gram form the fp16
 *   operands are the correlation matrix D^-1 H D^-1 (D = diag(sqrt(H_kk))) and E_i D; H itself
 *   is accumulated in fp32 over token chunks and summed in fp64. Layers with N < 256 or
 *   M < 256 use fp32 operands instead (see AWQ_FORM_GRAM above; relative error ~1e-6).
 *   The scale table s_i is left in the workspace: fp32 [n_grid][K] at byte offset 256.
 * losses out, fp64 [n_grid]; best out, int32 [1] = i*; s_best out, fp32 [K] = s_{i*}.
 * flags  in/out: NONFINITE_W, X_F16_RANGE, NONFINITE_LOSS.
 * ws     device workspace of at least awq_search_workspace_bytes(M, N, K, xdt, cfg) bytes
 *        (dominated by the n_grid * N * K fp16 error stack; the Gram form adds K * K fp16 and
 *        shares the stack's memory with the transposed X and the partial sums of H).
 * Errors: as for awq_act_stats, plus AWQ_ERR_CONFIG for an invalid cfg (bits, group, n_grid,
 *         s_floor or form) and AWQ_ERR_SHAPE for the Gram form's K and M limits.
 * ---------------------------------------------------------------------------------------- */
size_t awq_search_workspace_bytes(int64_t M, int64_t N, int64_t K, awq_dtype xdt,
                                  const awq_cfg* cfg);
awq_status awq_search_layer(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                            const void* X, awq_dtype xdt, int64_t M, const float* sx,
                            const awq_cfg* cfg, double* losses, int32_t* best, float* s_best,
                            uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_search_layers -- one alpha for several weights that read the same input X (the q, k and v
 * projections after one norm, or gate and up): [notes] 方法 folds s^-1 into the operator that
 * produces X (see awq_fold_scale), so all of X's consumers must share s. The search above runs
 * on the rows of W[0], W[1], ... stacked (no copy is made): L_i is the mean of squares over all
 * sum_l N[l] outputs.
 * W      host array of n_w device pointers, each [N[l], K] row-major, dtype wdt, 16-byte
 *        aligned; N host array of n_w row counts; 1 <= n_w <= 64.
 * The workspace is awq_search_workspace_bytes(M, sum_l N[l], K, xdt, cfg). Everything else as
 * awq_search_layer.
 * ---------------------------------------------------------------------------------------- */
awq_status awq_search_layers(const void* const* W, const int64_t* N, int32_t n_w,
                             awq_dtype wdt, int64_t K, const void* X, awq_dtype xdt, int64_t M,
                             const float* sx, const awq_cfg* cfg, double* losses,
                             int32_t* best, float* s_best, uint32_t* flags, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_stats_search_layers -- awq_act_stats followed by awq_search_layers on the same X, in one
 *   call: sx is an output, as in awq_stats_search_layer (identical to awq_act_stats's). Everything
 *   else as awq_search_layers.
 * ---------------------------------------------------------------------------------------- */
awq_status awq_stats_search_layers(const void* const* W, const int64_t* N, int32_t n_w,
                                   awq_dtype wdt, int64_t K, const void* X, awq_dtype xdt,
                                   int64_t M, const awq_cfg* cfg, float* sx, double* losses,
                                   int32_t* best, float* s_best, uint32_t* flags, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_fold_scale -- fold s^-1 into the previous operator's parameters, in place ([notes] 方法,
 * further optimisations: fuse the input's down-scaling into the previous operator).
 * prev   device [rows, cols] with row stride ld elements, dtype AWQ_F16, AWQ_BF16 or AWQ_F32.
 * s      device fp32: [cols] for axis 1 (a norm weight or bias as rows = 1, cols = K), [rows]
 *        for axis 0 (a previous linear layer's output channels, prev = its weight [K, *]).
 * Each element becomes fp32(fp32(p) / s[channel]), rounded once to prev's dtype (nearest even).
 * After folding, pass s16 = NULL to w4a16_gemm.
 * flags  in/out: FOLD_RANGE.
 * Errors: AWQ_ERR_NULL, AWQ_ERR_DTYPE, AWQ_ERR_SHAPE (sizes, ld < cols, axis, misalignment).
 * ---------------------------------------------------------------------------------------- */
awq_status awq_fold_scale(void* prev, awq_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                          const float* s, int32_t axis, uint32_t* flags, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_search_layer_profiled -- awq_search_layer plus the duration of each of its kernels,
 * measured with HIP events recorded between the launches on `stream`. Unlike every other call
 * it BLOCKS the host until the stream has finished the search (it reads the events back).
 * stage_ms  host array of AWQ_SEARCH_STAGES floats (milliseconds), in the order
 *           scale table; X preparation (direct: X to fp16, 0 when X is fp16; Gram: transpose
 *           to fp16 X^T, 0 when X is fp16: X^T X then reads X itself); X^T X (0 in the direct form); d and the correlation operand (0 in
 *           the direct form); max|W| (Gram: max|W d|); quantize + error stack; loss
 *           contraction; finalize.
 * Errors: as awq_search_layer; AWQ_ERR_NULL when stage_ms is NULL; AWQ_ERR_HIP when an event
 *         call fails.
 * ---------------------------------------------------------------------------------------- */
#define AWQ_SEARCH_STAGES 8
awq_status awq_search_layer_profiled(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                                     const void* X, awq_dtype xdt, int64_t M, const float* sx,
                                     const awq_cfg* cfg, double* losses, int32_t* best,
                                     float* s_best, uint32_t* flags, void* ws, size_t ws_bytes,
                                     hipStream_t stream, float* stage_ms);

/* ------------------------------------------------------------------------------------------
 * awq_stats_search_layer -- awq_act_stats followed by awq_search_layer on the same X, in one
 *   call ([notes] 方法: s_X is a statistic of the layer input, the grid search uses it).
 * sx     out, fp32 [K]: what awq_act_stats writes for this X, bit for bit (fp64 sums of 256
 *        tokens per chunk, reduced by the same final pass; with fp16 X these sums are exact,
 *        so their order does not matter, unless AWQ_FLAG_STATS_INEXACT is raised); the search
 *        then uses it.
 * The statistics pass runs first, then the search.
 * stage_ms  NULL: asynchronous, like awq_search_layer. Non-NULL: host array of
 *        AWQ_SEARCH_STAGES floats filled as by awq_search_layer_profiled (this call then BLOCKS
 *        until the stream has finished it), the statistics counted in the X preparation stage.
 * ws     device workspace of at least awq_search_workspace_bytes(M, N, K, xdt, cfg) bytes.
 * flags  in/out: those of awq_act_stats and of awq_search_layer.
 * Errors: as awq_search_layer (sx is an output here); AWQ_ERR_SHAPE also when M > 256 * 65535.
 * ---------------------------------------------------------------------------------------- */
awq_status awq_stats_search_layer(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                                  const void* X, awq_dtype xdt, int64_t M, const awq_cfg* cfg,
                                  float* sx, double* losses, int32_t* best, float* s_best,
                                  uint32_t* flags, void* ws, size_t ws_bytes,
                                  hipStream_t stream, float* stage_ms);

/* ------------------------------------------------------------------------------------------
 * awq_clip_search -- clipping of the scaled-up weights, one of the further optimisations listed
 * in [notes] 方法 (the page gives no details; the reading below is this library's).
 * For every output row n and group g of input channels, each ratio r_j of the grid in
 * awq_cfg is tried: the group of W s is clipped to [-c, c], c = fp32(r_j max|w s|), quantized
 * exactly as in awq_search_layer (so that Delta = c / (2^(b-1)-1)), and scored by the output
 * error the group causes on its own,
 *   err_j[n, g] = sum_m ( sum_{k in g} X[m,k] E[n,k] )^2,  E = Q(W s)/s - W,
 * evaluated as E_g H_gg E_g^T with the group's diagonal block of H = X^T X, in the conditioned
 * form of the Gram-form search: the error rows and the correlation block each as the sum of a
 * high and a low fp16 part (about 2^-22 relative), three MFMA products accumulated in fp32, the
 * final sum against the fp32 error rows. H is formed from X rounded to fp16 (exact for fp16 X;
 * for fp32 / bf16 X that rounding, up to 2^-11 per element, is the larger error).
 * clip[n, g] = r of the smallest error (the lowest j on ties).
 * W        [N, K], dtype wdt (AWQ_F16 or AWQ_F32); X [M, K] (row stride K), dtype xdt;
 * s        fp32 [K], the scale to clip at (typically s_best of awq_search_layer).
 * cfg      bits, group, zero_point, n_clip, clip_min (the other fields are not read).
 * clip     out, fp32 [N, K/group]: the chosen ratios (pass them to awq_pack_int4).
 * clip_err out, fp32 [n_clip, N, K/group] or NULL: err_j[n, g] for every ratio.
 * flags    in/out: NONFINITE_W, X_F16_RANGE, STEP_UNDERFLOW.
 * ws       device workspace of at least awq_clip_workspace_bytes(M, N, K, xdt, cfg) bytes
 *          (the transposed fp16 X dominates: K * M * 2 bytes).
 * Limits: K a multiple of cfg->group, at least 128 and at most 2^22, M <= 2^23 - 128. Groups of
 *         128 or 64 channels, symmetric or zero-point codes (cfg->zero_point).
 * Errors: AWQ_ERR_NULL, AWQ_ERR_SHAPE, AWQ_ERR_DTYPE, AWQ_ERR_CONFIG (also n_clip, clip_min),
 *         AWQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------------------------- */
size_t awq_clip_workspace_bytes(int64_t M, int64_t N, int64_t K, awq_dtype xdt,
                                const awq_cfg* cfg);
awq_status awq_clip_search(const void* W, awq_dtype wdt, int64_t N, int64_t K, const void* X,
                           awq_dtype xdt, int64_t M, const float* s, const awq_cfg* cfg,
                           float* clip, float* clip_err, uint32_t* flags, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_clip_search_gram -- the clipping search of awq_clip_search right after a Gram-form
 * awq_search_layer / awq_search_layers on the same X: H_gg and d are taken from that search's
 * workspace (its d = sqrt(diag X^T X) and the diagonal blocks of its correlation operand), so X
 * is not read again. Same ratios grid, error, choice and outputs as awq_clip_search; the errors
 * differ from it only by the rounding of the two preparations (their X^T X is summed over
 * different token chunks).
 * W, s, clip, clip_err, flags  as in awq_clip_search (W: any weight that read that X, e.g. each
 *          of q, k, v after awq_search_layers).
 * cfg      as in awq_clip_search, with form == AWQ_FORM_GRAM and the n_grid of the search (they
 *          locate the operand in its workspace; the search records both there).
 * search_ws, search_ws_bytes  the search's workspace (device), at least
 *          awq_clip_search_gram_ws_bytes(K, cfg) bytes; read only. The last call that wrote it
 *          must be that search, with the same K and cfg->n_grid. Checked on the device: if the
 *          workspace holds no Gram-form operand for this K and n_grid (a direct-form search,
 *          another K or grid size, or a search that did not reach that point),
 *          AWQ_FLAG_NO_GRAM is raised and clip and clip_err are not written.
 * Limits: as awq_clip_search, and K <= 32768 (the Gram form's limit).
 * Errors: AWQ_ERR_NULL, AWQ_ERR_SHAPE, AWQ_ERR_DTYPE, AWQ_ERR_CONFIG (also form != GRAM),
 *         AWQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------------------------- */
size_t awq_clip_search_gram_ws_bytes(int64_t K, const awq_cfg* cfg);
awq_status awq_clip_search_gram(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                                const float* s, const awq_cfg* cfg, const void* search_ws,
                                size_t search_ws_bytes, float* clip, float* clip_err,
                                uint32_t* flags, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_pack_int4 -- the stored result of [eng] 三 (QuantLinear(q_weight, scales_per_group,
 * awq_scale)).
 * W        [N, K], dtype wdt (AWQ_F16 or AWQ_F32); s fp32 [K] (typically s_best).
 * clip     fp32 [N, K/group] clip ratios in (0, 1] (typically from awq_clip_search), or NULL
 *          for none: the group of W s is clipped to +-fp32(r max|w s|) before quantization.
 *          A ratio outside (0, 1] sets AWQ_FLAG_CLIP_RANGE and that group is packed unclipped.
 * qweight  out, uint32 [N, K/8]: qweight[n,j] = sum_t (q[n,8j+t] & 0xF) << 4t, the codes of
 *          the same quantization as awq_search_layer / awq_clip_search (bit-identical);
 *          unsigned 0 .. 2^bits-1 with cfg->zero_point.
 * scales16 out, fp16 bits [N, K/group]: fp16(Delta), round to nearest even.
 * zeros    out, uint8 [N, K/group]: z, required with cfg->zero_point and NULL without.
 * s16      out, fp16 bits [K]: fp16(s).
 * codes    out, int8 [N, K] or NULL (not written).
 * flags    in/out: NONFINITE_W, SCALE16_OVERFLOW, SCALE16_SUBNORMAL, STEP_UNDERFLOW, CLIP_RANGE.
 * Errors: AWQ_ERR_NULL (also zeros missing with cfg->zero_point), AWQ_ERR_SHAPE, AWQ_ERR_DTYPE,
 *         AWQ_ERR_CONFIG (also zeros given without cfg->zero_point).
 * ---------------------------------------------------------------------------------------- */
awq_status awq_pack_int4(const void* W, awq_dtype wdt, int64_t N, int64_t K, const float* s,
                         const float* clip, const awq_cfg* cfg, uint32_t* qweight,
                         uint16_t* scales16, uint8_t* zeros, uint16_t* s16, int8_t* codes,
                         uint32_t* flags, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * w4a16_gemm -- QuantLinear.forward of [eng] 三 on the packed artefacts:
 *   Y[m,n] = sum_k (A[m,k] / s16[k]) * c(q[n,k]) * scales16[n, k/group]
 * with c(q) = sext4(q) for symmetric codes, or q - zeros[n, k/group] for zero-point codes.
 * A        fp16 bits [M, K]; qweight uint32 [N, K/8]; scales16 fp16 bits [N, K/group];
 *          zeros uint8 [N, K/group] for zero-point codes, or NULL for symmetric ones;
 *          s16 fp16 bits [K], or NULL when s^-1 has been folded into the producer of A (then
 *          Y = A (c(q) * step)^T); Y out, fp16 bits [M, N]. group 128 or 64; K % 128 == 0,
 *          K <= 32768.
 * Arithmetic: no fp16 value holds 1/s or A/s directly, so no s (a dead channel's s_floor
 * included) can overflow fp16. With one activation row, a' = fp32(A rcp(s)) is stored as
 * fp16(a' 2^-e) with one power of two per 128-channel block (its largest |value| in
 * [2^14, 2^15)), multiplied with the exact codes in fp32 (v_dot2_f32_f16). With more rows the
 * weight operand is fp16(c(q) r_k), r_k = fp16(2^b rcp(s_k)) with 2^b per 128-channel block (its
 * largest r_k in [2^10, 2^11)), against the fp16 activations. Accumulation is fp32; the group
 * step (times the block's power of two) multiplies the fp32 partial of each group; Y is rounded
 * once to fp16 (relative Frobenius error ~3e-4). A channel keeps full fp16 precision while the
 * s values of its 128-channel block span less than 2^24.
 * Errors: AWQ_ERR_NULL, AWQ_ERR_SHAPE (M < 1, N < 1, K % 128, K > 32768), AWQ_ERR_CONFIG.
 * ---------------------------------------------------------------------------------------- */
awq_status w4a16_gemm(const uint16_t* A, int64_t M, int64_t N, int64_t K, int32_t group,
                      const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                      const uint16_t* s16, uint16_t* Y, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * w4a16_gemm_ws -- w4a16_gemm with a workspace: the same operation, arguments, arithmetic and
 * errors. Where it pays, K is split over workgroups and a second kernel adds the slices' fp32
 * partial sums in a fixed slice order (results do not depend on scheduling; they may differ
 * from w4a16_gemm's in the last bits of Y, which adds in another order):
 *   33 <= M <= 64; 17 <= M <= 32 with N >= 8192; 16 <= M <= 32 with K >= 8192: workgroups of
 *     64 weight rows and all M rows;
 *   M > 64 while the 128 x 64 output tiles number fewer than 256 (CUs would idle): the tiled
 *     kernel on slices of at least 8 steps of 128 channels.
 * Elsewhere it is w4a16_gemm and needs no workspace.
 * ws       device workspace, 16-byte aligned, of at least w4a16_gemm_workspace_bytes(M, N, K,
 *          group) bytes (0: ws may be NULL): scratch for the slices' partial sums, any
 *          contents. With slices the call launches two kernels on `stream` (the slices, then
 *          their sum).
 * Calls that share a workspace must not overlap (one stream, or events between them).
 * Errors: as w4a16_gemm; AWQ_ERR_WORKSPACE when ws is needed and NULL or smaller than required,
 *         or is not 16-byte aligned.
 * ---------------------------------------------------------------------------------------- */
size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group);
awq_status w4a16_gemm_ws(const uint16_t* A, int64_t M, int64_t N, int64_t K, int32_t group,
                         const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                         const uint16_t* s16, uint16_t* Y, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * awq_act_stats_noalloc -- awq_act_stats for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same inputs,
 * outputs, flags and results (bit for bit) as awq_act_stats, without the workspace argument: the
 * scratch lives in a static device array of AWQ_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held until the process ends. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); on the first call made on a device it looks the array's device
 * address up once (hipGetSymbolAddress).
 * Runs on the current device; `stream` must belong to it. Calls that overlap on one GPU share the
 * array and race: order them (one stream, or events). The array keeps the last call's contents;
 * every byte a call reads it has written first, so nothing needs clearing.
 * Limit: awq_act_stats_workspace_bytes(M, K) <= AWQ_NOALLOC_SCRATCH_BYTES (32 MiB), i.e.
 * ceil(M / 256) * K <= about 3.7 million (65536 tokens: K <= 14563); larger shapes return
 * AWQ_ERR_WORKSPACE before any HIP call.
 * Errors: as awq_act_stats; AWQ_ERR_WORKSPACE for shapes beyond the limit; AWQ_ERR_HIP when the
 * device or the array's address cannot be obtained, or a launch fails.
 * ---------------------------------------------------------------------------------------- */
#define AWQ_NOALLOC_SCRATCH_BYTES (32u << 20)
awq_status awq_act_stats_noalloc(const void* X, awq_dtype xdt, int64_t M, int64_t K,
                                 int64_t ldx, float* sx, uint32_t* flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_H_ */
