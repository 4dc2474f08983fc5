// extern "C" entry points of libawq (declared in include/awq.h): argument validation, workspace
// layout and the launch sequence of each call. Nothing here allocates, frees or synchronises;
// every host-checkable error returns before the first HIP call.
#include <math.h>
#include <stdint.h>

#include "../../include/awq.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(awq_dtype d) { return d == AWQ_F32 || d == AWQ_F16 || d == AWQ_BF16; }

awq_status check_cfg(const awq_cfg* cfg) {
  if (!cfg) return AWQ_ERR_NULL;
  if (cfg->bits != 3 && cfg->bits != 4) return AWQ_ERR_CONFIG;
  if (cfg->group != 128 && cfg->group != 64) return AWQ_ERR_CONFIG;
  if (cfg->zero_point != 0 && cfg->zero_point != 1) return AWQ_ERR_CONFIG;
  if (cfg->n_grid < 2 || cfg->n_grid > 64) return AWQ_ERR_CONFIG;
  if (!(cfg->s_floor > 0.0f) || !isfinite(cfg->s_floor)) return AWQ_ERR_CONFIG;
  if (cfg->form != AWQ_FORM_DIRECT && cfg->form != AWQ_FORM_GRAM) return AWQ_ERR_CONFIG;
  return AWQ_OK;
}

// Largest accepted extent of one dimension; keeps every element index and tile index in range.
constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxSearchK = int64_t(1) << 22;
constexpr int64_t kMaxW4A16K = 32768;   // the W4A16 kernels keep per-channel tables in LDS
// Gram form: the K x K operand is stored (2 GiB at K = 32768); 256 rows of the transposed X
// must fit a 32-bit buffer range.
constexpr int64_t kMaxGramK = 32768;
constexpr int64_t kMaxGramMp = (int64_t(1) << 23) - awq::kGramMAlign;

// Layers with fewer than awq::kPreciseRows weight rows or awq::kPreciseTokens tokens (256 each)
// take the losses from the fp32 vector-ALU contraction (lossvalu.hip) on an fp32 error stack, in either
// form; the Gram form still prepares its operand (awq_clip_search_gram reads it).
bool precise_path(int64_t M, int64_t N) {
  return N < awq::kPreciseRows || M < awq::kPreciseTokens;
}

struct SearchLayout {
  size_t ctrl, S, X16, E, partials, total;
  bool precise;                    // fp32 error stack and the vector-ALU contraction
  size_t d64, d32, B, Blo, Xt, Hpart;   // Gram form only (Xt and Hpart share memory with E)
  size_t stats;                    // chunk partials of s_X when the search takes it (in Hpart
                                   // or in E: both are written only after s_X is final)
  int64_t tiles_per_alpha;
  awq::GramPlan plan;
};

// Direct form: ctrl | S | X16 (non-fp16 X) | E stack | partials.
// Gram form:   ctrl | S | d64 | d32 | B | Blo | partials | union(Xt + Hpart, E stack); Xt and
//              the H partials are dead before the error stack is written. Blo (the low-order
//              parts of B's diagonal 256 x 256 blocks) serves the clipping search only.
SearchLayout search_layout(int64_t M, int64_t N, int64_t K, awq_dtype xdt, int n_grid,
                           int form) {
  SearchLayout L{};
  L.precise = precise_path(M, N);
  const int64_t tilesN = (N + awq::kLossBN - 1) / awq::kLossBN;
  size_t off = 0;
  L.ctrl = off;
  off += align_up(sizeof(awq::SearchCtrl));
  L.S = off;
  off += align_up((size_t)n_grid * (size_t)K * sizeof(float));
  const size_t e_bytes = align_up((size_t)n_grid * (size_t)N * (size_t)K * (L.precise ? 4 : 2));
  const int64_t valu_tiles = awq::loss_valu_tiles(M, N);
  const size_t stats_bytes = align_up(awq::stats_workspace_bytes(M, K));
  if (form == AWQ_FORM_GRAM) {
    L.plan = awq::gram_plan(M, K);
    L.tiles_per_alpha = L.precise ? valu_tiles : tilesN * L.plan.t;
    L.d64 = off;
    off += align_up((size_t)K * sizeof(double));
    L.d32 = off;
    off += align_up((size_t)K * sizeof(float));
    L.B = off;
    off += align_up((size_t)K * (size_t)K * 2);
    L.Blo = off;
    off += align_up((size_t)L.plan.t * (size_t)(awq::kLossBM * awq::kLossBN) * 2);
    L.partials = off;
    off += align_up((size_t)n_grid * (size_t)L.tiles_per_alpha * sizeof(double));
    const size_t xt_bytes = align_up((size_t)K * (size_t)L.plan.Mp * 2);
    size_t h_bytes = align_up((size_t)L.plan.S * (size_t)L.plan.T *
                              (size_t)(awq::kLossBM * awq::kLossBN) * sizeof(float));
    if (h_bytes < stats_bytes) h_bytes = stats_bytes;
    L.Xt = off;
    L.Hpart = off + xt_bytes;
    L.stats = L.Hpart;
    L.E = off;
    off += (xt_bytes + h_bytes > e_bytes) ? xt_bytes + h_bytes : e_bytes;
  } else {
    const int64_t tilesM = (M + awq::kLossBM - 1) / awq::kLossBM;
    L.tiles_per_alpha = L.precise ? valu_tiles : tilesM * tilesN;
    L.X16 = off;
    if (xdt != AWQ_F16 && !L.precise) off += align_up((size_t)M * (size_t)K * 2);
    L.E = off;
    L.stats = off;
    off += (e_bytes > stats_bytes) ? e_bytes : stats_bytes;
    L.partials = off;
    off += align_up((size_t)n_grid * (size_t)L.tiles_per_alpha * sizeof(double));
  }
  L.total = off;
  return L;
}

awq_status hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

}  // namespace

extern "C" {

const char* awq_status_string(awq_status status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERR_NULL: return "AWQ_ERR_NULL: a required pointer is NULL";
    case AWQ_ERR_SHAPE: return "AWQ_ERR_SHAPE: shape, stride or alignment not accepted";
    case AWQ_ERR_DTYPE: return "AWQ_ERR_DTYPE: dtype not accepted by this call";
    case AWQ_ERR_CONFIG: return "AWQ_ERR_CONFIG: invalid awq_cfg or group";
    case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE: workspace missing or too small";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP: kernel launch failed";
  }
  return "unknown awq_status";
}

int32_t awq_version(void) { return 10700; }

size_t awq_act_stats_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 1 || M > kMaxDim || K > kMaxDim) return 0;
  return align_up(awq::stats_workspace_bytes(M, K));
}

awq_status awq_act_stats(const void* X, awq_dtype xdt, int64_t M, int64_t K, int64_t ldx,
                         float* sx, uint32_t* flags, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!X || !sx || !flags) return AWQ_ERR_NULL;
  if (!valid_dtype(xdt)) return AWQ_ERR_DTYPE;
  if (M < 1 || K < 8 || K % 8 || ldx < K || ldx % 8 || M > kMaxDim || K > kMaxDim ||
      ldx > kMaxDim || !aligned16(X) || awq::stats_chunks(M) > 65535)
    return AWQ_ERR_SHAPE;
  if (!ws || ws_bytes < awq_act_stats_workspace_bytes(M, K)) return AWQ_ERR_WORKSPACE;
  return hip_status(awq::launch_stats(X, (int)xdt, M, K, ldx, sx, flags, ws, stream));
}

namespace {

// Shape rules of awq_search_layer beyond the per-dimension limits.
// K >= 128 for every group size: the contractions take at least four 32-channel K steps.
bool search_shape_ok(int64_t M, int64_t N, int64_t K, const awq_cfg* cfg) {
  if (M < 1 || N < 1 || K < 128 || K % cfg->group || M > kMaxDim || N > kMaxDim ||
      K > kMaxSearchK)
    return false;
  if (cfg->form == AWQ_FORM_GRAM) {
    const int64_t Mp = (M + awq::kGramMAlign - 1) / awq::kGramMAlign * awq::kGramMAlign;
    if (K > kMaxGramK || Mp > kMaxGramMp) return false;
  }
  return true;
}

}  // namespace

size_t awq_search_workspace_bytes(int64_t M, int64_t N, int64_t K, awq_dtype xdt,
                                  const awq_cfg* cfg) {
  if (check_cfg(cfg) != AWQ_OK || !valid_dtype(xdt)) return 0;
  if (!search_shape_ok(M, N, K, cfg)) return 0;
  return search_layout(M, N, K, xdt, cfg->n_grid, cfg->form).total;
}

namespace {

// Shared body of the search calls: the weights Ws[0..n_w) (N_l rows each, all reading the same
// X) are searched together, their rows stacked in one error stack. With sx_out non-null (and sx
// null), s_X is computed first into sx_out and used. With `ev` non-null (2 * AWQ_SEARCH_STAGES events), stage j is bracketed
// by ev[2j] and ev[2j + 1].
constexpr int kMaxSharedWeights = 64;

awq_status search_impl(const void* const* Ws, const int64_t* Ns, int n_w, awq_dtype wdt,
                       int64_t K, const void* X, awq_dtype xdt, int64_t M, const float* sx,
                       float* sx_out, const awq_cfg* cfg, double* losses, int32_t* best,
                       float* s_best, uint32_t* flags, void* ws, size_t ws_bytes,
                       hipStream_t stream, hipEvent_t* ev) {
  if (!Ws || !Ns || !X || !(sx || sx_out) || !cfg || !losses || !best || !s_best || !flags)
    return AWQ_ERR_NULL;
  if (n_w < 1 || n_w > kMaxSharedWeights) return AWQ_ERR_SHAPE;
  int64_t N = 0;
  for (int l = 0; l < n_w; ++l) {
    if (!Ws[l]) return AWQ_ERR_NULL;
    if (Ns[l] < 1 || Ns[l] > kMaxDim || !aligned16(Ws[l])) return AWQ_ERR_SHAPE;
    N += Ns[l];
  }
  const awq_status cs = check_cfg(cfg);
  if (cs != AWQ_OK) return cs;
  if (wdt != AWQ_F16 && wdt != AWQ_F32) return AWQ_ERR_DTYPE;
  if (!valid_dtype(xdt)) return AWQ_ERR_DTYPE;
  // K <= 2^22 keeps the loss kernel's 32-bit buffer offsets (256 rows x 2K bytes) in range
  if (!search_shape_ok(M, N, K, cfg) || !aligned16(X)) return AWQ_ERR_SHAPE;
  if (sx_out && awq::stats_chunks(M) > 65535) return AWQ_ERR_SHAPE;
  const SearchLayout L = search_layout(M, N, K, xdt, cfg->n_grid, cfg->form);
  if ((int64_t)L.tiles_per_alpha * cfg->n_grid > (int64_t(1) << 31) - 1) return AWQ_ERR_SHAPE;
  if (!ws || ws_bytes < L.total || !aligned16(ws)) return AWQ_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  auto* ctrl = reinterpret_cast<awq::SearchCtrl*>(base + L.ctrl);
  auto* S = reinterpret_cast<float*>(base + L.S);
  auto* E = reinterpret_cast<uint16_t*>(base + L.E);
  auto* partials = reinterpret_cast<double*>(base + L.partials);
  auto* stats = reinterpret_cast<double*>(base + L.stats);
  auto* Xt = reinterpret_cast<uint16_t*>(base + L.Xt);
  const bool gram = cfg->form == AWQ_FORM_GRAM;
  const bool direct = gram && xdt == AWQ_F16 && awq::gram_direct_x(L.plan, K);
  // the Gram form's fp16 stack holds E d (column-scaled); the fp32 stack of small layers holds E
  const float* dcol = (gram && !L.precise) ? reinterpret_cast<const float*>(base + L.d32)
                                           : nullptr;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(base + L.B);
  const uint16_t* X16 = static_cast<const uint16_t*>(X);

  hipError_t e = hipSuccess;
  auto mark = [&](int idx) {
    if (ev && e == hipSuccess) e = hipEventRecord(ev[idx], stream);
  };
  // X preparation: the statistics when the search takes them, then the transpose (Gram form,
  // unless X^T X reads fp16 X directly) or the fp16 copy of a non-fp16 X (direct form)
  auto x_prep = [&]() {
    mark(2 * 1);
    if (gram) {
      if (sx_out && e == hipSuccess)
        e = awq::launch_stats(X, (int)xdt, M, K, K, sx_out, flags, stats, stream);
      if (!direct && e == hipSuccess)
        e = awq::launch_gram_transpose(X, (int)xdt, M, K, L.plan.Mp, Xt, flags, stream);
    } else {
      if (sx_out && e == hipSuccess)
        e = awq::launch_stats(X, (int)xdt, M, K, K, sx_out, flags, stats, stream);
      if (e == hipSuccess && xdt != AWQ_F16 && !L.precise) {
        auto* x16 = reinterpret_cast<uint16_t*>(base + L.X16);
        e = awq::launch_x_to_f16(X, (int)xdt, M * K, x16, flags, stream);
        X16 = x16;
      }
    }
    mark(2 * 1 + 1);
  };
  // s_X must be final before the scale table; otherwise X is prepared after it
  if (sx_out) {
    x_prep();
    sx = sx_out;
  }
  mark(2 * 0);
  if (e == hipSuccess)
    e = awq::launch_search_prep(sx, (int)K, cfg->n_grid, cfg->s_floor, S, ctrl, stream);
  mark(2 * 0 + 1);
  if (!sx_out) x_prep();
  // X^T X (stage 2), then d and the correlation operand (stage 3)
  mark(2 * 2);
  if (gram) {
    if (e == hipSuccess)
      e = awq::launch_gram_hmat(Xt, K, L.plan, reinterpret_cast<float*>(base + L.Hpart),
                                reinterpret_cast<double*>(base + L.d64),
                                reinterpret_cast<float*>(base + L.d32),
                                reinterpret_cast<uint16_t*>(base + L.B),
                                reinterpret_cast<uint16_t*>(base + L.Blo), &ctrl->gram_k, stream,
                                ev ? ev[2 * 2 + 1] : nullptr, ev ? ev[2 * 3] : nullptr,
                                direct ? X16 : nullptr, M);
  } else {
    mark(2 * 2 + 1);
    mark(2 * 3);
  }
  mark(2 * 3 + 1);
  mark(2 * 4);
  for (int l = 0; l < n_w && e == hipSuccess; ++l)
    e = awq::launch_absmax(Ws[l], (int)wdt, Ns[l], K, dcol, ctrl, flags, stream);
  mark(2 * 4 + 1);
  mark(2 * 5);
  int64_t row = 0;
  for (int l = 0; l < n_w && e == hipSuccess; ++l) {
    // the Gram form's fp16 stack is K-blocked ([K / 32][N][32] per grid point): this weight's
    // first row is row `row` of K block 0
    void* dst = L.precise ? static_cast<void*>(reinterpret_cast<float*>(base + L.E) + row * K)
                          : static_cast<void*>(E + row * (dcol ? 32 : K));
    e = awq::launch_quantize_stack(Ws[l], (int)wdt, Ns[l], K, S, cfg->n_grid, cfg->bits,
                                   cfg->group, cfg->zero_point != 0, dcol, ctrl, dst, L.precise,
                                   N, flags, stream);
    row += Ns[l];
  }
  mark(2 * 5 + 1);
  mark(2 * 6);
  if (e == hipSuccess) {
    if (L.precise)
      e = awq::launch_loss_valu(X, (int)xdt, M, K, reinterpret_cast<const float*>(base + L.E), N,
                                cfg->n_grid, partials, stream);
    else if (gram)
      e = awq::launch_gram_loss(E, N, K, B, cfg->n_grid, partials, stream);
    else
      e = awq::launch_lossgemm(X16, M, K, E, N, cfg->n_grid, partials, stream);
  }
  mark(2 * 6 + 1);
  mark(2 * 7);
  if (e == hipSuccess)
    e = awq::launch_finalize(partials, L.tiles_per_alpha, cfg->n_grid, M, N, K, S, ctrl, losses,
                             best, s_best, flags, stream);
  mark(2 * 7 + 1);
  return hip_status(e);
}

// Runs search_impl with 2 * AWQ_SEARCH_STAGES events and reads the stage durations back.
extern "C++" template <class F>
awq_status run_profiled(float* stage_ms, F&& run) {
  hipEvent_t ev[2 * AWQ_SEARCH_STAGES] = {};
  int made = 0;
  for (; made < 2 * AWQ_SEARCH_STAGES; ++made)
    if (hipEventCreate(&ev[made]) != hipSuccess) break;
  awq_status st = AWQ_ERR_HIP;
  if (made == 2 * AWQ_SEARCH_STAGES) {
    st = run(ev);
    if (st == AWQ_OK && hipEventSynchronize(ev[2 * AWQ_SEARCH_STAGES - 1]) != hipSuccess)
      st = AWQ_ERR_HIP;
    for (int j = 0; st == AWQ_OK && j < AWQ_SEARCH_STAGES; ++j)
      if (hipEventElapsedTime(&stage_ms[j], ev[2 * j], ev[2 * j + 1]) != hipSuccess)
        st = AWQ_ERR_HIP;
  }
  for (int j = 0; j < made; ++j) (void)hipEventDestroy(ev[j]);
  return st;
}

}  // namespace

awq_status awq_search_layer(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                            const void* X, awq_dtype xdt, int64_t M, const float* sx,
                            const awq_cfg* cfg, double* losses, int32_t* best, float* s_best,
                            uint32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!W || !sx) return AWQ_ERR_NULL;
  return search_impl(&W, &N, 1, wdt, K, X, xdt, M, sx, nullptr, cfg, losses, best, s_best,
                     flags, ws, ws_bytes, stream, nullptr);
}

awq_status awq_search_layers(const void* const* W, const int64_t* N, int32_t n_w,
                             awq_dtype wdt, int64_t K, const void* X, awq_dtype xdt, int64_t M,
                             const float* sx, const awq_cfg* cfg, double* losses,
                             int32_t* best, float* s_best, uint32_t* flags, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!sx) return AWQ_ERR_NULL;
  return search_impl(W, N, n_w, wdt, K, X, xdt, M, sx, nullptr, cfg, losses, best, s_best,
                     flags, ws, ws_bytes, stream, nullptr);
}

awq_status awq_stats_search_layers(const void* const* W, const int64_t* N, int32_t n_w,
                                   awq_dtype wdt, int64_t K, const void* X, awq_dtype xdt,
                                   int64_t M, const awq_cfg* cfg, float* sx, double* losses,
                                   int32_t* best, float* s_best, uint32_t* flags, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  if (!sx) return AWQ_ERR_NULL;
  return search_impl(W, N, n_w, wdt, K, X, xdt, M, nullptr, sx, cfg, losses, best, s_best,
                     flags, ws, ws_bytes, stream, nullptr);
}

awq_status awq_search_layer_profiled(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                                     const void* X, awq_dtype xdt, int64_t M, const float* sx,
                                     const awq_cfg* cfg, double* losses, int32_t* best,
                                     float* s_best, uint32_t* flags, void* ws, size_t ws_bytes,
                                     hipStream_t stream, float* stage_ms) {
  if (!stage_ms || !W || !sx) return AWQ_ERR_NULL;
  return run_profiled(stage_ms, [&](hipEvent_t* ev) {
    return search_impl(&W, &N, 1, wdt, K, X, xdt, M, sx, nullptr, cfg, losses, best, s_best,
                       flags, ws, ws_bytes, stream, ev);
  });
}

awq_status awq_stats_search_layer(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                                  const void* X, awq_dtype xdt, int64_t M, const awq_cfg* cfg,
                                  float* sx, double* losses, int32_t* best, float* s_best,
                                  uint32_t* flags, void* ws, size_t ws_bytes,
                                  hipStream_t stream, float* stage_ms) {
  if (!W || !sx) return AWQ_ERR_NULL;
  if (!stage_ms)
    return search_impl(&W, &N, 1, wdt, K, X, xdt, M, nullptr, sx, cfg, losses, best, s_best,
                       flags, ws, ws_bytes, stream, nullptr);
  return run_profiled(stage_ms, [&](hipEvent_t* ev) {
    return search_impl(&W, &N, 1, wdt, K, X, xdt, M, nullptr, sx, cfg, losses, best, s_best,
                       flags, ws, ws_bytes, stream, ev);
  });
}

awq_status awq_pack_int4(const void* W, awq_dtype wdt, int64_t N, int64_t K, const float* s,
                         const float* clip, const awq_cfg* cfg, uint32_t* qweight,
                         uint16_t* scales16, uint8_t* zeros, uint16_t* s16, int8_t* codes,
                         uint32_t* flags, hipStream_t stream) {
  if (!W || !s || !cfg || !qweight || !scales16 || !s16 || !flags) return AWQ_ERR_NULL;
  const awq_status cs = check_cfg(cfg);
  if (cs != AWQ_OK) return cs;
  if (cfg->zero_point && !zeros) return AWQ_ERR_NULL;
  if (!cfg->zero_point && zeros) return AWQ_ERR_CONFIG;
  if (wdt != AWQ_F16 && wdt != AWQ_F32) return AWQ_ERR_DTYPE;
  if (N < 1 || K < 128 || K % cfg->group || N > kMaxDim ||
      K > kMaxDim || !aligned16(W) || !aligned16(s) || !aligned16(s16) ||
      (codes && (reinterpret_cast<uintptr_t>(codes) & 7u)))
    return AWQ_ERR_SHAPE;
  if (clip && (reinterpret_cast<uintptr_t>(clip) & 3u)) return AWQ_ERR_SHAPE;
  return hip_status(awq::launch_pack(W, (int)wdt, N, K, s, clip, cfg->bits, cfg->group, qweight,
                                     scales16, zeros, s16, codes, flags, stream));
}

namespace {

struct ClipLayout {
  size_t d64, d32, Bd, Bdl, Xt, Hpart, total;
  awq::GramPlan plan;
};

ClipLayout clip_layout(int64_t M, int64_t K) {
  ClipLayout L{};
  L.plan = awq::gram_plan(M, K, /*diag=*/true);
  size_t off = 0;
  L.d64 = off;
  off += align_up((size_t)K * sizeof(double));
  L.d32 = off;
  off += align_up((size_t)K * sizeof(float));
  L.Bd = off;
  off += align_up((size_t)L.plan.t * (size_t)(awq::kLossBM * awq::kLossBN) * 2);
  L.Bdl = off;
  off += align_up((size_t)L.plan.t * (size_t)(awq::kLossBM * awq::kLossBN) * 2);
  L.Xt = off;
  off += align_up((size_t)K * (size_t)L.plan.Mp * 2);
  L.Hpart = off;
  off += align_up((size_t)L.plan.S * (size_t)L.plan.T *
                  (size_t)(awq::kLossBM * awq::kLossBN) * sizeof(float));
  L.total = off;
  return L;
}

awq_status check_clip_cfg(const awq_cfg* cfg) {
  const awq_status cs = check_cfg(cfg);
  if (cs != AWQ_OK) return cs;
  if (cfg->n_clip < 2 || cfg->n_clip > 64) return AWQ_ERR_CONFIG;
  if (!(cfg->clip_min > 0.0f && cfg->clip_min < 1.0f)) return AWQ_ERR_CONFIG;
  return AWQ_OK;
}

bool clip_shape_ok(int64_t M, int64_t N, int64_t K, const awq_cfg* cfg) {
  if (M < 1 || N < 1 || K < 128 || K % cfg->group || M > kMaxDim || N > kMaxDim ||
      K > kMaxSearchK)
    return false;
  const int64_t Mp = (M + awq::kGramMAlign - 1) / awq::kGramMAlign * awq::kGramMAlign;
  return Mp <= kMaxGramMp;
}

}  // namespace

size_t awq_clip_workspace_bytes(int64_t M, int64_t N, int64_t K, awq_dtype xdt,
                                const awq_cfg* cfg) {
  if (check_clip_cfg(cfg) != AWQ_OK || !valid_dtype(xdt)) return 0;
  if (!clip_shape_ok(M, N, K, cfg)) return 0;
  return clip_layout(M, K).total;
}

awq_status awq_clip_search(const void* W, awq_dtype wdt, int64_t N, int64_t K, const void* X,
                           awq_dtype xdt, int64_t M, const float* s, const awq_cfg* cfg,
                           float* clip, float* clip_err, uint32_t* flags, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!W || !X || !s || !cfg || !clip || !flags) return AWQ_ERR_NULL;
  const awq_status cs = check_clip_cfg(cfg);
  if (cs != AWQ_OK) return cs;
  if (wdt != AWQ_F16 && wdt != AWQ_F32) return AWQ_ERR_DTYPE;
  if (!valid_dtype(xdt)) return AWQ_ERR_DTYPE;
  if (!clip_shape_ok(M, N, K, cfg) || !aligned16(W) || !aligned16(X) || !aligned16(s))
    return AWQ_ERR_SHAPE;
  const ClipLayout L = clip_layout(M, K);
  if (!ws || ws_bytes < L.total || !aligned16(ws)) return AWQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  auto* d32 = reinterpret_cast<float*>(base + L.d32);
  auto* Bd = reinterpret_cast<uint16_t*>(base + L.Bd);
  auto* Bdl = reinterpret_cast<uint16_t*>(base + L.Bdl);
  hipError_t e = awq::launch_gram_prepare(X, (int)xdt, M, K, L.plan,
                                          reinterpret_cast<uint16_t*>(base + L.Xt),
                                          reinterpret_cast<float*>(base + L.Hpart),
                                          reinterpret_cast<double*>(base + L.d64), d32, Bd, Bdl,
                                          nullptr, flags, stream, nullptr);
  if (e == hipSuccess)
    e = awq::launch_clip_search(W, (int)wdt, N, K, s, d32, Bd, (int64_t)awq::kLossBM * awq::kLossBN,
                                (int64_t)awq::kLossBN * 32, Bdl, nullptr, 0,
                                cfg->n_clip, cfg->clip_min, cfg->bits, cfg->group,
                                cfg->zero_point != 0, clip, clip_err, flags, stream);
  return hip_status(e);
}

size_t awq_clip_search_gram_ws_bytes(int64_t K, const awq_cfg* cfg) {
  if (check_clip_cfg(cfg) != AWQ_OK || cfg->form != AWQ_FORM_GRAM) return 0;
  if (K < 128 || K % cfg->group || K > kMaxGramK) return 0;
  const SearchLayout L = search_layout(awq::kGramMAlign, 1, K, AWQ_F16, cfg->n_grid,
                                       AWQ_FORM_GRAM);
  return L.Blo + (size_t)L.plan.t * (size_t)(awq::kLossBM * awq::kLossBN) * 2;
}

awq_status awq_clip_search_gram(const void* W, awq_dtype wdt, int64_t N, int64_t K,
                                const float* s, const awq_cfg* cfg, const void* search_ws,
                                size_t search_ws_bytes, float* clip, float* clip_err,
                                uint32_t* flags, hipStream_t stream) {
  if (!W || !s || !cfg || !clip || !flags || !search_ws) return AWQ_ERR_NULL;
  const awq_status cs = check_clip_cfg(cfg);
  if (cs != AWQ_OK) return cs;
  if (cfg->form != AWQ_FORM_GRAM) return AWQ_ERR_CONFIG;
  if (wdt != AWQ_F16 && wdt != AWQ_F32) return AWQ_ERR_DTYPE;
  if (N < 1 || N > kMaxDim || K < 128 || K % cfg->group || K > kMaxGramK || !aligned16(W) ||
      !aligned16(s))
    return AWQ_ERR_SHAPE;
  const size_t need = awq_clip_search_gram_ws_bytes(K, cfg);
  if (search_ws_bytes < need || !aligned16(search_ws)) return AWQ_ERR_WORKSPACE;
  // the search's operand: its offsets depend on K and n_grid only (not on M or N)
  const SearchLayout L = search_layout(awq::kGramMAlign, 1, K, AWQ_F16, cfg->n_grid,
                                       AWQ_FORM_GRAM);
  const char* base = static_cast<const char*>(search_ws);
  const auto* ctrl = reinterpret_cast<const awq::SearchCtrl*>(base + L.ctrl);
  return hip_status(awq::launch_clip_search(
      W, (int)wdt, N, K, s, reinterpret_cast<const float*>(base + L.d32),
      reinterpret_cast<const uint16_t*>(base + L.B), (int64_t)awq::kLossBN * K + awq::kLossBN * 32,
      32 * K,
      reinterpret_cast<const uint16_t*>(base + L.Blo), ctrl, cfg->n_grid, cfg->n_clip, cfg->clip_min, cfg->bits, cfg->group,
      cfg->zero_point != 0, clip, clip_err, flags, stream));
}

awq_status awq_fold_scale(void* prev, awq_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                          const float* s, int32_t axis, uint32_t* flags, hipStream_t stream) {
  if (!prev || !s || !flags) return AWQ_ERR_NULL;
  if (!valid_dtype(dtype)) return AWQ_ERR_DTYPE;
  const size_t es = dtype == AWQ_F32 ? 4 : 2;
  if (rows < 1 || cols < 1 || ld < cols || rows > kMaxDim || cols > kMaxDim || ld > kMaxDim ||
      (axis != 0 && axis != 1) || (reinterpret_cast<uintptr_t>(prev) % es) ||
      (reinterpret_cast<uintptr_t>(s) & 3u))
    return AWQ_ERR_SHAPE;
  return hip_status(awq::launch_fold(prev, (int)dtype, rows, cols, ld, s, axis, flags, stream));
}

awq_status w4a16_gemm(const uint16_t* A, int64_t M, int64_t N, int64_t K, int32_t group,
                      const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                      const uint16_t* s16, uint16_t* Y, hipStream_t stream) {
  if (!A || !qweight || !scales16 || !Y) return AWQ_ERR_NULL;   // s16 NULL: s folded away
  if (group != 128 && group != 64) return AWQ_ERR_CONFIG;
  if (M < 1 || N < 1 || K < 128 || K % 128 || M > kMaxDim || N > kMaxDim || K > kMaxW4A16K ||
      !aligned16(A) || !aligned16(qweight) || (s16 && !aligned16(s16)))
    return AWQ_ERR_SHAPE;
  return hip_status(awq::launch_w4a16(A, M, N, K, group, qweight, scales16, zeros, s16, Y,
                                      stream));
}

size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if ((group != 128 && group != 64) || M < 1 || N < 1 || K < 128 || K % 128 || M > kMaxDim ||
      N > kMaxDim || K > kMaxW4A16K)
    return 0;
  if (M > 64) return awq::w4a16_tiled_plan(M, N, K, true).ws_bytes;
  if (!awq::w4a16_prefer_split(M, N, K)) return 0;
  return awq::w4a16_splitk_plan(M, N, K).ws_bytes;
}

awq_status w4a16_gemm_ws(const uint16_t* A, int64_t M, int64_t N, int64_t K, int32_t group,
                         const uint32_t* qweight, const uint16_t* scales16, const uint8_t* zeros,
                         const uint16_t* s16, uint16_t* Y, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!A || !qweight || !scales16 || !Y) return AWQ_ERR_NULL;
  if (group != 128 && group != 64) return AWQ_ERR_CONFIG;
  if (M < 1 || N < 1 || K < 128 || K % 128 || M > kMaxDim || N > kMaxDim || K > kMaxW4A16K ||
      !aligned16(A) || !aligned16(qweight) || (s16 && !aligned16(s16)))
    return AWQ_ERR_SHAPE;
  if (ws && !aligned16(ws)) return AWQ_ERR_WORKSPACE;
  if (M > 64) {
    const awq::W4a16TiledPlan tp = awq::w4a16_tiled_plan(M, N, K, true);
    if (tp.S == 1)
      return hip_status(awq::launch_w4a16(A, M, N, K, group, qweight, scales16, zeros, s16, Y,
                                          stream));
    if (!ws || ws_bytes < tp.ws_bytes) return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_w4a16_tiled_split(A, M, N, K, group, qweight, scales16, zeros,
                                                    s16, Y, ws, ws_bytes, stream));
  }
  if (!awq::w4a16_prefer_split(M, N, K))
    return hip_status(awq::launch_w4a16(A, M, N, K, group, qweight, scales16, zeros, s16, Y,
                                        stream));
  const awq::W4a16SplitPlan p = awq::w4a16_splitk_plan(M, N, K);
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes)) return AWQ_ERR_WORKSPACE;
  return hip_status(awq::launch_w4a16_splitk(A, M, N, K, group, qweight, scales16, zeros, s16, Y,
                                             ws, ws_bytes, stream));
}

}  // extern "C"
