// C ABI entry points: host-side argument checks, then launches on the
// caller's stream.  A failed check returns before anything is enqueued.
#include "mdlm_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

namespace mdlm {
namespace {
thread_local char g_error[512];
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MDLM_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MDLM_OK;
}

// Checking mode's step for entry points that take document offsets (and,
// with `p`, noise levels).
static int check_docs(const char* fn, const int32_t* cu, int32_t n_docs, int64_t n,
                      const double* p, hipStream_t st) {
  if (!checking_enabled() || n_docs <= 0) return MDLM_OK;
  return run_checks(fn, st, [&](int32_t* word) {
    hipError_t e = launch_check_offsets(cu, n_docs, n, word, st);
    if (e == hipSuccess && p) e = launch_check_probs(p, n_docs, word, st);
    return e;
  });
}

// Checking mode's step for entry points that take a row list.
static int check_row_list(const char* fn, const int32_t* row_idx, const int32_t* tgt,
                          const float* w, const int32_t* n_rows, int64_t max_rows,
                          int64_t n_tokens, int32_t V, hipStream_t st) {
  if (!checking_enabled() || max_rows <= 0) return MDLM_OK;
  return run_checks(fn, st, [&](int32_t* word) {
    return launch_check_rows(row_idx, tgt, w, n_rows, max_rows, n_tokens, V, word, st);
  });
}

}  // namespace mdlm

using namespace mdlm;

extern "C" {

int mdlm_version(void) { return (1 << 16) | 0; }

const char* mdlm_last_error(void) { return g_error; }

int mdlm_corrupt(const int32_t* x0, int64_t n_tokens, const int32_t* cu_seqlens,
                 int32_t n_docs, uint64_t seed, double eps, int32_t noise, int32_t mask_id,
                 int32_t rand_vocab, int32_t* xt, uint8_t* corrupted, double* p_doc,
                 int32_t* doc_counts, void* stream) {
  clear_error();
  if (n_tokens < 0) return fail(MDLM_EINVAL, "mdlm_corrupt: n_tokens < 0");
  if (n_tokens > INT32_MAX)
    return fail(MDLM_EUNSUPPORTED, "mdlm_corrupt: n_tokens must be below 2^31");
  if (n_docs < 0) return fail(MDLM_EINVAL, "mdlm_corrupt: n_docs < 0");
  if (n_docs == 0 && n_tokens > 0)
    return fail(MDLM_EINVAL, "mdlm_corrupt: tokens given but n_docs = 0");
  if (!(eps > 0.0 && eps <= 1.0)) return fail(MDLM_EINVAL, "mdlm_corrupt: eps must lie in (0, 1]");
  if (noise != MDLM_NOISE_ABSORB && noise != MDLM_NOISE_UNIFORM)
    return fail(MDLM_EINVAL, "mdlm_corrupt: unknown noise mode %d", noise);
  if (noise == MDLM_NOISE_UNIFORM && rand_vocab < 1)
    return fail(MDLM_EINVAL, "mdlm_corrupt: rand_vocab must be >= 1");
  if (n_tokens > 0 && (!x0 || !xt || !corrupted))
    return fail(MDLM_EINVAL, "mdlm_corrupt: null token pointer");
  if (n_docs > 0 && (!cu_seqlens || !p_doc || !doc_counts))
    return fail(MDLM_EINVAL, "mdlm_corrupt: null document pointer");
  if (const int rc = check_docs("mdlm_corrupt", cu_seqlens, n_docs, n_tokens, nullptr,
                                reinterpret_cast<hipStream_t>(stream)))
    return rc;
  if (launch_corrupt(x0, n_tokens, cu_seqlens, n_docs, seed, eps, noise, mask_id, rand_vocab,
                     xt, corrupted, p_doc, doc_counts,
                     reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch("mdlm_corrupt");
  return MDLM_OK;
}

int mdlm_corrupt_mixture(const int32_t* x0, int64_t n_tokens, const int32_t* cu_seqlens,
                         int32_t n_docs, uint64_t seed, double eps, double mixture_prob,
                         int32_t mask_id, int32_t rand_vocab, int32_t* xt,
                         uint8_t* corrupted, double* p_doc, int32_t* doc_counts,
                         void* stream) {
  clear_error();
  const char* fn = "mdlm_corrupt_mixture";
  if (n_tokens < 0) return fail(MDLM_EINVAL, "%s: n_tokens < 0", fn);
  if (n_tokens > INT32_MAX) return fail(MDLM_EUNSUPPORTED, "%s: n_tokens must be below 2^31", fn);
  if (n_docs < 0) return fail(MDLM_EINVAL, "%s: n_docs < 0", fn);
  if (n_docs == 0 && n_tokens > 0) return fail(MDLM_EINVAL, "%s: tokens given but n_docs = 0", fn);
  if (!(eps > 0.0 && eps <= 1.0)) return fail(MDLM_EINVAL, "%s: eps must lie in (0, 1]", fn);
  if (!(mixture_prob >= 0.0 && mixture_prob <= 1.0))
    return fail(MDLM_EINVAL, "%s: mixture_prob must lie in [0, 1]", fn);
  if (rand_vocab < 1) return fail(MDLM_EINVAL, "%s: rand_vocab must be >= 1", fn);
  if (n_tokens > 0 && (!x0 || !xt || !corrupted))
    return fail(MDLM_EINVAL, "%s: null token pointer", fn);
  if (n_docs > 0 && (!cu_seqlens || !p_doc || !doc_counts))
    return fail(MDLM_EINVAL, "%s: null document pointer", fn);
  if (const int rc = check_docs(fn, cu_seqlens, n_docs, n_tokens, nullptr,
                                reinterpret_cast<hipStream_t>(stream)))
    return rc;
  if (launch_corrupt(x0, n_tokens, cu_seqlens, n_docs, seed, eps, kNoiseMixture, mask_id,
                     rand_vocab, xt, corrupted, p_doc, doc_counts,
                     reinterpret_cast<hipStream_t>(stream), mixture_prob) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

size_t mdlm_corrupt_compact_workspace_bytes(int64_t n_tokens) {
  return corrupt_compact_workspace_bytes(n_tokens);
}

int mdlm_corrupt_compact(const int32_t* x0, int64_t n_tokens, const int32_t* cu_seqlens,
                         int32_t n_docs, uint64_t seed, double eps, int32_t noise,
                         int32_t mask_id, int32_t rand_vocab, int32_t align, int32_t* xt,
                         uint8_t* corrupted, double* p_doc, int32_t* doc_counts,
                         int32_t* row_idx, int32_t* tgt, float* w, int32_t* n_rows,
                         void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const char* fn = "mdlm_corrupt_compact";
  if (n_tokens < 0) return fail(MDLM_EINVAL, "%s: n_tokens < 0", fn);
  if (n_tokens > INT32_MAX) return fail(MDLM_EUNSUPPORTED, "%s: n_tokens must be below 2^31", fn);
  if (n_docs < 0) return fail(MDLM_EINVAL, "%s: n_docs < 0", fn);
  if (n_docs == 0 && n_tokens > 0) return fail(MDLM_EINVAL, "%s: tokens given but n_docs = 0", fn);
  if (!(eps > 0.0 && eps <= 1.0)) return fail(MDLM_EINVAL, "%s: eps must lie in (0, 1]", fn);
  if (noise != MDLM_NOISE_ABSORB && noise != MDLM_NOISE_UNIFORM)
    return fail(MDLM_EINVAL, "%s: unknown noise mode %d", fn, noise);
  if (noise == MDLM_NOISE_UNIFORM && rand_vocab < 1)
    return fail(MDLM_EINVAL, "%s: rand_vocab must be >= 1", fn);
  if (align != MDLM_ALIGNED && align != MDLM_SHIFTED)
    return fail(MDLM_EINVAL, "%s: unknown alignment %d", fn, align);
  if (!n_rows) return fail(MDLM_EINVAL, "%s: null n_rows", fn);
  if (n_tokens > 0 && (!x0 || !xt || !row_idx || !tgt || !w))
    return fail(MDLM_EINVAL, "%s: null token pointer", fn);
  if (n_docs > 0 && (!cu_seqlens || !p_doc || !doc_counts))
    return fail(MDLM_EINVAL, "%s: null document pointer", fn);
  const size_t need = corrupt_compact_workspace_bytes(n_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MDLM_EWORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes,
                need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 8) != 0)
    return fail(MDLM_EINVAL, "%s: workspace must be 8-byte aligned", fn);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (const int rc = check_docs(fn, cu_seqlens, n_docs, n_tokens, nullptr, st)) return rc;
  if (launch_corrupt_compact(x0, n_tokens, cu_seqlens, n_docs, seed, eps, noise, mask_id,
                             rand_vocab, align, xt, corrupted, p_doc, doc_counts, row_idx, tgt,
                             w, n_rows, workspace, st) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

size_t mdlm_compact_workspace_bytes(int64_t n_tokens) {
  return compact_workspace_bytes(n_tokens, 0, MDLM_WEIGHT_INV_P);
}

size_t mdlm_compact_rows_workspace_bytes(int64_t n_tokens, int32_t n_docs, int32_t weighting) {
  if (n_docs < 0 || weighting < MDLM_WEIGHT_INV_P || weighting > MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED)
    return 0;
  return compact_workspace_bytes(n_tokens, n_docs, weighting);
}

// Shared checks and launch of both compaction entry points.
static int compact_common(const char* fn, bool need_mask, const uint8_t* corrupted,
                          const uint8_t* eligible,
                          const int32_t* x0, int64_t n_tokens, const int32_t* cu_seqlens,
                          int32_t n_docs, const double* p_doc, int32_t align, int32_t weighting,
                          double scale, double clip, int32_t* row_idx, int32_t* tgt, float* w,
                          int32_t* n_rows, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (n_tokens < 0) return fail(MDLM_EINVAL, "%s: n_tokens < 0", fn);
  if (n_tokens > INT32_MAX)
    return fail(MDLM_EUNSUPPORTED, "%s: n_tokens must be below 2^31", fn);
  if (n_docs < 0 || (n_docs == 0 && n_tokens > 0))
    return fail(MDLM_EINVAL, "%s: bad n_docs %d", fn, n_docs);
  if (align != MDLM_ALIGNED && align != MDLM_SHIFTED)
    return fail(MDLM_EINVAL, "%s: unknown alignment %d", fn, align);
  if (weighting < MDLM_WEIGHT_INV_P || weighting > MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED)
    return fail(MDLM_EINVAL, "%s: unknown weighting %d", fn, weighting);
  if (!isfinite(scale)) return fail(MDLM_EINVAL, "%s: weight_scale must be finite", fn);
  if (weighting == MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED && !(clip > 0.0))
    return fail(MDLM_EINVAL, "%s: weight_clip must be > 0", fn);
  if (!n_rows) return fail(MDLM_EINVAL, "%s: null n_rows", fn);
  const bool need_p = weighting != MDLM_WEIGHT_MEAN;
  if (n_tokens > 0 && (!x0 || !cu_seqlens || !row_idx || !tgt || !w || (need_p && !p_doc) ||
                       (need_mask && !corrupted)))
    return fail(MDLM_EINVAL, "%s: null pointer", fn);
  const size_t need = compact_workspace_bytes(n_tokens, n_docs, weighting);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MDLM_EWORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes,
                need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 4) != 0)
    return fail(MDLM_EINVAL, "%s: workspace must be 4-byte aligned", fn);
  if (const int rc = check_docs(fn, cu_seqlens, n_docs, n_tokens, need_p ? p_doc : nullptr,
                                reinterpret_cast<hipStream_t>(stream)))
    return rc;
  if (launch_compact(corrupted, eligible, x0, n_tokens, cu_seqlens, n_docs, p_doc, align,
                     weighting, scale, clip, row_idx, tgt, w, n_rows, workspace,
                     reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_compact_masked(const uint8_t* corrupted, const int32_t* x0, int64_t n_tokens,
                        const int32_t* cu_seqlens, int32_t n_docs, const double* p_doc,
                        int32_t align, int32_t* row_idx, int32_t* tgt, float* w,
                        int32_t* n_rows, void* workspace, size_t workspace_bytes,
                        void* stream) {
  clear_error();
  return compact_common("mdlm_compact_masked", true, corrupted, nullptr, x0, n_tokens, cu_seqlens,
                        n_docs, p_doc, align, MDLM_WEIGHT_INV_P, 1.0, 0.0, row_idx, tgt, w,
                        n_rows, workspace, workspace_bytes, stream);
}

int mdlm_compact_masked_noalloc(const uint8_t* corrupted, const int32_t* x0, int64_t n_tokens,
                                const int32_t* cu_seqlens, int32_t n_docs, const double* p_doc,
                                int32_t align, int32_t* row_idx, int32_t* tgt, float* w,
                                int32_t* n_rows, void* stream) {
  clear_error();
  const char* fn = "mdlm_compact_masked_noalloc";
  if (n_tokens > kNoAllocMaxTokens)
    return fail(MDLM_EUNSUPPORTED, "%s: n_tokens = %lld exceeds the %lld tokens its scratch "
                "array serves (use mdlm_compact_masked with a workspace)", fn,
                (long long)n_tokens, (long long)kNoAllocMaxTokens);
  void* scratch = nullptr;
  const size_t need = compact_workspace_bytes(n_tokens, n_docs, MDLM_WEIGHT_INV_P);
  if (need > 0 && compact_scratch(&scratch) != hipSuccess)
    return fail(MDLM_EHIP, "%s: no scratch array on this device", fn);
  if (need > compact_scratch_bytes())
    return fail(MDLM_EUNSUPPORTED, "%s: workspace of %zu bytes exceeds the scratch array", fn,
                need);
  return compact_common(fn, true, corrupted, nullptr, x0, n_tokens, cu_seqlens, n_docs, p_doc,
                        align, MDLM_WEIGHT_INV_P, 1.0, 0.0, row_idx, tgt, w, n_rows, scratch,
                        compact_scratch_bytes(), stream);
}

int mdlm_compact_corrective(const uint8_t* codes, const int32_t* x0, int64_t n_tokens,
                            const int32_t* cu_seqlens, int32_t n_docs, const double* p_doc,
                            int32_t align, double noise_token_wt, double clean_token_wt,
                            int32_t* row_idx, int32_t* tgt, float* w, int32_t* n_rows,
                            void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const char* fn = "mdlm_compact_corrective";
  if (n_tokens < 0) return fail(MDLM_EINVAL, "%s: n_tokens < 0", fn);
  if (n_tokens > INT32_MAX)
    return fail(MDLM_EUNSUPPORTED, "%s: n_tokens must be below 2^31", fn);
  if (n_docs < 0 || (n_docs == 0 && n_tokens > 0))
    return fail(MDLM_EINVAL, "%s: bad n_docs %d", fn, n_docs);
  if (align != MDLM_ALIGNED && align != MDLM_SHIFTED)
    return fail(MDLM_EINVAL, "%s: unknown alignment %d", fn, align);
  if (!isfinite(noise_token_wt) || !isfinite(clean_token_wt))
    return fail(MDLM_EINVAL, "%s: token weights must be finite", fn);
  if (!n_rows) return fail(MDLM_EINVAL, "%s: null n_rows", fn);
  if (n_tokens > 0 && (!codes || !x0 || !cu_seqlens || !p_doc || !row_idx || !tgt || !w))
    return fail(MDLM_EINVAL, "%s: null pointer", fn);
  const size_t need = compact_workspace_bytes(n_tokens, n_docs, MDLM_WEIGHT_INV_P);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MDLM_EWORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes,
                need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 4) != 0)
    return fail(MDLM_EINVAL, "%s: workspace must be 4-byte aligned", fn);
  if (const int rc = check_docs(fn, cu_seqlens, n_docs, n_tokens, p_doc,
                                reinterpret_cast<hipStream_t>(stream)))
    return rc;
  if (launch_compact_corrective(codes, x0, n_tokens, cu_seqlens, n_docs, p_doc, align,
                                noise_token_wt, clean_token_wt, row_idx, tgt, w, n_rows,
                                workspace, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_compact_rows(const uint8_t* corrupted, const uint8_t* eligible, const int32_t* x0,
                      int64_t n_tokens, const int32_t* cu_seqlens, int32_t n_docs,
                      const double* p_doc, int32_t align, int32_t weighting,
                      double weight_scale, double weight_clip, int32_t* row_idx, int32_t* tgt,
                      float* w, int32_t* n_rows, void* workspace, size_t workspace_bytes,
                      void* stream) {
  clear_error();
  return compact_common("mdlm_compact_rows", false, corrupted, eligible, x0, n_tokens, cu_seqlens,
                        n_docs, p_doc, align, weighting, weight_scale, weight_clip, row_idx, tgt,
                        w, n_rows, workspace, workspace_bytes, stream);
}

static bool head_sizes_ok(int64_t max_rows, int32_t H, int32_t V, int32_t dtype) {
  return max_rows >= 0 && max_rows <= INT32_MAX && H > 0 && V > 0 &&
         (dtype == MDLM_F32 || dtype == MDLM_BF16);
}

size_t mdlm_head_ce_workspace_bytes(int64_t max_rows, int32_t H, int32_t V, int32_t dtype) {
  if (!head_sizes_ok(max_rows, H, V, dtype)) return 0;
  return head_ce_workspace_bytes(max_rows, H, V, dtype, false, false);
}

size_t mdlm_head_ce_workspace_min_bytes(int64_t max_rows, int32_t H, int32_t V,
                                        int32_t dtype) {
  if (!head_sizes_ok(max_rows, H, V, dtype)) return 0;
  return head_ce_workspace_bytes(max_rows, H, V, dtype, true, false);
}

size_t mdlm_head_ce_dw_workspace_bytes(int64_t max_rows, int32_t H, int32_t V) {
  if (!head_sizes_ok(max_rows, H, V, MDLM_BF16)) return 0;
  return head_ce_workspace_bytes(max_rows, H, V, MDLM_BF16, false, true);
}

size_t mdlm_head_ce_dw_workspace_min_bytes(int64_t max_rows, int32_t H, int32_t V) {
  if (!head_sizes_ok(max_rows, H, V, MDLM_BF16)) return 0;
  return head_ce_workspace_bytes(max_rows, H, V, MDLM_BF16, true, true);
}

// Shared checks and launch of both fused head + CE entry points.
static int head_common(const char* fn, const void* hidden, const void* W, int32_t dtype,
                       int64_t n_tokens, int32_t H, int32_t V, const int32_t* row_idx,
                       const int32_t* tgt, const float* w, const int32_t* n_rows,
                       int64_t max_rows, float softcap, float* loss, float* row_ce,
                       void* d_hidden, float* dW, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (dtype != MDLM_F32 && dtype != MDLM_BF16)
    return fail(MDLM_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (n_tokens < 0 || H <= 0 || V <= 0)
    return fail(MDLM_EINVAL, "%s: bad sizes n_tokens=%lld H=%d V=%d", fn, (long long)n_tokens,
                H, V);
  if (max_rows < 0 || max_rows > n_tokens)
    return fail(MDLM_EINVAL, "%s: max_rows must lie in [0, n_tokens]", fn);
  if (n_tokens > INT32_MAX) return fail(MDLM_EUNSUPPORTED, "%s: n_tokens must be below 2^31", fn);
  if (H % 64 != 0) return fail(MDLM_EUNSUPPORTED, "%s: H = %d is not a multiple of 64", fn, H);
  // the bf16 kernels address hidden (gathered rows) and W (the dH product)
  // through 32-bit byte offsets
  if (dtype == MDLM_BF16 && (n_tokens * (int64_t)H * 2 >= (int64_t)1 << 32 ||
                             (int64_t)V * H * 2 >= (int64_t)1 << 32))
    return fail(MDLM_EUNSUPPORTED, "%s: bf16 hidden and W must each be below 4 GiB", fn);
  if (!(softcap >= 0.f) || !isfinite(softcap))
    return fail(MDLM_EINVAL, "%s: softcap must be finite and >= 0", fn);
  if (!loss) return fail(MDLM_EINVAL, "%s: null loss", fn);
  if (max_rows > 0 && (!hidden || !W || !row_idx || !tgt || !w || !n_rows))
    return fail(MDLM_EINVAL, "%s: null input pointer", fn);
  if (dtype == MDLM_BF16 && max_rows > 0 &&
      ((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(W)) % 16) != 0)
    return fail(MDLM_EINVAL, "%s: hidden and W must be 16-byte aligned", fn);
  if (dW && (reinterpret_cast<uintptr_t>(dW) % 16) != 0)
    return fail(MDLM_EINVAL, "%s: dW must be 16-byte aligned", fn);
  if (d_hidden && (reinterpret_cast<uintptr_t>(d_hidden) % 16) != 0)
    return fail(MDLM_EINVAL, "%s: d_hidden must be 16-byte aligned", fn);
  const size_t need =
      max_rows > 0 ? head_ce_workspace_bytes(max_rows, H, V, dtype, true, dW != nullptr) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MDLM_EWORKSPACE, "%s: workspace of %zu bytes, need at least %zu", fn,
                workspace_bytes, need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) % 256) != 0)
    return fail(MDLM_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (const int rc = check_row_list(fn, row_idx, tgt, w, n_rows, max_rows, n_tokens, V,
                                    reinterpret_cast<hipStream_t>(stream)))
    return rc;
  HeadCeArgs a;
  a.hidden = hidden;
  a.W = W;
  a.dtype = dtype;
  a.n_tokens = n_tokens;
  a.H = H;
  a.V = V;
  a.row_idx = row_idx;
  a.tgt = tgt;
  a.w = w;
  a.n_rows = n_rows;
  a.max_rows = max_rows;
  a.softcap = softcap;
  a.loss = loss;
  a.row_ce = row_ce;
  a.d_hidden = d_hidden;
  a.dW = dW;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  if (launch_head_ce(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_fused_head_ce_fwd_bwd(const void* hidden, const void* W, int32_t dtype,
                               int64_t n_tokens, int32_t H, int32_t V,
                               const int32_t* row_idx, const int32_t* tgt, const float* w,
                               const int32_t* n_rows, int64_t max_rows, float softcap,
                               float* loss, float* row_ce, void* d_hidden, void* workspace,
                               size_t workspace_bytes, void* stream) {
  clear_error();
  return head_common("mdlm_fused_head_ce_fwd_bwd", hidden, W, dtype, n_tokens, H, V, row_idx,
                     tgt, w, n_rows, max_rows, softcap, loss, row_ce, d_hidden, nullptr,
                     workspace, workspace_bytes, stream);
}

int mdlm_fused_head_ce_fwd_bwd_dw(const void* hidden, const void* W, int64_t n_tokens,
                                  int32_t H, int32_t V, const int32_t* row_idx,
                                  const int32_t* tgt, const float* w, const int32_t* n_rows,
                                  int64_t max_rows, float softcap, float* loss, float* row_ce,
                                  void* d_hidden, float* dW, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  clear_error();
  const char* fn = "mdlm_fused_head_ce_fwd_bwd_dw";
  if (!dW) return fail(MDLM_EINVAL, "%s: null dW", fn);
  return head_common(fn, hidden, W, MDLM_BF16, n_tokens, H, V, row_idx, tgt, w, n_rows,
                     max_rows, softcap, loss, row_ce, d_hidden, dW, workspace, workspace_bytes,
                     stream);
}

int mdlm_scale(const void* x, void* y, int32_t dtype, int64_t n, const float* scale,
               void* stream) {
  clear_error();
  const char* fn = "mdlm_scale";
  if (dtype != MDLM_F32 && dtype != MDLM_BF16)
    return fail(MDLM_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (n < 0) return fail(MDLM_EINVAL, "%s: n < 0", fn);
  if (n > 0 && (!x || !y || !scale)) return fail(MDLM_EINVAL, "%s: null pointer", fn);
  if (n > 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) % 16) != 0)
    return fail(MDLM_EINVAL, "%s: x and y must be 16-byte aligned", fn);
  if (launch_scale(x, y, dtype, n, scale, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_check_offsets(const int32_t* cu_seqlens, int32_t n_docs, int64_t n_tokens,
                       int32_t* status, void* stream) {
  clear_error();
  const char* fn = "mdlm_check_offsets";
  if (n_docs < 0 || n_tokens < 0) return fail(MDLM_EINVAL, "%s: bad sizes", fn);
  if (!cu_seqlens || !status) return fail(MDLM_EINVAL, "%s: null pointer", fn);
  if (launch_check_offsets(cu_seqlens, n_docs, n_tokens, status,
                           reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_check_probs(const double* p_doc, int32_t n_docs, int32_t* status, void* stream) {
  clear_error();
  const char* fn = "mdlm_check_probs";
  if (n_docs < 0) return fail(MDLM_EINVAL, "%s: n_docs < 0", fn);
  if ((n_docs > 0 && !p_doc) || !status) return fail(MDLM_EINVAL, "%s: null pointer", fn);
  if (launch_check_probs(p_doc, n_docs, status, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_check_rows(const int32_t* row_idx, const int32_t* tgt, const float* w,
                    const int32_t* n_rows, int64_t max_rows, int64_t n_tokens, int32_t V,
                    int32_t* status, void* stream) {
  clear_error();
  const char* fn = "mdlm_check_rows";
  if (max_rows < 0 || n_tokens < 0 || V < 0) return fail(MDLM_EINVAL, "%s: bad sizes", fn);
  if (!n_rows || !status || (max_rows > 0 && !row_idx))
    return fail(MDLM_EINVAL, "%s: null pointer", fn);
  if (launch_check_rows(row_idx, tgt, w, n_rows, max_rows, n_tokens, V, status,
                        reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return check_launch(fn);
  return MDLM_OK;
}

int mdlm_set_checking(int enable) { return set_checking(enable); }

}  // extern "C"
