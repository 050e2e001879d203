// Device-side precondition checks.
//
// The entry points never read device data on the host, so the conditions
// the header states on device-resident inputs (cumulative document offsets
// rising from 0 to n_tokens, row indices and targets in range, finite
// weights, noise levels in (0, 1]) are not checked on the hot path.  These
// kernels check them on demand: each ORs violation bits (MDLM_CHECK_*) into a
// caller-owned device word, and only reads its inputs.  The trainer the pages
// describe refuses inputs it cannot train correctly instead of training on
// them anyway (Axolotl diffusion docs, "Packed training": the default
// overflow policy raises on an oversized example; the note after the model
// table: a configuration without a native profile is refused, not trained
// as something else), which is what checking mode does here: with checking on
// (mdlm_set_checking, or MDLM_CHECK=1 in the environment at the first
// call), each entry point runs the checks of its own device inputs first,
// waits for them, and returns MDLM_EINVAL without enqueueing its work when
// one fails.
#include "mdlm_internal.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdlib.h>
#include <string.h>

namespace mdlm {
namespace {

constexpr int kThreads = 256;

// Status word of checking mode, one per device (each device holds its own
// copy); used only under g_check_mutex.
__device__ __align__(16) int32_t g_check_word;

std::mutex g_check_mutex;
std::atomic<int> g_checking{-1};  // -1: not yet read from the environment

// ORs `bits` into *status once per wave that saw a violation.
__device__ __forceinline__ void report(bool bad, int32_t bits, int32_t* status) {
  const uint64_t any = __ballot(bad);
  if (any && (threadIdx.x & 63) == __ffsll((unsigned long long)any) - 1) atomicOr(status, bits);
}

// Offsets: cu[0] = 0, cu[n_docs] = n, cu[i-1] <= cu[i]; one thread per entry.
__global__ void __launch_bounds__(kThreads)
check_offsets_kernel(const int32_t* __restrict__ cu, int32_t n_docs, int64_t n,
                     int32_t* __restrict__ status) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  bool bad = false;
  if (i <= n_docs) {
    const int64_t c = cu[i];
    bad = c < 0 || c > n;
    if (i == 0) bad = bad || c != 0;
    if (i == n_docs) bad = bad || c != n;
    if (i > 0) bad = bad || (int64_t)cu[i - 1] > c;
  }
  report(bad, MDLM_CHECK_OFFSETS, status);
}

// Noise levels in (0, 1].
__global__ void __launch_bounds__(kThreads)
check_probs_kernel(const double* __restrict__ p, int32_t n_docs, int32_t* __restrict__ status) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool bad = i < n_docs && !(p[i] > 0.0 && p[i] <= 1.0);
  report(bad, MDLM_CHECK_PROB, status);
}

// The row list of the fused head: the device row count within [0, max_rows],
// and for every listed row its index in [0, n_tokens), its target in [0, V)
// and a finite weight (tgt and w optional).
__global__ void __launch_bounds__(kThreads)
check_rows_kernel(const int32_t* __restrict__ row_idx, const int32_t* __restrict__ tgt,
                  const float* __restrict__ w, const int32_t* __restrict__ n_rows_ptr,
                  int64_t max_rows, int64_t n_tokens, int32_t V, int32_t* __restrict__ status) {
  const int32_t nr = *n_rows_ptr;
  if (blockIdx.x == 0 && threadIdx.x == 0 && (nr < 0 || nr > max_rows))
    atomicOr(status, MDLM_CHECK_ROW_COUNT);
  const int64_t n_rows = nr < 0 ? 0 : (nr > max_rows ? max_rows : nr);
  for (int64_t base = (int64_t)blockIdx.x * kThreads; base < n_rows;
       base += (int64_t)gridDim.x * kThreads) {
    const int64_t j = base + threadIdx.x;
    bool bad_r = false, bad_t = false, bad_w = false;
    if (j < n_rows) {
      const int64_t r = row_idx[j];
      bad_r = r < 0 || r >= n_tokens;
      if (tgt) bad_t = tgt[j] < 0 || tgt[j] >= V;
      if (w) bad_w = !isfinite(w[j]);
    }
    report(bad_r, MDLM_CHECK_ROW_INDEX, status);
    report(bad_t, MDLM_CHECK_TARGET, status);
    report(bad_w, MDLM_CHECK_WEIGHT, status);
  }
}

__global__ void clear_word_kernel(int32_t* p) { *p = 0; }

unsigned blocks_for(int64_t n) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + kThreads - 1) / kThreads, 65535));
}

}  // namespace

hipError_t launch_check_offsets(const int32_t* cu, int32_t n_docs, int64_t n, int32_t* status,
                                hipStream_t stream) {
  check_offsets_kernel<<<blocks_for((int64_t)n_docs + 1), kThreads, 0, stream>>>(cu, n_docs, n,
                                                                              status);
  return hipGetLastError();
}

hipError_t launch_check_probs(const double* p, int32_t n_docs, int32_t* status,
                              hipStream_t stream) {
  if (n_docs <= 0) return hipSuccess;
  check_probs_kernel<<<blocks_for(n_docs), kThreads, 0, stream>>>(p, n_docs, status);
  return hipGetLastError();
}

hipError_t launch_check_rows(const int32_t* row_idx, const int32_t* tgt, const float* w,
                             const int32_t* n_rows, int64_t max_rows, int64_t n_tokens,
                             int32_t V, int32_t* status, hipStream_t stream) {
  check_rows_kernel<<<blocks_for(max_rows), kThreads, 0, stream>>>(row_idx, tgt, w, n_rows,
                                                                   max_rows, n_tokens, V,
                                                                   status);
  return hipGetLastError();
}

bool checking_enabled() {
  int v = g_checking.load();
  if (v < 0) {
    const char* e = getenv("MDLM_CHECK");
    v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    if (!g_checking.compare_exchange_strong(expected, v)) v = g_checking.load();
  }
  return v != 0;
}

int set_checking(int enable) {
  const int prev = checking_enabled() ? 1 : 0;
  g_checking.store(enable ? 1 : 0);
  return prev;
}

int run_checks(const char* fn, hipStream_t stream, const CheckEnqueue& enqueue) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
    return fail(MDLM_EHIP, "%s: checking mode could not query the stream", fn);
  if (cs != hipStreamCaptureStatusNone)
    return fail(MDLM_EINVAL,
                "%s: checking mode waits for its checks and cannot run under stream capture",
                fn);
  std::lock_guard<std::mutex> lock(g_check_mutex);
  int32_t* word = nullptr;
  // this device's copy of the status word
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&word), HIP_SYMBOL(g_check_word)) !=
          hipSuccess ||
      !word)
    return fail(MDLM_EHIP, "%s: checking mode: no status word on this device", fn);
  clear_word_kernel<<<1, 1, 0, stream>>>(word);
  if (hipGetLastError() != hipSuccess || enqueue(word) != hipSuccess)
    return check_launch(fn);
  int32_t bits = 0;
  if (hipMemcpyAsync(&bits, word, sizeof bits, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(MDLM_EHIP, "%s: checking mode could not read its status word", fn);
  if (bits == 0) return MDLM_OK;
  char what[160] = "";
  const struct {
    int32_t bit;
    const char* name;
  } names[] = {{MDLM_CHECK_OFFSETS, "cu_seqlens"},   {MDLM_CHECK_ROW_COUNT, "n_rows"},
               {MDLM_CHECK_ROW_INDEX, "row_idx"},    {MDLM_CHECK_TARGET, "tgt"},
               {MDLM_CHECK_WEIGHT, "w"},             {MDLM_CHECK_PROB, "p_doc"}};
  for (const auto& n : names)
    if (bits & n.bit) {
      if (what[0]) strncat(what, ", ", sizeof what - strlen(what) - 1);
      strncat(what, n.name, sizeof what - strlen(what) - 1);
    }
  return fail(MDLM_EINVAL, "%s: device inputs break their preconditions (%s; check bits 0x%x)",
              fn, what, bits);
}

}  // namespace mdlm
