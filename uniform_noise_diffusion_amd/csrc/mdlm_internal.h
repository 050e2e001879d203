// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <functional>

#include "mdlm.h"

namespace mdlm {

// Records a formatted message in the calling thread's error slot and returns
// `code`.
int fail(int code, const char* fmt, ...);
void clear_error();
// Maps the last launch error to MDLM_EHIP (with the kernel's name) or MDLM_OK.
int check_launch(const char* what);

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies and xors,
// the key advanced by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    // one 32 x 32 -> 64-bit multiply-add instruction per product gives both
    // halves (rather than separate high and low multiplies)
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c.x;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1,
                   (uint32_t)p0);
  }
  return c;
}

// Stream tags carried in counter word 3.
constexpr uint32_t kTagDocT = 0;
constexpr uint32_t kTagBernoulli = 1;
constexpr uint32_t kTagReplace = 2;
constexpr uint32_t kTagMix = 3;  // corrective mixture: mask or replace a corrupted token
// Corruption modes: the two noise modes of mdlm_corrupt, and the corrective
// mixture of mdlm_corrupt_mixture (mask bytes are then codes 1 / 2).
constexpr int32_t kNoiseMixture = 2;

// Index of the document holding token g: the b with cu[b] <= g < cu[b+1],
// searched among documents [lo, hi] (which must contain it).
__device__ __forceinline__ int find_doc(const int32_t* __restrict__ cu, int lo, int hi,
                                        int64_t g) {
  // first i in [lo+1, hi+1] with cu[i] > g, minus one
  int a = lo + 1, b = hi + 1;
  while (a < b) {
    const int mid = (a + b) >> 1;
    if ((int64_t)cu[mid] > g)
      b = mid;
    else
      a = mid + 1;
  }
  return a - 1;
}

// Document holding token g, found by one whole wave (every lane passes the
// same g) with a 64-ary search: each round, 64 evenly spaced candidate
// documents are tested at once and the range shrinks 64-fold, so 32,768
// documents take three rounds of loads instead of fifteen.  Returns the same
// value on every lane.
__device__ __forceinline__ int wave_find_doc(const int32_t* __restrict__ cu, int n_docs,
                                             int64_t g) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n_docs - 1;  // the answer lies in [lo, hi]
  while (hi - lo + 1 > 64) {
    const int64_t span = (int64_t)hi - lo + 1;
    const int c = lo + (int)(span * lane / 64);
    const uint64_t b = __ballot((int64_t)cu[c + 1] > g);
    if (b == 0) {
      lo = lo + (int)(span * 63 / 64) + 1;
    } else {
      const int f = __ffsll((unsigned long long)b) - 1;
      const int cf = lo + (int)(span * f / 64);
      if (f > 0) lo = lo + (int)(span * (f - 1) / 64) + 1;
      hi = cf;
    }
  }
  const int c = lo + lane;
  const uint64_t b = __ballot(c <= hi && (int64_t)cu[c + 1] > g);
  return lo + __ffsll((unsigned long long)b) - 1;
}

// Document of token g among documents [0, nd) of a block whose offsets
// (cu[dlo] .. cu[dlo + nd]) are cached in LDS as s_cu[0 .. nd]; returns the
// local index.
__device__ __forceinline__ int lds_find_doc(const int32_t* s_cu, int nd, int64_t g) {
  int a = 1, b = nd;  // first i in [1, nd] with s_cu[i] > g, minus one
  while (a < b) {
    const int mid = (a + b) >> 1;
    if ((int64_t)s_cu[mid] > g)
      b = mid;
    else
      a = mid + 1;
  }
  return a - 1;
}

// Document offsets cu[lo + i] of a block that caches them in LDS as
// s_cu[i] when `cached`.  The uncached read goes through a buffer resource:
// written as plain loads, the two reads are merged by the compiler into one
// load through a selected generic pointer, i.e. a flat load that the cached
// case pays too.  The resource spans 2^30 offsets past lo (byte offsets fit
// 32 bits); offsets beyond that read as zero, which only a block spanning
// over 2^30 (empty) documents could reach.
struct DocOffsets {
  const int32_t* s_cu;
  __amdgpu_buffer_rsrc_t rsrc;
  bool cached;
  __device__ __forceinline__ DocOffsets(const int32_t* s, const int32_t* cu, int lo, int n_docs,
                                        bool c)
      : s_cu(s),
        rsrc(__builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(cu + lo), (short)0,
            (int)(uint32_t)(4 * (((int64_t)n_docs + 1 - lo) < ((int64_t)1 << 30)
                                     ? ((int64_t)n_docs + 1 - lo)
                                     : ((int64_t)1 << 30))),
            0x00020000)),
        cached(c) {}
  __device__ __forceinline__ int64_t operator[](int i) const {
    if (cached) return s_cu[i];
    return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, 4u * (uint32_t)i, 0, 0);
  }
};

// ---- launchers implemented in the kernel translation units ---------------
// noise: MDLM_NOISE_ABSORB, MDLM_NOISE_UNIFORM or kNoiseMixture (then
// mixture_prob in [0, 1] is the share of corrupted tokens replaced)
hipError_t launch_corrupt(const int32_t* x0, int64_t n_tokens, const int32_t* cu,
                          int32_t n_docs, uint64_t seed, double eps, int32_t noise,
                          int32_t mask_id, int32_t rand_vocab, int32_t* xt,
                          uint8_t* corrupted, double* p_doc, int32_t* doc_counts,
                          hipStream_t stream, double mixture_prob = 0.0,
                          int32_t* tile_counts = nullptr);

// Tokens per tile of the row list: one compaction tile, and one corruption
// block, whose per-tile corrupted counts the one-call path hands to the
// compaction's scan.
constexpr int kRowTile = 4096;

size_t compact_workspace_bytes(int64_t n_tokens, int32_t n_docs, int32_t weighting);
// mdlm_compact_masked_noalloc: the largest stream its device scratch array
// serves, that array's size, and (looked up once per device) its address on
// the current device
constexpr int64_t kNoAllocMaxTokens = (int64_t)1 << 28;
size_t compact_scratch_bytes();
hipError_t compact_scratch(void** ptr);
// the corrective mixture's row list (mdlm_compact_corrective); workspace as
// for the inverse-p weighting
hipError_t launch_compact_corrective(const uint8_t* codes, const int32_t* x0, int64_t n,
                                     const int32_t* cu, int32_t n_docs, const double* p_doc,
                                     int32_t align, double noise_wt, double clean_wt,
                                     int32_t* row_idx, int32_t* tgt, float* w, int32_t* n_rows,
                                     void* workspace, hipStream_t stream);
hipError_t launch_compact(const uint8_t* corrupted, const uint8_t* eligible, const int32_t* x0,
                          int64_t n_tokens, const int32_t* cu, int32_t n_docs,
                          const double* p_doc, int32_t align, int32_t weighting, double scale,
                          double clip, int32_t* row_idx, int32_t* tgt, float* w,
                          int32_t* n_rows, void* workspace, hipStream_t stream,
                          bool counts_given = false);

// corruption and the inverse-p row list in one pass (mdlm_corrupt_compact)
size_t corrupt_compact_workspace_bytes(int64_t n_tokens);
hipError_t launch_corrupt_compact(const int32_t* x0, int64_t n, const int32_t* cu,
                                  int32_t n_docs, uint64_t seed, double eps, int32_t noise,
                                  int32_t mask_id, int32_t rand_vocab, int32_t align,
                                  int32_t* xt, uint8_t* corrupted, double* p_doc,
                                  int32_t* doc_counts, int32_t* row_idx, int32_t* tgt,
                                  float* w, int32_t* n_rows, void* workspace,
                                  hipStream_t stream);

struct HeadCeArgs {
  const void* hidden;
  const void* W;
  int32_t dtype;
  int64_t n_tokens;
  int32_t H;
  int32_t V;
  const int32_t* row_idx;
  const int32_t* tgt;
  const float* w;
  const int32_t* n_rows;
  int64_t max_rows;
  float softcap;
  float* loss;
  float* row_ce;
  void* d_hidden;
  float* dW;  // head-weight gradient [V][H] or null (bf16 only)
  void* workspace;
  size_t workspace_bytes;
};

size_t head_ce_workspace_bytes(int64_t max_rows, int32_t H, int32_t V, int32_t dtype,
                               bool minimal, bool dw);
hipError_t launch_head_ce(const HeadCeArgs& a, hipStream_t stream);
// y = *scale * x over n entries of `dtype` (x and y 16-byte aligned; y may be x)
hipError_t launch_scale(const void* x, void* y, int32_t dtype, int64_t n, const float* scale,
                        hipStream_t stream);

// ---- device-side precondition checks (check.hip) -------------------------
// Each ORs MDLM_CHECK_* bits into *status; inputs are only read.
hipError_t launch_check_offsets(const int32_t* cu, int32_t n_docs, int64_t n, int32_t* status,
                                hipStream_t stream);
hipError_t launch_check_probs(const double* p, int32_t n_docs, int32_t* status,
                              hipStream_t stream);
hipError_t launch_check_rows(const int32_t* row_idx, const int32_t* tgt, const float* w,
                             const int32_t* n_rows, int64_t max_rows, int64_t n_tokens,
                             int32_t V, int32_t* status, hipStream_t stream);
// Checking mode: off unless MDLM_CHECK is set (not "0") at the first query,
// or switched by set_checking (which returns the previous setting).
bool checking_enabled();
int set_checking(int enable);
// Enqueues checks into a cleared status word (the argument) on `stream`.
typedef std::function<hipError_t(int32_t*)> CheckEnqueue;
// Checking mode's step before an entry point's launches: runs `enqueue`,
// waits for it and returns MDLM_OK, or MDLM_EINVAL naming the broken
// preconditions (nothing of the entry point's own work enqueued).
int run_checks(const char* fn, hipStream_t stream, const CheckEnqueue& enqueue);

}  // namespace mdlm
