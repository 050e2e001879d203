// Per-document noise levels and per-token corruption.
//
// Method: LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row (t ~ U(0,1)
// per sequence, mask probability p = (1 - 1e-3) t + 1e-3); diffusiongemma card,
// "Finetuning notes" (uniform-random ids at a per-example rate t ~ U(eps, 1));
// Axolotl diffusion docs, "Packed training" (documents in a packed stream stay
// isolated, so each draws its own t).
//
// Layout: one thread owns 4 consecutive tokens, which is exactly the output of
// one Philox call per stream, so each token costs a quarter of a call (two
// quarters under uniform noise).  A block covers 1024 tokens; the documents it
// touches are found once per block and per-document counts are gathered in LDS
// before one global atomic per (block, document).
#include "mdlm_internal.h"

namespace mdlm {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerThread = 4;
constexpr int kTokPerBlock = kThreads * kTokPerThread;
constexpr int kLdsDocs = 1024;

__global__ void __launch_bounds__(kThreads)
noise_level_kernel(int32_t n_docs, uint32_t k0, uint32_t k1, double eps,
                   double* __restrict__ p_doc, int32_t* __restrict__ doc_counts) {
#pragma clang fp contract(off)
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= n_docs) return;
  const uint4 r = philox4x32_10(make_uint4((uint32_t)b, 0u, 0u, kTagDocT), k0, k1);
  const double t = (double)(r.x >> 8) * 0x1p-24;
  // evaluated as (1 - eps), times t, plus eps; each step rounded, no fusion
  const double one_minus_eps = 1.0 - eps;
  const double scaled = one_minus_eps * t;
  p_doc[b] = eps + scaled;
  doc_counts[b] = 0;
}

__device__ __forceinline__ uint32_t threshold_of(double p) {
  // ceil(p * 2^24): exact, p in (0, 1]
  return (uint32_t)ceil(p * 16777216.0);
}

template <bool kUniform, bool kVec>
__global__ void __launch_bounds__(kThreads)
corrupt_kernel(const int32_t* __restrict__ x0, int64_t n, const int32_t* __restrict__ cu,
               int32_t n_docs, uint32_t k0, uint32_t k1, const double* __restrict__ p_doc,
               int32_t mask_id, uint32_t rand_vocab, int32_t* __restrict__ xt,
               uint8_t* __restrict__ corrupted, int32_t* __restrict__ doc_counts) {
  __shared__ int s_dlo, s_dhi;
  __shared__ int s_cnt[kLdsDocs];

  const int64_t blk0 = (int64_t)blockIdx.x * kTokPerBlock;
  const int64_t blk1 = min(blk0 + kTokPerBlock, n);
  if (threadIdx.x == 0) s_dlo = find_doc(cu, 0, n_docs - 1, blk0);
  if (threadIdx.x == 1) s_dhi = find_doc(cu, 0, n_docs - 1, blk1 - 1);
  for (int i = threadIdx.x; i < kLdsDocs; i += kThreads) s_cnt[i] = 0;
  __syncthreads();
  const int dlo = s_dlo, dhi = s_dhi;
  const bool lds_counts = (dhi - dlo) < kLdsDocs;

  const int64_t g0 = blk0 + (int64_t)threadIdx.x * kTokPerThread;
  if (g0 < n) {
    const uint64_t q = (uint64_t)g0 >> 2;
    const uint4 r1 = philox4x32_10(
        make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagBernoulli), k0, k1);
    uint4 r2 = make_uint4(0, 0, 0, 0);
    if (kUniform)
      r2 = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagReplace),
                         k0, k1);
    const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
    const uint32_t w2[4] = {r2.x, r2.y, r2.z, r2.w};

    int32_t in[4], out[4];
    uint8_t flag[4];
    const int cnt_here = (int)min<int64_t>(kTokPerThread, n - g0);
    if (kVec && cnt_here == kTokPerThread) {
      const int4 v = *reinterpret_cast<const int4*>(x0 + g0);
      in[0] = v.x; in[1] = v.y; in[2] = v.z; in[3] = v.w;
    } else {
#pragma unroll
      for (int k = 0; k < kTokPerThread; ++k) in[k] = k < cnt_here ? x0[g0 + k] : 0;
    }

    int d = find_doc(cu, dlo, dhi, g0);
    int64_t d_end = cu[d + 1];
    uint32_t thr = threshold_of(p_doc[d]);
    int run = 0;  // corrupted tokens of document d seen so far by this thread
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) {
      const int64_t g = g0 + k;
      flag[k] = 0;
      out[k] = in[k];
      if (k < cnt_here) {
        if (g >= d_end) {
          if (run) {
            if (lds_counts && d <= dhi) atomicAdd(&s_cnt[d - dlo], run);
            else atomicAdd(&doc_counts[d], run);
            run = 0;
          }
          // (bounded by the last document even if cu_seqlens is malformed)
          do { ++d; d_end = cu[d + 1]; } while (g >= d_end && d < n_docs - 1);
          thr = threshold_of(p_doc[d]);
        }
        if ((w1[k] >> 8) < thr) {
          flag[k] = 1;
          ++run;
          if (kUniform)
            out[k] = (int32_t)(((uint64_t)w2[k] * rand_vocab) >> 32);
          else
            out[k] = mask_id;
        }
      }
    }
    if (run) {
      if (lds_counts && d <= dhi) atomicAdd(&s_cnt[d - dlo], run);
      else atomicAdd(&doc_counts[d], run);
    }
    if (kVec && cnt_here == kTokPerThread) {
      *reinterpret_cast<int4*>(xt + g0) = make_int4(out[0], out[1], out[2], out[3]);
      const uint32_t packed = (uint32_t)flag[0] | ((uint32_t)flag[1] << 8) |
                              ((uint32_t)flag[2] << 16) | ((uint32_t)flag[3] << 24);
      *reinterpret_cast<uint32_t*>(corrupted + g0) = packed;
    } else {
      for (int k = 0; k < cnt_here; ++k) {
        xt[g0 + k] = out[k];
        corrupted[g0 + k] = flag[k];
      }
    }
  }
  if (lds_counts) {
    __syncthreads();
    for (int i = threadIdx.x; i <= dhi - dlo; i += kThreads)
      if (s_cnt[i]) atomicAdd(&doc_counts[dlo + i], s_cnt[i]);
  }
}

}  // namespace

hipError_t launch_corrupt(const int32_t* x0, int64_t n, const int32_t* cu, int32_t n_docs,
                          uint64_t seed, double eps, int32_t noise, int32_t mask_id,
                          int32_t rand_vocab, int32_t* xt, uint8_t* corrupted,
                          double* p_doc, int32_t* doc_counts, hipStream_t stream) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  if (n_docs > 0) {
    noise_level_kernel<<<(n_docs + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
        n_docs, k0, k1, eps, p_doc, doc_counts);
  }
  if (n > 0) {
    const bool vec = ((uintptr_t)x0 % 16 == 0) && ((uintptr_t)xt % 16 == 0) &&
                     ((uintptr_t)corrupted % 4 == 0);
    const unsigned grid = (unsigned)((n + kTokPerBlock - 1) / kTokPerBlock);
    const uint32_t rv = (uint32_t)rand_vocab;
    if (noise == MDLM_NOISE_UNIFORM) {
      if (vec)
        corrupt_kernel<true, true><<<grid, kThreads, 0, stream>>>(
            x0, n, cu, n_docs, k0, k1, p_doc, mask_id, rv, xt, corrupted, doc_counts);
      else
        corrupt_kernel<true, false><<<grid, kThreads, 0, stream>>>(
            x0, n, cu, n_docs, k0, k1, p_doc, mask_id, rv, xt, corrupted, doc_counts);
    } else {
      if (vec)
        corrupt_kernel<false, true><<<grid, kThreads, 0, stream>>>(
            x0, n, cu, n_docs, k0, k1, p_doc, mask_id, rv, xt, corrupted, doc_counts);
      else
        corrupt_kernel<false, false><<<grid, kThreads, 0, stream>>>(
            x0, n, cu, n_docs, k0, k1, p_doc, mask_id, rv, xt, corrupted, doc_counts);
    }
  }
  return hipGetLastError();
}

}  // namespace mdlm
