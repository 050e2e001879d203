// Per-document noise levels and per-token corruption.
//
// Method: LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row (one
// t ~ U(0,1) for each sequence, masking probability p = (1 - 1e-3) t + 1e-3);
// diffusiongemma card, "Finetuning notes" (uniformly drawn ids, each example
// with its own rate t ~ U(eps, 1));
// Axolotl diffusion docs, "Packed training" (documents in a packed stream stay
// isolated, so each draws its own t).  The corrective mixture (same card and
// row: mixture_prob and noise_token_wt, no formula given) is read as
// absorbing corruption in which a corrupted token takes the uniform-noise id
// instead of the mask token when a fourth Philox stream's word falls under
// ceil(mixture_prob 2^24); its output byte is then a code (1 masked, 2
// replaced) rather than a flag.
//
// Layout: a block covers 4096 tokens in four rounds; in round j thread t owns
// the 4 consecutive tokens starting at 4 (t + 256 j), exactly the output of one
// Philox call per stream, and a wave's loads and stores are contiguous.  The
// documents a block touches are found once (from hints the noise-level
// kernel leaves when documents are short, else by a wave-wide search) and
// their offsets and thresholds cached in LDS; corrupted counts are summed per
// wave and document before one LDS atomic, and one global atomic per (block,
// document).  A wave whose 256 tokens share a document takes a branch-free
// path (the kernel is bound by instruction issue, not by memory, otherwise).
// A stream of one block needs no noise-level launch: the block draws the
// noise levels itself.
#include "mdlm_internal.h"

#include <algorithm>

namespace mdlm {
namespace {

constexpr int kThreads = 256;
constexpr int kRounds = 4;
constexpr int kTokPerBlock = kThreads * 4 * kRounds;  // 4096 by default
static_assert(kRounds <= 64, "one lane per round finds a wave's window documents");
static_assert(kTokPerBlock == kRowTile, "a corruption block is one tile of the row list");
#ifndef MDLM_CORRUPT_PRELOAD
#define MDLM_CORRUPT_PRELOAD 1
#endif
// a full block loads all its tokens before locating its documents
constexpr bool kPreload = MDLM_CORRUPT_PRELOAD;
constexpr int kLdsDocs = 1024;                        // documents cached per block
// A document writes the block-range hints (see noise_level_kernel) of at
// most this many blocks; blocks past them search instead.
constexpr int kHintBlocks = 64;
// Hints are used when documents average fewer tokens than this.  With longer
// documents the search for a block's documents is shallow and its reads hit
// in L2 (they are shared by neighbouring blocks), while reading a hint always
// misses: 4,096-token documents at 2^27 tokens measured 221 us with the
// search, 229 with hints; lognormal documents of mean 296, 296 and 260.
constexpr int64_t kHintMaxMeanLen = 1024;

// Per document b: p_b, a zero count, and hints for corrupt_kernel.  The hints
// go into xt, which corrupt_kernel overwrites afterwards: for each block of
// kTokPerBlock tokens whose first token document b holds, b at the block's
// first slot; for each block of two or more tokens whose last token it
// holds, b at the block's second slot (at most kHintBlocks blocks each).  A
// block reads its two slots before writing any token and checks them
// against the offsets, so a slot nobody wrote is harmless.
// p_b = eps + (1 - eps) t_b for document b, t_b from its Philox word.
__device__ __forceinline__ double doc_p(int b, uint32_t k0, uint32_t k1, double eps) {
#pragma clang fp contract(off)
  const uint4 r = philox4x32_10(make_uint4((uint32_t)b, 0u, 0u, kTagDocT), k0, k1);
  const double t = (double)(r.x >> 8) * 0x1p-24;
  // evaluated as (1 - eps), times t, plus eps; each step rounded, no fusion
  const double one_minus_eps = 1.0 - eps;
  const double scaled = one_minus_eps * t;
  return eps + scaled;
}

// With tile_counts: the first n_tiles entries are cleared as well (one per
// thread), for corrupt_kernel to add each block's count to.
__global__ void __launch_bounds__(kThreads)
noise_level_kernel(int32_t n_docs, uint32_t k0, uint32_t k1, double eps,
                   double* __restrict__ p_doc, int32_t* __restrict__ doc_counts,
                   const int32_t* __restrict__ cu, int64_t n, int32_t* __restrict__ xt,
                   bool hints, int32_t* __restrict__ tile_counts, int64_t n_tiles) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (tile_counts && i < n_tiles) tile_counts[i] = 0;
  if (i >= n_docs) return;
  const int b = (int)i;
  p_doc[b] = doc_p(b, k0, k1, eps);
  doc_counts[b] = 0;
  if (!hints) return;
  const int64_t s = cu[b], e = cu[b + 1];
  if (!(0 <= s && s < e && e <= n)) return;
  // blocks starting inside [s, e)
  int64_t k = (s + kTokPerBlock - 1) / kTokPerBlock;
  for (int c = 0; c < kHintBlocks && k * kTokPerBlock < e; ++c, ++k) xt[k * kTokPerBlock] = b;
  // blocks of two or more tokens ending inside [s, e)
  k = s / kTokPerBlock;
  for (int c = 0; c < kHintBlocks && k * kTokPerBlock < e; ++c, ++k) {
    const int64_t last = min((k + 1) * kTokPerBlock, n) - 1;
    if (last >= s && last < e && last > k * kTokPerBlock) xt[k * kTokPerBlock + 1] = b;
  }
}

__device__ __forceinline__ uint32_t threshold_of(double p) {
  // ceil(p * 2^24): exact, p in (0, 1]
  return (uint32_t)ceil(p * 16777216.0);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Four consecutive tokens g0..g0+3 (g0 a multiple of 4), loaded as v, with
// Bernoulli thresholds t0..t3: writes xt and the mask bytes (with the
// mixture: codes 1 masked / 2 replaced) and returns the four corruption
// flags as bits 0, 8, 16, 24.
template <int kMode>
__device__ __forceinline__ uint32_t corrupt4_core(int4 v, int64_t g0, uint32_t t0, uint32_t t1,
                                                  uint32_t t2, uint32_t t3, uint32_t k0,
                                                  uint32_t k1, int32_t mask_id,
                                                  uint32_t rand_vocab, uint32_t thr_mix,
                                                  int32_t* __restrict__ xt,
                                                  uint8_t* __restrict__ corrupted) {
  const uint64_t q = (uint64_t)g0 >> 2;
  const uint4 r1 =
      philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagBernoulli), k0, k1);
  uint4 r2 = make_uint4(0, 0, 0, 0), r3 = make_uint4(0, 0, 0, 0);
  if (kMode != MDLM_NOISE_ABSORB)
    r2 = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagReplace), k0, k1);
  if (kMode == kNoiseMixture)
    r3 = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagMix), k0, k1);
  const bool c0 = (r1.x >> 8) < t0, c1 = (r1.y >> 8) < t1;
  const bool c2 = (r1.z >> 8) < t2, c3 = (r1.w >> 8) < t3;
  // replaced (rather than masked) when corrupted
  auto rep = [&](uint32_t w3) {
    return kMode == MDLM_NOISE_UNIFORM || (kMode == kNoiseMixture && (w3 >> 8) < thr_mix);
  };
  const bool p0 = rep(r3.x), p1 = rep(r3.y), p2 = rep(r3.z), p3 = rep(r3.w);
  auto out = [&](bool c, bool pr, uint32_t w2, int32_t x) {
    return c ? (pr ? (int32_t)(((uint64_t)w2 * rand_vocab) >> 32) : mask_id) : x;
  };
  *reinterpret_cast<int4*>(xt + g0) = make_int4(out(c0, p0, r2.x, v.x), out(c1, p1, r2.y, v.y),
                                                out(c2, p2, r2.z, v.z), out(c3, p3, r2.w, v.w));
  const uint32_t bits =
      (uint32_t)c0 | ((uint32_t)c1 << 8) | ((uint32_t)c2 << 16) | ((uint32_t)c3 << 24);
  uint32_t codes = bits;
  if (kMode == kNoiseMixture)
    codes += ((uint32_t)(c0 && p0) | ((uint32_t)(c1 && p1) << 8) |
              ((uint32_t)(c2 && p2) << 16) | ((uint32_t)(c3 && p3) << 24));
  *reinterpret_cast<uint32_t*>(corrupted + g0) = codes;
  return bits;
}

// corrupt4_core for four tokens of one document (threshold thr); returns the
// wave's corrupted count (every lane of the wave must call it).
template <int kMode>
__device__ __forceinline__ int corrupt4(int4 v, int64_t g0, uint32_t thr, uint32_t k0,
                                        uint32_t k1, int32_t mask_id, uint32_t rand_vocab,
                                        uint32_t thr_mix, int32_t* __restrict__ xt,
                                        uint8_t* __restrict__ corrupted) {
  const uint32_t bits = corrupt4_core<kMode>(v, g0, thr, thr, thr, thr, k0, k1, mask_id,
                                             rand_vocab, thr_mix, xt, corrupted);
  int c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) c += __popcll(__ballot((bits >> (8 * k)) & 1u));
  return c;
}

template <int kMode, bool kVec>
__global__ void __launch_bounds__(kThreads)
corrupt_kernel(const int32_t* __restrict__ x0, int64_t n, const int32_t* __restrict__ cu,
               int32_t n_docs, uint32_t k0, uint32_t k1, const double* __restrict__ p_doc,
               int32_t mask_id, uint32_t rand_vocab, uint32_t thr_mix, int32_t* __restrict__ xt,
               uint8_t* __restrict__ corrupted, int32_t* __restrict__ doc_counts, bool hints,
               double* __restrict__ p_out, double eps, int32_t* __restrict__ tile_counts) {
  __shared__ int s_dlo, s_dhi;
  __shared__ int32_t s_cu[kLdsDocs + 1];
  __shared__ int s_cnt[kLdsDocs];
  __shared__ uint32_t s_thr[kLdsDocs];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t blk0 = (int64_t)blockIdx.x * kTokPerBlock;
  const int64_t blk1 = min(blk0 + kTokPerBlock, n);
  // A full block issues the loads of all its tokens first, so that they are
  // in flight while the block finds its documents and fills its tables.
  const bool full = kVec && kPreload && blk1 - blk0 == kTokPerBlock;
  int4 vpre[kRounds];
  if (full) {
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
      vpre[j] = *reinterpret_cast<const int4*>(x0 + blk0 + 4 * (int64_t)(tid + kThreads * j));
  }
  // The block's first and last documents and their offsets and thresholds
  // in LDS.  With hints: the documents noise_level_kernel left in this
  // block's first two xt slots (read before this block writes them), taken
  // when the offsets confirm them; otherwise, or without hints, searched for.
  auto fill = [&](int lo, int count) {
    for (int i = tid; i <= count; i += kThreads) s_cu[i] = cu[lo + i];
    for (int i = tid; i < count; i += kThreads) {
      s_cnt[i] = 0;
      s_thr[i] = threshold_of(p_doc[lo + i]);
    }
  };
  int dlo = 0, nd = 0;
  bool hinted = false;
  if (p_out) {
    // The whole stream in this one block, at most kLdsDocs documents: the
    // noise levels are drawn here (no noise_level_kernel), every document
    // is in the table, and the counts are cleared before any is added to.
    for (int b = tid; b < n_docs; b += kThreads) {
      const double p = doc_p(b, k0, k1, eps);
      p_out[b] = p;
      doc_counts[b] = 0;
      s_cu[b] = cu[b];
      s_cnt[b] = 0;
      s_thr[b] = threshold_of(p);
    }
    if (tid == 0) {
      s_cu[n_docs] = cu[n_docs];
      if (tile_counts) tile_counts[0] = 0;  // (the waves add to it after the barrier)
    }
    nd = n_docs;
    hinted = true;
    __syncthreads();
  } else if (hints) {
    // Every thread reads the two slots (the same values block-wide); no
    // thread writes a token before the barrier that follows the table fill,
    // so every read sees the hints.
    const int h0 = xt[blk0];
    const int h1 = blk1 - blk0 >= 2 ? xt[blk0 + 1] : h0;
    dlo = h0;
    const int64_t nd_hint = (int64_t)h1 - h0 + 1;
    nd = (int)min<int64_t>(max<int64_t>(nd_hint, 0), kLdsDocs);
    hinted = h0 >= 0 && nd_hint >= 1 && nd_hint <= kLdsDocs && h1 < n_docs;
    if (hinted) {
      fill(dlo, nd);
      __syncthreads();
      hinted =
          s_cu[0] <= blk0 && blk0 < s_cu[1] && s_cu[nd - 1] <= blk1 - 1 && blk1 - 1 < s_cu[nd];
    }
    // (a failed check falls through to the search, whose barrier precedes
    // its own table fill, after every thread's check has read s_cu)
  }
  if (!hinted) {
    if (wave == 0) {
      const int d = wave_find_doc(cu, n_docs, blk0);
      if (lane == 0) s_dlo = d;
    } else if (wave == 1) {
      const int d = wave_find_doc(cu, n_docs, blk1 - 1);
      if (lane == 0) s_dhi = d;
    }
    __syncthreads();
    dlo = s_dlo;
    nd = s_dhi - s_dlo + 1;
    if (nd <= kLdsDocs) fill(dlo, nd);
    __syncthreads();
  }
  const bool cached = nd <= kLdsDocs;
  // The document range of this wave's window in each round (256 tokens from
  // 4 (64 wave + 256 j)): lane j finds round j's, as first local document |
  // (last - first) << 16; the rounds read it with a lane read.
  int win = 0;
  if (cached && nd > 1 && lane < kRounds) {
    const int64_t ws = blk0 + 4 * (int64_t)(64 * wave + kThreads * lane);
    if (ws < blk1) {
      const int d0 = lds_find_doc(s_cu, nd, ws);
      const int d1 = lds_find_doc(s_cu, nd, min(ws + 256, blk1) - 1);
      win = d0 | ((d1 - d0) << 16);
    }
  }
  // Bernoulli threshold of local document d (from LDS when cached)
  auto thr_of = [&](int d) { return cached ? s_thr[d] : threshold_of(p_doc[dlo + d]); };
  const DocOffsets cu_at(s_cu, cu, dlo, n_docs, cached);  // cu[dlo + i]
  // With tile_counts (cleared beforehand): the block's corrupted tokens (its
  // 4096 tokens are one tile of the row list), added once per wave from each
  // thread's share.
  int tile_mine = 0;
  auto add_tile_count = [&]() {
    const int c = wave_sum(tile_mine);
    if (lane == 0 && c) atomicAdd(&tile_counts[blockIdx.x], c);
  };

  // Whole block in one document: all four rounds' loads are issued first.
  if (kVec && cached && nd == 1 && blk1 - blk0 == kTokPerBlock) {
    int4 v[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
      v[j] = full ? vpre[j]
                  : *reinterpret_cast<const int4*>(x0 + blk0 + 4 * (int64_t)(tid + kThreads * j));
    const uint32_t thr = s_thr[0];
    int c = 0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
      c += corrupt4<kMode>(v[j], blk0 + 4 * (int64_t)(tid + kThreads * j), thr, k0, k1,
                           mask_id, rand_vocab, thr_mix, xt, corrupted);
    if (lane == 0 && c) atomicAdd(&doc_counts[dlo], c);
    if (tile_counts && lane == 0 && c) atomicAdd(&tile_counts[blockIdx.x], c);
    return;
  }

#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t g0 = blk0 + 4 * (int64_t)(tid + kThreads * j);
    // Fast paths for a wave whose 256 tokens all exist (wave-uniform tests):
    // all in one document (one threshold, ballot counts), or spread over at
    // most four documents (per-token document index from three wave-uniform
    // boundaries, ballot counts per document).  Neither walks or branches
    // per token.
    const int64_t gw = blk0 + 4 * (int64_t)(64 * wave + kThreads * j);
    if (kVec && cached && gw + 256 <= n) {
      int dw = 0, span = 0;
      if (nd > 1) {
        const int pk = __shfl(win, j, 64);
        dw = pk & 0xffff;
        span = pk >> 16;
      }
      const int4 v = full ? vpre[j] : *reinterpret_cast<const int4*>(x0 + g0);
      if (span == 0) {
        const int c = corrupt4<kMode>(v, g0, s_thr[dw], k0, k1, mask_id, rand_vocab, thr_mix,
                                      xt, corrupted);
        if (lane == 0 && c) atomicAdd(&s_cnt[dw], c);
        if (lane == 0) tile_mine += c;
        continue;
      }
      if (span <= 3) {
        // start of local documents dw+1..dw+3 (past the span: never reached)
        const int64_t b1 = s_cu[dw + 1];
        const int64_t b2 = span >= 2 ? (int64_t)s_cu[dw + 2] : INT64_MAX;
        const int64_t b3 = span >= 3 ? (int64_t)s_cu[dw + 3] : INT64_MAX;
        const uint32_t th0 = s_thr[dw], th1 = s_thr[dw + 1];
        const uint32_t th2 = s_thr[dw + min(span, 2)], th3 = s_thr[dw + span];
        int idx[4];
        uint32_t tk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t g = g0 + k;
          idx[k] = (int)(g >= b1) + (int)(g >= b2) + (int)(g >= b3);
          tk[k] = idx[k] == 0 ? th0 : idx[k] == 1 ? th1 : idx[k] == 2 ? th2 : th3;
        }
        const uint32_t bits = corrupt4_core<kMode>(v, g0, tk[0], tk[1], tk[2], tk[3], k0, k1,
                                                   mask_id, rand_vocab, thr_mix, xt, corrupted);
        tile_mine += __popc(bits);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i > span) break;
          int c = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            c += __popcll(__ballot(((bits >> (8 * k)) & 1u) && idx[k] == i));
          if (lane == 0 && c) atomicAdd(&s_cnt[dw + i], c);
        }
        continue;
      }
    }
    const bool active = g0 < n;
    int dl[4] = {0, 0, 0, 0};  // local document index of each token (-1: none)
    uint32_t flag_bits = 0;
    if (active) {
      const uint64_t q = (uint64_t)g0 >> 2;
      const uint4 r1 = philox4x32_10(
          make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagBernoulli), k0, k1);
      uint4 r2 = make_uint4(0, 0, 0, 0), r3 = make_uint4(0, 0, 0, 0);
      if (kMode != MDLM_NOISE_ABSORB)
        r2 = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagReplace), k0,
                           k1);
      if (kMode == kNoiseMixture)
        r3 = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagMix), k0, k1);
      const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
      const uint32_t w2[4] = {r2.x, r2.y, r2.z, r2.w};
      const uint32_t w3[4] = {r3.x, r3.y, r3.z, r3.w};
      uint32_t code_bits = 0;  // the stored mask bytes (codes with the mixture)
      const int cnt_here = (int)min<int64_t>(4, n - g0);
      int32_t in[4];
      if (kVec && cnt_here == 4) {
        const int4 v = full ? vpre[j] : *reinterpret_cast<const int4*>(x0 + g0);
        in[0] = v.x; in[1] = v.y; in[2] = v.z; in[3] = v.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) in[k] = k < cnt_here ? x0[g0 + k] : 0;
      }
      // document of the first token, then walk forward
      int d = cached ? lds_find_doc(s_cu, nd, g0) : find_doc(cu, dlo, dlo + nd - 1, g0) - dlo;
      int64_t d_end = cu_at[d + 1];
      uint32_t thr = thr_of(d);
      int32_t out[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t g = g0 + k;
        out[k] = in[k];
        dl[k] = -1;
        if (k < cnt_here) {
          if (g >= d_end) {
            do {
              ++d;
              d_end = cu_at[d + 1];
            } while (g >= d_end && d < nd - 1);
            thr = thr_of(d);
          }
          dl[k] = d;
          if ((w1[k] >> 8) < thr) {
            flag_bits |= 1u << (8 * k);
            const bool replaced = kMode == MDLM_NOISE_UNIFORM ||
                                  (kMode == kNoiseMixture && (w3[k] >> 8) < thr_mix);
            code_bits |= (kMode == kNoiseMixture && replaced ? 2u : 1u) << (8 * k);
            out[k] = replaced ? (int32_t)(((uint64_t)w2[k] * rand_vocab) >> 32) : mask_id;
          }
        }
      }
      if (kVec && cnt_here == 4) {
        *reinterpret_cast<int4*>(xt + g0) = make_int4(out[0], out[1], out[2], out[3]);
        *reinterpret_cast<uint32_t*>(corrupted + g0) = code_bits;
      } else {
        for (int k = 0; k < cnt_here; ++k) {
          xt[g0 + k] = out[k];
          corrupted[g0 + k] = (uint8_t)((code_bits >> (8 * k)) & 0xffu);
        }
      }
    }
    tile_mine += __popc(flag_bits);
    // Per-document counts.  Active lanes form a prefix of the wave and their
    // documents rise with the lane.  When the wave's tokens lie in one
    // document, ballots count its corrupted tokens; otherwise tokens in the
    // wave's first or last document are summed across the wave and any others
    // (short documents) are added per lane.
    const uint64_t act = __ballot(active);
    if (act != 0) {
      int last_local = -1;
#pragma unroll
      for (int k = 0; k < 4; ++k) last_local = max(last_local, dl[k]);
      const int d_first = __shfl(dl[0], 0, 64);
      const int d_last = __shfl(last_local, 63 - __clzll((long long)act), 64);
      if (d_first == d_last) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) c += __popcll(__ballot((flag_bits >> (8 * k)) & 1u));
        if (lane == 0 && c) {
          if (cached) atomicAdd(&s_cnt[d_first], c);
          else atomicAdd(&doc_counts[dlo + d_first], c);
        }
      } else {
        int c_first = 0, c_last = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int bit = (flag_bits >> (8 * k)) & 1;
          if (dl[k] == d_first) c_first += bit;
          else if (dl[k] == d_last) c_last += bit;
          else if (dl[k] >= 0 && bit) {
            if (cached) atomicAdd(&s_cnt[dl[k]], 1);
            else atomicAdd(&doc_counts[dlo + dl[k]], 1);
          }
        }
        c_first = wave_sum(c_first);
        c_last = wave_sum(c_last);
        if (lane == 0) {
          if (c_first) {
            if (cached) atomicAdd(&s_cnt[d_first], c_first);
            else atomicAdd(&doc_counts[dlo + d_first], c_first);
          }
          if (c_last) {
            if (cached) atomicAdd(&s_cnt[d_last], c_last);
            else atomicAdd(&doc_counts[dlo + d_last], c_last);
          }
        }
      }
    }
  }
  if (cached) {
    __syncthreads();
    for (int i = tid; i < nd; i += kThreads)
      if (s_cnt[i]) atomicAdd(&doc_counts[dlo + i], s_cnt[i]);
  }
  if (tile_counts) add_tile_count();
}

}  // namespace

hipError_t launch_corrupt(const int32_t* x0, int64_t n, const int32_t* cu, int32_t n_docs,
                          uint64_t seed, double eps, int32_t noise, int32_t mask_id,
                          int32_t rand_vocab, int32_t* xt, uint8_t* corrupted,
                          double* p_doc, int32_t* doc_counts, hipStream_t stream,
                          double mixture_prob, int32_t* tile_counts) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const bool hints = n > 0 && n < (int64_t)n_docs * kHintMaxMeanLen;
  // one block over at most kLdsDocs documents: it draws the noise levels too
  const bool single = n > 0 && n <= kTokPerBlock && n_docs <= kLdsDocs;
  const int64_t tiles = n > 0 ? (n + kTokPerBlock - 1) / kTokPerBlock : 0;
  if ((n_docs > 0 || tile_counts) && !single) {
    const int64_t threads = std::max<int64_t>(n_docs, tile_counts ? tiles : 0);
    if (threads > 0)
      noise_level_kernel<<<(unsigned)((threads + kThreads - 1) / kThreads), kThreads, 0,
                           stream>>>(n_docs, k0, k1, eps, p_doc, doc_counts, cu, n, xt, hints,
                                     tile_counts, tiles);
  }
  if (n > 0) {
    const unsigned grid = (unsigned)tiles;
    const uint32_t rv = (uint32_t)rand_vocab;
    // ceil(mixture_prob * 2^24): exact (power-of-two scaling), 0 .. 2^24
    const uint32_t thr_mix = (uint32_t)ceil(mixture_prob * 16777216.0);
    const bool vec = ((uintptr_t)x0 % 16 == 0) && ((uintptr_t)xt % 16 == 0) &&
                     ((uintptr_t)corrupted % 4 == 0);
#define MDLM_CORRUPT_LAUNCH(M, VEC)                                                       \
  corrupt_kernel<M, VEC><<<grid, kThreads, 0, stream>>>(x0, n, cu, n_docs, k0, k1,         \
                                                        single ? nullptr : p_doc,          \
                                                        mask_id, rv, thr_mix, xt, corrupted, \
                                                        doc_counts, hints && !single,      \
                                                        single ? p_doc : nullptr, eps,     \
                                                        tile_counts)
    if (noise == MDLM_NOISE_UNIFORM) {
      if (vec) MDLM_CORRUPT_LAUNCH(MDLM_NOISE_UNIFORM, true);
      else MDLM_CORRUPT_LAUNCH(MDLM_NOISE_UNIFORM, false);
    } else if (noise == kNoiseMixture) {
      if (vec) MDLM_CORRUPT_LAUNCH(kNoiseMixture, true);
      else MDLM_CORRUPT_LAUNCH(kNoiseMixture, false);
    } else {
      if (vec) MDLM_CORRUPT_LAUNCH(MDLM_NOISE_ABSORB, true);
      else MDLM_CORRUPT_LAUNCH(MDLM_NOISE_ABSORB, false);
    }
#undef MDLM_CORRUPT_LAUNCH
  }
  return hipGetLastError();
}

}  // namespace mdlm
