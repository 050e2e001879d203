// Ordered stream compaction of the scored rows.
//
// Method: LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row (CE only
// on masked tokens, divided by p); Axolotl diffusion docs, model table
// (aligned vs shifted logits) and "Batching" (logits computed only at label
// slots).  Each scored token g of document b yields, in ascending g,
//   ALIGNED: (row g,   target x0[g], weight 1 / (p_b N))
//   SHIFTED: (row g-1, target x0[g], weight 1 / (p_b N)), skipping g = cu[b].
//
// Four passes, none of which waits on another block:
//   1. tile_docs_kernel: one thread per document records, for every 4096-token
//      tile whose first or last token the document holds, that document --
//      each tile learns the range of documents it touches without a search;
//   2. count_kernel: one wave per tile counts its scored tokens (1 byte per
//      token read, four 16-byte loads in flight per lane);
//   3. group_scan_kernel: each block scans 1024 tile counts into offsets
//      within the group (in place) and writes the group's total;
//   4. scatter_kernel: each block adds the totals of the groups before its own
//      to its offset, re-reads its tile in four 1024-token rounds, ranks each
//      round's scored tokens with ballots, stages (row, target, weight) in
//      LDS and writes them with coalesced stores.
// A stream of one tile whose weights need no totals runs pass 4 alone.
// A tile's document offsets and weights are cached in LDS when it touches at
// most 1024 documents (682 with the corrective mixture's second table); a
// wave whose 256 tokens of a round touch at most four documents finds each
// token's document by comparisons with wave-uniform boundaries instead of a
// search.
//
// The corrective mixture's list (same card and row: noise_token_wt and
// clean_token_wt, no formula given) uses the same passes: the codes are the
// mask when clean tokens carry no weight, every token is listed otherwise,
// and the scatter picks each row's weight by its code from two per-document
// LDS tables (1 / (p_b N), noise_token_wt / (p_b N)) and one scalar
// (clean_token_wt / N).
#include "mdlm_internal.h"

#include <algorithm>
#include <mutex>

namespace mdlm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = kRowTile;      // tokens per tile (4096)
#ifndef MDLM_COMPACT_LDS_DOCS
#define MDLM_COMPACT_LDS_DOCS 1024
#endif
constexpr int kLdsDocs = MDLM_COMPACT_LDS_DOCS;  // documents cached per tile
constexpr int kGroup = 1024;         // tiles per scan group (one block)
constexpr int kRoundTok = kThreads * 4;  // tokens per scatter round: 1024
#ifndef MDLM_SCATTER_BUFS
#define MDLM_SCATTER_BUFS 1
#endif
// staging buffers: two drop the barrier that protects reuse, at the cost of
// LDS (and so of resident blocks)
constexpr int kBufs = MDLM_SCATTER_BUFS;

__global__ void set_int_kernel(int32_t* p, int32_t v) { *p = v; }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Bit 8k set iff byte k of w is nonzero: bit 0 of each byte becomes the OR
// of that byte's bits (shifts that only move bits down within a byte's low
// nibble).
__device__ __forceinline__ uint32_t nonzero_flags(uint32_t w) {
  uint32_t x = w | (w >> 4);
  x |= x >> 2;
  x |= x >> 1;
  return x & 0x01010101u;
}

// Which tokens are scored before the alignment rule: corrupted and eligible.
// kC / kE say whether each mask is present (an absent mask scores every
// token); they are compile-time so the token loops carry no pointer tests.
template <bool kC, bool kE>
struct RowMasks {
  const uint8_t* corrupted;
  const uint8_t* eligible;
  __device__ __forceinline__ bool at(int64_t g) const {
    return (!kC || corrupted[g]) && (!kE || eligible[g]);
  }
  // the 4 tokens at g (4-byte aligned, all in range): byte k is nonzero iff
  // token g + k is scored (a single mask's bytes as they are)
  __device__ __forceinline__ uint32_t word(int64_t g) const {
    if (kC && !kE) return *reinterpret_cast<const uint32_t*>(corrupted + g);
    if (kE && !kC) return *reinterpret_cast<const uint32_t*>(eligible + g);
    uint32_t f = 0x01010101u;
    if (kC) f &= nonzero_flags(*reinterpret_cast<const uint32_t*>(corrupted + g));
    if (kE) f &= nonzero_flags(*reinterpret_cast<const uint32_t*>(eligible + g));
    return f;
  }
  // flags of the 16 tokens at off (16-byte aligned, all in range)
  __device__ __forceinline__ uint4 flags16(int64_t off) const {
    uint4 f = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
    if (kC) {
      const uint4 v = *reinterpret_cast<const uint4*>(corrupted + off);
      f.x &= nonzero_flags(v.x); f.y &= nonzero_flags(v.y);
      f.z &= nonzero_flags(v.z); f.w &= nonzero_flags(v.w);
    }
    if (kE) {
      const uint4 v = *reinterpret_cast<const uint4*>(eligible + off);
      f.x &= nonzero_flags(v.x); f.y &= nonzero_flags(v.y);
      f.z &= nonzero_flags(v.z); f.w &= nonzero_flags(v.w);
    }
    return f;
  }
  __device__ __forceinline__ bool aligned16() const {
    return (!kC || (uintptr_t)corrupted % 16 == 0) && (!kE || (uintptr_t)eligible % 16 == 0);
  }
};

// How rows are weighted (see mdlm_compact_rows).
struct WeightArgs {
  int32_t mode;
  double scale, clip;
  const double* p_doc;
  int64_t n;                   // tokens in the call
  const int32_t* doc_rows;     // example-mean mode: scored rows per document
  const int32_t* n_examples;   // example-mean mode: documents with a scored row
};

// Weight of the rows of document b, in fp64 rounded once to fp32.
__device__ __forceinline__ float doc_weight(const WeightArgs& a, int b, int64_t total_rows,
                                            int32_t n_examples) {
#pragma clang fp contract(off)
  if (a.mode == MDLM_WEIGHT_MEAN) return (float)(a.scale / (double)total_rows);
  if (a.mode == MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED) {
    const int32_t nb = a.doc_rows[b];
    if (nb <= 0) return 0.f;  // (no row of such a document is ever written)
    double x = 1.0 / (1.0 - a.p_doc[b]);
    x = fmin(x, a.clip);
    return (float)(a.scale * x / ((double)nb * (double)n_examples));
  }
  return (float)(a.scale / (a.p_doc[b] * (double)a.n));
}

// Set bits of b at lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t b) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// For each tile k, the documents holding its first token (tile_lo[k]) and its
// last token (tile_hi[k]).  A non-empty document holds exactly the tokens
// [cu[b], cu[b+1]), so each tile boundary token has exactly one writer.
// Offsets that break the preconditions (negative, decreasing, past n) are
// clipped to [0, n] first, so every write stays inside the two tables; the
// tables' contents are then unspecified, and tile_range clamps what it reads.
// With start_mask (tile counts of corrupted tokens given, shifted rows): a
// document whose first token is marked takes that token out of its tile's
// count, which then counts the tile's scored rows.
__global__ void __launch_bounds__(kThreads)
tile_docs_kernel(const int32_t* __restrict__ cu, int32_t n_docs, int64_t n,
                 int32_t* __restrict__ tile_lo, int32_t* __restrict__ tile_hi,
                 const uint8_t* __restrict__ start_mask, int32_t* __restrict__ tile_counts) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= n_docs) return;
  const int64_t beg = max<int64_t>(cu[b], 0), end = min<int64_t>(cu[b + 1], n);
  if (beg >= end) return;
  if (start_mask && start_mask[beg]) atomicSub(&tile_counts[beg / kTile], 1);
  // tiles whose first token 4096 k lies in [beg, end)
  for (int64_t k = (beg + kTile - 1) / kTile; k * kTile < end; ++k) tile_lo[k] = b;
  // tiles whose last token min(4096 (k + 1), n) - 1 lies in [beg, end)
  const int64_t n_tiles = (n + kTile - 1) / kTile;
  for (int64_t k = beg / kTile; k < n_tiles; ++k) {
    const int64_t last = min<int64_t>((k + 1) * kTile, n) - 1;
    if (last >= end) break;
    if (last >= beg) tile_hi[k] = b;
  }
}

// Document range [dlo, dhi] of tile t (clamped so that even offsets that
// break the preconditions stay in range).
__device__ __forceinline__ void tile_range(const int32_t* __restrict__ tile_lo,
                                           const int32_t* __restrict__ tile_hi, int32_t n_docs,
                                           int64_t t, int* dlo, int* dhi) {
  *dlo = min(max(tile_lo[t], 0), n_docs - 1);
  *dhi = min(max(tile_hi[t], *dlo), n_docs - 1);
}

// One wave per tile: the number of scored tokens of the tile.
template <bool kShifted, bool kC, bool kE>
__global__ void __launch_bounds__(kThreads)
count_kernel(RowMasks<kC, kE> mk, int64_t n, const int32_t* __restrict__ cu, int32_t n_docs,
             const int32_t* __restrict__ tile_lo, const int32_t* __restrict__ tile_hi,
             int64_t n_tiles, int32_t* __restrict__ tile_counts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= n_tiles) return;
  const int64_t t0 = t * kTile, t1 = min(t0 + kTile, n);
  int cnt = 0;
  if (t1 - t0 == kTile && mk.aligned16()) {
    uint4 f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = mk.flags16(t0 + 1024 * i + 16 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      cnt += __popc(f[i].x) + __popc(f[i].y) + __popc(f[i].z) + __popc(f[i].w);
  } else {
    for (int64_t g = t0 + lane; g < t1; g += 64) cnt += mk.at(g);
  }
  if (kShifted) {
    // a scored first token of a (non-empty) document has no row
    int dlo, dhi;
    tile_range(tile_lo, tile_hi, n_docs, t, &dlo, &dhi);
    for (int i = dlo + lane; i <= dhi; i += 64) {
      const int64_t beg = cu[i], end = cu[i + 1];
      if (beg < end && beg >= t0 && beg < t1 && mk.at(beg)) --cnt;
    }
  }
  cnt = wave_sum(cnt);
  // (negative only when the offsets break their preconditions)
  if (lane == 0) tile_counts[t] = max(cnt, 0);
}

// Example-mean weighting, pass 1: one wave per document counts its scored
// rows, 16 mask bytes per lane per load; bytes outside the document (or its
// first token, with shifted logits) are masked off.
template <bool kShifted, bool kC, bool kE>
__global__ void __launch_bounds__(kThreads)
doc_rows_kernel(RowMasks<kC, kE> mk, int64_t n, const int32_t* __restrict__ cu,
                int32_t n_docs, int32_t* __restrict__ doc_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (b >= n_docs) return;
  const int64_t lo = (int64_t)cu[b] + (kShifted ? 1 : 0);
  const int64_t hi = min<int64_t>(cu[b + 1], n);
  int cnt = 0;
  if (mk.aligned16()) {
    for (int64_t off = (lo & ~(int64_t)15) + 16 * lane; off < hi; off += 1024) {
      uint32_t f[4] = {0u, 0u, 0u, 0u};
      if (off + 16 <= n) {
        const uint4 v = mk.flags16(off);
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
      } else {
        for (int i = 0; i < 16 && off + i < n; ++i)
          f[i >> 2] |= (uint32_t)mk.at(off + i) << (8 * (i & 3));
      }
      // keep the bytes of [lo, hi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t base = off + 4 * q;
        const int s0 = (int)min<int64_t>(max<int64_t>(lo - base, 0), 4);
        const int s1 = (int)min<int64_t>(max<int64_t>(hi - base, 0), 4);
        const uint64_t keep = ((1ull << (8 * s1)) - 1) & ~((1ull << (8 * s0)) - 1);
        cnt += __popc(f[q] & (uint32_t)keep);
      }
    }
  } else {
    for (int64_t g = lo + lane; g < hi; g += 64) cnt += mk.at(g);
  }
  cnt = wave_sum(cnt);
  if (lane == 0) doc_rows[b] = cnt;
}

// Example-mean weighting, pass 2: the number of documents with a scored row.
__global__ void __launch_bounds__(1024)
examples_kernel(const int32_t* __restrict__ doc_rows, int32_t n_docs,
                int32_t* __restrict__ n_examples) {
  __shared__ int s_part[1024 / 64];
  int c = 0;
  for (int b = threadIdx.x; b < n_docs; b += 1024) c += doc_rows[b] > 0;
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < 1024 / 64; ++i) t += s_part[i];
    *n_examples = t;
  }
}

// Mean and example-mean weightings: every document's weight into a table
// (the mean's needs the total row count, summed from the group totals).
__global__ void __launch_bounds__(kThreads)
doc_weights_kernel(WeightArgs wa, int32_t n_docs, const int32_t* __restrict__ group_sums,
                   int32_t n_groups, float* __restrict__ w_doc) {
  __shared__ int s_total;
  if (threadIdx.x < 64) {
    int tot = 0;
    if (wa.mode == MDLM_WEIGHT_MEAN)
      for (int g = threadIdx.x; g < n_groups; g += 64) tot += group_sums[g];
    tot = wave_sum(tot);
    if (threadIdx.x == 0) s_total = tot;
  }
  __syncthreads();
  const int32_t n_examples = wa.mode == MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED ? *wa.n_examples : 0;
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b < n_docs) w_doc[b] = doc_weight(wa, b, s_total, n_examples);
}

// Per group of 1024 tiles: counts -> exclusive offsets within the group (in
// place) and the group's total.
__global__ void __launch_bounds__(kGroup)
group_scan_kernel(int32_t* __restrict__ tile_counts, int64_t n_tiles,
                  int32_t* __restrict__ group_sums) {
  __shared__ int s_wave[kGroup / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i = (int64_t)blockIdx.x * kGroup + tid;
  // (negative only when the offsets break their preconditions)
  const int v = i < n_tiles ? max(tile_counts[i], 0) : 0;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kGroup / 64; ++w) {
    const int x = s_wave[w];
    if (w < wave) before += x;
    total += x;
  }
  if (i < n_tiles) tile_counts[i] = before + incl - v;
  if (tid == 0) group_sums[blockIdx.x] = total;
}

// Per-token weights of the corrective mixture (kCode): a token's code byte
// picks the masked weight (the document's scale / (p_b N) with scale 1), the
// replaced weight (noise_wt / (p_b N)) or the clean weight (clean_wt / N).
struct CodeWeights {
  const uint8_t* codes;  // [n] codes 0 clean / 1 masked / 2 replaced
  double noise_wt;
  float clean_w;
};

// Scatter: four rounds per tile; in round j thread t owns the 4 consecutive
// tokens at 1024 j + 4 t, so every load is contiguous across the wave.
template <bool kShifted, bool kVec, bool kC, bool kE, bool kCode = false>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(const uint8_t* __restrict__ corrupted, const uint8_t* __restrict__ eligible,
               const int32_t* __restrict__ x0, int64_t n,
               const int32_t* __restrict__ cu, int32_t n_docs,
               const int32_t* __restrict__ tile_lo, const int32_t* __restrict__ tile_hi,
               const double* __restrict__ p_doc, double scale,
               const float* __restrict__ w_doc, const int32_t* __restrict__ tile_offsets,
               const int32_t* __restrict__ group_sums, int32_t n_groups,
               int32_t* __restrict__ row_idx, int32_t* __restrict__ tgt, float* __restrict__ w,
               int32_t* __restrict__ n_rows, CodeWeights cwt, bool single) {
  // the code-weight form holds a second weight table in the same LDS budget
  constexpr int kDocs = kCode ? kLdsDocs * 2 / 3 : kLdsDocs;
  __shared__ int32_t s_cu[kDocs + 1];
  __shared__ float s_wd[kDocs];
  __shared__ float s_wd2[kCode ? kDocs : 1];  // replaced-token weights
  __shared__ int s_wsum[kBufs][kWaves];
  __shared__ int32_t s_row[kBufs][kRoundTok];
  __shared__ int32_t s_tgt[kBufs][kRoundTok];
  __shared__ float s_w[kBufs][kRoundTok];
  __shared__ int s_base;

  // (the masks arrive as restrict-qualified parameters so that their loads
  // are known not to alias the row stores)
  const RowMasks<kC, kE> mk{corrupted, eligible};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTile;
  // `single`: the whole stream is this one tile, run without the count and
  // scan passes (every document, offset 0, and the row count written here)
  int dlo = 0, dhi = n_docs - 1;
  if (!single) tile_range(tile_lo, tile_hi, n_docs, tile, &dlo, &dhi);
  const int nd = dhi - dlo + 1;
  const bool cached = nd <= kDocs;
  // per-document weight: scale / (p_b N) computed here, or from the table
  // of the other weightings
  auto weight_of_doc = [&](int b) {
#pragma clang fp contract(off)
    return w_doc ? w_doc[b] : (float)(scale / (p_doc[b] * (double)n));
  };
  auto weight2_of_doc = [&](int b) {
#pragma clang fp contract(off)
    return (float)(cwt.noise_wt / (p_doc[b] * (double)n));
  };
  if (cached) {
    for (int i = tid; i <= nd; i += kThreads) s_cu[i] = cu[dlo + i];
    for (int i = tid; i < nd; i += kThreads) s_wd[i] = weight_of_doc(dlo + i);
    if (kCode)
      for (int i = tid; i < nd; i += kThreads) s_wd2[i] = weight2_of_doc(dlo + i);
  }
  // the weight of a selected token from its code and its document's weights
  auto by_code = [&](uint32_t code, float wm, float wr) {
    return code == 1u ? wm : code == 2u ? wr : cwt.clean_w;
  };
  const int grp = (int)(tile / kGroup);
  if (single) {
    if (tid == 0) s_base = 0;
  } else if (wave == 0) {
    // this tile's offset: its place in its group plus the groups before it
    int b = 0;
    for (int g = lane; g < grp; g += 64) b += group_sums[g];
    b = wave_sum(b);
    if (lane == 0) s_base = b + tile_offsets[tile];
  } else if (wave == 1 && tile == 0) {
    int tot = 0;
    for (int g = lane; g < n_groups; g += 64) tot += group_sums[g];
    tot = wave_sum(tot);
    if (lane == 0) *n_rows = tot;
  }
  __syncthreads();
  int64_t out = s_base;

  for (int j = 0; j < kTile / kRoundTok; ++j) {
    const int buf = j % kBufs;
    const int64_t g0 = t0 + (int64_t)kRoundTok * j + 4 * tid;
    const int64_t gw = t0 + (int64_t)kRoundTok * j + 256 * wave;
    uint32_t sel = 0;
    int32_t vals[4] = {0, 0, 0, 0};
    float wts[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t mv = 0;  // byte k nonzero iff token g0 + k is corrupted and eligible
    uint32_t cv = 0;  // (kCode) byte k: the code of token g0 + k
    const int cnt_here = g0 < n ? (int)min<int64_t>(4, n - g0) : 0;
    if (kVec && cnt_here == 4) {
      mv = mk.word(g0);
      if (kCode) cv = kC && !kE ? mv : *reinterpret_cast<const uint32_t*>(cwt.codes + g0);
      const int4 xv = *reinterpret_cast<const int4*>(x0 + g0);
      vals[0] = xv.x; vals[1] = xv.y; vals[2] = xv.z; vals[3] = xv.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < cnt_here) {
          mv |= (uint32_t)mk.at(g0 + k) << (8 * k);
          if (kCode) cv |= (uint32_t)cwt.codes[g0 + k] << (8 * k);
          vals[k] = x0[g0 + k];
        }
    }
    bool done = false;
    if (kVec && cached && gw + 256 <= n) {
      // wave-uniform: the round's 256 tokens of this wave touch local
      // documents dw .. dw + span
      const int dw = lds_find_doc(s_cu, nd, gw);
      const int span = lds_find_doc(s_cu, nd, gw + 255) - dw;
      if (span <= 3) {
        const int64_t b0 = s_cu[dw], b1 = s_cu[dw + 1];
        const int64_t b2 = span >= 2 ? (int64_t)s_cu[dw + 2] : INT64_MAX;
        const int64_t b3 = span >= 3 ? (int64_t)s_cu[dw + 3] : INT64_MAX;
        const float w0 = s_wd[dw], w1 = s_wd[dw + min(span, 1)];
        const float w2 = s_wd[dw + min(span, 2)], w3 = s_wd[dw + span];
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        if (kCode) {
          r0 = s_wd2[dw];
          r1 = s_wd2[dw + min(span, 1)];
          r2 = s_wd2[dw + min(span, 2)];
          r3 = s_wd2[dw + span];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t g = g0 + k;
          const int idx = (int)(g >= b1) + (int)(g >= b2) + (int)(g >= b3);
          const int64_t beg = idx == 0 ? b0 : idx == 1 ? b1 : idx == 2 ? b2 : b3;
          const float wk = idx == 0 ? w0 : idx == 1 ? w1 : idx == 2 ? w2 : w3;
          if (((mv >> (8 * k)) & 0xffu) && (!kShifted || g != beg)) {
            sel |= 1u << k;
            if (kCode) {
              const float rk = idx == 0 ? r0 : idx == 1 ? r1 : idx == 2 ? r2 : r3;
              wts[k] = by_code((cv >> (8 * k)) & 0xffu, wk, rk);
            } else {
              wts[k] = wk;
            }
          }
        }
        done = true;
      }
    }
    if (!done && mv != 0) {
      int d = cached ? lds_find_doc(s_cu, nd, g0) : find_doc(cu, dlo, dhi, g0) - dlo;
      const DocOffsets cu_at(s_cu, cu, dlo, n_docs, cached);  // cu[dlo + i]
      int64_t d_beg = cu_at[d];
      int64_t d_end = cu_at[d + 1];
      auto weight_of = [&](int dd) { return cached ? s_wd[dd] : weight_of_doc(dlo + dd); };
      auto weight2_of = [&](int dd) { return cached ? s_wd2[dd] : weight2_of_doc(dlo + dd); };
      float wd = weight_of(d);
      float wr = kCode ? weight2_of(d) : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t g = g0 + k;
        if (k < cnt_here && ((mv >> (8 * k)) & 0xffu)) {
          if (g >= d_end) {
            // (bounded by the last document even if cu_seqlens is malformed)
            do {
              ++d;
              d_end = cu_at[d + 1];
            } while (g >= d_end && d < nd - 1);
            d_beg = cu_at[d];
            wd = weight_of(d);
            if (kCode) wr = weight2_of(d);
          }
          if (!kShifted || g != d_beg) {
            sel |= 1u << k;
            wts[k] = kCode ? by_code((cv >> (8 * k)) & 0xffu, wd, wr) : wd;
          }
        }
      }
    }

    // rank: selected tokens of lower lanes in the wave, then lower waves
    int below = 0, wave_total = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t b = __ballot((sel >> k) & 1u);
      below += lanes_below(b);
      wave_total += __popcll(b);
    }
    if (lane == 0) s_wsum[buf][wave] = wave_total;
    __syncthreads();
    int pos = below, round_total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int v = s_wsum[buf][i];
      if (i < wave) pos += v;
      round_total += v;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (sel & (1u << k)) {
        const int64_t g = g0 + k;
        s_row[buf][pos] = (int32_t)(kShifted ? g - 1 : g);
        s_tgt[buf][pos] = vals[k];
        s_w[buf][pos] = wts[k];
        ++pos;
      }
    }
    __syncthreads();
    // (offsets that break their preconditions can misplace rows; the bounds
    // test keeps every store inside the n-entry row buffers regardless)
    for (int i = tid; i < round_total; i += kThreads) {
      const int64_t o = out + i;
      if (o < n) {
        row_idx[o] = s_row[buf][i];
        tgt[o] = s_tgt[buf][i];
        w[o] = s_w[buf][i];
      }
    }
    out += round_total;
    // with one buffer, the next round's staging must wait for this copy
    if (kBufs == 1) __syncthreads();
  }
  if (single && tid == 0) *n_rows = (int32_t)out;
}

}  // namespace

size_t compact_workspace_bytes(int64_t n_tokens, int32_t n_docs, int32_t weighting) {
  if (n_tokens <= 0) return 0;
  const int64_t tiles = (n_tokens + kTile - 1) / kTile;
  const int64_t groups = (tiles + kGroup - 1) / kGroup;
  // counts, first and last document per tile; one total per group; for the
  // example-mean weighting, scored rows per document and the example count
  size_t words = 3 * (size_t)tiles + (size_t)groups;
  if (weighting != MDLM_WEIGHT_INV_P) words += (size_t)std::max(n_docs, 0);  // weights
  if (weighting == MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED) words += (size_t)std::max(n_docs, 0) + 1;
  return words * sizeof(int32_t);
}

namespace {

struct Launch {
  int64_t n;
  const int32_t* cu;
  int32_t n_docs;
  int64_t tiles, groups;
  int32_t *counts, *tile_lo, *tile_hi, *group_sums, *doc_rows, *n_examples;
  float* w_doc;  // per-document weights (mean and example-mean weightings), else null
  const int32_t* x0;
  WeightArgs wa;
  int32_t *row_idx, *tgt;
  float* w;
  int32_t* n_rows;
  bool vec;
  hipStream_t stream;
  CodeWeights cwt;  // corrective mixture only
  bool single;      // one tile, per-document weights needing no totals: scatter alone
  bool counts_given;  // the tile counts are in place (from the corruption pass)
};

// The passes after tile_docs_kernel, for one combination of alignment and
// masks present.
template <bool kShifted, bool kC, bool kE, bool kCode = false>
void run_passes(const Launch& L, RowMasks<kC, kE> mk) {
  hipStream_t st = L.stream;
  if (L.single) {
    if (L.vec)
      scatter_kernel<kShifted, true, kC, kE, kCode><<<1, kThreads, 0, st>>>(
          mk.corrupted, mk.eligible, L.x0, L.n, L.cu, L.n_docs, nullptr, nullptr, L.wa.p_doc,
          L.wa.scale, nullptr, nullptr, nullptr, 0, L.row_idx, L.tgt, L.w, L.n_rows, L.cwt,
          true);
    else
      scatter_kernel<kShifted, false, kC, kE, kCode><<<1, kThreads, 0, st>>>(
          mk.corrupted, mk.eligible, L.x0, L.n, L.cu, L.n_docs, nullptr, nullptr, L.wa.p_doc,
          L.wa.scale, nullptr, nullptr, nullptr, 0, L.row_idx, L.tgt, L.w, L.n_rows, L.cwt,
          true);
    return;
  }
  if (L.wa.mode == MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED) {
    const unsigned g = (unsigned)((L.n_docs + kWaves - 1) / kWaves);
    doc_rows_kernel<kShifted, kC, kE><<<g, kThreads, 0, st>>>(mk, L.n, L.cu, L.n_docs,
                                                              L.doc_rows);
    examples_kernel<<<1, 1024, 0, st>>>(L.doc_rows, L.n_docs, L.n_examples);
  }
  if (!L.counts_given) {
    const unsigned count_grid = (unsigned)((L.tiles + kWaves - 1) / kWaves);
    count_kernel<kShifted, kC, kE><<<count_grid, kThreads, 0, st>>>(
        mk, L.n, L.cu, L.n_docs, L.tile_lo, L.tile_hi, L.tiles, L.counts);
  }
  group_scan_kernel<<<(unsigned)L.groups, kGroup, 0, st>>>(L.counts, L.tiles, L.group_sums);
  if (L.w_doc)
    doc_weights_kernel<<<(unsigned)((L.n_docs + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        L.wa, L.n_docs, L.group_sums, (int32_t)L.groups, L.w_doc);
  if (L.vec)
    scatter_kernel<kShifted, true, kC, kE, kCode><<<(unsigned)L.tiles, kThreads, 0, st>>>(
        mk.corrupted, mk.eligible, L.x0, L.n, L.cu, L.n_docs, L.tile_lo, L.tile_hi, L.wa.p_doc,
        L.wa.scale, L.w_doc,
        L.counts, L.group_sums, (int32_t)L.groups, L.row_idx, L.tgt, L.w, L.n_rows, L.cwt,
        false);
  else
    scatter_kernel<kShifted, false, kC, kE, kCode><<<(unsigned)L.tiles, kThreads, 0, st>>>(
        mk.corrupted, mk.eligible, L.x0, L.n, L.cu, L.n_docs, L.tile_lo, L.tile_hi, L.wa.p_doc,
        L.wa.scale, L.w_doc,
        L.counts, L.group_sums, (int32_t)L.groups, L.row_idx, L.tgt, L.w, L.n_rows, L.cwt,
        false);
}

}  // namespace

hipError_t launch_compact(const uint8_t* corrupted, const uint8_t* eligible, const int32_t* x0,
                          int64_t n, const int32_t* cu, int32_t n_docs, const double* p_doc,
                          int32_t align, int32_t weighting, double scale, double clip,
                          int32_t* row_idx, int32_t* tgt, float* w, int32_t* n_rows,
                          void* workspace, hipStream_t stream, bool counts_given) {
  if (n <= 0) {
    set_int_kernel<<<1, 1, 0, stream>>>(n_rows, 0);
    return hipGetLastError();
  }
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t groups = (tiles + kGroup - 1) / kGroup;
  int32_t* counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* tile_lo = counts + tiles;
  int32_t* tile_hi = tile_lo + tiles;
  int32_t* group_sums = tile_hi + tiles;
  WeightArgs wa{weighting, scale, clip, p_doc, n, nullptr, nullptr};
  // after the group totals: (mean, example mean) one weight per document;
  // (example mean) scored rows per document and the example count
  float* w_doc = nullptr;
  int32_t* doc_rows = nullptr;
  int32_t* n_examples = nullptr;
  if (weighting != MDLM_WEIGHT_INV_P) w_doc = reinterpret_cast<float*>(group_sums + groups);
  if (weighting == MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED) {
    doc_rows = reinterpret_cast<int32_t*>(w_doc + n_docs);
    n_examples = doc_rows + n_docs;
    wa.doc_rows = doc_rows;
    wa.n_examples = n_examples;
  }
  // a single tile with per-document weights needs none of the passes before
  // the scatter
  const bool single = tiles == 1 && weighting == MDLM_WEIGHT_INV_P;
  const bool shifted = align == MDLM_SHIFTED;
  // (given counts are of corrupted tokens: only with the mask alone)
  counts_given = counts_given && corrupted && !eligible;
  if (!single)
    tile_docs_kernel<<<(n_docs + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
        cu, n_docs, n, tile_lo, tile_hi, counts_given && shifted ? corrupted : nullptr, counts);
  const bool vec = ((uintptr_t)x0 % 16 == 0) && ((uintptr_t)corrupted % 4 == 0) &&
                   ((uintptr_t)eligible % 4 == 0);
  const Launch L{n,        cu,     n_docs, tiles,     groups, counts,    tile_lo,
                 tile_hi,  group_sums, doc_rows, n_examples, w_doc, x0, wa,
                 row_idx,  tgt,    w,      n_rows,    vec,    stream,    CodeWeights{},
                 single,   counts_given};
  const int key = (shifted ? 4 : 0) | (corrupted ? 2 : 0) | (eligible ? 1 : 0);
  switch (key) {
    case 0: run_passes<false, false, false>(L, {corrupted, eligible}); break;
    case 1: run_passes<false, false, true>(L, {corrupted, eligible}); break;
    case 2: run_passes<false, true, false>(L, {corrupted, eligible}); break;
    case 3: run_passes<false, true, true>(L, {corrupted, eligible}); break;
    case 4: run_passes<true, false, false>(L, {corrupted, eligible}); break;
    case 5: run_passes<true, false, true>(L, {corrupted, eligible}); break;
    case 6: run_passes<true, true, false>(L, {corrupted, eligible}); break;
    default: run_passes<true, true, true>(L, {corrupted, eligible}); break;
  }
  return hipGetLastError();
}

hipError_t launch_compact_corrective(const uint8_t* codes, const int32_t* x0, int64_t n,
                                     const int32_t* cu, int32_t n_docs, const double* p_doc,
                                     int32_t align, double noise_wt, double clean_wt,
                                     int32_t* row_idx, int32_t* tgt, float* w, int32_t* n_rows,
                                     void* workspace, hipStream_t stream) {
  if (n <= 0) {
    set_int_kernel<<<1, 1, 0, stream>>>(n_rows, 0);
    return hipGetLastError();
  }
  const int64_t tiles = (n + kTile - 1) / kTile;
  const int64_t groups = (tiles + kGroup - 1) / kGroup;
  int32_t* counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* tile_lo = counts + tiles;
  int32_t* tile_hi = tile_lo + tiles;
  int32_t* group_sums = tile_hi + tiles;
  // masked rows: the inverse-p weight with scale 1
  WeightArgs wa{MDLM_WEIGHT_INV_P, 1.0, 0.0, p_doc, n, nullptr, nullptr};
  const bool single = tiles == 1;
  if (!single)
    tile_docs_kernel<<<(n_docs + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
        cu, n_docs, n, tile_lo, tile_hi, nullptr, nullptr);
  const bool vec = ((uintptr_t)x0 % 16 == 0) && ((uintptr_t)codes % 4 == 0);
  const CodeWeights cwt{codes, noise_wt, (float)(clean_wt / (double)n)};
  const Launch L{n,        cu,     n_docs,  tiles,   groups, counts,  tile_lo,
                 tile_hi,  group_sums, nullptr, nullptr, nullptr, x0,  wa,
                 row_idx,  tgt,    w,       n_rows,  vec,    stream,  cwt,
                 single,   false};
  const bool shifted = align == MDLM_SHIFTED;
  // without clean rows the codes are the selection mask (nonzero: corrupted
  // either way); with them every token is a row
  const bool clean = clean_wt != 0.0;
  if (shifted) {
    if (clean) run_passes<true, false, false, true>(L, {nullptr, nullptr});
    else run_passes<true, true, false, true>(L, {codes, nullptr});
  } else {
    if (clean) run_passes<false, false, false, true>(L, {nullptr, nullptr});
    else run_passes<false, true, false, true>(L, {codes, nullptr});
  }
  return hipGetLastError();
}

// ---- the allocation-free variant of mdlm_compact_masked -------------------
// Its workspace is `scratch`, a file-scope device array sized for
// kNoAllocMaxTokens tokens; each device holds its own copy, whose address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and kept.  Host code passes that address, never the array's name (which is
// a host-side stand-in), to the kernels.  Nothing in it needs clearing: the
// passes write every word they later read.  Calls on one device share the
// array, so calls that overlap on one device race.
namespace {

constexpr int64_t kNoAllocTiles = (kNoAllocMaxTokens + kTile - 1) / kTile;
constexpr int64_t kNoAllocWords = 3 * kNoAllocTiles + (kNoAllocTiles + kGroup - 1) / kGroup;

__device__ __align__(256) int32_t scratch[kNoAllocWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // per device, once looked up

}  // namespace

static_assert(kNoAllocWords * sizeof(int32_t) ==
                  3 * kNoAllocTiles * sizeof(int32_t) +
                      ((kNoAllocTiles + kGroup - 1) / kGroup) * sizeof(int32_t),
              "scratch holds the inverse-p workspace of kNoAllocMaxTokens tokens");

hipError_t compact_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t compact_scratch_bytes() { return (size_t)kNoAllocWords * sizeof(int32_t); }

}  // namespace mdlm
