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
//   2. count_kernel: each block counts the scored tokens of one tile (1 byte
//      per token read);
//   3. scan_kernel: one block turns the per-tile counts into exclusive
//      offsets in place and writes the total to n_rows;
//   4. scatter_kernel: each block re-reads its tile in four 1024-token rounds,
//      ranks each round's scored tokens with a block scan, stages (row,
//      target, weight) in LDS and writes them at its offset with coalesced
//      stores.
// A tile's document offsets are cached in LDS when it touches at most 2048
// documents.
#include "mdlm_internal.h"

#include <algorithm>

namespace mdlm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTokPerThread = 16;
constexpr int kTile = kThreads * kTokPerThread;  // 4096 tokens
constexpr int kLdsDocs = 2048;                   // documents cached per tile
constexpr int kScanThreads = 1024;

__global__ void set_int_kernel(int32_t* p, int32_t v) { *p = v; }

// The 16 mask bytes of this thread's tokens [g0, g0 + cnt).
__device__ __forceinline__ void load_mask(const uint8_t* __restrict__ corrupted, int64_t g0,
                                          int cnt, uint8_t (&m)[kTokPerThread]) {
  if (cnt == kTokPerThread && ((uintptr_t)(corrupted + g0) % 16 == 0)) {
    const uint4 v = *reinterpret_cast<const uint4*>(corrupted + g0);
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) m[k] = (words[k >> 2] >> (8 * (k & 3))) & 0xff;
  } else {
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) m[k] = k < cnt ? corrupted[g0 + k] : 0;
  }
}

// For each tile k, the documents holding its first token (tile_lo[k]) and its
// last token (tile_hi[k]).  A non-empty document holds exactly the tokens
// [cu[b], cu[b+1]), so each tile boundary token has exactly one writer.
__global__ void __launch_bounds__(kThreads)
tile_docs_kernel(const int32_t* __restrict__ cu, int32_t n_docs, int64_t n,
                 int32_t* __restrict__ tile_lo, int32_t* __restrict__ tile_hi) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= n_docs) return;
  const int64_t beg = cu[b], end = min<int64_t>(cu[b + 1], n);
  if (beg >= end) return;
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

// Loads the tile's document range and caches the documents' offsets in s_cu
// when there are at most kLdsDocs of them.  Returns whether they were cached.
// Contains one barrier.
__device__ __forceinline__ bool tile_docs(const int32_t* __restrict__ cu, int32_t n_docs,
                                          const int32_t* __restrict__ tile_lo,
                                          const int32_t* __restrict__ tile_hi, int* dlo_out,
                                          int* dhi_out, int32_t* s_cu) {
  // (clamped so that even offsets that break the preconditions stay in range)
  const int dlo = min(max(tile_lo[blockIdx.x], 0), n_docs - 1);
  const int dhi = min(max(tile_hi[blockIdx.x], dlo), n_docs - 1);
  const int nd = dhi - dlo + 1;
  const bool cached = nd <= kLdsDocs;
  if (cached)
    for (int i = threadIdx.x; i <= nd; i += kThreads) s_cu[i] = cu[dlo + i];
  __syncthreads();
  *dlo_out = dlo;
  *dhi_out = dhi;
  return cached;
}

template <bool kShifted>
__global__ void __launch_bounds__(kThreads)
count_kernel(const uint8_t* __restrict__ corrupted, int64_t n, const int32_t* __restrict__ cu,
             int32_t n_docs, const int32_t* __restrict__ tile_lo, const int32_t* __restrict__ tile_hi,
             int32_t* __restrict__ tile_counts) {
  __shared__ int32_t s_cu[kLdsDocs + 1];
  __shared__ int s_sum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTile;
  const int64_t t1 = min(t0 + kTile, n);
  const int64_t g0 = t0 + (int64_t)tid * kTokPerThread;
  int cnt = 0;
  if (g0 < n) {
    uint8_t m[kTokPerThread];
    load_mask(corrupted, g0, (int)min<int64_t>(kTokPerThread, n - g0), m);
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) cnt += m[k] != 0;
  }
  if (kShifted) {
    // a corrupted first token of a (non-empty) document is not scored
    int dlo, dhi;
    const bool cached = tile_docs(cu, n_docs, tile_lo, tile_hi, &dlo, &dhi, s_cu);
    const int nd = dhi - dlo + 1;
    for (int i = tid; i < nd; i += kThreads) {
      const int64_t beg = cached ? s_cu[i] : cu[dlo + i];
      const int64_t end = cached ? s_cu[i + 1] : cu[dlo + i + 1];
      if (beg < end && beg >= t0 && beg < t1 && corrupted[beg]) --cnt;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if (lane == 0) s_sum[wave] = cnt;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int i = 0; i < kWaves; ++i) t += s_sum[i];
    tile_counts[blockIdx.x] = t;
  }
}

// Exclusive scan of the per-tile counts in place (one block; each thread
// takes a run of consecutive counts per pass), total -> n_rows.
constexpr int kScanRun = 32;
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(int32_t* __restrict__ tile_counts, int64_t n_tiles, int32_t* __restrict__ n_rows) {
  __shared__ int64_t s_wave[kScanThreads / 64];
  __shared__ int64_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < n_tiles; base += (int64_t)kScanThreads * kScanRun) {
    const int64_t i0 = base + (int64_t)tid * kScanRun;
    int32_t v[kScanRun];
    int64_t run = 0;
#pragma unroll
    for (int k = 0; k < kScanRun; ++k) {
      v[k] = i0 + k < n_tiles ? tile_counts[i0 + k] : 0;
      run += v[k];
    }
    int64_t incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int64_t before = s_carry, total = 0;
    for (int wv = 0; wv < kScanThreads / 64; ++wv) {
      if (wv < wave) before += s_wave[wv];
      total += s_wave[wv];
    }
    int64_t acc = before + incl - run;
#pragma unroll
    for (int k = 0; k < kScanRun; ++k) {
      if (i0 + k < n_tiles) tile_counts[i0 + k] = (int32_t)acc;
      acc += v[k];
    }
    __syncthreads();
    if (tid == 0) s_carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_rows = (int32_t)s_carry;
}

// Scatter: four rounds per tile; in round j thread t owns the 4 consecutive
// tokens at 1024 j + 4 t, so every load is contiguous across the wave.  Each
// round ranks its scored tokens with a block scan, stages them in LDS and
// writes them at the tile offset plus the rounds before it.
constexpr int kRoundTok = kThreads * 4;  // 1024
template <bool kShifted, bool kVec>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(const uint8_t* __restrict__ corrupted, const int32_t* __restrict__ x0, int64_t n,
               const int32_t* __restrict__ cu, int32_t n_docs,
               const int32_t* __restrict__ tile_lo, const int32_t* __restrict__ tile_hi,
               const double* __restrict__ p_doc,
               const int32_t* __restrict__ tile_offsets, int32_t* __restrict__ row_idx,
               int32_t* __restrict__ tgt, float* __restrict__ w) {
  __shared__ int s_wave_sum[kWaves];
  __shared__ int32_t s_cu[kLdsDocs + 1];
  __shared__ int32_t s_row[kRoundTok];
  __shared__ int32_t s_tgt[kRoundTok];
  __shared__ float s_w[kRoundTok];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTile;
  int dlo, dhi;
  const bool cached = tile_docs(cu, n_docs, tile_lo, tile_hi, &dlo, &dhi, s_cu);
  const int nd = dhi - dlo + 1;
  int64_t out = tile_offsets[blockIdx.x];

  for (int j = 0; j < kTile / kRoundTok; ++j) {
    const int64_t g0 = t0 + (int64_t)kRoundTok * j + 4 * tid;
    uint32_t sel = 0;
    int32_t vals[4] = {0, 0, 0, 0};
    float wts[4] = {0.f, 0.f, 0.f, 0.f};
    if (g0 < n) {
      const int cnt_here = (int)min<int64_t>(4, n - g0);
      uint8_t m[4];
      if (kVec && cnt_here == 4) {
        const uint32_t mv = *reinterpret_cast<const uint32_t*>(corrupted + g0);
        const int4 xv = *reinterpret_cast<const int4*>(x0 + g0);
#pragma unroll
        for (int k = 0; k < 4; ++k) m[k] = (mv >> (8 * k)) & 0xff;
        vals[0] = xv.x; vals[1] = xv.y; vals[2] = xv.z; vals[3] = xv.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          m[k] = k < cnt_here ? corrupted[g0 + k] : 0;
          vals[k] = k < cnt_here ? x0[g0 + k] : 0;
        }
      }
      if (m[0] | m[1] | m[2] | m[3]) {
        int d = cached ? lds_find_doc(s_cu, nd, g0) : find_doc(cu, dlo, dhi, g0) - dlo;
        int64_t d_beg = cached ? s_cu[d] : cu[dlo + d];
        int64_t d_end = cached ? s_cu[d + 1] : cu[dlo + d + 1];
        float wd = (float)(1.0 / (p_doc[dlo + d] * (double)n));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t g = g0 + k;
          if (k < cnt_here && m[k]) {
            if (g >= d_end) {
              // (bounded by the last document even if cu_seqlens is malformed)
              do {
                ++d;
                d_end = cached ? s_cu[d + 1] : cu[dlo + d + 1];
              } while (g >= d_end && d < nd - 1);
              d_beg = cached ? s_cu[d] : cu[dlo + d];
              wd = (float)(1.0 / (p_doc[dlo + d] * (double)n));
            }
            if (!kShifted || g != d_beg) {
              sel |= 1u << k;
              wts[k] = wd;
            }
          }
        }
      }
    }
    const int cnt = __popc(sel);

    // block-exclusive scan of the per-thread counts
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave_sum[wave] = incl;
    __syncthreads();
    int wave_off = 0, round_total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int v = s_wave_sum[i];
      if (i < wave) wave_off += v;
      round_total += v;
    }
    int pos = wave_off + incl - cnt;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (sel & (1u << k)) {
        const int64_t g = g0 + k;
        s_row[pos] = (int32_t)(kShifted ? g - 1 : g);
        s_tgt[pos] = vals[k];
        s_w[pos] = wts[k];
        ++pos;
      }
    }
    __syncthreads();
    for (int i = tid; i < round_total; i += kThreads) {
      row_idx[out + i] = s_row[i];
      tgt[out + i] = s_tgt[i];
      w[out + i] = s_w[i];
    }
    out += round_total;
    __syncthreads();  // staging and wave sums are reused by the next round
  }
}

}  // namespace

size_t compact_workspace_bytes(int64_t n_tokens) {
  if (n_tokens <= 0) return 0;
  const int64_t tiles = (n_tokens + kTile - 1) / kTile;
  return 3 * (size_t)tiles * sizeof(int32_t);  // counts, first and last document
}

hipError_t launch_compact(const uint8_t* corrupted, const int32_t* x0, int64_t n,
                          const int32_t* cu, int32_t n_docs, const double* p_doc,
                          int32_t align, int32_t* row_idx, int32_t* tgt, float* w,
                          int32_t* n_rows, void* workspace, hipStream_t stream) {
  if (n <= 0) {
    set_int_kernel<<<1, 1, 0, stream>>>(n_rows, 0);
    return hipGetLastError();
  }
  const int64_t tiles = (n + kTile - 1) / kTile;
  int32_t* counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* tile_lo = counts + tiles;
  int32_t* tile_hi = tile_lo + tiles;
  const unsigned grid = (unsigned)tiles;
  tile_docs_kernel<<<(n_docs + kThreads - 1) / kThreads, kThreads, 0, stream>>>(cu, n_docs, n,
                                                                                tile_lo, tile_hi);
  const bool vec = ((uintptr_t)x0 % 16 == 0) && ((uintptr_t)corrupted % 4 == 0);
  if (align == MDLM_SHIFTED) {
    count_kernel<true><<<grid, kThreads, 0, stream>>>(corrupted, n, cu, n_docs, tile_lo, tile_hi,
                                                      counts);
    scan_kernel<<<1, kScanThreads, 0, stream>>>(counts, tiles, n_rows);
    if (vec)
      scatter_kernel<true, true><<<grid, kThreads, 0, stream>>>(
          corrupted, x0, n, cu, n_docs, tile_lo, tile_hi, p_doc, counts, row_idx, tgt, w);
    else
      scatter_kernel<true, false><<<grid, kThreads, 0, stream>>>(
          corrupted, x0, n, cu, n_docs, tile_lo, tile_hi, p_doc, counts, row_idx, tgt, w);
  } else {
    count_kernel<false><<<grid, kThreads, 0, stream>>>(corrupted, n, cu, n_docs, tile_lo,
                                                       tile_hi, counts);
    scan_kernel<<<1, kScanThreads, 0, stream>>>(counts, tiles, n_rows);
    if (vec)
      scatter_kernel<false, true><<<grid, kThreads, 0, stream>>>(
          corrupted, x0, n, cu, n_docs, tile_lo, tile_hi, p_doc, counts, row_idx, tgt, w);
    else
      scatter_kernel<false, false><<<grid, kThreads, 0, stream>>>(
          corrupted, x0, n, cu, n_docs, tile_lo, tile_hi, p_doc, counts, row_idx, tgt, w);
  }
  return hipGetLastError();
}

}  // namespace mdlm
