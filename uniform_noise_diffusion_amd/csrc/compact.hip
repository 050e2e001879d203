// Ordered stream compaction of the scored rows.
//
// Method: LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row (CE only
// on masked tokens, divided by p); Axolotl diffusion docs, model table
// (aligned vs shifted logits) and "Batching" (logits computed only at label
// slots).  Each scored token g of document b yields, in ascending g,
//   ALIGNED: (row g,   target x0[g], weight 1 / (p_b N))
//   SHIFTED: (row g-1, target x0[g], weight 1 / (p_b N)), skipping g = cu[b].
//
// One pass over the mask: a block takes a 4096-token tile (16 per thread),
// counts its scored tokens with wavefront ballots, publishes the count, and
// obtains its output offset by looking back over its predecessors' published
// counts and prefixes (Merrill & Garland, "Single-pass Parallel Prefix Scan
// with Decoupled Look-back", 2016).  Tiles are numbered by an atomic ticket
// taken at block start, so every tile a block waits on is already running.
// Rows are staged in LDS and written out with coalesced stores.
#include "mdlm_internal.h"

#include <algorithm>

namespace mdlm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTokPerThread = 16;
constexpr int kTile = kThreads * kTokPerThread;  // 4096 tokens

// Tile status word: two flag bits over a 62-bit count.
constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagPrefix = 2ull << 62;
constexpr uint64_t kValueMask = (1ull << 62) - 1;

// workspace: [0, 256) ticket counter, then one status word per tile
constexpr size_t kStatusOffset = 256;

__global__ void compact_init_kernel(uint64_t* __restrict__ ws, int64_t n_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (int64_t)gridDim.x * blockDim.x)
    ws[i] = 0;
}

__global__ void set_int_kernel(int32_t* p, int32_t v) { *p = v; }

template <bool kShifted>
__global__ void __launch_bounds__(kThreads)
compact_kernel(const uint8_t* __restrict__ corrupted, const int32_t* __restrict__ x0,
               int64_t n, const int32_t* __restrict__ cu, int32_t n_docs,
               const double* __restrict__ p_doc, int32_t* __restrict__ row_idx,
               int32_t* __restrict__ tgt, float* __restrict__ w,
               int32_t* __restrict__ n_rows, uint32_t* __restrict__ ticket,
               uint64_t* __restrict__ status, int64_t n_tiles) {
  __shared__ int s_tile, s_dlo, s_dhi;
  __shared__ int s_wave_sum[kWaves];
  __shared__ int64_t s_prefix;
  __shared__ int32_t s_row[kTile];
  __shared__ int32_t s_tgt[kTile];
  __shared__ float s_w[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_tile = (int)atomicAdd(ticket, 1u);
  __syncthreads();
  const int64_t tile = s_tile;
  const int64_t t0 = tile * kTile;
  const int64_t t1 = min(t0 + kTile, n);
  if (tid == 0) s_dlo = find_doc(cu, 0, n_docs - 1, t0);
  if (tid == 1) s_dhi = find_doc(cu, 0, n_docs - 1, t1 - 1);
  __syncthreads();

  // ---- this thread's 16 tokens: mask bits, targets, documents ------------
  const int64_t g0 = t0 + (int64_t)tid * kTokPerThread;
  uint32_t sel = 0;
  int32_t vals[kTokPerThread];
  float wts[kTokPerThread];
  if (g0 < n) {
    const int cnt_here = (int)min<int64_t>(kTokPerThread, n - g0);
    uint8_t m[kTokPerThread];
    if (cnt_here == kTokPerThread && ((uintptr_t)(corrupted + g0) % 16 == 0)) {
      const uint4 v = *reinterpret_cast<const uint4*>(corrupted + g0);
      const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < kTokPerThread; ++k) m[k] = (words[k >> 2] >> (8 * (k & 3))) & 0xff;
    } else {
#pragma unroll
      for (int k = 0; k < kTokPerThread; ++k) m[k] = k < cnt_here ? corrupted[g0 + k] : 0;
    }
    int d = find_doc(cu, s_dlo, s_dhi, g0);
    int64_t d_beg = cu[d], d_end = cu[d + 1];
    float wd = (float)(1.0 / (p_doc[d] * (double)n));
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) {
      const int64_t g = g0 + k;
      vals[k] = 0;
      wts[k] = 0.f;
      if (k < cnt_here && m[k]) {
        if (g >= d_end) {
          do { ++d; d_end = cu[d + 1]; } while (g >= d_end && d < n_docs - 1);
          d_beg = cu[d];
          wd = (float)(1.0 / (p_doc[d] * (double)n));
        }
        if (!kShifted || g != d_beg) {
          sel |= 1u << k;
          vals[k] = x0[g];
          wts[k] = wd;
        }
      }
    }
  }
  const int cnt = __popc(sel);

  // ---- block-exclusive scan of the per-thread counts ---------------------
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wave_sum[wave] = incl;
  __syncthreads();
  int wave_off = 0, tile_total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int s = s_wave_sum[i];
    if (i < wave) wave_off += s;
    tile_total += s;
  }
  const int excl = wave_off + incl - cnt;

  // ---- decoupled look-back for the tile's global offset ------------------
  if (tid == 0) {
    int64_t prefix = 0;
    if (tile == 0) {
      __hip_atomic_store(&status[0], kFlagPrefix | (uint64_t)tile_total, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(&status[tile], kFlagAggregate | (uint64_t)tile_total,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int64_t pred = tile - 1;
      while (true) {
        uint64_t s;
        do {
          s = __hip_atomic_load(&status[pred], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((s & ~kValueMask) == 0) __builtin_amdgcn_s_sleep(1);
        } while ((s & ~kValueMask) == 0);
        prefix += (int64_t)(s & kValueMask);
        if (s & kFlagPrefix) break;
        --pred;
      }
      __hip_atomic_store(&status[tile], kFlagPrefix | (uint64_t)(prefix + tile_total),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_prefix = prefix;
    if (tile == n_tiles - 1) *n_rows = (int32_t)(prefix + tile_total);
  }

  // ---- stage the tile's rows in LDS, then write them out coalesced -------
  {
    int pos = excl;
#pragma unroll
    for (int k = 0; k < kTokPerThread; ++k) {
      if (sel & (1u << k)) {
        const int64_t g = g0 + k;
        s_row[pos] = (int32_t)(kShifted ? g - 1 : g);
        s_tgt[pos] = vals[k];
        s_w[pos] = wts[k];
        ++pos;
      }
    }
  }
  __syncthreads();
  const int64_t base = s_prefix;
  for (int i = tid; i < tile_total; i += kThreads) {
    row_idx[base + i] = s_row[i];
    tgt[base + i] = s_tgt[i];
    w[base + i] = s_w[i];
  }
}

}  // namespace

size_t compact_workspace_bytes(int64_t n_tokens) {
  if (n_tokens <= 0) return 0;
  const int64_t tiles = (n_tokens + kTile - 1) / kTile;
  return kStatusOffset + (size_t)tiles * sizeof(uint64_t);
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
  uint64_t* ws = reinterpret_cast<uint64_t*>(workspace);
  const int64_t words = (int64_t)(kStatusOffset / sizeof(uint64_t)) + tiles;
  const unsigned init_grid = (unsigned)std::min<int64_t>((words + 255) / 256, 1024);
  compact_init_kernel<<<init_grid, 256, 0, stream>>>(ws, words);
  uint32_t* ticket = reinterpret_cast<uint32_t*>(ws);
  uint64_t* status = ws + kStatusOffset / sizeof(uint64_t);
  if (align == MDLM_SHIFTED)
    compact_kernel<true><<<(unsigned)tiles, kThreads, 0, stream>>>(
        corrupted, x0, n, cu, n_docs, p_doc, row_idx, tgt, w, n_rows, ticket, status, tiles);
  else
    compact_kernel<false><<<(unsigned)tiles, kThreads, 0, stream>>>(
        corrupted, x0, n, cu, n_docs, p_doc, row_idx, tgt, w, n_rows, ticket, status, tiles);
  return hipGetLastError();
}

}  // namespace mdlm
