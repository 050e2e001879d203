// Corruption and the scored-row list in one pass over the tokens.
//
// Method: LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row (one
// t ~ U(0,1) for each sequence, masking probability p = (1 - 1e-3) t + 1e-3,
// the CE of each masked token scaled by 1/p); diffusiongemma card,
// "Finetuning notes" (uniformly drawn ids, each example with its own rate);
// Axolotl diffusion docs, model table (aligned vs shifted logits) and
// "Packed training" (documents stay isolated).  The outputs are exactly
// those of corruption followed by compaction with inverse-p weights: the
// same Philox words decide the same tokens, and the rows come out in
// ascending token order with the same targets and fp32 weights.
//
// The separate calls read the tokens twice and the corruption mask once more
// (about 19 bytes of traffic per token at a masked share of one half); here
// each 4096-token tile is visited once: its tokens are read, corrupted and
// written back, and its scored rows are written straight to their place in
// the list -- 9 bytes per token plus 12 per scored row, 15 at one half.
// A tile's place in the list is the number of scored rows in all tiles
// before it, found by a decoupled look-back (Merrill and Garland, "Single-
// pass Parallel Prefix Scan with Decoupled Look-back", 2016): each tile
// publishes its own row count as soon as it has it, then sums its
// predecessors' published counts back to the nearest one whose inclusive
// total is already known, and publishes its own inclusive total.  Tiles are
// handed out in order by an atomic ticket, so every tile a block waits on
// belongs to a block that is already running; a running block publishes its
// count without waiting on anyone, so every wait ends.  The descriptors are
// single 64-bit words (state in the high half, count in the low half) read
// and written with device-scope atomics, which keep them coherent across the
// chip's L2 caches without fences.
//
// Passes: prep_kernel (per document: p_b, a zero count, and the first and
// last document of each tile it bounds; per tile: a cleared descriptor; the
// ticket cleared), then fused_kernel.  A stream of one tile runs one block
// of fused_kernel alone, which draws the noise levels itself.
#include "mdlm_internal.h"

#include <algorithm>

namespace mdlm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRounds = 4;
constexpr int kRoundTok = kThreads * 4;          // 1024 tokens per round
constexpr int kTile = kRoundTok * kRounds;       // 4096 tokens per tile
constexpr int kLdsDocs = 512;                    // documents cached per tile
// Look-back waits are bounded (a correct launch never comes near): past the
// bound a tile writes no rows and sets the call's row count to -1.
constexpr uint32_t kSpinLimit = 1u << 20;
// The row count before the last tile sets it (multi-tile streams): the last
// tile replaces it by compare-and-swap, a tile whose wait expired by -1 with
// an exchange, so -1 stands whichever comes first.
constexpr int32_t kRowsUnset = INT32_MIN;

// descriptor states (high 32 bits)
constexpr uint64_t kNotReady = 0, kAggregate = 1, kInclusive = 2;

__device__ __forceinline__ uint64_t desc_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void desc_store(uint64_t* p, uint64_t state, uint32_t count) {
  __hip_atomic_store(p, (state << 32) | count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// p_b = eps + (1 - eps) t_b for document b, t_b from its Philox word (the
// order of corruption's noise levels: (1 - eps), times t, plus eps).
__device__ __forceinline__ double doc_p(int b, uint32_t k0, uint32_t k1, double eps) {
#pragma clang fp contract(off)
  const uint4 r = philox4x32_10(make_uint4((uint32_t)b, 0u, 0u, kTagDocT), k0, k1);
  const double t = (double)(r.x >> 8) * 0x1p-24;
  const double one_minus_eps = 1.0 - eps;
  const double scaled = one_minus_eps * t;
  return eps + scaled;
}

__device__ __forceinline__ uint32_t threshold_of(double p) {
  return (uint32_t)ceil(p * 16777216.0);  // ceil(p 2^24), exact
}

__device__ __forceinline__ float weight_of(double p, int64_t n) {
#pragma clang fp contract(off)
  return (float)(1.0 / (p * (double)n));
}

__device__ __forceinline__ int lanes_below(uint64_t b) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

struct Ws {
  uint64_t* desc;     // [tiles]
  int32_t* tile_lo;   // [tiles] first document of each tile
  int32_t* tile_hi;   // [tiles] last document
  uint32_t* ticket;   // [1]
};

// Per document: p_b, cleared count, and the tile bounds (a non-empty
// document writes the tiles whose first or last token it holds; offsets
// outside [0, n] are clipped so that every write stays in the tables).  Per
// tile: a cleared descriptor.  Thread 0 clears the ticket and sets the row
// count to kRowsUnset (with no tiles, to 0).
__global__ void __launch_bounds__(kThreads)
prep_kernel(int32_t n_docs, int64_t n, int64_t tiles, uint32_t k0, uint32_t k1, double eps,
            const int32_t* __restrict__ cu, double* __restrict__ p_doc,
            int32_t* __restrict__ doc_counts, int32_t* __restrict__ n_rows, Ws ws) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i == 0) {
    *n_rows = tiles > 0 ? kRowsUnset : 0;
    if (tiles > 0) *ws.ticket = 0;
  }
  if (i < tiles) ws.desc[i] = 0;
  if (i >= n_docs) return;
  const int b = (int)i;
  p_doc[b] = doc_p(b, k0, k1, eps);
  doc_counts[b] = 0;
  const int64_t beg = max<int64_t>(cu[b], 0), end = min<int64_t>(cu[b + 1], n);
  if (beg >= end) return;
  for (int64_t k = (beg + kTile - 1) / kTile; k * kTile < end; ++k) ws.tile_lo[k] = b;
  for (int64_t k = beg / kTile; k < tiles; ++k) {
    const int64_t last = min<int64_t>((k + 1) * kTile, n) - 1;
    if (last >= end) break;
    if (last >= beg) ws.tile_hi[k] = b;
  }
}

struct Args {
  const int32_t* x0;
  int64_t n;
  const int32_t* cu;
  int32_t n_docs;
  uint32_t k0, k1;
  double eps;
  int32_t mask_id;
  uint32_t rand_vocab;
  int32_t* xt;
  uint8_t* corrupted;  // nullable
  double* p_doc;
  int32_t* doc_counts;
  int32_t* row_idx;
  int32_t* tgt;
  float* w;
  int32_t* n_rows;
  Ws ws;
  int64_t tiles;
  bool single;  // the whole stream is one tile: no prep pass, no look-back
};

// One block per 4096-token tile, four rounds of 1024 tokens; in round j
// thread t owns the 4 consecutive tokens at 1024 j + 4 t (one Philox call
// per stream), so loads and stores are contiguous across each wave.
template <int kNoise, bool kShifted, bool kVec>
__global__ void __launch_bounds__(kThreads) fused_kernel(Args a) {
  __shared__ int32_t s_cu[kLdsDocs + 1];
  __shared__ uint32_t s_thr[kLdsDocs];
  __shared__ float s_wd[kLdsDocs];
  __shared__ int s_cnt[kLdsDocs];
  __shared__ int s_wsum[kRounds][kWaves];
  __shared__ int32_t s_row[kRoundTok];
  __shared__ int32_t s_tgt[kRoundTok];
  __shared__ float s_w[kRoundTok];
  __shared__ int64_t s_tile;
  __shared__ int s_dlo, s_dhi;
  __shared__ int64_t s_base;
  __shared__ int64_t s_lb_part[kWaves];
  __shared__ bool s_lb_inc[kWaves], s_lb_timeout[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    const int64_t t = a.single ? 0 : (int64_t)atomicAdd(a.ws.ticket, 1u);
    s_tile = t;
    if (a.single) {
      s_dlo = 0;
      s_dhi = a.n_docs - 1;
    } else {
      const int lo = min(max(a.ws.tile_lo[t], 0), a.n_docs - 1);
      s_dlo = lo;
      s_dhi = min(max(a.ws.tile_hi[t], lo), a.n_docs - 1);
    }
  }
  __syncthreads();
  const int64_t tile = s_tile;
  const int64_t t0 = tile * kTile, t1 = min(t0 + kTile, a.n);
  const bool full = kVec && t1 - t0 == kTile;
  // the tile's tokens first, so that they are in flight while the tables fill
  int4 v[kRounds];
  if (full) {
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
      v[j] = *reinterpret_cast<const int4*>(a.x0 + t0 + kRoundTok * j + 4 * tid);
  }
  const int dlo = s_dlo, nd = s_dhi - s_dlo + 1;
  const bool cached = nd <= kLdsDocs;
  if (cached) {
    for (int i = tid; i <= nd; i += kThreads) s_cu[i] = a.cu[dlo + i];
    for (int i = tid; i < nd; i += kThreads) {
      double p;
      if (a.single) {
        p = doc_p(dlo + i, a.k0, a.k1, a.eps);
        a.p_doc[dlo + i] = p;
        a.doc_counts[dlo + i] = 0;
      } else {
        p = a.p_doc[dlo + i];
      }
      s_thr[i] = threshold_of(p);
      s_wd[i] = weight_of(p, a.n);
      s_cnt[i] = 0;
    }
  } else if (a.single) {
    for (int b = tid; b < a.n_docs; b += kThreads) {
      a.p_doc[b] = doc_p(b, a.k0, a.k1, a.eps);
      a.doc_counts[b] = 0;
    }
  }
  __syncthreads();

  // ---- pass over the tile: corrupt, count, rank --------------------------
  uint32_t sel_all = 0;  // bit 4 j + k: token 4 t + k of round j is scored
  int below[kRounds];    // scored tokens of lower lanes of this wave, per round
  float wts[kRounds][4];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t g0 = t0 + kRoundTok * j + 4 * tid;
    const int cnt_here = g0 < t1 ? (int)min<int64_t>(4, t1 - g0) : 0;
    int32_t in[4] = {0, 0, 0, 0};
    if (full) {
      in[0] = v[j].x; in[1] = v[j].y; in[2] = v[j].z; in[3] = v[j].w;
    } else if (kVec && cnt_here == 4) {
      const int4 x = *reinterpret_cast<const int4*>(a.x0 + g0);
      in[0] = x.x; in[1] = x.y; in[2] = x.z; in[3] = x.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < cnt_here) in[k] = a.x0[g0 + k];
    }
    // each token's document: local index, start, threshold and weight
    int dl[4] = {-1, -1, -1, -1};
    uint32_t thr[4] = {0, 0, 0, 0};
    float wd[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t beg[4] = {0, 0, 0, 0};
    if (cnt_here > 0) {
      int d = cached ? lds_find_doc(s_cu, nd, g0) : find_doc(a.cu, dlo, dlo + nd - 1, g0) - dlo;
      int64_t d_beg = cached ? s_cu[d] : a.cu[dlo + d];
      int64_t d_end = cached ? s_cu[d + 1] : a.cu[dlo + d + 1];
      auto load_doc = [&](int dd, uint32_t* th, float* ww) {
        if (cached) {
          *th = s_thr[dd];
          *ww = s_wd[dd];
        } else {
          // (a one-tile stream draws its noise levels in this launch: taken
          // again here rather than read back from other threads' stores)
          const double p = a.single ? doc_p(dlo + dd, a.k0, a.k1, a.eps) : a.p_doc[dlo + dd];
          *th = threshold_of(p);
          *ww = weight_of(p, a.n);
        }
      };
      uint32_t th;
      float ww;
      load_doc(d, &th, &ww);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t g = g0 + k;
        if (k < cnt_here) {
          if (g >= d_end) {
            // (bounded by the tile's last document even if the offsets are
            // malformed)
            do {
              ++d;
              d_end = cached ? s_cu[d + 1] : a.cu[dlo + d + 1];
            } while (g >= d_end && d < nd - 1);
            d_beg = cached ? s_cu[d] : a.cu[dlo + d];
            load_doc(d, &th, &ww);
          }
          dl[k] = d;
          thr[k] = th;
          wd[k] = ww;
          beg[k] = d_beg;
        }
      }
    }
    // the Bernoulli words (and the replacement words under uniform noise)
    const uint64_t q = (uint64_t)g0 >> 2;
    uint32_t w1[4] = {0, 0, 0, 0}, w2[4] = {0, 0, 0, 0};
    if (cnt_here > 0) {
      const uint4 r1 = philox4x32_10(
          make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagBernoulli), a.k0, a.k1);
      w1[0] = r1.x; w1[1] = r1.y; w1[2] = r1.z; w1[3] = r1.w;
      if (kNoise == MDLM_NOISE_UNIFORM) {
        const uint4 r2 = philox4x32_10(
            make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, kTagReplace), a.k0, a.k1);
        w2[0] = r2.x; w2[1] = r2.y; w2[2] = r2.z; w2[3] = r2.w;
      }
    }
    int32_t out[4];
    uint32_t mbits = 0, sel = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool c = k < cnt_here && (w1[k] >> 8) < thr[k];
      out[k] = c ? (kNoise == MDLM_NOISE_UNIFORM
                        ? (int32_t)(((uint64_t)w2[k] * a.rand_vocab) >> 32)
                        : a.mask_id)
                 : in[k];
      mbits |= (uint32_t)c << (8 * k);
      if (c && (!kShifted || g0 + k != beg[k])) sel |= 1u << k;
      wts[j][k] = wd[k];
    }
    if (kVec && cnt_here == 4) {
      *reinterpret_cast<int4*>(a.xt + g0) = make_int4(out[0], out[1], out[2], out[3]);
      if (a.corrupted) *reinterpret_cast<uint32_t*>(a.corrupted + g0) = mbits;
    } else {
      for (int k = 0; k < cnt_here; ++k) {
        a.xt[g0 + k] = out[k];
        if (a.corrupted) a.corrupted[g0 + k] = (uint8_t)((mbits >> (8 * k)) & 1u);
      }
    }
    // corrupted counts per document: the wave's tokens lie in documents
    // d_first .. d_last (rising with the lane); the first and last are summed
    // across the wave, any between them (short documents) added per lane
    {
      const uint64_t act = __ballot(cnt_here > 0);
      if (act != 0) {
        int last_local = -1;
#pragma unroll
        for (int k = 0; k < 4; ++k) last_local = max(last_local, dl[k]);
        const int d_first = __shfl(dl[0], 0, 64);
        const int d_last = __shfl(last_local, 63 - __clzll((long long)act), 64);
        int c_first = 0, c_last = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int bit = (mbits >> (8 * k)) & 1;
          if (dl[k] == d_first) c_first += bit;
          else if (dl[k] == d_last) c_last += bit;
          else if (dl[k] >= 0 && bit) {
            if (cached) atomicAdd(&s_cnt[dl[k]], 1);
            else atomicAdd(&a.doc_counts[dlo + dl[k]], 1);
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          c_first += __shfl_xor(c_first, off, 64);
          c_last += __shfl_xor(c_last, off, 64);
        }
        if (lane == 0) {
          if (c_first) {
            if (cached) atomicAdd(&s_cnt[d_first], c_first);
            else atomicAdd(&a.doc_counts[dlo + d_first], c_first);
          }
          if (c_last && d_last != d_first) {
            if (cached) atomicAdd(&s_cnt[d_last], c_last);
            else atomicAdd(&a.doc_counts[dlo + d_last], c_last);
          }
        }
      }
    }
    // ranks of this round's scored tokens within the wave
    int bl = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t b = __ballot((sel >> k) & 1u);
      bl += lanes_below(b);
      tot += __popcll(b);
    }
    below[j] = bl;
    if (lane == 0) s_wsum[j][wave] = tot;
    sel_all |= sel << (4 * j);
  }
  __syncthreads();
  // the tile's per-document counts, and its row total
  if (cached)
    for (int i = tid; i < nd; i += kThreads)
      if (s_cnt[i]) atomicAdd(&a.doc_counts[dlo + i], s_cnt[i]);
  int total = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j)
#pragma unroll
    for (int i = 0; i < kWaves; ++i) total += s_wsum[j][i];

  // ---- the tile's place in the row list ----------------------------------
  if (a.single) {
    if (tid == 0) {
      s_base = 0;
      *a.n_rows = total;
    }
  } else if (tile == 0) {
    if (tid == 0) {
      desc_store(&a.ws.desc[0], kInclusive, (uint32_t)total);
      s_base = 0;
      if (a.tiles == 1) atomicCAS(a.n_rows, kRowsUnset, total);
    }
  } else {
    // Every wave takes part: one round trip reads the 256 descriptors
    // before the tile (wave w, lane l: tile j - 64 w - l), which bounds how
    // far behind the inclusive totals can fall when tiles arrive fast.
    if (tid == 0) desc_store(&a.ws.desc[tile], kAggregate, (uint32_t)total);
    int64_t base = 0;
    int64_t j = tile - 1;
    uint32_t spins = 0;
    while (true) {
      const int64_t idx = j - (64 * wave + lane);
      uint64_t d = idx >= 0 ? desc_load(&a.ws.desc[idx]) : (kInclusive << 32);
      bool timed_out = false;
      while (__ballot((d >> 32) == kNotReady) != 0) {
        if (++spins > kSpinLimit) {
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        if ((d >> 32) == kNotReady) d = desc_load(&a.ws.desc[idx]);
      }
      // this wave's nearest inclusive total (lowest lane), and its counts up
      // to it (all 64 without one)
      const uint64_t inc = __ballot((d >> 32) == kInclusive);
      const int stop = inc ? __ffsll((unsigned long long)inc) - 1 : 63;
      int64_t part = lane <= stop ? (int64_t)(uint32_t)d : 0;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
      if (lane == 0) {
        s_lb_part[wave] = part;
        s_lb_inc[wave] = inc != 0;
        s_lb_timeout[wave] = timed_out;
      }
      __syncthreads();
      bool any_timeout = false, found = false;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        any_timeout = any_timeout || s_lb_timeout[w];
        if (!found) {
          base += s_lb_part[w];
          found = s_lb_inc[w];
        }
      }
      __syncthreads();  // (the slots are rewritten by the next window)
      if (any_timeout) {
        if (tid == 0) {
          // a tile whose wait expired writes no rows (s_base past the list)
          // and marks the call's row count
          desc_store(&a.ws.desc[tile], kInclusive, (uint32_t)total);
          s_base = a.n;
          atomicExch(a.n_rows, -1);
        }
        break;
      }
      if (found) {
        if (tid == 0) {
          desc_store(&a.ws.desc[tile], kInclusive, (uint32_t)(base + total));
          s_base = base;
          if (tile == a.tiles - 1) atomicCAS(a.n_rows, kRowsUnset, (int32_t)(base + total));
        }
        break;
      }
      j -= 64 * kWaves;
    }
  }
  __syncthreads();
  int64_t out_pos = s_base;

  // ---- the rows, round by round, staged for coalesced stores ------------
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    int pos = below[j], round_total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int c = s_wsum[j][i];
      if (i < wave) pos += c;
      round_total += c;
    }
    const int64_t g0 = t0 + kRoundTok * j + 4 * tid;
    const uint32_t sel = (sel_all >> (4 * j)) & 0xFu;
    // targets: this thread's clean tokens of round j (registers, or reread)
    int32_t in[4] = {0, 0, 0, 0};
    if (sel) {
      if (full) {
        in[0] = v[j].x; in[1] = v[j].y; in[2] = v[j].z; in[3] = v[j].w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if ((sel >> k) & 1u) in[k] = a.x0[g0 + k];
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if ((sel >> k) & 1u) {
        s_row[pos] = (int32_t)(kShifted ? g0 + k - 1 : g0 + k);
        s_tgt[pos] = in[k];
        s_w[pos] = wts[j][k];
        ++pos;
      }
    }
    __syncthreads();
    for (int i = tid; i < round_total; i += kThreads) {
      const int64_t o = out_pos + i;
      if (o < a.n) {  // (only offsets that break their preconditions reach past)
        a.row_idx[o] = s_row[i];
        a.tgt[o] = s_tgt[i];
        a.w[o] = s_w[i];
      }
    }
    out_pos += round_total;
    __syncthreads();
  }
}

__global__ void set_rows_kernel(int32_t* p, int32_t v) { *p = v; }

template <int kNoise, bool kShifted>
void launch_fused(const Args& a, bool vec, unsigned grid, hipStream_t st) {
  if (vec)
    fused_kernel<kNoise, kShifted, true><<<grid, kThreads, 0, st>>>(a);
  else
    fused_kernel<kNoise, kShifted, false><<<grid, kThreads, 0, st>>>(a);
}

}  // namespace

size_t corrupt_compact_workspace_bytes(int64_t n_tokens) {
  if (n_tokens <= 0) return 0;
  const int64_t tiles = (n_tokens + kTile - 1) / kTile;
  // descriptors (8 B), first and last document (4 + 4 B) per tile; the ticket
  return (size_t)tiles * 16 + 16;
}

hipError_t launch_corrupt_compact(const int32_t* x0, int64_t n, const int32_t* cu,
                                  int32_t n_docs, uint64_t seed, double eps, int32_t noise,
                                  int32_t mask_id, int32_t rand_vocab, int32_t align,
                                  int32_t* xt, uint8_t* corrupted, double* p_doc,
                                  int32_t* doc_counts, int32_t* row_idx, int32_t* tgt,
                                  float* w, int32_t* n_rows, void* workspace,
                                  hipStream_t stream) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int64_t tiles = n > 0 ? (n + kTile - 1) / kTile : 0;
  Args a{};
  a.x0 = x0;
  a.n = n;
  a.cu = cu;
  a.n_docs = n_docs;
  a.k0 = k0;
  a.k1 = k1;
  a.eps = eps;
  a.mask_id = mask_id;
  a.rand_vocab = (uint32_t)rand_vocab;
  a.xt = xt;
  a.corrupted = corrupted;
  a.p_doc = p_doc;
  a.doc_counts = doc_counts;
  a.row_idx = row_idx;
  a.tgt = tgt;
  a.w = w;
  a.n_rows = n_rows;
  a.tiles = tiles;
  if (n <= 0) {
    // no tokens: the noise levels still (the prep pass writes a row count of
    // 0 when there are no tiles), or just the empty list
    if (n_docs > 0)
      prep_kernel<<<(unsigned)((n_docs + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
          n_docs, 0, 0, k0, k1, eps, cu, p_doc, doc_counts, n_rows, Ws{});
    else
      set_rows_kernel<<<1, 1, 0, stream>>>(n_rows, 0);
    return hipGetLastError();
  }
  char* ws = reinterpret_cast<char*>(workspace);
  a.ws.desc = reinterpret_cast<uint64_t*>(ws);
  a.ws.tile_lo = reinterpret_cast<int32_t*>(ws + tiles * 8);
  a.ws.tile_hi = a.ws.tile_lo + tiles;
  a.ws.ticket = reinterpret_cast<uint32_t*>(a.ws.tile_hi + tiles);
  a.single = tiles == 1;
  if (!a.single) {
    const int64_t threads = std::max<int64_t>(tiles, n_docs);
    prep_kernel<<<(unsigned)((threads + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
        n_docs, n, tiles, k0, k1, eps, cu, p_doc, doc_counts, n_rows, a.ws);
  }
  const bool vec = ((uintptr_t)x0 % 16 == 0) && ((uintptr_t)xt % 16 == 0) &&
                   ((uintptr_t)corrupted % 4 == 0);
  const unsigned grid = (unsigned)tiles;
  const bool shifted = align == MDLM_SHIFTED;
  if (noise == MDLM_NOISE_UNIFORM) {
    if (shifted) launch_fused<MDLM_NOISE_UNIFORM, true>(a, vec, grid, stream);
    else launch_fused<MDLM_NOISE_UNIFORM, false>(a, vec, grid, stream);
  } else {
    if (shifted) launch_fused<MDLM_NOISE_ABSORB, true>(a, vec, grid, stream);
    else launch_fused<MDLM_NOISE_ABSORB, false>(a, vec, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace mdlm
