// Fused frozen-LM-head + cross-entropy, forward and gradient w.r.t. hidden.
//
// Method: Axolotl diffusion docs, "Adapters, merging and inference" (full-
// vocabulary CE computed from hidden states through a plain linear head,
// without materialising vocabulary logits); LLaDA-8B-MDLM-LoRA card,
// "Training" table (CE on masked tokens divided by p; output layer frozen);
// diffusiongemma card, "Finetuning notes" (softcap applied exactly once).
//
// Pipeline for M scored rows (M lives on the device; grids are persistent and
// read it there):
//   0. (gradient with the preferred workspace) stash_ref_kernel: each row's
//      reference R, its capped target logit in log2 units from a plain dot
//      product; its spare blocks clear d_hidden.
//   1. logits_kernel<fwd>: z = W h over 256 x 256 (vocab x row) tiles, or
//      320 x 256 without a softcap, K = H, on bf16 MFMA with
//      fp32 accumulation.  Operands go from global memory straight into a
//      two-stage LDS ring (no register staging), two waves per SIMD.  The
//      epilogue caps, takes each row's partial (m_h, sum 2^(s-m_h)) over each
//      half of the tile (128 or 160 entries; m_h: the half's maximum) and
//      picks the target logit.  Logits never leave registers.  With the
//      preferred workspace and the gradient wanted, the epilogue also stashes
//      2^(s - rho) zhat' (zhat' = 1 - (zhat/c)^2 with a softcap c, else 1) in
//      G as bf16, the softmax up to a known factor: rho is R unless m_h lies
//      more than kStashSpan above it, which flags the row.
//   2. merge_kernel: per row, combine the partials into the log-sum-exp and
//      CE; per-block sums of w * CE in fp64.
//   3. fixed-order sum of the block sums -> loss: by block 0 of the first
//      stash_scale_kernel launch when the stash is used, else by loss_kernel.
//   4. (gradient) G = w (softmax - onehot) zhat' as bf16, either from the
//      stash (stash_scale_kernel multiplies by w 2^(rho - lse) and rewrites
//      the target entries, for the flagged rows only unless dW is wanted) or,
//      with a smaller workspace, per vocabulary chunk [v0, v1) by
//      logits_kernel<grad>, which recomputes the tiles.  dh_kernel forms
//      dH = G W over 256 x 256 (row x hidden) tiles with W read through LDS
//      transpose loads, split along the vocabulary into S slices chosen on
//      the device so that the tile x slice units fill the grid; for the rows
//      left as stash it forms sum_v q_v W_v instead.
//   5. d_hidden = 0 (zero_kernel, or step 0), then scatter_kernel: d_hidden[row_idx[j]]
//      = sum of the S slices of dH[j], in the hidden dtype; for stash rows
//      times the row factor w 2^(R - lse), plus the exact target term.
//   6. (trained head only) the remaining stash rows become G,
//      gather_rows_kernel copies the scored rows of hidden into the
//      workspace and dw_kernel forms dW = G^T Hs over 256 x 256 (vocab x
//      hidden) tiles, K = scored rows, per vocabulary chunk.
#include "mdlm_internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace mdlm {
namespace {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kThreads = 256;         // reduction and utility kernels
#ifndef MDLM_GEMM_WAVES
#define MDLM_GEMM_WAVES 8
#endif
// MFMA kernels: kWaves waves over a 256 x 256 tile.  Each wave owns 128 rows
// of operand A and 256 / (kWaves / 2) rows of operand B (kNJ 32-row blocks).
constexpr int kWaves = MDLM_GEMM_WAVES;
constexpr int kGemmThreads = 64 * kWaves;
constexpr int kNJ = 16 / kWaves;          // 32-row B blocks per wave
constexpr int kWB = 32 * kNJ;             // B rows per wave
constexpr int kLoads = 32 / kWaves;       // 1 KiB loads per operand per wave
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves");
constexpr int kTile = 256;            // rows of each operand tile
constexpr int kBK = 64;               // K elements per main-loop step
constexpr int kKRow = kBK * 2;        // bytes per row of a K-major tile (128)
constexpr int kNRow = kTile * 2;      // bytes per row of an N-major tile (512)
// The 32-row blocks of the tile's scored rows are dealt to the waves in turn:
// block j of a wave sits kRowStride rows after its block j-1, so that the
// blocks holding the first n rows of a partial tile fall evenly on the two
// waves of each SIMD pair.
constexpr int kRowStride = 32 * (kWaves / 2);
constexpr int kOpBytes = kTile * kKRow;       // one operand tile: 32 KiB
constexpr int kStageBytes = 2 * kOpBytes;     // A + B: 64 KiB
constexpr int kLdsBytes = 2 * kStageBytes;    // two stages: 128 KiB
#ifndef MDLM_STASH
#define MDLM_STASH 1
#endif
#ifndef MDLM_WIDE_TILE
#define MDLM_WIDE_TILE 1
#endif
constexpr int kMaxSplit = 8;          // K-splits of the dH product
#ifndef MDLM_DH_ROWS
#define MDLM_DH_ROWS 320
#endif
// The dH product's tile: kDhRows scored rows (kDhNI 32-row blocks per wave)
// by kTile hidden columns.
constexpr int kDhRows = MDLM_DH_ROWS;
constexpr int kDhNI = kDhRows / 64;
constexpr int kDhABytes = kDhRows * kKRow;            // G's K-major tile
constexpr int kDhALoads = kDhABytes / 1024 / kWaves;  // its 1 KiB loads per wave
constexpr int kDhStageBytes = kDhABytes + kOpBytes;   // G + W
static_assert(kDhRows % 64 == 0 && kDhALoads * 1024 * kWaves == kDhABytes,
              "whole 1 KiB loads per wave");
static_assert(2 * kDhStageBytes <= 160 * 1024, "two stages in LDS");
// The stash of a half tile is taken relative to the row's reference R (its
// target logit) when the half tile's maximum m_h is at most kStashSpan above
// R (log2 units), so entries stay below 2^64 and sums of them far below the
// fp32 range; otherwise relative to m_h, and the row takes the per-half-tile
// scaling pass.
constexpr float kStashSpan = 64.f;
constexpr int kMergeRows = 4;         // rows per merge block (one per wave)
constexpr int kGrid = 256;            // persistent grid: one workgroup per CU
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr size_t kAlign = 256;
static_assert(kTile * kKRow == 64 * kNRow, "K-major and N-major tiles share a size");

#define MDLM_LDS __attribute__((address_space(3)))
#define MDLM_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ int logical_block() {
  // Consecutive logical ids on one XCD: the hardware hands workgroup b to XCD
  // b % 8, so ids are regrouped to let one XCD's concurrently running tiles
  // share operand rows in its L2.
  const int per_xcd = gridDim.x >> 3;
  return (gridDim.x & 7) ? (int)blockIdx.x
                         : (int)((blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3));
}

// Tile (r, c) of an nr x nc grid for the linear index t, visited in blocks of
// gr x gc tiles: bands of gr rows one after another, the blocks of a band
// along c, each block row by row.  The tiles running at one time on an XCD
// then form a block (a few rows and columns of operand slabs instead of one
// row against every column, or the reverse), and the XCDs running beside it
// walk the same band, so that its slabs are fetched once for all of them.
// A bijection onto the grid for any sizes (edge bands and blocks are
// smaller).
__device__ __forceinline__ void grouped_tile(int64_t t, int nr, int nc, int gr, int gc, int* r,
                                             int* c) {
  const int64_t band = (int64_t)gr * nc;
  const int br = (int)(t / band);
  const int64_t rem = t - (int64_t)br * band;
  const int sr = min(gr, nr - br * gr);
  const int64_t blk = (int64_t)sr * gc;
  const int bc = (int)(rem / blk);
  const int64_t rem2 = rem - (int64_t)bc * blk;
  const int sc = min(gc, nc - bc * gc);
  *r = br * gr + (int)(rem2 / sc);
  *c = bc * gc + (int)(rem2 - (rem2 / sc) * sc);
}

__device__ __forceinline__ float softcap_fwd(float z, float c, float inv_c, float* dcap) {
  // c * tanh(z / c) with tanh(x) = 1 - 2 / (1 + e^{2x}); saturates cleanly.
  const float e = __builtin_amdgcn_exp2f(z * inv_c * (2.0f * kLog2e));
  const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
  *dcap = 1.0f - th * th;
  return c * th;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16_t a = (bf16_t)lo, b = (bf16_t)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// LDS swizzles.  K-major tile rows are 128 bytes (eight 16-byte chunks); the
// chunk index is xor-ed with a function of the row so that 16 consecutive
// rows read at one logical chunk hit distinct banks.  N-major tile rows are
// 512 bytes; their chunk index is xor-ed with 4 * (row % 4), which spreads the
// four rows of a transpose read over distinct banks.
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_n(int r) { return (r & 3) << 2; }

// 16 bytes per lane from a buffer into LDS: lane l's bytes land at lds + 16 l.
// Offsets past the resource's byte count read as zeros (the descriptor's
// range check), so tiles that overhang an operand need no clamping.
__device__ __forceinline__ void buf2l(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (MDLM_LDS void*)lds, 16, voff, soff, 0, 0);
}

// Raw (unformatted) buffer descriptor over `bytes` bytes from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t capped = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)capped,
                                           0x00020000);
}

// Calls f(integral_constant<int, min(n, N)>) for a wave-uniform n >= 0, so
// that a loop can be specialised on how many of a wave's blocks are in use.
template <int N, typename F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= N)
      f(std::integral_constant<int, N>{});
    else
      with_count<N - 1>(n, f);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Keeps the scheduler from moving instructions across this point: used so a
// step's MFMAs (and the loads interleaved with them) stay ahead of the next
// wait.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short shortx4;

// Four K-consecutive bf16 of one column of an N-major LDS tile (transpose
// read): in each group of 16 lanes, lane j names row j / 4 of a 4 x 16 block
// (its columns 4 (j % 4) .. 4 (j % 4) + 3); lane i then receives column i of
// that block, rows 0..3.
__device__ __forceinline__ shortx4 ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MDLM_LDS shortx4*)(p));
}

// Entry at offset dt (0 <= dt < 32 NA, bit 2 clear) of a lane's 16 NA
// entries of row block j, where entry e of block i sits at offset
// 32 i + 8 (e / 4) + e % 4: a select tree on the bits of dt (63 selects for
// four blocks) rather than one compare per entry.
__device__ __forceinline__ float sel(bool c, float a, float b) { return c ? a : b; }

template <int NA>
__device__ __forceinline__ float pick_entry(const f32x16 (&acc)[NA][kNJ], int j, int dt) {
  // (selects on values, never on array elements: a conditional lvalue would
  // select addresses and force the arrays into scratch memory)
  static_assert(NA == 4 || NA == 5, "four or five blocks");
  const bool b0 = dt & 1, b1 = dt & 2, b3 = dt & 8, b4 = dt & 16, b5 = dt & 32, b6 = dt & 64,
             b7 = dt & 128;
  float g[4 * NA];  // g[4 i + q]: entry 4 q + (dt % 4) of block i
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x0 = acc[i][j][4 * q], x1 = acc[i][j][4 * q + 1];
      const float x2 = acc[i][j][4 * q + 2], x3 = acc[i][j][4 * q + 3];
      g[4 * i + q] = sel(b1, sel(b0, x3, x2), sel(b0, x1, x0));
    }
  float h8[2 * NA], h4[NA];
#pragma unroll
  for (int k = 0; k < 2 * NA; ++k) h8[k] = sel(b3, g[2 * k + 1], g[2 * k]);
#pragma unroll
  for (int k = 0; k < NA; ++k) h4[k] = sel(b4, h8[2 * k + 1], h8[2 * k]);
  const float lo = sel(b6, sel(b5, h4[3], h4[2]), sel(b5, h4[1], h4[0]));
  if constexpr (NA == 5) return sel(b7, h4[4], lo);
  return lo;
}

// --------------------------------------------------------------------------
// Logits tiles: forward partials or gradient chunk.
// --------------------------------------------------------------------------
struct LogitsArgs {
  const bf16_t* W;
  const bf16_t* hidden;
  int64_t n_tokens;
  int H;
  int V;
  const int32_t* row_idx;
  const int32_t* tgt;
  const float* w;
  const int32_t* n_rows;
  int max_rows;
  float softcap;
  float inv_softcap;
  int v_begin;  // vocabulary range of this launch
  int v_end;
  float2* partial;  // fwd: [max_rows][n_part] (max, sum) per half tile, in log2
                    // units (row-major, so that a row's partials are contiguous)
  int n_part;       // 2 ceil(V / tile rows): 256, or 320 (see logits_kernel)
  float* ztgt;      // [max_rows] capped target logit x log2(e) (fwd writes, grad reads)
  const float* lse; // grad: [max_rows]
  bf16_t* G;        // grad, or fwd with the stash: [max_rows][ldg], column = v - v_begin
  int64_t ldg;
  const float* rref;  // fwd with the stash: [max_rows] per-row reference, log2 units
  int* row_flag;      // fwd with the stash: [max_rows] set where the reference was not used
};

// Waits for this wave's LDS accesses and until at most n of its memory
// operations are outstanding, then joins the workgroup's barrier.  Written
// as one asm block: in front of each barrier it emits itself (from
// __syncthreads or the barrier builtin), the compiler waits for every
// outstanding memory operation, which would also retire loads meant to stay
// in flight across it and stores nothing after it depends on.  (Vector
// memory operations complete in issue order, so n counts those issued after
// the ones waited for; n = 63, the counter's limit, waits for none.)
template <int n>
__device__ __forceinline__ void wait_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

// The K loop of the MFMA kernels over steps [kb, ke) of kBK: two LDS stages
// s0 and s1, operands loaded straight into LDS by issue(stage, k0), and
// fragments read by ra(stage, kk, f) and rb(stage, kk, f) for 16-deep slice
// kk.  Each step's barrier sits before its last slice, whose fragments are
// already in registers: after the barrier its MFMAs run while the step two
// ahead is loaded into the stage just finished and the first fragments of
// the next stage are read, so no wave waits on LDS latency after a barrier.
// At the barrier every wave is past its reads of the current stage and has
// waited for its own loads into the next one.  The loads of the two steps
// past ke read in-range bytes or zeros and are never consumed; the wait at
// the end retires them.  Only the first NI A blocks and NJ B blocks take
// part (NI NJ = 0: loads and barriers only); kReads counts a slice's LDS
// read instructions (transpose reads twice).
template <int NI, int NJ, int kReads, int kNIMax = 4, int kV = 2 * kLoads, typename ReadA,
          typename ReadB, typename Issue>
__device__ __forceinline__ void kloop_pipe(f32x16 (&acc)[kNIMax][kNJ], int kb, int ke, char* s0,
                                           char* s1, ReadA ra, ReadB rb, Issue issue) {
  // kNIMax: A blocks per wave (the accumulator rows); kV: loads per issue()
  constexpr int kMfma = NI * NJ;
  constexpr int kSlices = kBK / 16;
  bf16x8 af[2][kNIMax], bfr[2][kNJ];
  auto mfmas = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j],
                                                            0, 0, 0);
  };
  // the previous tile is done with both stages (its LDS reads; its stores
  // may still be in flight)
  wait_barrier<63>();
  issue(s0, kb * kBK);
  issue(s1, (kb + 1) * kBK);
  // s0's loads only (the kV loads into s1 stay in flight)
  wait_barrier<kV>();
  if constexpr (kMfma > 0) {
    ra(s0, 0, af[0]);
    rb(s0, 0, bfr[0]);
  }
  auto step = [&](char* cur, char* nxt, int kt) __attribute__((always_inline)) {
    if constexpr (kMfma > 0) {
#pragma unroll
      for (int kk = 0; kk + 1 < kSlices; ++kk) {
        ra(cur, kk + 1, af[(kk + 1) & 1]);
        rb(cur, kk + 1, bfr[(kk + 1) & 1]);
        mfmas(kk & 1);
      }
      // each slice's MFMAs alternated one for one with the next slice's reads
#pragma unroll
      for (int kk = 0; kk + 1 < kSlices; ++kk) {
#pragma unroll
        for (int x = 0; x < kMfma; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (x < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int x = kMfma; x < kReads; ++x) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    sched_fence();
    wait_barrier<0>();
    issue(cur, (kt + 2) * kBK);
    if constexpr (kMfma > 0) {
      ra(nxt, 0, af[0]);
      rb(nxt, 0, bfr[0]);
      mfmas((kSlices - 1) & 1);
      // the last slice's MFMAs, each after one load and before one read
#pragma unroll
      for (int x = 0; x < kMfma; ++x) {
        if (x < kV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (x < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int x = kMfma; x < kV; ++x) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
      for (int x = kMfma; x < kReads; ++x) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    sched_fence();
  };
  // two steps per trip so that each access names its stage statically
  int kt = kb;
  for (; kt + 2 <= ke; kt += 2) {
    step(s0, s1, kt);
    step(s1, s0, kt + 1);
  }
  if (kt < ke) step(s0, s1, kt);
  wait_vmem();
}

// Tile of 64 kNA vocabulary rows (operand A, rows of W) by 256 scored rows
// (operand B, rows of hidden gathered through row_idx), K = H.  Wave w owns
// vocabulary rows 32 kNA (w % 2) .. + 32 kNA - 1 and the scored-row blocks
// 32 (w / 2) + kRowStride j .. +31, j < kNJ: a kNA x kNJ grid of 32 x 32
// MFMA blocks, of which only those holding scored rows are computed.
// kStash (forward only): the epilogue also keeps the tile's unnormalised
// softmax, 2^(s - rho) zhat', as bf16 in G, so that the gradient needs no
// second pass over the logits.  rho is the row's reference R (see
// kStashSpan) or, far above it, the row's maximum m_h over the wave's half
// of the tile.  The partials are (m_h, sum 2^(s - m_h)) either way, the same
// as without the stash.
// kNA: 32-row blocks of W per wave, so a vocabulary tile of 64 kNA rows
// (256, or 320 for the forward pass without a softcap), each
// wave owning half of it: 32 kNA entries per row and partial.
template <bool kGrad, bool kCap, bool kStash = false, int kNA = 4>
__global__ void __launch_bounds__(kGemmThreads, 1) logits_kernel(LogitsArgs a) {
  static_assert(!(kGrad && kStash), "the stash is written by the forward pass");
  static_assert(kNA == 4 || (kNA == 5 && !kGrad && !kCap), "320 rows: forward, no softcap");
  constexpr int kVT = 64 * kNA;            // vocabulary rows of a tile
  constexpr int kHalf = 32 * kNA;          // a wave's entries per row
  constexpr int kAB = kVT * kKRow;         // W's bytes in a stage
  constexpr int kSB = kAB + kOpBytes;      // W + the scored rows
  static_assert(2 * kSB <= 160 * 1024, "two stages in LDS");
  // the two stages are separate objects so that the compiler can tell a
  // prefetch into one from reads of the other
  __shared__ __attribute__((aligned(1024))) char smem0[kSB];
  __shared__ __attribute__((aligned(1024))) char smem1[kSB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = wave & 1, wb = wave >> 1;
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int n_mt = (n_rows + kTile - 1) / kTile;
  const int n_vt = (a.v_end - a.v_begin + kVT - 1) / kVT;
  const int64_t n_tiles = (int64_t)n_mt * n_vt;
  const int KT = a.H / kBK;

  // fragment-read offsets (bytes within a stage)
  const int fx = swz_k(lane & 15), khalf = lane >> 5;
  const int a_off = (wa * kHalf + (lane & 31)) * kKRow;
  const int b_off = kAB + (32 * wb + (lane & 31)) * kKRow;
  // direct-load roles: load q (0..kNA-1) of this wave fills W rows
  // 8 (kNA wave + q) .. +7, load q (0..kLoads-1) the scored rows
  // 8 (kLoads wave + q) .. +7; lane l supplies row 8 (...) + l / 8 at
  // physical chunk l % 8
  const int lrow = lane >> 3, lphys = lane & 7;
  const int wpar = (kNA * wave) & 1;

  for (int64_t t = logical_block(); t < n_tiles; t += gridDim.x) {
    // bands of 8 vocabulary tiles (W, the larger operand, shared by the
    // XCDs of a band), blocks of 8 x 4 (measured against 4 x 8, 2 x 16,
    // 16 x 2 and 32 x 1: 0.4% faster than 4 x 8 per call on llada8b-1x4096,
    // 1.5% on packed, 0.6% on canvas with its 256-row tiles)
    int vt, mt;
    grouped_tile(t, n_vt, n_mt, 8, 4, &vt, &mt);
    const int v0 = a.v_begin + vt * kVT;
    const int m0 = mt * kTile;

    // A: rows v0.. of W, read as one buffer that ends at v_end (rows past it
    // read as zeros).  Row r = 8 (kNA wave + q) + l / 8 has r % 8 = l / 8
    // and (r / 8) % 2 = wpar ^ (q % 2), so its swizzled chunk depends on q
    // only through q % 2: two lane offsets serve all loads, the rest is
    // scalar.
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(a.W + (int64_t)v0 * a.H, (int64_t)(a.v_end - v0) * a.H * 2);
    uint32_t a_voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
      a_voff[par] = (uint32_t)((lrow * a.H + 8 * (lphys ^ lrow ^ par ^ wpar)) * 2);
    // B: gathered rows of hidden; rows past n_rows point past the buffer
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.hidden, a.n_tokens * a.H * 2);
    uint32_t b_voff[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int r = 8 * (kLoads * wave + q) + lrow;
      const int m = m0 + r;
      int64_t row = -1;
      if (m < n_rows) {
        row = a.row_idx[m];
        if (row >= a.n_tokens) row = -1;
      }
      b_voff[q] = row < 0 ? 0xFFFFFFF0u
                          : (uint32_t)((row * a.H + 8 * (lphys ^ swz_k(r))) * 2);
    }
    f32x16 acc[kNA][kNJ];
#pragma unroll
    for (int i = 0; i < kNA; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto issue = [&](char* stage, int k0) {
      char* sa = stage + (kNA * wave) * 1024;
      char* sb = stage + kAB + (kLoads * wave) * 1024;
#pragma unroll
      for (int q = 0; q < kNA; ++q) {
        buf2l(ra, sa + q * 1024, a_voff[q & 1],
              (uint32_t)((8 * (kNA * wave + q) * a.H + k0) * 2));
        if (q < kLoads) buf2l(rb, sb + q * 1024, b_voff[q], (uint32_t)(k0 * 2));
      }
    };
    // this wave's blocks that hold scored rows (a prefix of its kNJ)
    const int nv = min(kTile, n_rows - m0);
    const int kj = max(0, (nv - 32 * wb + kRowStride - 1) / kRowStride);
    // the epilogue's per-row inputs, loaded before the K loop so that they
    // arrive during it (the loop's waits keep later loads from moving up);
    // the five-block tile, whose registers are full, loads them in the
    // epilogue instead
    constexpr bool kPre = kNA == 4;
    int tg_pre[kNJ];
    float ref_pre[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      const int m = m0 + 32 * wb + kRowStride * j + (lane & 31);
      const bool mv = m < n_rows;
      tg_pre[j] = kPre && mv ? a.tgt[m] : -1;
      ref_pre[j] = kPre && kStash && mv ? a.rref[m] : 0.f;
    }
    // the K loop, specialised on that count (the waves of a workgroup run
    // the same loads and barriers whatever their count)
    auto kloop = [&](auto nj_tag) __attribute__((always_inline)) {
      constexpr int NJ = decltype(nj_tag)::value;
      kloop_pipe<kNA, NJ, kNA + NJ, kNA, kNA + kLoads>(
          acc, 0, KT, smem0, smem1,
          [&](const char* base, int kk, bf16x8(&f)[kNA]) __attribute__((always_inline)) {
            const int coff = ((2 * kk + khalf) ^ fx) * 16;
#pragma unroll
            for (int i = 0; i < kNA; ++i)
              f[i] = *reinterpret_cast<const bf16x8*>(base + a_off + i * 32 * kKRow + coff);
          },
          [&](const char* base, int kk, bf16x8(&f)[kNJ]) __attribute__((always_inline)) {
            const int coff = ((2 * kk + khalf) ^ fx) * 16;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              f[j] = *reinterpret_cast<const bf16x8*>(base + b_off + j * kRowStride * kKRow + coff);
          },
          issue);
    };
    with_count<kNJ>(kj, kloop);
    // the variants that write G stage it through the stage memory, which
    // other waves may still be reading (their last K step) or filling (the
    // unconsumed prefetch) until all of them are here
    if constexpr (kStash || kGrad) __syncthreads();

    // ---- epilogue ---------------------------------------------------------
    // (the lane index passes through an empty asm so that the epilogue's
    // lane offsets are formed here, per tile, rather than hoisted out of the
    // tile loop and held in registers across the K loop)
    int el = lane;
    asm volatile("" : "+v"(el));
    // Accumulator element e of block (i, j) on lane l holds vocabulary entry
    // vl + 32i + 8(e/4) + e%4, vl = v0 + wa*kHalf + 4(l/32), for row
    // m0 + 32 wb + kRowStride j + l%32.  A row's target sits in this lane's registers
    // iff its offset dt from vl lies in [0, kHalf) with bit 2 clear.  Only the
    // tile that straddles v_end masks entries past the vocabulary.
    const int vl = v0 + wa * kHalf + 4 * (el >> 5);
    const int lim = a.v_end - vl;
    // G goes out through LDS: a lane's 4-entry pieces of a block land in
    // this wave's own 32 rows of 2 kHalf bytes (256 or 320; pitch 16 B more,
    // so that any 16 consecutive rows start on distinct 4-bank groups, the
    // writes do not conflict on banks, and every address is one base plus a
    // constant) and leave as whole row segments, 16 B a lane, instead of 8 B
    // in each of 32 rows per store.  The blocks of a wave reuse the region.
    constexpr int kPitch = 2 * kHalf + 16;
    static_assert(4 * 32 * kPitch <= kSB, "staging fits a stage");
    char* const st = (wave < 4 ? smem0 : smem1) + (wave & 3) * (32 * kPitch);
    auto stage_put = [&](int i, int q, uint2 v) __attribute__((always_inline)) {
      *reinterpret_cast<uint2*>(st + (el & 31) * kPitch + 8 * (el >> 5) + 16 * (4 * i + q)) =
          v;
    };
    auto stage_flush = [&](int j) __attribute__((always_inline)) {
      // LDS work of one wave completes in order; the wait and the clobbers
      // keep the compiler from moving the reads above this block's writes
      // or the next block's writes above them.  The stores go through a
      // buffer that ends at row n_rows, so rows past it are dropped by the
      // hardware (no branch), and share one lane offset.
      sched_fence();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int rb = m0 + 32 * wb + kRowStride * j;
      const int col = v0 - a.v_begin + wa * kHalf;
      const __amdgpu_buffer_rsrc_t rg =
          make_rsrc(a.G + (int64_t)rb * a.ldg + col, (int64_t)(n_rows - rb) * a.ldg * 2 - 2 * col);
      if constexpr (kNA == 4) {
        // 16 lanes per 256-byte row segment, four rows per store
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          v[k] = *reinterpret_cast<const u32x4*>(st + ((el >> 4) + 4 * k) * kPitch +
                                                 16 * (el & 15));
        asm volatile("" ::: "memory");
        const uint32_t voff = (uint32_t)(((el >> 4) * a.ldg + 8 * (el & 15)) * 2);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          __builtin_amdgcn_raw_buffer_store_b128(v[k], rg, voff, (uint32_t)(8 * k * a.ldg), 0);
      } else {
        // 320-byte rows as a 256-byte segment (16 lanes a row, four rows a
        // store, as above) and a 64-byte one (4 lanes a row, sixteen rows a
        // store): lane offsets plus scalar ones.  G is ldg columns wide (a
        // multiple of 256), so the last tile's pieces from column ldg on
        // (entries past the vocabulary, all zeros) are not stored.
        static_assert(kNA == 5, "256 + 64 bytes per row");
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          v[k] = *reinterpret_cast<const u32x4*>(st + ((el >> 4) + 4 * k) * kPitch +
                                                 16 * (el & 15));
        u32x4 t[2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
          t[k] = *reinterpret_cast<const u32x4*>(st + ((el >> 2) + 16 * k) * kPitch + 256 +
                                                 16 * (el & 3));
        asm volatile("" ::: "memory");
        const uint32_t voff = (uint32_t)(((el >> 4) * a.ldg + 8 * (el & 15)) * 2);
        if (col + 8 * (el & 15) < a.ldg) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(v[k], rg, voff, (uint32_t)(8 * k * a.ldg), 0);
        }
        const uint32_t toff = (uint32_t)(((el >> 2) * a.ldg + 128 + 8 * (el & 3)) * 2);
        if (col + 128 + 8 * (el & 3) < a.ldg) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(t[k], rg, toff, (uint32_t)(32 * k * a.ldg), 0);
        }
      }
      sched_fence();
    };
    auto epilogue = [&](auto full_tag) __attribute__((always_inline)) {
      constexpr bool kFull = decltype(full_tag)::value;
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        if (j >= kj) break;  // (no scored row in this block or the next)
        const int m = m0 + 32 * wb + kRowStride * j + (el & 31);
        const bool mvalid = m < n_rows;
        const int tg = kPre ? tg_pre[j] : mvalid ? a.tgt[m] : -1;
        const int dt = tg - vl;
        const bool holds_tgt = (unsigned)dt < (unsigned)kHalf && (dt & 4) == 0;
        if (!kGrad) {
          // The accumulators of row block j become, in place, the scaled
          // logits s = z log2(e) (capped first), or without a cap the logits
          // z themselves, scaled where they are used: the maximum and the
          // target are scaled after the selection (a positive factor
          // commutes with max, and each is rounded once, as before), and
          // 2^(s - mref) takes s - mref as one fma.  (In place: a copy
          // would hold a second set of the block's values in registers.)
          constexpr bool kRaw = !kCap;
          float mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < kNA; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int off = 32 * i + 8 * (e >> 2) + (e & 3);
              float zc = acc[i][j][e], dc;
              if (kCap) zc = softcap_fwd(zc, a.softcap, a.inv_softcap, &dc);
              float sc = kRaw ? zc : zc * kLog2e;
              if (!kFull) sc = off < lim ? sc : -INFINITY;
              acc[i][j][e] = sc;
              mx = fmaxf(mx, sc);
            }
          // (the target is never past the vocabulary, so never masked)
          if (mvalid && holds_tgt) {
            const float pt = pick_entry(acc, j, dt);
            a.ztgt[m] = kRaw ? pt * kLog2e : pt;
          }
          // the row's maximum over this wave's kHalf entries (two lanes hold
          // half each); -inf when all of them lie past the vocabulary
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          if (kRaw) mx *= kLog2e;
          const float mref = mx == -INFINITY ? 0.f : mx;
          // the stash is 2^(s - rho) = 2^(s - mref) fs with rho = R when m_h
          // is within kStashSpan of it (fs <= 2^64; it may underflow to 0
          // where m_h is far below R, whose entries are then negligible),
          // else rho = m_h and the row is flagged
          float fs = 1.f;
          if (kStash) {
            const float R = kPre ? ref_pre[j] : mvalid ? a.rref[m] : 0.f;
            const bool near = !(mx - R > kStashSpan);
            if (!near && mvalid && el < 32) a.row_flag[m] = 1;
            fs = mx == -INFINITY ? 0.f : near ? __builtin_amdgcn_exp2f(mx - R) : 1.f;
          }
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < kNA; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float g[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float sc = acc[i][j][4 * q + r];
                const float e2 = __builtin_amdgcn_exp2f(kRaw ? __builtin_fmaf(sc, kLog2e, -mref)
                                                             : sc - mref);
                sum += e2;
                if (kStash) {
                  float gv = e2 * fs;
                  if (kCap) {
                    const float th = sc * kLn2 * a.inv_softcap;
                    gv *= 1.f - th * th;
                  }
                  if (!kFull) gv = 32 * i + 8 * q + r < lim ? gv : 0.f;
                  g[r] = gv;
                }
              }
              if (kStash)
                stage_put(i, q, make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])));
            }
            // (five blocks: the sum is formed block by block, so that the
            // block's exponentials are not all held until the end for it)
            if constexpr (kNA == 5) asm volatile("" : "+v"(sum));
          }
          if (kStash) stage_flush(j);
          sum += __shfl_xor(sum, 32, 64);
          if (el < 32 && mvalid)
            a.partial[(int64_t)m * a.n_part + 2 * ((v0 - a.v_begin) / kVT) + wa] =
                make_float2(mx, sum);
        } else {
          // G = w p cap' everywhere, then the target entry is rewritten with
          // w (p - 1) cap' from the capped target logit the forward pass kept
          // (the same tile product).  Lanes of rows past n_rows stage
          // zeros that are never stored.
          const float lse2 = mvalid ? a.lse[m] * kLog2e : 0.f;
          const float wm = mvalid ? a.w[m] : 0.f;
#pragma unroll
          for (int i = 0; i < kNA; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float g[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int off = 32 * i + 8 * q + r;
                float zc = acc[i][j][4 * q + r], dc = 1.f;
                if (kCap) zc = softcap_fwd(zc, a.softcap, a.inv_softcap, &dc);
                const float p = __builtin_amdgcn_exp2f(zc * kLog2e - lse2);
                g[r] = kCap ? p * dc * wm : p * wm;
                if (!kFull) g[r] = off < lim ? g[r] : 0.f;
              }
              stage_put(i, q, make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])));
            }
          if (mvalid && holds_tgt) {
            const float zt2 = a.ztgt[m];
            float dc = 1.f;
            if (kCap) {
              const float th = zt2 * kLn2 * a.inv_softcap;
              dc = 1.f - th * th;
            }
            const float p = __builtin_amdgcn_exp2f(zt2 - lse2);
            // (over the piece this lane staged above: program order)
            *reinterpret_cast<bf16_t*>(st + (el & 31) * kPitch + 2 * (tg - (v0 + wa * kHalf))) =
                (bf16_t)((p - 1.f) * dc * wm);
          }
          stage_flush(j);
        }
      }
    };
    if (v0 + kVT <= a.v_end)
      epilogue(std::true_type{});
    else
      epilogue(std::false_type{});
  }
}

// --------------------------------------------------------------------------
// dH = G W over one vocabulary chunk, split along K into S slices.
// --------------------------------------------------------------------------
struct DhArgs {
  const bf16_t* G;
  int64_t ldg;
  const bf16_t* W;
  int H;
  int v_begin;
  int v_end;
  const int32_t* n_rows;
  int max_rows;
  float* part;  // [kMaxSplit][max_rows][H] fp32, slice s in part + s * max_rows * H
  int accumulate;
};

// Number of K-slices: the fewest (up to kMaxSplit) that keep the grid busy,
// measured by the share of workgroup slots the tile x slice units fill.
__host__ __device__ __forceinline__ int dh_splits(int64_t tiles, int grid, int ki) {
  if (tiles <= 0) return 1;
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= kMaxSplit && s <= ki; ++s) {
    const int64_t units = tiles * s;
    const int64_t rounds = (units + grid - 1) / grid;
    const double eff = (double)units / (double)(rounds * grid);
    if (eff > best_eff + 0.02) {
      best = s;
      best_eff = eff;
    }
  }
  return best;
}

// Tile of kDhRows scored rows (operand A, rows of G) by 256 hidden columns
// (operand B, columns of W read through transpose loads), K = vocabulary.
// Wave w owns the row blocks 32 (w % 2) + 64 i .. +31, i < kDhNI (dealt in turn,
// so that a partial tile's rows fall evenly on both SIMD pairs; only blocks
// holding scored rows are computed) and columns kWB (w / 2) .. +kWB-1.
__global__ void __launch_bounds__(kGemmThreads, 1) dh_kernel(DhArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem0[kDhStageBytes];
  __shared__ __attribute__((aligned(1024))) char smem1[kDhStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = wave & 1, wb = wave >> 1;
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int n_mt = (n_rows + kDhRows - 1) / kDhRows;
  const int n_ht = (a.H + kTile - 1) / kTile;
  const int64_t T = (int64_t)n_mt * n_ht;
  const int KI = (a.v_end - a.v_begin + kBK - 1) / kBK;
  if (T == 0 || KI == 0) return;
  const int S = dh_splits(T, gridDim.x, KI);

  const int fx = swz_k(lane & 15), khalf = lane >> 5;
  const int a_off = (32 * wa + (lane & 31)) * kKRow;
  // transpose-read roles: group g = lane / 16 covers K rows 8 (g / 2) .. +7 of
  // a 16-deep slice and columns 16 (g % 2) .. +15 of a 32-column block
  const int jl = lane & 15, grp = lane >> 4;
  const int tr_row = 8 * (grp >> 1) + (jl >> 2);
  int b_col_off[kNJ];
#pragma unroll
  for (int j = 0; j < kNJ; ++j) {
    const int col = wb * kWB + 32 * j + 16 * (grp & 1) + 4 * (jl & 3);
    b_col_off[j] = (((col >> 3) ^ swz_n(tr_row)) * 16) + ((col >> 2) & 1) * 8;
  }
  const int lrow = lane >> 3, lphys = lane & 7;       // K-major loads
  const int nrow = lane >> 5, nphys = lane & 31;      // N-major loads

  const int64_t units = T * S;
  for (int64_t u = logical_block(); u < units; u += gridDim.x) {
    const int s = (int)(u / T);
    const int64_t tile = u % T;
    // bands of 8 row tiles (G, the larger operand, shared by the XCDs of a
    // band), blocks of 8 x 4
    int mt, ht;
    grouped_tile(tile, n_mt, n_ht, 8, 4, &mt, &ht);
    const int m0 = mt * kDhRows, h0 = ht * kTile;
    const int kb = (int)((int64_t)KI * s / S), ke = (int)((int64_t)KI * (s + 1) / S);

    // load q (0..kLoads-1): K-major rows 8 (kLoads wave + q) + l / 8 of G,
    // N-major rows 2 (kLoads wave + q) + l / 32 of W.  Both swizzles depend on q only through
    // q % 2, so two lane offsets per operand serve all loads.  G rows past
    // n_rows and W rows past v_end read as zeros.
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(a.G + (int64_t)m0 * a.ldg, (int64_t)(n_rows - m0) * a.ldg * 2);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(a.W + (int64_t)a.v_begin * a.H, (int64_t)(a.v_end - a.v_begin) * a.H * 2);
    // (G's load q fills LDS rows 8 (kDhALoads wave + q) .. +7, whose swizzle
    // parity is that of kDhALoads wave + q)
    const int wpar = (kDhALoads & 1) ? (wave & 1) : 0;
    uint32_t a_voff[2], b_voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      a_voff[par] = (uint32_t)((lrow * a.ldg + 8 * (lphys ^ lrow ^ par ^ wpar)) * 2);
      const int cn = nphys ^ swz_n(2 * par + nrow);
      // columns past H read the following row (finite values whose products
      // land only in columns that are never stored)
      b_voff[par] = (uint32_t)((nrow * a.H + h0 + 8 * cn) * 2);
    }
    f32x16 acc[kDhNI][kNJ];
#pragma unroll
    for (int i = 0; i < kDhNI; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto issue = [&](char* stage, int k0) {
      char* sa = stage + (kDhALoads * wave) * 1024;
      char* sb = stage + kDhABytes + (kLoads * wave) * 1024;
#pragma unroll
      for (int q = 0; q < (kDhALoads > kLoads ? kDhALoads : kLoads); ++q) {
        if (q < kDhALoads)
          buf2l(ra, sa + q * 1024, a_voff[q & 1],
                (uint32_t)((8 * (kDhALoads * wave + q) * a.ldg + k0) * 2));
        if (q < kLoads)
          buf2l(rb, sb + q * 1024, b_voff[q & 1],
                (uint32_t)((2 * (kLoads * wave + q) + k0) * a.H * 2));
      }
    };
    // this wave's row blocks that hold scored rows (a prefix of its kDhNI)
    const int nv = min(kDhRows, n_rows - m0);
    const int ki = max(0, (nv - 32 * wa + 63) / 64);
    auto kloop = [&](auto ni_tag) __attribute__((always_inline)) {
      constexpr int NI = decltype(ni_tag)::value;
      kloop_pipe<NI, kNJ, NI + 2 * kNJ, kDhNI, kDhALoads + kLoads>(
          acc, kb, ke, smem0, smem1,
          [&](const char* base, int kk, bf16x8(&f)[kDhNI]) __attribute__((always_inline)) {
            const int coff = ((2 * kk + khalf) ^ fx) * 16;
#pragma unroll
            for (int i = 0; i < NI; ++i)
              f[i] = *reinterpret_cast<const bf16x8*>(base + a_off + i * 64 * kKRow + coff);
          },
          [&](const char* base, int kk, bf16x8(&f)[kNJ]) __attribute__((always_inline)) {
            const char* brow_p = base + kDhABytes + (16 * kk + tr_row) * kNRow;
#pragma unroll
            for (int j = 0; j < kNJ; ++j) {
              const shortx4 lo = ds_read_tr(brow_p + b_col_off[j]);
              const shortx4 hi = ds_read_tr(brow_p + 4 * kNRow + b_col_off[j]);
              const short v8 __attribute__((__vector_size__(16))) = {
                  lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              f[j] = __builtin_bit_cast(bf16x8, v8);
            }
          },
          issue);
    };
    with_count<kDhNI>(ki, kloop);

    // acc element e of block (i, j) on lane l: row m0 + 32 wa + 64 i + 8(e/4)
    // + 4(l/32) + e%4, column h0 + wb*kWB + 32j + l%32.
    float* out = a.part + (int64_t)s * a.max_rows * a.H;
#pragma unroll
    for (int i = 0; i < kDhNI; ++i) {
      if (i >= ki) break;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * wa + 64 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m >= n_rows) continue;
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
          const int h = h0 + wb * kWB + 32 * j + (lane & 31);
          if (h < a.H) {
            float* p = out + (int64_t)m * a.H + h;
            *p = a.accumulate ? *p + acc[i][j][e] : acc[i][j][e];
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// dW = G^T Hs over one vocabulary chunk (a trainable head's gradient).
// --------------------------------------------------------------------------
struct DwArgs {
  const bf16_t* G;   // [max_rows][ldg], column v - v_begin
  int64_t ldg;
  const bf16_t* Hs;  // [max_rows][H]: hidden[row_idx[m]] for m < n_rows
  int H;
  int v_begin;
  int v_end;
  const int32_t* n_rows;
  int max_rows;
  float* dW;         // [V][H]
};

// Tile of 256 vocabulary entries (operand A: columns of G) by 256 hidden
// columns (operand B: columns of Hs), K = scored rows.  Both operands are
// N-major in memory (rows of G and of Hs), staged as 64-row x 512-byte LDS
// tiles and read through transpose loads.  Wave w owns vocabulary entries
// 128 (w % 2) .. +127 and hidden columns kWB (w / 2) .. +kWB-1.  Rows past
// n_rows read as zeros through the buffer range check; the buffer bases move
// with the K step so every offset stays within 32 bits.
__global__ void __launch_bounds__(kGemmThreads, 1) dw_kernel(DwArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char smem1[kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = wave & 1, wb = wave >> 1;
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int n_vt = (a.v_end - a.v_begin + kTile - 1) / kTile;
  const int n_ht = (a.H + kTile - 1) / kTile;
  const int64_t T = (int64_t)n_vt * n_ht;
  const int KT = (n_rows + kBK - 1) / kBK;

  // transpose-read roles (as in dh_kernel)
  const int jl = lane & 15, grp = lane >> 4;
  const int tr_row = 8 * (grp >> 1) + (jl >> 2);
  auto col_off = [&](int col) {
    return (((col >> 3) ^ swz_n(tr_row)) * 16) + ((col >> 2) & 1) * 8;
  };
  int a_col_off[4], b_col_off[kNJ];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_col_off[i] = col_off(wa * 128 + 32 * i + 16 * (grp & 1) + 4 * (jl & 3));
#pragma unroll
  for (int j = 0; j < kNJ; ++j)
    b_col_off[j] = col_off(wb * kWB + 32 * j + 16 * (grp & 1) + 4 * (jl & 3));
  const int nrow = lane >> 5, nphys = lane & 31;  // N-major loads

  for (int64_t t = logical_block(); t < T; t += gridDim.x) {
    // bands of 4 vocabulary tiles (G, the larger operand), blocks of 4 x 8
    int vt, ht;
    grouped_tile(t, n_vt, n_ht, 4, 8, &vt, &ht);
    const int v0 = vt * kTile;  // column of G
    const int h0 = ht * kTile;
    uint32_t a_voff[2], b_voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int cn = nphys ^ swz_n(2 * par + nrow);
      a_voff[par] = (uint32_t)((nrow * a.ldg + 8 * cn) * 2);
      b_voff[par] = (uint32_t)((nrow * a.H + 8 * cn) * 2);
    }
    f32x16 acc[4][kNJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto issue = [&](char* stage, int k0) {
      // rows k0.. of both operands; past n_rows the ranges are empty
      const int64_t rows_left = (int64_t)n_rows - k0;
      const __amdgpu_buffer_rsrc_t ra =
          make_rsrc(a.G + (int64_t)k0 * a.ldg + v0, rows_left * a.ldg * 2 - (int64_t)v0 * 2);
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(a.Hs + (int64_t)k0 * a.H + h0, rows_left * a.H * 2 - (int64_t)h0 * 2);
      char* sa = stage + (kLoads * wave) * 1024;
#pragma unroll
      for (int q = 0; q < kLoads; ++q) {
        const int r = 2 * (kLoads * wave + q);
        buf2l(ra, sa + q * 1024, a_voff[q & 1], (uint32_t)(r * a.ldg * 2));
        buf2l(rb, sa + kOpBytes + q * 1024, b_voff[q & 1], (uint32_t)(r * a.H * 2));
      }
    };
    // the K loop of the other MFMA kernels (each step's barrier before its
    // last slice; the prefetch past the last row reads empty ranges)
    kloop_pipe<4, kNJ, 2 * 4 + 2 * kNJ>(
        acc, 0, KT, smem0, smem1,
        [&](const char* base, int kk, bf16x8(&f)[4]) __attribute__((always_inline)) {
          const char* arow_p = base + (16 * kk + tr_row) * kNRow;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const shortx4 lo = ds_read_tr(arow_p + a_col_off[i]);
            const shortx4 hi = ds_read_tr(arow_p + 4 * kNRow + a_col_off[i]);
            const short v8 __attribute__((__vector_size__(16))) = {
                lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            f[i] = __builtin_bit_cast(bf16x8, v8);
          }
        },
        [&](const char* base, int kk, bf16x8(&f)[kNJ]) __attribute__((always_inline)) {
          const char* brow_p = base + kOpBytes + (16 * kk + tr_row) * kNRow;
#pragma unroll
          for (int j = 0; j < kNJ; ++j) {
            const shortx4 lo = ds_read_tr(brow_p + b_col_off[j]);
            const shortx4 hi = ds_read_tr(brow_p + 4 * kNRow + b_col_off[j]);
            const short v8 __attribute__((__vector_size__(16))) = {
                lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            f[j] = __builtin_bit_cast(bf16x8, v8);
          }
        },
        issue);

    // acc element e of block (i, j) on lane l: vocabulary entry v_begin + v0
    // + wa*128 + 32i + 8(e/4) + 4(l/32) + e%4, hidden column h0 + wb*kWB +
    // 32j + l%32.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = a.v_begin + v0 + wa * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (v >= a.v_end) continue;
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
          const int h = h0 + wb * kWB + 32 * j + (lane & 31);
          if (h < a.H) a.dW[(int64_t)v * a.H + h] = acc[i][j][e];
        }
      }
  }
}

// Hs[m] = hidden[row_idx[m]] for the scored rows (zeros for an out-of-range
// index), 16 bytes per thread.
__global__ void __launch_bounds__(kThreads)
gather_rows_kernel(const bf16_t* __restrict__ hidden, const int32_t* __restrict__ row_idx,
                   const int32_t* __restrict__ n_rows_ptr, int max_rows, int64_t n_tokens, int H,
                   bf16_t* __restrict__ Hs) {
  const int n_rows = min(*n_rows_ptr, max_rows);
  const int n16 = H / 8;  // H is a multiple of 64
  for (int m = blockIdx.x; m < n_rows; m += gridDim.x) {
    const int64_t r = row_idx[m];
    const bool ok = r >= 0 && r < n_tokens;
    const uint4* src = reinterpret_cast<const uint4*>(hidden + (ok ? r : 0) * H);
    uint4* dst = reinterpret_cast<uint4*>(Hs + (int64_t)m * H);
    for (int i = threadIdx.x; i < n16; i += kThreads)
      dst[i] = ok ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  }
}

// --------------------------------------------------------------------------
// Reductions.
// --------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
merge_kernel(const float2* __restrict__ partial, int n_part, int max_rows,
             const float* __restrict__ ztgt, const int32_t* __restrict__ tgt, int V,
             const float* __restrict__ w, const int32_t* __restrict__ n_rows_ptr,
             float* __restrict__ lse_out, float* __restrict__ row_ce,
             double* __restrict__ block_sums) {
  __shared__ double contrib[kMergeRows];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_rows = min(*n_rows_ptr, max_rows);
  const int j = blockIdx.x * kMergeRows + wave;
  double c = 0.0;
  if (j < n_rows) {
    float mx = -INFINITY, s = 0.f;
    for (int t = lane; t < n_part; t += 64) {
      const float2 p = partial[(int64_t)j * n_part + t];
      const float nm = fmaxf(mx, p.x);
      if (nm != -INFINITY)
        s = s * __builtin_amdgcn_exp2f(mx - nm) + p.y * __builtin_amdgcn_exp2f(p.x - nm);
      mx = nm;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(mx, off, 64), os = __shfl_xor(s, off, 64);
      const float nm = fmaxf(mx, om);
      if (nm != -INFINITY)
        s = s * __builtin_amdgcn_exp2f(mx - nm) + os * __builtin_amdgcn_exp2f(om - nm);
      mx = nm;
    }
    const float lse2 = mx + __log2f(s);
    const float lse = lse2 * kLn2;
    const int tg = tgt[j];
    // ztgt holds the capped target logit in log2 units
    const float ce = (tg >= 0 && tg < V) ? (lse2 - ztgt[j]) * kLn2 : NAN;
    if (lane == 0) {
      lse_out[j] = lse;
      if (row_ce) row_ce[j] = ce;
    }
    c = (double)w[j] * (double)ce;
  }
  if (lane == 0) contrib[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kMergeRows; ++i) t += contrib[i];
    block_sums[blockIdx.x] = t;
  }
}

// The stash's per-row reference: the capped target logit in log2 units,
// computed on its own (one wave per row, fp32), and a cleared fallback flag.
// Rows whose hidden row or target lies outside its range get 0.  The first
// ref_blocks blocks do this; any blocks after them clear d_hidden (z16
// 16-byte words at zp, then z_tail bytes), which would otherwise take a
// launch of its own.
__global__ void __launch_bounds__(kThreads)
stash_ref_kernel(const bf16_t* __restrict__ hidden, const bf16_t* __restrict__ W, int H, int V,
                 const int32_t* __restrict__ row_idx, const int32_t* __restrict__ tgt,
                 const int32_t* __restrict__ n_rows_ptr, int max_rows, int64_t n_tokens,
                 float softcap, float inv_softcap, float* __restrict__ rref,
                 int* __restrict__ row_flag, int ref_blocks, uint4* __restrict__ zp,
                 int64_t z16, uint8_t* __restrict__ ztail, int64_t z_tail) {
  if ((int)blockIdx.x >= ref_blocks) {
    const int64_t zb = blockIdx.x - ref_blocks, nzb = gridDim.x - ref_blocks;
    for (int64_t i = zb * kThreads + threadIdx.x; i < z16; i += nzb * kThreads)
      zp[i] = make_uint4(0, 0, 0, 0);
    if (zb == 0)
      for (int64_t i = threadIdx.x; i < z_tail; i += kThreads) ztail[i] = 0;
    return;
  }
  const int n_rows = min(*n_rows_ptr, max_rows);
  const int lane = threadIdx.x & 63;
  for (int j = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); j < n_rows;
       j += ref_blocks * (kThreads / 64)) {
    const int64_t r = row_idx[j];
    const int tg = tgt[j];
    float acc = 0.f;
    const bool ok = r >= 0 && r < n_tokens && tg >= 0 && tg < V;
    if (ok) {
      const bf16_t* hr = hidden + r * H;
      const bf16_t* wr = W + (int64_t)tg * H;
      for (int k = lane * 8; k < H; k += 512) {
        const uint4 x = *reinterpret_cast<const uint4*>(hr + k);
        const uint4 y = *reinterpret_cast<const uint4*>(wr + k);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc += __uint_as_float(xs[q] << 16) * __uint_as_float(ys[q] << 16);
          acc += __uint_as_float(xs[q] & 0xFFFF0000u) * __uint_as_float(ys[q] & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) {
      float z = acc, dc;
      if (softcap > 0.f) z = softcap_fwd(z, softcap, inv_softcap, &dc);
      rref[j] = ok ? z * kLog2e : 0.f;
      row_flag[j] = 0;
    }
  }
}

// Turns the forward pass's stash into G: entry v of row m becomes
// w_m 2^(rho - lse2_m) times the stashed 2^(s - rho) zhat' (rho: the
// reference the forward pass used for the half tile holding v, R_m or the
// half's maximum, decided again here by the same test; so the factor is
// w_m p zhat'), and the target entry w_m (p - 1) zhat' from the capped target
// logit.  `which` selects the rows: those the forward pass flagged (1), the
// others (0; they keep the stash until then, and their dH is finished by
// scatter_kernel), or all (-1).  One block per row at a time (so that rows
// left out cost one flag read), 16-byte groups of eight entries per thread.
constexpr int kScaleSeg = kThreads * 8;

// The loss: a fixed-order sum of the merge kernel's block sums by one block
// of kThreads threads (strided per thread, then a tree), whichever kernel
// runs it.
__device__ __forceinline__ void sum_block_sums(const double* __restrict__ block_sums, int n,
                                               float* __restrict__ loss, double* s) {
  double t = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) t += block_sums[i];
  s[threadIdx.x] = t;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) s[threadIdx.x] += s[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)s[0];
}

__global__ void __launch_bounds__(kThreads)
stash_scale_kernel(bf16_t* __restrict__ G, int64_t ldg, const float2* __restrict__ partial,
                   int n_part, int half, int max_rows, const float* __restrict__ lse, const float* __restrict__ ztgt,
                   const int32_t* __restrict__ tgt, const float* __restrict__ w,
                   const int32_t* __restrict__ n_rows_ptr, int V, float inv_softcap,
                   const float* __restrict__ rref, const int* __restrict__ row_flag,
                   int which, const double* __restrict__ block_sums, int n_bsum,
                   float* __restrict__ loss) {
  // (with block_sums) block 0 also sums the loss, saving its own launch
  if (block_sums && blockIdx.x == 0) {
    __shared__ double s[kThreads];
    sum_block_sums(block_sums, n_bsum, loss, s);
  }
  const int n_rows = min(*n_rows_ptr, max_rows);
  for (int m = blockIdx.x; m < n_rows; m += gridDim.x) {
    if (which >= 0 && row_flag[m] != which) continue;
    const float lse2 = lse[m] * kLog2e;
    const float wm = w[m];
    const float R = rref[m];
    const int tg = tgt[m];
    float gt = 0.f;  // the target entry
    if (tg >= 0 && tg < V) {
      const float zt2 = ztgt[m];
      float dc = 1.f;
      if (inv_softcap > 0.f) {
        const float th = zt2 * kLn2 * inv_softcap;
        dc = 1.f - th * th;
      }
      gt = (__builtin_amdgcn_exp2f(zt2 - lse2) - 1.f) * dc * wm;
    }
    uint4* grow = reinterpret_cast<uint4*>(G + (int64_t)m * ldg);
    // the columns the partials cover (n_part partials of `half` entries;
    // the stash beyond them, if any, lies past the vocabulary and is not read)
    const int vend = (int)min(ldg, (int64_t)n_part * half);
    // four 16-byte groups in flight per thread
    for (int v0 = (int)threadIdx.x * 8; v0 < vend; v0 += 4 * kScaleSeg) {
      uint4 in[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int v = v0 + b * kScaleSeg;
        if (v < vend) in[b] = grow[v / 8];
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int v = v0 + b * kScaleSeg;
        if (v >= vend) break;
        const float mh = partial[(int64_t)m * n_part + v / half].x;
        const float rho = mh - R > kStashSpan ? mh : R;
        const float f = wm * __builtin_amdgcn_exp2f(rho - lse2);
        const uint32_t wd[4] = {in[b].x, in[b].y, in[b].z, in[b].w};
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = __uint_as_float(wd[k] << 16) * f;
          x[2 * k + 1] = __uint_as_float(wd[k] & 0xFFFF0000u) * f;
        }
        const int dt = tg - v;
        if ((unsigned)dt < 8u && tg < V) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = dt == e ? gt : x[e];
        }
        grow[v / 8] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                 pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads)
loss_kernel(const double* __restrict__ block_sums, int n, float* __restrict__ loss) {
  __shared__ double s[kThreads];
  sum_block_sums(block_sums, n, loss, s);
}

__global__ void set_float_kernel(float* p, float v) { *p = v; }

__global__ void zero_kernel(uint4* __restrict__ p, int64_t n16, uint8_t* __restrict__ tail,
                            int64_t n_tail) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < n_tail; i += blockDim.x) tail[i] = 0;
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

// Rows whose dH slices were formed from the stash q (relative to the row's
// reference R) rather than from G.  Off the target, G = f q with the row
// factor f = w 2^(R - lse2); at the target t, G_t = w (p_t - 1) zhat'_t.  The
// slices hold sum_v q_v W_v in fp32, so dH = f (sum - q_t W_t) + G_t W_t,
// with q_t the stashed bf16 entry itself: its product with W_t is exact in
// fp32 and is taken out before the scaling.
struct StashFix {
  const float* rref;
  const int* row_flag;  // rows flagged here were finished by the scaling pass
  const float* lse;
  const float* ztgt;
  const float* w;
  const int32_t* tgt;
  const bf16_t* G;
  int64_t ldg;
  const bf16_t* W;
  int V;
  float inv_softcap;
};

// d_hidden[row_idx[j]] = sum over the K-slices of dH[j] (with the stash
// correction for rows that need it), for every scored row.
template <typename T>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(const float* __restrict__ part, int H, int grid, int v_span,
               const int32_t* __restrict__ row_idx, const int32_t* __restrict__ n_rows_ptr,
               int max_rows, int64_t n_tokens, T* __restrict__ d_hidden, StashFix fx) {
  const int n_rows = min(*n_rows_ptr, max_rows);
  // (the dH product's tile grid and split, as dh_kernel counts them)
  const int64_t tiles = (int64_t)((n_rows + kDhRows - 1) / kDhRows) * ((H + kTile - 1) / kTile);
  const int S = dh_splits(tiles, grid, (v_span + kBK - 1) / kBK);
  const int64_t slice = (int64_t)max_rows * H;
  for (int j = blockIdx.x; j < n_rows; j += gridDim.x) {
    const int64_t r = row_idx[j];
    if (r < 0 || r >= n_tokens) continue;
    float f = 1.f, qt = 0.f, gt = 0.f;
    const bf16_t* wt = nullptr;
    if (fx.rref && fx.row_flag[j] == 0) {
      const float lse2 = fx.lse[j] * kLog2e;
      const float wm = fx.w[j];
      f = wm * __builtin_amdgcn_exp2f(fx.rref[j] - lse2);
      const int tg = fx.tgt[j];
      if (tg >= 0 && tg < fx.V) {
        const float zt2 = fx.ztgt[j];
        float dc = 1.f;
        if (fx.inv_softcap > 0.f) {
          const float th = zt2 * kLn2 * fx.inv_softcap;
          dc = 1.f - th * th;
        }
        qt = (float)fx.G[(int64_t)j * fx.ldg + tg];
        gt = wm * (__builtin_amdgcn_exp2f(zt2 - lse2) - 1.f) * dc;
        wt = fx.W + (int64_t)tg * H;
      }
    }
    // four consecutive columns per thread (H is a multiple of 64)
    for (int h = 4 * (int)threadIdx.x; h < H; h += 4 * kThreads) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < S; ++k) {
        const float4 p = *reinterpret_cast<const float4*>(part + k * slice + (int64_t)j * H + h);
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
      }
      float d[4] = {f * acc.x, f * acc.y, f * acc.z, f * acc.w};
      if (wt) {
        const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
        const uint2 wb = *reinterpret_cast<const uint2*>(wt + h);
        const float wv[4] = {__uint_as_float(wb.x << 16), __uint_as_float(wb.x & 0xFFFF0000u),
                             __uint_as_float(wb.y << 16), __uint_as_float(wb.y & 0xFFFF0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = f * fmaf(-qt, wv[e], a4[e]) + gt * wv[e];
      }
      if constexpr (std::is_same<T, bf16_t>::value) {
        *reinterpret_cast<uint2*>(d_hidden + r * H + h) =
            make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) d_hidden[r * H + h + e] = from_f32<T>(d[e]);
      }
    }
  }
}

// --------------------------------------------------------------------------
// fp32 path: plain per-row dot products on the vector ALUs.
// --------------------------------------------------------------------------
struct F32Args {
  const float* W;
  const float* hidden;
  int64_t n_tokens;
  int H;
  int V;
  const int32_t* row_idx;
  const int32_t* tgt;
  const float* w;
  const int32_t* n_rows;
  int max_rows;
  float softcap;
  float inv_softcap;
  float2* partial;  // [max_rows][n_part], one (max, sum) per 256-entry tile
  int n_part;       // ceil(V/kTile)
  float* ztgt;
  const float* lse;
  float* G;  // [max_rows][V]
};

template <bool kGrad>
__global__ void __launch_bounds__(kThreads) f32_logits_kernel(F32Args a) {
  __shared__ float2 red[kThreads / 64];
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int m = blockIdx.x;
  if (m >= n_rows) return;
  const int64_t r = a.row_idx[m];
  const bool row_ok = r >= 0 && r < a.n_tokens;
  const int v = blockIdx.y * kThreads + threadIdx.x;
  const bool vok = v < a.V;
  float z = 0.f;
  if (vok && row_ok) {
    const float* h = a.hidden + r * a.H;
    const float* wr = a.W + (int64_t)v * a.H;
    for (int k = 0; k < a.H; ++k) z = fmaf(h[k], wr[k], z);
  }
  float dc = 1.f;
  if (a.softcap > 0.f) z = softcap_fwd(z, a.softcap, a.inv_softcap, &dc);
  const int tg = a.tgt[m];
  if (!kGrad) {
    if (vok && v == tg) a.ztgt[m] = z * kLog2e;
    const float s = vok ? z * kLog2e : -INFINITY;
    float mx = s;
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float e = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s - mx);
    for (int off = 32; off >= 1; off >>= 1) e += __shfl_xor(e, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(mx, e);
    __syncthreads();
    if (threadIdx.x == 0) {
      float M = -INFINITY;
      for (int i = 0; i < kThreads / 64; ++i) M = fmaxf(M, red[i].x);
      float S = 0.f;
      if (M != -INFINITY)
        for (int i = 0; i < kThreads / 64; ++i)
          S += red[i].y * __builtin_amdgcn_exp2f(red[i].x - M);
      a.partial[(int64_t)m * a.n_part + blockIdx.y] = make_float2(M, S);
    }
  } else if (vok) {
    float p = __builtin_amdgcn_exp2f(z * kLog2e - a.lse[m] * kLog2e);
    if (v == tg) p -= 1.f;
    a.G[(int64_t)m * a.V + v] = p * dc * a.w[m];
  }
}

__global__ void __launch_bounds__(kThreads)
f32_dh_kernel(F32Args a, float* __restrict__ d_hidden) {
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int m = blockIdx.x;
  if (m >= n_rows) return;
  const int64_t r = a.row_idx[m];
  if (r < 0 || r >= a.n_tokens) return;
  const int h = blockIdx.y * kThreads + threadIdx.x;
  if (h >= a.H) return;
  const float* g = a.G + (int64_t)m * a.V;
  float s = 0.f;
  for (int v = 0; v < a.V; ++v) s = fmaf(g[v], a.W[(int64_t)v * a.H + h], s);
  d_hidden[r * a.H + h] = s;
}

// --------------------------------------------------------------------------
// Workspace layout.
// --------------------------------------------------------------------------
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t partial, ztgt, lse, bsum, rref, flag, Hs, part, G, total;
  int n_vt, n_bsum;
};

// Fixed part of the layout; G gets whatever follows.  `dw`: room for the
// gathered scored rows of the head-weight gradient.
Layout fixed_layout(int64_t max_rows, int H, int V, int dtype, bool grad, bool dw = false) {
  Layout L{};
  L.n_vt = (V + kTile - 1) / kTile;
  L.n_bsum = (int)((max_rows + kMergeRows - 1) / kMergeRows);
  size_t off = 0;
  L.partial = off; off = align_up(off + (size_t)2 * L.n_vt * max_rows * sizeof(float2));
  L.ztgt = off;    off = align_up(off + (size_t)max_rows * sizeof(float));
  L.lse = off;     off = align_up(off + (size_t)max_rows * sizeof(float));
  L.bsum = off;    off = align_up(off + (size_t)std::max(L.n_bsum, 1) * sizeof(double));
  L.rref = off;    off = align_up(off + (size_t)max_rows * sizeof(float));
  L.flag = off;    off = align_up(off + (size_t)max_rows * sizeof(int));
  L.Hs = off;
  if (dw) off = align_up(off + (size_t)max_rows * H * sizeof(bf16_t));
  L.part = L.G = off;
  if (grad && dtype == MDLM_BF16) {
    L.part = off;
    off = align_up(off + (size_t)kMaxSplit * max_rows * H * sizeof(float));
    L.G = off;
  } else if (grad) {
    L.G = off;
    off = align_up(off + (size_t)max_rows * V * sizeof(float));
  }
  L.total = off;
  return L;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

// The preferred workspace holds G for the whole vocabulary, so the gradient
// runs as one chunk; the minimum holds one 256-wide vocabulary chunk.
size_t head_ce_workspace_bytes(int64_t max_rows, int32_t H, int32_t V, int32_t dtype,
                               bool minimal, bool dw) {
  Layout L = fixed_layout(max_rows, H, V, dtype, true, dw);
  if (dtype != MDLM_BF16 || max_rows == 0) return L.total;
  const int64_t vc = minimal ? kTile : round_up(V, kTile);
  return L.total + align_up((size_t)max_rows * vc * sizeof(bf16_t));
}

hipError_t launch_head_ce(const HeadCeArgs& x, hipStream_t stream) {
  const bool want_dh = x.d_hidden != nullptr;
  const bool want_dw = x.dW != nullptr;  // (bf16 only; checked by the caller)
  const bool grad = want_dh || want_dw;
  const int64_t max_rows = x.max_rows;
  char* ws = reinterpret_cast<char*>(x.workspace);
  const size_t elt = x.dtype == MDLM_BF16 ? 2 : 4;

  // d_hidden = 0: its own launch here, or (bf16 with the stash) in the
  // spare blocks of stash_ref_kernel below
  const size_t dh_bytes = want_dh ? (size_t)x.n_tokens * x.H * elt : 0;
  const int64_t dh16 = (int64_t)(dh_bytes / 16), dh_tail = (int64_t)(dh_bytes % 16);
  const unsigned dh_blocks =
      (unsigned)std::max<int64_t>(1, std::min<int64_t>((dh16 + 255) / 256, 4096));
  uint8_t* dh_tail_ptr = reinterpret_cast<uint8_t*>(x.d_hidden) + dh16 * 16;
  auto zero_dh = [&]() {
    if (dh_bytes)
      zero_kernel<<<dh_blocks, 256, 0, stream>>>(reinterpret_cast<uint4*>(x.d_hidden), dh16,
                                                 dh_tail_ptr, dh_tail);
  };
  if (want_dw && max_rows == 0) {
    // no kernel below runs: dW = 0 here (otherwise dw_kernel writes every
    // entry, zeros included, whatever the device row count)
    const size_t bytes = (size_t)x.V * x.H * sizeof(float);
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t tail = (int64_t)(bytes % 16);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n16 + 255) / 256, 4096));
    zero_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<uint4*>(x.dW), n16,
                                          reinterpret_cast<uint8_t*>(x.dW) + n16 * 16, tail);
  }
  if (max_rows == 0) {
    zero_dh();
    set_float_kernel<<<1, 1, 0, stream>>>(x.loss, 0.f);
    return hipGetLastError();
  }

  Layout L = fixed_layout(max_rows, x.H, x.V, x.dtype, grad, want_dw);
  float2* partial = reinterpret_cast<float2*>(ws + L.partial);
  float* ztgt = reinterpret_cast<float*>(ws + L.ztgt);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  double* bsum = reinterpret_cast<double*>(ws + L.bsum);
  const float inv_cap = x.softcap > 0.f ? 1.0f / x.softcap : 0.f;

  int device = 0, cus = kGrid;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    cus = kGrid;
  const int grid = std::max(8, std::min(kGrid, cus / 8 * 8));

  // bf16 gradient: vocabulary chunks sized by the workspace given.  When G
  // holds the whole vocabulary the forward pass stashes the unnormalised
  // softmax there and the gradient needs no second logits pass.
  int64_t vc = 0;
  if (grad && x.dtype == MDLM_BF16) {
    const size_t g_room = x.workspace_bytes - L.total;
    vc = (int64_t)(g_room / ((size_t)max_rows * sizeof(bf16_t))) / kTile * kTile;
    vc = std::min<int64_t>(vc, round_up(x.V, kTile));
  }
  const bool stash = MDLM_STASH && grad && x.dtype == MDLM_BF16 && vc >= x.V;
  if (!stash) zero_dh();
  // The bf16 forward pass without a softcap takes vocabulary tiles of 320
  // rows (five 32-row blocks per wave), with a softcap 256: one partial per
  // wave's half of a tile, `half` entries each.  (The gradient recompute
  // reads only the log-sum-exp and the target logit.)
  const bool wide = MDLM_WIDE_TILE && x.dtype == MDLM_BF16 && x.softcap <= 0.f;
  const int half = wide ? 160 : kTile / 2;
  const int n_part_f = 2 * (int)((x.V + 2 * half - 1) / (2 * half));
  bf16_t* G = reinterpret_cast<bf16_t*>(ws + L.G);
  float* rref = reinterpret_cast<float*>(ws + L.rref);
  int* row_flag = reinterpret_cast<int*>(ws + L.flag);

  if (x.dtype == MDLM_BF16) {
    LogitsArgs la{};
    la.W = reinterpret_cast<const bf16_t*>(x.W);
    la.hidden = reinterpret_cast<const bf16_t*>(x.hidden);
    la.n_tokens = x.n_tokens;
    la.H = x.H;
    la.V = x.V;
    la.row_idx = x.row_idx;
    la.tgt = x.tgt;
    la.w = x.w;
    la.n_rows = x.n_rows;
    la.max_rows = (int)max_rows;
    la.softcap = x.softcap;
    la.inv_softcap = inv_cap;
    la.v_begin = 0;
    la.v_end = x.V;
    la.partial = partial;
    la.n_part = n_part_f;
    la.ztgt = ztgt;
    la.G = G;
    la.ldg = vc;
    la.rref = rref;
    la.row_flag = row_flag;
    if (stash) {
      const int ref_blocks = (int)std::min<int64_t>((max_rows + 3) / 4, 16384);
      const unsigned zb = dh_bytes ? dh_blocks : 0;
      stash_ref_kernel<<<(unsigned)ref_blocks + zb, kThreads, 0, stream>>>(
          la.hidden, la.W, x.H, x.V, x.row_idx, x.tgt, x.n_rows, (int)max_rows, x.n_tokens,
          x.softcap, inv_cap, rref, row_flag, ref_blocks,
          reinterpret_cast<uint4*>(x.d_hidden), dh16, dh_tail_ptr, dh_tail);
      if (x.softcap > 0.f)
        logits_kernel<false, true, true><<<grid, kGemmThreads, 0, stream>>>(la);
      else if (wide)
        logits_kernel<false, false, true, 5><<<grid, kGemmThreads, 0, stream>>>(la);
      else
        logits_kernel<false, false, true><<<grid, kGemmThreads, 0, stream>>>(la);
    } else if (x.softcap > 0.f) {
      logits_kernel<false, true><<<grid, kGemmThreads, 0, stream>>>(la);
    } else if (wide) {
      logits_kernel<false, false, false, 5><<<grid, kGemmThreads, 0, stream>>>(la);
    } else {
      logits_kernel<false, false><<<grid, kGemmThreads, 0, stream>>>(la);
    }
  } else {
    F32Args fa{};
    fa.W = reinterpret_cast<const float*>(x.W);
    fa.hidden = reinterpret_cast<const float*>(x.hidden);
    fa.n_tokens = x.n_tokens;
    fa.H = x.H;
    fa.V = x.V;
    fa.row_idx = x.row_idx;
    fa.tgt = x.tgt;
    fa.w = x.w;
    fa.n_rows = x.n_rows;
    fa.max_rows = (int)max_rows;
    fa.softcap = x.softcap;
    fa.inv_softcap = inv_cap;
    fa.partial = partial;
    fa.n_part = L.n_vt;
    fa.ztgt = ztgt;
    dim3 g((unsigned)max_rows, (unsigned)L.n_vt);
    f32_logits_kernel<false><<<g, kThreads, 0, stream>>>(fa);
  }
  // (bf16: one partial per half tile; fp32: one per 256-entry tile)
  const int n_part = x.dtype == MDLM_BF16 ? n_part_f : L.n_vt;
  merge_kernel<<<L.n_bsum, kThreads, 0, stream>>>(partial, n_part, (int)max_rows, ztgt, x.tgt,
                                                  x.V, x.w, x.n_rows, lse, x.row_ce, bsum);
  // with the stash the loss is summed by the first scaling launch below
  if (!stash) loss_kernel<<<1, kThreads, 0, stream>>>(bsum, L.n_bsum, x.loss);
  if (!grad) return hipGetLastError();

  if (x.dtype == MDLM_F32) {
    F32Args fa{};
    fa.W = reinterpret_cast<const float*>(x.W);
    fa.hidden = reinterpret_cast<const float*>(x.hidden);
    fa.n_tokens = x.n_tokens;
    fa.H = x.H;
    fa.V = x.V;
    fa.row_idx = x.row_idx;
    fa.tgt = x.tgt;
    fa.w = x.w;
    fa.n_rows = x.n_rows;
    fa.max_rows = (int)max_rows;
    fa.softcap = x.softcap;
    fa.inv_softcap = inv_cap;
    fa.lse = lse;
    fa.G = reinterpret_cast<float*>(ws + L.G);
    dim3 g((unsigned)max_rows, (unsigned)L.n_vt);
    f32_logits_kernel<true><<<g, kThreads, 0, stream>>>(fa);
    dim3 g2((unsigned)max_rows, (unsigned)((x.H + kThreads - 1) / kThreads));
    f32_dh_kernel<<<g2, kThreads, 0, stream>>>(fa, reinterpret_cast<float*>(x.d_hidden));
    return hipGetLastError();
  }

  float* part = reinterpret_cast<float*>(ws + L.part);
  // With the stash: the rows the forward pass flagged become G here; the
  // others keep the stash through the dH product (scatter_kernel finishes
  // their dH) and become G only before a dW product, which needs G itself.
  auto scale_rows = [&](int which, bool with_loss) {
    const unsigned sgrid = (unsigned)std::min<int64_t>(max_rows, (int64_t)cus * 8);
    stash_scale_kernel<<<sgrid, kThreads, 0, stream>>>(
        G, vc, partial, n_part_f, half, (int)max_rows, lse, ztgt, x.tgt, x.w, x.n_rows, x.V,
        inv_cap, rref, row_flag, which, with_loss ? bsum : nullptr, L.n_bsum, x.loss);
  };
  if (stash) scale_rows(want_dh ? 1 : -1, true);

  LogitsArgs la{};
  la.W = reinterpret_cast<const bf16_t*>(x.W);
  la.hidden = reinterpret_cast<const bf16_t*>(x.hidden);
  la.n_tokens = x.n_tokens;
  la.H = x.H;
  la.V = x.V;
  la.row_idx = x.row_idx;
  la.tgt = x.tgt;
  la.w = x.w;
  la.n_rows = x.n_rows;
  la.max_rows = (int)max_rows;
  la.softcap = x.softcap;
  la.inv_softcap = inv_cap;
  la.lse = lse;
  la.ztgt = ztgt;
  la.G = G;
  la.ldg = vc;

  DwArgs wa{};
  bf16_t* Hs = reinterpret_cast<bf16_t*>(ws + L.Hs);
  if (want_dw) {
    gather_rows_kernel<<<(unsigned)std::min<int64_t>(max_rows, 65535), kThreads, 0, stream>>>(
        la.hidden, x.row_idx, x.n_rows, (int)max_rows, x.n_tokens, x.H, Hs);
    wa.G = G;
    wa.ldg = vc;
    wa.Hs = Hs;
    wa.H = x.H;
    wa.n_rows = x.n_rows;
    wa.max_rows = (int)max_rows;
    wa.dW = x.dW;
  }

  DhArgs da{};
  da.G = G;
  da.ldg = vc;
  da.W = la.W;
  da.H = x.H;
  da.n_rows = x.n_rows;
  da.max_rows = (int)max_rows;
  da.part = part;

  // every chunk uses the same slice count (it depends on the chunk width only
  // through the number of K steps, which is at least kMaxSplit unless the
  // chunk is narrower than 512)
  auto scatter = [&](const StashFix& fix) {
    scatter_kernel<bf16_t><<<(unsigned)std::min<int64_t>(max_rows, 65536), kThreads, 0,
                             stream>>>(part, x.H, grid, (int)std::min<int64_t>(vc, x.V),
                                       x.row_idx, x.n_rows, (int)max_rows, x.n_tokens,
                                       reinterpret_cast<bf16_t*>(x.d_hidden), fix);
  };

  if (stash) {
    // one chunk: G (or the stash) spans the vocabulary
    if (want_dh) {
      da.v_begin = 0;
      da.v_end = x.V;
      da.accumulate = 0;
      dh_kernel<<<grid, kGemmThreads, 0, stream>>>(da);
      StashFix fix{};
      fix.rref = rref;
      fix.row_flag = row_flag;
      fix.lse = lse;
      fix.ztgt = ztgt;
      fix.w = x.w;
      fix.tgt = x.tgt;
      fix.G = G;
      fix.ldg = vc;
      fix.W = la.W;
      fix.V = x.V;
      fix.inv_softcap = inv_cap;
      scatter(fix);  // (reads the stashed target entries: before they are scaled)
    }
    if (want_dw) {
      if (want_dh) scale_rows(0, false);
      wa.v_begin = 0;
      wa.v_end = x.V;
      dw_kernel<<<grid, kGemmThreads, 0, stream>>>(wa);
    }
    return hipGetLastError();
  }

  int chunk = 0;
  for (int64_t v0 = 0; v0 < x.V; v0 += vc, ++chunk) {
    const int v1 = (int)std::min<int64_t>(x.V, v0 + vc);
    la.v_begin = (int)v0;
    la.v_end = v1;
    if (x.softcap > 0.f)
      logits_kernel<true, true><<<grid, kGemmThreads, 0, stream>>>(la);
    else
      logits_kernel<true, false><<<grid, kGemmThreads, 0, stream>>>(la);
    if (want_dh) {
      da.v_begin = (int)v0;
      da.v_end = v1;
      da.accumulate = chunk > 0;
      dh_kernel<<<grid, kGemmThreads, 0, stream>>>(da);
    }
    if (want_dw) {
      wa.v_begin = (int)v0;
      wa.v_end = v1;
      dw_kernel<<<grid, kGemmThreads, 0, stream>>>(wa);
    }
  }
  if (want_dh) scatter(StashFix{});
  return hipGetLastError();
}

}  // namespace mdlm
