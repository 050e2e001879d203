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
//   1. logits_kernel<fwd>: z = W h over 256x128 (vocab x row) tiles, K = H,
//      on bf16 MFMA with fp32 accumulation, operands staged through LDS.  The
//      epilogue caps, takes each row's (max, sum 2^(s-max)) over the tile's
//      256 vocabulary entries and picks the target logit.  Logits never leave
//      registers.
//   2. merge_kernel: per row, combine the per-tile partials into the
//      log-sum-exp and CE; per-block sums of w * CE in fp64.
//   3. loss_kernel: fixed-order sum of the block sums -> loss.
//   4. (gradient) for each vocabulary chunk [v0, v1):
//      logits_kernel<grad> recomputes the chunk's tiles and writes
//      G = w (softmax - onehot) zhat' as bf16 into a bounded workspace;
//      dh_kernel accumulates dH += G W over the chunk (tiles of 128 rows x 256
//      hidden columns, whole tiles per workgroup, the leftover tiles split
//      along K), dh_fixup_kernel sums the split tiles in a fixed order.
//   5. zero_kernel + scatter_kernel: d_hidden = 0, then d_hidden[row_idx[j]]
//      = dH[j] in the hidden dtype.
#include "mdlm_internal.h"

#include <math.h>

#include <algorithm>

namespace mdlm {
namespace {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kThreads = 256;
constexpr int kBK = 64;               // K elements per main-loop step
constexpr int kStride = kBK + 8;      // LDS row pitch in elements (144 bytes)
constexpr int kLA = 256, kLB = 128;   // logits tile: vocab rows x scored rows
constexpr int kDA = 128, kDB = 256;   // dH tile: scored rows x hidden columns
constexpr int kMergeRows = 4;         // rows per merge block (one per wave)
constexpr int kGrid = 256;            // persistent grid: one workgroup per CU
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr size_t kAlign = 256;

static_assert((kLA + kLB) == (kDA + kDB), "both GEMMs share one LDS footprint");
constexpr int kLdsElems = 2 * (kLA + kLB) * kStride;

__device__ __forceinline__ int logical_block() {
  // Consecutive logical ids on one XCD: the hardware hands workgroup b to XCD
  // b % 8, so ids are regrouped to let one XCD's concurrently running tiles
  // share operand rows in its L2.
  const int per_xcd = gridDim.x >> 3;
  return (gridDim.x & 7) ? (int)blockIdx.x
                         : (int)((blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3));
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

// One 64-deep K step of a wave's (32*NI) x (32*NJ) tile.  `as`/`bs` point at
// this lane's operand row in LDS (row = wave base + lane % 32, column offset
// (lane / 32) * 8).  Blocks whose mask bit is clear (rows past the end) are
// skipped; the masks are wave-uniform.
template <int NI, int NJ>
__device__ __forceinline__ void mma_step(const bf16_t* __restrict__ as,
                                         const bf16_t* __restrict__ bs,
                                         f32x16 (&acc)[NI][NJ], uint32_t imask,
                                         uint32_t jmask) {
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    bf16x8 af[NI], bfr[NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(as + i * 32 * kStride + kk * 16);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(bs + j * 32 * kStride + kk * 16);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (((imask >> i) & 1u) && ((jmask >> j) & 1u))
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0,
                                                              0);
  }
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
  float2* partial;  // fwd: [ceil(V/kLA)][max_rows] (max, sum) in log2 units
  float* ztgt;      // fwd: [max_rows] capped target logit
  const float* lse; // grad: [max_rows]
  bf16_t* G;        // grad: [max_rows][ldg], column = v - v_begin
  int64_t ldg;
};

template <bool kGrad>
__global__ void __launch_bounds__(kThreads, 1) logits_kernel(LogitsArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[kLdsElems];
  __shared__ float2 red[2][kLB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wa = wave >> 1, wb = wave & 1;
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int n_mt = (n_rows + kLB - 1) / kLB;
  const int n_vt = (a.v_end - a.v_begin + kLA - 1) / kLA;
  const int64_t n_tiles = (int64_t)n_mt * n_vt;
  const int KT = a.H / kBK;
  const bool capped = a.softcap > 0.f;
  const int kc = tid & 7, rsub = tid >> 3;

  for (int64_t t = logical_block(); t < n_tiles; t += gridDim.x) {
    const int vt = (int)(t / n_mt), mt = (int)(t % n_mt);
    const int v0 = a.v_begin + vt * kLA;
    const int m0 = mt * kLB;

    // ---- operand row pointers for this thread's global loads -------------
    const bf16_t* a_ptr = a.W + (int64_t)(v0 + rsub) * a.H + kc * 8;
    uint32_t a_ok = 0;
#pragma unroll
    for (int c = 0; c < kLA / 32; ++c)
      if (v0 + 32 * c + rsub < a.v_end) a_ok |= 1u << c;
    const bf16_t* b_ptr[kLB / 32];
#pragma unroll
    for (int c = 0; c < kLB / 32; ++c) {
      const int m = m0 + 32 * c + rsub;
      b_ptr[c] = nullptr;
      if (m < n_rows) {
        const int64_t r = a.row_idx[m];
        if (r >= 0 && r < a.n_tokens) b_ptr[c] = a.hidden + r * a.H + kc * 8;
      }
    }
    uint32_t imask = 0, jmask = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v0 + wa * 128 + 32 * i < a.v_end) imask |= 1u << i;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (m0 + wb * 64 + 32 * j < n_rows) jmask |= 1u << j;

    uint4 ra[kLA / 32], rb[kLB / 32];
    auto gload = [&](int k0) {
#pragma unroll
      for (int c = 0; c < kLA / 32; ++c)
        ra[c] = ((a_ok >> c) & 1u)
                    ? *reinterpret_cast<const uint4*>(a_ptr + (int64_t)c * 32 * a.H + k0)
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kLB / 32; ++c)
        rb[c] = b_ptr[c] ? *reinterpret_cast<const uint4*>(b_ptr[c] + k0)
                         : make_uint4(0, 0, 0, 0);
    };
    auto lstore = [&](int buf) {
      bf16_t* as = lds + buf * (kLA + kLB) * kStride;
      bf16_t* bs = as + kLA * kStride;
#pragma unroll
      for (int c = 0; c < kLA / 32; ++c)
        *reinterpret_cast<uint4*>(as + (32 * c + rsub) * kStride + kc * 8) = ra[c];
#pragma unroll
      for (int c = 0; c < kLB / 32; ++c)
        *reinterpret_cast<uint4*>(bs + (32 * c + rsub) * kStride + kc * 8) = rb[c];
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gload((kt + 1) * kBK);
      const bf16_t* base = lds + (kt & 1) * (kLA + kLB) * kStride;
      const bf16_t* as = base + (wa * 128 + (lane & 31)) * kStride + (lane >> 5) * 8;
      const bf16_t* bs = base + (kLA + wb * 64 + (lane & 31)) * kStride + (lane >> 5) * 8;
      mma_step<4, 2>(as, bs, acc, imask, jmask);
      if (kt + 1 < KT) lstore((kt + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    // Accumulator element e of block (i, j) on lane l holds vocabulary entry
    // v0 + wa*128 + 32i + 8(e/4) + 4(l/32) + e%4 for row m0 + wb*64 + 32j + l%32.
    const int vl = v0 + wa * 128 + 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wb * 64 + 32 * j + (lane & 31);
      const bool mvalid = m < n_rows;
      const int tg = mvalid ? a.tgt[m] : -1;
      if (!kGrad) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int v = vl + 32 * i + 8 * (e >> 2) + (e & 3);
            float zc = acc[i][j][e], dc;
            if (capped) zc = softcap_fwd(zc, a.softcap, a.inv_softcap, &dc);
            if (mvalid && v == tg) a.ztgt[m] = zc;
            const float s = v < a.v_end ? zc * kLog2e : -INFINITY;
            acc[i][j][e] = s;
            mx = fmaxf(mx, s);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        float sum = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f(acc[i][j][e] - mx);
        }
        sum += __shfl_xor(sum, 32, 64);
        if (lane < 32) red[wa][wb * 64 + 32 * j + lane] = make_float2(mx, sum);
      } else if (mvalid) {
        const float lse2 = a.lse[m] * kLog2e;
        const float wm = a.w[m];
        bf16_t* grow = a.G + (int64_t)m * a.ldg - a.v_begin;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float g[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int v = vl + 32 * i + 8 * q + r;
              float zc = acc[i][j][4 * q + r], dc = 1.f;
              if (capped) zc = softcap_fwd(zc, a.softcap, a.inv_softcap, &dc);
              float p = __builtin_amdgcn_exp2f(zc * kLog2e - lse2);
              if (v == tg) p -= 1.f;
              g[r] = v < a.v_end ? p * dc * wm : 0.f;
            }
            const int v = vl + 32 * i + 8 * q;
            *reinterpret_cast<uint2*>(grow + v) =
                make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
          }
      }
    }
    if (!kGrad) {
      __syncthreads();
      if (wa == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = wb * 64 + 32 * j + (lane & 31);
          const int m = m0 + col;
          if (lane < 32 && m < n_rows) {
            const float2 p0 = red[0][col], p1 = red[1][col];
            const float mx = fmaxf(p0.x, p1.x);
            float s = 0.f;
            if (mx != -INFINITY)
              s = p0.y * __builtin_amdgcn_exp2f(p0.x - mx) +
                  p1.y * __builtin_amdgcn_exp2f(p1.x - mx);
            a.partial[(int64_t)((v0 - a.v_begin) / kLA) * a.max_rows + m] = make_float2(mx, s);
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// dH += G W over one vocabulary chunk.
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
  float* dh;     // [max_rows][H] fp32
  float* slots;  // [kGrid][kDA * kDB] split-tile partials
  int accumulate;
};

// The 8x8 transpose of bf16 held as 8 rows of uint4 (row = v, 8 h each) into
// 8 rows of uint4 (row = h, 8 v each).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo_row = reinterpret_cast<const uint32_t*>(&in[2 * q])[s >> 1];
      const uint32_t hi_row = reinterpret_cast<const uint32_t*>(&in[2 * q + 1])[s >> 1];
      o[q] = (s & 1) ? ((lo_row >> 16) | (hi_row & 0xFFFF0000u))
                     : ((lo_row & 0xFFFFu) | (hi_row << 16));
    }
    out[s] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__device__ __forceinline__ void dh_tile(const DhArgs& a, bf16_t* lds, int n_rows, int n_mt,
                                        int64_t tile, int k_beg, int k_end, float* out,
                                        int64_t ld_out, bool to_slot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wa = wave >> 1, wb = wave & 1;
  const int mt = (int)(tile % n_mt), ht = (int)(tile / n_mt);
  const int m0 = mt * kDA, h0 = ht * kDB;
  const int kc = tid & 7, rsub = tid >> 3;
  // A = G rows (K contiguous)
  const bf16_t* a_ptr = a.G + (int64_t)(m0 + rsub) * a.ldg + kc * 8;
  uint32_t a_ok = 0;
#pragma unroll
  for (int c = 0; c < kDA / 32; ++c)
    if (m0 + 32 * c + rsub < n_rows) a_ok |= 1u << c;
  // B = W^T: this thread loads an 8 (v) x 8 (h) block and transposes it
  const int gv = lane & 7, gh = 8 * wave + (lane >> 3);
  const bool h_ok = h0 + 8 * gh < a.H;
  const bf16_t* b_ptr = a.W + (int64_t)(a.v_begin + 8 * gv) * a.H + h0 + 8 * gh;
  uint32_t imask = 0, jmask = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (m0 + wa * 64 + 32 * i < n_rows) imask |= 1u << i;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (h0 + wb * 128 + 32 * j < a.H) jmask |= 1u << j;

  uint4 ra[kDA / 32], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int c = 0; c < kDA / 32; ++c)
      ra[c] = ((a_ok >> c) & 1u)
                  ? *reinterpret_cast<const uint4*>(a_ptr + (int64_t)c * 32 * a.ldg + k0)
                  : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bool ok = h_ok && (a.v_begin + k0 + 8 * gv + r < a.v_end);
      rb[r] = ok ? *reinterpret_cast<const uint4*>(b_ptr + (int64_t)(k0 + r) * a.H)
                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    bf16_t* as = lds + buf * (kDA + kDB) * kStride;
    bf16_t* bs = as + kDA * kStride;
#pragma unroll
    for (int c = 0; c < kDA / 32; ++c)
      *reinterpret_cast<uint4*>(as + (32 * c + rsub) * kStride + kc * 8) = ra[c];
    uint4 tr[8];
    transpose8x8(rb, tr);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<uint4*>(bs + (8 * gh + s) * kStride + 8 * gv) = tr[s];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  gload(k_beg * kBK);
  lstore(0);
  __syncthreads();
  for (int kt = k_beg; kt < k_end; ++kt) {
    const int buf = (kt - k_beg) & 1;
    if (kt + 1 < k_end) gload((kt + 1) * kBK);
    const bf16_t* base = lds + buf * (kDA + kDB) * kStride;
    const bf16_t* as = base + (wa * 64 + (lane & 31)) * kStride + (lane >> 5) * 8;
    const bf16_t* bs = base + (kDA + wb * 128 + (lane & 31)) * kStride + (lane >> 5) * 8;
    mma_step<2, 4>(as, bs, acc, imask, jmask);
    if (kt + 1 < k_end) lstore(buf ^ 1);
    __syncthreads();
  }

  // acc element e of block (i, j) on lane l: row m0 + wa*64 + 32i + 8(e/4) +
  // 4(l/32) + e%4, column h0 + wb*128 + 32j + l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rl = wa * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cl = wb * 128 + 32 * j + (lane & 31);
        if (to_slot) {
          out[(int64_t)rl * kDB + cl] = acc[i][j][e];
        } else if (m0 + rl < n_rows && h0 + cl < a.H) {
          float* p = out + (int64_t)(m0 + rl) * ld_out + h0 + cl;
          *p = a.accumulate ? *p + acc[i][j][e] : acc[i][j][e];
        }
      }
    }
}

__device__ __forceinline__ void dh_schedule(int n_rows, int H, int v_begin, int v_end,
                                            int* n_mt, int64_t* T, int* KI, int64_t* full,
                                            int* R, int* SB) {
  *n_mt = (n_rows + kDA - 1) / kDA;
  const int n_ht = (H + kDB - 1) / kDB;
  *T = (int64_t)(*n_mt) * n_ht;
  *KI = (v_end - v_begin + kBK - 1) / kBK;
  *full = *T / gridDim.x;
  *R = (int)(*T % gridDim.x);
  *SB = *R ? (int)gridDim.x / *R : 0;
  if (*SB > *KI) *SB = *KI;
}

__global__ void __launch_bounds__(kThreads, 1) dh_kernel(DhArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[kLdsElems];
  const int n_rows = min(*a.n_rows, a.max_rows);
  int n_mt, KI, R, SB;
  int64_t T, full;
  dh_schedule(n_rows, a.H, a.v_begin, a.v_end, &n_mt, &T, &KI, &full, &R, &SB);
  if (T == 0 || KI == 0) return;
  const int lw = logical_block();
  // whole tiles: every workgroup runs the same K range at the same time
  for (int64_t r = 0; r < full; ++r)
    dh_tile(a, lds, n_rows, n_mt, r * gridDim.x + lw, 0, KI, a.dh, a.H, false);
  // leftover tiles, each split into SB K-slices
  if (R && lw < R * SB) {
    const int64_t tile = full * gridDim.x + lw / SB;
    const int s = lw % SB;
    const int kb = (int)((int64_t)KI * s / SB), ke = (int)((int64_t)KI * (s + 1) / SB);
    dh_tile(a, lds, n_rows, n_mt, tile, kb, ke, a.slots + (int64_t)lw * kDA * kDB, kDB, true);
  }
}

// Sums the K-slices of each leftover tile in slice order and adds them to dH.
__global__ void __launch_bounds__(kThreads) dh_fixup_kernel(DhArgs a, int grid) {
  const int n_rows = min(*a.n_rows, a.max_rows);
  const int n_mt = (n_rows + kDA - 1) / kDA;
  const int n_ht = (a.H + kDB - 1) / kDB;
  const int64_t T = (int64_t)n_mt * n_ht;
  const int KI = (a.v_end - a.v_begin + kBK - 1) / kBK;
  if (T == 0 || KI == 0) return;
  const int64_t full = T / grid;
  const int R = (int)(T % grid);
  int SB = R ? grid / R : 0;
  if (SB > KI) SB = KI;
  const int r = blockIdx.x;
  if (r >= R) return;
  const int64_t tile = full * grid + r;
  const int mt = (int)(tile % n_mt), ht = (int)(tile / n_mt);
  const int m0 = mt * kDA, h0 = ht * kDB;
  for (int idx = threadIdx.x; idx < kDA * kDB; idx += kThreads) {
    const int rl = idx / kDB, cl = idx % kDB;
    if (m0 + rl >= n_rows || h0 + cl >= a.H) continue;
    float s = 0.f;
    for (int k = 0; k < SB; ++k) s += a.slots[(int64_t)(r * SB + k) * kDA * kDB + idx];
    float* p = a.dh + (int64_t)(m0 + rl) * a.H + h0 + cl;
    *p = a.accumulate ? *p + s : s;
  }
}

// --------------------------------------------------------------------------
// Reductions.
// --------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
merge_kernel(const float2* __restrict__ partial, int n_vt, int max_rows,
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
    for (int t = lane; t < n_vt; t += 64) {
      const float2 p = partial[(int64_t)t * max_rows + j];
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
    const float lse = (mx + __log2f(s)) * kLn2;
    const int tg = tgt[j];
    const float ce = (tg >= 0 && tg < V) ? lse - ztgt[j] : NAN;
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

__global__ void __launch_bounds__(kThreads)
loss_kernel(const double* __restrict__ block_sums, int n, float* __restrict__ loss) {
  __shared__ double s[kThreads];
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

// d_hidden[row_idx[j]] = dH[j] for every scored row j.
template <typename T>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(const float* __restrict__ dh, int H, const int32_t* __restrict__ row_idx,
               const int32_t* __restrict__ n_rows_ptr, int max_rows, int64_t n_tokens,
               T* __restrict__ d_hidden) {
  const int n_rows = min(*n_rows_ptr, max_rows);
  for (int j = blockIdx.x; j < n_rows; j += gridDim.x) {
    const int64_t r = row_idx[j];
    if (r < 0 || r >= n_tokens) continue;
    for (int h = threadIdx.x; h < H; h += kThreads)
      d_hidden[r * H + h] = from_f32<T>(dh[(int64_t)j * H + h]);
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
  float2* partial;
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
    if (vok && v == tg) a.ztgt[m] = z;
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
      a.partial[(int64_t)blockIdx.y * a.max_rows + m] = make_float2(M, S);
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
  size_t partial, ztgt, lse, bsum, dh, slots, G, total;
  int64_t vc;   // vocabulary chunk width of the gradient pass
  int64_t ldg;  // row pitch of G in elements
  int n_vt, n_bsum;
};

// Fixed part of the layout; G gets whatever follows.
Layout fixed_layout(int64_t max_rows, int H, int V, int dtype, bool grad) {
  Layout L{};
  const int tile = dtype == MDLM_BF16 ? kLA : kThreads;
  L.n_vt = (V + tile - 1) / tile;
  L.n_bsum = (int)((max_rows + kMergeRows - 1) / kMergeRows);
  size_t off = 0;
  L.partial = off; off = align_up(off + (size_t)L.n_vt * max_rows * sizeof(float2));
  L.ztgt = off;    off = align_up(off + (size_t)max_rows * sizeof(float));
  L.lse = off;     off = align_up(off + (size_t)max_rows * sizeof(float));
  L.bsum = off;    off = align_up(off + (size_t)std::max(L.n_bsum, 1) * sizeof(double));
  L.dh = L.slots = L.G = off;
  if (grad && dtype == MDLM_BF16) {
    L.dh = off;    off = align_up(off + (size_t)max_rows * H * sizeof(float));
    L.slots = off; off = align_up(off + (size_t)kGrid * kDA * kDB * sizeof(float));
    L.G = off;
  } else if (grad) {
    L.G = off;
    off = align_up(off + (size_t)max_rows * V * sizeof(float));
  }
  L.total = off;
  return L;
}

// The bf16 gradient chunk prefers G to stay near 192 MiB so that it and the
// matching slice of W can be served from the 256 MiB Infinity Cache.
constexpr size_t kPreferredGBytes = 192ull << 20;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

size_t head_ce_workspace_bytes(int64_t max_rows, int32_t H, int32_t V, int32_t dtype,
                               bool minimal) {
  Layout L = fixed_layout(max_rows, H, V, dtype, true);
  if (dtype != MDLM_BF16 || max_rows == 0) return L.total;
  const int64_t vfull = round_up(V, kLA);
  int64_t vc = kLA;
  if (!minimal) {
    vc = (int64_t)(kPreferredGBytes / ((size_t)max_rows * sizeof(bf16_t))) / kLA * kLA;
    vc = std::max<int64_t>(kLA, std::min(vc, vfull));
  }
  return L.total + align_up((size_t)max_rows * vc * sizeof(bf16_t));
}

hipError_t launch_head_ce(const HeadCeArgs& x, hipStream_t stream) {
  const bool grad = x.d_hidden != nullptr;
  const int64_t max_rows = x.max_rows;
  char* ws = reinterpret_cast<char*>(x.workspace);
  const size_t elt = x.dtype == MDLM_BF16 ? 2 : 4;

  if (grad) {
    const size_t bytes = (size_t)x.n_tokens * x.H * elt;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t tail = (int64_t)(bytes % 16);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n16 + 255) / 256, 4096));
    if (bytes)
      zero_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<uint4*>(x.d_hidden), n16,
                                            reinterpret_cast<uint8_t*>(x.d_hidden) + n16 * 16,
                                            tail);
  }
  if (max_rows == 0) {
    set_float_kernel<<<1, 1, 0, stream>>>(x.loss, 0.f);
    return hipGetLastError();
  }

  Layout L = fixed_layout(max_rows, x.H, x.V, x.dtype, grad);
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
    la.ztgt = ztgt;
    logits_kernel<false><<<grid, kThreads, 0, stream>>>(la);
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
    fa.ztgt = ztgt;
    dim3 g((unsigned)max_rows, (unsigned)L.n_vt);
    f32_logits_kernel<false><<<g, kThreads, 0, stream>>>(fa);
  }
  merge_kernel<<<L.n_bsum, kThreads, 0, stream>>>(partial, L.n_vt, (int)max_rows, ztgt, x.tgt,
                                                  x.V, x.w, x.n_rows, lse, x.row_ce, bsum);
  loss_kernel<<<1, kThreads, 0, stream>>>(bsum, L.n_bsum, x.loss);
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

  // bf16 gradient: vocabulary chunks sized by the workspace given
  const size_t g_room = x.workspace_bytes - L.total;
  int64_t vc = (int64_t)(g_room / ((size_t)max_rows * sizeof(bf16_t))) / kLA * kLA;
  vc = std::min<int64_t>(vc, round_up(x.V, kLA));
  float* dh = reinterpret_cast<float*>(ws + L.dh);
  float* slots = reinterpret_cast<float*>(ws + L.slots);
  bf16_t* G = reinterpret_cast<bf16_t*>(ws + L.G);

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
  la.G = G;
  la.ldg = vc;

  DhArgs da{};
  da.G = G;
  da.ldg = vc;
  da.W = la.W;
  da.H = x.H;
  da.n_rows = x.n_rows;
  da.max_rows = (int)max_rows;
  da.dh = dh;
  da.slots = slots;

  int chunk = 0;
  for (int64_t v0 = 0; v0 < x.V; v0 += vc, ++chunk) {
    const int v1 = (int)std::min<int64_t>(x.V, v0 + vc);
    la.v_begin = (int)v0;
    la.v_end = v1;
    logits_kernel<true><<<grid, kThreads, 0, stream>>>(la);
    da.v_begin = (int)v0;
    da.v_end = v1;
    da.accumulate = chunk > 0;
    dh_kernel<<<grid, kThreads, 0, stream>>>(da);
    dh_fixup_kernel<<<grid, kThreads, 0, stream>>>(da, grid);
  }
  if (x.dtype == MDLM_BF16)
    scatter_kernel<bf16_t><<<(unsigned)std::min<int64_t>(max_rows, 65536), kThreads, 0, stream>>>(
        dh, x.H, x.row_idx, x.n_rows, (int)max_rows, x.n_tokens,
        reinterpret_cast<bf16_t*>(x.d_hidden));
  return hipGetLastError();
}

}  // namespace mdlm
