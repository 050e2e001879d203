// Measurement kernels: a one-pass streaming copy and an MFMA issue loop, the
// achievable-peak references for the loss path's roofline.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mdlm_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

constexpr int kChains = 8;  // independent accumulators per wave

__global__ void __launch_bounds__(512) mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int mdlm_probe_copy(const void* src, void* dst, int64_t n16, void* stream) {
  if (n16 <= 0) return 0;
  const int64_t blocks = (n16 + 255) / 256;
  copy_kernel<<<(unsigned)blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n16);
  return (int)hipGetLastError();
}

int mdlm_probe_mfma(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (blocks < 1 || blocks > 65535 || iters < 1) return (int)hipErrorInvalidValue;
  mfma_kernel<<<blocks, 512, 0, reinterpret_cast<hipStream_t>(stream)>>>(out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
