// y = g x with a device scalar g: the upstream gradient applied to d_hidden.
//
// LLaDA-8B-MDLM-LoRA card, "Training" table, "Objective" row: the loss is
// what the trainer backpropagates through; by the chain rule the gradient
// of g * loss is g * d_hidden, and the fused call forms d_hidden for g = 1.
// g is read on the device, so a backward pass needs no host read of it.
#include "mdlm_internal.h"

#include <algorithm>

namespace mdlm {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16_t;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16_t a = (bf16_t)lo, b = (bf16_t)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Eight bf16 entries per 16-byte word, each product in fp32 rounded once to
// bf16 (ties to even); the entries past the last whole word one at a time.
__global__ void __launch_bounds__(kThreads)
scale_bf16_kernel(const uint4* x, uint4* y, int64_t n,  // (y may be x)
                  const float* __restrict__ scale) {
  const float f = *scale;
  const int64_t n16 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = x[i];
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r[k] = pack2(__uint_as_float(wd[k] << 16) * f, __uint_as_float(wd[k] & 0xFFFF0000u) * f);
    y[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
  if (blockIdx.x == 0) {
    const bf16_t* xs = reinterpret_cast<const bf16_t*>(x);
    bf16_t* ys = reinterpret_cast<bf16_t*>(y);
    for (int64_t i = n16 * 8 + threadIdx.x; i < n; i += kThreads) ys[i] = (bf16_t)((float)xs[i] * f);
  }
}

// Four fp32 entries per 16-byte word, then the tail.
__global__ void __launch_bounds__(kThreads)
scale_f32_kernel(const float4* x, float4* y, int64_t n,  // (y may be x)
                 const float* __restrict__ scale) {
  const float f = *scale;
  const int64_t n16 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const float4 v = x[i];
    y[i] = make_float4(v.x * f, v.y * f, v.z * f, v.w * f);
  }
  if (blockIdx.x == 0) {
    const float* xs = reinterpret_cast<const float*>(x);
    float* ys = reinterpret_cast<float*>(y);
    for (int64_t i = n16 * 4 + threadIdx.x; i < n; i += kThreads) ys[i] = xs[i] * f;
  }
}

}  // namespace

hipError_t launch_scale(const void* x, void* y, int32_t dtype, int64_t n, const float* scale,
                        hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t words = n / (dtype == MDLM_BF16 ? 8 : 4);
  const unsigned grid =
      (unsigned)std::max<int64_t>(1, std::min<int64_t>((words + kThreads - 1) / kThreads, 8192));
  if (dtype == MDLM_BF16)
    scale_bf16_kernel<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x),
                                                     reinterpret_cast<uint4*>(y), n, scale);
  else
    scale_f32_kernel<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const float4*>(x),
                                                    reinterpret_cast<float4*>(y), n, scale);
  return hipGetLastError();
}

}  // namespace mdlm
