// The input of an MoE layer taken from a residual stream h (fp32 [T][d]):
// bf16(h) as it is, or through the pre-MoE norm.
//
// The pages name RMSNorm (per-head QK RMSNorm in the attention of "feat(laguna):
// Laguna-S-2.1 decode on the CUDA engine", a fused add-RMSNorm op) but do not
// define the norm in front of the MoE block; the norm here is the standard
// RMSNorm, x = h / sqrt(mean(h^2) + eps) * gamma, rounded to bf16 (nearest
// even).
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {

// fp32 -> bf16 (round to nearest even) of n8 groups of 8 values.
__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* __restrict__ h, uint16_t* __restrict__ x,
                                                     size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4* hp = reinterpret_cast<const float4*>(h + 8 * i);
  const float4 a = hp[0], b = hp[1];
  *reinterpret_cast<u32x4*>(x + 8 * i) =
      u32x4{float_to_bf16_bits(a.x) | ((uint32_t)float_to_bf16_bits(a.y) << 16),
            float_to_bf16_bits(a.z) | ((uint32_t)float_to_bf16_bits(a.w) << 16),
            float_to_bf16_bits(b.x) | ((uint32_t)float_to_bf16_bits(b.y) << 16),
            float_to_bf16_bits(b.z) | ((uint32_t)float_to_bf16_bits(b.w) << 16)};
}

hipError_t launch_f32_to_bf16(const float* h, uint16_t* x, size_t n, hipStream_t st) {
  const size_t n8 = n / 8;
  hipLaunchKernelGGL(k_f32_to_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, h, x, n8);
  return hipGetLastError();
}

// RMSNorm, one workgroup of 256 threads per token.  Thread i sums the squares of the 8-value groups
// i, i + 256, ... in that order; the 256 sums meet across each wavefront (DPP steps) and then across
// the 4 wavefronts in LDS, in a fixed order, so the result does not depend on scheduling.  Then
// x = bf16((h * r) * gamma) with r = 1 / sqrt(sum / d + eps) (IEEE square root and division).
__global__ __launch_bounds__(256) void k_rmsnorm_bf16(const float* __restrict__ h, const float* __restrict__ gamma,
                                                      float eps, uint16_t* __restrict__ x, int d) {
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = h + (size_t)blockIdx.x * d;
  const int n8 = d / 8;
  float ss = 0.f;
  for (int g = tid; g < n8; g += 256) {
    const float4 a = reinterpret_cast<const float4*>(row)[2 * g], b = reinterpret_cast<const float4*>(row)[2 * g + 1];
    ss = fmaf(a.x, a.x, ss); ss = fmaf(a.y, a.y, ss); ss = fmaf(a.z, a.z, ss); ss = fmaf(a.w, a.w, ss);
    ss = fmaf(b.x, b.x, ss); ss = fmaf(b.y, b.y, ss); ss = fmaf(b.z, b.z, ss); ss = fmaf(b.w, b.w, ss);
  }
  ss = wave_sum_hi(ss);  // valid in lanes 48..63
  if (lane == 63) part[wave] = ss;
  __syncthreads();
  const float total = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(total / (float)d + eps);
  uint16_t* out = x + (size_t)blockIdx.x * d;
  for (int g = tid; g < n8; g += 256) {
    const float4 a = reinterpret_cast<const float4*>(row)[2 * g], b = reinterpret_cast<const float4*>(row)[2 * g + 1];
    const float4 ga = reinterpret_cast<const float4*>(gamma)[2 * g], gb = reinterpret_cast<const float4*>(gamma)[2 * g + 1];
    *reinterpret_cast<u32x4*>(out + 8 * g) =
        u32x4{float_to_bf16_bits(a.x * r * ga.x) | ((uint32_t)float_to_bf16_bits(a.y * r * ga.y) << 16),
              float_to_bf16_bits(a.z * r * ga.z) | ((uint32_t)float_to_bf16_bits(a.w * r * ga.w) << 16),
              float_to_bf16_bits(b.x * r * gb.x) | ((uint32_t)float_to_bf16_bits(b.y * r * gb.y) << 16),
              float_to_bf16_bits(b.z * r * gb.z) | ((uint32_t)float_to_bf16_bits(b.w * r * gb.w) << 16)};
  }
}

hipError_t launch_rmsnorm_bf16(const float* h, const float* gamma, float eps, uint16_t* x, int T, int d,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm_bf16, dim3(T), dim3(256), 0, st, h, gamma, eps, x, d);
  return hipGetLastError();
}

}  // namespace moe
