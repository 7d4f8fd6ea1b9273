// Router of the MoE expert layer: logits l = W_r x, sigmoid scores, and the
// biased top-k selection with unbiased, normalised weights.
//
// Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine"
// (thewafflehaus/butter pull request 69): a sigmoid top-10 router with a
// score-correction bias.  The bias only ranks (key = s + b); the weights are
// the chosen experts' sigmoid scores normalised to sum to 1; ties go to the
// lower expert id and the k choices are listed by descending key.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Small T: one wavefront per expert streams its router row once per group of
// 8 tokens (the row stays in L2 for the next group) and reduces each dot
// product across the wave.  Lane l reads 16 contiguous bytes of the row at
// 4l + 256m, so each load instruction covers 1 KB of the row.
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, const float* __restrict__ W,
                                                     float* __restrict__ logits, int T, int d, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float* wr = W + (size_t)e * d;
  for (int t0 = 0; t0 < T; t0 += 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int c = 4 * lane; c < d; c += 256) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (t0 + i < T) {
          const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + i) * d + c);
          float a = acc[i];
          a = fmaf(wv.x, bf16_bits_to_float(xv.x & 0xFFFFu), a);
          a = fmaf(wv.y, bf16_bits_to_float(xv.x >> 16), a);
          a = fmaf(wv.z, bf16_bits_to_float(xv.y & 0xFFFFu), a);
          a = fmaf(wv.w, bf16_bits_to_float(xv.y >> 16), a);
          acc[i] = a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = wave_sum(acc[i]);
      if (lane == 0 && t0 + i < T) logits[(size_t)(t0 + i) * E + e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Larger T: bf16 MFMA.  x is bf16 already; each fp32 router weight is split
// into hi = bf16(w) and lo = bf16(w - hi) so that two bf16 MFMAs reproduce
// the fp32 product to about 2^-17 relative.  A workgroup computes 64 tokens x
// 64 experts; wave w owns experts [16w, 16w+16) of the block and all 64
// tokens (four 16x16x32 MFMA tiles per K-step, hi and lo).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ W,
                                                     float* __restrict__ logits, int T, int d, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int t0 = blockIdx.x * 64;
  const int e0 = blockIdx.y * 64 + wave * 16;
  if (e0 >= E) return;  // whole wave idle: no barriers in this kernel
  const bool e_ok = (e0 + n) < E;
  const float* wrow = W + (size_t)(e_ok ? e0 + n : 0) * d + 8 * G;
  const uint16_t* xrow[4];
  bool t_ok[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = t0 + 16 * mt + n;
    t_ok[mt] = t < T;
    xrow[mt] = x + (size_t)(t_ok[mt] ? t : 0) * d + 8 * G;
  }
  floatx4 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d; k0 += 32) {
    float wv[8];
    if (e_ok) {
      const float4 w0 = *reinterpret_cast<const float4*>(wrow + k0);
      const float4 w1 = *reinterpret_cast<const float4*>(wrow + k0 + 4);
      wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
      wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) wv[i] = 0.f;
    }
    bf16x8 bhi, blo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)wv[i];
      bhi[i] = h;
      blo[i] = (__bf16)(wv[i] - (float)h);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      u32x4 av = {0u, 0u, 0u, 0u};
      if (t_ok[mt]) av = ld16(xrow[mt] + k0);
      const bf16x8 a = __builtin_bit_cast(bf16x8, av);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo, acc[mt], 0, 0, 0);
    }
  }
  // D layout: lane holds column n (expert) of rows 4G..4G+3 (tokens).
  if (!e_ok) return;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * mt + 4 * G + i;
      if (t < T) logits[(size_t)t * E + e0 + n] = acc[mt][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wavefront per token.  Lane l holds experts l, l+64, ...; each
// of the k rounds takes the lane-local best untaken (key, id) and reduces it
// across the wave with the total order (larger key first, then lower id).
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int T, int E,
                                              int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  constexpr int kPer = kMaxExperts / 64;
  float key[kPer], sc[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float s = sigmoidf_(logits[(size_t)t * E + e]);
      float kv = s + bias[e];
      if (kv != kv) kv = -INFINITY;  // a NaN score ranks last but stays selectable
      key[i] = kv;
      sc[i] = s;
    } else {
      key[i] = -INFINITY;
      sc[i] = 0.f;
      taken |= 1u << i;
    }
  }
  float my_s = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1u) && (key[i] > best || (key[i] == best && e < bi))) {
        best = key[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ob = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    float s_sel = 0.f;
    if ((bi & 63) == lane) {
      const int i = bi >> 6;
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (q == i) {
          taken |= 1u << q;
          s_sel = sc[q];
        }
    }
    s_sel = __shfl(s_sel, bi & 63, 64);
    if (lane == j) {
      my_s = s_sel;
      my_id = bi;
    }
  }
  float tot = 0.f;
  for (int j = 0; j < k; ++j) tot += __shfl(my_s, j, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = my_s / tot;
  }
}

hipError_t launch_router_gemv(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_router_gemv, dim3((s.E + 3) / 4), dim3(256), 0, st, x, w_router, logits, s.T, s.d, s.E);
  return hipGetLastError();
}

hipError_t launch_router_mfma(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_router_mfma, dim3((s.T + 63) / 64, (s.E + 63) / 64), dim3(256), 0, st, x, w_router, logits,
                     s.T, s.d, s.E);
  return hipGetLastError();
}

hipError_t launch_topk(const Shape& s, const float* logits, const float* bias, int32_t* topk_ids, float* topk_w,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_topk, dim3((s.T + 3) / 4), dim3(256), 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  return hipGetLastError();
}

}  // namespace moe
