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
// Small T: one workgroup of 256 threads per expert.  Thread i holds 4
// consecutive router weights at 4i + 1024m (m < NM), loaded once for all
// tokens; tokens are processed TB at a time and each dot product is reduced
// across the wavefront (DPP) and then across the 4 wavefronts in LDS.
template <int NM, int TB>
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, const float* __restrict__ W,
                                                     float* __restrict__ logits, int T, int d, int E) {
  __shared__ float red[4][TB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const float* wr = W + (size_t)e * d;
  float4 wv[NM];
  bool ok[NM];
  int col[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int c = 4 * tid + 1024 * m;
    ok[m] = c < d;
    col[m] = ok[m] ? c : d - 4;  // clamped: every load in bounds, masked below
    wv[m] = *reinterpret_cast<const float4*>(wr + col[m]);
  }
  for (int t0 = 0; t0 < T; t0 += TB) {
    uint2 xv[TB][NM];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int t = min(t0 + i, T - 1);
#pragma unroll
      for (int m = 0; m < NM; ++m) xv[i][m] = *reinterpret_cast<const uint2*>(x + (size_t)t * d + col[m]);
    }
    float acc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      float a = 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        float p = wv[m].x * bf16_bits_to_float(xv[i][m].x & 0xFFFFu);
        p = fmaf(wv[m].y, bf16_bits_to_float(xv[i][m].x >> 16), p);
        p = fmaf(wv[m].z, bf16_bits_to_float(xv[i][m].y & 0xFFFFu), p);
        p = fmaf(wv[m].w, bf16_bits_to_float(xv[i][m].y >> 16), p);
        a += ok[m] ? p : 0.f;
      }
      acc[i] = wave_sum(a);
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < TB; ++i) red[wave][i] = acc[i];
    }
    __syncthreads();
    if (tid < TB && t0 + tid < T)
      logits[(size_t)(t0 + tid) * E + e] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    __syncthreads();
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
// Top-k: one wavefront per token.  Lane l holds experts l, l+64, ... as
// 64-bit sort keys (order-preserving bits of s + b, then the complement of
// the expert id), so "larger key, then lower id" is a plain unsigned max.
// Each of the k rounds takes the lane's best untaken key and reduces it over
// the wavefront: four DPP steps inside each 16-lane row, then the four row
// winners are compared in scalar registers.  Every lane ends with the winner.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  if (f != f) return 1u;  // NaN ranks below every number but above empty slots
  if (f == 0.f) f = 0.f;  // -0 and +0 are the same key (then the lower id wins)
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step_dpp(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = (uint32_t)dpp_i<CTRL>((int)hi), ol = (uint32_t)dpp_i<CTRL>((int)lo);
  const bool take = (oh > hi) || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}

template <int NPER>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int T, int E,
                                              int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint32_t key[NPER];
  float sc[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float s = sigmoidf_(logits[(size_t)t * E + e]);
      key[i] = ordered_bits(s + bias[e]);
      sc[i] = s;
    } else {
      key[i] = 0u;  // empty slot: never wins (every real key is >= 1)
      sc[i] = 0.f;
    }
  }
  float my_s = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t hi = 0u, lo = 0u;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint32_t l2 = ~(uint32_t)(lane + 64 * i);
      if (key[i] > hi || (key[i] == hi && l2 > lo)) {
        hi = key[i];
        lo = l2;
      }
    }
    argmax_step_dpp<kDppXor1>(hi, lo);
    argmax_step_dpp<kDppXor2>(hi, lo);
    argmax_step_dpp<kDppHalfMirror>(hi, lo);
    argmax_step_dpp<kDppMirror>(hi, lo);
    // every lane of a 16-lane row holds the row's best; combine the four rows in scalar registers
    {
      uint32_t bh = (uint32_t)__builtin_amdgcn_readlane((int)hi, 0), bl = (uint32_t)__builtin_amdgcn_readlane((int)lo, 0);
#pragma unroll
      for (int r = 1; r < 4; ++r) {
        const uint32_t oh = (uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r);
        const uint32_t ol = (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
        if (oh > bh || (oh == bh && ol > bl)) {
          bh = oh;
          bl = ol;
        }
      }
      hi = bh;
      lo = bl;
    }
    const int win = (int)~lo;
    float s_sel = 0.f;
    if ((win & 63) == lane) {
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i == (win >> 6)) {
          key[i] = 0u;  // taken
          s_sel = sc[i];
        }
    }
    s_sel = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_sel), win & 63));
    if (lane == j) {
      my_s = s_sel;
      my_id = win;
    }
  }
  float tot = 0.f;
  for (int j = 0; j < k; ++j)  // slot order, same value in every lane
    tot += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_s), j));
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = my_s / tot;
  }
}

template <int NM>
static void router_gemv_tb(const Shape& s, const uint16_t* x, const float* w_router, float* logits, hipStream_t st) {
  const dim3 grid(s.E), block(256);
  if (s.T == 1) hipLaunchKernelGGL((k_router_gemv<NM, 1>), grid, block, 0, st, x, w_router, logits, s.T, s.d, s.E);
  else if (s.T <= 4) hipLaunchKernelGGL((k_router_gemv<NM, 4>), grid, block, 0, st, x, w_router, logits, s.T, s.d, s.E);
  else hipLaunchKernelGGL((k_router_gemv<NM, 8>), grid, block, 0, st, x, w_router, logits, s.T, s.d, s.E);
}

hipError_t launch_router_gemv(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st) {
  const int nm = (s.d + 1023) / 1024;
  if (nm <= 1) router_gemv_tb<1>(s, x, w_router, logits, st);
  else if (nm <= 2) router_gemv_tb<2>(s, x, w_router, logits, st);
  else if (nm <= 4) router_gemv_tb<4>(s, x, w_router, logits, st);
  else router_gemv_tb<8>(s, x, w_router, logits, st);
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
  const dim3 grid((s.T + 3) / 4), block(256);
  const int nper = (s.E + 63) / 64;
  if (nper <= 1) hipLaunchKernelGGL(k_topk<1>, grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else if (nper <= 2) hipLaunchKernelGGL(k_topk<2>, grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else if (nper <= 4) hipLaunchKernelGGL(k_topk<4>, grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else if (nper <= 8) hipLaunchKernelGGL(k_topk<8>, grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else hipLaunchKernelGGL(k_topk<16>, grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  return hipGetLastError();
}

}  // namespace moe
