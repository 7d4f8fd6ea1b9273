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
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.x;
  const float* wr = W + (size_t)e * d;
  float4 wv[NM];
  float okf[NM];
  int col[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int c = 4 * tid + 1024 * m;
    okf[m] = c < d ? 1.f : 0.f;
    col[m] = c < d ? c : d - 4;  // clamped: every load in bounds, masked below
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
        a = fmaf(okf[m], p, a);
      }
      acc[i] = wave_sum_hi(a);
    }
    if (lane == 63) {
#pragma unroll
      for (int i = 0; i < TB; ++i) red[wave][i] = acc[i];
    }
    __syncthreads();
    if (tid < TB && t0 + tid < T)
      logits[(size_t)(t0 + tid) * E + e] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    __syncthreads();
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

// ---------------------------------------------------------------------------
// Larger T: bf16 MFMA.  x is bf16 already; each fp32 router weight is split
// into hi = bf16(w) and lo = bf16(w - hi) so that two bf16 MFMAs reproduce
// the fp32 product to about 2^-17 relative.  A workgroup computes one 16 x 16
// tile (16 tokens x 16 experts); its four wavefronts take interleaved quarters
// of K (steps of 32) and their partial tiles are summed in LDS in a fixed
// order.  With 16 x 16 tiles the grid has T/16 * E/16 workgroups, enough
// wavefronts per SIMD to hide the load latency without software pipelining.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRouterUnroll = 8;  // K steps whose loads are issued together

__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ W,
                                                     float* __restrict__ logits, int T, int d, int E) {
  __shared__ floatx4 part[4][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  // Workgroups go round-robin over the 8 XCDs (own L2 each).  When the expert blocks divide evenly,
  // XCD x takes a fixed eighth of them for every token block, so each L2 holds only its eighth of
  // the router weights while the token blocks stream past.
  const int neb = (E + 15) / 16;
  int eb, tb;
  if (neb % 8 == 0) {
    const int per = neb / 8, item = blockIdx.x >> 3;
    eb = (blockIdx.x & 7) * per + item % per;
    tb = item / per;
  } else {
    eb = blockIdx.x % neb;
    tb = blockIdx.x / neb;
  }
  const int t0 = tb * 16, e0 = eb * 16;
  const int t = min(t0 + n, T - 1), e = min(e0 + n, E - 1);  // clamped rows: computed, never stored
  const uint16_t* xrow = x + (size_t)t * d + 8 * G;
  const float* wrow = W + (size_t)e * d + 8 * G;
  const int nsteps = d / 32;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](const u32x4& a, const float4& w0, const float4& w1) __attribute__((always_inline)) {
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    bf16x8 bhi, blo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)wv[i];
      bhi[i] = h;
      blo[i] = (__bf16)(wv[i] - (float)h);
    }
    const bf16x8 a8 = __builtin_bit_cast(bf16x8, a);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, bhi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, blo, acc, 0, 0, 0);
  };
  // wave w takes steps w, w+4, w+8, ...: whole batches of kRouterUnroll steps with all loads issued
  // first, then the remaining steps one at a time
  int s0 = wave;
  for (; s0 + 4 * (kRouterUnroll - 1) < nsteps; s0 += 4 * kRouterUnroll) {
    u32x4 av[kRouterUnroll];
    float4 w0[kRouterUnroll], w1[kRouterUnroll];
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) {
      av[u] = ld16(xrow + 32 * (s0 + 4 * u));
      w0[u] = *reinterpret_cast<const float4*>(wrow + 32 * (s0 + 4 * u));
      w1[u] = *reinterpret_cast<const float4*>(wrow + 32 * (s0 + 4 * u) + 4);
    }
#pragma unroll
    for (int u = 0; u < kRouterUnroll; ++u) step(av[u], w0[u], w1[u]);
  }
  for (; s0 < nsteps; s0 += 4)
    step(ld16(xrow + 32 * s0), *reinterpret_cast<const float4*>(wrow + 32 * s0),
         *reinterpret_cast<const float4*>(wrow + 32 * s0 + 4));
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  const floatx4 r = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  // D layout: lane holds column n (expert e0+n) of rows 4G..4G+3 (tokens)
  if (e0 + n >= E) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = t0 + 4 * G + i;
    if (tt < T) logits[(size_t)tt * E + e0 + n] = r[i];
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wavefront per token.  Lane l holds experts l, l+64, ... as
// order-preserving unsigned keys of s + b (empty and taken slots hold 0,
// below every real key).  Each of the k rounds finds the largest key (per
// lane, then four DPP max steps inside each 16-lane row, then the four row
// maxima in scalar registers) and then the lowest expert id that holds it,
// from one ballot per key register: ties go to the lower id.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  if (f != f) return 1u;  // NaN ranks below every number but above empty slots
  if (f == 0.f) f = 0.f;  // -0 and +0 are the same key (then the lower id wins)
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)dpp_i<CTRL>((int)v);
  return o > v ? o : v;
}

// Selection for one token by one wavefront: writes ids[0..k) and w[0..k).
template <int NPER>
__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, const float* __restrict__ bias,
                                          int32_t* __restrict__ ids, float* __restrict__ w, int E, int k, int lane) {
  uint32_t key[NPER];
  float sc[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float s = sigmoidf_(lrow[e]);
      key[i] = ordered_bits(s + bias[e]);
      sc[i] = s;
    } else {
      key[i] = 0u;
      sc[i] = 0.f;
    }
  }
  float my_s = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) m = key[i] > m ? key[i] : m;
    m = dpp_max_u32<kDppXor1>(m);
    m = dpp_max_u32<kDppXor2>(m);
    m = dpp_max_u32<kDppHalfMirror>(m);
    m = dpp_max_u32<kDppMirror>(m);
    uint32_t M = (uint32_t)__builtin_amdgcn_readlane((int)m, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)m, 16 * r);
      M = o > M ? o : M;
    }
    // lowest expert id holding M: the first key register with a hit, then its lowest lane
    int win = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(key[i] == M);
      if (!found && hit != 0) {
        win = 64 * i + (int)__builtin_ctzll(hit);
        found = true;
      }
    }
    float s_sel = sc[0];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      if ((win >> 6) == i) s_sel = sc[i];
      if (lane + 64 * i == win) key[i] = 0u;  // taken
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
    ids[lane] = my_id;
    w[lane] = my_s / tot;
  }
}

template <int NPER>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int T, int E,
                                              int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave<NPER>(logits + (size_t)t * E, bias, ids + (size_t)t * k, w + (size_t)t * k, E, k, lane);
}

hipError_t launch_router_mfma(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st) {
  const dim3 grid(((s.T + 15) / 16) * ((s.E + 15) / 16)), block(256);
  hipLaunchKernelGGL(k_router_mfma, grid, block, 0, st, x, w_router, logits, s.T, s.d, s.E);
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
