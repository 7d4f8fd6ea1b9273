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
#include "topk.hpp"


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
// the fp32 product to about 2^-17 relative.  A workgroup computes 16*TA
// tokens x 256 experts over one of kRouterParts contiguous parts of K with 8
// wavefronts: wavefront w takes the 64-expert block w % 4 and half w / 4 of
// every chunk's K steps, and the two halves are added in LDS at the end
// (lower half first).  Every workgroup streams its part of the router
// weights for all of its experts, so where 128-token tiles still give 256
// workgroups the token tile is 128: over all 256 experts with 4 wavefronts
// and whole K steps (T >= 4096 at E = 256), or over 128 experts with 4
// wavefronts and two K halves (T = 2048), reading the weights half as often
// as 64-token tiles.  When that gives few workgroups (small T) a workgroup
// takes one 64-expert block and splits every chunk's K steps over 8
// wavefronts instead, whose sums are added in LDS in wavefront order, with
// the token tile shrunk to 32 or 16 rows when 64-row tiles give fewer than
// 128 workgroups.  The token tile is brought into LDS first, 1 KiB of
// every token row per chunk of 16 K steps, with buffer loads straight into
// LDS (rows past T read as zeros), so the activation operand never waits on
// HBM inside the K loop; each wavefront streams its weights from memory into
// MFMA registers -- lane (n, G) takes 8 consecutive K values of weight row
// n -- with the next two K steps of 32 in flight, and splits them there.
// Workgroups go round-robin over the 8 XCDs and workgroup b takes K part
// b % kRouterParts, so each XCD keeps the same part of the router weights in
// its L2 while the token tiles stream past.  The weights are the MFMA A
// operand: a lane ends with 4 consecutive experts of one token, stored as
// one 16-byte piece.  Every part writes its own partial logits [part][T][E];
// the top-k sums the parts in order, so the result is fixed.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRtExp = 64, kRtK = 32;  // experts per wavefront, K per step
constexpr int kRtChunk = 16;           // K steps per LDS chunk: 1 KiB of each token row
constexpr int kRtXRow = kRtChunk * kRtK * 2 + 16;  // LDS bytes per token row (padded against bank conflicts)
static_assert(kRouterParts == 8, "one K part of the router weights per XCD");

typedef float float2v __attribute__((ext_vector_type(2)));
// hi = bf16(w) (round to nearest even), lo = bf16(w - hi); w - hi is exact in fp32, and the bf16 pair
// hi is turned back into fp32 by placing each half in the top 16 bits
__device__ __forceinline__ void split_pair(float w0, float w1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{w0, w1}, bf16x2));
  const float r0 = w0 - __builtin_bit_cast(float, hi << 16);
  const float r1 = w1 - __builtin_bit_cast(float, hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{r0, r1}, bf16x2));
}
__device__ __forceinline__ void split_hi_lo(const float4 a, const float4 b, bf16x8& hi, bf16x8& lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split_pair(a.x, a.y, h0, l0);
  split_pair(a.z, a.w, h1, l1);
  split_pair(b.x, b.y, h2, l2);
  split_pair(b.z, b.w, h3, l3);
  hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
  lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

// TA 16-token blocks, EB 64-expert blocks per workgroup, every chunk's K steps split over KS wavefronts
// x16 (may be nullptr): the workgroups of one token tile and K part also write that part of the fp16
// pair-ordered copy of x for the grouped gate+up, each a contiguous share of the tile's rows, from the
// bf16 tile they staged in LDS (every element of x is written once).
template <int TA, int EB, int KS>
__global__ __launch_bounds__(64 * EB * KS) void k_router_mfma(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ W,
                                                              float* __restrict__ logits, int T, int d, int E,
                                                              _Float16* __restrict__ x16) {
  constexpr int kRtBlocks = EB, kRtWaves = EB * KS;
  static_assert(16 * TA % kRtWaves == 0, "token rows split evenly over the wavefronts");
  static_assert(16 * TA * kRtXRow >= kRtBlocks * 4 * TA * 64 * 16, "the K-part sums fit in the token tile");
  __shared__ __attribute__((aligned(16))) char xs[16 * TA * kRtXRow];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int blk = wave % kRtBlocks, kh = wave / kRtBlocks;
  const int part = blockIdx.x % kRouterParts, item = blockIdx.x / kRouterParts;
  const int neb = (E + kRtBlocks * kRtExp - 1) / (kRtBlocks * kRtExp);
  const int t0 = (item / neb) * 16 * TA, e0 = ((item % neb) * kRtBlocks + blk) * kRtExp;
  const bool active = e0 < E;  // uniform over the wavefront; idle ones still stage tokens and meet the barriers
  logits += (size_t)part * T * E;
  const int nst = d / kRtK;
  const int st0 = (nst * part) / kRouterParts, ns = (nst * (part + 1)) / kRouterParts - st0;
  const int rows = min(16 * TA, T - t0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)t0 * d, (uint32_t)((size_t)rows * d * 2));
  // weight rows past E re-read row E-1 and are never stored
  const float* wr[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) wr[b] = W + (size_t)min(e0 + 16 * b + n, E - 1) * d + (size_t)st0 * kRtK + 8 * G;
  floatx4 acc[4][TA];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int a = 0; a < TA; ++a) acc[b][a] = floatx4{0.f, 0.f, 0.f, 0.f};
  float4 wl[2][4][2];
#define MOE_RT_LOAD(S, s)                                                    \
  _Pragma("unroll") for (int b = 0; b < 4; ++b) {                            \
    wl[S][b][0] = *reinterpret_cast<const float4*>(wr[b] + (s) * kRtK);      \
    wl[S][b][1] = *reinterpret_cast<const float4*>(wr[b] + (s) * kRtK + 4);  \
  }
// all 16 hi products before the 16 lo ones: consecutive MFMAs on one accumulator stay 16 apart
#define MOE_RT_MMA(S, s)                                                     \
  {                                                                          \
    bf16x8 xb[TA], hi[4], lo[4];                                             \
    _Pragma("unroll") for (int a = 0; a < TA; ++a) xb[a] = __builtin_bit_cast( \
        bf16x8, *reinterpret_cast<const u32x4*>(xs + (16 * a + n) * kRtXRow + ((s) - c0) * kRtK * 2 + 16 * G)); \
    _Pragma("unroll") for (int b = 0; b < 4; ++b) split_hi_lo(wl[S][b][0], wl[S][b][1], hi[b], lo[b]); \
    _Pragma("unroll") for (int b = 0; b < 4; ++b)                            \
      _Pragma("unroll") for (int a = 0; a < TA; ++a)                         \
        acc[b][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[b], xb[a], acc[b][a], 0, 0, 0); \
    _Pragma("unroll") for (int b = 0; b < 4; ++b)                            \
      _Pragma("unroll") for (int a = 0; a < TA; ++a)                         \
        acc[b][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[b], xb[a], acc[b][a], 0, 0, 0); \
  }
  for (int c0 = 0; c0 < ns; c0 += kRtChunk) {
    const int cn = min(kRtChunk, ns - c0);
    const int k0 = c0 + (cn * kh) / KS, kn = c0 + (cn * (kh + 1)) / KS - k0;  // this wavefront's K steps
    if (c0 > 0) {  // every wavefront is done reading the previous chunk
      vm_lgkm_wait<0>();
      tile_barrier();
    }
    // the chunk: wavefront w loads rows w, w + 8, ... with one 1 KiB instruction per row; lanes past
    // the chunk read on along the row (zeros past the tile) into padding that is never read
#pragma unroll
    for (int i = 0; i < 16 * TA / kRtWaves; ++i) {
      const int r = wave + kRtWaves * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(xs + r * kRtXRow), 16,
                                               r * d * 2 + (st0 + c0) * kRtK * 2 + 16 * lane, 0, 0, 0);
    }
    // the first two weight steps are issued behind the chunk, so waiting for all but them waits for
    // exactly the chunk
    if (active && kn > 1) {
      MOE_RT_LOAD(0, k0);
      MOE_RT_LOAD(1, k0 + 1);
      vm_wait<16>();
    } else if (active && kn == 1) {
      MOE_RT_LOAD(0, k0);
      vm_wait<8>();
    } else {
      vm_wait<0>();
    }
    tile_barrier();  // every row of the chunk is in LDS
    if (active) {
      for (int s = k0; s < k0 + kn; s += 2) {
        MOE_RT_MMA(0, s);
        if (s + 2 < k0 + kn) MOE_RT_LOAD(0, s + 2);
        if (s + 1 < k0 + kn) {
          MOE_RT_MMA(1, s + 1);
          if (s + 3 < k0 + kn) MOE_RT_LOAD(1, s + 3);
        }
      }
    }
    if (x16 != nullptr) {  // uniform; the chunk stays in LDS until the next chunk's barrier
      const int eb = item % neb;
      const int r0 = (16 * TA * eb) / neb, r1 = min((16 * TA * (eb + 1)) / neb, rows);
      const int per_row = cn * (kRtK / 8);  // 16-byte groups of 8 values per row of the chunk
      for (int i = threadIdx.x; i < (r1 - r0) * per_row; i += 64 * kRtWaves) {
        const int r = r0 + i / per_row, g = i % per_row;
        const u32x4 v = *reinterpret_cast<const u32x4*>(xs + r * kRtXRow + 16 * g);
        *reinterpret_cast<u32x4*>(x16 + (size_t)(t0 + r) * d + (size_t)(st0 + c0) * kRtK + 8 * g) =
            x8_bf16_to_f16_pairs(v);
      }
    }
  }
#undef MOE_RT_LOAD
#undef MOE_RT_MMA
  // the other K parts hand their sums to part 0 through LDS (the token tile is no longer read), one
  // after another in part order
  floatx4* red = reinterpret_cast<floatx4*>(xs) + (size_t)blk * 4 * TA * 64 + lane;
  for (int r = 1; r < KS; ++r) {
    vm_lgkm_wait<0>();
    tile_barrier();
    if (kh == r && active) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int a = 0; a < TA; ++a) red[(b * TA + a) * 64] = acc[b][a];
    }
    vm_lgkm_wait<0>();
    tile_barrier();
    if (kh == 0 && active && r + 1 < KS) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int a = 0; a < TA; ++a) acc[b][a] += red[(b * TA + a) * 64];
    }
  }
  if (kh != 0 || !active) return;
  // D layout (weights as A): lane holds token n of each 16-token block, experts 4G .. 4G+3
  const bool vec = (E & 3) == 0;  // rows of the logits 16-byte aligned
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int e = e0 + 16 * b + 4 * G;
#pragma unroll
    for (int a = 0; a < TA; ++a) {
      const floatx4 v = KS > 1 ? acc[b][a] + red[(b * TA + a) * 64] : acc[b][a];
      const int t = t0 + 16 * a + n;
      if (t >= T || e >= E) continue;
      float* dst = logits + (size_t)t * E + e;
      if (vec && e + 3 < E) {
        *reinterpret_cast<floatx4*>(dst) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e + i < E) dst[i] = v[i];
      }
    }
  }
}

template <int NPER, int NPARTS>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int T, int E,
                                              int k) {
  __shared__ TopkLds sm[4];
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  topk_wave<NPER, NPARTS>(logits + (size_t)t * E, (size_t)T * E, bias, ids + (size_t)t * k, w + (size_t)t * k, E,
                          k, lane, sm[wv]);
}

template <int TA, int EB, int KS>
static void router_mfma_cfg(const Shape& s, const uint16_t* x, const float* w_router, float* logits, hipStream_t st,
                            _Float16* x16) {
  const int ntt = (s.T + 16 * TA - 1) / (16 * TA), neb = (s.E + EB * kRtExp - 1) / (EB * kRtExp);
  const dim3 grid(ntt * neb * kRouterParts), block(64 * EB * KS);
  hipLaunchKernelGGL((k_router_mfma<TA, EB, KS>), grid, block, 0, st, x, w_router, logits, s.T, s.d, s.E, x16);
}

hipError_t launch_router_mfma(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st, _Float16* x16) {
  const int ntt4 = (s.T + 63) / 64, ntt8 = (s.T + 127) / 128, neb4 = (s.E + 4 * kRtExp - 1) / (4 * kRtExp);
  if (ntt8 * neb4 * kRouterParts >= 256)
    router_mfma_cfg<8, 4, 1>(s, x, w_router, logits, st, x16);  // 128 tokens x 256 experts per workgroup
  else if (ntt8 * ((s.E + 2 * kRtExp - 1) / (2 * kRtExp)) * kRouterParts >= 256)
    router_mfma_cfg<8, 2, 2>(s, x, w_router, logits, st, x16);  // 128 tokens x 128 experts x 2 K halves
  else if (ntt4 * neb4 * kRouterParts >= 128)
    router_mfma_cfg<4, 4, 2>(s, x, w_router, logits, st, x16);  // 64 tokens x 256 experts x 2 K halves
  else {
    // small T: 64 experts x 8 K parts per workgroup, and the largest token tile (64, 32 or 16) that still
    // gives 128 workgroups (T = 64: 11.7 -> 7.7 us with 16 tokens)
    const int neb1 = (s.E + kRtExp - 1) / kRtExp;
    if (ntt4 * neb1 * kRouterParts >= 128)
      router_mfma_cfg<4, 1, 8>(s, x, w_router, logits, st, x16);
    else if (((s.T + 31) / 32) * neb1 * kRouterParts >= 128)
      router_mfma_cfg<2, 1, 8>(s, x, w_router, logits, st, x16);
    else
      router_mfma_cfg<1, 1, 8>(s, x, w_router, logits, st, x16);
  }
  return hipGetLastError();
}

template <int NPARTS>
static hipError_t launch_topk_parts(const Shape& s, const float* logits, const float* bias, int32_t* topk_ids,
                                    float* topk_w, hipStream_t st) {
  const dim3 grid((s.T + 3) / 4), block(256);
  const int nper = (s.E + 63) / 64;
  if (nper <= 1)
    hipLaunchKernelGGL((k_topk<1, NPARTS>), grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else if (nper <= 2)
    hipLaunchKernelGGL((k_topk<2, NPARTS>), grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else if (nper <= 4)
    hipLaunchKernelGGL((k_topk<4, NPARTS>), grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else if (nper <= 8)
    hipLaunchKernelGGL((k_topk<8, NPARTS>), grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  else
    hipLaunchKernelGGL((k_topk<16, NPARTS>), grid, block, 0, st, logits, bias, topk_ids, topk_w, s.T, s.E, s.k);
  return hipGetLastError();
}

hipError_t launch_topk(const Shape& s, const float* logits, int nparts, const float* bias, int32_t* topk_ids,
                       float* topk_w, hipStream_t st) {
  if (nparts == 1) return launch_topk_parts<1>(s, logits, bias, topk_ids, topk_w, st);
  if (nparts == kRouterParts) return launch_topk_parts<kRouterParts>(s, logits, bias, topk_ids, topk_w, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
