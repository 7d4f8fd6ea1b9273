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
// the fp32 product to about 2^-17 relative.  A workgroup computes a tile of
// 32 tokens x 64 experts: K advances 64 at a time through a double-buffered
// LDS stage (32 x 64 bf16 activations, 64 x 64 fp32 weights, rows padded so
// that the 16 rows one MFMA operand reads fall in distinct banks).  Wavefront
// w takes tokens 16(w&1) .. +15 and experts 32(w>>1) .. +31 (two 16 x 16
// tiles, each with a hi and a lo MFMA per K step of 32).  K is split in
// kRtSplit contiguous parts (blockIdx.y), each writing its own partial logits
// [part][T][E]; the top-k sums the parts in order, so the result is fixed.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRtT = 32, kRtE = 64, kRtK = 64;
constexpr int kRtSplit = kRouterParts;  // K parts, each its own workgroup; partial logits summed by the top-k
constexpr int kRtXStride = kRtK * 2 + 16;  // bytes per activation row in LDS (144)
constexpr int kRtWStride = kRtK * 4 + 16;  // bytes per weight row in LDS (272)

__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ W,
                                                     float* __restrict__ logits, int T, int d, int E) {
  __shared__ __attribute__((aligned(16))) char xs[2][kRtT * kRtXStride];
  __shared__ __attribute__((aligned(16))) char ws[2][kRtE * kRtWStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, G = lane >> 4;
  // Workgroups go round-robin over the 8 XCDs (own L2 each).  When the expert blocks and the XCDs
  // divide evenly, each XCD keeps a fixed share of the expert blocks for every token block, so its L2
  // holds only its share of the router weights while the token blocks stream past.
  const int neb = (E + kRtE - 1) / kRtE;
  int eb, tb;
  if (neb <= 8 && 8 % neb == 0) {
    eb = blockIdx.x % neb;  // blockIdx % 8 is the XCD, so XCD x always gets expert block x % neb
    tb = blockIdx.x / neb;
  } else if (neb % 8 == 0) {
    const int per = neb / 8, item = blockIdx.x >> 3;
    eb = (blockIdx.x & 7) * per + item % per;
    tb = item / per;
  } else {
    eb = blockIdx.x % neb;
    tb = blockIdx.x / neb;
  }
  const int t0 = tb * kRtT, e0 = eb * kRtE;
  // staging: thread -> one 16-byte piece of the activation tile and four of the weight tile
  const int xr = tid >> 3, xc = tid & 7;                     // 32 rows x 8 pieces
  const uint16_t* xsrc = x + (size_t)min(t0 + xr, T - 1) * d + 8 * xc;
  const int wr0 = tid >> 4, wc = tid & 15;  // 64 rows x 16 pieces: rows wr0 + 16j
  const float* wsrc = W + (size_t)min(e0 + wr0, E - 1) * d + 4 * wc;
  const size_t wstep = (size_t)16 * d;  // 16 rows further down (clamped rows only at the end of E)
  const int wlast = E - 1 - e0 - wr0;   // rows beyond E re-read row E-1: j > wlast/16 is clamped
  // this workgroup's part of K: stages [st0, st1) of 64 columns
  const int nst_all = (d + kRtK - 1) / kRtK;
  const int st0 = (nst_all * (int)blockIdx.y) / kRtSplit, st1 = (nst_all * ((int)blockIdx.y + 1)) / kRtSplit;
  const bool half_tail = (d % kRtK) != 0 && st1 == nst_all;  // the last stage holds only one K step of 32
  logits += (size_t)blockIdx.y * T * E;
  const int wt = wave & 1, we = wave >> 1;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  u32x4 xv;
  float4 wv0, wv1, wv2, wv3;
#define MOE_RT_LOAD(st)                                                                             \
  {                                                                                                  \
    /* K columns past the end (half stage) re-read the stage's first half: loaded, never used */    \
    const int k0_ = (st) * kRtK;                                                                     \
    xv = ld16(xsrc + ((k0_ + 8 * xc < d) ? k0_ : k0_ - 32));                                         \
    const int kw_ = (k0_ + 4 * wc < d) ? k0_ : k0_ - 32;                                            \
    wv0 = *reinterpret_cast<const float4*>(wsrc + kw_);                                              \
    wv1 = *reinterpret_cast<const float4*>(wsrc + (16 <= wlast ? wstep : 0) + kw_);                   \
    wv2 = *reinterpret_cast<const float4*>(wsrc + (32 <= wlast ? 2 * wstep : 0) + kw_);               \
    wv3 = *reinterpret_cast<const float4*>(wsrc + (48 <= wlast ? 3 * wstep : 0) + kw_);               \
  }
#define MOE_RT_STORE(buf)                                                                           \
  {                                                                                                  \
    *reinterpret_cast<u32x4*>(xs[buf] + xr * kRtXStride + 16 * xc) = xv;                             \
    char* w_ = ws[buf] + wr0 * kRtWStride + 16 * wc;                                                 \
    *reinterpret_cast<float4*>(w_) = wv0;                                                            \
    *reinterpret_cast<float4*>(w_ + 16 * kRtWStride) = wv1;                                          \
    *reinterpret_cast<float4*>(w_ + 32 * kRtWStride) = wv2;                                          \
    *reinterpret_cast<float4*>(w_ + 48 * kRtWStride) = wv3;                                          \
  }
  if (st0 < st1) {
    MOE_RT_LOAD(st0);
    MOE_RT_STORE(0);
  }
  __syncthreads();
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    if (st + 1 < st1) MOE_RT_LOAD(st + 1);  // in flight while this stage is computed
    const int nk = (half_tail && st == st1 - 1) ? 1 : 2;  // uniform
    for (int kk = 0; kk < nk; ++kk) {
      const bf16x8 a8 = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(xs[buf] + (16 * wt + n) * kRtXStride + 64 * kk + 16 * G));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* wrow = ws[buf] + (32 * we + 16 * j + n) * kRtWStride + 128 * kk + 32 * G;
        const float4 w0 = *reinterpret_cast<const float4*>(wrow);
        const float4 w1 = *reinterpret_cast<const float4*>(wrow + 16);
        bf16x8 bhi, blo;
        bhi[0] = (__bf16)w0.x; bhi[1] = (__bf16)w0.y; bhi[2] = (__bf16)w0.z; bhi[3] = (__bf16)w0.w;
        bhi[4] = (__bf16)w1.x; bhi[5] = (__bf16)w1.y; bhi[6] = (__bf16)w1.z; bhi[7] = (__bf16)w1.w;
        blo[0] = (__bf16)(w0.x - (float)bhi[0]); blo[1] = (__bf16)(w0.y - (float)bhi[1]);
        blo[2] = (__bf16)(w0.z - (float)bhi[2]); blo[3] = (__bf16)(w0.w - (float)bhi[3]);
        blo[4] = (__bf16)(w1.x - (float)bhi[4]); blo[5] = (__bf16)(w1.y - (float)bhi[5]);
        blo[6] = (__bf16)(w1.z - (float)bhi[6]); blo[7] = (__bf16)(w1.w - (float)bhi[7]);
        floatx4& acc = j ? acc1 : acc0;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, blo, acc, 0, 0, 0);
      }
    }
    if (st + 1 < st1) {
      __syncthreads();  // every wavefront is done with buffer buf ^ 1 (read two stages ago)
      MOE_RT_STORE(buf ^ 1);
      __syncthreads();
    }
  }
#undef MOE_RT_LOAD
#undef MOE_RT_STORE
  const floatx4 accs[2] = {acc0, acc1};
  // D layout: lane holds column n (expert) of rows 4G..4G+3 (tokens) of each 16 x 16 tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + 32 * we + 16 * j + n;
    if (e >= E) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * wt + 4 * G + i;
      if (t < T) logits[(size_t)t * E + e] = accs[j][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wavefront per token.  Lane l holds experts l, l+64, ... as
// order-preserving unsigned keys of s + b (lanes past E hold 0, below every
// real key).  The k-th largest key tau is found bit by bit from the top: a
// candidate bit stays set when at least k keys are >= the candidate (one
// ballot and popcount per key register), so the search costs 32 short steps
// whatever k is.  The chosen experts are the keys above tau and, of the keys
// equal to tau, the lowest ids (ties go to the lower id).  They are compacted
// into LDS; each finds its slot by counting the chosen keys that rank before
// it (a larger key, or an equal key and a lower id), and the weights are
// normalised by the sum of the chosen scores taken in slot order.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  if (f != f) return 1u;  // NaN ranks below every number but above empty slots
  if (f == 0.f) f = 0.f;  // -0 and +0 are the same key (then the lower id wins)
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkLds {  // one wavefront's staging: the chosen entries in id order, then in slot order
  uint32_t key[kMaxTopK];
  int32_t id[kMaxTopK];
  float s[kMaxTopK];
  int32_t slot_id[kMaxTopK];
  float slot_s[kMaxTopK];
};

__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }

// Selection for one token by one wavefront: writes ids[0..k) and w[0..k).  The wavefront reads
// back only what its own lanes wrote to LDS: LDS operations of one wavefront are ordered.
template <int NPER, int NPARTS>
__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, size_t part_stride,
                                          const float* __restrict__ bias, int32_t* __restrict__ ids,
                                          float* __restrict__ w, int E, int k, int lane, TopkLds& sm) {
  // every load first, from clamped indices: one memory round trip
  float lg[NPARTS][NPER], bs[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    bs[i] = bias[e];
#pragma unroll
    for (int p = 0; p < NPARTS; ++p) lg[p][i] = lrow[p * part_stride + e];
  }
  uint32_t key[NPER];
  float sc[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    float l = lg[0][i];
#pragma unroll
    for (int p = 1; p < NPARTS; ++p) l += lg[p][i];  // partial logits, in order
    sc[i] = sigmoidf_(l);
    const uint32_t valid = lane + 64 * i < E ? 0xFFFFFFFFu : 0u;
    key[i] = ordered_bits(sc[i] + bs[i]) & valid;
  }
  // tau: the largest value with at least k keys >= it, i.e. the k-th largest key
  uint32_t tau = 0u;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) cnt += popc(__builtin_amdgcn_ballot_w64(key[i] >= cand));
    tau = cnt >= k ? cand : tau;
  }
  // chosen: every key above tau (fewer than k), then the lowest ids among the keys equal to tau
  uint64_t chosen[NPER];
  int need = k;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    chosen[i] = __builtin_amdgcn_ballot_w64(key[i] > tau);
    need -= popc(chosen[i]);
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    uint64_t eq = __builtin_amdgcn_ballot_w64(key[i] == tau);
    while (need > 0 && eq != 0) {
      const uint64_t low = eq & (~eq + 1u);
      chosen[i] |= low;
      eq ^= low;
      --need;
    }
  }
  // compact the k chosen entries into LDS in id order
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const uint64_t m = chosen[i];
    if ((m >> lane) & 1u) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      sm.key[pos] = key[i];
      sm.id[pos] = lane + 64 * i;
      sm.s[pos] = sc[i];
    }
    base += popc(m);
  }
  // lane r < k takes entry r and counts the entries that rank before it: its slot
  const int r = min(lane, k - 1);
  const uint32_t K = sm.key[r];
  const int I = sm.id[r];
  const float S = sm.s[r];
  int slot = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t Kj = (uint32_t)__builtin_amdgcn_readlane((int)K, j);
    const int Ij = __builtin_amdgcn_readlane(I, j);
    slot += (Kj > K || (Kj == K && Ij < I)) ? 1 : 0;
  }
  if (lane < k) {
    sm.slot_id[slot] = I;
    sm.slot_s[slot] = S;
  }
  const int q = min(lane, k - 1);
  const int my_id = sm.slot_id[q];
  const float my_s = sm.slot_s[q];
  float tot = 0.f;
  for (int j = 0; j < k; ++j)  // slot order, same value in every lane
    tot += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_s), j));
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = my_s / tot;
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

hipError_t launch_router_mfma(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st) {
  const dim3 grid(((s.T + kRtT - 1) / kRtT) * ((s.E + kRtE - 1) / kRtE), kRtSplit), block(256);
  hipLaunchKernelGGL(k_router_mfma, grid, block, 0, st, x, w_router, logits, s.T, s.d, s.E);
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
