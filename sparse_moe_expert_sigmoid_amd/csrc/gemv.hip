// Small-T path: gathered Q4 GEMVs.
//
// Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine": decode runs
// the chosen experts as gathered Q4 GEMVs (moe_gather_q4 and the SwiGLU-fused
// moe_gather_q4_swiglu), with gate and up fused and the shared expert taken
// through the same gather.  Page thewafflehaus/FFAI pull request 72,
// "ffai_add3": routed terms are summed first, then the shared expert.
//
// Every (token, slot) pair is a job that streams its expert's rows straight
// from HBM with 16-byte loads; each job's activation slice stays in
// registers for all the rows a wavefront handles.  No routing build is
// needed: jobs read topk_ids directly.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Gate+up with SwiGLU.  grid = (ceil(max(I, Is)/16), P + T); a workgroup of 4
// wavefronts covers 16 h-rows of one job, a wavefront 4 h-rows (4 gate rows
// and the 4 matching up rows).  Lane l owns Q4 blocks 2l and 2l+1 of every
// 128-block chunk of the row (32 contiguous code bytes, 4 scale bytes).
// h is written in fp32: h_r[p][I] for pair p, h_s[t][Is] for the shared expert.
template <int NCH>
__global__ __launch_bounds__(256) void k_gemv_gateup(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                                                     Q4 w13, Q4 s13, float* __restrict__ h_r, float* __restrict__ h_s,
                                                     int T, int d, int k, int I, int Is, uint32_t mask, uint32_t magic) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int job = blockIdx.y;
  const int P = T * k;
  int t, Iw;
  const uint8_t* qs;
  const uint16_t* sc;
  float* out;
  if (job < P) {
    t = job / k;
    const int e = ids[job];
    Iw = I;
    qs = w13.qs + (size_t)e * (2 * (size_t)I) * (d / 2);
    sc = w13.sc + (size_t)e * (2 * (size_t)I) * (d / 32);
    out = h_r + (size_t)job * I;
  } else {
    t = job - P;
    Iw = Is;
    qs = s13.qs;
    sc = s13.sc;
    out = h_s + (size_t)t * Is;
  }
  const int i0 = blockIdx.x * 16 + wave * 4;
  if (i0 >= Iw) return;  // Iw % 32 == 0: a wavefront's 4 rows are all valid or all past the end
  const int nb = d / 32;
  const size_t qstride = d / 2, sstride = d / 32;

  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    // Block indices past the row end are clamped to a valid block (so every load is issued
    // unconditionally and stays in bounds) and their contribution is masked to zero.
    int bi[2];
    bool ok[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 128 * c + 2 * lane + bb;
      ok[bb] = b < nb;
      bi[bb] = ok[bb] ? b : nb - 1;
    }
    // 1) activation slices of this lane's blocks (L2-resident), issued first
    u32x4 u[2][4];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) u[bb][dw] = ld16(x + (size_t)t * d + 32 * bi[bb] + 8 * dw);
    // 2) weight codes and scales of 8 rows: all loads in flight before any arithmetic
    u32x4 q[8][2];
    uint32_t sv[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = (r < 4) ? (i0 + r) : (Iw + i0 + r - 4);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        q[r][bb] = ld16(qs + row * qstride + 16 * (size_t)bi[bb]);
        sv[r][bb] = sc[row * sstride + bi[bb]];
      }
    }
    // 3) activation pairs and block sums
    uint32_t xp[2][4][4];
    float xs[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      float sum = 0.f;
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        x_bf16_pairs(u[bb][dw], xp[bb][dw]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          sum += bf16_bits_to_float(u[bb][dw][m] & 0xFFFFu) + bf16_bits_to_float(u[bb][dw][m] >> 16);
      }
      xs[bb] = ok[bb] ? sum : 0.f;
    }
    // 4) dot products
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        float dot = 0.f;
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          uint32_t cp[4];
          codes_bf16_pairs(q[r][bb][dw], mask, magic, cp);
#pragma unroll
          for (int m = 0; m < 4; ++m) dot = dot2_bf16(cp[m], xp[bb][dw][m], dot);
        }
        const float dsc = ok[bb] ? fp16_bits_to_float(sv[r][bb]) : 0.f;
        acc[r] = fmaf(dsc, fmaf(-136.f, xs[bb], dot), acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = wave_sum(acc[r]);
  if (lane < 4) {
    float g = acc[0], u = acc[4];
#pragma unroll
    for (int r = 1; r < 4; ++r)
      if (lane == r) {
        g = acc[r];
        u = acc[4 + r];
      }
    out[i0 + lane] = siluf_(g) * u;
  }
}

// ---------------------------------------------------------------------------
// Down projection fused with the combine.  grid = (ceil(d/16), T); the
// workgroup has min(k+1, 16) wavefronts that take the slots j = wave,
// wave + nw, ... (slot k is the shared expert).  A wavefront computes the
// 16 output rows of its slot, two rows at a time (one per 32-lane half);
// lane l%32 owns block l%32 (+32c) of the row and keeps the matching 32 h
// values in registers.  Partial dot products meet in LDS and one thread per
// row sums them in slot order: y = sum_j w_j * dot_j, then + shared.
template <int NCH>
__global__ __launch_bounds__(1024) void k_gemv_down_combine(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ topk_w, Q4 w2, Q4 s2,
                                                            const float* __restrict__ h_r,
                                                            const float* __restrict__ h_s, float* __restrict__ y,
                                                            int T, int d, int k, int I, int Is) {
  __shared__ float part[kMaxTopK + 1][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * 16;
  const int half = lane >> 5, bl = lane & 31;
  for (int slot = wave; slot <= k; slot += nw) {
    const uint8_t* qs;
    const uint16_t* sc;
    const float* h;
    int Kw;
    if (slot < k) {
      const int e = ids[(size_t)t * k + slot];
      Kw = I;
      qs = w2.qs + (size_t)e * d * (I / 2);
      sc = w2.sc + (size_t)e * d * (I / 32);
      h = h_r + ((size_t)t * k + slot) * I;
    } else {
      Kw = Is;
      qs = s2.qs;
      sc = s2.sc;
      h = h_s + (size_t)t * Is;
    }
    const int nbk = Kw / 32;
    const size_t qstride = Kw / 2, sstride = Kw / 32;
    // clamped block and row indices: every load is issued unconditionally and stays in bounds
    int bi[NCH];
    bool ok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int b = bl + 32 * c;
      ok[c] = b < nbk;
      bi[c] = ok[c] ? b : nbk - 1;
    }
    // 1) the matching h values (L2-resident)
    float hv[NCH][32];
    float hsum[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 f = *reinterpret_cast<const float4*>(h + 32 * bi[c] + 4 * v);
        hv[c][4 * v + 0] = f.x;
        hv[c][4 * v + 1] = f.y;
        hv[c][4 * v + 2] = f.z;
        hv[c][4 * v + 3] = f.w;
        s += (f.x + f.y) + (f.z + f.w);
      }
      hsum[c] = s;
    }
    constexpr int RB = 8 / NCH;  // rows per load batch
#pragma unroll
    for (int r0 = 0; r0 < 8; r0 += RB) {
      // 2) codes and scales of RB rows for this lane's blocks, all in flight together
      u32x4 q[RB][NCH];
      uint32_t sv[RB][NCH];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int n = min(n0 + 2 * (r0 + rr) + half, d - 1);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          q[rr][c] = ld16(qs + n * qstride + 16 * (size_t)bi[c]);
          sv[rr][c] = sc[n * sstride + bi[c]];
        }
      }
      // 3) dot products: codes converted exactly with v_cvt_f32_ubyte, offset folded per block
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float dot = 0.f;
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const uint32_t lo = q[rr][c][dw] & 0x0F0F0F0Fu, hi = (q[rr][c][dw] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) {
              dot = fmaf(hv[c][8 * dw + 2 * bt], (float)((lo >> (8 * bt)) & 0xFFu), dot);
              dot = fmaf(hv[c][8 * dw + 2 * bt + 1], (float)((hi >> (8 * bt)) & 0xFFu), dot);
            }
          }
          const float dsc = ok[c] ? fp16_bits_to_float(sv[rr][c]) : 0.f;
          acc = fmaf(dsc, fmaf(-8.f, hsum[c], dot), acc);
        }
        acc = half_wave_sum(acc);
        if (bl == 0) part[slot][2 * (r0 + rr) + half] = acc;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int n = n0 + threadIdx.x;
    if (n < d) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) acc = fmaf(topk_w[(size_t)t * k + j], part[j][threadIdx.x], acc);
      y[(size_t)t * d + n] = acc + part[k][threadIdx.x];
    }
  }
}

hipError_t launch_gemv_gateup(const Shape& s, const uint16_t* x, const int32_t* topk_ids, Q4 w13, Q4 s13,
                              float* h_r, float* h_s, hipStream_t st) {
  const int Imax = s.I > s.Is ? s.I : s.Is;
  dim3 grid((Imax + 15) / 16, s.T * s.k + s.T);
  if (s.d <= 4096)
    hipLaunchKernelGGL(k_gemv_gateup<1>, grid, dim3(256), 0, st, x, topk_ids, w13, s13, h_r, h_s, s.T, s.d, s.k, s.I,
                       s.Is, 0x000F000Fu, 0x43004300u);
  else
    hipLaunchKernelGGL(k_gemv_gateup<2>, grid, dim3(256), 0, st, x, topk_ids, w13, s13, h_r, h_s, s.T, s.d, s.k, s.I,
                       s.Is, 0x000F000Fu, 0x43004300u);
  return hipGetLastError();
}

hipError_t launch_gemv_down_combine(const Shape& s, const int32_t* topk_ids, const float* topk_w, Q4 w2, Q4 s2,
                                    const float* h_r, const float* h_s, float* y, hipStream_t st) {
  const int nw = (s.k + 1) < 16 ? (s.k + 1) : 16;
  const int Imax = s.I > s.Is ? s.I : s.Is;
  dim3 grid((s.d + 15) / 16, s.T);
  if (Imax <= 1024)
    hipLaunchKernelGGL(k_gemv_down_combine<1>, grid, dim3(64 * nw), 0, st, topk_ids, topk_w, w2, s2, h_r, h_s, y, s.T,
                       s.d, s.k, s.I, s.Is);
  else
    hipLaunchKernelGGL(k_gemv_down_combine<2>, grid, dim3(64 * nw), 0, st, topk_ids, topk_w, w2, s2, h_r, h_s, y, s.T,
                       s.d, s.k, s.I, s.Is);
  return hipGetLastError();
}

}  // namespace moe
