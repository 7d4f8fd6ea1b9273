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
// and the 4 matching up rows).  Lane l owns Q4 blocks l and l + 64 of every
// 128-block chunk of the row, so that each load instruction of a wavefront
// covers 1 KiB of contiguous codes (or 128 contiguous scale bytes).
// h is written in fp16 (h_r[p][I] for pair p, h_s[t][Is] for the shared
// expert), each group of 8 stored in the pair order of the down kernel: slot
// i of a group holds element 0,4,1,5,2,6,3,7 [i].
template <int NCH>
__global__ __launch_bounds__(256) void k_gemv_gateup(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                                                     Q4 w13, Q4 s13, _Float16* __restrict__ h_r, _Float16* __restrict__ h_s,
                                                     int T, int d, int k, int I, int Is, uint32_t mask, uint32_t magic) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int job = blockIdx.y;
  const int P = T * k;
  int t, Iw;
  const uint8_t* qs;
  const uint16_t* sc;
  _Float16* out;
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
    float okf[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 128 * c + 64 * bb + lane;
      ok[bb] = b < nb;
      okf[bb] = ok[bb] ? 1.f : 0.f;
      bi[bb] = ok[bb] ? b : nb - 1;
    }
    // 1) activation slices of this lane's blocks (L2-resident), issued first
    u32x4 u[2][4];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) u[bb][dw] = ld16(x + (size_t)t * d + 32 * bi[bb] + 8 * dw);
    // 2) weight codes of 8 rows and their scales: all loads in flight before any arithmetic.  Scales
    // are stored in 16-row groups ([rows/16][K/32][16]); the 4 gate (and the 4 up) rows of this
    // wavefront lie in one group, so one 8-byte load per block brings all four.
    u32x4 q[8][2];
    uint2 sg[2][2];  // [gate/up][bb]: fp16 scales of rows +0..+3
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = (r < 4) ? (i0 + r) : (Iw + i0 + r - 4);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) q[r][bb] = ld16(qs + row * qstride + 16 * (size_t)bi[bb]);
    }
#pragma unroll
    for (int gu = 0; gu < 2; ++gu) {
      const int r0 = gu ? Iw + i0 : i0;  // i0 % 4 == 0: rows r0 .. r0+3 share a 16-row group
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
        sg[gu][bb] = *reinterpret_cast<const uint2*>(sc + ((size_t)(r0 >> 4) * sstride + bi[bb]) * 16 + (r0 & 15));
    }
    uint32_t sv[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const uint2 v = sg[r >> 2][bb];
        const uint32_t d = ((r & 3) < 2) ? v.x : v.y;
        sv[r][bb] = (r & 1) ? (d >> 16) : (d & 0xFFFFu);
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
        // masked by a multiply (not a select), so that the scale load is never made conditional
        const float dsc = fp16_bits_to_float(sv[r][bb]) * okf[bb];
        acc[r] = fmaf(dsc, fmaf(-136.f, xs[bb], dot), acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = wave_sum_hi(acc[r]);
  if (lane >= 60) {  // lanes 60..63 hold the sums; lane 60 + r writes h-row i0 + r
    float g = acc[0], u = acc[4];
#pragma unroll
    for (int r = 1; r < 4; ++r)
      if (lane == 60 + r) {
        g = acc[r];
        u = acc[4 + r];
      }
    const int i = i0 + lane - 60;
    out[(i & ~7) + perm_slot(i & 7)] = (_Float16)(siluf_(g) * u);
  }
}

// ---------------------------------------------------------------------------
// Down projection fused with the combine.  grid = (ceil(d/16), T); the
// workgroup has min(k+1, 16) wavefronts that take the slots j = wave,
// wave + nw, ... (slot k is the shared expert).  A wavefront computes the
// 16 output rows of its slot, two rows at a time (32-lane half h takes rows
// 8h .. 8h+7); lane l%32 owns block l%32 (+32c) of the row and keeps the matching 32 h
// values in registers.  Partial dot products meet in LDS and one thread per
// row sums them in slot order: y = sum_j w_j * dot_j, then + shared.
//
// Dot products use v_dot2_f32_f16 on fp16 codes built with one and-or each:
// for a dword w of codes (element m in bits 4m..4m+3), w & 0x000F000F placed
// in the mantissa of 1024.0 gives the pair (1024 + e0, 1024 + e4), and
// w & 0x00F000F0 gives (1024 + 16 e1, 1024 + 16 e5), both exact; w >> 8 gives
// elements 2, 6 and 3, 7 the same way.  h arrives in the matching pair order
// (h0,h4) (h1,h5) (h2,h6) (h3,h7); the pairs that meet a 16x code are taken
// as h/16 (exact).  With A = sum of h over the 1024+q pairs and B over the
// 1024+16q pairs, a block's dot is 1024 A + 64 B + sum h*q, so starting each
// block's accumulation at -(1032 A + 72 B) leaves sum h*(q - 8).
template <int NCH>
__global__ __launch_bounds__(1024) void k_gemv_down_combine(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ topk_w, Q4 w2, Q4 s2,
                                                            const _Float16* __restrict__ h_r,
                                                            const _Float16* __restrict__ h_s, float* __restrict__ y,
                                                            int T, int d, int k, int I, int Is, uint32_t mask_lo,
                                                            uint32_t mask_hi, uint32_t magic) {
  __shared__ float part[kMaxTopK + 1][16];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * 16;
  const int half = lane >> 5, bl = lane & 31;
  for (int slot = wave; slot <= k; slot += nw) {
    const uint8_t* qs;
    const uint16_t* sc;
    const _Float16* h;
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
    float okf[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int b = bl + 32 * c;
      okf[c] = b < nbk ? 1.f : 0.f;
      bi[c] = b < nbk ? b : nbk - 1;
    }
    // 1) the matching h values (L2-resident): pairs, the 1024+16q pairs pre-divided by 16
    u32x4 hp[NCH][4];
    float c0[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 v = ld16(h + 32 * bi[c] + 8 * g);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const half2v hv = as_half2(v[m]);
          const float s2v = (float)hv[0] + (float)hv[1];
          if (m & 1) {
            sb += s2v;
            v[m] = __builtin_bit_cast(uint32_t, hv * half2v{(_Float16)0.0625f, (_Float16)0.0625f});
          } else {
            sa += s2v;
          }
        }
        hp[c][g] = v;
      }
      c0[c] = -(1032.f * sa + 72.f * sb);
    }
    // 2) codes and scales of RB row pairs for this lane's blocks, all in flight together; 3) dots
    // Half h of the wavefront takes rows n0 + 8h .. n0 + 8h + 7 (n0 % 16 == 0, d % 32 == 0: all valid),
    // so the 8 scales a lane needs for its block are 16 contiguous bytes of the [rows/16][K/32][16]
    // scale layout: one load per chunk.
    u32x4 sc8[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) sc8[c] = ld16(sc + ((size_t)(n0 >> 4) * sstride + bi[c]) * 16 + 8 * half);
    constexpr int RB = 8 / NCH;
#pragma unroll
    for (int r0 = 0; r0 < 8; r0 += RB) {
      u32x4 q[RB][NCH];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int n = n0 + 8 * half + r0 + rr;
#pragma unroll
        for (int c = 0; c < NCH; ++c) q[rr][c] = ld16(qs + n * qstride + 16 * (size_t)bi[c]);
      }
      float acc[RB];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        acc[rr] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float dot = c0[c];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t w = q[rr][c][g], w8 = w >> 8;
            dot = dot2_f16(and_or(w, mask_lo, magic), hp[c][g][0], dot);
            dot = dot2_f16(and_or(w, mask_hi, magic), hp[c][g][1], dot);
            dot = dot2_f16(and_or(w8, mask_lo, magic), hp[c][g][2], dot);
            dot = dot2_f16(and_or(w8, mask_hi, magic), hp[c][g][3], dot);
          }
          const int k8 = r0 + rr;  // compile-time: halfword k8 of the lane's 8 scales
          const uint32_t sbits = (sc8[c][k8 >> 1] >> (16 * (k8 & 1))) & 0xFFFFu;
          // masked by a multiply (not a select), so that no load is made conditional
          acc[rr] = fmaf(fp16_bits_to_float(sbits) * okf[c], dot, acc[rr]);
        }
      }
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) acc[rr] = half_wave_sum_hi(acc[rr]);
      if (bl == 16) {
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) part[slot][8 * half + r0 + rr] = acc[rr];
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
                              _Float16* h_r, _Float16* h_s, hipStream_t st) {
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
                                    const _Float16* h_r, const _Float16* h_s, float* y, hipStream_t st) {
  const int nw = (s.k + 1) < 16 ? (s.k + 1) : 16;
  const int Imax = s.I > s.Is ? s.I : s.Is;
  dim3 grid((s.d + 15) / 16, s.T);
  if (Imax <= 1024)
    hipLaunchKernelGGL(k_gemv_down_combine<1>, grid, dim3(64 * nw), 0, st, topk_ids, topk_w, w2, s2, h_r, h_s, y, s.T,
                       s.d, s.k, s.I, s.Is, 0x000F000Fu, 0x00F000F0u, 0x64006400u);
  else
    hipLaunchKernelGGL(k_gemv_down_combine<2>, grid, dim3(64 * nw), 0, st, topk_ids, topk_w, w2, s2, h_r, h_s, y, s.T,
                       s.d, s.k, s.I, s.Is, 0x000F000Fu, 0x00F000F0u, 0x64006400u);
  return hipGetLastError();
}

}  // namespace moe
