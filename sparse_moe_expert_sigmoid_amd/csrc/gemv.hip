// Small-T path: gathered Q4 GEMVs.
//
// Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine": decode runs
// the chosen experts as gathered Q4 GEMVs (moe_gather_q4 and the SwiGLU-fused
// moe_gather_q4_swiglu), with gate and up fused and the shared expert taken
// through the same gather.  Page thewafflehaus/FFAI pull request 72,
// "ffai_add3": routed terms are summed first, then the shared expert.
//
// Every (token, slot) pair is a job that streams its expert's rows straight
// from HBM.  The Q4 matrices are stored in 16-row groups (codes
// [rows/16][K/32][16][16 B], scales [rows/16][K/32][16]), so a wavefront
// reads one 16-row x 4-block tile -- 1 KiB of contiguous codes and 128
// contiguous scale bytes -- per load instruction; lane (n, G) gets row n,
// block G of the tile.  The activation slice a lane needs changes with G and
// with the tile, so each wavefront stages its part of the activations in LDS
// once, already in the operand pair order.  No routing build is needed: jobs
// read topk_ids directly.
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "topk.hpp"

namespace moe {

// 4-block tiles per row group a wavefront loads together before any arithmetic: the gate+up takes its
// whole quarter of K (8 tiles at d = 4096) at once; the down pass (8 tiles at I = 1024) goes in two
// batches of 4, so that the first batch's arithmetic overlaps the second's loads (0.26 us less per
// decode step on MI355X; the gate+up loses 1.3 us the same way)
constexpr int kGemvTiles = 8;
constexpr int kDownTiles = 4;
static_assert(kMaxGemvBlocksPerWave == kWave, "activation staging gives every lane one block");

// ---------------------------------------------------------------------------
// Gate+up with SwiGLU.  grid = (ceil(max(I, Is)/16), P + T); a workgroup of 4
// wavefronts covers 16 h-rows (one 16-row group of gate rows and the matching
// group of up rows) of one job; wavefront w takes the w-th quarter of K.  For
// each 4-block tile a lane holds one gate and one up code block (row n, block
// G).  The arithmetic is the down kernel's (below): codes become the fp16
// pairs (1024 + e0, 1024 + e4) and (1024 + 16 e1, 1024 + 16 e5) with one
// and-or each (elements 2, 6 and 3, 7 from the dword shifted by 8), x is
// staged as the matching fp16 pairs with the 16x pairs pre-divided by 16, and
// each block's v_dot2_f32_f16 chain starts at -(1032 A + 1152 B) (A the sum of
// the plain pairs, B of the divided ones), leaving sum x (q - 8).  x is
// rounded to fp16 (exact for bf16 values inside the fp16 normal range).
// Partial sums meet across G (lane exchanges) and across the 4 quarters (LDS).
// h is written in fp16 (h_r[p][I] for pair p, h_s[t][Is] for the shared
// expert), each group of 8 stored in the pair order of the down kernel: slot
// i of a group holds element 0,4,1,5,2,6,3,7 [i].
//
// Both kernels are compiled without floating-point contraction (the multiply-adds meant as one FMA are
// written as fmaf): the instantiations used by the separate calls and by moe_layer_forward then round
// alike, bit for bit.
//
// NPER = 0: the expert of each pair comes from ids.  NPER > 0 (the key registers per lane of the
// selection, ceil(E/64)): a routed workgroup selects its token's experts itself from the router's
// logits with one wavefront (the same selection as the top-k launch, so the same experts, order and
// weights), and the workgroup of row group 0 and slot 0 writes the selection to ids and topk_w for
// the down pass; this takes the top-k launch off the decode step.

// v plus its value in lane l ^ 16 (XOR16) or l ^ 32: gfx950 lane swaps between rows / halves of the
// wavefront, no LDS round trip.  The swap returns {first operand, second operand} after the exchange.
template <int XOR>
__device__ __forceinline__ float add_lane_xor(float v, int lane) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  if constexpr (XOR == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return v + __builtin_bit_cast(float, ((lane >> 4) & 1) ? p[0] : p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return v + __builtin_bit_cast(float, lane >= 32 ? p[0] : p[1]);
  }
}

template <int NPER>
__global__ __launch_bounds__(256) void k_gemv_gateup(const uint16_t* __restrict__ x, int32_t* __restrict__ ids,
                                                     Q4 w13, Q4 s13, _Float16* __restrict__ h_r, _Float16* __restrict__ h_s,
                                                     int T, int d, int k, int I, int Is, uint32_t mask_lo, uint32_t mask_hi,
                                                     uint32_t magic, const float* __restrict__ logits,
                                                     const float* __restrict__ bias, float* __restrict__ topk_w, int E) {
#pragma clang fp contract(off)
  // x of this wavefront's quarter of K, per block: 16 dwords of fp16 pairs and the block's starting value
  __shared__ __attribute__((aligned(16))) uint32_t xs[4][kMaxGemvBlocksPerWave][16];
  __shared__ float xsum[4][kMaxGemvBlocksPerWave];
  __shared__ float red[4][2][16];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int job = blockIdx.y;
  const int P = T * k;
  const int i0 = blockIdx.x * 16;
  const bool routed = job < P;  // uniform over the workgroup
  const int Iw = routed ? I : Is;
  if (i0 >= Iw) return;  // uniform over the workgroup (Iw % 32 == 0): no barrier is skipped by part of it
  const int t = routed ? job / k : job - P;
  const int nkb = d / 32;
  const int ntile = (nkb + 3) / 4;
  const int tw0 = (ntile * wave) / 4, tw1 = (ntile * (wave + 1)) / 4;  // this wavefront's tiles
  const int b0 = 4 * tw0;                                               // its first block
  // x of this wavefront's blocks: lane l takes block b0 + l (clamped; blocks past the wavefront's last
  // one are never read; a quarter of K holds at most 64 blocks as d <= 8192).  The loads go out first,
  // so that with NPER > 0 the selection's logit loads are in flight with them.
  const int bl = min(b0 + lane, nkb - 1);
  const uint16_t* xb = x + (size_t)t * d + 32 * bl;
  u32x4 xr[4];
#pragma unroll
  for (int dw = 0; dw < 4; ++dw) xr[dw] = ld16(xb + 8 * dw);
  // the expert of this job and the slot whose h row it writes: with the selection inside (NPER > 0) job
  // (t, j) takes the j-th chosen expert in id order, which needs only the chosen set, and writes the row
  // of that expert's slot; the slot order and the weights for the down pass are written by the workgroup
  // of row group 0 and j = 0, while its weight loads are in flight
  int e = 0, hslot = routed ? job % k : 0;
  uint64_t chosen[NPER > 0 ? NPER : 1];
  uint32_t key[NPER > 0 ? NPER : 1];
  float ssc[NPER > 0 ? NPER : 1];
  bool rank_pending = false;
  __shared__ TopkLds tsm;
  if constexpr (NPER > 0) {
    // every wavefront finds the chosen set itself (the same bits in each), so no barrier hands it over
    if (routed) {
      topk_chosen<NPER, 1>(logits + (size_t)t * E, 0, bias, E, k, lane, chosen, key, ssc);
      e = __builtin_amdgcn_readfirstlane(topk_nth_chosen<NPER>(chosen, job % k));
      hslot = __builtin_amdgcn_readfirstlane(topk_slot_of<NPER>(chosen, key, e, lane));
      rank_pending = wave == 0 && blockIdx.x == 0 && job % k == 0;
    }
  } else {
    if (routed) e = ids[job];
  }
  auto rank_write = [&]() __attribute__((always_inline)) {
    if constexpr (NPER > 0) {
      if (rank_pending) {  // uniform over the wavefront
        topk_rank_write<NPER>(chosen, key, ssc, ids + (size_t)t * k, topk_w + (size_t)t * k, k, lane, tsm, true);
        rank_pending = false;
      }
    }
  };
  const uint8_t* qs = routed ? w13.qs + (size_t)e * (2 * (size_t)I) * (d / 2) : s13.qs;
  const uint16_t* sc = routed ? w13.sc + (size_t)e * (2 * (size_t)I) * (d / 32) : s13.sc;
  _Float16* out = routed ? h_r + ((size_t)t * k + hslot) * I : h_s + (size_t)t * Is;
  const size_t grp_bytes = (size_t)nkb * 256;  // one 16-row group of codes
  const uint8_t* qg = qs + (size_t)(i0 >> 4) * grp_bytes;          // gate rows i0 .. i0+15
  const uint8_t* qu = qs + (size_t)((Iw + i0) >> 4) * grp_bytes;   // up rows Iw+i0 ..
  const uint16_t* sg = sc + (size_t)(i0 >> 4) * nkb * 16;
  const uint16_t* su = sc + (size_t)((Iw + i0) >> 4) * nkb * 16;
  // stage x as fp16 pairs in the dot-product order, with each block's starting value
  {
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const u32x4 u = xr[dw];
      float xf[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        xf[2 * m] = clamp_f16_range(bf16_bits_to_float(u[m] & 0xFFFFu));  // saturated to the fp16 range
        xf[2 * m + 1] = clamp_f16_range(bf16_bits_to_float(u[m] >> 16));
      }
      const half2v p0 = {(_Float16)xf[0], (_Float16)xf[4]};
      const half2v p1 = {(_Float16)(0.0625f * xf[1]), (_Float16)(0.0625f * xf[5])};
      const half2v p2 = {(_Float16)xf[2], (_Float16)xf[6]};
      const half2v p3 = {(_Float16)(0.0625f * xf[3]), (_Float16)(0.0625f * xf[7])};
      sa += ((float)p0[0] + (float)p0[1]) + ((float)p2[0] + (float)p2[1]);
      sb += ((float)p1[0] + (float)p1[1]) + ((float)p3[0] + (float)p3[1]);
      *reinterpret_cast<u32x4*>(xs[wave][lane] + 4 * dw) =
          u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    }
    xsum[wave][lane] = -fmaf(1032.f, sa, 1152.f * sb);
  }
  wave_lds_sync();  // the tiles below read the blocks other lanes staged
  // codes and scales of up to kGemvTiles tiles per batch, all in flight before any arithmetic; blocks
  // past the row end (last tile) re-read the row's last block and weigh zero.
  u32x4 cg[kGemvTiles], cu[kGemvTiles];
  uint32_t dg[kGemvTiles], du[kGemvTiles];
  int blk[kGemvTiles];
#define MOE_GU_LOAD(TB)                                                        \
  _Pragma("unroll") for (int j = 0; j < kGemvTiles; ++j) {                     \
    const int b = min(4 * min((TB) + j, tw1 - 1) + G, nkb - 1);               \
    blk[j] = b;                                                                \
    cg[j] = ld16(qg + (size_t)b * 256 + 16 * n);                               \
    cu[j] = ld16(qu + (size_t)b * 256 + 16 * n);                               \
    dg[j] = sg[(size_t)b * 16 + n];                                            \
    du[j] = su[(size_t)b * 16 + n];                                            \
  }
  float accg = 0.f, accu = 0.f;
  for (int tb = tw0; tb < tw1; tb += kGemvTiles) {
    MOE_GU_LOAD(tb);
    rank_write();  // the slot order and weights while this batch of weights is in flight
#pragma unroll
    for (int j = 0; j < kGemvTiles; ++j) {
      const int b = 4 * (tb + j) + G;  // the block this lane owns in tile tb + j
      const float use = (tb + j < tw1 && b < nkb) ? 1.f : 0.f;
      const int lb = blk[j] - b0;      // its slot in the staged x
      const u32x4* xp = reinterpret_cast<const u32x4*>(xs[wave][lb]);
      float dotg = xsum[wave][lb], dotu = dotg;
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const u32x4 xv = xp[dw];
        const uint32_t wg = cg[j][dw], wg8 = wg >> 8, wu = cu[j][dw], wu8 = wu >> 8;
        dotg = dot2_f16(and_or(wg, mask_lo, magic), xv[0], dotg);
        dotu = dot2_f16(and_or(wu, mask_lo, magic), xv[0], dotu);
        dotg = dot2_f16(and_or(wg, mask_hi, magic), xv[1], dotg);
        dotu = dot2_f16(and_or(wu, mask_hi, magic), xv[1], dotu);
        dotg = dot2_f16(and_or(wg8, mask_lo, magic), xv[2], dotg);
        dotu = dot2_f16(and_or(wu8, mask_lo, magic), xv[2], dotu);
        dotg = dot2_f16(and_or(wg8, mask_hi, magic), xv[3], dotg);
        dotu = dot2_f16(and_or(wu8, mask_hi, magic), xv[3], dotu);
      }
      // masked by a multiply (not a select), so that no load is made conditional
      accg = fmaf(fp16_bits_to_float(dg[j]) * use, dotg, accg);
      accu = fmaf(fp16_bits_to_float(du[j]) * use, dotu, accu);
    }
  }
#undef MOE_GU_LOAD
  rank_write();  // a wavefront without K tiles of its own
  // sum over G (lanes n, n+16, n+32, n+48), then over the 4 quarters in order
  accg = add_lane_xor<16>(accg, lane);
  accu = add_lane_xor<16>(accu, lane);
  accg = add_lane_xor<32>(accg, lane);
  accu = add_lane_xor<32>(accu, lane);
  if (lane < 16) {
    red[wave][0][lane] = accg;
    red[wave][1][lane] = accu;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int r = threadIdx.x;
    const float g = ((red[0][0][r] + red[1][0][r]) + red[2][0][r]) + red[3][0][r];
    const float u = ((red[0][1][r] + red[1][1][r]) + red[2][1][r]) + red[3][1][r];
    const int i = i0 + r;
    out[(i & ~7) + perm_slot(i & 7)] = to_f16_sat(siluf_(g) * u);
  }
}

// ---------------------------------------------------------------------------
// Down projection fused with the combine.  grid = (d/16, T); the workgroup
// has min(k+1, 16) wavefronts that take the slots j = wave, wave + nw, ...
// (slot k is the shared expert).  A wavefront computes the 16 output rows of
// its slot (one 16-row group) over all of K = I, one 4-block tile per load
// instruction; it stages the slot's h in LDS first.  Partial dot products
// meet across G (lane exchanges), then in LDS, and one thread per row sums
// them in slot order: y = sum_j w_j * dot_j, then + shared.
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
__global__ __launch_bounds__(1024) void k_gemv_down_combine(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ topk_w, Q4 w2, Q4 s2,
                                                            const _Float16* __restrict__ h_r,
                                                            const _Float16* __restrict__ h_s, const float* residual,
                                                            float* y, uint16_t* __restrict__ y_bf16,
                                                            int T, int d, int k, int I, int Is, uint32_t mask_lo,
                                                            uint32_t mask_hi, uint32_t magic) {
#pragma clang fp contract(off)
  // per wavefront: the slot's h, per block 16 dwords of fp16 pairs (the 16x pairs pre-divided by 16)
  // and the block's starting value -(1032 A + 72 B)
  __shared__ __attribute__((aligned(16))) uint32_t hsm[16][kMaxGemvBlocksPerWave][16];
  __shared__ float hc0[16][kMaxGemvBlocksPerWave];
  __shared__ float part[kMaxTopK + 1][16];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int nw = blockDim.x >> 6;
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * 16;  // one 16-row group (d % 32 == 0: all rows valid)
  for (int slot = wave; slot <= k; slot += nw) {
    // the slot's h first: its address does not depend on the expert id, so these loads are in flight
    // while the id is read (lane l takes block l, clamped; blocks past nkb are never read; nkb <= 64 as
    // I <= 2048)
    const int Kw = slot < k ? I : Is;
    const _Float16* h = slot < k ? h_r + ((size_t)t * k + slot) * I : h_s + (size_t)t * Is;
    const int nkb = Kw / 32;
    const int bl = min(lane, nkb - 1);
    u32x4 hv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) hv[g] = ld16(h + 32 * bl + 8 * g);
    const uint8_t* qs;
    const uint16_t* sc;
    if (slot < k) {
      const int e = ids[(size_t)t * k + slot];
      qs = w2.qs + (size_t)e * d * (I / 2);
      sc = w2.sc + (size_t)e * d * (I / 32);
    } else {
      qs = s2.qs;
      sc = s2.sc;
    }
    const int ntile = (nkb + 3) / 4;
    const uint8_t* qg = qs + (size_t)(n0 >> 4) * nkb * 256;
    const uint16_t* sg = sc + (size_t)(n0 >> 4) * nkb * 16;
    // codes and scales of up to kDownTiles tiles per batch, all in flight before any arithmetic;
    // the first batch is issued before h is staged, so that the two loads overlap
    u32x4 cq[kDownTiles];
    uint32_t dq[kDownTiles];
    int blk[kDownTiles];
#define MOE_DN_LOAD(TB)                                                        \
    _Pragma("unroll") for (int j = 0; j < kDownTiles; ++j) {                   \
      const int b = min(4 * min((TB) + j, ntile - 1) + G, nkb - 1);           \
      blk[j] = b;                                                              \
      cq[j] = ld16(qg + (size_t)b * 256 + 16 * n);                             \
      dq[j] = sg[(size_t)b * 16 + n];                                          \
    }
    MOE_DN_LOAD(0);
    // stage h
    {
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 v = hv[g];
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
        *reinterpret_cast<u32x4*>(hsm[wave][lane] + 4 * g) = v;
      }
      hc0[wave][lane] = -fmaf(1032.f, sa, 72.f * sb);
    }
    wave_lds_sync();  // the tiles below read the blocks other lanes staged
    float acc = 0.f;
    for (int tb = 0; tb < ntile; tb += kDownTiles) {
      if (tb != 0) MOE_DN_LOAD(tb);
#pragma unroll
      for (int j = 0; j < kDownTiles; ++j) {
        const float use = (tb + j < ntile && 4 * (tb + j) + G < nkb) ? 1.f : 0.f;
        const u32x4* hp = reinterpret_cast<const u32x4*>(hsm[wave][blk[j]]);
        float dot = hc0[wave][blk[j]];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 hv = hp[g];
          const uint32_t w = cq[j][g], w8 = w >> 8;
          dot = dot2_f16(and_or(w, mask_lo, magic), hv[0], dot);
          dot = dot2_f16(and_or(w, mask_hi, magic), hv[1], dot);
          dot = dot2_f16(and_or(w8, mask_lo, magic), hv[2], dot);
          dot = dot2_f16(and_or(w8, mask_hi, magic), hv[3], dot);
        }
        // masked by a multiply (not a select), so that no load is made conditional
        acc = fmaf(fp16_bits_to_float(dq[j]) * use, dot, acc);
      }
    }
#undef MOE_DN_LOAD
    acc = add_lane_xor<16>(acc, lane);
    acc = add_lane_xor<32>(acc, lane);
    if (lane < 16) part[slot][lane] = clamp_f16_range(acc);  // each expert's output saturates as on the grouped path
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int r = n0 + threadIdx.x;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(topk_w[(size_t)t * k + j], part[j][threadIdx.x], acc);
    float v = acc + part[k][threadIdx.x];
    if (residual) v += residual[(size_t)t * d + r];  // after routed + shared; residual may be y itself
    y[(size_t)t * d + r] = v;
    if (y_bf16) y_bf16[(size_t)t * d + r] = float_to_bf16_bits(v);
  }
}

hipError_t launch_gemv_gateup(const Shape& s, const uint16_t* x, const int32_t* topk_ids, Q4 w13, Q4 s13,
                              _Float16* h_r, _Float16* h_s, hipStream_t st) {
  const int Imax = s.I > s.Is ? s.I : s.Is;
  dim3 grid((Imax + 15) / 16, s.T * s.k + s.T);
  hipLaunchKernelGGL(k_gemv_gateup<0>, grid, dim3(256), 0, st, x, const_cast<int32_t*>(topk_ids), w13, s13, h_r, h_s,
                     s.T, s.d, s.k, s.I, s.Is, 0x000F000Fu, 0x00F000F0u, 0x64006400u, nullptr, nullptr, nullptr, s.E);
  return hipGetLastError();
}

template <int NPER>
static void gateup_select_nper(const Shape& s, const uint16_t* x, const float* logits, const float* bias,
                               int32_t* topk_ids, float* topk_w, Q4 w13, Q4 s13, _Float16* h_r, _Float16* h_s,
                               hipStream_t st) {
  const int Imax = s.I > s.Is ? s.I : s.Is;
  dim3 grid((Imax + 15) / 16, s.T * s.k + s.T);
  hipLaunchKernelGGL(k_gemv_gateup<NPER>, grid, dim3(256), 0, st, x, topk_ids, w13, s13, h_r, h_s, s.T, s.d, s.k, s.I,
                     s.Is, 0x000F000Fu, 0x00F000F0u, 0x64006400u, logits, bias, topk_w, s.E);
}

hipError_t launch_gemv_gateup_select(const Shape& s, const uint16_t* x, const float* logits, const float* bias,
                                     int32_t* topk_ids, float* topk_w, Q4 w13, Q4 s13, _Float16* h_r, _Float16* h_s,
                                     hipStream_t st) {
  const int nper = (s.E + 63) / 64;
  if (nper <= 1) gateup_select_nper<1>(s, x, logits, bias, topk_ids, topk_w, w13, s13, h_r, h_s, st);
  else if (nper <= 2) gateup_select_nper<2>(s, x, logits, bias, topk_ids, topk_w, w13, s13, h_r, h_s, st);
  else if (nper <= 4) gateup_select_nper<4>(s, x, logits, bias, topk_ids, topk_w, w13, s13, h_r, h_s, st);
  else if (nper <= 8) gateup_select_nper<8>(s, x, logits, bias, topk_ids, topk_w, w13, s13, h_r, h_s, st);
  else gateup_select_nper<16>(s, x, logits, bias, topk_ids, topk_w, w13, s13, h_r, h_s, st);
  return hipGetLastError();
}

hipError_t launch_gemv_down_combine(const Shape& s, const int32_t* topk_ids, const float* topk_w, Q4 w2, Q4 s2,
                                    const _Float16* h_r, const _Float16* h_s, const float* residual, float* y,
                                    uint16_t* y_bf16, hipStream_t st) {
  const int nw = (s.k + 1) < 16 ? (s.k + 1) : 16;
  dim3 grid(s.d / 16, s.T);
  hipLaunchKernelGGL(k_gemv_down_combine, grid, dim3(64 * nw), 0, st, topk_ids, topk_w, w2, s2, h_r, h_s, residual, y, y_bf16, s.T, s.d,
                     s.k, s.I, s.Is, 0x000F000Fu, 0x00F000F0u, 0x64006400u);
  return hipGetLastError();
}

}  // namespace moe
