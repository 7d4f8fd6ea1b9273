// Grouped path: gate+up (SwiGLU epilogue) and down as grouped GEMMs on the
// fp16 MFMA units of gfx950, then a fixed-order combine.
//
// Page "feat(laguna): batched prefill with tensor-core projections, fused
// MoE, CTA scheduling": grouped-GEMM MoE with on-device descriptors, fused
// gate+up expert stacks, descending-size expert order plus N-banded
// workgroup order for weight reuse in cache.  Page thewafflehaus/FFAI pull
// request 72 (Nemotron MoE commits): activations gathered on read through the
// router-sorted token indices (no separate gather pass), per-pair outputs
// combined by a deterministic scatter-add, routed terms summed before the
// shared expert ("ffai_add3"), and a K-loop that never reads past the weight
// buffer when K is not a multiple of the tile ("tile-select fix").
//
// Work items: for each group (expert, or the shared expert as group E) in
// schedule order, its M-tiles of up to 128 rows times the N-bands of the
// output.  Default order is band-major inside a group (all M-tiles of one
// weight band adjacent), and the launch index is remapped so that each XCD
// (own L2) receives a contiguous run of items.  The grid is sized for the
// largest possible tile count; surplus workgroups exit at once, so the launch
// shape does not depend on device data and the call can be graph-captured.
//
// Inner loop (per 128-wide K step): the workgroup stages its 128 activation
// rows x 128 columns as fp16 in LDS (double-buffered); each wavefront owns
// four 16-column weight slices, loads one 16-byte Q4 block per slice and
// lane, dequantises it in registers straight into the B-operand layout of
// v_mfma_f32_16x16x32_f16 and multiplies it against every 16-row slice of
// the activation tile.  K is permuted consistently: MFMA k-lane group G of
// step s holds elements 32G + 8s .. 32G + 8s + 7 of the 128-wide chunk, which
// are exactly dword s of Q4 block G.
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "../../include/moe_q4.h"

namespace moe {

// LDS tile: 128 rows x 128 halves (256 B) per buffer, no padding.  The 16 B
// chunk c of row r is stored in slot c ^ (r & 15), so the 16 lanes that read
// one MFMA operand (16 rows, same chunk) hit 16 different slots, i.e. all 64
// banks once.  Tiles arrive by global_load_lds_dwordx4: one instruction moves
// 64 x 16 B into 1 KB of consecutive LDS (4 rows), lane l filling slot l%16
// of row l/16, so the swizzle is applied on the global address side.
constexpr int kRowBytes = kGroupedBK * 2;

struct GArgs {
  const _Float16* a_r;      // A rows: gate+up -> x16 [T][d] (gathered); down -> h_r [P][I] (sorted rows)
  const _Float16* a_s;      // A rows of the shared group: gate+up -> x16; down -> h_s [T][Is]
  Q4 wr;                    // routed stack (w13 or w2)
  Q4 ws;                    // shared expert (s13 or s2)
  _Float16* h_r;            // gate+up outputs
  _Float16* h_s;
  float* y_r;               // down outputs
  float* y_s;
  const int* counts;
  const int* offsets;
  const int* sorted_pair;
  const int* group_order;
  const int* mt_prefix;
  int T, d, E, k, I, Is;
  int nbands;
  uint32_t flags;
};

typedef __attribute__((address_space(3))) void lds_void;

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_grouped(GArgs a) {
  constexpr int BM = kGroupedBM, BK = kGroupedBK;
  constexpr int BANDW = GATEUP ? kGateUpBandCols : kDownBandCols;
  __shared__ __attribute__((aligned(1024))) char As[2][BM * kRowBytes];
  __shared__ int s_prefix[kMaxExperts + 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngroups = a.E + 1;
  for (int i = tid; i <= ngroups; i += 256) s_prefix[i] = a.mt_prefix[i];
  __syncthreads();
  const int nb = a.nbands;
  const int n_items = s_prefix[ngroups] * nb;
  if ((int)blockIdx.x >= n_items) return;
  const int item = xcd_remap(blockIdx.x, n_items);
  int lo = 0, hi = ngroups;  // s_prefix[lo]*nb <= item < s_prefix[hi]*nb
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_prefix[mid] * nb <= item) lo = mid; else hi = mid;
  }
  const int rank = lo;
  const int g = a.group_order[rank];
  const int nmt = s_prefix[rank + 1] - s_prefix[rank];
  const int local = item - s_prefix[rank] * nb;
  int band, mtile;
  if (a.flags & MOE_FLAG_NO_BANDING) {
    mtile = local / nb;
    band = local % nb;
  } else {
    band = local / nmt;
    mtile = local % nmt;
  }
  const bool shared = (g == a.E);
  const int cnt = shared ? a.T : a.counts[g];
  const int Iw = shared ? a.Is : a.I;
  const int Kdim = GATEUP ? a.d : Iw;
  const int Ndim = GATEUP ? Iw : a.d;
  if (band * BANDW >= Ndim) return;  // uniform across the workgroup
  const int m0 = mtile * BM;
  const int mlen = min(BM, cnt - m0);
  const int rbase = shared ? m0 : a.offsets[g] + m0;  // first output row (token or sorted position)
  const size_t wrows = GATEUP ? 2 * (size_t)Iw : (size_t)a.d;
  const uint8_t* Wq = shared ? a.ws.qs : a.wr.qs + (size_t)g * wrows * (Kdim / 2);
  const uint16_t* Ws = shared ? a.ws.sc : a.wr.sc + (size_t)g * wrows * (Kdim / 32);

  // ---- A rows staged by this wavefront: rows 32*wave + 4*i + lane/16, slot lane%16
  const char* abase = reinterpret_cast<const char*>(shared ? a.a_s : a.a_r);
  uint32_t aoff[8];  // byte offset of the row start, plus the swizzled chunk
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 32 * wave + 4 * i + (lane >> 4);
    const int rr = row < mlen ? row : 0;  // rows past the group read row 0: finite, and discarded
    size_t arow;
    if (GATEUP)
      arow = shared ? (size_t)(m0 + rr) : (size_t)(a.sorted_pair[a.offsets[g] + m0 + rr] / a.k);
    else
      arow = shared ? (size_t)(m0 + rr) : (size_t)(a.offsets[g] + m0 + rr);
    const int chunk = (lane & 15) ^ (row & 15);
    aoff[i] = (uint32_t)(arow * (size_t)Kdim * 2 + 16 * chunk);
  }
  const bool ktail = (Kdim % BK) != 0;
  auto issue_a = [&](int it, int buf) {
    const uint32_t kb = (uint32_t)it * BK * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t off = aoff[i] + kb;
      // a chunk past the end of the row reads the tile's first chunk instead: finite data that
      // meets zero weights (the weight K tail is zero-filled)
      if (ktail && (int)(it * BK + 8 * ((lane & 15) ^ ((32 * wave + 4 * i + (lane >> 4)) & 15))) >= Kdim)
        off = aoff[i] - 16 * (uint32_t)((lane & 15) ^ ((32 * wave + 4 * i + (lane >> 4)) & 15)) + kb;
      __builtin_amdgcn_global_load_lds(abase + off, (lds_void*)&As[buf][(32 * wave + 4 * i) * kRowBytes], 16, 0, 0);
    }
  };

  // ---- this wavefront's weight rows: four 16-row slices
  const int n = lane & 15, G = lane >> 4;
  int wrow[4];
  bool nok[4];
  int c0;
  if (GATEUP) {
    c0 = band * BANDW + wave * 32;  // h columns c0 .. c0+31: gate rows, then the matching up rows
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = c0 + 16 * (ns & 1);
      nok[ns] = col < Iw;
      wrow[ns] = (ns < 2 ? 0 : Iw) + (nok[ns] ? col : 0) + n;
    }
  } else {
    c0 = band * BANDW + wave * 64;  // output columns c0 .. c0+63
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = c0 + 16 * ns;
      nok[ns] = col < a.d;
      wrow[ns] = (nok[ns] ? col : 0) + n;
    }
  }
  const size_t qstride = Kdim / 2, sstride = Kdim / 32;
  const int nkb = Kdim / 32;
  const int nit = (Kdim + BK - 1) / BK;

  u32x4 q[4];
  uint32_t sc[4];
  auto load_w = [&](int it, u32x4* qd, uint32_t* sd) {
    const int blk = it * 4 + G;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      if (nok[ns] && blk < nkb) {  // never read past the row: the K tail is zero-filled
        qd[ns] = ld16(Wq + wrow[ns] * qstride + 16 * (size_t)blk);
        sd[ns] = Ws[wrow[ns] * sstride + blk];
      } else {
        qd[ns] = u32x4{0u, 0u, 0u, 0u};
        sd[ns] = 0u;
      }
    }
  };

  floatx4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[mt][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

  load_w(0, q, sc);
  issue_a(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // all counters: the first tile has landed in LDS
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nit;
    u32x4 qn[4];
    uint32_t sn[4];
    if (more) {
      issue_a(it + 1, cur ^ 1);
      load_w(it + 1, qn, sn);
    }
    half2v d2[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const _Float16 dv = __builtin_bit_cast(_Float16, (uint16_t)sc[ns]);
      d2[ns] = half2v{dv, dv};
    }
    const char* Acur = As[cur];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 b[4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) b[ns] = dequant8_f16(q[ns][s], d2[ns]);
      const int slot = (4 * G + s) ^ n;  // row mt*16 + n has (row & 15) == n
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        if (mt * 16 < mlen) {
          const half8 am = *reinterpret_cast<const half8*>(Acur + (mt * 16 + n) * kRowBytes + 16 * slot);
#pragma unroll
          for (int ns = 0; ns < 4; ++ns)
            if (nok[ns]) acc[mt][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, b[ns], acc[mt][ns], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        q[ns] = qn[ns];
        sc[ns] = sn[ns];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // next tile in LDS, next weights in registers
    __syncthreads();
  }

  // ---- epilogue.  D layout: lane holds column n of rows 4G..4G+3 of each 16x16 tile.
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt * 16 >= mlen) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * G + i;
      if (row >= mlen) continue;
      if (GATEUP) {
        _Float16* out = shared ? a.h_s : a.h_r;
#pragma unroll
        for (int xh = 0; xh < 2; ++xh) {
          if (!nok[xh]) continue;
          const float gv = acc[mt][xh][i], uv = acc[mt][2 + xh][i];
          out[(size_t)(rbase + row) * Iw + c0 + 16 * xh + n] = (_Float16)(siluf_(gv) * uv);
        }
      } else {
        float* out = shared ? a.y_s : a.y_r;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          if (!nok[ns]) continue;
          out[(size_t)(rbase + row) * a.d + c0 + 16 * ns + n] = acc[mt][ns][i];
        }
      }
    }
  }
}

// bf16 -> fp16 copy of the activations for the gate+up A operand.  The
// conversion is exact inside the fp16 range; round-toward-zero saturates
// values beyond it to +-65504.
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, _Float16* __restrict__ x16,
                                                  size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  u32x4 v = ld16(x + 8 * i);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float lo = __builtin_bit_cast(float, v[m] << 16);
    const float hi = __builtin_bit_cast(float, v[m] & 0xFFFF0000u);
    v[m] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  *reinterpret_cast<u32x4*>(x16 + 8 * i) = v;
}

// Combine: y[t] = (sum_j w[t,j] * y_pair[pair_pos[t*k+j]]) + y_shared[t], j ascending, no atomics.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ topk_w, const int* __restrict__ pair_pos,
                                                 const float* __restrict__ y_r, const float* __restrict__ y_s,
                                                 float* __restrict__ y, int d, int k) {
  const int per_row = (d + 1023) / 1024;
  const int t = blockIdx.x / per_row;
  const int col = ((blockIdx.x % per_row) * 256 + threadIdx.x) * 4;
  if (col >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int pp = pair_pos[(size_t)t * k + j];
    if (pp < 0) continue;
    const float w = topk_w[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y_r + (size_t)pp * d + col);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  const float4 s = *reinterpret_cast<const float4*>(y_s + (size_t)t * d + col);
  *reinterpret_cast<float4*>(y + (size_t)t * d + col) =
      make_float4(acc.x + s.x, acc.y + s.y, acc.z + s.z, acc.w + s.w);
}

int grouped_max_mtiles(const Shape& s) {
  // sum_e ceil(c_e / BM) <= floor(P / BM) + min(E, P), plus the shared group
  const long P = (long)s.T * s.k;
  const long routed = P / kGroupedBM + (P < s.E ? P : s.E);
  return (int)(routed + (s.T + kGroupedBM - 1) / kGroupedBM);
}

static GArgs make_args(const Shape& s, const Routing& r, uint32_t flags) {
  GArgs a{};
  a.counts = r.counts;
  a.offsets = r.offsets;
  a.sorted_pair = r.sorted_pair;
  a.group_order = r.group_order;
  a.mt_prefix = r.mt_prefix;
  a.T = s.T; a.d = s.d; a.E = s.E; a.k = s.k; a.I = s.I; a.Is = s.Is;
  a.flags = flags;
  return a;
}

hipError_t launch_grouped_gateup(const Shape& s, const uint16_t* x, const Routing& r, Q4 w13, Q4 s13,
                                 const GroupedOut& o, uint32_t flags, hipStream_t st) {
  const size_t n8 = (size_t)s.T * s.d / 8;
  hipLaunchKernelGGL(k_x_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, x, o.x16, n8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GArgs a = make_args(s, r, flags);
  a.a_r = o.x16;
  a.a_s = o.x16;
  a.wr = w13;
  a.ws = s13;
  a.h_r = o.h_r;
  a.h_s = o.h_s;
  const int Imax = s.I > s.Is ? s.I : s.Is;
  a.nbands = (Imax + kGateUpBandCols - 1) / kGateUpBandCols;
  const long grid = (long)grouped_max_mtiles(s) * a.nbands;
  hipLaunchKernelGGL(k_grouped<true>, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_grouped_down(const Shape& s, const Routing& r, Q4 w2, Q4 s2, const GroupedOut& o, uint32_t flags,
                               hipStream_t st) {
  GArgs a = make_args(s, r, flags);
  a.a_r = o.h_r;
  a.a_s = o.h_s;
  a.wr = w2;
  a.ws = s2;
  a.y_r = o.y_pair;
  a.y_s = o.y_s;
  a.nbands = (s.d + kDownBandCols - 1) / kDownBandCols;
  const long grid = (long)grouped_max_mtiles(s) * a.nbands;
  hipLaunchKernelGGL(k_grouped<false>, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const float* topk_w, const Routing& r, const GroupedOut& o, float* y,
                          hipStream_t st) {
  dim3 grid(((s.d + 1023) / 1024) * s.T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, st, topk_w, r.pair_pos, o.y_pair, o.y_s, y, s.d, s.k);
  return hipGetLastError();
}

}  // namespace moe
