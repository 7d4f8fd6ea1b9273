// W4A8 and W8A8 variants of the grouped path: MXFP4 or MXFP8 expert weights times FP8 activations on
// the block-scaled MFMA of gfx950.
//
// Page thewafflehaus/FFAI pull request 72 ("Nemotron-Nano-30B GB10 prefill quality + speed wins"):
// W4A8 and W8A8 grouped MoE (fp8 activations times fp4 or fp8 weights) beside the Q4 W4A16 path; the
// fp4 MoE weights are the Q4 weights requantised to a block-scaled fp4 grid, and the fp8 activations
// carry a per-token scale applied to the product.  Here the fp4 grid is e2m1 (the fp8 one e4m3) in
// blocks of 32 with a shared power-of-two exponent (one byte, bias 127), the block formats that
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies directly: one such MFMA takes, per lane, one 32-value
// block of one weight row (MXFP8: two half blocks) as its weight operand with that block's exponent as
// its scale, so the main loop has no dequantisation at all.  Activations (x, then h) are e4m3 with one fp32 scale per row
// (amax / 448), applied to the fp32 accumulators in the epilogues.
//
// Operand layout of the MFMA (16 x 16 x 128, checked on the GPU against a host product): the fp4
// operand lane (n, G) = (l % 16, l / 16) holds row n, K values 32G .. 32G+31 (value j in nibble j,
// low nibble first), i.e. block G of the 128-value K step, and supplies block G's scale; the fp8
// operand lane (n, G) holds column n, K values 16G .. 16G+15 in its first four dwords and
// 64 + 16G .. 64 + 16G + 15 in the last four; the result is the 16 x 16 fp32 tile with lane (n, G)
// holding rows 4G .. 4G+3 of column n.  With the weights as the fp4 operand the tile comes out
// transposed, as on the W4A16 path: lane (n, G) holds, for activation row n, four consecutive
// output columns.
//
// Work items, schedule order, XCD remapping and the launch shape are those of the W4A16 grouped
// GEMM (grouped.hip); the K loop is 128 values per iteration with the next one or two steps'
// operands in flight (activation tiles in LDS, weight blocks in registers).  d, I and I_shared must be multiples of 128.
#include <type_traits>

#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_q4.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kMxBM = kGroupedBM;            // rows per M-tile of the routing build
constexpr int kMxBK = 128;                   // K per iteration: one MFMA
constexpr int kMxWaves = kGroupedWaves;
constexpr int kMxThreads = 64 * kMxWaves;
constexpr int kMxRowBytes = kMxBK;           // fp8 activations: 128 B per row and iteration
constexpr int kMxGateUpBandCols = kGateUpBandCols;
constexpr int kMxDownBandCols = kDownBandCols;
constexpr uint32_t kMxOffsetOOB = 0xFFFFFFF0u;
// Rows a workgroup computes: the whole 96-row M-tile, or (BME = 48) one half of it, so that the MXFP8
// weights' doubled registers fit beside the accumulators.  The activation tile arrives in BME / 8
// load instructions of 8 rows x 128 B; wavefront w issues instructions w, w + 4, w + 8.
template <int BME> constexpr int kMxLoadInst = BME / 8;
template <int BME> constexpr int kMxLoadsPerWave = (BME / 8 + kMxWaves - 1) / kMxWaves;
static_assert(64 * 16 == 8 * kMxRowBytes, "one load instruction fills 8 rows");

// LDS tile: row r holds its 128 fp8 values as 8 chunks of 16 B, chunk c in slot c ^ ((r >> 1) & 7):
// the 16 lanes that read one chunk of 16 consecutive rows (two rows per 256-byte bank line) hit 16
// different bank groups.
__device__ __forceinline__ int mx_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

struct MxArgs {
  const uint8_t* a_r;       // fp8 rows: gate+up -> x8 [T][d] (gathered); down -> h8_r [P][I] (sorted rows)
  const uint8_t* a_s;       // shared group: gate+up -> x8; down -> h8_s [T][Is]
  const float* as_r;        // fp32 row scales of a_r rows: gate+up -> xs [T]; down -> hs_r [P]
  const float* as_s;        // ... of a_s rows: gate+up -> xs [T]; down -> hs_s [T]
  uint32_t a_r_bytes, a_s_bytes;
  const uint8_t* wr_codes;  // routed stack (w13 or w2): e2m1 or e4m3 codes in 16-row groups
  const uint8_t* wr_exp;    //   and the blocks' biased exponents
  const uint8_t* ws_codes;  // shared expert
  const uint8_t* ws_exp;
  _Float16* h_r;            // gate+up outputs, natural column order
  _Float16* h_s;
  _Float16* y_r;            // down outputs
  _Float16* y_s;
  const int* counts;
  const int* offsets;
  const int* sorted_pair;
  const int* group_order;
  const int* mt_prefix;
  int T, d, E, k, I, Is;
  int nbands;
  int order;
};

__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Weight element formats (the MFMA's operand format codes): e2m1 (MXFP4) or e4m3 (MXFP8).
constexpr int kFmtFp4 = 4;
constexpr int kFmtFp8 = 0;
// Per weight format: bytes of one 32-element block, and the 16-byte loads a lane makes per slice and step.
template <int WF> constexpr int kBlockBytes = WF == kFmtFp4 ? 16 : 32;
template <int WF> constexpr int kWLoads = WF == kFmtFp4 ? 1 : 2;

template <bool GATEUP, int WF, int BME, int NS, int NMT>
__device__ __forceinline__ void mx_tile(const MxArgs& a, char* As0, char* As1, char* As2, char* Aout,
                                        const __amdgpu_buffer_rsrc_t& rq,
                                        const __amdgpu_buffer_rsrc_t& rs, const __amdgpu_buffer_rsrc_t& ra,
                                        const uint32_t (&aoff)[kMxLoadsPerWave<BME>], const int (&qns)[4],
                                        const int (&sns)[4], const bool (&nok)[4], int nit, int c0, int wave,
                                        int lane, int mlen, int rbase, int m0, int Iw, bool shared) {
  const int n = lane & 15, G = lane >> 4;
  // The ring's stages are separate LDS objects (stage numbers are compile-time constants below), so the
  // compiler can tell that reading one stage does not depend on the loads still filling the other and
  // puts no wait for them in front of the reads.
  auto ring = [&](int buf) __attribute__((always_inline)) { return buf == 0 ? As0 : buf == 1 ? As1 : As2; };
  auto issue_a = [&](int it, int buf) {
#pragma unroll
    for (int i = 0; i < kMxLoadsPerWave<BME>; ++i) {
      const int inst = wave + kMxWaves * i;  // uniform
      if (inst < kMxLoadInst<BME>)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(ring(buf) + 8 * inst * kMxRowBytes), 16,
                                                 (int)aoff[i], it * kMxBK, 0, 0);
    }
  };
  // This lane's weights of every slice, from the step's 4 blocks of 16 rows (4 KiB-aligned runs of
  // 4 x 16 x kBlockBytes bytes), and the exponent byte of block G of row n.  MXFP4: lane (n, G) takes
  // the 16 bytes of block G of row n (its 32 values in order).  MXFP8: lane (n, G) takes values
  // 16G .. 16G+15 and 64 + 16G .. 64 + 16G + 15 of the 128 (the MFMA's fp8 operand layout): half G % 2
  // of blocks G / 2 and 2 + G / 2.
  constexpr int BB = kBlockBytes<WF>, NW = kWLoads<WF>;
  const int wo0 = WF == kFmtFp4 ? 16 * lane : (G >> 1) * 16 * BB + n * BB + 16 * (G & 1);
  auto load_w = [&](int it, u32x4 (*qd)[NW], uint32_t* sd) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
#pragma unroll
      for (int h = 0; h < NW; ++h)
        qd[ns][h] = __builtin_amdgcn_raw_buffer_load_b128(rq, wo0 + h * 2 * 16 * BB, qns[ns] + it * 64 * BB, 0);
      sd[ns] = __builtin_amdgcn_raw_buffer_load_b8(rs, lane, sns[ns] + it * 64, 0);
    }
  };

  floatx4 acc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[mt][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the fp8 operand of slice mt: chunks G and 4 + G of activation row 16 mt + n
  const int sw = (n >> 1) & 7;
  const uint32_t off0 = (uint32_t)(n * kMxRowBytes + 16 * (G ^ sw)), off1 = (uint32_t)(n * kMxRowBytes + 16 * ((4 + G) ^ sw));
  auto aread = [&](const char* At, int mt) __attribute__((always_inline)) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(At + mt * 16 * kMxRowBytes + off0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(At + mt * 16 * kMxRowBytes + off1);
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto compute = [&](int buf, const u32x4 (*q)[NW], const uint32_t* sc) __attribute__((always_inline)) {
    const char* At = ring(buf);
    v8i w[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const u32x4 lo = q[ns][0], hi = NW > 1 ? q[ns][NW - 1] : u32x4{0u, 0u, 0u, 0u};
      w[ns] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    v8i x0 = aread(At, 0);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      v8i x1;
      if (mt + 1 < NMT) x1 = aread(At, mt + 1);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
        // weights (format WF) as the A operand with their block exponent; activations (e4m3, format 0)
        // as the B operand with exponent 127 (scale 1)
        acc[mt][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[ns], x0, acc[mt][ns], WF, kFmtFp8, 0,
                                                                         (int)sc[ns], 0, 127);
      if (mt + 1 < NMT) x0 = x1;
    }
  };

  // NS-stage pipeline (2 or 3): while step `it` is computed, the activation tiles (LDS) and weight
  // blocks (registers) of the next NS - 1 steps are in flight.  A step's loads are nA tile loads (this
  // wavefront's share) and NWL weight loads, so with three stages the wait before step `it` leaves the
  // next step's nA + NWL in flight.
  static_assert(NS == 2 || NS == 3, "two or three stages");
  u32x4 q[NS][4][NW];
  uint32_t sc[NS][4];
  constexpr int NI = kMxLoadInst<BME>;
  const int nA = (NI % kMxWaves == 0 || wave < NI % kMxWaves) ? (NI + kMxWaves - 1) / kMxWaves : NI / kMxWaves;
  constexpr int NWL = 4 * NW + 4;
  issue_a(0, 0);
  load_w(0, q[0], sc[0]);
  if (NS == 3 && 1 < nit) {
    issue_a(1, 1);
    load_w(1, q[1 % NS], sc[1 % NS]);
  }
  auto step = [&](int it, auto st_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    constexpr int nx = (st + NS - 1) % NS;  // stage of step it + NS - 1
    if (NS == 3 && it + 1 < nit) {
      if (nA == 3) vm_lgkm_wait<3 + NWL>();
      else if (nA == 2) vm_lgkm_wait<2 + NWL>();
      else vm_lgkm_wait<1 + NWL>();
    } else {
      vm_lgkm_wait<0>();
    }
    tile_barrier();  // every wavefront's part of tile `it` is in LDS; the stage refilled below was last
                     // read by step it - 1
    if (it + NS - 1 < nit) {
      issue_a(it + NS - 1, nx);
      load_w(it + NS - 1, q[nx], sc[nx]);
    }
    compute(st, q[st], sc[st]);
  };
  int it0 = 0;
  for (; it0 + NS <= nit; it0 += NS) {
    step(it0 + 0, std::integral_constant<int, 0>{});
    step(it0 + 1, std::integral_constant<int, 1>{});
    if constexpr (NS == 3) step(it0 + 2, std::integral_constant<int, 2 % NS>{});
  }
  if (it0 < nit) step(it0, std::integral_constant<int, 0>{});
  if (NS == 3 && it0 + 1 < nit) step(it0 + 1, std::integral_constant<int, 1>{});

  // ---- epilogue: lane (n, G) holds, for activation row 16 mt + n, output columns 4G .. 4G+3 of each
  // 16-column slice; the row's activation scale multiplies them.
  const float* rsc = shared ? a.as_s : a.as_r;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int row = mt * 16 + n;
    const bool live = row < mlen;
    const int rr = live ? row : 0;
    float s;
    if (GATEUP)
      s = shared ? rsc[m0 + rr] : rsc[a.sorted_pair[rbase + rr] / a.k];  // the token's x scale
    else
      s = rsc[rbase + rr];  // the h row's scale (token row for the shared group)
    if (GATEUP) {
      _Float16* out = shared ? a.h_s : a.h_r;
#pragma unroll
      for (int xh = 0; xh < 2; ++xh) {
        // h columns c0 + 16 xh + 4G + i: SiLU(gate) * up, gate rows in slices 0, 1 and up rows in 2, 3
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = s * acc[mt][xh][i], uv = s * acc[mt][2 + xh][i];
          hv[i] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
        }
        const uint2 v = {__builtin_bit_cast(uint32_t, half2v{to_f16_sat(hv[0]), to_f16_sat(hv[1])}),
                         __builtin_bit_cast(uint32_t, half2v{to_f16_sat(hv[2]), to_f16_sat(hv[3])})};
        const int col = c0 + 16 * xh + 4 * G;
        if (live && nok[xh]) *reinterpret_cast<uint2*>(out + (size_t)(rbase + row) * Iw + col) = v;
      }
    } else {
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) acc[mt][ns] *= s;
    }
  }
  if (!GATEUP) {
    // the down tile leaves through LDS so that every store writes whole rows; the staging region is
    // stage 0 of the ring, enlarged (every wavefront is done reading its last tile first; no load into it
    // is in flight after the last step's wait)
    tile_barrier();
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 16 + n;
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const half2v p0 = {to_f16_sat(acc[mt][ns][0]), to_f16_sat(acc[mt][ns][1])};
        const half2v p1 = {to_f16_sat(acc[mt][ns][2]), to_f16_sat(acc[mt][ns][3])};
        const int chunk = 8 * wave + 2 * ns + (G >> 1);
        *reinterpret_cast<uint2*>(Aout + row * (kMxDownBandCols * 2) + ((chunk ^ (row & 31)) * 16) + 8 * (G & 1)) =
            uint2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
      }
    }
    vm_lgkm_wait<0>();
    tile_barrier();
    constexpr int C = kMxDownBandCols / 8, R = kMxThreads / C;
    static_assert(R * C == kMxThreads && 16 % R == 0, "whole rows per pass");
    _Float16* out = shared ? a.y_s : a.y_r;
    const int tid = (int)threadIdx.x, chunk = tid % C;
    const int col = c0 - 64 * wave + 8 * chunk;
#pragma unroll
    for (int i = 0; i < 16 * NMT / R; ++i) {
      const int row = R * i + tid / C;
      const u32x4 v = *reinterpret_cast<const u32x4*>(Aout + row * (kMxDownBandCols * 2) + ((chunk ^ (row & 31)) * 16));
      if (row < mlen && col < a.d) *reinterpret_cast<u32x4*>(out + (size_t)(rbase + row) * a.d + col) = v;
    }
  }
}

template <bool GATEUP, int WF>
__global__ __launch_bounds__(kMxThreads, 8 / kMxWaves) void k_grouped_mx(MxArgs a) {
  // MXFP8 weights: every M-tile is two work items of 48 rows (launch indices b and b + 8 of the same
  // XCD, adjacent in time, so the second reads the weight band from L2)
  constexpr bool HALF = WF == kFmtFp8;
  constexpr int BME = HALF ? kMxBM / 2 : kMxBM;
  // three pipeline stages (measured against two: MXFP8 gate+up -8%, down -3%, MXFP4 gate+up -1%); the
  // down projection's output staging reuses stage 0, so that two workgroups per CU still fit
  constexpr int NS = 3;
  constexpr int BANDW = GATEUP ? kMxGateUpBandCols : kMxDownBandCols;
  constexpr int kStage = BME * kMxRowBytes, kOut = GATEUP ? 0 : BME * kMxDownBandCols * 2;
  __shared__ __attribute__((aligned(1024))) char As0[kStage > kOut ? kStage : kOut];
  __shared__ __attribute__((aligned(1024))) char As1[kStage];
  __shared__ __attribute__((aligned(1024))) char As2[kStage];
  char* const Aout = As0;
  __shared__ int s_prefix[kMaxExperts + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = ufl(tid >> 6);
  const int ngroups = a.E + 1;
  for (int i = tid; i <= ngroups; i += kMxThreads) s_prefix[i] = a.mt_prefix[i];
  __syncthreads();
  const int nb = a.nbands;
  const int n_mt = ufl(s_prefix[ngroups]);
  const int bx = blockIdx.x;
  const int hsel = HALF ? (bx >> 3) & 1 : 0;
  // work item -> (group rank, band, M-tile), as on the W4A16 path
  int rank, band, mtile;
  {
    const int bid = HALF ? (((bx >> 4) << 3) | (bx & 7)) : bx;
    const int order = (a.order == 1 && nb % 8 != 0) ? 2 : a.order;
    const int nbx = order == 1 ? nb / 8 : nb;
    int item;
    if (order == 0) {
      const int sl = bid >> 3;
      item = (((sl >> 3) << 3) + (bid & 7)) * 8 + (sl & 7);
    } else {
      item = order == 1 ? bid >> 3 : bid;
    }
    if (item >= n_mt * nbx) return;
    int lo = 0, hi = ngroups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ufl(s_prefix[mid]) * nbx <= item) lo = mid; else hi = mid;
    }
    rank = lo;
    const int p0 = ufl(s_prefix[rank]);
    const int nmt = ufl(s_prefix[rank + 1]) - p0;
    const int local = item - p0 * nbx;
    if (order == 1) {
      band = 8 * (local / nmt) + (bid & 7);
      mtile = local % nmt;
    } else if (order == 0 && GATEUP) {
      // gate+up: a group's M-tiles of one band adjacent (same run of 8 items, same XCD), so a
      // multi-tile group streams each weight band from HBM about once; the activation rows, 8 MB of fp8
      // in all, are the ones read again (measured: gate+up -1% at T=2048, -4% at T=8192; the down
      // projection, whose h rows are 2.5x x's bytes, is faster M-tile-major)
      mtile = local % nmt;
      band = local / nmt;
    } else {
      mtile = local / nbx;
      band = local % nbx;
    }
  }
  const int g = ufl(a.group_order[rank]);
  const bool shared = (g == a.E);
  const int cnt = shared ? a.T : ufl(a.counts[g]);
  const int Iw = shared ? a.Is : a.I;
  const int Kdim = GATEUP ? a.d : Iw;
  const int Ndim = GATEUP ? Iw : a.d;
  if (band * BANDW >= Ndim) return;
  const int m0 = mtile * kMxBM + hsel * BME;
  if (cnt - m0 <= 0) return;  // the lower half of a tile with at most 48 rows
  const int mlen = min(BME, cnt - m0);
  const int gbase = shared ? 0 : ufl(a.offsets[g]);
  const int rbase = gbase + m0;
  const uint32_t wrows = GATEUP ? 2u * (uint32_t)Iw : (uint32_t)a.d;
  const uint32_t qstride = (uint32_t)Kdim / 32 * kBlockBytes<WF>, nkb = (uint32_t)Kdim / 32;
  const uint8_t* Wq = shared ? a.ws_codes : a.wr_codes + (size_t)g * wrows * qstride;
  const uint8_t* We = shared ? a.ws_exp : a.wr_exp + (size_t)g * wrows * nkb;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Wq, wrows * qstride);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(We, wrows * nkb);
  const __amdgpu_buffer_rsrc_t ra = shared ? make_rsrc(a.a_s, a.a_s_bytes) : make_rsrc(a.a_r, a.a_r_bytes);

  // activation rows staged by this wavefront: rows 8 inst + lane/8 of its load instructions inst =
  // wave + 4i, slot lane%8
  uint32_t aoff[kMxLoadsPerWave<BME>];
#pragma unroll
  for (int i = 0; i < kMxLoadsPerWave<BME>; ++i) {
    const int row = 8 * (wave + kMxWaves * i) + (lane >> 3);
    const int rr = row < mlen ? row : 0;
    uint32_t arow;
    if (GATEUP)
      arow = shared ? (uint32_t)(m0 + rr) : (uint32_t)(a.sorted_pair[rbase + rr] / a.k);
    else
      arow = (uint32_t)(rbase + rr);
    // the chunk that belongs in slot lane % 8 of this row; rows past the group read nothing (zeros)
    const int chunk = mx_slot(row, lane & 7);
    aoff[i] = row < mlen ? arow * (uint32_t)Kdim + 16u * (uint32_t)chunk : kMxOffsetOOB;
  }
  const int nit = Kdim / kMxBK;
  // this wavefront's weight rows: four 16-row slices (gate+up: gate columns c0.., c0+16.., then the
  // matching up rows; down: output columns c0 + 16 ns)
  int rowbase[4];
  bool nok[4];
  int c0;
  if (GATEUP) {
    c0 = band * BANDW + wave * 32;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = c0 + 16 * (ns & 1);
      nok[ns] = col < Iw;
      rowbase[ns] = (ns < 2 ? 0 : Iw) + (nok[ns] ? col : 0);
    }
  } else {
    c0 = band * BANDW + wave * 64;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = c0 + 16 * ns;
      nok[ns] = col < a.d;
      rowbase[ns] = nok[ns] ? col : 0;
    }
  }
  // codes [rows/16][K/32][16][block bytes] and exponents [rows/16][K/32][16]: slice ns's iteration
  // `it` is 64 blocks' worth of codes from ((rowbase/16)*(K/32) + 4 it)*16 blocks and 64 exponent bytes
  // from ((rowbase/16)*(K/32) + 4 it)*16; lane l takes exponent byte l
  int qns[4], sns[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    qns[ns] = ufl((int)((uint32_t)(rowbase[ns] / 16) * nkb * 16u * (uint32_t)kBlockBytes<WF>));
    sns[ns] = ufl((int)((uint32_t)(rowbase[ns] / 16) * nkb * 16u));
  }
#define MX_TILE(NMT)                                                                                      \
  mx_tile<GATEUP, WF, BME, NS, NMT>(a, As0, As1, As2, Aout, rq, rs, ra, aoff, qns, sns, nok, nit, c0, wave, lane, mlen, \
                                rbase, m0, Iw, shared)
  const int nmt16 = (mlen + 15) >> 4;
  if constexpr (BME == 48) {
    if (nmt16 == 1) MX_TILE(1);
    else if (nmt16 == 2) MX_TILE(2);
    else MX_TILE(3);
  } else {
    switch (nmt16) {
      case 1: MX_TILE(1); break;
      case 2: MX_TILE(2); break;
      case 3: MX_TILE(3); break;
      case 4: MX_TILE(4); break;
      case 5: MX_TILE(5); break;
      default: MX_TILE(6); break;
    }
  }
#undef MX_TILE
}

// ---------------------------------------------------------------------------- row quantisation
// e4m3 code of a finite fp32 value: nearest e4m3 value, ties to the even mantissa, saturating at
// +-448; the sign bit is kept for values that round to zero.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float a = fabsf(v);
  uint32_t c;
  if (!(a < 448.f)) {
    c = 0x7E;
  } else if (a < 0.015625f) {                  // subnormal range: steps of 2^-9
    c = (uint32_t)rintf(a * 512.f);            // 0 .. 8 (8 is the smallest normal, code 0x08)
  } else {
    int ex;
    (void)frexpf(a, &ex);                      // a = m * 2^ex, m in [0.5, 1): exponent e = ex - 1
    const int e = ex - 1;
    const uint32_t r = (uint32_t)rintf(ldexpf(a, 3 - e));  // 8 .. 16 (16 carries into the next exponent)
    c = (uint32_t)(8 * e + 48) + r;
    c = c > 0x7Eu ? 0x7Eu : c;
  }
  return c | (__builtin_signbit(v) ? 0x80u : 0u);
}

// ---------------------------------------------------------------------------- requantisation
// One Q4 block (16 code bytes, fp16 scale) -> 16 bytes of e2m1 codes and the biased shared
// exponent: values w = (q - 8) * d (exact in fp32), E = floor(log2 max|w|) - 2 (E = -127 for an
// all-zero block), codes = w / 2^E rounded to the nearest e2m1 value, ties to the even mantissa,
// saturating at +-6.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | (__builtin_signbit(v) ? 8u : 0u);
}

// WF = fp8 (MXFP8): E = floor(log2 max|w|) - 8, 32 e4m3 codes (value j at byte j), saturating at +-448.
template <int WF>
__global__ __launch_bounds__(256) void k_q4_to_mx(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ sc,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ exps,
                                                  size_t nblocks) {
  constexpr int emax = WF == kFmtFp4 ? 2 : 8;  // largest exponent of the element format
  for (size_t b = (size_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += (size_t)gridDim.x * 256) {
    const u32x4 v = ld16(qs + 16 * b);
    const float d = (float)__builtin_bit_cast(_Float16, sc[b]);
    int qmax = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = (int)((v[w] >> (4 * j)) & 0xF) - 8;
        qmax = max(qmax, q < 0 ? -q : q);
      }
    const float amax = (float)qmax * fabsf(d);
    int e = -127;
    if (amax > 0.f) {
      int ex;
      (void)frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
      e = min(max(ex - 1 - emax, -127), 127);
    }
    if constexpr (WF == kFmtFp4) {
      u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int q = (int)((v[w] >> (4 * j)) & 0xF) - 8;
          const float val = ldexpf((float)q * d, -e);  // exact: a power-of-two scaling of an exact product
          o |= e2m1_code(val) << (4 * j);
        }
        out[w] = o;
      }
      *reinterpret_cast<u32x4*>(codes + 16 * b) = out;
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int q = (int)((v[2 * half + w] >> (4 * j)) & 0xF) - 8;
            const float val = ldexpf((float)q * d, -e);
            out[2 * w + j / 4] |= e4m3_code(val) << (8 * (j % 4));
          }
        *reinterpret_cast<u32x4*>(codes + 32 * b + 16 * half) = out;
      }
    }
    exps[b] = (uint8_t)(e + 127);
  }
}

// One workgroup per row (any K % 4 == 0): s = amax / 448 (1 for an all-zero row), codes = e4m3(x / s), both
// divisions correctly rounded in fp32.  IN_F16: the input row is fp16 (h), else bf16 (x).  NIT > 0: the
// row fits in NIT groups of 4 values per thread (K <= 1024 NIT) and is read once, kept in registers;
// NIT = 0: any K, the row read twice.
template <bool IN_F16, int NIT>
__global__ __launch_bounds__(256) void k_rows_fp8(const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                                                  float* __restrict__ scale, int K) {
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* src = in + (size_t)r * K;
  auto val = [&](uint16_t b) { return IN_F16 ? (float)__builtin_bit_cast(_Float16, b) : bf16_bits_to_float(b); };
  auto amax4 = [&](uint2 u) {
    return fmaxf(fmaxf(fabsf(val((uint16_t)(u.x & 0xFFFF))), fabsf(val((uint16_t)(u.x >> 16)))),
                 fmaxf(fabsf(val((uint16_t)(u.y & 0xFFFF))), fabsf(val((uint16_t)(u.y >> 16)))));
  };
  constexpr int NR = NIT > 0 ? NIT : 1;
  uint2 keep[NR];
  float m = 0.f;
  if constexpr (NIT > 0) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int i = 4 * tid + 1024 * j;
      keep[j] = i < K ? *reinterpret_cast<const uint2*>(src + i) : uint2{0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NIT; ++j) m = fmaxf(m, amax4(keep[j]));
  } else {
    for (int i = 4 * tid; i < K; i += 4 * 256) m = fmaxf(m, amax4(*reinterpret_cast<const uint2*>(src + i)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  if (tid == 0) scale[r] = s;
  auto store = [&](int i, uint2 u) {
    const uint32_t c0 = e4m3_code(__fdiv_rn(val((uint16_t)(u.x & 0xFFFF)), s));
    const uint32_t c1 = e4m3_code(__fdiv_rn(val((uint16_t)(u.x >> 16)), s));
    const uint32_t c2 = e4m3_code(__fdiv_rn(val((uint16_t)(u.y & 0xFFFF)), s));
    const uint32_t c3 = e4m3_code(__fdiv_rn(val((uint16_t)(u.y >> 16)), s));
    *reinterpret_cast<uint32_t*>(out + (size_t)r * K + i) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  };
  if constexpr (NIT > 0) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int i = 4 * tid + 1024 * j;
      if (i < K) store(i, keep[j]);
    }
  } else {
    for (int i = 4 * tid; i < K; i += 4 * 256) store(i, *reinterpret_cast<const uint2*>(src + i));
  }
}

// One wavefront per row, the row held in registers (a single pass over it): lane l takes the 16-byte
// chunks l, l + 64, ... (8 values each, coalesced), the row's amax is a wavefront reduction, and the
// codes leave as 8 bytes per chunk.  The same arithmetic as k_rows_fp8, for K % 8 == 0 and
// K <= 512 * NCH (short rows, where a workgroup per row would leave most lanes idle).  One launch can
// take two matrices: rows * K, then rows2 * K2 (the routed and the shared h).
template <bool IN_F16, int NCH>
__global__ __launch_bounds__(256) void k_rows_fp8_wave(const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                                                       float* __restrict__ scale, int rows, int K,
                                                       const uint16_t* __restrict__ in2, uint8_t* __restrict__ out2,
                                                       float* __restrict__ scale2, int rows2, int K2) {
  const int lane = threadIdx.x & 63;
  int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  // rows past the first matrix's belong to the second (rows2 = 0: none); the choice is per wavefront
  if (r >= rows) {
    r -= rows;
    if (r >= rows2) return;  // whole wavefronts
    in = in2;
    out = out2;
    scale = scale2;
    K = K2;
  }
  const uint16_t* src = in + (size_t)r * K;
  const int nch = K / 8;
  auto val = [&](uint32_t b) { return IN_F16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)b) : bf16_bits_to_float(b); };
  u32x4 v[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nch ? ld16(src + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, fmaxf(fabsf(val(v[i][w] & 0xFFFF)), fabsf(val(v[i][w] >> 16))));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float s = m > 0.f ? __fdiv_rn(m, 448.f) : 1.f;
  if (lane == 0) scale[r] = s;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      uint32_t o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t a = v[i][2 * h], b = v[i][2 * h + 1];
        o[h] = e4m3_code(__fdiv_rn(val(a & 0xFFFF), s)) | (e4m3_code(__fdiv_rn(val(a >> 16), s)) << 8) |
               (e4m3_code(__fdiv_rn(val(b & 0xFFFF), s)) << 16) | (e4m3_code(__fdiv_rn(val(b >> 16), s)) << 24);
      }
      *reinterpret_cast<uint2*>(out + (size_t)r * K + 8 * c) = uint2{o[0], o[1]};
    }
  }
}

}  // namespace

hipError_t launch_q4_to_mx(size_t nblocks, const uint8_t* qs, const uint16_t* sc, uint8_t* codes, uint8_t* exps,
                           bool fp8, hipStream_t st) {
  if (nblocks == 0) return hipSuccess;
  const size_t want = (nblocks + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  if (fp8) hipLaunchKernelGGL(k_q4_to_mx<kFmtFp8>, dim3(grid), dim3(256), 0, st, qs, sc, codes, exps, nblocks);
  else hipLaunchKernelGGL(k_q4_to_mx<kFmtFp4>, dim3(grid), dim3(256), 0, st, qs, sc, codes, exps, nblocks);
  return hipGetLastError();
}

hipError_t launch_rows_fp8(const uint16_t* in, bool in_f16, int rows, int K, uint8_t* out, float* scale,
                           hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  // short rows (K <= 1024, K % 8 == 0): one wavefront per row, the row in registers; longer ones: one
  // workgroup per row, the row in registers up to K = 8192 (one read), else read twice
  if (K % 8 == 0 && K <= 1024) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (in_f16)
      hipLaunchKernelGGL((k_rows_fp8_wave<true, 2>), grid, dim3(256), 0, st, in, out, scale, rows, K, nullptr,
                         nullptr, nullptr, 0, 0);
    else
      hipLaunchKernelGGL((k_rows_fp8_wave<false, 2>), grid, dim3(256), 0, st, in, out, scale, rows, K, nullptr,
                         nullptr, nullptr, 0, 0);
    return hipGetLastError();
  }
  const int nit = (K + 1023) / 1024;
#define MOE_ROWS_BLOCK(N)                                                                               \
  if (in_f16) hipLaunchKernelGGL((k_rows_fp8<true, N>), dim3(rows), dim3(256), 0, st, in, out, scale, K); \
  else hipLaunchKernelGGL((k_rows_fp8<false, N>), dim3(rows), dim3(256), 0, st, in, out, scale, K);
  if (nit <= 2) { MOE_ROWS_BLOCK(2) }
  else if (nit <= 4) { MOE_ROWS_BLOCK(4) }
  else if (nit <= 8) { MOE_ROWS_BLOCK(8) }
  else { MOE_ROWS_BLOCK(0) }
#undef MOE_ROWS_BLOCK
  return hipGetLastError();
}

hipError_t launch_w4a8_forward(const Shape& s, const uint16_t* x, const Routing& r, const MxWeights& w,
                               const W4A8Scratch& o, const float* topk_w, float* y, uint32_t flags, bool fp8,
                               hipStream_t st) {
  const int P = s.T * s.k;
  hipError_t e = launch_rows_fp8(x, false, s.T, s.d, o.x8, o.xs, st);
  if (e != hipSuccess) return e;
  MxArgs a{};
  a.counts = r.counts;
  a.offsets = r.offsets;
  a.sorted_pair = r.sorted_pair;
  a.group_order = r.group_order;
  a.mt_prefix = r.mt_prefix;
  a.T = s.T; a.d = s.d; a.E = s.E; a.k = s.k; a.I = s.I; a.Is = s.Is;
  a.order = (flags & MOE_FLAG_NO_BANDING) ? 2 : (flags & MOE_FLAG_BAND_MAJOR) ? 1 : 0;
  const long mtiles = grouped_max_mtiles(s);
  // gate+up
  a.a_r = o.x8; a.a_s = o.x8; a.as_r = o.xs; a.as_s = o.xs;
  a.a_r_bytes = a.a_s_bytes = (uint32_t)((size_t)s.T * s.d);
  a.wr_codes = w.w13_codes; a.wr_exp = w.w13_exp; a.ws_codes = w.s13_codes; a.ws_exp = w.s13_exp;
  a.h_r = o.h_r; a.h_s = o.h_s;
  const int Imax = s.I > s.Is ? s.I : s.Is;
  a.nbands = (Imax + kMxGateUpBandCols - 1) / kMxGateUpBandCols;
  long grid = (mtiles * a.nbands + 63) / 64 * 64;  // MXFP8: two half-tile items per launch-order item
  if (fp8) hipLaunchKernelGGL((k_grouped_mx<true, kFmtFp8>), dim3((unsigned)(2 * grid)), dim3(kMxThreads), 0, st, a);
  else hipLaunchKernelGGL((k_grouped_mx<true, kFmtFp4>), dim3((unsigned)grid), dim3(kMxThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // h rows to fp8 (routed rows by sorted position, then the shared expert's token rows): one launch of
  // the wavefront-per-row kernel for both when their rows are short enough, else one launch each
  const uint16_t* hr = reinterpret_cast<const uint16_t*>(o.h_r);
  const uint16_t* hs = reinterpret_cast<const uint16_t*>(o.h_s);
  if (s.I <= 1024 && s.Is <= 1024) {  // multiples of 128 (checked on the host)
    hipLaunchKernelGGL((k_rows_fp8_wave<true, 2>), dim3((unsigned)((P + s.T + 3) / 4)), dim3(256), 0, st, hr, o.h8_r,
                       o.hs_r, P, s.I, hs, o.h8_s, o.hs_s, s.T, s.Is);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    if ((e = launch_rows_fp8(hr, true, P, s.I, o.h8_r, o.hs_r, st)) != hipSuccess) return e;
    if ((e = launch_rows_fp8(hs, true, s.T, s.Is, o.h8_s, o.hs_s, st)) != hipSuccess) return e;
  }
  // down
  a.a_r = o.h8_r; a.a_s = o.h8_s; a.as_r = o.hs_r; a.as_s = o.hs_s;
  a.a_r_bytes = (uint32_t)((size_t)P * s.I);
  a.a_s_bytes = (uint32_t)((size_t)s.T * s.Is);
  a.wr_codes = w.w2_codes; a.wr_exp = w.w2_exp; a.ws_codes = w.s2_codes; a.ws_exp = w.s2_exp;
  a.y_r = o.y_pair; a.y_s = o.y_s;
  a.nbands = (s.d + kMxDownBandCols - 1) / kMxDownBandCols;
  grid = (mtiles * a.nbands + 63) / 64 * 64;
  if (fp8) hipLaunchKernelGGL((k_grouped_mx<false, kFmtFp8>), dim3((unsigned)(2 * grid)), dim3(kMxThreads), 0, st, a);
  else hipLaunchKernelGGL((k_grouped_mx<false, kFmtFp4>), dim3((unsigned)grid), dim3(kMxThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GroupedOut go{};
  go.y_pair = o.y_pair;
  go.y_s = o.y_s;
  return launch_combine(s, topk_w, r, go, nullptr, y, nullptr, st);
}

}  // namespace moe
