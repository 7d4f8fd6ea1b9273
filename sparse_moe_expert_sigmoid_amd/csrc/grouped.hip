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
// schedule order, its M-tiles of up to 96 rows times the N-bands of the
// output, M-tile-major by default (the bands of one M-tile adjacent; runs of
// 8 items per XCD so that the workgroups sharing an activation tile share an
// L2), or band-major (all M-tiles of one weight band on one XCD) on request.
// The grid is sized for the
// largest possible tile count; surplus workgroups exit at once, so the launch
// shape does not depend on device data and the call can be graph-captured.
//
// Inner loop (per 128-wide K step): the workgroup stages its 96 activation
// rows x 128 columns as fp16 in LDS (double-buffered); each wavefront owns
// four 16-column weight slices, loads one 16-byte Q4 block per slice and
// lane, dequantises it in registers straight into the B-operand layout of
// v_mfma_f32_16x16x32_f16 (as weight / 16, undone in the epilogue) and
// multiplies it against every 16-row slice of the activation tile, whose
// fragments are read from LDS two slices ahead.  K is permuted consistently: MFMA k-lane group G of
// step s holds elements 32G + 8s .. 32G + 8s + 7 of the 128-wide chunk, which
// are exactly dword s of Q4 block G.
#include <type_traits>

#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_q4.h"

namespace moe {

// LDS tile: 96 rows x 128 halves (256 B) per buffer, no padding.  The 16 B
// chunk c of row r is stored in slot c ^ (r & 15), so the 16 lanes that read
// one MFMA operand (16 rows, same chunk) hit 16 different slots, i.e. all 64
// banks once.  Tiles arrive by buffer_load_dwordx4 ... lds: one instruction
// moves 64 x 16 B into 1 KB of consecutive LDS (4 rows), lane l filling slot
// l%16 of row l/16, so the swizzle is applied on the global offset side.
//
// All global loads are buffer loads whose per-lane offset is fixed for the
// whole K loop; the K advance is a scalar offset, so the main loop spends
// its vector instructions on dequantisation, not on address arithmetic.
constexpr int kRowBytes = kGroupedBK * 2;
constexpr int kTileBytes = kGroupedBM * kRowBytes;  // 24 KB
constexpr int kStages = 2;        // pipeline depth (LDS ring of kStages activation tiles)
constexpr int kGroupedThreads = 64 * kGroupedWaves;
constexpr int kTileLoads = kTileBytes / (kGroupedThreads * 16);  // buffer_load ... lds per lane per tile
constexpr int kLoadsPerStep = kTileLoads + 8;        // vector-memory ops per lane per K step (+4 code blocks, 4 scales)
constexpr int kRowsPerWave = kGroupedBM / kGroupedWaves;  // activation rows staged by each wavefront
// A buffer offset past every buffer this path addresses (all are below 2^32 - 64 bytes): buffer
// loads at it return zeros without a memory access.  The range check uses the per-lane offset
// only, so it holds whatever scalar offset the K loop adds.
constexpr uint32_t kOffsetOOB = 0xFFFFFFF0u;

struct GArgs {
  const _Float16* a_r;      // A rows: gate+up -> x16 [T][d] (gathered); down -> h_r [P][I] (sorted rows)
  const _Float16* a_s;      // A rows of the shared group: gate+up -> x16; down -> h_s [T][Is]
  uint32_t a_r_bytes, a_s_bytes;
  Q4 wr;                    // routed stack (w13 or w2)
  Q4 ws;                    // shared expert (s13 or s2)
  _Float16* h_r;            // gate+up outputs (element order permuted in groups of 8)
  _Float16* h_s;
  _Float16* y_r;            // down outputs (fp16)
  _Float16* y_s;
  const int* counts;
  const int* offsets;
  const int* sorted_pair;
  const int* group_order;
  const int* mt_prefix;
  int T, d, E, k, I, Is;
  int nbands;
  int order;                // work-item order (see k_grouped)
  uint32_t flags;
  uint32_t dq_mask, dq_magic;
};


__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Per-tile state handed from the work-item decode to the main loop.
struct TileCtx {
  __amdgpu_buffer_rsrc_t rq, rs, ra;
  uint32_t aoff[kTileLoads];
  uint32_t qoff, soff;         // per-lane part of the weight offsets (row n, block G)
  uint32_t qoff_tail, soff_tail;  // the same, block clamped to the row's last, for the K tail iteration
  int qns[4], sns[4];          // per-slice part (uniform): slice ns's first code row, first scale group
  uint32_t rdo;                // LDS read offset of row n (chunk swizzle applied per K-step)
  int gx;                      // 4G ^ n: swizzled chunk of K-step s is gx ^ s
  bool nok[4];
  int c0, wave, nit, nkb, Kdim, Iw, mlen, rbase, G, n, lane;
  uint32_t dq_mask, dq_magic;  // 0x000F000F (uniform) and 0x64006400 (kept in a VGPR)
  bool ktail, shared;
};

// Main loop and epilogue of one tile with NMT active 16-row slices (known
// at compile time, so the K loop has no per-MFMA conditions).  Slices of the
// wavefront's four 16-column weight slices that lie past the N edge are
// computed on a valid row and discarded in the epilogue.
template <bool GATEUP, int NMT>
__device__ __forceinline__ void grouped_tile(const GArgs& a, const TileCtx& c, char* As) {
  constexpr int BK = kGroupedBK;
  auto issue_a = [&](int it, int buf) {
    const int kb = it * BK * 2;
    if (c.ktail && it == c.nit - 1) {  // uniform
#pragma unroll
      for (int i = 0; i < kTileLoads; ++i) {
        // a chunk past the row end re-reads the tile's first chunk of the same row: finite data
        // that meets zero weights (the weights' K tail is masked to zero below)
        const int chunk = (c.lane & 15) ^ ((kRowsPerWave * c.wave + 4 * i + (c.lane >> 4)) & 15);
        const uint32_t off = c.aoff[i] - (it * BK + 8 * chunk >= c.Kdim ? 16u * (uint32_t)chunk : 0u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            c.ra, (lds_void*)(As + buf * kTileBytes + (kRowsPerWave * c.wave + 4 * i) * kRowBytes), 16, (int)off, kb,
            0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTileLoads; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            c.ra, (lds_void*)(As + buf * kTileBytes + (kRowsPerWave * c.wave + 4 * i) * kRowBytes), 16,
            (int)c.aoff[i], kb, 0, 0);
    }
  };
  auto load_w = [&](int it, u32x4* qd, uint32_t* sd) {
    // in the K tail iteration, lanes whose block lies past the row end re-read the row's last block
    // (their scale is masked to zero): every access stays inside the weight matrix
    const bool tail = c.ktail && it == c.nit - 1;  // uniform
    const uint32_t qo = tail ? c.qoff_tail : c.qoff, so = tail ? c.soff_tail : c.soff;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      qd[ns] = __builtin_amdgcn_raw_buffer_load_b128(c.rq, (int)qo, c.qns[ns] + it * 1024, 0);
      sd[ns] = __builtin_amdgcn_raw_buffer_load_b16(c.rs, (int)so, c.sns[ns] + it * 128, 0);
    }
  };

  floatx4 acc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[mt][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One K iteration (4 MFMA K-steps of 32) on LDS buffer `buf`.  Within a K-step the activation
  // fragment of each 16-row slice is read from LDS just before its four MFMAs (one slice ahead), and
  // the four weight fragments of the next K-step are dequantised between the MFMAs.  The loop body has
  // no branches around the MFMAs, so the accumulators keep their registers across iterations.
  auto compute = [&](int buf, const u32x4* q, const half2v* d2, bool general) __attribute__((always_inline)) {
    const char* At = As + buf * kTileBytes;
    SmallScale ss[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) ss[ns] = small_scale(d2[ns]);
    // common form; redone in the general form when a scale of this iteration is outside its range
    // (`general` is uniform, so this is a scalar branch that is normally not taken)
    auto deq = [&](uint32_t w, int ns) __attribute__((always_inline)) {
      half8 r = dequant8_small(w, ss[ns]);
      if (__builtin_expect(general, 0)) r = dequant8_general(w, d2[ns], c.dq_mask, c.dq_magic);
      return r;
    };
    half8 b_cur[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) b_cur[ns] = deq(q[ns][0], ns);
    // activation fragments are read two 16-row slices ahead, across K-step boundaries
    constexpr int NI = 4 * NMT;
    auto aread = [&](int idx) __attribute__((always_inline)) {
      return *reinterpret_cast<const half8*>(At + c.rdo + 16 * (c.gx ^ (idx / NMT)) + (idx % NMT) * 16 * kRowBytes);
    };
    half8 a0 = aread(0), a1 = aread(NI > 1 ? 1 : 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 b_nxt[4];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int idx = s * NMT + mt;
        half8 a2;
        if (idx + 2 < NI) a2 = aread(idx + 2);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          // weights as the A operand: the tile comes out transposed (see the epilogue)
          acc[mt][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b_cur[ns], a0, acc[mt][ns], 0, 0, 0);
        if (s < 3 && mt < 4) b_nxt[mt] = deq(q[mt][s + 1], mt);
        a0 = a1;
        if (idx + 2 < NI) a1 = a2;
      }
      if (s < 3) {
#pragma unroll
        for (int ns = NMT; ns < 4; ++ns) b_nxt[ns] = deq(q[ns][s + 1], ns);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) b_cur[ns] = b_nxt[ns];
      }
    }
  };
  // Scales of iteration `it` (the K tail's blocks weigh zero), and whether any scale the wavefront uses
  // in this iteration is outside the range of the common dequantisation form.
  auto run_step = [&](int buf, const u32x4* q, const uint32_t* sc_in, int it) __attribute__((always_inline)) {
    half2v d2[4];
    const bool tail = c.ktail && it == c.nit - 1;  // uniform
    bool small = true;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      // the step's loads have landed: no register in flight is overwritten here
      const uint32_t bits = (tail && it * 4 + c.G >= c.nkb) ? 0u : sc_in[ns];
      small = small && small_scale_ok(bits);
      const _Float16 dv = __builtin_bit_cast(_Float16, (uint16_t)bits);
      d2[ns] = half2v{dv, dv};
    }
    compute(buf, q, d2, __builtin_amdgcn_ballot_w64(!small) != 0);
  };

  // kStages-deep pipeline: while step `it` is computed, the activation tiles and weight blocks of
  // steps it+1 .. it+kStages-1 are in flight (LDS ring of kStages tiles, weights in registers).
  constexpr int NS = kStages;
  u32x4 q[NS][4];
  uint32_t sc[NS][4];
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    if (st < c.nit) {
      issue_a(st, st);
      load_w(st, q[st], sc[st]);
    }
  }
  // Wait until step `it` has landed (younger steps stay in flight), then barrier.
  auto arrive = [&](int it) __attribute__((always_inline)) {
    const int younger = min(NS - 2, c.nit - 1 - it);
    static_assert(kStages <= 3, "the waits below cover up to two younger steps");
    if (younger >= 2) vm_lgkm_wait<2 * kLoadsPerStep>();
    else if (younger == 1) vm_lgkm_wait<kLoadsPerStep>();
    else vm_lgkm_wait<0>();
    tile_barrier();  // every wavefront's part of tile `it` is in LDS; tile it-1 is no longer read
  };
  // Main loop over whole groups of NS steps: the compute is unconditional (only the load issue and the
  // wait depth depend on the trip count), so the accumulators stay in their registers.
  int it0 = 0;
  for (; it0 + NS <= c.nit; it0 += NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int it = it0 + st;
      arrive(it);
      if (it + NS - 1 < c.nit) {
        const int nxt = (st + NS - 1) % NS;  // folded: st is an unrolled constant
        issue_a(it + NS - 1, nxt);
        load_w(it + NS - 1, q[nxt], sc[nxt]);
      }
      run_step(st, q[st], sc[st], it);
    }
  }
  // The remaining nit % NS steps (their loads were issued above or in the prologue).
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    const int it = it0 + st;
    if (it < c.nit) {
      arrive(it);
      run_step(st, q[st], sc[st], it);
    }
  }

  // ---- epilogue.  With the weights as the A operand, lane (n, G) holds, for activation row
  // mt*16 + n, the four consecutive output columns 4G .. 4G+3 of each 16-column slice, divided by 16
  // (the dequantised weights are weight / 16; the products and sums scale exactly).
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int row = mt * 16 + c.n;
    const bool live = row < c.mlen;
    if (GATEUP) {
      _Float16* out = c.shared ? a.h_s : a.h_r;
#pragma unroll
      for (int xh = 0; xh < 2; ++xh) {
        // h columns c0 + 16xh + 4G + i; SiLU(gate) * up with a fast exponential and reciprocal
        half2v h[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float hv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float gv = 16.f * acc[mt][xh][2 * j + e], uv = 16.f * acc[mt][2 + xh][2 * j + e];
            hv[e] = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
          }
          h[j] = half2v{to_f16_sat(hv[0]), to_f16_sat(hv[1])};
        }
        // h is stored in the dequant pair order inside each group of 8 columns (slot 2m holds column
        // m, slot 2m+1 column m+4): lanes G and G^1 (16 lanes apart) hold the two halves of a group.
        // The even lane writes slots 0..3 (its columns 0, 1 with the partner's 4, 5), the odd lane
        // slots 4..7 (the partner's 2, 3 with its own 6, 7).
        const bool odd = c.G & 1;
        const uint32_t give = __builtin_bit_cast(uint32_t, odd ? h[0] : h[1]);
        const half2v got = as_half2((uint32_t)__shfl_xor((int)give, 16, 64));
        const half2v mine = odd ? h[1] : h[0];
        const half2v lo = odd ? got : mine, hi = odd ? mine : got;  // lo: columns of the even lane
        const uint2 v = {__builtin_bit_cast(uint32_t, half2v{lo[0], hi[0]}),
                         __builtin_bit_cast(uint32_t, half2v{lo[1], hi[1]})};
        const int col = c.c0 + 16 * xh + 8 * (c.G >> 1) + 4 * (c.G & 1);
        if (live && c.nok[xh]) *reinterpret_cast<uint2*>(out + (size_t)(c.rbase + row) * c.Iw + col) = v;
      }
    }
  }
  if (!GATEUP) {
    // The down tile goes out through LDS so that every store writes whole rows: 96 x 256 fp16 = the
    // activation ring, 512 B per row, 16-byte chunk j of row r in slot j ^ (r & 31) (the 16 lanes that
    // write one column chunk for 16 rows hit 16 different bank groups).
    static_assert(kStages * kTileBytes >= kGroupedBM * kDownBandCols * 2, "the output tile fits in the ring");
    vm_lgkm_wait<0>();
    tile_barrier();  // every wavefront is done reading the activation ring
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = mt * 16 + c.n;
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const half2v p0 = {to_f16_sat(16.f * acc[mt][ns][0]), to_f16_sat(16.f * acc[mt][ns][1])};
        const half2v p1 = {to_f16_sat(16.f * acc[mt][ns][2]), to_f16_sat(16.f * acc[mt][ns][3])};
        const int chunk = 8 * c.wave + 2 * ns + (c.G >> 1);
        *reinterpret_cast<uint2*>(As + row * (kDownBandCols * 2) + ((chunk ^ (row & 31)) * 16) + 8 * (c.G & 1)) =
            uint2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
      }
    }
    vm_lgkm_wait<0>();
    tile_barrier();
    // thread t stores chunk t % 32 of rows t / 32, t / 32 + 8, ...: one wavefront store covers two rows
    _Float16* out = c.shared ? a.y_s : a.y_r;
    const int tid = (int)threadIdx.x, chunk = tid & 31;
    const int col = c.c0 - 64 * c.wave + 8 * chunk;  // d % 32 == 0: a chunk is all inside d or all past it
#pragma unroll
    for (int i = 0; i < 2 * NMT; ++i) {
      const int row = 8 * i + (tid >> 5);
      const u32x4 v = *reinterpret_cast<const u32x4*>(As + row * (kDownBandCols * 2) + ((chunk ^ (row & 31)) * 16));
      if (row < c.mlen && col < a.d) *reinterpret_cast<u32x4*>(out + (size_t)(c.rbase + row) * a.d + col) = v;
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kGroupedThreads, 8 / kGroupedWaves) void k_grouped(GArgs a) {
  constexpr int BM = kGroupedBM, BK = kGroupedBK;
  constexpr int BANDW = GATEUP ? kGateUpBandCols : kDownBandCols;
  __shared__ __attribute__((aligned(1024))) char As[kStages * kTileBytes];
  __shared__ int s_prefix[kMaxExperts + 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = ufl(tid >> 6);
  const int ngroups = a.E + 1;
  for (int i = tid; i <= ngroups; i += kGroupedThreads) s_prefix[i] = a.mt_prefix[i];
  __syncthreads();
  const int nb = a.nbands;
  const int n_mt = ufl(s_prefix[ngroups]);
  // Work item -> (group rank, band, M-tile).  Workgroups are dispatched round-robin over the 8 XCDs
  // (own L2 each).  With a multiple of 8 bands, XCD x takes the bands = x (mod 8) of every group, in
  // schedule order: each XCD gets the same mix of group sizes (balanced), and all M-tiles that read
  // one weight band run on one XCD, adjacent in time.  Otherwise items go round-robin in schedule order.
  int rank, band, mtile;
  {
    // Work items in schedule order of the groups.  Workgroups are dispatched round-robin over the 8
    // XCDs (own L2 each), so the launch index is remapped (uniform choice, a.order):
    //  0: items are M-tile-major (the bands of one M-tile adjacent) and every run of 8 consecutive
    //     items goes to one XCD: the workgroups that share an activation tile share an L2;
    //  1: band-major inside a group, XCD x taking the bands = x (mod 8) of every group: all M-tiles
    //     that read one weight band run on one XCD, adjacent in time (needs nbands % 8 == 0);
    //  2: items M-tile-major in launch order.
    const int bid = blockIdx.x;
    const int order = (a.order == 1 && nb % 8 != 0) ? 2 : a.order;
    const int nbx = order == 1 ? nb / 8 : nb;  // bands per group seen by this walk
    int item;
    if (order == 0) {
      const int sl = bid >> 3;
      item = (((sl >> 3) << 3) + (bid & 7)) * 8 + (sl & 7);
    } else {
      item = order == 1 ? bid >> 3 : bid;
    }
    if (item >= n_mt * nbx) return;
    int lo = 0, hi = ngroups;  // s_prefix[lo]*nbx <= item < s_prefix[hi]*nbx
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
  if (band * BANDW >= Ndim) return;  // uniform across the workgroup
  const int m0 = mtile * BM;
  const int mlen = min(BM, cnt - m0);
  const int gbase = shared ? 0 : ufl(a.offsets[g]);
  const int rbase = gbase + m0;  // first output row (token for the shared group, else sorted position)
  const uint32_t wrows = GATEUP ? 2u * (uint32_t)Iw : (uint32_t)a.d;
  const uint32_t qstride = (uint32_t)Kdim / 2, sstride = (uint32_t)Kdim / 32;
  const uint8_t* Wq = shared ? a.ws.qs : a.wr.qs + (size_t)g * wrows * qstride;
  const uint16_t* Ws = shared ? a.ws.sc : a.wr.sc + (size_t)g * wrows * sstride;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Wq, wrows * qstride);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(Ws, wrows * sstride * 2);
  const __amdgpu_buffer_rsrc_t ra = shared ? make_rsrc(a.a_s, a.a_s_bytes) : make_rsrc(a.a_r, a.a_r_bytes);

  // ---- activation rows staged by this wavefront: rows kRowsPerWave*wave + 4*i + lane/16, slot lane%16
  uint32_t aoff[kTileLoads];
#pragma unroll
  for (int i = 0; i < kTileLoads; ++i) {
    const int row = kRowsPerWave * wave + 4 * i + (lane >> 4);
    const int rr = row < mlen ? row : 0;
    uint32_t arow;
    if (GATEUP)
      arow = shared ? (uint32_t)(m0 + rr) : (uint32_t)(a.sorted_pair[rbase + rr] / a.k);
    else
      arow = (uint32_t)(rbase + rr);
    // Rows past the group get an offset beyond the buffer: the load still counts in vmcnt but
    // fetches nothing and fills its LDS slot with zeros (those rows are never stored).
    aoff[i] = row < mlen ? arow * (uint32_t)Kdim * 2u + 16u * (uint32_t)((lane & 15) ^ (row & 15)) : kOffsetOOB;
  }
  const int nit = (Kdim + BK - 1) / BK;
  const bool ktail = (Kdim % BK) != 0;
  // ---- this wavefront's weight rows: four 16-row slices; slice ns starts at weight row rowbase[ns]
  // (uniform), lane (n, G) reads row rowbase[ns] + n, block G of every 4-block K chunk
  const int n = lane & 15, G = lane >> 4;
  int rowbase[4];
  bool nok[4];
  int c0;
  if (GATEUP) {
    c0 = band * BANDW + wave * 32;  // h columns c0 .. c0+31: gate rows, then the matching up rows
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = c0 + 16 * (ns & 1);
      nok[ns] = col < Iw;
      rowbase[ns] = (ns < 2 ? 0 : Iw) + (nok[ns] ? col : 0);
    }
  } else {
    c0 = band * BANDW + wave * 64;  // output columns c0 .. c0+63
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = c0 + 16 * ns;
      nok[ns] = col < a.d;
      rowbase[ns] = nok[ns] ? col : 0;
    }
  }
  const int nkb = Kdim / 32;

  TileCtx c;
  c.rq = rq; c.rs = rs; c.ra = ra;
#pragma unroll
  for (int i = 0; i < kTileLoads; ++i) c.aoff[i] = aoff[i];
  // Codes and scales are stored in 16-row groups: codes [rows/16][K/32][16][16 B], scales
  // [rows/16][K/32][16].  Slice ns (16 rows from rowbase[ns], a multiple of 16) has the 16 code blocks
  // of block column b at byte ((rowbase/16)*(K/32) + b)*256 and their scales at ((rowbase/16)*(K/32) +
  // b)*32, so per 4-block iteration lane (n, G) reads bytes 16*lane of one contiguous KiB of codes and
  // bytes 2*lane of one 128-byte run of scales.
  const int Glast = (nkb - 1) - 4 * (nit - 1);  // last valid block of the final iteration, relative
  const int Gt = G < Glast ? G : Glast;
  c.qoff = 16u * (uint32_t)lane;
  c.soff = 2u * (uint32_t)lane;
  c.qoff_tail = 16u * (uint32_t)(n + 16 * Gt);
  c.soff_tail = 2u * (uint32_t)(n + 16 * Gt);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    c.qns[ns] = ufl((int)((uint32_t)(rowbase[ns] / 16) * qstride * 16u));
    c.sns[ns] = ufl((int)((uint32_t)(rowbase[ns] / 16) * sstride * 32u));
    c.nok[ns] = nok[ns];
  }
  c.rdo = (uint32_t)(n * kRowBytes);
  c.gx = (4 * G) ^ n;
  c.c0 = c0; c.wave = wave; c.nit = nit; c.nkb = nkb; c.Kdim = Kdim; c.Iw = Iw; c.mlen = mlen; c.rbase = rbase;
  c.G = G; c.n = n; c.lane = lane; c.ktail = ktail; c.shared = shared;
  c.dq_mask = a.dq_mask;
  c.dq_magic = a.dq_magic;
  switch ((mlen + 15) >> 4) {
    case 1: grouped_tile<GATEUP, 1>(a, c, As); break;
    case 2: grouped_tile<GATEUP, 2>(a, c, As); break;
    case 3: grouped_tile<GATEUP, 3>(a, c, As); break;
    case 4: grouped_tile<GATEUP, 4>(a, c, As); break;
    case 5: grouped_tile<GATEUP, 5>(a, c, As); break;
    default: grouped_tile<GATEUP, 6>(a, c, As); break;
  }
}

// bf16 -> fp16 copy of the activations for the gate+up A operand, stored in
// the dequant pair order inside every group of 8 (x0 x4 x1 x5 x2 x6 x3 x7).
// The conversion is exact inside the fp16 normal range, rounds to nearest
// even in the subnormal range and saturates values beyond it to +-65504
// (the same conversion as the small-T path's staging).
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, _Float16* __restrict__ x16,
                                                  size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  *reinterpret_cast<u32x4*>(x16 + 8 * i) = x8_bf16_to_f16_pairs(ld16(x + 8 * i));
}

// Combine: y[t] = (sum_j w[t,j] * y_pair[pair_pos[t*k+j]]) + y_shared[t], j ascending, no atomics.
// Per-pair and shared outputs arrive in fp16; every thread sums 8 columns in fp32.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ topk_w, const int* __restrict__ pair_pos,
                                                 const _Float16* __restrict__ y_r, const _Float16* __restrict__ y_s,
                                                 const float* residual, float* y, uint16_t* __restrict__ y_bf16,
                                                 int d, int k) {
  const int per_row = (d + 2047) / 2048;
  const int t = blockIdx.x / per_row;
  const int col = ((blockIdx.x % per_row) * 256 + threadIdx.x) * 8;
  if (col >= d) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const u32x4 sv = ld16(y_s + (size_t)t * d + col);
  // up to kCombineBatch pair rows in flight at once; slots past k (and pairs without a row) read a real
  // row of y_pair and weigh 0, so the sum over j stays in slot order and no load is conditional
  constexpr int kCombineBatch = 16;
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    u32x4 v[kCombineBatch];
    float wj[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int j = min(j0 + u, k - 1);
      const int pp = pair_pos[(size_t)t * k + j];
      wj[u] = (j0 + u < k && pp >= 0) ? topk_w[(size_t)t * k + j] : 0.f;
      v[u] = ld16(y_r + (size_t)(pp < 0 ? 0 : pp) * d + col);
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const half2v h = as_half2(v[u][m]);
        acc[2 * m] = fmaf(wj[u], (float)h[0], acc[2 * m]);
        acc[2 * m + 1] = fmaf(wj[u], (float)h[1], acc[2 * m + 1]);
      }
    }
  }
  float4 o0, o1;
  {
    const half2v h0 = as_half2(sv[0]), h1 = as_half2(sv[1]), h2 = as_half2(sv[2]), h3 = as_half2(sv[3]);
    o0 = make_float4(acc[0] + (float)h0[0], acc[1] + (float)h0[1], acc[2] + (float)h1[0], acc[3] + (float)h1[1]);
    o1 = make_float4(acc[4] + (float)h2[0], acc[5] + (float)h2[1], acc[6] + (float)h3[0], acc[7] + (float)h3[1]);
  }
  if (residual) {  // after routed + shared; residual may be y itself (each thread reads what it then writes)
    const float4* ro = reinterpret_cast<const float4*>(residual + (size_t)t * d + col);
    const float4 r0 = ro[0], r1 = ro[1];
    o0 = make_float4(o0.x + r0.x, o0.y + r0.y, o0.z + r0.z, o0.w + r0.w);
    o1 = make_float4(o1.x + r1.x, o1.y + r1.y, o1.z + r1.z, o1.w + r1.w);
  }
  float4* yo = reinterpret_cast<float4*>(y + (size_t)t * d + col);
  yo[0] = o0;
  yo[1] = o1;
  if (y_bf16) {
    const uint32_t b0 = float_to_bf16_bits(o0.x) | ((uint32_t)float_to_bf16_bits(o0.y) << 16);
    const uint32_t b1 = float_to_bf16_bits(o0.z) | ((uint32_t)float_to_bf16_bits(o0.w) << 16);
    const uint32_t b2 = float_to_bf16_bits(o1.x) | ((uint32_t)float_to_bf16_bits(o1.y) << 16);
    const uint32_t b3 = float_to_bf16_bits(o1.z) | ((uint32_t)float_to_bf16_bits(o1.w) << 16);
    *reinterpret_cast<u32x4*>(y_bf16 + (size_t)t * d + col) = u32x4{b0, b1, b2, b3};
  }
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
  a.order = (flags & MOE_FLAG_NO_BANDING) ? 2 : (flags & MOE_FLAG_BAND_MAJOR) ? 1 : 0;
  a.dq_mask = 0x000F000Fu;
  a.dq_magic = 0x64006400u;
  return a;
}

hipError_t launch_grouped_gateup(const Shape& s, const uint16_t* x, const Routing& r, Q4 w13, Q4 s13,
                                 const GroupedOut& o, uint32_t flags, hipStream_t st, bool x16_ready) {
  if (!x16_ready) {
    const size_t n8 = (size_t)s.T * s.d / 8;
    hipLaunchKernelGGL(k_x_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, x, o.x16, n8);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  GArgs a = make_args(s, r, flags);
  a.a_r = o.x16;
  a.a_s = o.x16;
  a.a_r_bytes = a.a_s_bytes = (uint32_t)((size_t)s.T * s.d * 2);
  a.wr = w13;
  a.ws = s13;
  a.h_r = o.h_r;
  a.h_s = o.h_s;
  const int Imax = s.I > s.Is ? s.I : s.Is;
  a.nbands = (Imax + kGateUpBandCols - 1) / kGateUpBandCols;
  const long grid = ((long)grouped_max_mtiles(s) * a.nbands + 63) / 64 * 64;  // whole runs of 8 x 8 items
  hipLaunchKernelGGL(k_grouped<true>, dim3((unsigned)grid), dim3(kGroupedThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_grouped_down(const Shape& s, const Routing& r, Q4 w2, Q4 s2, const GroupedOut& o, uint32_t flags,
                               hipStream_t st) {
  GArgs a = make_args(s, r, flags);
  a.a_r = o.h_r;
  a.a_s = o.h_s;
  a.a_r_bytes = (uint32_t)((size_t)s.T * s.k * s.I * 2);
  a.a_s_bytes = (uint32_t)((size_t)s.T * s.Is * 2);
  a.wr = w2;
  a.ws = s2;
  a.y_r = o.y_pair;
  a.y_s = o.y_s;
  a.nbands = (s.d + kDownBandCols - 1) / kDownBandCols;
  const long grid = ((long)grouped_max_mtiles(s) * a.nbands + 63) / 64 * 64;  // whole runs of 8 x 8 items
  hipLaunchKernelGGL(k_grouped<false>, dim3((unsigned)grid), dim3(kGroupedThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const float* topk_w, const Routing& r, const GroupedOut& o,
                          const float* residual, float* y, uint16_t* y_bf16, hipStream_t st) {
  dim3 grid(((s.d + 2047) / 2048) * s.T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, st, topk_w, r.pair_pos, o.y_pair, o.y_s, residual, y, y_bf16, s.d,
                     s.k);
  return hipGetLastError();
}

}  // namespace moe
