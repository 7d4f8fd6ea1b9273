// Host-visible launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Device pointers into the caller's routing workspace.
struct Routing {
  float* logits;       // [T][E]
  int* counts;         // [E+1]
  int* offsets;        // [E+1]
  int* sorted_pair;    // [P]
  int* pair_pos;       // [P]
  int* row_expert;     // [P]
  int* group_order;    // [E+1]
  int* mt_prefix;      // [E+2]
  int* chunk_counts;   // [chunks][E]
};

struct Shape {
  int T, d, E, k, I, Is;
};

struct Q4 {
  const uint8_t* qs;
  const uint16_t* sc;
};

// router.hip
hipError_t launch_router_gemv(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st);
// writes kRouterParts partial logit arrays [part][T][E] (K split in that many parts)
constexpr int kRouterParts = 8;
// x16 (may be nullptr): also write the fp16 pair-ordered copy of x that launch_grouped_gateup reads
hipError_t launch_router_mfma(const Shape& s, const uint16_t* x, const float* w_router, float* logits,
                              hipStream_t st, _Float16* x16 = nullptr);
// logits: nparts partial arrays [nparts][T][E], summed in order
hipError_t launch_topk(const Shape& s, const float* logits, int nparts, const float* bias, int32_t* topk_ids,
                       float* topk_w, hipStream_t st);

// build.hip
hipError_t launch_build(const Shape& s, const int32_t* topk_ids, const Routing& r, uint32_t flags,
                        hipStream_t st);

// gemv.hip  (small-T path)
hipError_t launch_gemv_gateup(const Shape& s, const uint16_t* x, const int32_t* topk_ids, Q4 w13, Q4 s13,
                              _Float16* h_r, _Float16* h_s, hipStream_t st);
// the same, each routed workgroup selecting its token's experts from the router's logits [T][E] (one
// part) and the bias; the selection is also written to topk_ids / topk_w [T][k] for the down pass
hipError_t launch_gemv_gateup_select(const Shape& s, const uint16_t* x, const float* logits, const float* bias,
                                     int32_t* topk_ids, float* topk_w, Q4 w13, Q4 s13, _Float16* h_r, _Float16* h_s,
                                     hipStream_t st);
// residual: optional fp32 [T][d] added after the routed + shared sum (may be y itself; nullptr = none);
// y_bf16: optional bf16 [T][d] copy of y, rounded to nearest even (nullptr = none)
hipError_t launch_gemv_down_combine(const Shape& s, const int32_t* topk_ids, const float* topk_w, Q4 w2, Q4 s2,
                                    const _Float16* h_r, const _Float16* h_s, const float* residual, float* y,
                                    uint16_t* y_bf16, hipStream_t st);

// grouped.hip  (grouped path)
struct GroupedOut {
  _Float16* x16;   // [T][d]   fp16 copy of x
  _Float16* h_r;   // [P][I]   sorted rows
  _Float16* h_s;   // [T][Is]
  _Float16* y_pair;  // [P][d]   sorted rows
  _Float16* y_s;     // [T][d]
};
int grouped_max_mtiles(const Shape& s);
// x16_ready: o.x16 already holds the fp16 copy of x (written by launch_router_mfma)
hipError_t launch_grouped_gateup(const Shape& s, const uint16_t* x, const Routing& r, Q4 w13, Q4 s13,
                                 const GroupedOut& o, uint32_t flags, hipStream_t st, bool x16_ready = false);
hipError_t launch_grouped_down(const Shape& s, const Routing& r, Q4 w2, Q4 s2, const GroupedOut& o,
                               uint32_t flags, hipStream_t st);
// residual and y_bf16 as for launch_gemv_down_combine
hipError_t launch_combine(const Shape& s, const float* topk_w, const Routing& r, const GroupedOut& o,
                          const float* residual, float* y, uint16_t* y_bf16, hipStream_t st);

// pack.hip: n_mats row-major Q4 matrices [rows][K] -> the 16-row-group layout (rows % 16 == 0, K % 32 == 0)
hipError_t launch_q4_pack(size_t n_mats, int rows, int K, const uint8_t* qs_in, const uint16_t* sc_in,
                          uint8_t* qs_out, uint16_t* sc_out, hipStream_t st);

// w4a8.hip: MXFP4 weights x FP8 activations on the grouped path
struct MxWeights {
  const uint8_t* w13_codes; const uint8_t* w13_exp;   // MXFP4 or MXFP8 codes / block exponents, 16-row groups
  const uint8_t* w2_codes;  const uint8_t* w2_exp;
  const uint8_t* s13_codes; const uint8_t* s13_exp;
  const uint8_t* s2_codes;  const uint8_t* s2_exp;
};
struct W4A8Scratch {
  uint8_t* x8;  float* xs;     // [T][d] e4m3 codes of x, [T] row scales
  _Float16* h_r; _Float16* h_s;  // [P][I] (sorted rows), [T][Is]
  uint8_t* h8_r; float* hs_r;  // [P][I], [P]
  uint8_t* h8_s; float* hs_s;  // [T][Is], [T]
  _Float16* y_pair; _Float16* y_s;  // [P][d] (sorted rows), [T][d]
};
// nblocks Q4 blocks (16 code bytes + one fp16 scale each) -> MXFP4 (16 bytes of e2m1 codes, same nibble
// order) or with fp8 MXFP8 (32 e4m3 codes), and biased block exponents, block b to block b
hipError_t launch_q4_to_mx(size_t nblocks, const uint8_t* qs, const uint16_t* sc, uint8_t* codes, uint8_t* exps,
                           bool fp8, hipStream_t st);
// rows x K values (bf16 bits, or fp16 when in_f16; K % 4 == 0) -> e4m3 codes and fp32 row scales
hipError_t launch_rows_fp8(const uint16_t* in, bool in_f16, int rows, int K, uint8_t* out, float* scale,
                           hipStream_t st);
// d, I, Is % 128 == 0; routing built for the grouped path; fp8: MXFP8 weights (W8A8), else MXFP4 (W4A8)
hipError_t launch_w4a8_forward(const Shape& s, const uint16_t* x, const Routing& r, const MxWeights& w,
                               const W4A8Scratch& o, const float* topk_w, float* y, uint32_t flags, bool fp8,
                               hipStream_t st);

// norm.hip
// x[i] = bf16(h[i]) for n values (n % 8 == 0), round to nearest even
hipError_t launch_f32_to_bf16(const float* h, uint16_t* x, size_t n, hipStream_t st);
// x[t] = bf16(h[t] / sqrt(mean(h[t]^2) + eps) * gamma) for T rows of d values (d % 8 == 0)
hipError_t launch_rmsnorm_bf16(const float* h, const float* gamma, float eps, uint16_t* x, int T, int d,
                               hipStream_t st);

}  // namespace moe
