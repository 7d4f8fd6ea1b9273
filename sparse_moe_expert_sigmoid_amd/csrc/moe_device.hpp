// Device-side helpers shared by the gfx950 kernels of the Q4 MoE expert layer.
//
// Q4 format (the library's own layout for the Q4-requantised expert weights
// of the "feat(laguna): Laguna-S-2.1 decode on the CUDA engine" page): a row
// of K values is K/32 blocks; block b is 16 bytes of codes (element 2i in the
// low nibble of byte i, element 2i+1 in the high nibble) and one fp16 scale;
// value = (q - 8) * scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- constants
constexpr int kWave = 64;
constexpr int kBlockK = 32;           // Q4 block length
constexpr int kGroupedBM = 96;        // grouped GEMM: rows per M-tile
constexpr int kGroupedBK = 128;       // grouped GEMM: K per main-loop iteration (4 blocks)
constexpr int kGroupedWaves = 4;                  // grouped GEMM: wavefronts per workgroup (two per CU)
constexpr int kGateUpBandCols = 32 * kGroupedWaves;  // grouped gate+up: h columns per workgroup
constexpr int kDownBandCols = 64 * kGroupedWaves;    // grouped down: output columns per workgroup
constexpr int kBuildChunk = 256;      // routing build: tokens per workgroup
constexpr int kMaxGemvBlocksPerWave = 64;  // small-T path: Q4 blocks of K a wavefront stages (K <= 2048 per wave)
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Reinterpret by value.  (clang's __builtin_bit_cast applied directly to an
// element of an ext_vector_type lvalue, as in bit_cast(v[m]), reads element 0
// whatever m is; routing the element through a by-value parameter avoids it.)
__device__ __forceinline__ half2v as_half2(uint32_t bits) { return __builtin_bit_cast(half2v, bits); }
__device__ __forceinline__ float fp16_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
// The fp16 activations of both paths (x for the expert projections, the SwiGLU output h, each
// expert's down-projection output) saturate: a value beyond the fp16 range becomes +-65504, one inside
// it rounds to nearest even.  Finite inputs therefore never give Inf or NaN.
constexpr float kF16Max = 65504.0f;
__device__ __forceinline__ float clamp_f16_range(float v) { return __builtin_amdgcn_fmed3f(v, -kF16Max, kF16Max); }
__device__ __forceinline__ _Float16 to_f16_sat(float v) { return (_Float16)clamp_f16_range(v); }

// fp32 -> bf16 bits, round to nearest with ties to even (add 0x7FFF plus the lowest kept bit, keep the
// top half; a carry into the exponent gives the next binade or infinity).  NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// (a & mask) | bits in one v_and_or_b32.  gfx9 VOP3 encodings take at most one scalar or literal
// operand, so the mask travels in an SGPR and `bits` in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask_s, uint32_t bits_v) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask_s), "v"(bits_v));
  return r;
}

// ---------------------------------------------------------------- dequant to fp16 (MFMA operand)
// Eight codes of one dword (element m in bits 4m..4m+3) -> eight fp16
// weights (q - 8) * d / 16, in the pair order (e0,e4) (e1,e5) (e2,e6)
// (e3,e7): each pair needs one mask (after at most one shift).  The
// activation operands are stored in the same order within every group of 8
// (see perm_slot).  The factor 1/16 keeps the common form at one shift per
// dword; the GEMM multiplies its fp32 accumulators by 16 (exact) before use.
// Both forms below give round((q - 8) * d) / 16, the same bits, while that
// value is an fp16 normal (always, for 2^-10 <= |d| < 2^-4).
//
// General form: the pair's nibbles placed in the low mantissa of 1024.0
// (v_and_or_b32 with 0x64006400) are exactly 1024 + q; minus 1032 (exact),
// times d (one rounding), times 1/16 (exact unless the result is subnormal).
__device__ __forceinline__ half8 dequant8_general(uint32_t w, half2v d2, uint32_t M, uint32_t C) {
  // M = 0x000F000F (SGPR), C = 0x64006400 (VGPR): p_j = (1024 + e_j, 1024 + e_{j+4}) as fp16 bits
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t t = w >> 4;
  const uint32_t p0 = and_or(w, M, C), p1 = and_or(t, M, C), p2 = and_or(w >> 8, M, C), p3 = and_or(t >> 8, M, C);
  const half2v r0 = ((__builtin_bit_cast(half2v, p0) - off) * d2) * sixteenth;
  const half2v r1 = ((__builtin_bit_cast(half2v, p1) - off) * d2) * sixteenth;
  const half2v r2 = ((__builtin_bit_cast(half2v, p2) - off) * d2) * sixteenth;
  const half2v r3 = ((__builtin_bit_cast(half2v, p3) - off) * d2) * sixteenth;
  return half8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Common form, for 2^-10 <= |d| < 2^-4 (and d = 0): a pair of nibbles masked
// in place into an fp16 with zero exponent is a pair of subnormals, exactly
// q * 2^-24 (bits 0..3 of each half) or q * 2^-20 (bits 4..7).  One packed
// FMA with (d * 2^20, -d/2) or (d * 2^16, -d/2) -- all exact, d * 2^20 <=
// 65504 -- gives (q - 8) * d / 16 with a single rounding, an fp16 normal for
// q != 8.  One shift, four ands, four FMAs per eight weights.
struct SmallScale {
  half2v mul_lo, mul_hi, add;  // (d * 2^20, ..), (d * 2^16, ..), (-d/2, ..)
};
__device__ __forceinline__ SmallScale small_scale(half2v d2) {
  const half2v k = {(_Float16)256.0f, (_Float16)256.0f};
  const half2v hi = d2 * k * k;
  return SmallScale{hi * half2v{(_Float16)16.0f, (_Float16)16.0f}, hi, d2 * half2v{(_Float16)-0.5f, (_Float16)-0.5f}};
}
// 2^-10 <= |d| < 2^-4, or d = 0 (false for inf and NaN)
__device__ __forceinline__ bool small_scale_ok(uint32_t d_bits) {
  const uint32_t m = d_bits & 0x7FFFu;
  return m - 0x1400u < 0x1800u || m == 0u;
}

__device__ __forceinline__ half8 dequant8_small(uint32_t w, const SmallScale& s) {
  const uint32_t w8 = w >> 8;
  const half2v r0 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, w & 0x000F000Fu), s.mul_lo, s.add);
  const half2v r1 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, w & 0x00F000F0u), s.mul_hi, s.add);
  const half2v r2 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, w8 & 0x000F000Fu), s.mul_lo, s.add);
  const half2v r3 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, w8 & 0x00F000F0u), s.mul_hi, s.add);
  return half8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Position, inside a group of 8 stored activations, of logical element c % 8
// (the inverse of the pair order above: stored slot i holds element
// 0,4,1,5,2,6,3,7 [i]).
__device__ __forceinline__ int perm_slot(int c8) { return (c8 < 4) ? 2 * c8 : 2 * (c8 - 4) + 1; }

// Buffer resource for raw (unstructured) loads; accesses at or past
// num_bytes return zero.  Word 3 is the gfx9-family raw-buffer format.
// s_waitcnt vmcnt(N), leaving the LDS and export counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt vmcnt(N) lgkmcnt(0): this wavefront's loads older than the N youngest have landed
// (including tile loads into LDS) and its own LDS reads are complete.
template <int N>
__device__ __forceinline__ void vm_lgkm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
// One wavefront hands data to its other lanes through LDS.  The hardware keeps a wavefront's LDS
// operations in order, but the compiler treats the lanes as separate threads and may move a read of
// another lane's slot above the write that fills it: this fence (wavefront scope, no barrier
// instruction) keeps every LDS access where the program puts it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier without a memory fence.  The ordering it needs comes from explicit waits: every
// wavefront waits for its own loads into LDS (and its LDS reads) before arriving, so after the barrier
// the new tile is in LDS and nobody still reads the buffer that is refilled next.
// (__syncthreads() would also wait for younger loads still in flight.)
__device__ __forceinline__ void tile_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void;  // LDS destination of buffer loads into LDS
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

// ---------------------------------------------------------------- pair order
// 8 consecutive 16-bit values (u0..u3, each a pair (x_2m, x_2m+1)) -> the
// pairs (x0,x4), (x1,x5), (x2,x6), (x3,x7): the order in which one dword of
// codes (element m in bits 4m..4m+3) is dequantised.
__device__ __forceinline__ void x_bf16_pairs(const u32x4 u, uint32_t out[4]) {
  out[0] = __builtin_amdgcn_perm(u[2], u[0], 0x05040100u);
  out[1] = __builtin_amdgcn_perm(u[2], u[0], 0x07060302u);
  out[2] = __builtin_amdgcn_perm(u[3], u[1], 0x05040100u);
  out[3] = __builtin_amdgcn_perm(u[3], u[1], 0x07060302u);
}

// 8 consecutive bf16 activations -> fp16 in that pair order (x0 x4 x1 x5 x2 x6 x3 x7), each value
// rounded to nearest even and saturated to +-65504 (exact inside the fp16 normal range).  The
// grouped path's fp16 activation copy is made with this, by the router or by its own pass.
__device__ __forceinline__ u32x4 x8_bf16_to_f16_pairs(u32x4 v) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float lo = __builtin_bit_cast(float, v[m] << 16);
    const float hi = __builtin_bit_cast(float, v[m] & 0xFFFF0000u);
    v[m] = __builtin_bit_cast(uint32_t, half2v{to_f16_sat(lo), to_f16_sat(hi)});
  }
  uint32_t o[4];
  x_bf16_pairs(v, o);  // the same 16-bit lane shuffle as for bf16 pairs
  return u32x4{o[0], o[1], o[2], o[3]};
}

// ---------------------------------------------------------------- GEMV helper
// v_dot2_f32_f16: two fp16 products added to an fp32 accumulator.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}

// ---------------------------------------------------------------- reductions
// DPP lane exchanges (no LDS traffic): quad xor 1, quad xor 2, mirror inside
// 8 lanes, mirror inside 16 lanes.  After the four steps every lane of a
// 16-lane row holds the row's reduction.  The gfx9 row broadcasts then carry
// lane 15 of each row into the next row (row_bcast:15) and lane 31 into rows
// 2 and 3 (row_bcast:31).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
constexpr int kDppBcast15 = 0x142;    // row_bcast:15
constexpr int kDppBcast31 = 0x143;    // row_bcast:31

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f_rows(float v) {  // rows outside ROW_MASK receive 0
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}
// Sum over each 32-lane half; the result is valid in lanes 16..31 (first
// half) and 48..63 (second half).
__device__ __forceinline__ float half_wave_sum_hi(float v) {
  v = row16_sum(v);
  return v + dpp_f_rows<kDppBcast15, 0xA>(v);
}
// Sum over the wavefront; the result is valid in lanes 48..63.
__device__ __forceinline__ float wave_sum_hi(float v) {
  v = half_wave_sum_hi(v);
  return v + dpp_f_rows<kDppBcast31, 0xC>(v);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
