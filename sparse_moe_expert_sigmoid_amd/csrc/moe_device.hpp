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
constexpr int kGemvMaxChunks = 2;     // small-T path: d <= 2 * 4096, I <= 2 * 1024
constexpr int kGroupedBM = 128;       // grouped GEMM: rows per M-tile
constexpr int kGroupedBK = 128;       // grouped GEMM: K per main-loop iteration (4 blocks)
constexpr int kGateUpBandCols = 128;  // grouped gate+up: h columns per workgroup
constexpr int kDownBandCols = 256;    // grouped down: output columns per workgroup
constexpr int kBuildChunk = 256;      // routing build: tokens per workgroup
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ uint32_t ld4(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ float fp16_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// ---------------------------------------------------------------- dequant to fp16 (MFMA operand)
// Eight codes of one dword -> eight fp16 weights (q - 8) * d in natural
// element order.  Each nibble is placed in the low mantissa bits of an fp16
// whose exponent makes it 1024 + q exactly; subtracting 1032 gives q - 8
// exactly, and one packed multiply by the scale rounds once to fp16.
__device__ __forceinline__ half8 dequant8_f16(uint32_t w, half2v d2) {
  const uint32_t t = w >> 4;  // byte j of t has element 2j+1 in its low nibble
  const half2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
  half8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // bytes: [w.b_j, -, t.b_j, -]  (perm pool: t = bytes 4..7, w = bytes 0..3)
    const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t p = __builtin_amdgcn_perm(t, w, sel);
    const uint32_t m = (p & 0x000F000Fu) | 0x64006400u;
    half2v v = __builtin_bit_cast(half2v, m);
    v = (v - off) * d2;
    r[2 * j] = v[0];
    r[2 * j + 1] = v[1];
  }
  return r;
}

// ---------------------------------------------------------------- GEMV helpers (bf16 dot2)
// For v_dot2_f32_bf16 the codes are mapped to bf16 values 1 + q/16 (exact:
// bits 0x3F80 | q << 3) and paired as (e0,e4), (e1,e5), (e2,e6), (e3,e7) of
// a dword, so that every pair comes from one shift and one and-or.  With
// x in matching pairs, sum x*(1 + q/16) = X + Q/16 where X = sum x and
// Q = sum x*q; the block's contribution is then d * (16*dot - 24*X) =
// d * (Q - 8X) = d * sum x*(q - 8).
__device__ __forceinline__ void codes_bf16_pairs(uint32_t w, uint32_t out[4]) {
  out[0] = ((w << 3) & 0x00780078u) | 0x3F803F80u;
  out[1] = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
  out[2] = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
  out[3] = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
}
// 8 consecutive bf16 values (u0..u3, each a pair (x_2m, x_2m+1)) -> pairs
// (x0,x4), (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ void x_bf16_pairs(const u32x4 u, uint32_t out[4]) {
  out[0] = __builtin_amdgcn_perm(u[2], u[0], 0x05040100u);
  out[1] = __builtin_amdgcn_perm(u[2], u[0], 0x07060302u);
  out[2] = __builtin_amdgcn_perm(u[3], u[1], 0x05040100u);
  out[3] = __builtin_amdgcn_perm(u[3], u[1], 0x07060302u);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float half_wave_sum(float v) {  // within each 32-lane half
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float siluf_(float z) { return z / (1.0f + expf(-z)); }

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Map launch index -> work item so that each XCD receives a contiguous
// run of the schedule: items that share a weight band then share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int n_items) {
  const int x = bid & 7, within = bid >> 3;
  const int q = n_items >> 3, rem = n_items & 7;
  return x * q + (x < rem ? x : rem) + within;
}

}  // namespace moe
