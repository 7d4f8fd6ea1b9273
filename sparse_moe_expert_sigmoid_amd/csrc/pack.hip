// Repack of row-major Q4 matrices into the library's 16-row groups, on the device.
//
// Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine" loads
// Q4-requantised expert weights once and keeps them resident; the pages fix
// no bit layout.  A caller holds each matrix [rows][K] row-major (codes
// [rows][K/2], element 2i in the low nibble of byte i; fp16 scales
// [rows][K/32]); the kernels read them in groups of 16 rows (codes
// [rows/16][K/32][16][16 B], scales [rows/16][K/32][16]), so that the 16 rows
// x 4 blocks one wavefront load takes are contiguous.  The repack moves whole
// 16-byte code blocks and their scales: a pure permutation, no arithmetic.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {

// One thread per Q4 block, in output order (the writes are contiguous; the reads gather 16 rows).
__global__ __launch_bounds__(256) void k_q4_pack(const uint8_t* __restrict__ qs_in, const uint16_t* __restrict__ sc_in,
                                                 uint8_t* __restrict__ qs_out, uint16_t* __restrict__ sc_out,
                                                 size_t nblocks, uint32_t rows, uint32_t nkb) {
  const uint32_t ngroups = rows / 16;
  for (size_t ob = (size_t)blockIdx.x * 256 + threadIdx.x; ob < nblocks; ob += (size_t)gridDim.x * 256) {
    // ob = ((m * ngroups + rg) * nkb + b) * 16 + r16
    const uint32_t r16 = (uint32_t)(ob & 15);
    size_t q = ob >> 4;
    const uint32_t b = (uint32_t)(q % nkb);
    q /= nkb;
    const uint32_t rg = (uint32_t)(q % ngroups);
    const size_t m = q / ngroups;
    const size_t ib = ((m * rows + (size_t)rg * 16 + r16) * nkb) + b;  // row-major block index
    *reinterpret_cast<u32x4*>(qs_out + 16 * ob) = ld16(qs_in + 16 * ib);
    sc_out[ob] = sc_in[ib];
  }
}

hipError_t launch_q4_pack(size_t n_mats, int rows, int K, const uint8_t* qs_in, const uint16_t* sc_in,
                          uint8_t* qs_out, uint16_t* sc_out, hipStream_t st) {
  const uint32_t nkb = (uint32_t)K / 32;
  const size_t nblocks = n_mats * (size_t)rows * nkb;
  const size_t want = (nblocks + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_q4_pack, dim3(grid), dim3(256), 0, st, qs_in, sc_in, qs_out, sc_out, nblocks, (uint32_t)rows,
                     nkb);
  return hipGetLastError();
}

}  // namespace moe
