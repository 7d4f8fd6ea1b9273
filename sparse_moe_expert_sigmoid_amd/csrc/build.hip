// On-device routing build for the grouped path.
//
// Page "feat(laguna): batched prefill with tensor-core projections, fused
// MoE, CTA scheduling": grouped-GEMM MoE whose descriptors are built on the
// device, scheduled in descending group size.  Page thewafflehaus/FFAI pull
// request 72 (Nemotron MoE commits): one fill pass reading the router's CSR
// offsets instead of a host round trip, router-sorted token indices, and the
// expert id of every sorted row expanded from the offsets.
//
// Output (pair p = t*k + j; groups = the E experts plus the shared expert as
// group E):
//   counts[E+1], offsets[E+1]      CSR over experts (counts[E] = T)
//   sorted_pair[P], pair_pos[P]    stable order by (expert, pair id) and its inverse
//   row_expert[P]                  expert of each sorted position
//   group_order[E+1]               schedule order of the groups
//   mt_prefix[E+2]                 exclusive prefix of M-tiles along group_order
//
// Two launches over chunks of 256 tokens (the second with one more workgroup
// that builds the group schedule while the others scatter).  Every token picks k distinct
// experts, so inside an expert the stable order is token order: the rank of
// token i of a chunk within expert e is the number of set bits below i in
// the chunk's bitmask of e, plus the counts of the earlier chunks.  The
// result does not depend on scheduling or atomic order.
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_q4.h"

namespace moe {

__global__ __launch_bounds__(256) void k_build_count(const int32_t* __restrict__ ids, int T, int k, int E,
                                                     int* __restrict__ chunk_counts) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kBuildChunk + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of v[0..n) in place (n <= 1024+2), 256 threads.
__device__ void block_exclusive_scan(int* v, int n, int* tmp /* [256] */) {
  const int tid = threadIdx.x;
  const int per = (n + 255) / 256;
  const int lo = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) local += v[lo + i];
  tmp[tid] = local;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  int run = tmp[tid] - local;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) {
      const int c = v[lo + i];
      v[lo + i] = run;
      run += c;
    }
  __syncthreads();
}

// Scatter (workgroups 0 .. nchunks-1, one per chunk of tokens) and the group
// schedule (workgroup nchunks, in parallel with them).
__global__ __launch_bounds__(256) void k_build_scatter(const int32_t* __restrict__ ids, int T, int k, int E,
                                                       int nchunks, uint32_t flags, Routing r) {
  __shared__ __attribute__((aligned(16))) int cnt[kMaxExperts + 4];
  __shared__ int off[kMaxExperts + 2];
  __shared__ int base[kMaxExperts + 2];
  __shared__ uint32_t masks[kMaxExperts * (kBuildChunk / 32)];
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const bool schedule = chunk == nchunks;  // uniform
  constexpr int W = kBuildChunk / 32;
  for (int e = tid; e < E; e += 256) {
    int c = 0, b = 0;
    int ch = 0;
    for (; ch + 8 <= nchunks; ch += 8) {  // eight loads in flight per step
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = r.chunk_counts[(size_t)(ch + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        c += v[u];
        if (ch + u < chunk) b += v[u];
      }
    }
    for (; ch < nchunks; ++ch) {
      const int v = r.chunk_counts[(size_t)ch * E + e];
      c += v;
      if (ch < chunk) b += v;
    }
    cnt[e] = c;
    off[e] = c;
    base[e] = b;
  }
  if (tid == 0) off[E] = 0;
  if (!schedule)
    for (int i = tid; i < E * W; i += 256) masks[i] = 0u;
  __syncthreads();
  block_exclusive_scan(off, E + 1, tmp);  // off[E] = number of valid pairs
  if (!schedule) {
    const int i = tid;
    const int t = chunk * kBuildChunk + i;
    if (t < T) {
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        if ((unsigned)e < (unsigned)E) atomicOr(&masks[e * W + (i >> 5)], 1u << (i & 31));
      }
    }
    __syncthreads();
    if (t < T) {
      for (int j = 0; j < k; ++j) {
        const int p = t * k + j;
        const int e = ids[(size_t)p];
        if ((unsigned)e >= (unsigned)E) {
          r.pair_pos[p] = -1;  // out-of-range id: the pair contributes nothing
          continue;
        }
        const int w = i >> 5;
        int rank = __popc(masks[e * W + w] & ((1u << (i & 31)) - 1u));
        for (int q = 0; q < w; ++q) rank += __popc(masks[e * W + q]);
        const int pos = off[e] + base[e] + rank;
        r.sorted_pair[pos] = p;
        r.pair_pos[p] = pos;
        r.row_expert[pos] = e;
      }
    }
    return;
  }
  // ---- group schedule -------------------------------------------------------
  const int ng = E + 1;
  for (int e = tid; e < E; e += 256) {
    r.counts[e] = cnt[e];
    r.offsets[e] = off[e];
  }
  if (tid == 0) {
    r.counts[E] = T;
    r.offsets[E] = off[E];
  }
  if (tid == 0) cnt[E] = T;
  if (tid < 3) cnt[ng + tid] = -1;  // padding to a multiple of 4: never ranks above a real count
  __syncthreads();
  // rank of group g: larger count first, ties to the lower id (or id order)
  const int n4 = (ng + 3) / 4;
  for (int g = tid; g < ng; g += 256) {
    const int cg = cnt[g];
    int rank;
    if (flags & MOE_FLAG_ID_ORDER) {
      rank = g;
    } else {
      rank = 0;
      for (int h4 = 0; h4 < n4; ++h4) {
        const int4 c4 = reinterpret_cast<const int4*>(cnt)[h4];
        const int h = 4 * h4;
        rank += (c4.x > cg) || (c4.x == cg && h < g);
        rank += (c4.y > cg) || (c4.y == cg && h + 1 < g);
        rank += (c4.z > cg) || (c4.z == cg && h + 2 < g);
        rank += (c4.w > cg) || (c4.w == cg && h + 3 < g);
      }
    }
    r.group_order[rank] = g;
    base[rank] = (cg + kGroupedBM - 1) / kGroupedBM;  // reuse: M-tiles per rank
  }
  __syncthreads();
  for (int q = tid; q <= ng; q += 256) off[q] = q < ng ? base[q] : 0;
  __syncthreads();
  block_exclusive_scan(off, ng + 1, tmp);  // off[ng] = total M-tiles
  for (int q = tid; q <= ng; q += 256) r.mt_prefix[q] = off[q];
}

hipError_t launch_build(const Shape& s, const int32_t* topk_ids, const Routing& r, uint32_t flags,
                        hipStream_t st) {
  const int nchunks = (s.T + kBuildChunk - 1) / kBuildChunk;
  hipLaunchKernelGGL(k_build_count, dim3(nchunks), dim3(256), 0, st, topk_ids, s.T, s.k, s.E, r.chunk_counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_build_scatter, dim3(nchunks + 1), dim3(256), 0, st, topk_ids, s.T, s.k, s.E, nchunks, flags,
                     r);
  return hipGetLastError();
}

}  // namespace moe
