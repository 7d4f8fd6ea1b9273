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
// One workgroup when every expert's token bitmask fits in LDS (k_build_small);
// otherwise two launches over chunks of 256 tokens (the second with one more
// workgroup that builds the group schedule while the others scatter).  Every token picks k distinct
// experts, so inside an expert the stable order is token order: the rank of
// token i of a chunk within expert e is the number of set bits below i in
// the chunk's bitmask of e, plus the counts of the earlier chunks.  The
// result does not depend on scheduling or atomic order.
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_q4.h"

namespace moe {

// f(j, e) for the k expert ids of token t, j ascending.  The ids are loaded 16 at a time, all in
// flight together (a load per id followed by its use would wait out one memory latency per id).
template <typename F>
__device__ __forceinline__ void for_each_id(const int32_t* __restrict__ ids, int t, int k, F&& f) {
  for (int j0 = 0; j0 < k; j0 += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = ids[(size_t)t * k + min(j0 + u, k - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (j0 + u < k) f(j0 + u, v[u]);
  }
}

// The ids of pairs p = p0 + NT*i (i < 4, p < P) for the one-workgroup build (P <= 4*NT), loaded together.
template <int NT>
__device__ __forceinline__ void load_pair_ids(const int32_t* __restrict__ ids, int p0, int P, int (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ids[min(p0 + NT * i, P - 1)];
}

__global__ __launch_bounds__(256) void k_build_count(const int32_t* __restrict__ ids, int T, int k, int E,
                                                     int* __restrict__ chunk_counts) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kBuildChunk + tid;
  if (t < T)
    for_each_id(ids, t, k, [&](int, int e) {
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    });
  __syncthreads();
  for (int e = tid; e < E; e += 256) chunk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of v[0..n) in place (n <= 1024+2) by NT threads: each thread sums a run of
// consecutive elements, the run sums are scanned inside each wavefront with lane shifts and across
// the NT/64 wavefronts through LDS, then every run is rewritten from its offset (two barriers).
template <int NT = 256>
__device__ void block_exclusive_scan(int* v, int n, int* tmp /* [NT/64] */) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) local += v[lo + i];
  int incl = local;  // inclusive scan of the run sums inside the wavefront
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += tmp[w];
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
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int off[kMaxExperts + 2];
  __shared__ int base[kMaxExperts + 2];
  __shared__ __attribute__((aligned(16))) uint32_t masks[kMaxExperts * (kBuildChunk / 32)];
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
    if (t < T)
      for_each_id(ids, t, k, [&](int, int e) {
        if ((unsigned)e < (unsigned)E) atomicOr(&masks[e * W + (i >> 5)], 1u << (i & 31));
      });
    __syncthreads();
    if (t < T)
      for_each_id(ids, t, k, [&](int j, int e) {
        const int p = t * k + j;
        if ((unsigned)e >= (unsigned)E) {
          r.pair_pos[p] = -1;  // out-of-range id: the pair contributes nothing
          return;
        }
        const int w = i >> 5;
        int rank = __popc(masks[e * W + w] & ((1u << (i & 31)) - 1u));
        for (int q = 0; q < w; ++q) rank += __popc(masks[e * W + q]);
        const int pos = off[e] + base[e] + rank;
        r.sorted_pair[pos] = p;
        r.pair_pos[p] = pos;
        r.row_expert[pos] = e;
      });
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
  // rank of group g: larger count first, ties to the lower id (or id order).  With the 64-bit key
  // count * 2^32 + (2^32 - 1 - g) (the chunk masks' LDS is free here) the rank is the number of larger
  // keys: one compare per group, two keys per LDS read.
  uint64_t* key = reinterpret_cast<uint64_t*>(masks);
  const int ng2 = (ng + 1) & ~1;  // padded with a zero key, below every real one
  __syncthreads();
  for (int g = tid; g < ng2; g += 256)
    key[g] = g < ng ? ((uint64_t)(uint32_t)cnt[g] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)g) : 0ull;
  __syncthreads();
  for (int g = tid; g < ng; g += 256) {
    const int cg = cnt[g];
    const uint64_t kg = key[g];
    int rank;
    if (flags & MOE_FLAG_ID_ORDER) {
      rank = g;
    } else {
      rank = 0;
#pragma unroll 8
      for (int h2 = 0; h2 < ng2 / 2; ++h2) {
        const ulonglong2 k2 = reinterpret_cast<const ulonglong2*>(key)[h2];
        rank += (int)(k2.x > kg) + (int)(k2.y > kg);
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


// ---------------------------------------------------------------------------
// The whole build in one workgroup of 1024 threads, for few pairs (T * k <= 4096) whose experts'
// token bitmasks fit in LDS (E * ceil(T/32) <= kBuildSmallWords words).  Bit t of expert e's mask is
// set when token t picked e, so the stable (expert, pair) order ranks a pair of token t inside its
// expert by the set bits before bit t: a per-word prefix (uint16, T < 65536) plus one popcount.
// Counts, offsets, ranks and the group schedule never leave the workgroup: one launch, no global
// histogram.
constexpr int kBuildSmallThreads = 1024;
constexpr int kBuildSmallWords = 20480;

__global__ __launch_bounds__(kBuildSmallThreads) void k_build_small(const int32_t* __restrict__ ids, int T, int k,
                                                                    int E, uint32_t flags, Routing r) {
  __shared__ uint32_t masks[kBuildSmallWords];
  __shared__ uint16_t pre[kBuildSmallWords];  // set bits of the expert's earlier words
  __shared__ int cnt[kMaxExperts + 2];
  __shared__ int off[kMaxExperts + 2];
  __shared__ __attribute__((aligned(16))) uint32_t key[kMaxExperts + 4];
  __shared__ int tmp[kBuildSmallThreads / 64];
  constexpr int NT = kBuildSmallThreads;
  const int tid = threadIdx.x;
  const int W = (T + 31) >> 5;
  const int P = T * k;
  const int ng = E + 1;
  for (int i = tid; i < E * W; i += NT) masks[i] = 0u;
  for (int e = tid; e <= E; e += NT) cnt[e] = 0;
  __syncthreads();
  int pid[4];  // P <= 4 * NT: this thread's pairs are tid + NT*i, i < 4
  load_pair_ids<NT>(ids, tid, P, pid);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + NT * i, e = pid[i];
    if (p < P && (unsigned)e < (unsigned)E) {
      const int t = p / k;
      atomicAdd(&cnt[e], 1);
      atomicOr(&masks[e * W + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += NT) off[e] = e < E ? cnt[e] : 0;
  if (tid == 0) cnt[E] = T;
  // per-word prefix of set bits inside each expert's mask
  for (int e = tid; e < E; e += NT) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      pre[e * W + w] = (uint16_t)run;
      run += __popc(masks[e * W + w]);
    }
  }
  // schedule keys: count * 2^11 + (2047 - g), one compare per group (counts <= T < 2^21)
  const int ng4 = (ng + 3) & ~3;  // padded with zero keys, below every real one
  for (int g = tid; g < ng4; g += NT)
    key[g] = g < ng ? ((uint32_t)(g < E ? cnt[g] : T) << 11) | (uint32_t)(2047 - g) : 0u;
  __syncthreads();
  block_exclusive_scan<NT>(off, E + 1, tmp);  // off[E] = number of valid pairs
  // ranks of the groups (larger count first, ties to the lower id; or id order)
  int my_rank = 0, my_tiles = 0;
  const int g = tid;
  if (g < ng) {
    if (flags & MOE_FLAG_ID_ORDER) {
      my_rank = g;
    } else {
      const uint32_t kg = key[g];
#pragma unroll 4
      for (int h4 = 0; h4 < ng4 / 4; ++h4) {
        const u32x4 k4 = reinterpret_cast<const u32x4*>(key)[h4];
        my_rank += (int)(k4[0] > kg) + (int)(k4[1] > kg) + (int)(k4[2] > kg) + (int)(k4[3] > kg);
      }
    }
    my_tiles = ((g < E ? cnt[g] : T) + kGroupedBM - 1) / kGroupedBM;
  }
  // scatter: position of a pair = offset of its expert + earlier pairs of the expert in token order
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + NT * i, e = pid[i];
    if (p >= P) continue;
    if ((unsigned)e >= (unsigned)E) {
      r.pair_pos[p] = -1;  // out-of-range id: the pair contributes nothing
      continue;
    }
    const int t = p / k, w = t >> 5;
    const int pos = off[e] + pre[e * W + w] + __popc(masks[e * W + w] & ((1u << (t & 31)) - 1u));
    r.sorted_pair[pos] = p;
    r.pair_pos[p] = pos;
    r.row_expert[pos] = e;
  }
  for (int e = tid; e < E; e += NT) {
    r.counts[e] = cnt[e];
    r.offsets[e] = off[e];
  }
  if (tid == 0) {
    r.counts[E] = T;
    r.offsets[E] = off[E];
  }
  __syncthreads();  // every read of off and cnt above is done: off takes the M-tiles in rank order
  for (int q = tid; q <= ng; q += NT) off[q] = 0;
  __syncthreads();
  if (g < ng) {
    r.group_order[my_rank] = g;
    off[my_rank] = my_tiles;
  }
  if (ng > NT) {  // E = 1024: the last group, by thread 0 (ranks are a permutation, no write collides)
    if (tid == 0) {
      const int gl = ng - 1;
      int rank = gl;
      if (!(flags & MOE_FLAG_ID_ORDER)) {
        rank = 0;
        for (int h = 0; h < ng; ++h) rank += (int)(key[h] > key[gl]);
      }
      r.group_order[rank] = gl;
      off[rank] = (T + kGroupedBM - 1) / kGroupedBM;
    }
  }
  __syncthreads();
  block_exclusive_scan<NT>(off, ng + 1, tmp);  // off[ng] = total M-tiles
  for (int q = tid; q <= ng; q += NT) r.mt_prefix[q] = off[q];
}

hipError_t launch_build(const Shape& s, const int32_t* topk_ids, const Routing& r, uint32_t flags,
                        hipStream_t st) {
  // one workgroup while the pairs are few (at most 4 per thread: 8.6 against 13 us at 640 pairs; at
  // 20480 pairs the two parallel launches take 22 us and one workgroup 47) and the masks fit
  if ((long long)s.E * ((s.T + 31) / 32) <= kBuildSmallWords && (long long)s.T * s.k <= 4LL * kBuildSmallThreads) {
    hipLaunchKernelGGL(k_build_small, dim3(1), dim3(kBuildSmallThreads), 0, st, topk_ids, s.T, s.k, s.E, flags, r);
    return hipGetLastError();
  }
  const int nchunks = (s.T + kBuildChunk - 1) / kBuildChunk;
  hipLaunchKernelGGL(k_build_count, dim3(nchunks), dim3(256), 0, st, topk_ids, s.T, s.k, s.E, r.chunk_counts);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_build_scatter, dim3(nchunks + 1), dim3(256), 0, st, topk_ids, s.T, s.k, s.E, nchunks, flags,
                     r);
  return hipGetLastError();
}

}  // namespace moe
