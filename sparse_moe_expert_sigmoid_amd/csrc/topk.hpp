// Expert selection by one wavefront (sigmoid top-k with a selection-only
// bias), shared by the top-k launch and the small-T gate+up GEMV that selects
// its own experts.
//
// Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine"
// (thewafflehaus/butter pull request 69): a sigmoid top-10 router with a
// score-correction bias.  The bias only ranks (key = s + b); the weights are
// the chosen experts' sigmoid scores normalised to sum to 1; ties go to the
// lower expert id and the k choices are listed by descending key.
#pragma once
#include "moe_device.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k: one wavefront per token.  Lane l holds experts l, l+64, ... as
// order-preserving unsigned keys of s + b (lanes past E hold 0, below every
// real key).  The k-th largest key tau is found bit by bit from the top: a
// candidate bit stays set when at least k keys are >= the candidate (one
// ballot and popcount per key register), so the search costs at most 32
// short steps whatever k is (it stops once a candidate splits off exactly k
// keys).  It starts below the bits that every contender shares: when at least
// k keys lie at or above the binade below the largest key's, tau is among
// them, so their common leading bits (AND and OR over the wavefront) are
// tau's; for scores in (0, 1) that skips the sign and exponent steps.  The
// scores come from the hardware exp2 and reciprocal (s = 1/2 exactly at a
// zero logit).  The chosen experts are the keys above tau and, of the keys
// equal to tau, the lowest ids (ties go to the lower id).  They are compacted
// into LDS; each finds its slot by counting the chosen keys that rank before
// it (a larger key, or an equal key and a lower id), and the weights are
// normalised by the sum of the chosen scores taken in slot order.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  if (f != f) return 1u;  // NaN ranks below every number but above empty slots
  if (f == 0.f) f = 0.f;  // -0 and +0 are the same key (then the lower id wins)
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkLds {  // one wavefront's staging: the chosen entries in id order, then in slot order
  uint32_t key[kMaxTopK];
  int32_t id[kMaxTopK];
  float s[kMaxTopK];
  int32_t slot_id[kMaxTopK];
  float slot_s[kMaxTopK];
};

__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }

// sigma(l) from v_exp_f32 and v_rcp_f32: exact at l = 0; the rounding of l * log2(e) sets the relative
// error, about |l| * 6e-8 (1e-6 at |l| = 16)
__device__ __forceinline__ float sigmoid_score(float l) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * l));
}

// max (OP 0), and (1) or or (2) of v over the wavefront, the same in every lane: four rotations within
// each row of 16 lanes (every lane then holds its row's value), then the four rows combined
template <int OP>
__device__ __forceinline__ uint32_t u32_op(uint32_t a, uint32_t b) {
  return OP == 0 ? (a > b ? a : b) : OP == 1 ? (a & b) : (a | b);
}
template <int OP>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  v = u32_op<OP>(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));  // row_ror:1
  v = u32_op<OP>(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));  // row_ror:2
  v = u32_op<OP>(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = u32_op<OP>(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return u32_op<OP>(u32_op<OP>(r0, r1), u32_op<OP>(r2, r3));
}

// The chosen set of one token, by one wavefront: bit l of chosen[i] set when expert l + 64 i is among the k
// chosen (exactly k bits over all registers); key[i] / sc[i] are lane l's keys and sigmoid scores.
template <int NPER, int NPARTS>
__device__ __forceinline__ void topk_chosen(const float* __restrict__ lrow, size_t part_stride,
                                            const float* __restrict__ bias, int E, int k, int lane,
                                            uint64_t (&chosen)[NPER], uint32_t (&key)[NPER], float (&sc)[NPER]) {
  // every load first, from clamped indices: one memory round trip
  float lg[NPARTS][NPER], bs[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    bs[i] = bias[e];
#pragma unroll
    for (int p = 0; p < NPARTS; ++p) lg[p][i] = lrow[p * part_stride + e];
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    float l = lg[0][i];
#pragma unroll
    for (int p = 1; p < NPARTS; ++p) l += lg[p][i];  // partial logits, in order
    sc[i] = sigmoid_score(l);
    const uint32_t valid = lane + 64 * i < E ? 0xFFFFFFFFu : 0u;
    key[i] = ordered_bits(sc[i] + bs[i]) & valid;
  }
  // tau: the largest value with at least k keys >= it, i.e. the k-th largest key, found bit by bit from
  // the top.  A candidate with exactly k keys at or above it already splits the k largest from the rest
  // (the k-th largest key is >= it, the next one below it): the search stops there with tau just under
  // the candidate, so that the keys above tau are those k and no tie is left to break.
  uint32_t tau = 0u;
  int top = 31;  // the first bit the search decides
  {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) m = max(m, key[i]);
    const uint32_t M = wave_reduce_u32<0>(m);
    // v0: the start of the binade below the largest key's (0 when that would leave the key range)
    const uint32_t v0 = M >= 0x01000000u ? (M & 0xFF800000u) - 0x00800000u : 0u;
    int n0 = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) n0 += popc(__builtin_amdgcn_ballot_w64(key[i] >= v0));
    if (n0 == k && v0 != 0u) {  // exactly k keys at or above v0: they are the k largest
      tau = v0 - 1u;
      top = -1;
    } else if (n0 >= k) {  // tau >= v0: tau shares the leading bits of every key >= v0
      uint32_t a = 0xFFFFFFFFu, o = 0u;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const bool c = key[i] >= v0;
        a &= c ? key[i] : 0xFFFFFFFFu;
        o |= c ? key[i] : 0u;
      }
      const uint32_t A = wave_reduce_u32<1>(a), O = wave_reduce_u32<2>(o);
      if (A == O) {  // every key >= v0 is the same value: that value is tau
        tau = A;
        top = -1;
      } else {
        top = 31 - __builtin_clz(A ^ O);
        tau = top == 31 ? 0u : (A & ~((2u << top) - 1u));
      }
    }
  }
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) cnt += popc(__builtin_amdgcn_ballot_w64(key[i] >= cand));
    if (cnt == k) {  // uniform over the wavefront
      tau = cand - 1u;
      break;
    }
    tau = cnt > k ? cand : tau;
  }
  // chosen: every key above tau (fewer than k), then the lowest ids among the keys equal to tau
  int need = k;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    chosen[i] = __builtin_amdgcn_ballot_w64(key[i] > tau);
    need -= popc(chosen[i]);
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    uint64_t eq = __builtin_amdgcn_ballot_w64(key[i] == tau);
    while (need > 0 && eq != 0) {
      const uint64_t low = eq & (~eq + 1u);
      chosen[i] |= low;
      eq ^= low;
      --need;
    }
  }
}

// Expert id of the j-th chosen expert (0 <= j < k) in id order.
template <int NPER>
__device__ __forceinline__ int topk_nth_chosen(const uint64_t (&chosen)[NPER], int j) {
  int e = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int c = popc(chosen[i]);
    if (j >= 0 && j < c) {
      uint64_t m = chosen[i];
      for (int q = 0; q < j; ++q) m &= m - 1u;  // drop the j lowest set bits
      e = 64 * i + (int)__builtin_ctzll(m);
    }
    j -= c;
  }
  return e;
}

// Slot (0 .. k-1: rank by descending key, equal keys by ascending id) of the chosen expert e.
template <int NPER>
__device__ __forceinline__ int topk_slot_of(const uint64_t (&chosen)[NPER], const uint32_t (&key)[NPER], int e,
                                            int lane) {
  uint32_t ke = 0u;
#pragma unroll
  for (int i = 0; i < NPER; ++i)  // uniform branches: e is the same in every lane
    if (e / 64 == i) ke = (uint32_t)__builtin_amdgcn_readlane((int)key[i], e % 64);
  int slot = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int id = lane + 64 * i;
    slot += popc(chosen[i] & __builtin_amdgcn_ballot_w64(key[i] > ke || (key[i] == ke && id < e)));
  }
  return slot;
}

// The slot order of a chosen set (topk_chosen) and the weights: writes ids[0..k) and w[0..k) (unless
// write is false) and leaves the ids and scores in slot order in sm.slot_id / sm.slot_s.  The lanes
// exchange entries through LDS, with wave_lds_sync between each write and the reads of other lanes.
template <int NPER>
__device__ __forceinline__ void topk_rank_write(const uint64_t (&chosen)[NPER], const uint32_t (&key)[NPER],
                                                const float (&sc)[NPER], int32_t* __restrict__ ids,
                                                float* __restrict__ w, int k, int lane, TopkLds& sm, bool write) {
  // compact the k chosen entries into LDS in id order
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const uint64_t m = chosen[i];
    if ((m >> lane) & 1u) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      sm.key[pos] = key[i];
      sm.id[pos] = lane + 64 * i;
      sm.s[pos] = sc[i];
    }
    base += popc(m);
  }
  wave_lds_sync();
  // lane r < k takes entry r and counts the entries that rank before it: its slot
  const int r = min(lane, k - 1);
  const uint32_t K = sm.key[r];
  const int I = sm.id[r];
  const float S = sm.s[r];
  int slot = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t Kj = (uint32_t)__builtin_amdgcn_readlane((int)K, j);
    const int Ij = __builtin_amdgcn_readlane(I, j);
    slot += (Kj > K || (Kj == K && Ij < I)) ? 1 : 0;
  }
  if (lane < k) {
    sm.slot_id[slot] = I;
    sm.slot_s[slot] = S;
  }
  wave_lds_sync();
  const int q = min(lane, k - 1);
  const int my_id = sm.slot_id[q];
  const float my_s = sm.slot_s[q];
  float tot = 0.f;
  for (int j = 0; j < k; ++j)  // slot order, same value in every lane
    tot += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_s), j));
  if (write && lane < k) {
    ids[lane] = my_id;
    w[lane] = my_s / tot;
  }
  wave_lds_sync();  // callers read sm.slot_id / sm.slot_s in any lane
}

// Selection for one token by one wavefront: writes ids[0..k) and w[0..k) (unless write is false) and
// leaves the ids and scores in slot order in sm.slot_id / sm.slot_s.
template <int NPER, int NPARTS>
__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, size_t part_stride,
                                          const float* __restrict__ bias, int32_t* __restrict__ ids,
                                          float* __restrict__ w, int E, int k, int lane, TopkLds& sm,
                                          bool write = true) {
  uint64_t chosen[NPER];
  uint32_t key[NPER];
  float sc[NPER];
  topk_chosen<NPER, NPARTS>(lrow, part_stride, bias, E, k, lane, chosen, key, sc);
  topk_rank_write<NPER>(chosen, key, sc, ids, w, k, lane, sm, write);
}

}  // namespace moe
