// moe_select.h -- expert selection: the top-k of one token's logits by value,
// ties to the lower expert index, and the softmax over the selected logits
// ([P273] Summary item 1: an in-kernel top-8 instead of a separate sort).
// Two forms: the four-wave rank selection of the persistent kernel (also used
// by the per-layer gate/up kernel), and a one-wave form for the router's last
// workgroup, which selects for several tokens at once (one per wave).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_decode.h"
#include "moe_device.h"

namespace moe {

// Order-preserving 32-bit key of a logit (a larger float gives a larger key);
// NaN counts as -inf and -0 as +0.  Never 0, which marks an empty or taken slot.
__device__ __forceinline__ uint32_t logit_key(float v) {
  if (v != v) v = -__builtin_inff();
  if (v == 0.0f) v = 0.0f;
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Expert selection ([P273] Summary item 1: the top-k runs inside the router's
// kernel), larger logit first and the lower expert id first among equal
// logits, in three steps:
//  1. waves 0..3 each take the experts e = 64w + lane + 256j and find their own
//     k best (by ranking within the wave for E <= 256, else by k wave-wide
//     picks), as 64-bit candidates key << 32 | ~id (0 where a wave has fewer
//     than k experts);
//  2. wave 0 ranks the 4k candidates against each other (all distinct), and
//     the candidate of rank r < k is slot r; the selected logits (and the
//     shared-gate logit) are copied out (the persistent kernel reuses the
//     logits' landing area for the routed rows right after);
//  3. later, off the critical path, wave 0 turns the copied logits into the
//     softmax weights (fp64, shifted by the largest, summed in slot order) and
//     the shared expert's sigmoid gate.
// Candidate slots per wave: wave w's candidates sit at kc*w + 0..k-1 (the rest
// of its kc slots hold 0), so 4*kc slots in all.
__device__ __forceinline__ int cand_stride(int k) { return k <= 8 ? 8 : 16; }

template <int NPL>
__device__ __forceinline__ void wave_topk(const float* lg, int E, int k, int kc, int w, unsigned long long* cand) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = 64 * w + lane + 256 * j;
    key[j] = (e < E) ? logit_key(lg[e]) : 0u;
  }
  if (lane >= k && lane < kc) cand[kc * w + lane] = 0ull;   // slots past k never rank
  for (int s = 0; s < k; ++s) {
    uint32_t hv = key[0], hid = (uint32_t)(64 * w + lane);
#pragma unroll
    for (int j = 1; j < NPL; ++j)
      if (key[j] > hv) { hv = key[j]; hid = (uint32_t)(64 * w + lane + 256 * j); }
    const uint32_t m = wave_max_u32(hv);
    const unsigned long long tied = __ballot(hv == m);
    // usually one lane holds the maximum: it takes its own key out and writes
    // the candidate; on a tie the lowest id among the tied lanes goes first
    uint32_t id = hid;
    bool win = (hv == m);
    if (__popcll(tied) != 1) {
      id = wave_min_u32(hv == m ? hid : 0xffffffffu);
      win = (hid == id);
    }
    if (win) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if ((uint32_t)(64 * w + lane + 256 * j) == id) key[j] = 0u;
      cand[kc * w + s] = m ? (((unsigned long long)m << 32) | (uint32_t)~id) : 0ull;
    }
  }
}

// Adds [k_i > c] to a_i for four keys.  The four compares write four
// separate SGPR-pair masks and only then do the four carry-in adds read
// them: the compiler's form puts every compare through VCC, each add waiting
// on its own compare, a chain of one compare, two wait states and one add
// per key.  Here each add reads a mask written three instructions earlier,
// which covers the wait states a VALU-written mask needs before a VALU reads
// it as a carry.
__device__ __forceinline__ void count4_above(unsigned long long k0, unsigned long long k1, unsigned long long k2,
                                             unsigned long long k3, unsigned long long c, int& a0, int& a1, int& a2,
                                             int& a3) {
  unsigned long long m0, m1, m2, m3;
  asm volatile(
      "v_cmp_gt_u64_e64 %4, %8, %12\n\t"
      "v_cmp_gt_u64_e64 %5, %9, %12\n\t"
      "v_cmp_gt_u64_e64 %6, %10, %12\n\t"
      "v_cmp_gt_u64_e64 %7, %11, %12\n\t"
      "v_addc_co_u32_e64 %0, %4, 0, %0, %4\n\t"
      "v_addc_co_u32_e64 %1, %5, 0, %1, %5\n\t"
      "v_addc_co_u32_e64 %2, %6, 0, %2, %6\n\t"
      "v_addc_co_u32_e64 %3, %7, 0, %3, %7"
      : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "=&s"(m0), "=&s"(m1), "=&s"(m2), "=&s"(m3)
      : "v"(k0), "v"(k1), "v"(k2), "v"(k3), "v"(c));
}

// Count of the 2*NP keys at `k2` (NP pairs) that are above c.  The loads go
// out in batches of 8 pairs, each batch before the compares of the previous
// one, and the count is kept in four separate sums.
template <int NP>
__device__ __forceinline__ int count_above(const ulonglong2* k2, unsigned long long c) {
  static_assert(NP % 8 == 0, "whole batches");
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  ulonglong2 v[8], nv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = k2[j];
#pragma unroll
  for (int b = 0; b < NP; b += 8) {
    if (b + 8 < NP) {
#pragma unroll
      for (int j = 0; j < 8; ++j) nv[j] = k2[b + 8 + j];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; j += 2) count4_above(v[j].x, v[j].y, v[j + 1].x, v[j + 1].y, c, a0, a1, a2, a3);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = nv[j];
  }
  return (a0 + a1) + (a2 + a3);
}

// E <= 256: wave w ranks its 64 experts against each other in parallel
// (one key per lane; 32 broadcast 16-byte LDS loads and 64 independent
// compares per lane, no dependent chain); the lanes ranked below k are the
// wave's candidates, already in order.  keys: 256 u64 of LDS.  cand_lg (or
// null) receives each candidate's logit beside it.
__device__ __forceinline__ void wave_rank_topk(const float* lg, int E, int k, int kc, int w,
                                               unsigned long long* keys, unsigned long long* cand,
                                               float* cand_lg = nullptr) {
  const int lane = threadIdx.x & 63;
  const int e = 64 * w + lane;
  const unsigned long long c = (e < E) ? (((unsigned long long)logit_key(lg[e]) << 32) | (uint32_t)~e) : 0ull;
  keys[e] = c;
  if (lane < kc) cand[kc * w + lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int rank = count_above<32>(reinterpret_cast<const ulonglong2*>(keys + 64 * w), c);
  if (rank < k && c != 0ull) {
    cand[kc * w + rank] = c;
    if (cand_lg) cand_lg[kc * w + rank] = lg[e];
  }
}

// (cand_lg: E <= 256 only)
__device__ __forceinline__ void topk_candidates(const float* lg, int E, int k, int wave, unsigned long long* keys,
                                                unsigned long long* cand, float* cand_lg = nullptr) {
  if (wave >= 4) return;
  const int kc = cand_stride(k);
  if (E <= 256) wave_rank_topk(lg, E, k, kc, wave, keys, cand, cand_lg);
  else if (E <= 512) wave_topk<2>(lg, E, k, kc, wave, cand);
  else wave_topk<4>(lg, E, k, kc, wave, cand);
}

// wave 0, after a barrier: slot ids -> sel[0..k), their logits -> lgsel[0..k),
// the shared-gate logit -> lgsel[k].  Each candidate counts the candidates
// above it over all 4*kc slots (unused slots hold 0, read with unrolled
// 16-byte loads).  For kc == 8 (32 slots) lanes L and L+32 both hold slot L
// and count half of the slots each; one cross-half lane swap adds the halves.
// For kc == 16 lane L holds slot L and counts all 64.  Returns true unless
// exactly k candidates rank below k (fewer than k valid experts).  With
// cand_lg (the candidates' logits, and at cand_lg[64] the shared-gate logit)
// the logits are not read again.
__device__ __forceinline__ bool rank_candidates(const float* lg, int E, int k, bool has_sg,
                                                const unsigned long long* cand, uint32_t* sel, float* lgsel,
                                                const float* cand_lg = nullptr) {
  const int lane = threadIdx.x & 63;
  const int kc = cand_stride(k);
  const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cand);
  unsigned long long c;
  int rank, ci;
  bool mine;
  if (kc == 8) {
    const int slot = lane & 31;
    ci = slot;
    c = ((slot & 7) < k) ? cand[slot] : 0ull;
    const int part = count_above<8>(c2 + 8 * (lane >> 5), c);
    const auto sw = __builtin_amdgcn_permlane32_swap(part, part, false, false);
    rank = (int)sw[0] + (int)sw[1];
    mine = lane < 32;
  } else {
    ci = lane;
    c = (lane < 4 * kc && (lane & (kc - 1)) < k) ? cand[lane] : 0ull;
    rank = count_above<32>(c2, c);
    mine = true;
  }
  const bool take = mine && c != 0ull && rank < k;
  if (take) {
    const uint32_t id = ~(uint32_t)c;
    sel[rank] = id;
    lgsel[rank] = cand_lg ? cand_lg[ci] : lg[id];
  }
  if (lane == 0) lgsel[k] = has_sg ? (cand_lg ? cand_lg[64] : lg[E]) : 0.0f;
  return __popcll(__ballot(take)) != k;
}

// The id of the candidate of rank r (0 <= r < k), found by every lane of the
// calling wave with rank_candidates' counting for kc == 8 (k <= 8); ok is
// false unless exactly k candidates rank below k and one of them has rank r.
__device__ __forceinline__ uint32_t candidate_of_rank(const unsigned long long* cand, int k, int r, bool& ok) {
  const int lane = threadIdx.x & 63;
  const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cand);
  const int slot = lane & 31;
  const unsigned long long c = ((slot & 7) < k) ? cand[slot] : 0ull;
  const int part = count_above<8>(c2 + 8 * (lane >> 5), c);
  const auto sw = __builtin_amdgcn_permlane32_swap(part, part, false, false);
  const int rank = (int)sw[0] + (int)sw[1];
  const bool take = lane < 32 && c != 0ull && rank < k;
  const unsigned long long m = __ballot(take && rank == r);
  ok = __popcll(__ballot(take)) == k && m != 0ull;
  const int src = m ? __ffsll((long long)m) - 1 : 0;
  return (uint32_t)__builtin_amdgcn_readlane((int)~(uint32_t)c, src);
}

// wave 0: routing weights sel[k..2k) and the shared gate sel[2k] from lgsel;
// scr: k doubles of LDS
__device__ __forceinline__ void routing_weights(int k, bool has_sg, const float* lgsel, uint32_t* sel, double* scr) {
  const int lane = threadIdx.x & 63;
  const double lmax = (double)lgsel[0];
  double arg = 0.0;
  if (lane < k) arg = (double)lgsel[lane] - lmax;
  else if (lane == k && has_sg) arg = -(double)lgsel[k];
  const double ex = exp(arg);
  if (lane < k) scr[lane] = ex;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  double sum = 0.0;
  for (int s = 0; s < k; ++s) sum += scr[s];   // slot order
  if (lane < k) sel[k + lane] = __float_as_uint((float)(ex / sum));
  else if (lane == k) sel[2 * k] = __float_as_uint(has_sg ? (float)(1.0 / (1.0 + ex)) : 0.0f);
}

// Wave-level top-k over E <= 64*NPL logits held in memory.  Each lane keeps
// its NPL 32-bit order keys (expert e = lane + 64j in slot j); a round takes
// the wave-wide maximum key and, among the experts holding it, the lowest
// index (the first slot j with a match, then its first lane), so slots come in
// rank order with ties to the lower index.  A taken key becomes 0, below
// every real key (logit_key: -0 counts as +0, as IEEE equality ties them,
// and NaN as -inf).
template <int NPL>
__device__ void wave_topk_softmax_n(const float* logits, int E, int k, int32_t* ids_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? logit_key(logits[e]) : 0u;
  }
  int my_id = 0;   // lane s < k: the id of slot s
  for (int s = 0; s < k; ++s) {
    uint32_t best = key[0];
#pragma unroll
    for (int j = 1; j < NPL; ++j) best = max(best, key[j]);
    const uint32_t wbest = wave_max_u32(best);
    int win = -1;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const unsigned long long m = __ballot(key[j] == wbest);
      if (win < 0 && m != 0ull) win = 64 * j + __ffsll((long long)m) - 1;
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (win == lane + 64 * j) key[j] = 0u;
    if (lane == s) my_id = win;
  }
  // softmax over the selected logits, shifted by the largest (slot 0), fp64:
  // lane s takes slot s's exponential, every lane sums them in slot order
  const double m = (double)logits[__shfl(my_id, 0)];
  const double ex = (lane < k) ? exp((double)logits[my_id] - m) : 0.0;
  double sum = 0.0;
  for (int s = 0; s < k; ++s) sum += __shfl(ex, s);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = (float)(ex / sum);
  }
}
// keys per lane from the expert count (the scan is the same, over fewer keys)
__device__ __forceinline__ void wave_topk_softmax(const float* logits, int E, int k, int32_t* ids_out, float* w_out) {
  static_assert(MOE_MAX_EXPERTS <= 16 * 64, "dispatch below covers up to 16 keys per lane");
  if (E <= 64) wave_topk_softmax_n<1>(logits, E, k, ids_out, w_out);
  else if (E <= 128) wave_topk_softmax_n<2>(logits, E, k, ids_out, w_out);
  else if (E <= 256) wave_topk_softmax_n<4>(logits, E, k, ids_out, w_out);
  else if (E <= 512) wave_topk_softmax_n<8>(logits, E, k, ids_out, w_out);
  else wave_topk_softmax_n<16>(logits, E, k, ids_out, w_out);
}

}  // namespace moe
