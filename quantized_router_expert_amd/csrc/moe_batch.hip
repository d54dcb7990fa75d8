// moe_batch.hip -- several tokens at once: experts grouped by the tokens that
// selected them.
//
// A group (the tokens whose top-k contains expert e) with at least group_min
// tokens reads its expert's rows once and multiplies them on the int8 matrix
// cores against the members' Q8_1 codes (v_mfma_i32_16x16x32_i8, one
// 32-element block per step), then scales and sums exactly as the
// single-token integer path does.  A smaller group takes that integer path
// (Q8_1 x v_dot4) for all its members at once, reading each weight task once.
// Either way every token gets the bit-identical value the batch-1 stage gives
// it: the grouped path is batch-invariant.  The shared expert is one group of
// all the tokens.  Norm, router and top-k run per token as at batch 1; the
// combine is per token in slot order.  The pages cover batch 1 only ([P359]
// Summary: the Q8_1 integer dot path); the grouping is this library's.
//
// MFMA operand layout (16x16x32, 8 elements per lane): lane l holds row l%16
// of A and column l%16 of B at k = 8*(l/16) .. +7, and rows 4*(l/16) .. +3 of
// column l%16 of D.
#include <algorithm>
#include <mutex>

#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kBThreads = 256;
constexpr int kBWaves = kBThreads / 64;
constexpr int kBRows = 16;                   // rows per wave
constexpr int kBRowsPerBlock = kBRows * kBWaves;

// ---------------------------------------------------------------- grouping
// Exclusive prefix sum over the block (blockDim.x a multiple of 64): a
// shuffle scan in each wave, then the wave totals; wsum holds one int per wave.
__device__ __forceinline__ long long block_excl_scan(long long v, long long* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  long long pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  __syncthreads();
  return pre + x - v;
}

// ids [n][k] -> cnt[e] tokens per expert, moff[e] first member, members (p = t*k + s,
// token order within an expert), dlist = the experts with cnt > 0 in increasing
// order, nd[0] = their number, err[0] = 1 if an id is outside [0, E).
__global__ __launch_bounds__(1024) void k_group(const int32_t* ids, int n, int k, int E, int gmin, int* cnt, int* moff,
                                                int* members, int* dlist, int* nd, int* blist, int* nb, int* err) {
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ long long tmp[1024 / 64];
  __shared__ int s_ids[MOE_MAX_BATCH * MOE_MAX_TOPK];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int P = n * k;
  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  for (int p = tid; p < P; p += 1024) s_ids[p] = ids[p];
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = s_ids[p];
    if (e < 0 || e >= E) s_bad = 1;
    else atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  const int c = (tid < E) ? s_cnt[tid] : 0;
  // one scan of (count, count > 0, count >= gmin) packed in 16-bit fields:
  // each total is at most n*k <= MOE_MAX_BATCH * MOE_MAX_TOPK = 1024 and E <= 1024
  static_assert(MOE_MAX_BATCH * MOE_MAX_TOPK < 65536 && MOE_MAX_EXPERTS <= 1024, "packed scan");
  const long long sc = block_excl_scan((long long)c | ((long long)(c > 0 ? 1 : 0) << 16) |
                                       ((long long)(c >= gmin ? 1 : 0) << 32), tmp);
  const int off = (int)(sc & 0xffff), pos = (int)((sc >> 16) & 0xffff), bpos = (int)((sc >> 32) & 0xffff);
  if (tid < E) {
    s_off[tid] = off;
    cnt[tid] = c;
    moff[tid] = off;
    if (c > 0) dlist[pos] = tid;
    if (c >= gmin) blist[bpos] = tid;
  }
  if (tid == 1023) {
    nd[0] = pos + (c > 0 ? 1 : 0);
    nb[0] = bpos + (c >= gmin ? 1 : 0);
  }
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = s_ids[p];
    if (e < 0 || e >= E) continue;
    const int t = p / k;
    int rank = 0;
    for (int q = 0; q < t * k; ++q) rank += (s_ids[q] == e) ? 1 : 0;
    members[s_off[e] + rank] = p;
  }
  if (tid == 0) err[0] = s_bad;
}

// ---------------------------------------------------------------- int8 matrix-core rows
// A group of group_min or more tokens multiplies its expert's rows on the
// int8 matrix cores (v_mfma_i32_16x16x32_i8: 16 rows x 16 tokens x one
// 32-element block).  The weight codes (Q4_K nibbles, Q5_K 5-bit codes, Q8_0
// bytes) and the tokens' Q8_1 codes go in as int8, so each sub-block's dot
// is the exact integer of the single-token path; each task (a 64-element
// K-quant group, or one Q8_0 block) is then scaled in fp64 by the same
// expression as the single-token row task, and the tasks of a row are summed
// in the same order: lane position p of a TP-lane group holds tasks p, p+64,
// ..., and the positions meet in a balanced binary tree (the lane-group
// reduction).  Every token of the group therefore gets the bit-identical
// value the batch-1 path gives it.  Wave w of the block takes positions
// [w TP/4, (w+1) TP/4) as a subtree; the four subtrees meet as
// (q0 + q1) + (q2 + q3).
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i mfma_i8(uint2 a, uint2 b) {
  const long la = (long)(((unsigned long long)a.y << 32) | a.x);
  const long lb = (long)(((unsigned long long)b.y << 32) | b.x);
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(la, lb, v4i{0, 0, 0, 0}, 0, 0, 0);
}

// codes of elements 8q .. 8q+7 of sub-block 2g + hi of a K-quant superblock, as int8
template <int TYPE>
__device__ __forceinline__ uint2 kq_codes8(const uint8_t* blk, int g, int q, int hi) {
  const int qs_off = (TYPE == MOE_TYPE_Q5_K) ? 48 : 16;
  const uint2 b = *reinterpret_cast<const uint2*>(blk + qs_off + 32 * g + 8 * q);
  uint2 r = make_uint2((b.x >> (4 * hi)) & 0x0f0f0f0fu, (b.y >> (4 * hi)) & 0x0f0f0f0fu);
  if (TYPE == MOE_TYPE_Q5_K) {
    const uint2 h = *reinterpret_cast<const uint2*>(blk + 16 + 8 * q);
    r.x |= ((h.x >> (2 * g + hi)) & 0x01010101u) << 4;
    r.y |= ((h.y >> (2 * g + hi)) & 0x01010101u) << 4;
  }
  return r;
}
// Q8_0 block t of a row: codes 8q .. 8q+7 (34-byte blocks: 2-byte aligned)
__device__ __forceinline__ uint2 q80_codes8(const uint8_t* row, int t, int q) {
  const uint16_t* c = reinterpret_cast<const uint16_t*>(row + 34L * t) + 1 + 4 * q;
  return make_uint2((uint32_t)c[0] | ((uint32_t)c[1] << 16), (uint32_t)c[2] | ((uint32_t)c[3] << 16));
}

// The fp64 value of task t of this lane's row (row lane % 16 of the 16; a
// row past nr gives an unused value) against the lane's 4 tokens (tile
// tokens 4*(lane/16) + i), for NM matrices of TYPE.  The tokens' codes are
// the MFMA's A operand and the weight codes its B operand, so each lane's
// results share one weight row and its scales are decoded once per task.
// codes8(blk, q) -> the codes 8q..8q+7 of Q8_1 block blk of tile token
// lane % 16 (zero for a missing token); ds(tok, blk) -> d and s of tile token
// tok's block blk (zero for a missing token).
template <int TYPE, int NM, class Codes, class DS>
__device__ __forceinline__ void i8_task(const uint8_t* const (&mats)[NM], long rb, int nr, int t, Codes codes8, DS ds,
                                        double (&v)[NM][4]) {
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const bool rv = r < nr;
  const long ro = (long)(rv ? r : 0) * rb;
  if (TYPE == MOE_TYPE_Q8_0) {
    const uint2 aq = codes8(t, q);
    float2 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = ds(4 * q + i, t);
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      uint2 wq = q80_codes8(mats[mi] + ro, t, q);
      if (!rv) wq = make_uint2(0u, 0u);
      const v4i D = mfma_i8(aq, wq);
      const float dw = f16_to_f32(*reinterpret_cast<const uint16_t*>(mats[mi] + ro + 34L * t));
#pragma unroll
      for (int i = 0; i < 4; ++i) v[mi][i] = (double)dw * (double)a[i].x * (double)D[i];
    }
    return;
  }
  const int b = t >> 2, g = t & 3;
  const int jlo = 8 * b + 2 * g;
  const uint2 alo = codes8(jlo, q), ahi = codes8(jlo + 1, q);
  float2 slo[4], shi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    slo[i] = ds(4 * q + i, jlo);
    shi[i] = ds(4 * q + i, jlo + 1);
  }
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) {
    const uint8_t* blk = mats[mi] + ro + (long)b * block_bytes(TYPE);
    uint2 wlo = kq_codes8<TYPE>(blk, g, q, 0), whi = kq_codes8<TYPE>(blk, g, q, 1);
    if (!rv) wlo = whi = make_uint2(0u, 0u);
    const v4i Dlo = mfma_i8(alo, wlo), Dhi = mfma_i8(ahi, whi);
    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
    int sclo, mlo, schi, mhi;
    kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g, sclo, mlo);
    kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g + 1, schi, mhi);
    const double d = (double)f16_to_f32(hdr.x);
    const double dmin = (double)f16_to_f32(hdr.x >> 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double t1 = d * (double)sclo * (double)slo[i].x * (double)Dlo[i];
      const double t2 = dmin * (double)mlo * (double)slo[i].y;
      const double t3 = d * (double)schi * (double)shi[i].x * (double)Dhi[i];
      const double t4 = dmin * (double)mhi * (double)shi[i].y;
      v[mi][i] = ((t1 - t2) + t3) - t4;
    }
  }
}

// This wave's subtree: positions p0 .. p0+N-1 (N a power of two <= 16), each
// the sum of tasks p, p+64, ... < T in order (0 past T), met pairwise in a
// balanced tree.  out[mi][i] = the subtree's value for the lane's row and
// token i.  A runtime loop with the task inlined once (the unrolled form did
// not fit the instruction cache): the partial sums of the tree live in five
// named levels, position n merging the levels of its trailing one bits (left
// operand first), as the unrolled tree does.
template <int NM>
__device__ __forceinline__ void tree_set(double (&d)[NM][4], const double (&s)[NM][4]) {
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) d[mi][i] = s[mi][i];
}
template <int NM>
__device__ __forceinline__ void tree_merge(const double (&left)[NM][4], double (&v)[NM][4]) {
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[mi][i] = left[mi][i] + v[mi][i];
}
// LV: the number of tree levels held, log2(N) + 1 for the largest N the
// instance serves (levels past it are never live, so they take no registers)
template <int TYPE, int NM, int LV, class Codes, class DS>
__device__ __forceinline__ void i8_subtree(const uint8_t* const (&mats)[NM], long rb, int nr, int T, int p0, int N,
                                           Codes codes8, DS ds, double (&out)[NM][4]) {
  static_assert(LV >= 1 && LV <= 5, "up to 16 positions per wave");
  double s0[NM][4], s1[NM][4], s2[NM][4], s3[NM][4], s4[NM][4];
#pragma unroll 1
  for (int n = 0; n < N; ++n) {
    const int p = p0 + n;
    double v[NM][4];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[mi][i] = 0.0;
#pragma unroll 1
    for (int t = p; t < T; t += 64) {
      double w[NM][4];
      i8_task<TYPE, NM>(mats, rb, nr, t, codes8, ds, w);
      if (t == p) tree_set<NM>(v, w);
      else {
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[mi][i] += w[mi][i];
      }
    }
    const int tz = __builtin_ctz(~(unsigned)n);   // trailing one bits of n (wave-uniform)
    if (tz >= 1) tree_merge<NM>(s0, v);
    if constexpr (LV > 2) if (tz >= 2) tree_merge<NM>(s1, v);
    if constexpr (LV > 3) if (tz >= 3) tree_merge<NM>(s2, v);
    if constexpr (LV > 4) if (tz >= 4) tree_merge<NM>(s3, v);
    switch (tz) {
      case 0: tree_set<NM>(s0, v); break;
      case 1: if constexpr (LV > 1) tree_set<NM>(s1, v); break;
      case 2: if constexpr (LV > 2) tree_set<NM>(s2, v); break;
      case 3: if constexpr (LV > 3) tree_set<NM>(s3, v); break;
      default: if constexpr (LV > 4) tree_set<NM>(s4, v); break;
    }
  }
  // the root: the level of N's single bit
  switch (N) {
    case 1: tree_set<NM>(out, s0); break;
    case 2: if constexpr (LV > 1) tree_set<NM>(out, s1); break;
    case 4: if constexpr (LV > 2) tree_set<NM>(out, s2); break;
    case 8: if constexpr (LV > 3) tree_set<NM>(out, s3); break;
    default: if constexpr (LV > 4) tree_set<NM>(out, s4); break;
  }
}

// The block's rows (nr <= 16) of NM matrices against one tile of tokens:
// every wave computes its subtree, the four meet in LDS (buf: kBWaves * NM * 4
// * 64 doubles) and wave 0 returns true with the row values in out.
constexpr size_t kI8Lds = sizeof(double) * kBWaves * 2 * 4 * 64;
constexpr size_t kStageLdsMax = 160 * 1024;   // a CU's LDS
template <int TYPE, int NM, class Codes, class DS>
__device__ __forceinline__ bool i8_rows(const uint8_t* const (&mats)[NM], long rb, int nr, int T, Codes codes8, DS ds,
                                        double* buf, double (&out)[NM][4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int TP = 4;
  while (TP < T && TP < 64) TP <<= 1;
  const int N = TP / kBWaves, p0 = wave * N;
  double c[NM][4];
  // up to 8 positions per wave (rows of up to 2048 K-quant elements) hold
  // four tree levels; more take the fifth
  if (N <= 8) i8_subtree<TYPE, NM, 4>(mats, rb, nr, T, p0, N, codes8, ds, c);
  else i8_subtree<TYPE, NM, 5>(mats, rb, nr, T, p0, N, codes8, ds, c);
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[((wave * NM + mi) * 4 + i) * 64 + lane] = c[mi][i];
  __syncthreads();
  if (wave != 0) return false;
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double q0 = buf[((0 * NM + mi) * 4 + i) * 64 + lane], q1 = buf[((1 * NM + mi) * 4 + i) * 64 + lane];
      const double q2 = buf[((2 * NM + mi) * 4 + i) * 64 + lane], q3 = buf[((3 * NM + mi) * 4 + i) * 64 + lane];
      out[mi][i] = (q0 + q1) + (q2 + q3);
    }
  return true;
}

// ---------------------------------------------------------------- group kernels
struct BGroupArgs {
  const int* cnt;
  const int* moff;
  const int* members;
  const int* dlist;
  const int* nd;
  const int* blist;         // the experts with group_min or more tokens, increasing
  const int* nb;
  const float* xn;          // [n][H]
  const uint8_t* xq;        // [n][H/32] Q8_1
  const uint8_t* gate;      // routed [E][F] rows
  const uint8_t* up;
  const uint8_t* down;      // routed [E][H] rows of Kp
  const uint8_t* sgate;     // shared [Fs] rows
  const uint8_t* sup;
  const uint8_t* sdown;     // shared [H] rows of Kps
  float* h;                 // [n][k][F]
  float* hs;                // [n][Fs]
  float* y;                 // [n][k][H]
  float* ys;                // [n][H]
  int n, k, H, E, F, Fs, Kp, Kps, gmin, has_sg;
  int stage_gu, stage_dn;   // matrix-core groups: rows (and gate/up activations) staged in LDS
  int stage_dma;            // gate/up rows streamed into LDS by buffer->LDS loads (whole KiB per block)
};

// The group of a block, and the block's chunk of that group's rows.  The
// big-group grids are (group, chunk, tile of 16 tokens); the small-group
// grids are (chunk, group), so that a group's chunks are dispatched one after
// another.  Either way group 0 is the shared expert's (when there is one):
// its workgroups, the heaviest, start first instead of being dispatched last
// and finishing after everything else.  block_group() returns false if the
// block has no group.
struct Group {
  bool shared;
  int e, ne, mbase;
};
template <bool BIG>
__device__ __forceinline__ int block_chunk() { return BIG ? (int)blockIdx.y : (int)blockIdx.x; }
// (BIG: the groups of group_min or more tokens only, the compact list)
template <bool BIG>
__device__ __forceinline__ bool block_group(const BGroupArgs& a, Group& gp) {
  const int gi = BIG ? (int)blockIdx.x : (int)blockIdx.y;
  gp.shared = a.has_sg && gi == 0;
  if (gp.shared) {
    gp.e = -1;
    gp.ne = a.n;
    gp.mbase = 0;
    return true;
  }
  const int li = gi - a.has_sg;   // index into the expert list
  if (li >= (BIG ? a.nb[0] : a.nd[0])) return false;
  gp.e = BIG ? a.blist[li] : a.dlist[li];
  gp.ne = a.cnt[gp.e];
  gp.mbase = a.moff[gp.e];
  return true;
}
// member m of the group -> token t and slot s (shared: slot -1)
__device__ __forceinline__ void member(const BGroupArgs& a, const Group& gp, int m, int& t, int& s) {
  if (gp.shared) { t = m; s = -1; return; }
  const int p = a.members[gp.mbase + m];
  t = p / a.k;
  s = p - t * a.k;
}

// ---------------------------------------------------------------- integer rows for several tokens
// A small group's members share the expert's rows: each task's weights are
// read and decoded once and dotted with every member's Q8_1 activations.
// Each member's value is the single-token row_task value, summed in the same
// order (task t, t+64, ..., then the lane-group tree), so it is bit-identical
// to running the rows once per member.
constexpr int kBSmallPerWave = 4;                       // rows per wave, small groups
constexpr int kBSmallRows = kBSmallPerWave * kBWaves;   // rows per block, small groups (gate/up)
static_assert(kBRows % kBSmallRows == 0, "a big group's block spans whole small-group blocks");
constexpr int kBigSpan = kBRows / kBSmallRows;              // gate/up: small-group blocks per big-group block

// A task's weight side, decoded once for all the members that use it: the
// int8 codes of its two sub-blocks (Q4_K nibbles; Q5_K with the fifth bit
// added) or of its Q8_0 block, and the fp64 factors the single-token task
// multiplies by (d*sc and dmin*m per sub-block; d for Q8_0).  task_member()
// then gives exactly row_task()'s value for one member's activations.
template <int TYPE>
struct TaskW {
  uint32_t lo[8], hi[8];
  double s_lo, m_lo, s_hi, m_hi;
};
// a task's weight bytes as loaded: K-quant header (4 dwords) and 32 code
// bytes (8), Q5_K also its 32 bytes of fifth bits (8); Q8_0 the 9 dwords
// from the dword boundary at or below the block (the block sits at 34t)
template <int TYPE>
struct TaskRaw {
  uint32_t v[TYPE == MOE_TYPE_Q5_K ? 20 : (TYPE == MOE_TYPE_Q8_0 ? 9 : 12)];
};
template <int TYPE>
__device__ __forceinline__ void task_raw(const uint8_t* row, int t, TaskRaw<TYPE>& r) {
  if (TYPE == MOE_TYPE_Q8_0) {
    const uint32_t* base = reinterpret_cast<const uint32_t*>(row + ((34 * t) & ~3));
#pragma unroll
    for (int i = 0; i < 9; ++i) r.v[i] = base[i];
    return;
  }
  const int b = t >> 2, g = t & 3;
  const uint8_t* blk = row + (long)b * block_bytes(TYPE);
  const uint4* q = reinterpret_cast<const uint4*>(blk + (TYPE == MOE_TYPE_Q5_K ? 48 : 16) + 32 * g);
  const uint4 h = *reinterpret_cast<const uint4*>(blk), q0 = q[0], q1 = q[1];
  r.v[0] = h.x; r.v[1] = h.y; r.v[2] = h.z; r.v[3] = h.w;
  r.v[4] = q0.x; r.v[5] = q0.y; r.v[6] = q0.z; r.v[7] = q0.w;
  r.v[8] = q1.x; r.v[9] = q1.y; r.v[10] = q1.z; r.v[11] = q1.w;
  if (TYPE == MOE_TYPE_Q5_K) {
    const uint4* hq = reinterpret_cast<const uint4*>(blk + 16);
    const uint4 h0 = hq[0], h1 = hq[1];
    r.v[12] = h0.x; r.v[13] = h0.y; r.v[14] = h0.z; r.v[15] = h0.w;
    r.v[16] = h1.x; r.v[17] = h1.y; r.v[18] = h1.z; r.v[19] = h1.w;
  }
}
template <int TYPE>
__device__ __forceinline__ void task_decode(const TaskRaw<TYPE>& r, int t, TaskW<TYPE>& w) {
  if (TYPE == MOE_TYPE_Q8_0) {
    // d in the low or the high half of the first dword; the codes 2 bytes on
    const bool sh = (34 * t) & 2;
    w.s_lo = (double)f16_to_f32(sh ? (r.v[0] >> 16) : (r.v[0] & 0xffffu));
#pragma unroll
    for (int i = 0; i < 8; ++i) w.lo[i] = sh ? r.v[i + 1] : __builtin_amdgcn_alignbyte(r.v[i + 1], r.v[i], 2);
    return;
  }
  const int g = t & 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t qs = r.v[4 + i];
    w.lo[i] = qs & 0x0f0f0f0fu;
    w.hi[i] = (qs >> 4) & 0x0f0f0f0fu;
    if (TYPE == MOE_TYPE_Q5_K) {
      const uint32_t qh = r.v[12 + i];
      w.lo[i] |= ((qh >> (2 * g)) & 0x01010101u) << 4;
      w.hi[i] |= ((qh >> (2 * g + 1)) & 0x01010101u) << 4;
    }
  }
  int sclo, mlo, schi, mhi;
  kquant_scale_min(r.v[1], r.v[2], r.v[3], 2 * g, sclo, mlo);
  kquant_scale_min(r.v[1], r.v[2], r.v[3], 2 * g + 1, schi, mhi);
  const double d = (double)f16_to_f32(r.v[0]);
  const double dmin = (double)f16_to_f32(r.v[0] >> 16);
  w.s_lo = d * (double)sclo;
  w.m_lo = dmin * (double)mlo;
  w.s_hi = d * (double)schi;
  w.m_hi = dmin * (double)mhi;
}
template <int TYPE>
__device__ __forceinline__ double task_member(const TaskW<TYPE>& w, int t, const ActLds& act) {
  if (TYPE == MOE_TYPE_Q8_0) {
    uint32_t a[8];
    lds_load8(act.codes + 32 * t, a);
    return w.s_lo * (double)act.d[t] * (double)q8_block_dot(w.lo, a);
  }
  const int jlo = 8 * (t >> 2) + 2 * (t & 3);
  uint32_t alo[8], ahi[8];
  lds_load8(act.codes + 32 * jlo, alo);
  lds_load8(act.codes + 32 * (jlo + 1), ahi);
  int lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo[i & 1] = __builtin_amdgcn_sdot4((int)w.lo[i], (int)alo[i], lo[i & 1], false);
    hi[i & 1] = __builtin_amdgcn_sdot4((int)w.hi[i], (int)ahi[i], hi[i & 1], false);
  }
  const double t1 = w.s_lo * (double)act.d[jlo] * (double)(lo[0] + lo[1]);
  const double t2 = w.m_lo * (double)act.s[jlo];
  const double t3 = w.s_hi * (double)act.d[jlo + 1] * (double)(hi[0] + hi[1]);
  const double t4 = w.m_hi * (double)act.s[jlo + 1];
  return ((t1 - t2) + t3) - t4;
}

// Row values of nrows rows of one wave for each of ne members (lanes and
// lane-group sums as in rows_dot: TP lanes per row, lane position p holding
// tasks p, p+64, ...): out[r * ldo + m] = row r against member m.  The
// members go one at a time (a run-time loop) over the task words decoded
// once per row pass, so the registers do not grow with the group.  Member m's
// Q8_1 codes are at codes + m*K, its block scales at dq/sq + m*(K/32).
template <int TYPE, class RowFn>
__device__ __forceinline__ void rows_dot_members(int nrows, int T, RowFn rowfn, const uint8_t* codes, const float* dq,
                                                 const float* sq, int K, int ne, double* out, int ldo) {
  int TP = 1;
  while (TP < T && TP < 64) TP <<= 1;
  const int rpi = 64 / TP;
  const int lane = threadIdx.x & 63;
  const int rl = lane / TP, t0 = lane - rl * TP;
  const int tt = (t0 < T) ? t0 : 0;
  const int nbk = K / 32;
  if (T <= 64) {   // one task per lane and row; the next pass's words load while this one computes
    auto row_of = [&](int r0) {
      const int ra = r0 + rl;
      return rowfn(ra < nrows ? ra : nrows - 1);
    };
    TaskRaw<TYPE> next;
    task_raw<TYPE>(row_of(0), tt, next);
    for (int r0 = 0; r0 < nrows; r0 += rpi) {
      const int ra = r0 + rl;
      const TaskRaw<TYPE> cur = next;
      if (r0 + rpi < nrows) task_raw<TYPE>(row_of(r0 + rpi), tt, next);
      TaskW<TYPE> w;
      task_decode<TYPE>(cur, tt, w);
#pragma unroll 1
      for (int m = 0; m < ne; ++m) {
        const ActLds act{codes + (long)m * K, dq + m * nbk, sq + m * nbk};
        double v = task_member<TYPE>(w, tt, act);
        if (t0 >= T) v = 0.0;
        v = group_sum_f64(v, TP);
        if (t0 == 0 && ra < nrows) out[ra * ldo + m] = v;
      }
    }
    return;
  }
  for (int r0 = 0; r0 < nrows; r0 += rpi) {
    const int ra = r0 + rl;
    const uint8_t* row = rowfn(ra < nrows ? ra : nrows - 1);
    {                // tasks t0, t0 + 64, ... summed in that order
#pragma unroll 1
      for (int m = 0; m < ne; ++m) {
        const ActLds act{codes + (long)m * K, dq + m * nbk, sq + m * nbk};
        double v = row_task<TYPE>(row, t0, act);
        for (int t = t0 + 64; t < T; t += 64) v += row_task<TYPE>(row, t, act);
        v = group_sum_f64(v, TP);
        if (t0 == 0 && ra < nrows) out[ra * ldo + m] = v;
      }
    }
  }
}

// bytes (a multiple of 16, 16-byte aligned both sides) from global to LDS by the block
__device__ __forceinline__ void copy_to_lds(uint8_t* dst, const uint8_t* src, long bytes) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (long i = threadIdx.x; i < (bytes >> 4); i += kBThreads) d4[i] = s4[i];
}

// `bytes` from global src straight into LDS dst by all waves of the block (the
// block waits with wait_vmem() and a barrier; dst needs room up to the next KiB)
__device__ __forceinline__ void dma_to_lds(uint8_t* dst, const uint8_t* src, uint32_t bytes) {
  stage_async(dst, src, bytes, threadIdx.x >> 6, 0, kBThreads / 64);
}

// Q8_1 activations of `nt` tokens unpacked into LDS (codes [nt][K], d/s [nt][K/32])
__device__ __forceinline__ void stage_xq(const uint8_t* xq_all, const int* toks, int nt, int K, uint8_t* codes,
                                         float* dq, float* sq) {
  const int nb = K / 32;
  for (int i = threadIdx.x; i < nt * nb; i += kBThreads) {
    const int j = i / nb, blk = i - j * nb;
    const uint8_t* src = xq_all + ((long)toks[j] * nb + blk) * kQ81Bytes;
    const uint32_t ds = *reinterpret_cast<const uint16_t*>(src) | ((uint32_t)reinterpret_cast<const uint16_t*>(src)[1] << 16);
    dq[j * nb + blk] = f16_to_f32(ds);
    sq[j * nb + blk] = f16_to_f32(ds >> 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (long)j * K + 32 * blk);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint8_t* c = src + 4 + 4 * w;
      dst[w] = (uint32_t)c[0] | ((uint32_t)c[1] << 8) | ((uint32_t)c[2] << 16) | ((uint32_t)c[3] << 24);
    }
  }
}

// gate/up + SwiGLU of one group, kBSmallRows (16) rows per block
// (BIG: the instance for groups of group_min or more tokens; the other
// instance takes the smaller groups, so each keeps its own register budget)
template <int ST, bool BIG>
__global__ __launch_bounds__(kBThreads) void k_bgu(BGroupArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Group gp;
  if (!block_group<BIG>(a, gp)) return;
  const int Fx = gp.shared ? a.Fs : a.F;
  const bool big = gp.ne >= a.gmin;
  if (big != BIG) return;
  // the chunk counts kBSmallRows-row chunks: a small group's block takes
  // one (kBSmallPerWave rows per wave); a big group's block takes kBigSpan
  // of them, kBRows rows whose K its waves split (the other blocks of its
  // span leave at once)
  if (big && (block_chunk<BIG>() % kBigSpan)) return;
  const int fb = block_chunk<BIG>() * kBSmallRows;
  if (fb >= Fx) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H;
  if constexpr (BIG) {
    // int8 matrix cores; blockIdx.z picks the tile of 16 tokens
    const int f0 = fb;
    const int nr = min(kBRows, Fx - f0);
    const int nb = H / 32;
    const long act_slot = (nb * kQ81Bytes + 1023) & ~1023L;   // a staged token's Q8_1 row, KiB-aligned
    double* buf = reinterpret_cast<double*>(smem);
    const int j = blockIdx.z;
    if (16 * j >= gp.ne) return;
    {
      const long rbw = gp.shared ? row_bytes(ST, H) : row_bytes(MOE_TYPE_Q4_K, H);
      const uint8_t* src0 = gp.shared ? a.sgate + f0 * rbw : a.gate + ((long)gp.e * a.F + f0) * rbw;
      const uint8_t* src1 = gp.shared ? a.sup + f0 * rbw : a.up + ((long)gp.e * a.F + f0) * rbw;
      const uint8_t* w0 = src0;
      const uint8_t* w1 = src1;
      const int nm = min(16, gp.ne - 16 * j);   // tokens of this tile
      __shared__ int s_tok[16];                  // token of tile position c
      if ((int)threadIdx.x < nm) {
        int tc, sc_;
        member(a, gp, 16 * j + (int)threadIdx.x, tc, sc_);
        s_tok[threadIdx.x] = tc;
      }
      const uint8_t* xq0 = a.xq;   // tile token c's blocks at xq0 + tokoff(c)
      bool staged = false;
      if (a.stage_gu) {
        // one bulk load of the block's rows and the tile's activations, so
        // the task loop reads LDS instead of waiting on memory per task
        uint8_t* wst = smem + kI8Lds;
        uint8_t* xst = wst + 2L * kBRows * rbw;
        if (a.stage_dma) {
          // the rows stream in, the activations behind them
          dma_to_lds(wst, src0, (uint32_t)(nr * rbw));
          dma_to_lds(wst + kBRows * rbw, src1, (uint32_t)(nr * rbw));
        } else {
          copy_to_lds(wst, src0, nr * rbw);
          copy_to_lds(wst + kBRows * rbw, src1, nr * rbw);
        }
        __syncthreads();   // s_tok
        // the tile's activations streamed the same way, token c's Q8_1 row
        // into its own KiB-aligned slot (the DMA pads each row to whole KiB)
        for (int c = 0; c < nm; ++c)
          dma_to_lds(xst + (long)c * act_slot, a.xq + (long)s_tok[c] * nb * kQ81Bytes, (uint32_t)(nb * kQ81Bytes));
        wait_vmem();
        w0 = wst;
        w1 = wst + kBRows * rbw;
        xq0 = xst;
        staged = true;
      }
      __syncthreads();
      auto tokoff = [&](int c) -> long { return staged ? (long)c * act_slot : (long)s_tok[c] * nb * kQ81Bytes; };
      const int cl = lane & 15;
      const bool mv = cl < nm;
      const uint8_t* xqt = xq0 + (mv ? tokoff(cl) : 0);
      auto codes8 = [&](int blk, int q) -> uint2 {
        if (!mv) return make_uint2(0u, 0u);
        const uint32_t* c = reinterpret_cast<const uint32_t*>(xqt + (long)blk * kQ81Bytes + 4 + 8 * q);
        return make_uint2(c[0], c[1]);
      };
      auto ds = [&](int c, int blk) -> float2 {
        if (c >= nm) return make_float2(0.f, 0.f);
        const uint32_t w = *reinterpret_cast<const uint32_t*>(xq0 + tokoff(c) + (long)blk * kQ81Bytes);
        return make_float2(f16_to_f32(w), f16_to_f32(w >> 16));
      };
      double gu[2][4];
      bool first;
      const uint8_t* const mats[2] = {w0, w1};
      if (gp.shared) first = i8_rows<ST, 2>(mats, rbw, nr, tasks_per_row(ST, H), codes8, ds, buf, gu);
      else first = i8_rows<MOE_TYPE_Q4_K, 2>(mats, rbw, nr, tasks_per_row(MOE_TYPE_Q4_K, H), codes8, ds, buf, gu);
      const int rr = lane & 15;   // the lane's row
      if (first && rr < nr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * (lane >> 4) + i;   // the lane's tokens
          if (c >= nm) continue;
          int t, s;
          member(a, gp, 16 * j + c, t, s);
          const float g = (float)gu[0][i], u = (float)gu[1][i];
          const float hv = (float)(silu_f64((double)g) * (double)u);
          if (gp.shared) a.hs[(long)t * a.Fs + f0 + rr] = hv;
          else a.h[((long)t * a.k + s) * a.F + f0 + rr] = hv;
        }
      }
    }
    return;
  }
  // a small group: the integer path, kBSmallPerWave rows of gate and up per
  // wave, all members at once
  int* toks = reinterpret_cast<int*>(smem);
  int* slots = toks + MOE_MAX_BATCH;
  uint8_t* codes = smem + 2 * sizeof(int) * MOE_MAX_BATCH;
  float* dq = reinterpret_cast<float*>(codes + (long)gp.ne * H);
  float* sq = dq + gp.ne * (H / 32);
  double* part = reinterpret_cast<double*>(smem + ((2 * sizeof(int) * MOE_MAX_BATCH + (long)gp.ne * H +
                                                    8L * gp.ne * (H / 32) + 15) & ~15L));
  for (int m = threadIdx.x; m < gp.ne; m += kBThreads) {
    int t, s;
    member(a, gp, m, t, s);
    toks[m] = t;
    slots[m] = s;
  }
  __syncthreads();
  stage_xq(a.xq, toks, gp.ne, H, codes, dq, sq);
  __syncthreads();
  const int fs = fb + wave * kBSmallPerWave;
  const int ns = max(0, min(kBSmallPerWave, Fx - fs));
  if (ns == 0) return;
  const int ne = gp.ne;
  double* pw = part + (long)wave * 2 * kBSmallPerWave * ne;   // [2 ns rows][ne]
  if (gp.shared) {
    const long rb = row_bytes(ST, H);
    rows_dot_members<ST>(2 * ns, tasks_per_row(ST, H), [&](int r) {
      return (r < ns) ? a.sgate + (fs + r) * rb : a.sup + (fs + r - ns) * rb;
    }, codes, dq, sq, H, ne, pw, ne);
  } else {
    const long rb = row_bytes(MOE_TYPE_Q4_K, H);
    const long base = ((long)gp.e * a.F + fs) * rb;
    rows_dot_members<MOE_TYPE_Q4_K>(2 * ns, tasks_per_row(MOE_TYPE_Q4_K, H), [&](int r) {
      return (r < ns) ? a.gate + base + r * rb : a.up + base + (r - ns) * rb;
    }, codes, dq, sq, H, ne, pw, ne);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  for (int o = lane; o < ns * ne; o += 64) {
    const int r = o / ne, m = o - r * ne;
    const float g = (float)pw[r * ne + m], u = (float)pw[(ns + r) * ne + m];
    const float hv = (float)(silu_f64((double)g) * (double)u);
    if (gp.shared) a.hs[(long)toks[m] * a.Fs + fs + r] = hv;
    else a.h[((long)toks[m] * a.k + slots[m]) * a.F + fs + r] = hv;
  }
}

// down rows of one group: 64 output rows per block for a small group, 16 for a
// big one (the chunk counts 16-row units)
template <int DT, int ST, bool BIG>
__global__ __launch_bounds__(kBThreads) void k_bdn(BGroupArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Group gp;
  if (!block_group<BIG>(a, gp)) return;
  const int H = a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool big = gp.ne >= a.gmin;
  if (big != BIG) return;
  // the chunk: a big group's block takes kBRows rows (its waves split K), a
  // small group's block kBRowsPerBlock rows (kBRows per wave)
  const int i0 = BIG ? block_chunk<BIG>() * kBRows : block_chunk<BIG>() * kBRowsPerBlock + wave * kBRows;
  if (big && i0 >= H) return;
  const int nr = max(0, min(kBRows, H - i0));
  const int Fx = gp.shared ? a.Fs : a.F;
  const int Kx = gp.shared ? a.Kps : a.Kp;
  auto hsrc = [&](int m) {
    int t, s;
    member(a, gp, m, t, s);
    return gp.shared ? a.hs + (long)t * a.Fs : a.h + ((long)t * a.k + s) * a.F;
  };
  if constexpr (BIG) {
    // int8 matrix cores; blockIdx.z picks the tile of 16 tokens, whose h is
    // quantised to Q8_1 in LDS (as for a small group), then the rows
    const int nb = Kx / 32;
    double* buf = reinterpret_cast<double*>(smem);
    uint8_t* codes = smem + kI8Lds;
    float* dq = reinterpret_cast<float*>(codes + 16L * Kx);
    float* sq = dq + 16 * nb;
    const int j = blockIdx.z;
    if (16 * j >= gp.ne) return;
    {
      const int nm = min(16, gp.ne - 16 * j);
      quantize_q81_blocks<1>(nm * nb, [&](int jj) -> const float* {
        const int mm = jj / nb, blk = jj - mm * nb;
        return (blk * 32 < Fx) ? hsrc(16 * j + mm) + 32 * blk : nullptr;
      }, [&](int jj) { return codes + 32L * jj; }, dq, sq, threadIdx.x, kBThreads);
      __syncthreads();
      const int c = lane & 15;
      const bool mv = c < nm;
      auto codes8 = [&](int blk, int q) -> uint2 {
        if (!mv) return make_uint2(0u, 0u);
        return *reinterpret_cast<const uint2*>(codes + (long)c * Kx + 32 * blk + 8 * q);
      };
      auto ds = [&](int c2, int blk) -> float2 {
        if (c2 >= nm) return make_float2(0.f, 0.f);
        return make_float2(dq[c2 * nb + blk], sq[c2 * nb + blk]);
      };
      double yv[1][4];
      bool first;
      const long rb = gp.shared ? row_bytes(ST, Kx) : row_bytes(DT, Kx);
      const uint8_t* src = gp.shared ? a.sdown + i0 * rb : a.down + ((long)gp.e * H + i0) * rb;
      const uint8_t* w0 = src;
      if (a.stage_dn) {   // the rows staged after the tile's codes (already behind a barrier)
        uint8_t* wst = reinterpret_cast<uint8_t*>(sq + 16 * nb);
        copy_to_lds(wst, src, nr * rb);
        __syncthreads();
        w0 = wst;
      }
      const uint8_t* const mats[1] = {w0};
      if (gp.shared) first = i8_rows<ST, 1>(mats, rb, nr, tasks_per_row(ST, Kx), codes8, ds, buf, yv);
      else first = i8_rows<DT, 1>(mats, rb, nr, tasks_per_row(DT, Kx), codes8, ds, buf, yv);
      const int rr = lane & 15;   // the lane's row
      if (first && rr < nr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c2 = 4 * (lane >> 4) + i;   // the lane's tokens
          if (c2 >= nm) continue;
          int t, s;
          member(a, gp, 16 * j + c2, t, s);
          if (gp.shared) a.ys[(long)t * H + i0 + rr] = (float)yv[0][i];
          else a.y[((long)t * a.k + s) * H + i0 + rr] = (float)yv[0][i];
        }
      }
    }
    return;
  }
  // small group: quantise each member's h to Q8_1 in LDS, then the integer rows
  const int nb = Kx / 32;
  int* toks = reinterpret_cast<int*>(smem);
  int* slots = toks + MOE_MAX_BATCH;
  uint8_t* codes = smem + 2 * sizeof(int) * MOE_MAX_BATCH;
  float* dq = reinterpret_cast<float*>(codes + (long)gp.ne * Kx);
  float* sq = dq + gp.ne * nb;
  double* part = reinterpret_cast<double*>(smem + ((2 * sizeof(int) * MOE_MAX_BATCH + (long)gp.ne * Kx +
                                                    8L * gp.ne * nb + 15) & ~15L));
  for (int m = threadIdx.x; m < gp.ne; m += kBThreads) {
    int t, s;
    member(a, gp, m, t, s);
    toks[m] = t;
    slots[m] = s;
  }
  __syncthreads();
  quantize_q81_blocks<1>(gp.ne * nb, [&](int j) -> const float* {
    const int m = j / nb, blk = j - m * nb;
    return (blk * 32 < Fx) ? hsrc(m) + 32 * blk : nullptr;
  }, [&](int j) { return codes + 32L * j; }, dq, sq, threadIdx.x, kBThreads);
  __syncthreads();
  if (nr == 0) return;
  const int ne = gp.ne;
  double* pw = part + (long)wave * kBRows * ne;   // [nr rows][ne]
  if (gp.shared) {
    const long rb = row_bytes(ST, Kx);
    rows_dot_members<ST>(nr, tasks_per_row(ST, Kx), [&](int r) { return a.sdown + (i0 + r) * rb; }, codes, dq, sq,
                         Kx, ne, pw, ne);
  } else {
    const long rb = row_bytes(DT, Kx);
    const uint8_t* base = a.down + ((long)gp.e * H + i0) * rb;
    rows_dot_members<DT>(nr, tasks_per_row(DT, Kx), [&](int r) { return base + r * rb; }, codes, dq, sq, Kx, ne, pw,
                         ne);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  for (int o = lane; o < nr * ne; o += 64) {
    const int r = o / ne, m = o - r * ne;
    const float yv = (float)pw[r * ne + m];
    if (gp.shared) a.ys[(long)toks[m] * H + i0 + r] = yv;
    else a.y[((long)toks[m] * a.k + slots[m]) * H + i0 + r] = yv;
  }
}

// routed = bf16(sum_s w_s y_s) in slot order; shared = bf16(gate * ys); NaN on bad ids
__global__ __launch_bounds__(256) void k_bcombine(const float* y, const float* ys, const float* wts, const float* sg,
                                                  const int* err, int k, int H, int has_sg, uint16_t* routed,
                                                  uint16_t* shared) {
  const int t = blockIdx.x;
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= H) return;
  if (err[0]) {
    routed[(long)t * H + i] = 0x7fc0u;
    if (has_sg) shared[(long)t * H + i] = 0x7fc0u;
    return;
  }
  double acc = 0.0;
  for (int s = 0; s < k; ++s) acc += (double)wts[(long)t * k + s] * (double)y[((long)t * k + s) * H + i];
  routed[(long)t * H + i] = f32_to_bf16((float)acc);
  if (has_sg) shared[(long)t * H + i] = f32_to_bf16((float)((double)sg[t] * (double)ys[(long)t * H + i]));
}

// ---------------------------------------------------------------- host side
static inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

BatchWs batch_ws_layout(const moe_layer_desc* d, int n) {
  BatchWs L;
  const int H = d->hidden, E = d->n_experts, k = d->top_k, F = d->ffn, Fs = d->shared_ffn;
  size_t o = 0;
  L.router = o; o += up256(sizeof(unsigned) * kCounterSlots) + up256(sizeof(float) * (size_t)n * (E + 1));
  L.cnt = o; o += up256(sizeof(int) * E);
  L.moff = o; o += up256(sizeof(int) * E);
  L.members = o; o += up256(sizeof(int) * (size_t)n * k);
  L.dlist = o; o += up256(sizeof(int) * E);
  L.nd = o; o += 256;
  L.blist = o; o += up256(sizeof(int) * E);
  L.nb = o; o += 256;
  L.err = o; o += 256;
  L.xn = o; o += up256(sizeof(float) * (size_t)n * H);
  L.xq = o; o += up256((size_t)n * (H / 32) * kQ81Bytes);
  L.ids = o; o += up256(sizeof(int32_t) * (size_t)n * k);
  L.wts = o; o += up256(sizeof(float) * (size_t)n * k);
  L.sg = o; o += up256(sizeof(float) * (size_t)n);
  L.h = o; o += up256(sizeof(float) * (size_t)n * k * F);
  L.hs = o; o += up256(sizeof(float) * (size_t)n * (Fs > 0 ? Fs : 1));
  L.y = o; o += up256(sizeof(float) * (size_t)n * k * H);
  L.ys = o; o += up256(sizeof(float) * (size_t)n * H);
  L.total = o;
  return L;
}

// toks/slots, the members' Q8_1 codes and block scales, and each wave's row
// values of every member (kBRows rows: the down rows; gate/up use half)
static size_t int_path_lds(int ne_max, int K) {
  return 2 * sizeof(int) * MOE_MAX_BATCH + (size_t)ne_max * K + 8 * (size_t)ne_max * (K / 32) + 16 +
         sizeof(double) * (size_t)ne_max * kBRows * kBWaves;
}

// The matrix-core groups and the integer-path groups write disjoint rows of
// h, hs, y and ys, so their kernels can run side by side: the matrix-core
// chain (gate/up, then down) goes to a second stream of the device, forked
// from the caller's stream after the grouping and joined before the combine.
// One such stream and its two events per device, made on the first call that
// is not being captured into a graph (a captured call before that runs both
// chains on the caller's stream).  The fork and join of one call happen under
// a lock, so that calls from several host threads cannot interleave the
// events' records and waits; their matrix-core chains then queue on the one
// side stream in call order.
namespace {
constexpr int kMaxDevices = 64;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// the device's side stream, or null (caller holds g_side_mu).  A failed query
// here only means the call keeps to one stream: its error is cleared, so that
// the launch path's own error check does not report it.
SideStream* side_stream(hipStream_t st) {
  auto none = []() -> SideStream* {
    (void)hipGetLastError();
    return nullptr;
  };
  int dev = -1;
  if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return none();
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.s) return &ss;
  if (ss.failed) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return none();
  if (cs != hipStreamCaptureStatusNone) return nullptr;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return none();
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return none();
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool ok = hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
                  hipEventCreateWithFlags(&e0, hipEventDisableTiming) == hipSuccess &&
                  hipEventCreateWithFlags(&e1, hipEventDisableTiming) == hipSuccess;
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) {
    if (e1) (void)hipEventDestroy(e1);
    if (e0) (void)hipEventDestroy(e0);
    if (s) (void)hipStreamDestroy(s);
    ss.failed = true;
    (void)hipGetLastError();
    return nullptr;
  }
  ss.s = s;
  ss.fork = e0;
  ss.join = e1;
  return &ss;
}
}  // namespace

int launch_grouped_ffn(const moe_layer_desc* d, const moe_layer_weights* w, const float* xn, const void* xq,
                       const int32_t* ids, const float* wts, const float* sg, int n, int gmin, uint16_t* routed,
                       uint16_t* shared, float* h, float* hs, uint8_t* ws, const BatchWs& L, hipStream_t st) {
  const int H = d->hidden, E = d->n_experts, k = d->top_k, F = d->ffn, Fs = d->shared_ffn;
  const int has_sg = Fs > 0;
  const int st_type = has_sg ? d->shared_type : MOE_TYPE_Q4_K;
  BGroupArgs a;
  a.cnt = reinterpret_cast<const int*>(ws + L.cnt);
  a.moff = reinterpret_cast<const int*>(ws + L.moff);
  a.members = reinterpret_cast<const int*>(ws + L.members);
  a.dlist = reinterpret_cast<const int*>(ws + L.dlist);
  a.nd = reinterpret_cast<const int*>(ws + L.nd);
  a.blist = reinterpret_cast<const int*>(ws + L.blist);
  a.nb = reinterpret_cast<const int*>(ws + L.nb);
  a.xn = xn;
  a.xq = static_cast<const uint8_t*>(xq);
  a.gate = static_cast<const uint8_t*>(w->gate);
  a.up = static_cast<const uint8_t*>(w->up);
  a.down = static_cast<const uint8_t*>(w->down);
  a.sgate = static_cast<const uint8_t*>(w->shared_gate);
  a.sup = static_cast<const uint8_t*>(w->shared_up);
  a.sdown = static_cast<const uint8_t*>(w->shared_down);
  a.h = h;
  a.hs = hs;
  a.y = reinterpret_cast<float*>(ws + L.y);
  a.ys = reinterpret_cast<float*>(ws + L.ys);
  a.n = n;
  a.k = k;
  a.H = H;
  a.E = E;
  a.F = F;
  a.Fs = Fs;
  a.Kp = pad_k(d->down_type, F);
  a.Kps = has_sg ? pad_k(st_type, Fs) : 0;
  a.gmin = gmin;
  a.has_sg = has_sg;
  a.stage_gu = a.stage_dn = a.stage_dma = 0;
  hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, st, ids, n, k, E, gmin, reinterpret_cast<int*>(ws + L.cnt),
                     reinterpret_cast<int*>(ws + L.moff), reinterpret_cast<int*>(ws + L.members),
                     reinterpret_cast<int*>(ws + L.dlist), reinterpret_cast<int*>(ws + L.nd),
                     reinterpret_cast<int*>(ws + L.blist), reinterpret_cast<int*>(ws + L.nb),
                     reinterpret_cast<int*>(ws + L.err));
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  // groups: at most min(E, n*k) distinct experts, plus the shared group
  const int ngroups = min(E, n * k) + has_sg;
  // groups of group_min or more tokens: at most n*k / group_min experts, plus the shared group
  const int ngroups_big = min(E, n * k / gmin) + has_sg;
  const int small = gmin - 1;   // largest group on the integer path
  const int fmax = max(F, Fs);
  const int ggu_chunks = (fmax + kBSmallRows - 1) / kBSmallRows;
  const dim3 ggu(ggu_chunks, ngroups);   // small groups: (chunk, group)
  const bool any_big = gmin <= n;   // a group (at least the shared one when n >= gmin) can reach group_min
  const size_t lds_gu = small > 0 ? int_path_lds(small > n ? n : small, H) : 0;
  // matrix-core groups stage their rows (and gate/up activations) in LDS when they fit
  const long rbw_max = std::max(row_bytes(MOE_TYPE_Q4_K, H), has_sg ? row_bytes(st_type, H) : 0L);
  const size_t gu_stage = 2 * kBRows * (size_t)rbw_max + 16 * (((size_t)(H / 32) * kQ81Bytes + 1023) & ~(size_t)1023);
  a.stage_gu = kI8Lds + gu_stage <= kStageLdsMax && (reinterpret_cast<uintptr_t>(xq) & 15) == 0;
  const size_t lds_gu_big = kI8Lds + (a.stage_gu ? gu_stage : 0);
  // streamed rows write whole KiB chunks: a block of kBRows rows must end on
  // a KiB boundary so a short block's zero padding stays inside its own area
  a.stage_dma = a.stage_gu && (kBRows * row_bytes(MOE_TYPE_Q4_K, H)) % 1024 == 0 &&
                (!has_sg || (kBRows * row_bytes(st_type, H)) % 1024 == 0);
  void* args[] = {&a};
  const bool q80 = st_type == MOE_TYPE_Q8_0;
  const void* fgs = q80 ? (const void*)k_bgu<MOE_TYPE_Q8_0, false> : (const void*)k_bgu<MOE_TYPE_Q4_K, false>;
  const void* fgb = q80 ? (const void*)k_bgu<MOE_TYPE_Q8_0, true> : (const void*)k_bgu<MOE_TYPE_Q4_K, true>;
  // x: the groups of group_min or more tokens (the compact list, as for
  // down), z: tiles of 16 tokens.  A grid over every group spent most of
  // the kernel dispatching workgroups that leave at once, one per CU at
  // this instance's LDS size
  const dim3 ggu_big(ngroups_big, ggu_chunks, (n + 15) / 16);
  const int kmax = max(a.Kp, a.Kps);
  const dim3 gdn(ngroups, (H + kBRows - 1) / kBRows);
  const size_t lds_dn = small > 0 ? int_path_lds(small > n ? n : small, kmax) : 0;
  size_t lds_dn_big = kI8Lds + 16 * (size_t)kmax + 2 * sizeof(float) * 16 * (size_t)(kmax / 32);
  const long rbd_max = std::max(row_bytes(d->down_type, a.Kp), has_sg ? row_bytes(st_type, a.Kps) : 0L);
  a.stage_dn = lds_dn_big + kBRows * (size_t)rbd_max <= kStageLdsMax;
  if (a.stage_dn) lds_dn_big += kBRows * (size_t)rbd_max;
  const void* fds;
  const void* fdb;
  if (d->down_type == MOE_TYPE_Q5_K) {
    fds = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bdn<MOE_TYPE_Q5_K, MOE_TYPE_Q8_0, false>
                                     : (const void*)k_bdn<MOE_TYPE_Q5_K, MOE_TYPE_Q4_K, false>;
    fdb = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bdn<MOE_TYPE_Q5_K, MOE_TYPE_Q8_0, true>
                                     : (const void*)k_bdn<MOE_TYPE_Q5_K, MOE_TYPE_Q4_K, true>;
  } else {
    fds = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bdn<MOE_TYPE_Q4_K, MOE_TYPE_Q8_0, false>
                                     : (const void*)k_bdn<MOE_TYPE_Q4_K, MOE_TYPE_Q4_K, false>;
    fdb = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bdn<MOE_TYPE_Q4_K, MOE_TYPE_Q8_0, true>
                                     : (const void*)k_bdn<MOE_TYPE_Q4_K, MOE_TYPE_Q4_K, true>;
  }
  const dim3 gdn_small((H + kBRowsPerBlock - 1) / kBRowsPerBlock, ngroups);   // (chunk, group)
  const dim3 gdn_big(ngroups_big, gdn.y, (n + 15) / 16);   // z: tiles of 16 tokens
  if ((small > 0 && (hipFuncSetAttribute(fgs, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_gu) != hipSuccess ||
                     hipFuncSetAttribute(fds, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dn) != hipSuccess)) ||
      (any_big && (hipFuncSetAttribute(fgb, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_gu_big) != hipSuccess ||
                   hipFuncSetAttribute(fdb, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dn_big) != hipSuccess)))
    return MOE_ERR_HIP;
  {
    std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
    SideStream* side = nullptr;
    if (small > 0 && any_big) {
      lock.lock();
      side = side_stream(st);
      if (!side) lock.unlock();
    }
    hipStream_t sb = st;   // the matrix-core chain's stream
    if (side) {
      if (hipEventRecord(side->fork, st) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
        return MOE_ERR_HIP;
      sb = side->s;
    }
    // the matrix-core chain first: its workgroups run longest
    int rc = MOE_OK;
    if (any_big && (hipLaunchKernel(fgb, ggu_big, dim3(kBThreads), args, lds_gu_big, sb) != hipSuccess ||
                    hipLaunchKernel(fdb, gdn_big, dim3(kBThreads), args, lds_dn_big, sb) != hipSuccess))
      rc = MOE_ERR_HIP;
    if (rc == MOE_OK && small > 0 &&
        (hipLaunchKernel(fgs, ggu, dim3(kBThreads), args, lds_gu, st) != hipSuccess ||
         hipLaunchKernel(fds, gdn_small, dim3(kBThreads), args, lds_dn, st) != hipSuccess))
      rc = MOE_ERR_HIP;
    // joined even after a failed launch, so that a capture is not left forked
    if (side && (hipEventRecord(side->join, sb) != hipSuccess || hipStreamWaitEvent(st, side->join, 0) != hipSuccess))
      rc = MOE_ERR_HIP;
    if (rc) return rc;
  }
  hipLaunchKernelGGL(k_bcombine, dim3(n, (H + 255) / 256), dim3(256), 0, st, a.y, a.ys, wts, sg,
                     reinterpret_cast<const int*>(ws + L.err), k, H, has_sg, routed, shared);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
