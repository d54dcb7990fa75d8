// moe_batch.hip -- several tokens at once: experts grouped by the tokens that
// selected them.
//
// A group (the tokens whose top-k contains expert e) with at least group_min
// tokens reads its expert's rows once and multiplies them on the matrix cores:
// weights decoded to f32 then rounded to bf16, activations bf16(xn) and
// bf16(h), fp32 accumulation (v_mfma_f32_16x16x32_bf16).  A smaller group
// takes the integer Q8_1 x v_dot4 path of the single-token stage for each of
// its tokens.  The shared expert is one group of all the tokens.  Norm, router
// and top-k run per token as at batch 1; the combine is per token in slot
// order.  The pages cover batch 1 only ([P359] Summary: the Q8_1 integer dot
// path); the grouping reading is stated with the oracle's grouped path.
//
// MFMA operand layout (16x16x32 bf16, checked on gfx950): lane l holds row
// l%16 of A and column l%16 of B at k = 8*(l/16) .. +7, and rows 4*(l/16) .. +3
// of column l%16 of D.  The k order inside a 64-element group is permuted the
// same way for both operands (lane group q takes elements 8q..8q+7 of the
// group's first half -- the low nibbles of bytes 8q..8q+7 of a K-quant group
// -- in one step and of its second half, the high nibbles, in the next), which
// leaves the dot product unchanged and lets each lane decode 8 contiguous
// bytes.
#include <algorithm>

#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBThreads = 256;
constexpr int kBWaves = kBThreads / 64;
constexpr int kBRows = 16;                   // rows per wave
constexpr int kBRowsPerBlock = kBRows * kBWaves;
constexpr int kMaxTiles = MOE_MAX_BATCH / 16;

// ---------------------------------------------------------------- grouping
__device__ __forceinline__ int block_excl_scan(int v, int* tmp) {
  // Hillis-Steele over blockDim.x (a power of two) values in LDS
  const int tid = threadIdx.x, n = blockDim.x;
  tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < n; o <<= 1) {
    const int add = (tid >= o) ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int incl = tmp[tid];
  __syncthreads();
  return incl - v;
}

// ids [n][k] -> cnt[e] tokens per expert, moff[e] first member, members (p = t*k + s,
// token order within an expert), dlist = the experts with cnt > 0 in increasing
// order, nd[0] = their number, err[0] = 1 if an id is outside [0, E).
__global__ __launch_bounds__(1024) void k_group(const int32_t* ids, int n, int k, int E, int* cnt, int* moff,
                                                int* members, int* dlist, int* nd, int* err) {
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int tmp[1024];
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
  const int off = block_excl_scan(c, tmp);
  const int pos = block_excl_scan(c > 0 ? 1 : 0, tmp);
  if (tid < E) {
    s_off[tid] = off;
    cnt[tid] = c;
    moff[tid] = off;
    if (c > 0) dlist[pos] = tid;
  }
  if (tid == 1023) nd[0] = pos + (c > 0 ? 1 : 0);
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

// ---------------------------------------------------------------- bf16 operands
// 8 weights of one 64-element group gg of a row (lane group q): lo = elements
// 64gg + 8q .. +7, hi = 64gg + 32 + 8q .. +7, each f32(w) rounded to bf16.
template <int TYPE>
__device__ __forceinline__ void weights_bf16(const uint8_t* row, int gg, int q, v8s& lo, v8s& hi) {
  if (TYPE == MOE_TYPE_Q8_0) {
    // blocks 2gg and 2gg+1, elements 8q..8q+7 of each (34-byte blocks: 2-byte aligned)
    const uint8_t* b0 = row + 34L * (2 * gg);
    const uint8_t* b1 = b0 + 34;
    const uint16_t* p0 = reinterpret_cast<const uint16_t*>(b0);
    const uint16_t* p1 = reinterpret_cast<const uint16_t*>(b1);
    const float d0 = f16_to_f32(p0[0]), d1 = f16_to_f32(p1[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t c0 = p0[1 + 4 * q + i], c1 = p1[1 + 4 * q + i];
      lo[2 * i] = (short)f32_to_bf16(d0 * (float)(int8_t)(c0 & 0xff));
      lo[2 * i + 1] = (short)f32_to_bf16(d0 * (float)(int8_t)(c0 >> 8));
      hi[2 * i] = (short)f32_to_bf16(d1 * (float)(int8_t)(c1 & 0xff));
      hi[2 * i + 1] = (short)f32_to_bf16(d1 * (float)(int8_t)(c1 >> 8));
    }
    return;
  }
  const int b = gg >> 2, g = gg & 3;
  const uint8_t* blk = row + (long)b * block_bytes(TYPE);
  const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
  const int qs_off = (TYPE == MOE_TYPE_Q5_K) ? 48 : 16;
  const uint2 qs = *reinterpret_cast<const uint2*>(blk + qs_off + 32 * g + 8 * q);
  uint2 qh = make_uint2(0, 0);
  if (TYPE == MOE_TYPE_Q5_K) qh = *reinterpret_cast<const uint2*>(blk + 16 + 8 * q);
  int sclo, mlo, schi, mhi;
  kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g, sclo, mlo);
  kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g + 1, schi, mhi);
  const float d = f16_to_f32(hdr.x), dmin = f16_to_f32(hdr.x >> 16);
  // each product below is exact in fp32; the subtraction rounds once: f32(w)
  const float alo = d * (float)sclo, ahi = d * (float)schi;
  const float mlo_f = dmin * (float)mlo, mhi_f = dmin * (float)mhi;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t byte = ((i < 4 ? qs.x : qs.y) >> (8 * (i & 3))) & 0xffu;
    int ql = (int)(byte & 15u), qhv = (int)(byte >> 4);
    if (TYPE == MOE_TYPE_Q5_K) {
      const uint32_t hb = ((i < 4 ? qh.x : qh.y) >> (8 * (i & 3))) & 0xffu;
      ql |= (int)((hb >> (2 * g)) & 1u) << 4;
      qhv |= (int)((hb >> (2 * g + 1)) & 1u) << 4;
    }
    lo[i] = (short)f32_to_bf16(alo * (float)ql - mlo_f);
    hi[i] = (short)f32_to_bf16(ahi * (float)qhv - mhi_f);
  }
}

// 8 activations bf16(x[base .. base+8)) (zero past n, or for a missing token)
__device__ __forceinline__ v8s acts_bf16(const float* x, int base, int n) {
  v8s r;
  if (!x || base >= n) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = 0;
    return r;
  }
  const float4 a = *reinterpret_cast<const float4*>(x + base);
  const float4 b = *reinterpret_cast<const float4*>(x + base + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (base + i < n) ? (short)f32_to_bf16(v[i]) : (short)0;
  return r;
}

__device__ __forceinline__ v4f mfma_bf16(v8s a, v8s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// One wave: rows r0.. (nr <= 16 valid) of one or two matrices (rowsA, rowsB
// may be null) of TYPE with K elements, against the activations of up to
// MOE_MAX_BATCH members (act(m) -> fp32 pointer of K_act values, K_act <= K;
// elements past K_act are zero), over the 64-element groups gg0, gg0 + ggs,
// ... of K.  accA/accB [kMaxTiles] receive D tiles.
template <int TYPE, class Act>
__device__ __forceinline__ void wave_mfma(const uint8_t* rowsA, const uint8_t* rowsB, long rb, int nr, int K, int ne,
                                          int K_act, Act act, v4f* accA, v4f* accB, int gg0, int ggs) {
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int ntiles = (ne + 15) >> 4;
#pragma unroll
  for (int j = 0; j < kMaxTiles; ++j) {
    accA[j] = v4f{0.f, 0.f, 0.f, 0.f};
    accB[j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const bool rv = r < nr;
  const uint8_t* ra = rowsA + (long)(rv ? r : 0) * rb;
  const uint8_t* rbp = rowsB ? rowsB + (long)(rv ? r : 0) * rb : nullptr;
  for (int gg = gg0; gg < K / 64; gg += ggs) {   // K-quant rows: 4 groups per superblock
    v8s alo, ahi, blo, bhi;
    weights_bf16<TYPE>(ra, gg, q, alo, ahi);
    if (!rv) alo = ahi = v8s{0, 0, 0, 0, 0, 0, 0, 0};
    if (rbp) {
      weights_bf16<TYPE>(rbp, gg, q, blo, bhi);
      if (!rv) blo = bhi = v8s{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kMaxTiles; ++j) {
      if (j >= ntiles) break;
      const int m = 16 * j + r;   // this lane's column: member m
      const float* x = (m < ne) ? act(m) : nullptr;
      const v8s xlo = acts_bf16(x, 64 * gg + 8 * q, K_act);
      const v8s xhi = acts_bf16(x, 64 * gg + 32 + 8 * q, K_act);
      accA[j] = mfma_bf16(alo, xlo, accA[j]);
      accA[j] = mfma_bf16(ahi, xhi, accA[j]);
      if (rbp) {
        accB[j] = mfma_bf16(blo, xlo, accB[j]);
        accB[j] = mfma_bf16(bhi, xhi, accB[j]);
      }
    }
  }
}

// The kBWaves waves of a block hold partial tiles over disjoint K groups:
// wave 0 ends with their sums, added in wave order (buf: kBWaves * kMaxTiles
// * 2 * 64 v4f of LDS).  Every wave of the block must call it.
constexpr size_t kBigLds = sizeof(v4f) * kBWaves * kMaxTiles * 2 * 64;
__device__ __forceinline__ void reduce_waves(v4f* accA, v4f* accB, int ntiles, bool two, v4f* buf) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kMaxTiles; ++j) {
    if (j < ntiles) {
      buf[((wave * kMaxTiles + j) * 2 + 0) * 64 + lane] = accA[j];
      if (two) buf[((wave * kMaxTiles + j) * 2 + 1) * 64 + lane] = accB[j];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < kMaxTiles; ++j) {
    if (j < ntiles) {
      v4f sa = buf[(j * 2 + 0) * 64 + lane], sb = v4f{0.f, 0.f, 0.f, 0.f};
      if (two) sb = buf[(j * 2 + 1) * 64 + lane];
      for (int w = 1; w < kBWaves; ++w) {
        sa += buf[((w * kMaxTiles + j) * 2 + 0) * 64 + lane];
        if (two) sb += buf[((w * kMaxTiles + j) * 2 + 1) * 64 + lane];
      }
      accA[j] = sa;
      accB[j] = sb;
    }
  }
}

// ---------------------------------------------------------------- group kernels
struct BGroupArgs {
  const int* cnt;
  const int* moff;
  const int* members;
  const int* dlist;
  const int* nd;
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
};

// the group of blockIdx.x: returns false if this block has no group
struct Group {
  bool shared;
  int e, ne, mbase;
};
__device__ __forceinline__ bool block_group(const BGroupArgs& a, Group& gp) {
  const int gi = blockIdx.x;
  gp.shared = a.has_sg && gi == (int)gridDim.x - 1;
  if (gp.shared) {
    gp.e = -1;
    gp.ne = a.n;
    gp.mbase = 0;
    return true;
  }
  if (gi >= a.nd[0]) return false;
  gp.e = a.dlist[gi];
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
// read once and dotted with up to kMulti members' Q8_1 activations.  Each
// member's value is the single-token row_task value, summed in the same
// order (task t, t+64, ..., then the lane-group tree), so it is bit-identical
// to running the rows once per member.
constexpr int kMulti = 4;
constexpr int kBSmallPerWave = 4;                       // rows per wave, small groups
constexpr int kBSmallRows = kBSmallPerWave * kBWaves;   // rows per block, small groups (gate/up)
static_assert(kBRows % kBSmallRows == 0, "a big group's block spans whole small-group blocks");
constexpr int kBigSpan = kBRows / kBSmallRows;              // gate/up: small-group blocks per big-group block
constexpr int kDnSpan = kBRowsPerBlock / kBRows;            // down: 16-row units per small-group block

template <int TYPE>
__device__ __forceinline__ void row_task_multi(const uint8_t* row, int t, const ActLds* acts, int ne, double v[kMulti]) {
  if (TYPE == MOE_TYPE_Q8_0) {
    float d;
    uint32_t w[8];
    q80_load(row, t, d, w);
#pragma unroll
    for (int m = 0; m < kMulti; ++m) {
      v[m] = 0.0;
      if (m < ne) {
        uint32_t av[8];
        lds_load8(acts[m].codes + 32 * t, av);
        v[m] = (double)d * (double)acts[m].d[t] * (double)q8_block_dot(w, av);
      }
    }
    return;
  }
  const int b = t >> 2, g = t & 3;
  const uint8_t* blk = row + (long)b * block_bytes(TYPE);
  const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
  uint32_t qs[8], qh[8];
  if (TYPE == MOE_TYPE_Q5_K) {
    lds_load8(blk + 16, qh);
    lds_load8(blk + 48 + 32 * g, qs);
  } else {
    lds_load8(blk + 16 + 32 * g, qs);
  }
  int sclo, mlo, schi, mhi;
  kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g, sclo, mlo);
  kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g + 1, schi, mhi);
  const double d = (double)f16_to_f32(hdr.x);
  const double dmin = (double)f16_to_f32(hdr.x >> 16);
  const int jlo = 8 * b + 2 * g;
#pragma unroll
  for (int m = 0; m < kMulti; ++m) {
    v[m] = 0.0;
    if (m < ne) {
      uint32_t alo[8], ahi[8];
      lds_load8(acts[m].codes + 32 * jlo, alo);
      lds_load8(acts[m].codes + 32 * (jlo + 1), ahi);
      int Dlo, Dhi;
      kquant_group_dots<TYPE == MOE_TYPE_Q5_K>(qs, qh, g, alo, ahi, Dlo, Dhi);
      const double t1 = d * (double)sclo * (double)acts[m].d[jlo] * (double)Dlo;
      const double t2 = dmin * (double)mlo * (double)acts[m].s[jlo];
      const double t3 = d * (double)schi * (double)acts[m].d[jlo + 1] * (double)Dhi;
      const double t4 = dmin * (double)mhi * (double)acts[m].s[jlo + 1];
      v[m] = ((t1 - t2) + t3) - t4;
    }
  }
}

// rows_dot for ne <= kMulti activation sets (ne wave-uniform): rowfn(r) gives
// row r's bytes; out[r * kMulti + m] receives row r against set m.
template <int TYPE, class RowFn>
__device__ __forceinline__ void rows_dot_multi(int nrows, int T, RowFn rowfn, const ActLds* acts, int ne, double* out,
                                               int wave, int nw) {
  int TP = 1;
  while (TP < T && TP < 64) TP <<= 1;
  const int rpi = 64 / TP;
  const int lane = threadIdx.x & 63;
  const int rl = lane / TP, t0 = lane - rl * TP;
  const int step = nw * rpi;
  const int tt = (t0 < T) ? t0 : 0;
  for (int r0 = wave * rpi; r0 < nrows; r0 += step) {
    const int ra = r0 + rl;
    const uint8_t* row = rowfn(ra < nrows ? ra : nrows - 1);
    double v[kMulti];
    row_task_multi<TYPE>(row, tt, acts, ne, v);
    if (t0 >= T) {
#pragma unroll
      for (int m = 0; m < kMulti; ++m) v[m] = 0.0;
    }
    for (int t = t0 + 64; t < T; t += 64) {
      double w[kMulti];
      row_task_multi<TYPE>(row, t, acts, ne, w);
#pragma unroll
      for (int m = 0; m < kMulti; ++m) v[m] += w[m];
    }
#pragma unroll
    for (int m = 0; m < kMulti; ++m)
      if (m < ne) v[m] = group_sum_f64(v[m], TP);
    if (t0 == 0 && ra < nrows) {
#pragma unroll
      for (int m = 0; m < kMulti; ++m)
        if (m < ne) out[ra * kMulti + m] = v[m];
    }
  }
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

// gate/up + SwiGLU of one group, 64 rows per block
template <int ST>
__global__ __launch_bounds__(kBThreads) void k_bgu(BGroupArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Group gp;
  if (!block_group(a, gp)) return;
  const int Fx = gp.shared ? a.Fs : a.F;
  const bool big = gp.ne >= a.gmin;
  // blockIdx.y counts kBSmallRows-row chunks: a small group's block takes
  // one (kBSmallPerWave rows per wave); a big group's block takes kBigSpan
  // of them, kBRows rows whose K its waves split (the other blocks of its
  // span leave at once)
  if (big && (blockIdx.y % kBigSpan)) return;
  const int fb = blockIdx.y * kBSmallRows;
  if (fb >= Fx) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H;
  if (big) {
    v4f ag[kMaxTiles], au[kMaxTiles];
    const int f0 = fb;
    const int nr = min(kBRows, Fx - f0);
    {
      auto act = [&](int m) {
        int t, s;
        member(a, gp, m, t, s);
        return a.xn + (long)t * H;
      };
      if (gp.shared) {
        const long rb = row_bytes(ST, H);
        wave_mfma<ST>(a.sgate + f0 * rb, a.sup + f0 * rb, rb, nr, H, gp.ne, H, act, ag, au, wave, kBWaves);
      } else {
        const long rb = row_bytes(MOE_TYPE_Q4_K, H);
        const long base = ((long)gp.e * a.F + f0) * rb;
        wave_mfma<MOE_TYPE_Q4_K>(a.gate + base, a.up + base, rb, nr, H, gp.ne, H, act, ag, au, wave, kBWaves);
      }
      const int ntiles = (gp.ne + 15) >> 4;
      reduce_waves(ag, au, ntiles, true, reinterpret_cast<v4f*>(smem));
      if (wave != 0) return;
#pragma unroll
      for (int j = 0; j < kMaxTiles; ++j) {
        if (j >= ntiles) break;
        const int m = 16 * j + (lane & 15);
        if (m >= gp.ne) continue;
        int t, s;
        member(a, gp, m, t, s);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * (lane >> 4) + i;
          if (rr >= nr) continue;
          const float g = ag[j][i], u = au[j][i];
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
  if (ns > 0) {
    double* pw = part + wave * 2 * kBSmallPerWave * kMulti;
    for (int m0 = 0; m0 < gp.ne; m0 += kMulti) {
      const int nm = min(kMulti, gp.ne - m0);
      ActLds acts[kMulti];
#pragma unroll
      for (int i = 0; i < kMulti; ++i) {
        const int m = m0 + min(i, nm - 1);
        acts[i] = ActLds{codes + (long)m * H, dq + m * (H / 32), sq + m * (H / 32)};
      }
      if (gp.shared) {
        const long rb = row_bytes(ST, H);
        rows_dot_multi<ST>(2 * ns, tasks_per_row(ST, H), [&](int r) {
          return (r < ns) ? a.sgate + (fs + r) * rb : a.sup + (fs + r - ns) * rb;
        }, acts, nm, pw, 0, 1);
      } else {
        const long rb = row_bytes(MOE_TYPE_Q4_K, H);
        const long base = ((long)gp.e * a.F + fs) * rb;
        rows_dot_multi<MOE_TYPE_Q4_K>(2 * ns, tasks_per_row(MOE_TYPE_Q4_K, H), [&](int r) {
          return (r < ns) ? a.gate + base + r * rb : a.up + base + (r - ns) * rb;
        }, acts, nm, pw, 0, 1);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      if (lane < ns * kMulti) {
        const int r = lane / kMulti, i = lane - r * kMulti;
        if (i < nm) {
          const float g = (float)pw[r * kMulti + i], u = (float)pw[(ns + r) * kMulti + i];
          const float hv = (float)(silu_f64((double)g) * (double)u);
          const int m = m0 + i;
          if (gp.shared) a.hs[(long)toks[m] * a.Fs + fs + r] = hv;
          else a.h[((long)toks[m] * a.k + slots[m]) * a.F + fs + r] = hv;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
  }
}

// down rows of one group, 64 output rows per block
template <int DT, int ST>
__global__ __launch_bounds__(kBThreads) void k_bdn(BGroupArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Group gp;
  if (!block_group(a, gp)) return;
  const int H = a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool big = gp.ne >= a.gmin;
  // blockIdx.y counts kBRows-row chunks: a big group's block takes one (its
  // waves split K), a small group's block kDnSpan of them, kBRows rows per
  // wave (the other blocks of its span leave at once)
  if (!big && (blockIdx.y % kDnSpan)) return;
  const int i0 = big ? blockIdx.y * kBRows : (blockIdx.y / kDnSpan) * kBRowsPerBlock + wave * kBRows;
  if (big && i0 >= H) return;
  const int nr = max(0, min(kBRows, H - i0));
  const int Fx = gp.shared ? a.Fs : a.F;
  const int Kx = gp.shared ? a.Kps : a.Kp;
  auto hsrc = [&](int m) {
    int t, s;
    member(a, gp, m, t, s);
    return gp.shared ? a.hs + (long)t * a.Fs : a.h + ((long)t * a.k + s) * a.F;
  };
  if (big) {
    v4f ay[kMaxTiles], dummy[kMaxTiles];
    {
      if (gp.shared) {
        const long rb = row_bytes(ST, Kx);
        wave_mfma<ST>(a.sdown + i0 * rb, nullptr, rb, nr, Kx, gp.ne, Fx, hsrc, ay, dummy, wave, kBWaves);
      } else {
        const long rb = row_bytes(DT, Kx);
        wave_mfma<DT>(a.down + ((long)gp.e * H + i0) * rb, nullptr, rb, nr, Kx, gp.ne, Fx, hsrc, ay, dummy, wave,
                      kBWaves);
      }
      const int ntiles = (gp.ne + 15) >> 4;
      reduce_waves(ay, dummy, ntiles, false, reinterpret_cast<v4f*>(smem));
      if (wave != 0) return;
#pragma unroll
      for (int j = 0; j < kMaxTiles; ++j) {
        if (j >= ntiles) break;
        const int m = 16 * j + (lane & 15);
        if (m >= gp.ne) continue;
        int t, s;
        member(a, gp, m, t, s);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * (lane >> 4) + i;
          if (rr >= nr) continue;
          if (gp.shared) a.ys[(long)t * H + i0 + rr] = ay[j][i];
          else a.y[((long)t * a.k + s) * H + i0 + rr] = ay[j][i];
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
  if (nr > 0) {
    double* pw = part + wave * kBRows * kMulti;
    for (int m0 = 0; m0 < gp.ne; m0 += kMulti) {
      const int nm = min(kMulti, gp.ne - m0);
      ActLds acts[kMulti];
#pragma unroll
      for (int i = 0; i < kMulti; ++i) {
        const int m = m0 + min(i, nm - 1);
        acts[i] = ActLds{codes + (long)m * Kx, dq + m * nb, sq + m * nb};
      }
      if (gp.shared) {
        const long rb = row_bytes(ST, Kx);
        rows_dot_multi<ST>(nr, tasks_per_row(ST, Kx), [&](int r) { return a.sdown + (i0 + r) * rb; }, acts, nm, pw, 0,
                           1);
      } else {
        const long rb = row_bytes(DT, Kx);
        const uint8_t* base = a.down + ((long)gp.e * H + i0) * rb;
        rows_dot_multi<DT>(nr, tasks_per_row(DT, Kx), [&](int r) { return base + r * rb; }, acts, nm, pw, 0, 1);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      for (int o = lane; o < nr * nm; o += 64) {
        const int r = o / nm, i = o - r * nm;
        const float yv = (float)pw[r * kMulti + i];
        const int m = m0 + i;
        if (gp.shared) a.ys[(long)toks[m] * H + i0 + r] = yv;
        else a.y[((long)toks[m] * a.k + slots[m]) * H + i0 + r] = yv;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
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

static size_t int_path_lds(int ne_max, int K) {
  return 2 * sizeof(int) * MOE_MAX_BATCH + (size_t)ne_max * K + 8 * (size_t)ne_max * (K / 32) + 16 +
         sizeof(double) * kMulti * 2 * kBRows * kBWaves;
}

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
  hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, st, ids, n, k, E, reinterpret_cast<int*>(ws + L.cnt),
                     reinterpret_cast<int*>(ws + L.moff), reinterpret_cast<int*>(ws + L.members),
                     reinterpret_cast<int*>(ws + L.dlist), reinterpret_cast<int*>(ws + L.nd),
                     reinterpret_cast<int*>(ws + L.err));
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  // groups: at most min(E, n*k) distinct experts, plus the shared group
  const int ngroups = min(E, n * k) + has_sg;
  const int small = gmin - 1;   // largest group on the integer path
  const int fmax = max(F, Fs);
  const dim3 ggu(ngroups, (fmax + kBSmallRows - 1) / kBSmallRows);
  const size_t lds_gu = std::max(small > 0 ? int_path_lds(small > n ? n : small, H) : (size_t)0, kBigLds);
  const void* fgu = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bgu<MOE_TYPE_Q8_0> : (const void*)k_bgu<MOE_TYPE_Q4_K>;
  if (hipFuncSetAttribute(fgu, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_gu) != hipSuccess) return MOE_ERR_HIP;
  void* args[] = {&a};
  if (hipLaunchKernel(fgu, ggu, dim3(kBThreads), args, lds_gu, st) != hipSuccess) return MOE_ERR_HIP;
  const int kmax = max(a.Kp, a.Kps);
  const dim3 gdn(ngroups, (H + kBRows - 1) / kBRows);
  const size_t lds_dn = std::max(small > 0 ? int_path_lds(small > n ? n : small, kmax) : (size_t)0, kBigLds);
  const void* fdn;
  if (d->down_type == MOE_TYPE_Q5_K)
    fdn = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bdn<MOE_TYPE_Q5_K, MOE_TYPE_Q8_0>
                                     : (const void*)k_bdn<MOE_TYPE_Q5_K, MOE_TYPE_Q4_K>;
  else
    fdn = (st_type == MOE_TYPE_Q8_0) ? (const void*)k_bdn<MOE_TYPE_Q4_K, MOE_TYPE_Q8_0>
                                     : (const void*)k_bdn<MOE_TYPE_Q4_K, MOE_TYPE_Q4_K>;
  if (hipFuncSetAttribute(fdn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dn) != hipSuccess) return MOE_ERR_HIP;
  if (hipLaunchKernel(fdn, gdn, dim3(kBThreads), args, lds_dn, st) != hipSuccess) return MOE_ERR_HIP;
  hipLaunchKernelGGL(k_bcombine, dim3(n, (H + 255) / 256), dim3(256), 0, st, a.y, a.ys, wts, sg,
                     reinterpret_cast<const int*>(ws + L.err), k, H, has_sg, routed, shared);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
