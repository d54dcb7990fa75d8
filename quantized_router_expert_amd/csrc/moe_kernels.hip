// moe_kernels.hip -- gfx950 kernels and the C ABI of the batch-1 decode MoE stage.
//
// Per-layer kernels (one launch each, used by the separate entry points, by
// moe_decode_layer and by the per-layer stack mode):
//   k_add_rmsnorm   a1: fold + RMSNorm + Q8_1, one workgroup per token
//   k_router_topk   a2+a3: fp32 GEMV rows (fp64 accumulate) + last-workgroup top-k/softmax
//   k_gate_up       a4 (+a6 gate/up): Q4_K/Q8_0 rows x Q8_1 + SwiGLU, rows staged in LDS
//   k_down_combine  a5 (+a6 down): Q8_1 of h in LDS, down rows x Q8_1, weighted combine
// Source pages: [P273] fused router GEMV+top-k + folded residual-norm;
// [P239] fused shared-expert launches; [P359] Q4_K shared-expert FFN kernels.
#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_select.h"
#include "moe_stack.h"

#include <string.h>

namespace moe {

// Areas that the DMA into LDS fills start at a KiB boundary of their own: it
// writes whole KiB chunks.
__host__ __device__ constexpr inline long kib_up(long bytes) { return (bytes + 1023) & ~1023L; }

// =====================================================================
// a1: residual add folded into RMSNorm, Q8_1 of the normed vector
// =====================================================================
// t = shared ? bf16(routed + shared) : routed ; u = bf16(residual + t) -> out_sum.
// sum(u^2) is reduced in fp64; r = 1/sqrt(mean + eps) in fp64; xn = f32((u*r)*w).
// With every vector 16-byte aligned, thread i handles elements 8i .. 8i+7,
// 8(i+256) .. with 16-byte accesses; otherwise element i, i+256, ...  The
// Q8_1 blocks are then quantised from LDS with four lanes per block (the same
// fp32 operations, so the same bytes, as the one-lane-per-element form).
__device__ __forceinline__ void unpack_bf16x8(uint4 v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffffu));
    f[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
  }
}
// One element of the fold: bf16(res + bf16(rt + sh)) (bf16(res + rt) without
// sh, res alone without rt) -- the same operations as norm_fold.
__device__ __forceinline__ uint16_t fold_elem(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, int i) {
  float t = 0.0f;
  if (rt && sh) t = bf16_to_f32(f32_to_bf16(bf16_to_f32(rt[i]) + bf16_to_f32(sh[i])));
  else if (rt) t = bf16_to_f32(rt[i]);
  return f32_to_bf16(bf16_to_f32(res[i]) + t);
}

// Q8_1 of the H values at xn_lds (LDS) into xq_out, four lanes per 32-block.
__device__ void q81_from_lds(const float* xn_lds, int H, uint8_t* xq_out) {
  // block j: lanes 4j .. 4j+3, values 8p .. 8p+7 each
  for (int i0 = threadIdx.x; i0 < H / 8; i0 += kNormThreads) {
    const int j = i0 >> 2, p = i0 & 3;
    const float4 a = reinterpret_cast<const float4*>(xn_lds + 32 * j + 8 * p)[0];
    const float4 b = reinterpret_cast<const float4*>(xn_lds + 32 * j + 8 * p)[1];
    float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float amax = 0.0f;
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      amax = fmaxf(amax, fabsf(x[i]));
      nan |= (x[i] != x[i]);
    }
    amax = fmaxf(amax, __uint_as_float(partner_dpp<0>(__float_as_uint(amax))));
    amax = fmaxf(amax, __uint_as_float(partner_dpp<1>(__float_as_uint(amax))));
    const bool slow = nan || !(amax == 0.0f || (amax >= 0x1p-100f && amax <= 0x1p100f));
    uint32_t q[2];
    uint32_t ds;
    if (__builtin_expect(__any(slow), 0)) ds = q81_group<4, true>(x, amax, q);
    else ds = q81_group<4, false>(x, amax, q);
    uint8_t* ob = xq_out + (long)j * kQ81Bytes;
    reinterpret_cast<uint32_t*>(ob + 4 + 8 * p)[0] = q[0];
    reinterpret_cast<uint32_t*>(ob + 4 + 8 * p)[1] = q[1];
    if (p == 0) *reinterpret_cast<uint32_t*>(ob) = ds;
  }
}

// The fold: u = bf16(res + t) into u_lds (and out_sum); returns this thread's
// part of sum(u^2).  vec: 8 elements per thread with 16-byte accesses.
__device__ double norm_fold(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, int H, uint16_t* out_sum,
                            float* u_lds, bool vec) {
  const int tid = threadIdx.x;
  double ss = 0.0;
  if (!vec) {
    for (int i = tid; i < H; i += kNormThreads) {
      float t = 0.0f;
      if (rt && sh) t = bf16_to_f32(f32_to_bf16(bf16_to_f32(rt[i]) + bf16_to_f32(sh[i])));
      else if (rt) t = bf16_to_f32(rt[i]);
      const uint16_t ub = f32_to_bf16(bf16_to_f32(res[i]) + t);
      if (out_sum) out_sum[i] = ub;
      const float u = bf16_to_f32(ub);
      u_lds[i] = u;
      ss += (double)u * (double)u;
    }
    return ss;
  }
  for (int c = tid; c < H / 8; c += kNormThreads) {
    float r8[8], t8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    unpack_bf16x8(reinterpret_cast<const uint4*>(res)[c], r8);
    if (rt) {
      unpack_bf16x8(reinterpret_cast<const uint4*>(rt)[c], t8);
      if (sh) {
        float s8[8];
        unpack_bf16x8(reinterpret_cast<const uint4*>(sh)[c], s8);
#pragma unroll
        for (int i = 0; i < 8; ++i) t8[i] = bf16_to_f32(f32_to_bf16(t8[i] + s8[i]));
      }
    }
    uint32_t ob[4];
    float u8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t ub = f32_to_bf16(r8[i] + t8[i]);
      u8[i] = bf16_to_f32(ub);
      ss += (double)u8[i] * (double)u8[i];
      if (i & 1) ob[i >> 1] |= (uint32_t)ub << 16;
      else ob[i >> 1] = ub;
    }
    if (out_sum) reinterpret_cast<uint4*>(out_sum)[c] = make_uint4(ob[0], ob[1], ob[2], ob[3]);
    reinterpret_cast<float4*>(u_lds)[2 * c] = make_float4(u8[0], u8[1], u8[2], u8[3]);
    reinterpret_cast<float4*>(u_lds)[2 * c + 1] = make_float4(u8[4], u8[5], u8[6], u8[7]);
  }
  return ss;
}

// The norm: sum(u^2) over the workgroup in fp64 (waves in order), r =
// 1/sqrt(mean + eps), xn = f32((u*r)*w) into xl (and xn_out).  w may be in
// LDS or global memory; vec: 4 elements per thread with 16-byte accesses.
__device__ void norm_scale(double ss, const float* w, int H, float eps, float* xn_out, const float* u_lds, float* xl,
                           double* red_lds, bool vec) {
  const int tid = threadIdx.x;
  ss = wave_sum_f64(ss);
  if ((tid & 63) == 0) red_lds[tid >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int wv = 0; wv < kNormThreads / 64; ++wv) tot += red_lds[wv];
  const double r = 1.0 / sqrt(tot / (double)H + (double)eps);
  if (!vec) {
    for (int i = tid; i < H; i += kNormThreads) {
      const float x = (float)(((double)u_lds[i] * r) * (double)w[i]);
      if (xn_out) xn_out[i] = x;
      xl[i] = x;
    }
    return;
  }
  for (int c = tid; c < H / 4; c += kNormThreads) {
    const float4 u = reinterpret_cast<const float4*>(u_lds)[c];
    const float4 wv = reinterpret_cast<const float4*>(w)[c];
    float4 x;
    x.x = (float)(((double)u.x * r) * (double)wv.x);
    x.y = (float)(((double)u.y * r) * (double)wv.y);
    x.z = (float)(((double)u.z * r) * (double)wv.z);
    x.w = (float)(((double)u.w * r) * (double)wv.w);
    if (xn_out) reinterpret_cast<float4*>(xn_out)[c] = x;
    reinterpret_cast<float4*>(xl)[c] = x;   // (each float4 is read and written by one thread)
  }
}

// Fold + norm + Q8_1 of one token by one workgroup.  xn goes to xn_lds when
// given (u stays in u_lds), else it replaces u in u_lds.
__device__ void norm_token_block(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, const float* w,
                                 int H, float eps, uint16_t* out_sum, float* xn_out, uint8_t* xq_out,
                                 float* u_lds, double* red_lds, int do_norm, float* xn_lds = nullptr) {
  const bool vec = ((reinterpret_cast<uintptr_t>(res) | reinterpret_cast<uintptr_t>(rt) |
                     reinterpret_cast<uintptr_t>(sh) | reinterpret_cast<uintptr_t>(out_sum) |
                     reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(xn_out)) & 15) == 0;
  const double ss = norm_fold(res, rt, sh, H, out_sum, u_lds, vec);
  if (!do_norm) return;
  float* const xl = xn_lds ? xn_lds : u_lds;
  norm_scale(ss, w, H, eps, xn_out, u_lds, xl, red_lds, vec);
  if (!xq_out) return;
  __syncthreads();
  q81_from_lds(xl, H, xq_out);
}

__global__ __launch_bounds__(kNormThreads) void k_add_rmsnorm(const uint16_t* res, const uint16_t* rt, const uint16_t* sh,
                                                               const float* w, int H, float eps, uint16_t* out_sum,
                                                               float* xn, uint8_t* xq, int do_norm) {
  __shared__ float u_lds[MOE_MAX_HIDDEN];
  __shared__ double red_lds[kNormThreads / 64];
  const long tok = blockIdx.x;
  norm_token_block(res + tok * H, rt ? rt + tok * H : nullptr, sh ? sh + tok * H : nullptr, w, H, eps,
                   out_sum ? out_sum + tok * H : nullptr, xn ? xn + tok * H : nullptr,
                   xq ? xq + tok * (H / 32) * kQ81Bytes : nullptr, u_lds, red_lds, do_norm);
}

// Plain Q8_1 of an fp32 vector (the layer input when the layer has no norm).
__global__ __launch_bounds__(kNormThreads) void k_quantize_q81(const float* x, int n, uint8_t* xq) {
  for (int i = blockIdx.x * kNormThreads + threadIdx.x; i < n; i += gridDim.x * kNormThreads) {
    Q81Lane q = quantize_q81_lane(x[i]);
    uint8_t* ob = xq + (long)(i >> 5) * kQ81Bytes;
    if ((i & 31) == 0) *reinterpret_cast<uint32_t*>(ob) = q.ds;
    ob[4 + (i & 31)] = (uint8_t)(int8_t)q.q;
  }
}

// =====================================================================
// a2 + a3: router GEMV + last-workgroup top-k + routing weights
// =====================================================================
// The workgroup's arrival on a grid-completion counter group at c0 (called by
// one thread after the workgroup's results are stored): true for the last of
// the gridDim.x workgroups to arrive.  The counters wrap back to zero.
__device__ __forceinline__ bool arrive_last(unsigned* c0, int cstride, int nsub) {
  if (nsub > 0) {
    const unsigned j = blockIdx.x % (unsigned)nsub;
    const unsigned nj = (gridDim.x - j + nsub - 1) / (unsigned)nsub;   // workgroups on sub-counter j
    const unsigned o1 = __builtin_amdgcn_atomic_inc32(c0 + (1 + j) * cstride, nj - 1, __ATOMIC_RELAXED, "agent");
    if (o1 != nj - 1) return false;
    const unsigned nz = min((unsigned)nsub, gridDim.x);   // sub-counters in use
    return __builtin_amdgcn_atomic_inc32(c0, nz - 1, __ATOMIC_RELAXED, "agent") == nz - 1;
  }
  const unsigned old = __builtin_amdgcn_atomic_inc32(c0, gridDim.x - 1, __ATOMIC_RELAXED, "agent");
  return old == gridDim.x - 1;
}

// grid (ceil(nrows / kRouterRpb), ceil(n_tok / kRouterTok)): workgroup x
// computes rows kRouterRpb*x .. (router row e < E, or the shared-gate row
// e == E) for up to kRouterTok tokens, so a row is read once per token group;
// the waves of a row take interleaved parts of it and their fp64 partial
// sums are added in wave order.  The last workgroup of a token group to
// finish selects for the group's tokens, one token per wave at a time.  It is
// found with wrapping atomic increments (each returns limit-1 to its last
// arrival and leaves 0 behind), one counter per 128-byte line when the
// workspace has room.  With nsub > 0 (the group's counters are slot 0, the
// top, and slots 1..nsub) workgroup x counts on sub-counter x % nsub and the
// last arrival of each sub-counter on the top one, so no counter takes more
// than about gridDim.x / nsub increments (increments of one address are
// performed one after another); with nsub == 0 all count on slot 0.
constexpr int kRouterRpb = 1;   // router rows per workgroup
__global__ __launch_bounds__(kRouterThreads) void k_router_topk(const float* xn, const float* W, const float* wsg,
                                                                 int n_tok, int H, int E, int k, float* logits,
                                                                 float* user_logits, int32_t* ids, float* wts,
                                                                 float* sg_out, unsigned* counters, int cstride,
                                                                 int nsub) {
  constexpr int kW = kRouterThreads / 64;
  constexpr int kWpr = kW / kRouterRpb;   // waves per row
  __shared__ double part[kW][kRouterTok];
  const int logits_stride = E + 1;
  const int tg = blockIdx.y;
  const int t0 = tg * kRouterTok;
  const int nt = min(kRouterTok, n_tok - t0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nrows = E + (wsg ? 1 : 0);
  const int row = blockIdx.x * kRouterRpb + wave / kWpr, qw = wave % kWpr;
  {
    double acc[kRouterTok];
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t) acc[t] = 0.0;
    if (row < nrows) {
      const float* wr = (row < E) ? W + (long)row * H : wsg;
      // every load of a step goes out before the first product: token slots
      // past nt read the last token again (their sums are never stored), so
      // no branch separates the loads
      for (int i = (qw * 64 + lane) * 4; i < H; i += 256 * kWpr) {
        const float4 a = *reinterpret_cast<const float4*>(wr + i);
        float4 b[kRouterTok];
#pragma unroll
        for (int t = 0; t < kRouterTok; ++t)
          b[t] = *reinterpret_cast<const float4*>(xn + (long)(t0 + min(t, nt - 1)) * H + i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kRouterTok; ++t) {
          acc[t] += (double)a.x * (double)b[t].x;
          acc[t] += (double)a.y * (double)b[t].y;
          acc[t] += (double)a.z * (double)b[t].z;
          acc[t] += (double)a.w * (double)b[t].w;
        }
      }
    }
    // the kRouterTok reductions are independent chains
    double red[kRouterTok];
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t) red[t] = wave_sum_f64(acc[t]);
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t)
        if (t < nt) part[wave][t] = red[t];
    }
    __syncthreads();
    if ((int)threadIdx.x < kRouterRpb * nt) {
      const int rr = threadIdx.x / nt, t = threadIdx.x - rr * nt;
      const int r = blockIdx.x * kRouterRpb + rr;
      if (r < nrows) {
        double v = part[rr * kWpr][t];
        for (int w2 = 1; w2 < kWpr; ++w2) v += part[rr * kWpr + w2][t];
        // agent-coherent store, complete before the counter moves: the
        // workgroup that finishes last reads it after invalidating its own
        // L2, so no workgroup has to write its L2 back (the release of an
        // acq_rel counter increment would)
        __hip_atomic_store(logits + (long)(t0 + t) * logits_stride + r, (float)v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }
  }
  __shared__ int is_last;
  __syncthreads();
  if (threadIdx.x == 0) is_last = arrive_last(counters + (long)tg * (nsub + 1) * cstride, cstride, nsub);
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int t = wave; t < nt; t += kRouterThreads / 64) {
    const float* lg = logits + (long)(t0 + t) * logits_stride;
    wave_topk_softmax(lg, E, k, ids + (long)(t0 + t) * k, wts + (long)(t0 + t) * k);
    if (lane == 0 && sg_out) sg_out[t0 + t] = wsg ? (float)sigmoid_f64((double)lg[E]) : 0.0f;
  }
  if (user_logits)
    for (int i = threadIdx.x; i < nt * E; i += kRouterThreads) {
      const int t = i / E, e = i - t * E;
      user_logits[(long)(t0 + t) * E + e] = logits[(long)(t0 + t) * logits_stride + e];
    }
}

// a1 + a2 for one token in one launch ([P273] Summary item 2: the residual
// fold and norm ahead of the router's GEMV).  Workgroup x (kNormThreads
// threads) owns router row x (the shared-gate row when x == E): it streams the
// row and the norm weight into LDS while it folds the token itself,
// normalises it (the same element mapping and fp64 reduction order in every
// workgroup, so the same xn everywhere) and stores the row's fp64 dot with xn.
// Workgroup 0 also writes xn and xq.  The selection runs in the next launch
// (k_gate_up), which also writes the folded sum: by then every read of the
// residual inputs is done, so out_sum may be one of them.
struct NormRouterArgs {
  const uint16_t* res;
  const uint16_t* rt;
  const uint16_t* sh;
  const float* norm_w;
  const float* W;          // [E][H]
  const float* wsg;        // [H] or null
  float* xn;               // or null
  uint8_t* xq;
  float* logits;           // [E + 1] workspace
  float* user_logits;      // [E] or null
  int H, E;
  float eps;
};

__global__ __launch_bounds__(kNormThreads) void k_norm_router(NormRouterArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ double red[kNormThreads / 64];
  const int H = a.H, x = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long hb = kib_up(4L * H);
  float* row = reinterpret_cast<float*>(smem);                 // H floats, padded to the next KiB
  float* nw = reinterpret_cast<float*>(smem + hb);             // the norm weight, likewise
  float* u = reinterpret_cast<float*>(smem + 2 * hb);          // H floats: the folded sum
  float* xn = u + H;                                            // H floats
  stage_async(reinterpret_cast<uint8_t*>(row), x < a.E ? a.W + (long)x * H : a.wsg, (uint32_t)(H * 4), wave, 0,
              kNormThreads / 64);
  stage_async(reinterpret_cast<uint8_t*>(nw), a.norm_w, (uint32_t)(H * 4), wave, 0, kNormThreads / 64);
  // the fold's loads queue behind the streamed rows, so both have landed after it
  const bool vec = ((reinterpret_cast<uintptr_t>(a.res) | reinterpret_cast<uintptr_t>(a.rt) |
                     reinterpret_cast<uintptr_t>(a.sh)) & 15) == 0;
  const double ss = norm_fold(a.res, a.rt, a.sh, H, nullptr, u, vec);
  wait_vmem();
  __syncthreads();
  norm_scale(ss, nw, H, a.eps, nullptr, u, xn, red, vec);
  __syncthreads();
  double acc = 0.0;
  for (int i = threadIdx.x * 4; i < H; i += kNormThreads * 4) {
    const float4 w4 = *reinterpret_cast<const float4*>(row + i);
    const float4 x4 = *reinterpret_cast<const float4*>(xn + i);
    acc += (double)w4.x * (double)x4.x;
    acc += (double)w4.y * (double)x4.y;
    acc += (double)w4.z * (double)x4.z;
    acc += (double)w4.w * (double)x4.w;
  }
  acc = wave_sum_f64(acc);
  __syncthreads();                       // every wave is done with red (the norm's sums)
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double v = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < kNormThreads / 64; ++w2) v += red[w2];
    a.logits[x] = (float)v;
    if (a.user_logits && x < a.E) a.user_logits[x] = (float)v;
  }
  if (x == 0) {
    for (int i = threadIdx.x * 4; a.xn && i < H; i += kNormThreads * 4)
      *reinterpret_cast<float4*>(a.xn + i) = *reinterpret_cast<const float4*>(xn + i);
    q81_from_lds(xn, H, a.xq);
  }
}

// =====================================================================
// Row staging and row dots from LDS
// =====================================================================
// Copy `bytes` (multiple of 16) from global to LDS with 16-byte loads by all threads.
__device__ __forceinline__ void stage_to_lds(uint8_t* dst, const uint8_t* src, long bytes, int nthreads) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  const int n16 = (int)(bytes >> 4);
  for (int i = threadIdx.x; i < n16; i += nthreads) d[i] = s[i];
}

// Q8_1 activations (global, 36-byte blocks) -> LDS codes/d/s.
__device__ void load_act_lds(const uint8_t* xq, int K, uint8_t* codes, float* d, float* s, int t0, int nthreads) {
  // the K/32 blocks are 9 dwords each (d|s, then 8 of codes): thread t0 + i
  // takes dwords i, i + nthreads, ..., four loads in flight before any store
  // (a dword past the end reads the last one again and is not stored)
  const int nb = K / 32, ndw = nb * 9;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(xq);
  for (int i0 = t0; i0 < ndw; i0 += 4 * nthreads) {
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[min(i0 + u * nthreads, ndw - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * nthreads;
      if (i < ndw) {
        const int b = i / 9, o = i - 9 * b;
        if (o == 0) {
          d[b] = f16_to_f32(v[u]);
          s[b] = f16_to_f32(v[u] >> 16);
        } else {
          reinterpret_cast<uint32_t*>(codes)[8 * b + o - 1] = v[u];
        }
      }
    }
  }
}

// All tasks of `nrows` rows of K elements staged back to back at `rows`:
// partial[r*T + t] = fp64 contribution of task t of row r.
// =====================================================================
// a4 (+ a6 gate/up): gate/up rows + SwiGLU
// =====================================================================
// Block b < k*cpe handles routed slot b/cpe, rows [(b%cpe)*R, +R); the rest
// handle the shared expert's rows.  Gate and up rows of a chunk are contiguous
// in memory and staged into LDS with 16-byte loads.
struct GateUpArgs {
  const uint8_t* xq;
  const int32_t* ids;      // the selected experts, or null: select from `logits`
  const float* logits;     // [E + 1] (selection; logit E is the shared gate's)
  int32_t* ids_out;        // selection: ids, weights and shared gate written by workgroup 0
  float* wts_out;
  float* sg_out;           // or null
  int has_sg;
  // the residual fold u = bf16(res + bf16(rt + sh)) -> out_sum, a slice per workgroup (or null)
  const uint16_t* res;
  const uint16_t* rt;
  const uint16_t* sh;
  uint16_t* out_sum;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* sgate;
  const uint8_t* sup;
  float* h;
  float* hs;
  int H, F, Fs, k, E, R, cpe, cps;
  int type, stype;
};


// the nr gate rows and nr up rows of a chunk by rows_dot (a row's tasks on
// lane groups, summed by the lane-group tree, two rows per lane in flight:
// the persistent kernel's row values bit for bit), then SwiGLU
template <int TYPE>
__device__ void gate_up_chunk(const uint8_t* stage, long up_off, int nr, int H, const ActLds& act, double* partial,
                              float* h_out) {
  const long rb = row_bytes(TYPE, H);
  rows_dot<TYPE>(2 * nr, tasks_per_row(TYPE, H), [&](int r) {
    return RowRef{(r < nr) ? stage + (long)r * rb : stage + up_off + (long)(r - nr) * rb, act};
  }, partial, (int)(threadIdx.x >> 6), (int)(blockDim.x >> 6));
  __syncthreads();
  for (int f = threadIdx.x; f < nr; f += blockDim.x) {
    const float g = (float)partial[f];
    const float u = (float)partial[nr + f];
    h_out[f] = (float)(silu_f64((double)g) * (double)u);
  }
}

// The gate and up rows are streamed straight into LDS (every KiB chunk in
// flight at once) as soon as the expert id is known; the activations are read
// behind them.
__global__ __launch_bounds__(kFfnThreads) void k_gate_up(GateUpArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int H = a.H;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const bool routed = b < a.k * a.cpe;
  const int type = routed ? MOE_TYPE_Q4_K : a.stype;
  const long rb = row_bytes(type, H);
  const long up_off = kib_up((long)a.R * rb);
  uint8_t* stage = smem;
  double* partial = reinterpret_cast<double*>(stage + 2 * up_off);
  uint8_t* codes = reinterpret_cast<uint8_t*>(partial + 2 * (long)a.R * tasks_per_row(type, H));
  float* dact = reinterpret_cast<float*>(codes + H);
  float* sact = dact + H / 32;
  int nr, f0;
  float* h_out;
  constexpr int kLastWave = kFfnThreads / 64 - 1;
  if (a.out_sum && wave == kLastWave) {   // this workgroup's slice of the folded residual sum (the last
    // wave: wave 0's loads are the selection's)
    const int cs = (H + gridDim.x - 1) / gridDim.x;
    const int iend = min(H, (b + 1) * cs);
    for (int i = b * cs + (threadIdx.x & 63); i < iend; i += 64) a.out_sum[i] = fold_elem(a.res, a.rt, a.sh, i);
  }
  if (routed) {
    const int slot = b / a.cpe;
    f0 = (b % a.cpe) * a.R;
    nr = min(a.R, a.F - f0);
    // the selection from the router launch's logits, as the persistent kernel
    // makes it: waves 0..3 land the logits in LDS and rank them (candidates),
    // wave 0 merges the candidates; waves 4..7 read the activations meanwhile
    __shared__ float s_lg[MOE_MAX_EXPERTS + 1];
    __shared__ unsigned long long s_keys[256], s_cand[4 * 16];
    __shared__ uint32_t s_sel[2 * MOE_MAX_TOPK + 1];
    __shared__ float s_lgsel[MOE_MAX_TOPK + 1];
    constexpr int kSelWaves = 4;
    static_assert(kFfnThreads / 64 > kSelWaves, "waves past the selecting ones read the activations");
    if (!a.ids && wave >= kSelWaves)
      load_act_lds(a.xq, H, codes, dact, sact, threadIdx.x - 64 * kSelWaves, blockDim.x - 64 * kSelWaves);
    if (!a.ids) {
      if (wave < kSelWaves) {
        // wave w lands the logits it ranks: experts 64w + lane + 256j
        const int lane = threadIdx.x & 63;
        for (int e = 64 * wave + lane; e < a.E; e += 64 * kSelWaves) s_lg[e] = a.logits[e];
        if (wave == 0 && lane == 0) s_lg[a.E] = a.has_sg ? a.logits[a.E] : 0.0f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        topk_candidates(s_lg, a.E, a.k, wave, s_keys, s_cand);
      }
      __syncthreads();
      if (wave == 0) rank_candidates(s_lg, a.E, a.k, a.has_sg, s_cand, s_sel, s_lgsel);
      __syncthreads();
    }
    const long e = a.ids ? a.ids[slot] : (long)s_sel[slot];
    if (e < 0 || e >= a.E) {  // an id outside the experts reads nothing and yields NaN
      for (int f = threadIdx.x; f < nr; f += blockDim.x) a.h[(long)slot * a.F + f0 + f] = __builtin_nanf("");
      return;
    }
    stage_async(stage, a.gate + (e * a.F + f0) * rb, (uint32_t)(nr * rb), wave, 0, kFfnThreads / 64);
    stage_async(stage + up_off, a.up + (e * a.F + f0) * rb, (uint32_t)(nr * rb), wave, 0, kFfnThreads / 64);
    h_out = a.h + (long)slot * a.F + f0;
    if (!a.ids && b == 0 && wave == 0) {   // ids, routing weights and gate, while the rows land
      routing_weights(a.k, a.has_sg, s_lgsel, s_sel, reinterpret_cast<double*>(s_cand));
      const int lane = threadIdx.x & 63;
      if (lane < a.k) {
        a.ids_out[lane] = (int32_t)s_sel[lane];
        a.wts_out[lane] = __uint_as_float(s_sel[a.k + lane]);
      }
      if (lane == 0 && a.sg_out) a.sg_out[0] = __uint_as_float(s_sel[2 * a.k]);
    }
  } else {
    f0 = (b - a.k * a.cpe) * a.R;
    nr = min(a.R, a.Fs - f0);
    stage_async(stage, a.sgate + f0 * rb, (uint32_t)(nr * rb), wave, 0, kFfnThreads / 64);
    stage_async(stage + up_off, a.sup + f0 * rb, (uint32_t)(nr * rb), wave, 0, kFfnThreads / 64);
    h_out = a.hs + f0;
  }
  if (!routed || a.ids) load_act_lds(a.xq, H, codes, dact, sact, threadIdx.x, blockDim.x);
  wait_vmem();
  __syncthreads();
  ActLds act{codes, dact, sact};
  if (type == MOE_TYPE_Q8_0) gate_up_chunk<MOE_TYPE_Q8_0>(stage, up_off, nr, H, act, partial, h_out);
  else gate_up_chunk<MOE_TYPE_Q4_K>(stage, up_off, nr, H, act, partial, h_out);
}

// =====================================================================
// a5 (+ a6 down): Q8_1 of h, down rows, weighted combine
// =====================================================================
struct DownArgs {
  const float* h;         // [k][F]
  const float* hs;        // [Fs]
  const int32_t* ids;
  const float* wts;
  const float* sg;        // [1]
  const uint8_t* down;    // [E][H] rows of Kp
  const uint8_t* sdown;   // [H] rows of Kps
  uint16_t* routed;
  uint16_t* shared;
  int H, F, Fs, k, E, Ro;
  int dtype, stype;
  int Kp, Kps;
};

// Q8_1 of n values (n multiple of 32) into LDS codes/d/s, zero blocks up to np.
__device__ void quantize_to_lds(const float* x, int n, int np, uint8_t* codes, float* d, float* s) {
  const int nthreads = blockDim.x;
  for (int i0 = 0; i0 < np; i0 += nthreads) {
    const int i = i0 + threadIdx.x;
    // whole 32-blocks per half wave: np is a multiple of 32 and nthreads of 64
    const float v = (i < n) ? x[i] : 0.0f;
    Q81Lane q = quantize_q81_lane(v);
    if (i < np) {
      codes[i] = (uint8_t)(int8_t)q.q;
      if ((i & 31) == 0) {
        d[i >> 5] = f16_to_f32(q.ds);
        s[i >> 5] = f16_to_f32(q.ds >> 16);
      }
    }
  }
}

template <int DT, int ST>
__device__ void down_combine_body(const DownArgs& a, uint8_t* smem) {
  const int nm = a.k + (a.Fs > 0 ? 1 : 0);
  const int Kp = a.Kp, Kps = a.Kps;
  // layout: codes [k][Kp] | codes_s [Kps] | d,s [k][Kp/32] | d,s [Kps/32] | stage | partials | y
  uint8_t* codes = smem;
  uint8_t* codes_s = codes + (long)a.k * Kp;
  float* dact = reinterpret_cast<float*>(codes_s + Kps);
  float* sact = dact + a.k * (Kp / 32);
  float* dsh = sact + a.k * (Kp / 32);
  float* ssh = dsh + Kps / 32;
  uint8_t* stage = reinterpret_cast<uint8_t*>((((uintptr_t)(ssh + Kps / 32)) + 15) & ~(uintptr_t)15);
  const long rb = row_bytes(DT, Kp);
  const long rbs = a.Fs > 0 ? row_bytes(ST, Kps) : 0;
  const long slot_bytes = kib_up((long)a.Ro * rb);   // each slot's rows start at a KiB boundary
  const int i0 = blockIdx.x * a.Ro;
  const int nr = min(a.Ro, a.H - i0);
  const int wave = threadIdx.x >> 6;
  uint8_t* stage_s = stage + (long)a.k * slot_bytes;
  double* partial = reinterpret_cast<double*>(stage_s + kib_up((long)a.Ro * rbs));
  const int T = tasks_per_row(DT, Kp);
  const int Ts = a.Fs > 0 ? tasks_per_row(ST, Kps) : 0;
  double* partial_s = partial + (long)a.k * a.Ro * T;
  float* y = reinterpret_cast<float*>(partial_s + (long)a.Ro * Ts);

  // the ids, the routing weights and the gate, read at once into LDS (the
  // row requests below are asm the compiler cannot move loads across: read
  // there, each id would be a round trip of its own)
  __shared__ float s_wts[MOE_MAX_TOPK], s_sg;
  __shared__ int32_t s_ids[MOE_MAX_TOPK];
  if ((int)threadIdx.x < a.k) {
    s_ids[threadIdx.x] = a.ids[threadIdx.x];
    s_wts[threadIdx.x] = a.wts[threadIdx.x];
  }
  if (threadIdx.x == 0) s_sg = a.Fs > 0 ? a.sg[0] : 0.0f;
  __syncthreads();
  bool bad_id = false;
  for (int s = 0; s < a.k; ++s) bad_id |= (s_ids[s] < 0 || s_ids[s] >= a.E);
  if (bad_id) {  // an id outside the experts reads nothing and yields NaN outputs
    for (int r = threadIdx.x; r < nr; r += blockDim.x) {
      a.routed[i0 + r] = 0x7fc0u;
      if (a.Fs > 0 && a.shared) a.shared[i0 + r] = 0x7fc0u;
    }
    return;
  }

  // stream the weight rows into LDS first so they are in flight during the quantisation
  for (int s = 0; s < a.k; ++s) {
    const long e = s_ids[s];
    stage_async(stage + (long)s * slot_bytes, a.down + (e * a.H + i0) * rb, (uint32_t)(nr * rb), wave, 0,
                kFfnThreads / 64);
  }
  if (a.Fs > 0) stage_async(stage_s, a.sdown + (long)i0 * rbs, (uint32_t)(nr * rbs), wave, 0, kFfnThreads / 64);
  // Q8_1 of every h: with 16-byte aligned h, four lanes per block and two
  // blocks in flight per lane (every load of a pass out before the first
  // quantisation); otherwise one lane per element
  const bool vec_h = (((uintptr_t)a.h | (uintptr_t)(a.Fs > 0 ? a.hs : nullptr)) & 15) == 0;
  if (vec_h) {
    const int nbk = Kp / 32, F = a.F, Fs = a.Fs;
    quantize_q81_groups<4, 3>(
        a.k * nbk, a.h,
        [nbk, F](int j) {
          const int s = j / nbk, jj = j - s * nbk;
          return 32 * jj < F ? s * F + 32 * jj : -1;
        },
        [codes](int j) { return codes + 32 * j; }, dact, sact, threadIdx.x, kFfnThreads);
    if (a.Fs > 0)
      quantize_q81_groups<4, 2>(
          Kps / 32, a.hs, [Fs](int j) { return 32 * j < Fs ? 32 * j : -1; },
          [codes_s](int j) { return codes_s + 32 * j; }, dsh, ssh, threadIdx.x, kFfnThreads);
  } else {
    for (int s = 0; s < a.k; ++s)
      quantize_to_lds(a.h + (long)s * a.F, a.F, Kp, codes + (long)s * Kp, dact + s * (Kp / 32), sact + s * (Kp / 32));
    if (a.Fs > 0) quantize_to_lds(a.hs, a.Fs, Kps, codes_s, dsh, ssh);
  }
  wait_vmem();
  __syncthreads();
  // the slots' rows by rows_dot (row i = row i % nr of slot i / nr: the
  // persistent kernel's row values bit for bit); the shared expert's rows as
  // one more slot in the same pass when its type and length are the routed ones
  const ActLds acts{codes_s, dsh, ssh};
  const bool one_pass = a.Fs > 0 && DT == ST && Kps == Kp;
  const int wave_n = (int)(blockDim.x >> 6);
  rows_dot<DT>((a.k + (one_pass ? 1 : 0)) * nr, T, [&](int i) {
    const int s = i / nr, r = i - s * nr;
    if (s == a.k) return RowRef{stage_s + (long)r * rbs, acts};
    return RowRef{stage + (long)s * slot_bytes + (long)r * rb,
                  ActLds{codes + (long)s * Kp, dact + s * (Kp / 32), sact + s * (Kp / 32)}};
  }, partial, wave, wave_n);
  if (a.Fs > 0 && !one_pass)
    rows_dot<ST>(nr, Ts, [&](int r) { return RowRef{stage_s + (long)r * rbs, acts}; }, partial + (long)a.k * nr, wave,
                 wave_n);
  __syncthreads();
  for (int i = threadIdx.x; i < nm * nr; i += blockDim.x) {
    const int m = i / nr, r = i - m * nr;
    y[m * a.Ro + r] = (float)partial[(long)m * nr + r];
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nr; r += blockDim.x) {
    double acc = 0.0;
    for (int s = 0; s < a.k; ++s) acc += (double)s_wts[s] * (double)y[s * a.Ro + r];
    a.routed[i0 + r] = f32_to_bf16((float)acc);
    if (a.Fs > 0 && a.shared) a.shared[i0 + r] = f32_to_bf16((float)((double)s_sg * (double)y[a.k * a.Ro + r]));
  }
}

// one instance per (down, shared) type pair, each with its own register budget
template <int DT, int ST>
__global__ __launch_bounds__(kFfnThreads) void k_down_combine(DownArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  down_combine_body<DT, ST>(a, smem);
}

// =====================================================================
// Test export: integer sub-block dots, through the same integer path
// =====================================================================
template <int TYPE>
__device__ void subblock_dots_row(const uint8_t* row, int K, const ActLds& act, int32_t* out) {
  const int T = tasks_per_row(TYPE, K);
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    if (TYPE == MOE_TYPE_Q8_0) {
      float d;
      uint32_t w[8], av[8];
      q80_load(row, t, d, w);
      lds_load8(act.codes + 32 * t, av);
      out[t] = q8_block_dot(w, av);
    } else {
      const int b = t >> 2, g = t & 3;
      const uint8_t* blk = row + (long)b * block_bytes(TYPE);
      uint32_t qs[8], qh[8], alo[8], ahi[8];
      if (TYPE == MOE_TYPE_Q5_K) {
        lds_load8(blk + 16, qh);
        lds_load8(blk + 48 + 32 * g, qs);
      } else {
        lds_load8(blk + 16 + 32 * g, qs);
      }
      lds_load8(act.codes + 32 * (8 * b + 2 * g), alo);
      lds_load8(act.codes + 32 * (8 * b + 2 * g + 1), ahi);
      int lo, hi;
      kquant_group_dots<TYPE == MOE_TYPE_Q5_K>(qs, qh, g, alo, ahi, lo, hi);
      out[8 * b + 2 * g] = lo;
      out[8 * b + 2 * g + 1] = hi;
    }
  }
}

__global__ __launch_bounds__(kFfnThreads) void k_subblock_dots(const uint8_t* rows, int type, int K, const uint8_t* xq,
                                                                int32_t* out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* codes = smem;
  float* d = reinterpret_cast<float*>(smem + K);
  float* s = d + K / 32;
  uint8_t* stage = reinterpret_cast<uint8_t*>((((uintptr_t)(s + K / 32)) + 15) & ~(uintptr_t)15);
  load_act_lds(xq, K, codes, d, s, threadIdx.x, blockDim.x);
  const long rb = row_bytes(type, K);
  stage_to_lds(stage, rows + blockIdx.x * rb, rb, blockDim.x);
  __syncthreads();
  ActLds act{codes, d, s};
  int32_t* o = out + (long)blockIdx.x * (K / 32);
  if (type == MOE_TYPE_Q4_K) subblock_dots_row<MOE_TYPE_Q4_K>(stage, K, act, o);
  else if (type == MOE_TYPE_Q5_K) subblock_dots_row<MOE_TYPE_Q5_K>(stage, K, act, o);
  else subblock_dots_row<MOE_TYPE_Q8_0>(stage, K, act, o);
}

// The persistent kernel's Q8_1 quantiser (four lanes per block, exact fast
// operations with a per-wave IEEE fallback) over n/32 blocks: 128 blocks per
// workgroup of 512 threads, staged through LDS as in the persistent kernel.
constexpr int kQ81TestThreads = 512, kQ81TestBlocks = 128;
__global__ __launch_bounds__(kQ81TestThreads) void k_test_q81_groups(const float* x, int nblk, uint8_t* xq) {
  __shared__ __attribute__((aligned(16))) float vals[32 * kQ81TestBlocks];
  __shared__ __attribute__((aligned(16))) uint8_t codes[32 * kQ81TestBlocks];
  __shared__ float dq[kQ81TestBlocks], sq[kQ81TestBlocks];
  const int b0 = blockIdx.x * kQ81TestBlocks;
  const int nb = min(kQ81TestBlocks, nblk - b0);
  for (int i = threadIdx.x; i < 32 * nb; i += kQ81TestThreads) vals[i] = x[(long)32 * b0 + i];
  __syncthreads();
  quantize_q81_groups<4, 1>(nb, vals, [](int j) { return 32 * j; }, [&](int j) { return codes + 32 * j; }, dq, sq,
                            (int)threadIdx.x, kQ81TestThreads);
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += kQ81TestThreads) {
    uint8_t* o = xq + (long)(b0 + j) * 36;
    const uint32_t ds = f32_to_f16(dq[j]) | (f32_to_f16(sq[j]) << 16);
    reinterpret_cast<uint16_t*>(o)[0] = (uint16_t)ds;
    reinterpret_cast<uint16_t*>(o)[1] = (uint16_t)(ds >> 16);
    for (int i = 0; i < 32; i += 2) reinterpret_cast<uint16_t*>(o + 4)[i / 2] = reinterpret_cast<const uint16_t*>(codes + 32 * j)[i / 2];
  }
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// =====================================================================
// Host side
// =====================================================================
static inline int launch_ok() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->hidden <= 0 || d->hidden % 256 || d->hidden > MOE_MAX_HIDDEN) return MOE_ERR_SHAPE;
  if (d->n_experts <= 0 || d->n_experts > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (d->top_k <= 0 || d->top_k > d->n_experts || d->top_k > MOE_MAX_TOPK) return MOE_ERR_SHAPE;
  if (d->ffn <= 0 || d->ffn % 32 || d->ffn > MOE_MAX_FFN) return MOE_ERR_SHAPE;
  if (d->shared_ffn < 0 || d->shared_ffn % 32 || d->shared_ffn > MOE_MAX_FFN) return MOE_ERR_SHAPE;
  if (d->gate_up_type != MOE_TYPE_Q4_K) return MOE_ERR_TYPE;
  if (d->down_type != MOE_TYPE_Q4_K && d->down_type != MOE_TYPE_Q5_K) return MOE_ERR_TYPE;
  if (d->shared_ffn > 0 && d->shared_type != MOE_TYPE_Q4_K && d->shared_type != MOE_TYPE_Q8_0) return MOE_ERR_TYPE;
  // Q8_0 rows are staged with 16-byte loads: a row must be a multiple of 16 bytes (K % 256 == 0)
  if (d->shared_ffn > 0 && d->shared_type == MOE_TYPE_Q8_0 && (d->shared_ffn % 256)) return MOE_ERR_SHAPE;
  if (d->norm != 0 && d->norm != 1) return MOE_ERR_SHAPE;
  if (!(d->eps >= 0.0f)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int check_weights(const moe_layer_desc* d, const moe_layer_weights* w) {
  if (!w) return MOE_ERR_NULL;
  if (!w->router_w || !w->gate || !w->up || !w->down) return MOE_ERR_NULL;
  if (d->norm && !w->norm_w) return MOE_ERR_NULL;
  if (d->shared_ffn > 0 && (!w->shared_gate_w || !w->shared_gate || !w->shared_up || !w->shared_down)) return MOE_ERR_NULL;
  const void* p16[] = {w->router_w, w->gate, w->up, w->down, w->shared_gate, w->shared_up, w->shared_down, w->shared_gate_w};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return MOE_ERR_ALIGN;
  if (w->norm_w && !aligned(w->norm_w, 4)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// ---------------------------------------------------------------- workspace layout
static inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const moe_layer_desc* d, int n_layers) {
  WsLayout L;
  size_t o = 0;
  L.counters = o; o += up256(sizeof(unsigned) * kCounterSlots);
  L.xn = o; o += up256(sizeof(float) * d->hidden);
  L.xq = o; o += up256((size_t)(d->hidden / 32) * kQ81Bytes);
  L.logits = o; o += up256(sizeof(float) * (d->n_experts + 1));
  L.ids = o; o += up256(sizeof(int32_t) * d->top_k);
  L.wts = o; o += up256(sizeof(float) * d->top_k);
  L.sg = o; o += up256(sizeof(float));
  L.h = o; o += up256(sizeof(float) * (size_t)d->top_k * d->ffn);
  L.hs = o; o += up256(sizeof(float) * (size_t)(d->shared_ffn > 0 ? d->shared_ffn : 1));
  L.res = o; o += up256(sizeof(uint16_t) * d->hidden);
  L.routed = o; o += up256(sizeof(uint16_t) * d->hidden);
  L.shared = o; o += up256(sizeof(uint16_t) * d->hidden);
  L.u1 = o; o += up256(sizeof(uint16_t) * d->hidden);
  L.table = o; o += up256(sizeof(moe_layer_weights) * (size_t)(n_layers > 0 ? n_layers : 1));
  L.bound = o; o += up256(sizeof(int) * 4);
  // exchange buffers of the persistent stack (their sizes do not depend on the grid)
  StackGeom g;
  if (stack_geometry(d, 256, &g) == MOE_OK) {
    stack_ws_layout(&g, o);
    L.stack = o;
    o = g.w_end;
  } else {
    L.stack = 0;
  }
  L.total = o;
  return L;
}

// ---------------------------------------------------------------- launch helpers
int launch_norm(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, const float* w, int H, int n_tok,
                float eps, uint16_t* out_sum, float* xn, void* xq, int do_norm, hipStream_t st) {
  hipLaunchKernelGGL(k_add_rmsnorm, dim3(n_tok), dim3(kNormThreads), 0, st, res, rt, sh, w, H, eps, out_sum, xn,
                     (uint8_t*)xq, do_norm);
  return launch_ok();
}

int launch_quantize(const float* x, int n, void* xq, hipStream_t st) {
  int blocks = (n + kNormThreads - 1) / kNormThreads;
  hipLaunchKernelGGL(k_quantize_q81, dim3(blocks), dim3(kNormThreads), 0, st, x, n, (uint8_t*)xq);
  return launch_ok();
}

int launch_router(const float* xn, const float* W, const float* wsg, int n_tok, int H, int E, int k, float* logits,
                  float* user_logits, int32_t* ids, float* wts, float* sg, unsigned* counters, hipStream_t st) {
  const int nrows = E + (wsg ? 1 : 0);
  const int ngroups = (n_tok + kRouterTok - 1) / kRouterTok;
  // one counter per 128-byte line when the counter area has room for it, and
  // eight sub-counters per token group when it has room for those too
  constexpr int kSub = 8;
  const bool split = ngroups * (kSub + 1) * 32 <= kCounterSlots;
  const int nsub = split ? kSub : 0;
  const int cstride = (split || ngroups * 32 <= kCounterSlots) ? 32 : 1;
  hipLaunchKernelGGL(k_router_topk, dim3((nrows + kRouterRpb - 1) / kRouterRpb, ngroups), dim3(kRouterThreads), 0, st,
                     xn, W, wsg, n_tok, H, E, k, logits, user_logits, ids, wts, sg, counters, cstride, nsub);
  return launch_ok();
}

int launch_norm_router(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, const float* norm_w, const float* W,
                       const float* wsg, int H, int E, float eps, float* xn, void* xq, float* logits,
                       float* user_logits, hipStream_t st) {
  NormRouterArgs a;
  a.res = res;
  a.rt = rt;
  a.sh = sh;
  a.norm_w = norm_w;
  a.W = W;
  a.wsg = wsg;
  a.xn = xn;
  a.xq = (uint8_t*)xq;
  a.logits = logits;
  a.user_logits = user_logits;
  a.H = H;
  a.E = E;
  a.eps = eps;
  const int nrows = E + (wsg ? 1 : 0);
  const size_t lds = 2 * (size_t)kib_up(4L * H) + 8 * (size_t)H;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)k_norm_router, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return MOE_ERR_HIP;
  hipLaunchKernelGGL(k_norm_router, dim3(nrows), dim3(kNormThreads), lds, st, a);
  return launch_ok();
}

size_t gate_up_lds(int H, int R, int rtype) {
  const long rb = row_bytes(rtype, H);
  size_t act = (size_t)H + 2 * sizeof(float) * (H / 32);
  size_t stage = 2 * (size_t)kib_up((long)R * rb);
  size_t part = sizeof(double) * 2 * (size_t)R * tasks_per_row(rtype, H);
  return stage + part + act;
}

// the kernel's static LDS (the selection's logits, keys and candidates) comes
// on top of the dynamic part
constexpr size_t kGateUpStaticLds = 8 * 1024;
int pick_gate_up_rows(int H, int rtype) {
  int R = kGateUpRows;
  while (R > 1 && gate_up_lds(H, R, rtype) > kLdsBudget - kGateUpStaticLds) R >>= 1;
  return R;
}

int launch_gate_up(const moe_layer_desc* d, const moe_layer_weights* w, const void* xq, const int32_t* ids, float* h,
                   float* hs, hipStream_t st, const GateUpSelect* sel) {
  GateUpArgs a;
  a.xq = (const uint8_t*)xq;
  a.ids = sel ? nullptr : ids;
  a.logits = sel ? sel->logits : nullptr;
  a.ids_out = sel ? sel->ids : nullptr;
  a.wts_out = sel ? sel->wts : nullptr;
  a.sg_out = sel ? sel->sg : nullptr;
  a.has_sg = d->shared_ffn > 0;
  a.res = sel ? sel->res : nullptr;
  a.rt = sel ? sel->rt : nullptr;
  a.sh = sel ? sel->sh : nullptr;
  a.out_sum = sel ? sel->out_sum : nullptr;
  a.gate = (const uint8_t*)w->gate;
  a.up = (const uint8_t*)w->up;
  a.sgate = (const uint8_t*)w->shared_gate;
  a.sup = (const uint8_t*)w->shared_up;
  a.h = h;
  a.hs = hs;
  a.H = d->hidden;
  a.F = d->ffn;
  a.Fs = d->shared_ffn;
  a.k = d->top_k;
  a.E = d->n_experts;
  a.type = d->gate_up_type;
  a.stype = d->shared_type;
  const int Rr = pick_gate_up_rows(d->hidden, MOE_TYPE_Q4_K);
  const int Rs = d->shared_ffn > 0 ? pick_gate_up_rows(d->hidden, d->shared_type) : Rr;
  a.R = Rr < Rs ? Rr : Rs;
  a.cpe = (a.F + a.R - 1) / a.R;
  a.cps = a.Fs > 0 ? (a.Fs + a.R - 1) / a.R : 0;
  size_t lds = gate_up_lds(a.H, a.R, MOE_TYPE_Q4_K);
  if (a.Fs > 0) {
    size_t l2 = gate_up_lds(a.H, a.R, a.stype);
    lds = l2 > lds ? l2 : lds;
  }
  const int nblk = a.k * a.cpe + a.cps;
  hipLaunchKernelGGL(k_gate_up, dim3(nblk), dim3(kFfnThreads), lds, st, a);
  return launch_ok();
}

size_t down_lds(const moe_layer_desc* d, int Ro) {
  const int Kp = pad_k(d->down_type, d->ffn);
  const int Kps = d->shared_ffn > 0 ? pad_k(d->shared_type, d->shared_ffn) : 0;
  const int k = d->top_k;
  size_t acts = (size_t)k * Kp + Kps + 2 * sizeof(float) * ((size_t)k * (Kp / 32) + Kps / 32) + 16;
  const long rb = row_bytes(d->down_type, Kp);
  const long rbs = d->shared_ffn > 0 ? row_bytes(d->shared_type, Kps) : 0;
  size_t stage = (size_t)k * kib_up((long)Ro * rb) + (size_t)kib_up((long)Ro * rbs);
  size_t part = sizeof(double) * ((size_t)k * Ro * tasks_per_row(d->down_type, Kp) +
                                  (size_t)Ro * (d->shared_ffn > 0 ? tasks_per_row(d->shared_type, Kps) : 0));
  size_t y = sizeof(float) * (size_t)(k + 1) * Ro;
  return acts + stage + part + y + 32;
}

int pick_down_rows(const moe_layer_desc* d) {
  int Ro = kDownRows;
  while (Ro > 1 && down_lds(d, Ro) > kLdsBudget) Ro >>= 1;
  return Ro;
}

int launch_down(const moe_layer_desc* d, const moe_layer_weights* w, const float* h, const float* hs, const int32_t* ids,
                const float* wts, const float* sg, uint16_t* routed, uint16_t* shared, hipStream_t st) {
  DownArgs a;
  a.h = h;
  a.hs = hs;
  a.ids = ids;
  a.wts = wts;
  a.sg = sg;
  a.down = (const uint8_t*)w->down;
  a.sdown = (const uint8_t*)w->shared_down;
  a.routed = routed;
  a.shared = shared;
  a.H = d->hidden;
  a.F = d->ffn;
  a.Fs = d->shared_ffn;
  a.k = d->top_k;
  a.E = d->n_experts;
  a.dtype = d->down_type;
  a.stype = d->shared_ffn > 0 ? d->shared_type : MOE_TYPE_Q4_K;
  a.Kp = pad_k(d->down_type, d->ffn);
  a.Kps = d->shared_ffn > 0 ? pad_k(d->shared_type, d->shared_ffn) : 0;
  a.Ro = pick_down_rows(d);
  if (down_lds(d, a.Ro) > kLdsBudget) return MOE_ERR_UNSUPPORTED;
  const int nblk = (a.H + a.Ro - 1) / a.Ro;
  const bool q5 = a.dtype == MOE_TYPE_Q5_K, s8 = a.stype == MOE_TYPE_Q8_0;
  auto fn = q5 ? (s8 ? k_down_combine<MOE_TYPE_Q5_K, MOE_TYPE_Q8_0> : k_down_combine<MOE_TYPE_Q5_K, MOE_TYPE_Q4_K>)
               : (s8 ? k_down_combine<MOE_TYPE_Q4_K, MOE_TYPE_Q8_0> : k_down_combine<MOE_TYPE_Q4_K, MOE_TYPE_Q4_K>);
  hipLaunchKernelGGL(fn, dim3(nblk), dim3(kFfnThreads), down_lds(d, a.Ro), st, a);
  return launch_ok();
}

int launch_fill(void* p, size_t n_u32, uint32_t v, hipStream_t st) {
  if (n_u32 == 0) return MOE_OK;
  int blocks = (int)((n_u32 + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, n_u32, v);
  return launch_ok();
}

// Plain streaming read of n16 16-byte words (the achievable HBM read rate):
// each lane folds its words with xor and one lane per block writes the result.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* p, size_t n16, uint32_t* out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {   // four loads in flight per lane
    const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride), d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a ^ b) ^ (c ^ d);
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9e3779b9u || threadIdx.x == 0) out[blockIdx.x] = r;
}

int launch_stream_read(const void* p, size_t bytes, uint32_t* out, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(256), 0, st, (const u32x4*)p, bytes / 16, out);
  return launch_ok();
}

int launch_test_q81_groups(const float* x, int n, void* xq, hipStream_t st) {
  const int nblk = n / 32;
  hipLaunchKernelGGL(k_test_q81_groups, dim3((nblk + kQ81TestBlocks - 1) / kQ81TestBlocks), dim3(kQ81TestThreads), 0,
                     st, x, nblk, (uint8_t*)xq);
  return launch_ok();
}

int launch_subblock_dots(const void* rows, int type, int K, int n_rows, const void* xq, int32_t* out, hipStream_t st) {
  size_t lds = (size_t)K + 2 * sizeof(float) * (K / 32) + 16 + row_bytes(type, K) + 16;
  hipLaunchKernelGGL(k_subblock_dots, dim3(n_rows), dim3(kFfnThreads), lds, st, (const uint8_t*)rows, type, K,
                     (const uint8_t*)xq, out);
  return launch_ok();
}

}  // namespace moe
