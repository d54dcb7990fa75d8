// Load-time requantisation of weight rows to Q4_K ([P359] Summary: the shared
// expert stored as Q8_0 and the routed down projection stored as Q5_K are
// re-quantised to Q4_K once, when the model is loaded, so that the per-token
// reads shrink).
//
// The quantiser is the min/max rule the library documents for this step: the
// source values are decoded exactly and rounded once to fp32; per 32-value
// sub-block lo = min(0, min x), hi = max x, step = (hi - lo)/15, off = -lo;
// d = f16(max step / 63), dmin = f16(max off / 63); sc and m are the nearest
// integers (ties to even) to step/d and off/dmin, clamped to 0..63; each code
// is the nearest integer to (x + dmin*m)/(d*sc), clamped to 0..15.  Every
// step is one fp32 operation rounded to nearest, so the bytes do not depend
// on how the work is split.
//
// One wave per 256-value superblock: lane l holds values 4l..4l+3, so the 8
// lanes of a sub-block reduce its min and max over DPP, and the sub-blocks'
// maxima meet over the rest of the wave.  The codes are packed through LDS.
#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kRqThreads = 256, kRqWaves = kRqThreads / 64;

static inline int rq_launch_ok() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

__device__ __forceinline__ uint16_t ld_u16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

// the lane's 4 source values (elements 4*lane .. 4*lane + 3 of the superblock)
template <int SRC>
__device__ __forceinline__ void rq_decode(const uint8_t* s, int lane, float x[4]) {
  if constexpr (SRC == MOE_TYPE_Q8_0) {
    // 8 blocks of 34 bytes; block lane/8, codes 4*(lane%8) .. +3 (2-byte aligned)
    const uint8_t* blk = s + 34 * (lane >> 3);
    const float d = f16_to_f32(ld_u16(blk));
    const uint32_t c = (uint32_t)ld_u16(blk + 2 + 4 * (lane & 7)) | ((uint32_t)ld_u16(blk + 4 + 4 * (lane & 7)) << 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = d * (float)(int8_t)(c >> (8 * i));   // exact: 11 x 8 bits
  } else {
    const uint4 hdr = *reinterpret_cast<const uint4*>(s);
    const int j = lane >> 3, p = j >> 1, hi = j & 1, l0 = 4 * (lane & 7);
    int sc, m;
    kquant_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
    const float d = f16_to_f32(hdr.x), dmin = f16_to_f32(hdr.x >> 16);
    const int qs_off = (SRC == MOE_TYPE_Q5_K) ? 48 : 16;
    const uint32_t qs = *reinterpret_cast<const uint32_t*>(s + qs_off + 32 * p + l0);
    uint32_t qh = 0;
    if constexpr (SRC == MOE_TYPE_Q5_K) qh = *reinterpret_cast<const uint32_t*>(s + 16 + l0);
    const float a = d * (float)sc, b = dmin * (float)m;   // both exact in fp32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = (int)((qs >> (8 * i + 4 * hi)) & 0xFu);
      if constexpr (SRC == MOE_TYPE_Q5_K) q |= (int)(((qh >> (8 * i)) >> (2 * p + hi)) & 1u) << 4;
      x[i] = a * (float)q - b;   // a*q exact (22 bits); one rounding of the difference
    }
  }
}

template <int LVL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __uint_as_float(partner_dpp<LVL>(__float_as_uint(v))));
}
template <int LVL>
__device__ __forceinline__ float dpp_min(float v) {
  return fminf(v, __uint_as_float(partner_dpp<LVL>(__float_as_uint(v))));
}
// maximum over the wave (the 8 sub-blocks' values agree within their groups)
__device__ __forceinline__ float groups_max(float v) {
  v = dpp_max<3>(v);
  const Pair32 a = swap16(__float_as_uint(v));
  v = fmaxf(__uint_as_float(a.a), __uint_as_float(a.b));
  const Pair32 c = swap32(__float_as_uint(v));
  return fmaxf(__uint_as_float(c.a), __uint_as_float(c.b));
}
__device__ __forceinline__ float plus_zero(float v) { return (v == 0.0f) ? 0.0f : v; }   // -0 -> +0

template <int SRC, int SB_BYTES>
__global__ __launch_bounds__(kRqThreads) void k_requant_q4k(const uint8_t* src, long n_sb, uint8_t* dst) {
  __shared__ __attribute__((aligned(16))) uint8_t qbuf[kRqWaves][256];
  __shared__ int scm[kRqWaves][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long sb = (long)blockIdx.x * kRqWaves + wave;
  if (sb >= n_sb) return;   // the whole wave leaves; no workgroup barrier follows
  float x[4];
  rq_decode<SRC>(src + sb * SB_BYTES, lane, x);
  // sub-block min / max over its 8 lanes
  float mn = fminf(fminf(x[0], x[1]), fminf(x[2], x[3]));
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mn = dpp_min<2>(dpp_min<1>(dpp_min<0>(mn)));
  mx = dpp_max<2>(dpp_max<1>(dpp_max<0>(mx)));
  const float lo = mn < 0.0f ? mn : 0.0f;
  const float step = (mx - lo) / 15.0f;
  const float off = 0.0f - lo;   // +0 for lo = 0 (the sign of a zero does not reach a decision)
  const float maxstep = plus_zero(groups_max(step)), maxoff = plus_zero(groups_max(off));
  const uint32_t d16 = f32_to_f16(maxstep / 63.0f), m16 = f32_to_f16(maxoff / 63.0f);
  const float d = f16_to_f32(d16), dmin = f16_to_f32(m16);
  const float ra = (d > 0.0f) ? rintf(step / d) : 0.0f, rb = (dmin > 0.0f) ? rintf(off / dmin) : 0.0f;
  const int sc = (int)fminf(fmaxf(ra, 0.0f), 63.0f), m = (int)fminf(fmaxf(rb, 0.0f), 63.0f);
  const float es = d * (float)sc, eo = dmin * (float)m;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int q = 0;
    if (es > 0.0f) q = (int)fminf(fmaxf(rintf((x[i] + eo) / es), 0.0f), 15.0f);
    packed |= (uint32_t)q << (8 * i);
  }
  reinterpret_cast<uint32_t*>(qbuf[wave])[lane] = packed;
  if ((lane & 7) == 0) {
    scm[wave][lane >> 3] = sc;
    scm[wave][8 + (lane >> 3)] = m;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  uint8_t* o = dst + sb * 144;
  // qs byte 32p + l = code 64p + l | code 64p + 32 + l << 4; lane writes bytes 2*lane, 2*lane + 1
  {
    const int i0 = 2 * lane, p = i0 >> 5, l = i0 & 31;
    const uint8_t* qb = qbuf[wave];
    const uint32_t b0 = qb[64 * p + l] | (qb[64 * p + 32 + l] << 4);
    const uint32_t b1 = qb[64 * p + l + 1] | (qb[64 * p + 33 + l] << 4);
    *reinterpret_cast<uint16_t*>(o + 16 + i0) = (uint16_t)(b0 | (b1 << 8));
  }
  if (lane == 0) {
    *reinterpret_cast<uint16_t*>(o) = (uint16_t)d16;
    *reinterpret_cast<uint16_t*>(o + 2) = (uint16_t)m16;
  }
  if (lane < 12) {
    const int* s8 = scm[wave];
    const int j = lane & 3;
    uint32_t v;
    if (lane < 4) v = (s8[j] & 63) | ((s8[j + 4] >> 4) << 6);
    else if (lane < 8) v = (s8[8 + j] & 63) | ((s8[8 + j + 4] >> 4) << 6);
    else v = (s8[j + 4] & 15) | ((s8[8 + j + 4] & 15) << 4);
    o[4 + lane] = (uint8_t)v;
  }
}

// The same quantiser with one lane per 32-value sub-block: lane L of a wave
// takes sub-block L % 8 of superblock 8w + L / 8, decodes its 32 values,
// reduces their min/max in the lane, meets the other 7 lanes of the
// superblock over DPP for the maxima, and quantises its 32 values.  Every
// value goes through the same fp32 operations as above, so the bytes are the
// same; the division count per value halves and most cross-lane steps go.
// Needs dst 16-byte aligned (16-byte stores).
template <int SRC, int SB_BYTES>
__global__ __launch_bounds__(kRqThreads) void k_requant_q4k_sub(const uint8_t* src, long n_sb, uint8_t* dst) {
  __shared__ int scm[kRqWaves][8][8][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 7, g8 = lane >> 3;
  const long sb = ((long)blockIdx.x * kRqWaves + wave) * 8 + g8;
  const bool live = sb < n_sb;   // a whole 8-lane group is live or not
  const uint8_t* s = src + (live ? sb : 0) * SB_BYTES;
  float x[32];
  if constexpr (SRC == MOE_TYPE_Q8_0) {
    const uint8_t* blk = s + 34 * j;
    const float d = f16_to_f32(ld_u16(blk));
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const uint32_t c = ld_u16(blk + 2 + i);
      x[i] = d * (float)(int8_t)(c & 0xffu);
      x[i + 1] = d * (float)(int8_t)(c >> 8);
    }
  } else {
    const uint4 hdr = *reinterpret_cast<const uint4*>(s);
    const int p = j >> 1, hi = j & 1;
    int sc, m;
    kquant_scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
    const float a = f16_to_f32(hdr.x) * (float)sc, b = f16_to_f32(hdr.x >> 16) * (float)m;   // exact
    const int qs_off = (SRC == MOE_TYPE_Q5_K) ? 48 : 16;
    const uint4* q4 = reinterpret_cast<const uint4*>(s + qs_off + 32 * p);
    const uint4 qa = q4[0], qb = q4[1];
    const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    uint32_t hw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if constexpr (SRC == MOE_TYPE_Q5_K) {
      const uint4* h4 = reinterpret_cast<const uint4*>(s + 16);
      const uint4 ha = h4[0], hb = h4[1];
      const uint32_t t[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) hw[i] = t[i];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      int q = (int)((qw[i >> 2] >> (8 * (i & 3) + 4 * hi)) & 0xFu);
      if constexpr (SRC == MOE_TYPE_Q5_K) q |= (int)(((hw[i >> 2] >> (8 * (i & 3))) >> (2 * p + hi)) & 1u) << 4;
      x[i] = a * (float)q - b;   // a*q exact (22 bits); one rounding of the difference
    }
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const float lo = mn < 0.0f ? mn : 0.0f;
  const float step = (mx - lo) / 15.0f;
  const float off = 0.0f - lo;
  // maxima over the 8 sub-blocks of the superblock (lanes 8*g8 .. +7)
  const float maxstep = plus_zero(dpp_max<2>(dpp_max<1>(dpp_max<0>(step))));
  const float maxoff = plus_zero(dpp_max<2>(dpp_max<1>(dpp_max<0>(off))));
  const uint32_t d16 = f32_to_f16(maxstep / 63.0f), m16 = f32_to_f16(maxoff / 63.0f);
  const float d = f16_to_f32(d16), dmin = f16_to_f32(m16);
  const float ra = (d > 0.0f) ? rintf(step / d) : 0.0f, rb = (dmin > 0.0f) ? rintf(off / dmin) : 0.0f;
  const int sc = (int)fminf(fmaxf(ra, 0.0f), 63.0f), m = (int)fminf(fmaxf(rb, 0.0f), 63.0f);
  const float es = d * (float)sc, eo = dmin * (float)m;
  // 32 codes as nibbles in byte l of w[] (low nibble for an even sub-block,
  // high for an odd one), then OR-ed with the partner sub-block's
  uint32_t w[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = 0;
      if (es > 0.0f) q = (int)fminf(fmaxf(rintf((x[4 * c + i] + eo) / es), 0.0f), 15.0f);
      v |= (uint32_t)q << (8 * i + 4 * (j & 1));
    }
    w[c] = v;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) w[c] |= partner_dpp<0>(w[c]);
  // the superblock's 8 (sc, m) pairs meet in LDS; lane 0 of the group packs the header
  scm[wave][g8][j][0] = sc;
  scm[wave][g8][j][1] = m;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  if (!live) return;
  uint8_t* o = dst + sb * 144;
  // qs bytes 32p .. 32p+31: the even lane of the pair writes the first 16, the odd one the second
  {
    const int p = j >> 1;
    uint4* q16 = reinterpret_cast<uint4*>(o + 16 + 32 * p + 16 * (j & 1));
    *q16 = (j & 1) ? make_uint4(w[4], w[5], w[6], w[7]) : make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (j == 0) {
    const int(*pm)[2] = scm[wave][g8];
    uint32_t by[12];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      by[i] = (uint32_t)((pm[i][0] & 63) | ((pm[i + 4][0] >> 4) << 6));
      by[4 + i] = (uint32_t)((pm[i][1] & 63) | ((pm[i + 4][1] >> 4) << 6));
      by[8 + i] = (uint32_t)((pm[i + 4][0] & 15) | ((pm[i + 4][1] & 15) << 4));
    }
    uint4 hv;
    hv.x = d16 | (m16 << 16);
    hv.y = by[0] | (by[1] << 8) | (by[2] << 16) | (by[3] << 24);
    hv.z = by[4] | (by[5] << 8) | (by[6] << 16) | (by[7] << 24);
    hv.w = by[8] | (by[9] << 8) | (by[10] << 16) | (by[11] << 24);
    *reinterpret_cast<uint4*>(o) = hv;
  }
}

int launch_requant_q4k(const void* src, int src_type, int n_rows, int K, void* dst, hipStream_t st) {
  const long n_sb = (long)n_rows * (K / 256);
  const dim3 grid((unsigned)((n_sb + kRqWaves - 1) / kRqWaves));
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* d = static_cast<uint8_t*>(dst);
  if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
    // one lane per sub-block: 8 superblocks per wave
    const dim3 g2((unsigned)((n_sb + 8 * kRqWaves - 1) / (8 * kRqWaves)));
    if (src_type == MOE_TYPE_Q8_0)
      hipLaunchKernelGGL((k_requant_q4k_sub<MOE_TYPE_Q8_0, 8 * kQ80Bytes>), g2, dim3(kRqThreads), 0, st, s, n_sb, d);
    else if (src_type == MOE_TYPE_Q5_K)
      hipLaunchKernelGGL((k_requant_q4k_sub<MOE_TYPE_Q5_K, kQ5KBytes>), g2, dim3(kRqThreads), 0, st, s, n_sb, d);
    else
      hipLaunchKernelGGL((k_requant_q4k_sub<MOE_TYPE_Q4_K, kQ4KBytes>), g2, dim3(kRqThreads), 0, st, s, n_sb, d);
    return rq_launch_ok();
  }
  if (src_type == MOE_TYPE_Q8_0)
    hipLaunchKernelGGL((k_requant_q4k<MOE_TYPE_Q8_0, 8 * kQ80Bytes>), grid, dim3(kRqThreads), 0, st, s, n_sb, d);
  else if (src_type == MOE_TYPE_Q5_K)
    hipLaunchKernelGGL((k_requant_q4k<MOE_TYPE_Q5_K, kQ5KBytes>), grid, dim3(kRqThreads), 0, st, s, n_sb, d);
  else
    hipLaunchKernelGGL((k_requant_q4k<MOE_TYPE_Q4_K, kQ4KBytes>), grid, dim3(kRqThreads), 0, st, s, n_sb, d);
  return rq_launch_ok();
}

}  // namespace moe
