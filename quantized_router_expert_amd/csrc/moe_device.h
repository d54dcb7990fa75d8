// moe_device.h -- device-side helpers of the gfx950 MoE decode library.
//
// Block formats (GGUF layouts; the source pages name the formats, [P359] Summary):
//   Q4_K 144 B: d f16 | dmin f16 | scales[12] | qs[128]
//   Q5_K 176 B: d f16 | dmin f16 | scales[12] | qh[32] | qs[128]
//   Q8_0  34 B: d f16 | q int8[32]
//   Q8_1  36 B: d f16 | s f16 | q int8[32]
// A K-quant superblock of 256 elements has 8 sub-blocks of 32 with a 6-bit
// scale sc_j and min m_j each; element value = d*sc_j*q - dmin*m_j.  Byte
// 32g+l of qs carries element 64g+l (low nibble) and 64g+32+l (high nibble).
//
// Arithmetic policy: every integer product of weight codes with activation
// codes goes through v_dot4_i32_i8 and is exact; the per-sub-block scaling,
// every reduction and every normalisation runs in fp64, and a value is
// rounded (to fp32, then to its storage type) only where it is stored.  The
// fp64 work is a few operations per 32 weights, far below what an HBM-bound
// kernel can hide, and it makes each stored value the correctly rounded
// result of the exact per-row sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_TYPE_Q8_0 8
#define MOE_TYPE_Q8_1 9
#define MOE_TYPE_Q4_K 12
#define MOE_TYPE_Q5_K 13

namespace moe {

constexpr int kQ4KBytes = 144;
constexpr int kQ5KBytes = 176;
constexpr int kQ80Bytes = 34;
constexpr int kQ81Bytes = 36;

// ---------------------------------------------------------------- global -> LDS streaming
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Wait for every vector-memory load the wave has issued (the DMA loads below
// are invisible to the compiler's own bookkeeping, so their consumers call this).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS (buffer_load ... lds):
// the wave's 64 lanes fill the 1 KiB at LDS address `lds` (M0) from byte
// offset `off` + 16 * lane of the buffer described by `rsrc`.  Issued from
// inline asm so the compiler does not track it: it would otherwise wait for
// every such load before any LDS read it cannot prove disjoint, which stalls
// the waves that compute while their next rows stream in.  The consumer waits
// explicitly (wait_vmem() in the issuing waves, then a barrier).
__device__ __forceinline__ void lds_dma_1k(v4u rsrc, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(off), "s"(rsrc)
               : "memory", "m0");
}

// Buffer descriptor with hardware range checking: loads past `bytes` read 0.
__device__ __forceinline__ v4u raw_rsrc(const void* p, uint32_t bytes) {
  const unsigned long long a = (unsigned long long)p;
  v4u r;
  r.x = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r.z = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000u;
  return r;
}

// Stream `bytes` from src into LDS dst (1 KiB per wave instruction); waves
// [w0, w0+nw) take chunks round-robin.  The loads hold no registers, so every
// chunk is in flight at once.  dst must have room for the byte count rounded
// up to 1 KiB: lanes past the source end read 0 (range-checked descriptor) and
// write that 0 into the padding.
__device__ __forceinline__ void stage_async(uint8_t* dst, const void* src, uint32_t bytes, int wave, int w0, int nw) {
  if (wave < w0 || wave >= w0 + nw || bytes == 0) return;
  const v4u r = raw_rsrc(src, bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)dst;
  const int lane = threadIdx.x & 63;
  const uint32_t nchunks = (bytes + 1023) >> 10;
  for (uint32_t c = wave - w0; c < nchunks; c += nw)
    lds_dma_1k(r, (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + (c << 10))), (c << 10) + lane * 16);
}

__host__ __device__ constexpr inline int block_bytes(int type) {
  return type == MOE_TYPE_Q4_K ? kQ4KBytes : type == MOE_TYPE_Q5_K ? kQ5KBytes : type == MOE_TYPE_Q8_0 ? kQ80Bytes : kQ81Bytes;
}
__host__ __device__ constexpr inline int block_elems(int type) {
  return (type == MOE_TYPE_Q4_K || type == MOE_TYPE_Q5_K) ? 256 : 32;
}
__host__ __device__ constexpr inline int pad_k(int type, int K) {
  return (K + block_elems(type) - 1) / block_elems(type) * block_elems(type);
}
__host__ __device__ constexpr inline long row_bytes(int type, int K) { return (long)(K / block_elems(type)) * block_bytes(type); }
// Independent work items ("tasks") per row: one per 64 elements for K-quants
// (a 32-byte group of qs = two sub-blocks), one per 32-element block for Q8_0.
__host__ __device__ constexpr inline int tasks_per_row(int type, int K) {
  return (type == MOE_TYPE_Q8_0) ? K / 32 : K / 64;
}

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// round to nearest, ties to even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // both results, then a select: a branch on NaN would cost an exec-mask
  // region per conversion
  const uint32_t u = __float_as_uint(f);
  const uint32_t rn = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;   // round to nearest even
  const uint32_t qn = (u >> 16) | 0x40u;                         // NaN stays a (quiet) NaN
  return (uint16_t)((f != f) ? qn : rn);
}
// binary16 <-> fp32 through the hardware conversions (exact one way, round to
// nearest even the other, subnormals kept).
__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h16 & 0xffffu));
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------------- lane exchange (wave64)
// Butterfly steps over groups of 2, 4, 8, 16, 32, 64 lanes, all on the VALU:
// DPP quad_perm [1,0,3,2] and [2,3,0,1] (xor 1, xor 2), row_half_mirror and
// row_mirror (partner 7-i / 15-i: equivalent to xor 4 / xor 8 once the smaller
// groups agree), and gfx950's permlane16/permlane32 swaps, whose two results
// are the values of lanes l & ~16 and l | 16 (resp. 32) in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
enum { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

struct Pair32 { uint32_t a, b; };  // values of the two lanes of a pair, same in both lanes
__device__ __forceinline__ Pair32 swap16(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {(uint32_t)r[0], (uint32_t)r[1]};
}
__device__ __forceinline__ Pair32 swap32(uint32_t v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {(uint32_t)r[0], (uint32_t)r[1]};
}

// partner value of a 32-bit lane value at butterfly level `lvl` (0..3: DPP)
template <int LVL>
__device__ __forceinline__ uint32_t partner_dpp(uint32_t v) {
  if (LVL == 0) return dpp_u32<kDppXor1>(v);
  if (LVL == 1) return dpp_u32<kDppXor2>(v);
  if (LVL == 2) return dpp_u32<kDppHalfMirror>(v);
  return dpp_u32<kDppMirror>(v);
}

__device__ __forceinline__ double dbl(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t lo32(double d) { return (uint32_t)__builtin_bit_cast(unsigned long long, d); }
__device__ __forceinline__ uint32_t hi32(double d) { return (uint32_t)(__builtin_bit_cast(unsigned long long, d) >> 32); }

template <int LVL>
__device__ __forceinline__ double sum_step_f64(double v) {
  if (LVL < 4) return v + dbl(partner_dpp<LVL>(lo32(v)), partner_dpp<LVL>(hi32(v)));
  const Pair32 l = (LVL == 4) ? swap16(lo32(v)) : swap32(lo32(v));
  const Pair32 h = (LVL == 4) ? swap16(hi32(v)) : swap32(hi32(v));
  return dbl(l.a, h.a) + dbl(l.b, h.b);   // same operand order in both lanes: identical results
}

// sum over aligned groups of `n` lanes (n a power of two, 1..64); every lane of a group gets the sum
__device__ __forceinline__ double group_sum_f64(double v, int n) {
  if (n >= 2) v = sum_step_f64<0>(v);
  if (n >= 4) v = sum_step_f64<1>(v);
  if (n >= 8) v = sum_step_f64<2>(v);
  if (n >= 16) v = sum_step_f64<3>(v);
  if (n >= 32) v = sum_step_f64<4>(v);
  if (n >= 64) v = sum_step_f64<5>(v);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) { return group_sum_f64(v, 64); }

__device__ __forceinline__ float half_wave_max_f32(float v) {  // within aligned groups of 32 lanes
  v = fmaxf(v, __uint_as_float(partner_dpp<0>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(partner_dpp<1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(partner_dpp<2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(partner_dpp<3>(__float_as_uint(v))));
  const Pair32 p = swap16(__float_as_uint(v));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ int half_wave_sum_i32(int v) {
  v += (int)partner_dpp<0>((uint32_t)v);
  v += (int)partner_dpp<1>((uint32_t)v);
  v += (int)partner_dpp<2>((uint32_t)v);
  v += (int)partner_dpp<3>((uint32_t)v);
  const Pair32 p = swap16((uint32_t)v);
  return (int)p.a + (int)p.b;
}

// wave-wide max of 64-bit unsigned keys; every lane gets it
template <int LVL>
__device__ __forceinline__ unsigned long long max_step_u64(unsigned long long v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  unsigned long long o;
  if (LVL < 4) {
    o = ((unsigned long long)partner_dpp<LVL>(hi) << 32) | partner_dpp<LVL>(lo);
    return o > v ? o : v;
  }
  const Pair32 l = (LVL == 4) ? swap16(lo) : swap32(lo);
  const Pair32 h = (LVL == 4) ? swap16(hi) : swap32(hi);
  const unsigned long long a = ((unsigned long long)h.a << 32) | l.a;
  const unsigned long long c = ((unsigned long long)h.b << 32) | l.b;
  return a > c ? a : c;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = max_step_u64<0>(v);
  v = max_step_u64<1>(v);
  v = max_step_u64<2>(v);
  v = max_step_u64<3>(v);
  v = max_step_u64<4>(v);
  return max_step_u64<5>(v);
}

// wave-wide max / min of 32-bit unsigned values; every lane gets the result
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, partner_dpp<0>(v));
  v = max(v, partner_dpp<1>(v));
  v = max(v, partner_dpp<2>(v));
  v = max(v, partner_dpp<3>(v));
  Pair32 p = swap16(v);
  v = max(p.a, p.b);
  p = swap32(v);
  return max(p.a, p.b);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, partner_dpp<0>(v));
  v = min(v, partner_dpp<1>(v));
  v = min(v, partner_dpp<2>(v));
  v = min(v, partner_dpp<3>(v));
  Pair32 p = swap16(v);
  v = min(p.a, p.b);
  p = swap32(v);
  return min(p.a, p.b);
}

// ---------------------------------------------------------------- Q8_1 quantiser
// One 32-element block held by 32 consecutive lanes (one value per lane).
// d32 = amax/127 and the codes x*(1/d32) are fp32 and correctly rounded (a
// float decides an integer here, so the precision is fixed, not widened);
// s = d16 * qsum in fp32 (exact: 11-bit d16 times |qsum| <= 4064), then fp16.
// The empty asm keeps the product a separate fp32 multiply: fused with the
// conversion into one mixed-precision fma with a +0 addend, a -0 product
// (d16 = 0, qsum < 0) would come out +0.
__device__ __forceinline__ uint32_t q81_s16(uint32_t d16, int qsum) {
  float sv = __fmul_rn(f16_to_f32(d16), (float)qsum);
  asm("" : "+v"(sv));
  return f32_to_f16(sv);
}
// codes round half away from zero; d and s = d16*sum(q) are stored as fp16.
struct Q81Lane {
  int q;            // this lane's code
  uint32_t ds;      // d16 | s16 << 16 (same in all 32 lanes)
};
__device__ __forceinline__ Q81Lane quantize_q81_lane(float x) {
  float amax = half_wave_max_f32(fabsf(x));
  Q81Lane r;
  if (amax == 0.0f) { r.q = 0; r.ds = 0u; return r; }
  float d32 = amax / 127.0f;
  float id = 1.0f / d32;
  float t = __fmul_rn(x, id);
  float qf = fminf(fmaxf(roundf(t), -127.0f), 127.0f);
  r.q = (int)qf;
  int qsum = half_wave_sum_i32(r.q);
  uint32_t d16 = f32_to_f16(d32);
  r.ds = d16 | (q81_s16(d16, qsum) << 16);
  return r;
}

// The same quantiser with one lane per 32-element block: the lane reads the
// block's 32 fp32 values from LDS (16-byte aligned), writes its 32 codes to
// dst (16-byte aligned) and returns d16 | s16 << 16.  Same fp32 operations,
// so the same bytes as quantize_q81_lane.
__device__ __forceinline__ uint32_t quantize_q81_block(const float* src, uint8_t* dst) {
  float x[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  if (amax == 0.0f) {
    d4[0] = make_uint4(0, 0, 0, 0);
    d4[1] = make_uint4(0, 0, 0, 0);
    return 0u;
  }
  const float d32 = amax / 127.0f;
  const float id = 1.0f / d32;
  uint32_t w[8];
  int qsum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t pk = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float qf = fminf(fmaxf(roundf(__fmul_rn(x[4 * j + i], id)), -127.0f), 127.0f);
      const int q = (int)qf;
      qsum += q;
      pk |= ((uint32_t)q & 0xffu) << (8 * i);
    }
    w[j] = pk;
  }
  d4[0] = make_uint4(w[0], w[1], w[2], w[3]);
  d4[1] = make_uint4(w[4], w[5], w[6], w[7]);
  const uint32_t d16 = f32_to_f16(d32);
  return d16 | (q81_s16(d16, qsum) << 16);
}

// The same quantiser spread over 8 consecutive lanes per block, 4 values per
// lane (lanes 8j..8j+7 of a wave share block j).  x4 = the lane's 4 values
// (elements 4p..4p+3 of the block, p = lane & 7).  Returns the lane's 4 codes
// packed little-endian; every lane of the group gets ds = d16 | s16 << 16.
// Same fp32 operations as quantize_q81_lane, so the same bytes.  All 8 lanes
// of a group must be active together.
__device__ __forceinline__ uint32_t quantize_q81_oct(float4 x4, uint32_t& ds) {
  float amax = fmaxf(fmaxf(fabsf(x4.x), fabsf(x4.y)), fmaxf(fabsf(x4.z), fabsf(x4.w)));
  amax = fmaxf(amax, __uint_as_float(partner_dpp<0>(__float_as_uint(amax))));
  amax = fmaxf(amax, __uint_as_float(partner_dpp<1>(__float_as_uint(amax))));
  amax = fmaxf(amax, __uint_as_float(partner_dpp<2>(__float_as_uint(amax))));
  // branch-free, so several blocks can be in flight in one lane: an all-zero
  // block computes with a stand-in scale and is replaced by zeros at the end
  const bool zero = (amax == 0.0f);
  const float d32 = (zero ? 1.0f : amax) / 127.0f;
  const float id = 1.0f / d32;
  const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
  uint32_t pk = 0;
  int qsum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float qf = fminf(fmaxf(roundf(__fmul_rn(xs[i], id)), -127.0f), 127.0f);
    const int q = (int)qf;
    qsum += q;
    pk |= ((uint32_t)q & 0xffu) << (8 * i);
  }
  qsum += (int)partner_dpp<0>((uint32_t)qsum);
  qsum += (int)partner_dpp<1>((uint32_t)qsum);
  qsum += (int)partner_dpp<2>((uint32_t)qsum);
  const uint32_t d16 = f32_to_f16(d32);
  ds = zero ? 0u : (d16 | (q81_s16(d16, qsum) << 16));
  return zero ? 0u : pk;
}

// Quantise nblk blocks with threads [tid0, tid0 + nthr) of the workgroup
// (nthr a multiple of 64): block j reads 32 fp32 values from src(j) (LDS,
// 16-byte aligned; nullptr = a zero block) and writes its codes to codes(j)
// (16-byte aligned), d and s to dq[j] and sq[j].  Each lane keeps up to U
// blocks in flight (independent dependency chains).
template <int U, class Src, class Dst>
__device__ __forceinline__ void quantize_q81_blocks(int nblk, Src src, Dst codes, float* dq, float* sq, int tid,
                                                    int nthr) {
  const int n = 8 * nblk;
  for (int i0 = tid; i0 < n; i0 += U * nthr) {
    float4 x4[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * nthr;
      ok[u] = i < n;   // the same for the 8 lanes of a block
      const float* sp = ok[u] ? src(i >> 3) : nullptr;
      x4[u] = sp ? reinterpret_cast<const float4*>(sp)[i & 7] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    uint32_t pk[U], ds[U];
#pragma unroll
    for (int u = 0; u < U; ++u) pk[u] = quantize_q81_oct(x4[u], ds[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * nthr;
      if (ok[u]) {
        const int j = i >> 3, p = i & 7;
        reinterpret_cast<uint32_t*>(codes(j))[p] = pk[u];
        if (p == 0) {
          dq[j] = f16_to_f32(ds[u]);
          sq[j] = f16_to_f32(ds[u] >> 16);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- Q8_1, four lanes per block
// Fast forms of the quantiser's fp32 operations that give the same values as
// the IEEE operations they replace, for the inputs they are used on:
//  * amax/127 as q = RN(amax * RN(1/127)) corrected once with the exact
//    remainder fma(-q, 127, amax): Markstein's correction step (P. Markstein,
//    IBM J. Res. Dev. 34(1), 1990), correctly rounded because RN(1/127) is the
//    correctly rounded reciprocal and q is within an ulp of the quotient;
//  * 1/d as one Newton step y + y*(1 - d*y) from the hardware reciprocal y;
//  * round-half-away-from-zero as an fp64 add of +-1/2 (exact: a 24-bit value
//    plus 1/2 needs at most 26 bits) followed by truncation.
// All three were compared with the IEEE operations over every fp32
// significand (exponents -120..120 for the first two, every |v| <= 128 for the
// rounding) with no difference.  Blocks whose maximum lies outside
// [2^-100, 2^100] (so that no intermediate leaves the normal range) or that
// hold a NaN take the IEEE operations instead; the choice is made per wave.
__device__ __forceinline__ float div127_rn(float a) {
  constexpr float y = 1.0f / 127.0f;
  const float q = a * y;
  const float r = __builtin_fmaf(-q, 127.0f, a);
  return __builtin_fmaf(r, y, q);
}
__device__ __forceinline__ float recip_rn(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, y, 1.0f), y, y);
}
__device__ __forceinline__ int round_away_i32(float v) {
  const double w = (double)v;
  return (int)(w + __builtin_copysign(0.5, w));
}
__device__ __forceinline__ uint32_t pack_i8x4(int q0, int q1, int q2, int q3) {
  return ((uint32_t)q0 & 0xffu) | (((uint32_t)q1 & 0xffu) << 8) | (((uint32_t)q2 & 0xffu) << 16) |
         ((uint32_t)q3 << 24);
}

// One block spread over LPB consecutive lanes (2 or 4), V = 32/LPB values
// each (x = elements V*p .. V*p+V-1 of the block, p = lane % LPB); amax = the
// block's max |x| (already reduced over the LPB lanes).  IEEE selects the
// plain IEEE operations.  Same bytes as quantize_q81_lane either way.  w gets
// the lane's V codes (little-endian, V/4 dwords); returns d16 | s16 << 16
// (same in the LPB lanes of the block).
template <int LPB, bool IEEE>
__device__ __forceinline__ uint32_t q81_group(const float* x, float amax, uint32_t* w) {
  constexpr int V = 32 / LPB;
  const bool zero = (amax == 0.0f);
  const float a = zero ? 1.0f : amax;   // stand-in scale for an all-zero block
  const float d32 = IEEE ? a / 127.0f : div127_rn(a);
  const float id = IEEE ? 1.0f / d32 : recip_rn(d32);
  int qsum = 0;
#pragma unroll
  for (int c = 0; c < V / 4; ++c) {
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = __fmul_rn(x[4 * c + i], id);
      // |t| <= 127(1 + 2^-22) when the fast operations apply: no clamp needed
      q[i] = IEEE ? (int)fminf(fmaxf(roundf(t), -127.0f), 127.0f) : round_away_i32(t);
    }
    w[c] = zero ? 0u : pack_i8x4(q[0], q[1], q[2], q[3]);
    qsum = __builtin_amdgcn_sdot4((int)w[c], 0x01010101, qsum, false);
  }
  qsum += (int)partner_dpp<0>((uint32_t)qsum);
  if (LPB >= 4) qsum += (int)partner_dpp<1>((uint32_t)qsum);
  const uint32_t d16 = f32_to_f16(d32);
  return zero ? 0u : (d16 | (q81_s16(d16, qsum) << 16));
}

// Quantise nblk blocks with threads [tid, ...) stepping by nthr (a multiple of
// 64), LPB lanes per block (2 or 4) and up to U blocks in flight per lane.
// Block j's 32 fp32 values are at base + off(j) (LDS, 16-byte aligned;
// off(j) < 0 = a zero block); its codes go to codes(j) (16-byte aligned), d
// and s to dq[j] and sq[j].
template <int LPB, int U, class Off, class Dst>
__device__ __forceinline__ void quantize_q81_groups(int nblk, const float* base, Off off, Dst codes, float* dq,
                                                    float* sq, int tid, int nthr) {
  constexpr int V = 32 / LPB;
  const int n = LPB * nblk;
  for (int i0 = tid; i0 < n; i0 += U * nthr) {
    float x[U][V], amax[U];
    bool live[U];
    bool slow = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * nthr;
      live[u] = i < n;   // the same for the LPB lanes of a block
      const int o = live[u] ? off(i / LPB) : -1;
      const float4* p = reinterpret_cast<const float4*>(base + (o < 0 ? 0 : o) + V * (i % LPB));
      float m = 0.0f;
      bool nan = false;
#pragma unroll
      for (int c = 0; c < V / 4; ++c) {
        const float4 v = p[c];
        const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[u][4 * c + e] = (o < 0) ? 0.0f : xs[e];
          m = fmaxf(m, fabsf(x[u][4 * c + e]));
          nan |= (x[u][4 * c + e] != x[u][4 * c + e]);
        }
      }
      m = fmaxf(m, __uint_as_float(partner_dpp<0>(__float_as_uint(m))));
      if (LPB >= 4) m = fmaxf(m, __uint_as_float(partner_dpp<1>(__float_as_uint(m))));
      amax[u] = m;
      slow |= nan || !(m == 0.0f || (m >= 0x1p-100f && m <= 0x1p100f));
    }
    uint32_t w[U][V / 4], ds[U];
    if (__builtin_expect(__any(slow), 0)) {
#pragma unroll
      for (int u = 0; u < U; ++u) ds[u] = q81_group<LPB, true>(x[u], amax[u], w[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) ds[u] = q81_group<LPB, false>(x[u], amax[u], w[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * nthr;
      if (live[u]) {
        const int j = i / LPB, p = i % LPB;
        uint32_t* dst = reinterpret_cast<uint32_t*>(codes(j)) + (V / 4) * p;
        if constexpr (V == 16) *reinterpret_cast<uint4*>(dst) = make_uint4(w[u][0], w[u][1], w[u][2], w[u][3]);
        else *reinterpret_cast<uint2*>(dst) = make_uint2(w[u][0], w[u][1]);
        if (p == 0) {
          dq[j] = f16_to_f32(ds[u]);
          sq[j] = f16_to_f32(ds[u] >> 16);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- K-quant scales
// 6-bit scale and min of sub-block j from the 12 scale bytes held as three
// dwords s0 (bytes 0..3), s1 (4..7), s2 (8..11).
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }
__device__ __forceinline__ void kquant_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j, int& sc, int& m) {
  // branch-free (lanes of a wave decode different sub-blocks)
  const int i = j & 3;
  const uint32_t b0 = byte_of(s0, i), b1 = byte_of(s1, i), b2 = byte_of(s2, i);
  const bool hi = j >= 4;
  sc = (int)(hi ? ((b2 & 0xfu) | ((b0 >> 6) << 4)) : (b0 & 63u));
  m = (int)(hi ? ((b2 >> 4) | ((b1 >> 6) << 4)) : (b1 & 63u));
}

// ---------------------------------------------------------------- integer dots
// 32-byte group g of a K-quant superblock against the two activation blocks it
// pairs with (sub-blocks 2g and 2g+1).  qs: 8 dwords of codes (low/high nibbles);
// qh: 8 dwords of fifth bits (Q5_K) or nullptr; alo/ahi: 8 dwords of int8 codes.
template <bool Q5>
__device__ __forceinline__ void kquant_group_dots(const uint32_t qs[8], const uint32_t* qh, int g,
                                                  const uint32_t alo[8], const uint32_t ahi[8], int& Dlo, int& Dhi) {
  int lo[2] = {0, 0}, hi[2] = {0, 0};   // two independent chains each (exact integer sums)
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t wl = qs[t] & 0x0f0f0f0fu;
    uint32_t wh = (qs[t] >> 4) & 0x0f0f0f0fu;
    if (Q5) {
      wl |= ((qh[t] >> (2 * g)) & 0x01010101u) << 4;
      wh |= ((qh[t] >> (2 * g + 1)) & 0x01010101u) << 4;
    }
    lo[t & 1] = __builtin_amdgcn_sdot4((int)wl, (int)alo[t], lo[t & 1], false);
    hi[t & 1] = __builtin_amdgcn_sdot4((int)wh, (int)ahi[t], hi[t & 1], false);
  }
  Dlo = lo[0] + lo[1];
  Dhi = hi[0] + hi[1];
}

__device__ __forceinline__ int q8_block_dot(const uint32_t w[8], const uint32_t a[8]) {
  int acc[2] = {0, 0};
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t & 1] = __builtin_amdgcn_sdot4((int)w[t], (int)a[t], acc[t & 1], false);
  return acc[0] + acc[1];
}

// Activations staged in LDS: int8 codes [K] (16-byte aligned), per-block d and s as float.
struct ActLds {
  const uint8_t* codes;
  const float* d;
  const float* s;
};

__device__ __forceinline__ void lds_load8(const uint8_t* p, uint32_t out[8]) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  uint4 a = v[0], b = v[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// One task of a K-quant row: superblock b, group g.  blk points at the block
// (LDS or global, 16-byte aligned).  Returns the exact fp64 contribution
//   d*sc_lo*da_lo*Dlo - dmin*m_lo*sa_lo + d*sc_hi*da_hi*Dhi - dmin*m_hi*sa_hi.
template <int TYPE>
__device__ __forceinline__ double kquant_task(const uint8_t* blk, int b, int g, const ActLds& act) {
  const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
  uint32_t qs[8], qh[8];
  if (TYPE == MOE_TYPE_Q5_K) {
    lds_load8(blk + 16, qh);
    lds_load8(blk + 48 + 32 * g, qs);
  } else {
    lds_load8(blk + 16 + 32 * g, qs);
  }
  const int jlo = 8 * b + 2 * g;
  uint32_t alo[8], ahi[8];
  lds_load8(act.codes + 32 * jlo, alo);
  lds_load8(act.codes + 32 * (jlo + 1), ahi);
  int Dlo, Dhi;
  kquant_group_dots<TYPE == MOE_TYPE_Q5_K>(qs, qh, g, alo, ahi, Dlo, Dhi);
  int sclo, mlo, schi, mhi;
  kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g, sclo, mlo);
  kquant_scale_min(hdr.y, hdr.z, hdr.w, 2 * g + 1, schi, mhi);
  const double d = (double)f16_to_f32(hdr.x);
  const double dmin = (double)f16_to_f32(hdr.x >> 16);
  const double t1 = d * (double)sclo * (double)act.d[jlo] * (double)Dlo;
  const double t2 = dmin * (double)mlo * (double)act.s[jlo];
  const double t3 = d * (double)schi * (double)act.d[jlo + 1] * (double)Dhi;
  const double t4 = dmin * (double)mhi * (double)act.s[jlo + 1];
  return ((t1 - t2) + t3) - t4;
}

// Read 34-byte Q8_0 block j of a row staged in LDS (row start 16-byte aligned):
// block offset 34j is 2-byte aligned, so dwords are assembled with a funnel shift.
__device__ __forceinline__ void q80_load(const uint8_t* row, int j, float& d, uint32_t w[8]) {
  const int off = 34 * j;
  const uint32_t* base = reinterpret_cast<const uint32_t*>(row + (off & ~3));
  const int sh = off & 3;  // 0 or 2
  uint32_t v[9];  // 36 bytes from the aligned base cover the block (may read 2 bytes past it)
#pragma unroll
  for (int t = 0; t < 9; ++t) v[t] = base[t];
  const uint32_t first = sh ? (v[0] >> 16) : (v[0] & 0xffffu);
  d = f16_to_f32(first);
  // codes start at byte off+2
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (sh == 0) w[t] = __builtin_amdgcn_alignbyte(v[t + 1], v[t], 2);
    else w[t] = v[t + 1];
  }
}

__device__ __forceinline__ double q80_task(const uint8_t* row, int j, const ActLds& act) {
  float d;
  uint32_t w[8], a[8];
  q80_load(row, j, d, w);
  lds_load8(act.codes + 32 * j, a);
  int D = q8_block_dot(w, a);
  return (double)d * (double)act.d[j] * (double)D;
}

template <int TYPE>
__device__ __forceinline__ double row_task(const uint8_t* row, int t, const ActLds& act) {
  if (TYPE == MOE_TYPE_Q8_0) return q80_task(row, t, act);
  const int b = t >> 2, g = t & 3;
  return kquant_task<TYPE>(row + (long)b * block_bytes(TYPE), b, g, act);
}

// A weight row and the activations it is dotted with.
struct RowRef {
  const uint8_t* row;
  ActLds act;
};

// Row values of nrows rows computed by lane groups: the T tasks of a row sit in
// TP = the next power of two >= min(T, 64) consecutive lanes (lanes past T add
// 0; with T > 64 a lane takes tasks t, t+64, ...), and a DPP/permlane sum over
// the group gives the row's fp64 value.  Waves [0, nw) split the rows (wave
// index `wave`); out[r] receives row r.  rowfn(r) returns the RowRef of row r.
// Each lane works on two rows at once (this round's and the next round's), so
// two independent dependency chains are in flight; the second is skipped when
// the wave has no row there.
template <int TYPE, class RowFn>
__device__ __forceinline__ void rows_dot(int nrows, int T, RowFn rowfn, double* out, int wave, int nw) {
  int TP = 1;
  while (TP < T && TP < 64) TP <<= 1;
  const int rpi = 64 / TP;
  const int lane = threadIdx.x & 63;
  const int rl = lane / TP, t0 = lane - rl * TP;
  const int step = nw * rpi;
  const int tt = (t0 < T) ? t0 : 0;
  for (int r0 = wave * rpi; r0 < nrows; r0 += 2 * step) {
    const int ra = r0 + rl, rb = r0 + step + rl;
    const bool two = (r0 + step) < nrows;   // wave-uniform
    const RowRef A = rowfn(ra < nrows ? ra : nrows - 1);
    double va = row_task<TYPE>(A.row, tt, A.act);
    double vb = 0.0;
    RowRef B = A;
    if (two) {
      B = rowfn(rb < nrows ? rb : nrows - 1);
      vb = row_task<TYPE>(B.row, tt, B.act);
    }
    if (t0 >= T) { va = 0.0; vb = 0.0; }
    for (int t = t0 + 64; t < T; t += 64) {
      va += row_task<TYPE>(A.row, t, A.act);
      if (two) vb += row_task<TYPE>(B.row, t, B.act);
    }
    va = group_sum_f64(va, TP);
    if (two) vb = group_sum_f64(vb, TP);
    if (t0 == 0) {
      if (ra < nrows) out[ra] = va;
      if (two && rb < nrows) out[rb] = vb;
    }
  }
}

__device__ __forceinline__ double silu_f64(double x) { return x / (1.0 + exp(-x)); }

// The value lane `src` (any lane of the wave) holds, as a double.
__device__ __forceinline__ double lane_f64(double v, int src) {
  const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)lo32(v));
  const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)hi32(v));
  return dbl((uint32_t)lo, (uint32_t)hi);
}

// SwiGLU outputs of npairs (gate row, up row) pairs: h_p = f32(silu(g_p) * u_p)
// with g_p, u_p the fp32-rounded row values.  A pair takes 2*TP consecutive
// lanes (TP = the next power of two >= min(T, 32)): the gate row's tasks in
// the first TP, the up row's in the next TP (a lane takes tasks t, t+TP, ...);
// each half is summed by a lane-group tree, the up sum travels to the gate
// half's first lane, which calls store(p, h).  Waves [0, nw) (index `wave`)
// take 32/TP pairs per pass, two passes' worth at a time (two independent
// chains per lane).  pairfn(p) returns {gate row, up row, activations}.
struct PairRef {
  const uint8_t* gate;
  const uint8_t* up;
  ActLds act;
};
template <int TYPE, class PairFn, class Store>
__device__ __forceinline__ void pair_h(int npairs, int T, PairFn pairfn, Store store, int wave, int nw) {
  int TP = 1;
  while (TP < T && TP < 32) TP <<= 1;
  const int ppw = 32 / TP;
  const int lane = threadIdx.x & 63;
  const int ps = lane / (2 * TP), half = (lane / TP) & 1, t0 = lane & (TP - 1);
  const int step = nw * ppw;
  for (int p0 = wave * ppw; p0 < npairs; p0 += 2 * step) {
    const int pa = p0 + ps, pb = p0 + step + ps;
    const bool two = (p0 + step) < npairs;   // wave-uniform
    const PairRef A = pairfn(pa < npairs ? pa : npairs - 1);
    const uint8_t* ra = half ? A.up : A.gate;
    double va = 0.0, vb = 0.0;
    PairRef B = A;
    const uint8_t* rb = ra;
    if (two) {
      B = pairfn(pb < npairs ? pb : npairs - 1);
      rb = half ? B.up : B.gate;
    }
    for (int t = t0; t < T; t += TP) {
      va += row_task<TYPE>(ra, t, A.act);
      if (two) vb += row_task<TYPE>(rb, t, B.act);
    }
    va = group_sum_f64(va, TP);
    const double ua = lane_f64(va, lane + TP < 64 ? lane + TP : lane);
    if (two) vb = group_sum_f64(vb, TP);
    const double ub = two ? lane_f64(vb, lane + TP < 64 ? lane + TP : lane) : 0.0;
    if (t0 == 0 && half == 0) {
      if (pa < npairs) store(pa, (float)(silu_f64((double)(float)va) * (double)(float)ua));
      if (two && pb < npairs) store(pb, (float)(silu_f64((double)(float)vb) * (double)(float)ub));
    }
  }
}
__device__ __forceinline__ double sigmoid_f64(double x) { return 1.0 / (1.0 + exp(-x)); }

}  // namespace moe
