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

__host__ __device__ inline int block_bytes(int type) {
  return type == MOE_TYPE_Q4_K ? kQ4KBytes : type == MOE_TYPE_Q5_K ? kQ5KBytes : type == MOE_TYPE_Q8_0 ? kQ80Bytes : kQ81Bytes;
}
__host__ __device__ inline int block_elems(int type) {
  return (type == MOE_TYPE_Q4_K || type == MOE_TYPE_Q5_K) ? 256 : 32;
}
__host__ __device__ inline int pad_k(int type, int K) {
  int b = block_elems(type);
  return (K + b - 1) / b * b;
}
__host__ __device__ inline long row_bytes(int type, int K) { return (long)(K / block_elems(type)) * block_bytes(type); }
// Independent work items ("tasks") per row: one per 64 elements for K-quants
// (a 32-byte group of qs = two sub-blocks), one per 32-element block for Q8_0.
__host__ __device__ inline int tasks_per_row(int type, int K) {
  return (type == MOE_TYPE_Q8_0) ? K / 32 : K / 64;
}

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// round to nearest, ties to even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// binary16 <-> fp32 through the hardware conversions (exact one way, round to
// nearest even the other, subnormals kept).
__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h16 & 0xffffu));
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------------- wave reductions (wave64)
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float half_wave_max_f32(float v) {  // within aligned groups of 32 lanes
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 32));
  return v;
}
__device__ __forceinline__ int half_wave_sum_i32(int v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 32);
  return v;
}

// ---------------------------------------------------------------- Q8_1 quantiser
// One 32-element block held by 32 consecutive lanes (one value per lane).
// d32 = amax/127 and the codes x*(1/d32) are fp32 and correctly rounded (a
// float decides an integer here, so the precision is fixed, not widened);
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
  float s = __fmul_rn(f16_to_f32(d16), (float)qsum);  // exact: 11-bit d16 times |qsum| <= 4064
  r.ds = d16 | (f32_to_f16(s) << 16);
  return r;
}

// ---------------------------------------------------------------- K-quant scales
// 6-bit scale and min of sub-block j from the 12 scale bytes held as three
// dwords s0 (bytes 0..3), s1 (4..7), s2 (8..11).
__device__ __forceinline__ uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xffu; }
__device__ __forceinline__ void kquant_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j, int& sc, int& m) {
  if (j < 4) {
    sc = (int)(byte_of(s0, j) & 63u);
    m = (int)(byte_of(s1, j) & 63u);
  } else {
    int i = j - 4;
    sc = (int)((byte_of(s2, i) & 0xfu) | ((byte_of(s0, i) >> 6) << 4));
    m = (int)((byte_of(s2, i) >> 4) | ((byte_of(s1, i) >> 6) << 4));
  }
}

// ---------------------------------------------------------------- integer dots
// 32-byte group g of a K-quant superblock against the two activation blocks it
// pairs with (sub-blocks 2g and 2g+1).  qs: 8 dwords of codes (low/high nibbles);
// qh: 8 dwords of fifth bits (Q5_K) or nullptr; alo/ahi: 8 dwords of int8 codes.
template <bool Q5>
__device__ __forceinline__ void kquant_group_dots(const uint32_t qs[8], const uint32_t* qh, int g,
                                                  const uint32_t alo[8], const uint32_t ahi[8], int& Dlo, int& Dhi) {
  int lo = 0, hi = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t wl = qs[t] & 0x0f0f0f0fu;
    uint32_t wh = (qs[t] >> 4) & 0x0f0f0f0fu;
    if (Q5) {
      wl |= ((qh[t] >> (2 * g)) & 0x01010101u) << 4;
      wh |= ((qh[t] >> (2 * g + 1)) & 0x01010101u) << 4;
    }
    lo = __builtin_amdgcn_sdot4((int)wl, (int)alo[t], lo, false);
    hi = __builtin_amdgcn_sdot4((int)wh, (int)ahi[t], hi, false);
  }
  Dlo = lo;
  Dhi = hi;
}

__device__ __forceinline__ int q8_block_dot(const uint32_t w[8], const uint32_t a[8]) {
  int acc = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_sdot4((int)w[t], (int)a[t], acc, false);
  return acc;
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

__device__ __forceinline__ double silu_f64(double x) { return x / (1.0 + exp(-x)); }
__device__ __forceinline__ double sigmoid_f64(double x) { return 1.0 / (1.0 + exp(-x)); }

}  // namespace moe
