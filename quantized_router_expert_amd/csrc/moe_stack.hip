// moe_stack.hip -- the whole L-layer MoE stack for one token in one cooperative launch.
//
// [P239] Summary: decode is graph- and launch-bound, so removing per-layer
// launches pays; [P273] Summary item 1: the top-k runs inside the router's
// kernel after a grid-completion handshake.  On gfx950 the same idea is taken
// further: every layer of the token runs inside one resident grid (one
// workgroup per CU), the phases of a layer hand data to each other through
// memory, and the weights that do not depend on the routing decision
// (norm weight, router rows, shared-expert rows) are streamed into LDS while
// the previous layer finishes.
//
// Per layer (G workgroups; workgroup b owns a fixed slice of every phase):
//   A  u = bf16(res + t), RMSNorm -> xn, xq (redundantly in every workgroup);
//      router row(s) b (+ the shared-gate row); shared gate/up rows -> hs
//   B  top-k + softmax (from all logits); routed gate/up rows of one slot -> h;
//      the routed down rows this workgroup needs are requested right away
//   C  Q8_1 of every h; down rows [b*RD, b*RD+RD) of all k slots + shared;
//      combine -> t = bf16(routed + shared) for those rows
// Exchanges: every produced value travels as an 8-byte word (32-bit payload,
// 32-bit epoch) written with one agent-coherent store, so a reader knows a
// word is current without a separate flag.  Only one workgroup per XCD (the
// leader, elected from the hardware XCC id) reads produced data from memory;
// it republishes into its XCD's L2 with plain stores, where the XCD's other
// workgroups read it with non-temporal loads.  Every wait is bounded: a spin
// limit sets an error word and the grid exits.
#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_stack.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kPollWaves = 4;   // waves 0..3 poll and load the routed gate/up rows
constexpr int kAuxSC1 = 16;     // agent-coherent (bypasses the XCD L2)
constexpr int kAuxNT = 2;       // non-temporal (bypasses L1, served by the XCD L2)
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xfu; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Stream `bytes` from src into LDS dst (1 KiB per wave instruction); waves
// [w0, w0+nw) take chunks round-robin.  dst must have room for the byte count
// rounded up to 1 KiB: lanes past the source end read 0 (bounds-checked
// buffer) and write that 0 into the padding.
__device__ __forceinline__ void stage_async(uint8_t* dst, const void* src, uint32_t bytes, int wave, int w0, int nw) {
  if (wave < w0 || wave >= w0 + nw || bytes == 0) return;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, bytes);
  const int lane = threadIdx.x & 63;
  const uint32_t nchunks = (bytes + 1023) >> 10;
  for (uint32_t c = wave - w0; c < nchunks; c += nw)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (c << 10)), 16, (c << 10) + lane * 16, 0, 0, 0);
}

__device__ __forceinline__ void ll_store(const __amdgpu_buffer_rsrc_t& r, uint32_t word, uint32_t payload, uint32_t epoch,
                                         int aux) {
  v2u v = {payload, epoch};
  if (aux == kAuxSC1) __builtin_amdgcn_raw_buffer_store_b64(v, r, word * 8, 0, kAuxSC1);
  else __builtin_amdgcn_raw_buffer_store_b64(v, r, word * 8, 0, 0);
}

// Poll n LL words until every epoch equals `epoch`, copying payloads to dst[].
// Waves [0, nw) split the words; every lane issues all of its loads of a
// round (up to kPollMax 16-byte word pairs) before checking any, so one
// memory round trip covers up to 64*nw*kPollMax pairs.  Returns false on the
// spin limit.
constexpr int kPollMax = 6;
template <int AUX>
__device__ __noinline__ bool poll_ll(const __amdgpu_buffer_rsrc_t& r, uint32_t n, uint32_t epoch, uint32_t* dst, int nw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave >= nw) return true;
  const uint32_t npairs = (n + 1) >> 1;
  const uint32_t stride = 64u * nw;
  for (uint32_t base = 0; base < npairs; base += stride * kPollMax) {
    const uint32_t first = base + wave * 64u + lane;
    uint32_t want = 0, done = 0;
#pragma unroll
    for (int m = 0; m < kPollMax; ++m)
      if (first + m * stride < npairs) want |= 1u << m;
    uint32_t spins = 0;
    for (;;) {
      uint4 v[kPollMax];
#pragma unroll
      for (int m = 0; m < kPollMax; ++m)
        if ((want & ~done) & (1u << m))
          v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (first + m * stride) * 16, 0, AUX));
#pragma unroll
      for (int m = 0; m < kPollMax; ++m) {
        if ((want & ~done) & (1u << m)) {
          const uint32_t p = first + m * stride;
          const bool second = (2 * p + 1 < n);
          if (v[m].y == epoch && (!second || v[m].w == epoch)) {
            dst[2 * p] = v[m].x;
            if (second) dst[2 * p + 1] = v[m].z;
            done |= 1u << m;
          }
        }
      }
      if (__all(done == want)) break;
      if (++spins > kSpinLimit) return false;
    }
  }
  return true;
}

// ---------------------------------------------------------------- row-dot helpers over LDS-staged rows
template <int TYPE>
__device__ __forceinline__ void tasks_to_partials(const uint8_t* rows, long rbytes, int nrows, int K, const ActLds& act,
                                                  double* partial) {
  const int T = tasks_per_row(TYPE, K);
  const int total = nrows * T;
  for (int i = threadIdx.x; i < total; i += kStackThreads) {
    const int r = i / T, t = i - r * T;
    partial[i] = row_task<TYPE>(rows + (long)r * rbytes, t, act);
  }
}

__device__ __forceinline__ double sum_row(const double* p, int T) {
  double a = 0.0;
  for (int t = 0; t < T; ++t) a += p[t];
  return a;
}

// block-wide fp64 sum (all threads get the result); red needs kStackThreads/64 doubles
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kStackThreads / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ unsigned long long key_of(float v, int e) {
  if (v != v) v = -__builtin_inff();
  if (v == 0.0f) v = 0.0f;
  const uint32_t b = __float_as_uint(v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xffffffffu - (uint32_t)e);
}

// wave 0: top-k of lg[0..E), softmax over the selected logits, sigmoid of lg[E] -> sel[] (ids, weights bits, gate bits)
__device__ __noinline__ void select_experts(const float* lg, int E, int k, bool has_sg, uint32_t* sel, double* scratch) {
  const int lane = threadIdx.x & 63;
  unsigned long long key[kTopkPerLane];
#pragma unroll
  for (int j = 0; j < kTopkPerLane; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? key_of(lg[e], e) : 0ull;
  }
  for (int s = 0; s < k; ++s) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int j = 0; j < kTopkPerLane; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int j = 0; j < kTopkPerLane; ++j)
      if (key[j] == best) key[j] = 0ull;
    if (lane == 0) sel[s] = 0xffffffffu - (uint32_t)(best & 0xffffffffull);
  }
  // softmax over the selected logits, shifted by the largest (slot 0), fp64:
  // lane s computes slot s's exponential, lane 0 sums them in slot order
  __builtin_amdgcn_wave_barrier();
  const double m = (double)lg[sel[0]];
  double p = 0.0;
  if (lane < k) p = exp((double)lg[sel[lane]] - m);
  if (lane < k) scratch[lane] = p;
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {
    double sum = 0.0;
    for (int s = 0; s < k; ++s) sum += scratch[s];
    scratch[MOE_MAX_TOPK] = sum;
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < k) sel[k + lane] = __float_as_uint((float)(p / scratch[MOE_MAX_TOPK]));
  if (lane == k) {
    sel[2 * k] = __float_as_uint(has_sg ? (float)sigmoid_f64((double)lg[E]) : 0.0f);
  }
}

__device__ __forceinline__ bool same_layer(const moe_layer_weights& p, const moe_layer_weights& q) {
  return p.norm_w == q.norm_w && p.router_w == q.router_w && p.shared_gate_w == q.shared_gate_w && p.gate == q.gate &&
         p.up == q.up && p.down == q.down && p.shared_gate == q.shared_gate && p.shared_up == q.shared_up &&
         p.shared_down == q.shared_down;
}

// ---------------------------------------------------------------- the kernel
template <int DT, int ST>
__global__ __launch_bounds__(kStackThreads) void k_stack(StackArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const StackGeom& g = a.g;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const int H = a.H, E = a.E, k = a.k, F = a.F, Fs = a.Fs;
  const bool has_sg = Fs > 0;

  float* res = reinterpret_cast<float*>(smem + g.o_res);
  float* xn = reinterpret_cast<float*>(smem + g.o_xn);
  uint8_t* xqc = smem + g.o_xqc;
  float* xqd = reinterpret_cast<float*>(smem + g.o_xqd);
  float* xqs = reinterpret_cast<float*>(smem + g.o_xqs);
  const float* nw = reinterpret_cast<const float*>(smem + g.o_nw);
  uint8_t* rrow = smem + g.o_rrow;
  uint8_t* sgu = smem + g.o_sgu;
  uint8_t* sdn = smem + g.o_sdn;
  uint8_t* rgu = smem + g.o_rgu;
  uint8_t* rdn = smem + g.o_rdn;
  uint8_t* hqc = smem + g.o_hqc;
  float* hqd = reinterpret_cast<float*>(smem + g.o_hqd);
  float* hqs = reinterpret_cast<float*>(smem + g.o_hqs);
  double* part = reinterpret_cast<double*>(smem + g.o_part);
  uint32_t* xbuf = reinterpret_cast<uint32_t*>(smem + g.o_xbuf);   // exchange landing area
  uint32_t* sel = reinterpret_cast<uint32_t*>(smem + g.o_sel);
  double* red = reinterpret_cast<double*>(smem + g.o_red);
  float* yv = reinterpret_cast<float*>(smem + g.o_y);
  double* smx = reinterpret_cast<double*>(smem + g.o_smx);

  __shared__ uint32_t s_gen, s_x, s_leader;
  __shared__ int s_fail;
  {
    // the bound pointer table must be the caller's stack
    bool ok = a.bound[0] == (int)kBoundMagic && a.bound[1] == a.L;
    if (ok) ok = same_layer(a.layers[0], a.first) && same_layer(a.layers[a.L - 1], a.last);
    if (!ok) {
      if (b == 0) {
        for (int i = tid; i < H; i += kStackThreads) a.output[i] = 0x7fc0u;
        if (tid == 0) __hip_atomic_store(reinterpret_cast<uint32_t*>(a.ws + g.w_ctrl) + kErrWord, 2u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
  }
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(a.ws + g.w_ctrl);
  const __amdgpu_buffer_rsrc_t r_ctrl = make_rsrc(ctrl, kStackCtrlBytes);
  if (tid == 0) {
    s_fail = 0;
    v2u gv = __builtin_amdgcn_raw_buffer_load_b64(r_ctrl, 0, 0, kAuxSC1);
    s_gen = gv.x;
    const unsigned x = xcc_id();
    const unsigned old = __hip_atomic_fetch_add(ctrl + kCensusWord + 16 * x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_x = x;
    s_leader = (old % (unsigned)g.per_xcc) == 0u;
  }
  __syncthreads();
  const uint32_t base = s_gen * (uint32_t)(3 * a.L + 2) + 1u;
  const unsigned x = s_x & 7u;
  const bool leader = s_leader != 0;

  const __amdgpu_buffer_rsrc_t r_t = make_rsrc(a.ws + g.w_t, (uint32_t)g.n_t * 8);
  const __amdgpu_buffer_rsrc_t r_lg = make_rsrc(a.ws + g.w_lg, (uint32_t)g.n_lg * 8);
  const __amdgpu_buffer_rsrc_t r_h = make_rsrc(a.ws + g.w_h, (uint32_t)g.n_h * 8);
  uint8_t* loc = a.ws + g.w_loc + (size_t)x * g.loc_stride;
  const __amdgpu_buffer_rsrc_t r_lt = make_rsrc(loc + g.l_t, (uint32_t)g.n_t * 8);
  const __amdgpu_buffer_rsrc_t r_ls = make_rsrc(loc + g.l_sel, (uint32_t)g.n_sel * 8);
  const __amdgpu_buffer_rsrc_t r_lh = make_rsrc(loc + g.l_hq, (uint32_t)g.n_hq * 8);

  const long rb_gu = row_bytes(MOE_TYPE_Q4_K, H);
  const long rb_sgu = has_sg ? row_bytes(ST, H) : 0;
  const long rb_dn = row_bytes(DT, g.Kp);
  const long rb_sdn = has_sg ? row_bytes(ST, g.Kps) : 0;
  const int row0 = b * g.RD;
  const int nrd = max(0, min(g.RD, H - row0));
  const int sf0 = b * g.SR;
  const int nsr = has_sg ? max(0, min(g.SR, Fs - sf0)) : 0;

  // weights that do not depend on the routing decision, for layer l
  auto prefetch_fixed = [&](int l) {
    const moe_layer_weights& w = a.layers[l];
    stage_async(smem + g.o_nw, w.norm_w, (uint32_t)(H * 4), wave, kPollWaves, kStackWaves - kPollWaves);
    for (int j = 0; j < g.RR; ++j) {
      const int r = b + j * g.G;
      const float* src = (r < E) ? w.router_w + (long)r * H : ((r == E && has_sg) ? w.shared_gate_w : nullptr);
      if (src) stage_async(rrow + (long)j * H * 4, src, (uint32_t)(H * 4), wave, kPollWaves, kStackWaves - kPollWaves);
    }
    if (nsr > 0) {
      stage_async(sgu, (const uint8_t*)w.shared_gate + sf0 * rb_sgu, (uint32_t)(nsr * rb_sgu), wave, kPollWaves,
                  kStackWaves - kPollWaves);
      stage_async(sgu + g.sgu_half, (const uint8_t*)w.shared_up + sf0 * rb_sgu, (uint32_t)(nsr * rb_sgu), wave,
                  kPollWaves, kStackWaves - kPollWaves);
    }
    if (has_sg && nrd > 0)
      stage_async(sdn, (const uint8_t*)w.shared_down + row0 * rb_sdn, (uint32_t)(nrd * rb_sdn), wave, kPollWaves,
                  kStackWaves - kPollWaves);
  };

  uint64_t* trace = reinterpret_cast<uint64_t*>(a.ws + g.w_trace);
  auto stamp = [&](int l, int i) {
    if (b == 0 && tid == 0 && l < kTraceLayers) {
      trace[l * kTraceSlots + i] = wall_clock64();
      if (i == 0) trace[l * kTraceSlots + 10] = clock64();
      if (i == 9) trace[l * kTraceSlots + 11] = clock64();
    }
  };

  auto fail_out = [&]() {
    if (tid == 0) __builtin_amdgcn_raw_buffer_store_b32(1u, r_ctrl, kErrWord * 4, 0, kAuxSC1);
  };

  // ---- layer-0 inputs: the token's residual, no previous outputs
  prefetch_fixed(0);
  for (int i = tid; i < H; i += kStackThreads) res[i] = bf16_to_f32(a.input[i]);

  for (int l = 0; l < a.L; ++l) {
    const uint32_t ep0 = base + 3u * l, ep1 = ep0 + 1u, ep2 = ep0 + 2u;
    const moe_layer_weights& w = a.layers[l];
    stamp(l, 0);
    // ================= R1: t of the previous layer
    if (l > 0) {
      const bool ok = leader ? poll_ll<kAuxSC1>(r_t, g.n_t, ep2 - 3u, xbuf, kPollWaves)
                             : poll_ll<kAuxNT>(r_lt, g.n_t, ep2 - 3u, xbuf, kPollWaves);
      if (!ok) s_fail = 1;
      __syncthreads();
      if (s_fail) { fail_out(); return; }
      if (leader)
        for (int i = tid; i < g.n_t; i += kStackThreads) ll_store(r_lt, i, xbuf[i], ep2 - 3u, 0);
      for (int i = tid; i < H; i += kStackThreads) {
        const uint32_t pr = xbuf[i >> 1];
        const float t = bf16_to_f32((uint16_t)((i & 1) ? (pr >> 16) : (pr & 0xffffu)));
        res[i] = bf16_to_f32(f32_to_bf16(res[i] + t));
      }
    }
    // ================= phase A: norm, router rows, shared gate/up rows
    stamp(l, 1);
    if (wave >= kPollWaves) wait_vmem();
    __syncthreads();
    stamp(l, 2);
    if (b == 0 && a.resid_out)
      for (int i = tid; i < H; i += kStackThreads) a.resid_out[(long)l * H + i] = f32_to_bf16(res[i]);
    double ss = 0.0;
    for (int i = tid; i < H; i += kStackThreads) ss += (double)res[i] * (double)res[i];
    ss = block_sum_f64(ss, red);
    const double rinv = 1.0 / sqrt(ss / (double)H + (double)a.eps);
    for (int i = tid; i < H; i += kStackThreads) xn[i] = (float)(((double)res[i] * rinv) * (double)nw[i]);
    __syncthreads();
    for (int j = tid; j < H / 32; j += kStackThreads) {
      const uint32_t ds = quantize_q81_block(xn + 32 * j, xqc + 32 * j);
      xqd[j] = f16_to_f32(ds);
      xqs[j] = f16_to_f32(ds >> 16);
    }
    __syncthreads();
    // router rows (fp64 dot of fp32 products), one wave per row
    for (int j = wave; j < g.RR; j += kStackWaves) {
      const int r = b + j * g.G;
      const bool real = (r < E) || (r == E && has_sg);
      if (!real) break;
      const float* wr = reinterpret_cast<const float*>(rrow + (long)j * H * 4);
      double acc = 0.0;
      for (int i = (tid & 63) * 4; i < H; i += 256) {
        const float4 wv = *reinterpret_cast<const float4*>(wr + i);
        const float4 xv = *reinterpret_cast<const float4*>(xn + i);
        acc += (double)wv.x * (double)xv.x;
        acc += (double)wv.y * (double)xv.y;
        acc += (double)wv.z * (double)xv.z;
        acc += (double)wv.w * (double)xv.w;
      }
      acc = wave_sum_f64(acc);
      if ((tid & 63) == 0) ll_store(r_lg, r, __float_as_uint((float)acc), ep0, kAuxSC1);
    }
    // shared gate/up rows -> hs (word k*F + f of the h exchange)
    if (nsr > 0) {
      const ActLds act{xqc, xqd, xqs};
      rows_dot<ST>(2 * nsr, tasks_per_row(ST, H), [&](int r) {
        return RowRef{(r < nsr) ? sgu + (long)r * rb_sgu : sgu + g.sgu_half + (long)(r - nsr) * rb_sgu, act};
      }, part, wave, kStackWaves);
      __syncthreads();
      if (tid < nsr) {
        const float gg = (float)part[tid];
        const float uu = (float)part[nsr + tid];
        const float hv = (float)(silu_f64((double)gg) * (double)uu);
        ll_store(r_h, k * F + sf0 + tid, __float_as_uint(hv), ep1, kAuxSC1);
      }
    }
    // ================= R2: logits -> selection
    stamp(l, 3);
    {
      const bool ok = leader ? poll_ll<kAuxSC1>(r_lg, g.n_lg, ep0, xbuf, kPollWaves)
                             : poll_ll<kAuxNT>(r_ls, g.n_sel, ep0, sel, kPollWaves);
      if (!ok) s_fail = 1;
      __syncthreads();
      if (s_fail) { fail_out(); return; }
      if (leader) {
        if (wave == 0) select_experts(reinterpret_cast<const float*>(xbuf), E, k, has_sg, sel, smx);
        __syncthreads();
        for (int i = tid; i < g.n_sel; i += kStackThreads) ll_store(r_ls, i, sel[i], ep0, 0);
        if (a.ids_out && x == 0)
          for (int s = tid; s < k; s += kStackThreads) a.ids_out[(long)l * k + s] = (int32_t)sel[s];
      }
    }
    stamp(l, 4);
    // ================= phase B: routed gate/up rows (this workgroup's slot and rows)
    const int p0 = b * g.RP;
    const int slot = p0 / F;
    const int f0 = p0 - slot * F;
    const int nrp = (slot < k) ? min(g.RP, F - f0) : 0;
    bool bad_id = false;
    for (int s = 0; s < k; ++s) bad_id |= (sel[s] >= (uint32_t)E);
    if (bad_id) { fail_out(); return; }
    if (nrp > 0 && wave < kPollWaves) {
      const long e = sel[slot];
      stage_async(rgu, (const uint8_t*)w.gate + (e * F + f0) * rb_gu, (uint32_t)(nrp * rb_gu), wave, 0, kPollWaves);
      stage_async(rgu + g.rgu_half, (const uint8_t*)w.up + (e * F + f0) * rb_gu, (uint32_t)(nrp * rb_gu), wave, 0,
                  kPollWaves);
    }
    if (nrd > 0 && wave >= kPollWaves) {
      for (int s = 0; s < k; ++s) {
        const long e = sel[s];
        stage_async(rdn + (long)s * g.rdn_slot, (const uint8_t*)w.down + (e * H + row0) * rb_dn, (uint32_t)(nrd * rb_dn),
                    wave, kPollWaves, kStackWaves - kPollWaves);
      }
    }
    if (wave < kPollWaves) wait_vmem();
    __syncthreads();
    stamp(l, 5);
    if (nrp > 0) {
      const ActLds act{xqc, xqd, xqs};
      rows_dot<MOE_TYPE_Q4_K>(2 * nrp, tasks_per_row(MOE_TYPE_Q4_K, H), [&](int r) {
        return RowRef{(r < nrp) ? rgu + (long)r * rb_gu : rgu + g.rgu_half + (long)(r - nrp) * rb_gu, act};
      }, part, wave, kStackWaves);
      __syncthreads();
      if (tid < nrp) {
        const float gg = (float)part[tid];
        const float uu = (float)part[nrp + tid];
        const float hv = (float)(silu_f64((double)gg) * (double)uu);
        ll_store(r_h, slot * F + f0 + tid, __float_as_uint(hv), ep1, kAuxSC1);
      }
    }
    // ================= R3: h -> Q8_1 codes of every slot (+ shared)
    stamp(l, 6);
    {
      const int nb_r = g.Kp / 32, nb_s = g.Kps / 32;
      const int nblk = k * nb_r + nb_s;           // Q8_1 blocks of all down inputs
      const int ncode_words = (k * g.Kp + g.Kps) / 4;
      // the leader polls the largest exchange with every wave (the down rows that
      // waves 4..7 requested in phase B have had the whole of phase B to land)
      const bool ok = leader ? poll_ll<kAuxSC1>(r_h, g.n_h, ep1, xbuf, kStackWaves)
                             : poll_ll<kAuxNT>(r_lh, g.n_hq, ep1, xbuf, kPollWaves);
      if (!ok) s_fail = 1;
      __syncthreads();
      if (s_fail) { fail_out(); return; }
      if (leader) {
        {
          // quantise, one lane per Q8_1 block: block j of slot s covers
          // h[s*F + 32j ..]; blocks past F (or Fs) are the zero padding
          for (int blk = tid; blk < nblk; blk += kStackThreads) {
            uint32_t ds = 0;
            uint8_t* codes;
            if (blk < k * nb_r) {
              const int s = blk / nb_r, jb = blk - s * nb_r;
              codes = hqc + (long)s * g.Kp + 32 * jb;
              if (jb * 32 < F) ds = quantize_q81_block(reinterpret_cast<const float*>(xbuf) + s * F + 32 * jb, codes);
              else *reinterpret_cast<uint4*>(codes) = make_uint4(0, 0, 0, 0), *reinterpret_cast<uint4*>(codes + 16) = make_uint4(0, 0, 0, 0);
            } else {
              const int jb = blk - k * nb_r;
              codes = hqc + (long)k * g.Kp + 32 * jb;
              if (jb * 32 < Fs) ds = quantize_q81_block(reinterpret_cast<const float*>(xbuf) + k * F + 32 * jb, codes);
              else *reinterpret_cast<uint4*>(codes) = make_uint4(0, 0, 0, 0), *reinterpret_cast<uint4*>(codes + 16) = make_uint4(0, 0, 0, 0);
            }
            hqd[blk] = f16_to_f32(ds);
            hqs[blk] = f16_to_f32(ds >> 16);
            xbuf[g.n_h + blk] = ds;     // the raw fp16 pair, for republishing
          }
          __syncthreads();
          const uint32_t* cw = reinterpret_cast<const uint32_t*>(hqc);
          for (int i = tid; i < ncode_words; i += kStackThreads) ll_store(r_lh, i, cw[i], ep1, 0);
          for (int i = tid; i < nblk; i += kStackThreads) ll_store(r_lh, ncode_words + i, xbuf[g.n_h + i], ep1, 0);
        }
      } else {
        uint32_t* cw = reinterpret_cast<uint32_t*>(hqc);
        for (int i = tid; i < ncode_words; i += kStackThreads) cw[i] = xbuf[i];
        for (int i = tid; i < nblk; i += kStackThreads) {
          const uint32_t ds = xbuf[ncode_words + i];
          hqd[i] = f16_to_f32(ds);
          hqs[i] = f16_to_f32(ds >> 16);
        }
      }
    }
    // ================= phase C: down rows of all slots + shared, combine
    stamp(l, 7);
    if (wave >= kPollWaves) wait_vmem();
    __syncthreads();
    stamp(l, 8);
    if (nrd > 0) {
      rows_dot<DT>(k * nrd, tasks_per_row(DT, g.Kp), [&](int r) {
        const int s = r / nrd, rr = r - s * nrd;
        return RowRef{rdn + (long)s * g.rdn_slot + (long)rr * rb_dn,
                      ActLds{hqc + (long)s * g.Kp, hqd + s * (g.Kp / 32), hqs + s * (g.Kp / 32)}};
      }, part, wave, kStackWaves);
      if (has_sg) {
        const ActLds acts{hqc + (long)k * g.Kp, hqd + k * (g.Kp / 32), hqs + k * (g.Kp / 32)};
        rows_dot<ST>(nrd, tasks_per_row(ST, g.Kps), [&](int r) { return RowRef{sdn + (long)r * rb_sdn, acts}; },
                     part + k * nrd, wave, kStackWaves);
      }
      __syncthreads();
      for (int i = tid; i < (k + 1) * nrd; i += kStackThreads) {
        const int m = i / nrd, r = i - m * nrd;
        yv[m * g.RD + r] = (m < k || has_sg) ? (float)part[m * nrd + r] : 0.0f;
      }
      __syncthreads();
      const float sgv = __uint_as_float(sel[2 * k]);
      for (int r2 = tid; 2 * r2 < nrd; r2 += kStackThreads) {
        uint32_t pr = 0;
        for (int h2 = 0; h2 < 2; ++h2) {
          const int r = 2 * r2 + h2;
          double acc = 0.0;
          for (int s = 0; s < k; ++s) acc += (double)__uint_as_float(sel[k + s]) * (double)yv[s * g.RD + r];
          const uint16_t routed = f32_to_bf16((float)acc);
          float t = bf16_to_f32(routed);
          if (has_sg) {
            const uint16_t shared = f32_to_bf16((float)((double)sgv * (double)yv[k * g.RD + r]));
            t = bf16_to_f32(f32_to_bf16(bf16_to_f32(routed) + bf16_to_f32(shared)));
          }
          pr |= (uint32_t)f32_to_bf16(t) << (16 * h2);
        }
        ll_store(r_t, (row0 >> 1) + r2, pr, ep2, kAuxSC1);
      }
    }
    __syncthreads();
    stamp(l, 9);
    if (l + 1 < a.L) prefetch_fixed(l + 1);
  }
  // ================= the fold a next layer would do: output = bf16(res + t)
  if (b == 0) {
    const uint32_t epl = base + 3u * (a.L - 1) + 2u;
    const bool ok = poll_ll<kAuxSC1>(r_t, g.n_t, epl, xbuf, kPollWaves);
    if (!ok) s_fail = 1;
    __syncthreads();
    if (s_fail) { fail_out(); return; }
    for (int i = tid; i < H; i += kStackThreads) {
      const uint32_t pr = xbuf[i >> 1];
      const float t = bf16_to_f32((uint16_t)((i & 1) ? (pr >> 16) : (pr & 0xffffu)));
      a.output[i] = f32_to_bf16(res[i] + t);
    }
    __syncthreads();
    if (tid == 0) {
      v2u nv = {s_gen + 1u, 0u};
      __builtin_amdgcn_raw_buffer_store_b64(nv, r_ctrl, 0, 0, kAuxSC1);
    }
  }
}

// ---------------------------------------------------------------- host side
static inline int up1k(long x) { return (int)((x + 1023) & ~1023L); }
static inline int up16(long x) { return (int)((x + 15) & ~15L); }

int stack_geometry(const moe_layer_desc* d, int G, StackGeom* out) {
  StackGeom g = {};
  const int H = d->hidden, E = d->n_experts, k = d->top_k, F = d->ffn, Fs = d->shared_ffn;
  const bool has_sg = Fs > 0;
  const int st = has_sg ? d->shared_type : MOE_TYPE_Q4_K;
  g.G = G;
  g.per_xcc = G / 8;
  g.Kp = pad_k(d->down_type, F);
  g.Kps = has_sg ? pad_k(st, Fs) : 0;
  g.RR = (E + (has_sg ? 1 : 0) + G - 1) / G;
  g.SR = has_sg ? (Fs + G - 1) / G : 0;
  g.RD = (H + G - 1) / G;
  if (g.RD & 1) g.RD += 1;                    // t travels in bf16 pairs
  g.RP = (k * F + G - 1) / G;
  while (F % g.RP) g.RP++;
  if ((long)g.RP * G < (long)k * F) return MOE_ERR_UNSUPPORTED;
  const long rb_gu = row_bytes(MOE_TYPE_Q4_K, H);
  const long rb_sgu = has_sg ? row_bytes(st, H) : 0;
  const long rb_dn = row_bytes(d->down_type, g.Kp);
  const long rb_sdn = has_sg ? row_bytes(st, g.Kps) : 0;
  g.n_t = H / 2;
  g.n_lg = E + (has_sg ? 1 : 0);
  g.n_h = k * F + Fs;
  g.n_sel = 2 * k + 1;
  const int nblk = k * (g.Kp / 32) + g.Kps / 32;
  g.n_hq = (k * g.Kp + g.Kps) / 4 + nblk;
  // LDS
  long o = 0;
  auto take = [&](long bytes) { long r = o; o += up16(bytes); return (int)r; };
  g.o_res = take(4L * H);
  g.o_xn = take(4L * H);
  g.o_xqc = take(H);
  g.o_xqd = take(4L * (H / 32));
  g.o_xqs = take(4L * (H / 32));
  g.o_nw = take(up1k(4L * H));
  g.o_rrow = take((long)g.RR * up1k(4L * H));
  g.sgu_half = up1k(g.SR * rb_sgu);
  g.o_sgu = take(2L * g.sgu_half);
  g.o_sdn = take(up1k(g.RD * rb_sdn));
  g.rgu_half = up1k(g.RP * rb_gu);
  g.o_rgu = take(2L * g.rgu_half);
  g.rdn_slot = up1k(g.RD * rb_dn);
  g.o_rdn = take((long)k * g.rdn_slot);
  g.o_hqc = take((long)k * g.Kp + g.Kps);
  g.o_hqd = take(4L * nblk);
  g.o_hqs = take(4L * nblk);
  long np = 2L * g.RP;                               // fp64 row values of one phase
  np = np > 2L * g.SR ? np : 2L * g.SR;
  np = np > (long)(k + 1) * g.RD ? np : (long)(k + 1) * g.RD;
  g.o_part = take(8L * np);
  long xb = g.n_h + nblk;                            // words landing from an exchange (h + fp16 pairs)
  xb = xb > g.n_t ? xb : g.n_t;
  xb = xb > g.n_lg ? xb : g.n_lg;
  xb = xb > g.n_hq ? xb : g.n_hq;
  // the exchange landing area is only written while the routed gate/up rows are
  // not in use (before they are staged, after they are consumed): share it
  if (4L * (xb + 2) <= 2L * g.rgu_half) g.o_xbuf = g.o_rgu;
  else g.o_xbuf = take(4L * (xb + 2));
  g.o_sel = take(4L * (g.n_sel + 1));
  g.o_red = take(8L * (kStackThreads / 64));
  g.o_y = take(4L * (k + 1) * g.RD);
  g.o_smx = take(8L * (MOE_MAX_TOPK + 1));
  g.lds = (int)o;
  if (g.lds < kStackMinLds) g.lds = kStackMinLds;   // keeps one workgroup per CU
  // workspace (exchange buffers after the per-layer region)
  out[0] = g;
  return MOE_OK;
}

void stack_ws_layout(StackGeom* g, size_t base) {
  size_t o = base;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~(size_t)255; return r; };
  g->w_ctrl = take(kStackCtrlBytes);
  g->w_t = take(8u * g->n_t);
  g->w_lg = take(8u * g->n_lg);
  g->w_h = take(8u * g->n_h);
  g->l_t = 0;
  g->l_sel = ((8u * g->n_t + 255) & ~(size_t)255);
  g->l_hq = g->l_sel + ((8u * g->n_sel + 255) & ~(size_t)255);
  g->loc_stride = g->l_hq + ((8u * g->n_hq + 255) & ~(size_t)255);
  g->w_loc = take(8 * g->loc_stride);
  g->w_trace = take(8u * kTraceLayers * kTraceSlots);
  g->w_end = o;
}

int device_cu_count(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

int launch_stack(const moe_layer_desc* d, int L, const moe_layer_weights* table_dev, const int* bound,
                 const moe_layer_weights& first, const moe_layer_weights& last, const uint16_t* input,
                 uint16_t* output, int32_t* ids_out, uint16_t* resid_out, uint8_t* ws, const StackGeom& g,
                 hipStream_t st) {
  StackArgs a;
  a.g = g;
  a.layers = table_dev;
  a.bound = bound;
  a.first = first;
  a.last = last;
  a.input = input;
  a.output = output;
  a.ids_out = ids_out;
  a.resid_out = resid_out;
  a.ws = ws;
  a.L = L;
  a.H = d->hidden;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.F = d->ffn;
  a.Fs = d->shared_ffn;
  a.eps = d->eps;
  const void* fn;
  const int dt = d->down_type;
  const int stt = d->shared_ffn > 0 ? d->shared_type : MOE_TYPE_Q4_K;
  if (dt == MOE_TYPE_Q5_K)
    fn = (stt == MOE_TYPE_Q8_0) ? (const void*)k_stack<MOE_TYPE_Q5_K, MOE_TYPE_Q8_0> : (const void*)k_stack<MOE_TYPE_Q5_K, MOE_TYPE_Q4_K>;
  else
    fn = (stt == MOE_TYPE_Q8_0) ? (const void*)k_stack<MOE_TYPE_Q4_K, MOE_TYPE_Q8_0> : (const void*)k_stack<MOE_TYPE_Q4_K, MOE_TYPE_Q4_K>;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, g.lds) != hipSuccess) return MOE_ERR_HIP;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(fn, dim3(g.G), dim3(kStackThreads), args, g.lds, st) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace moe
