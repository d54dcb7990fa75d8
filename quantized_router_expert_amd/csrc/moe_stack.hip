// moe_stack.hip -- the whole L-layer MoE stack for one token in one launch (every workgroup resident).
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
// word is current without a separate flag.  Every workgroup reads the words it
// needs straight from memory with agent-coherent loads (a per-XCD gatherer
// that republished into its L2 measured slower: the extra hop costs more than
// the contention it saves).  Every wait is bounded: a spin limit sets an
// error word and the grid exits.
#include <cstddef>
#include <cstring>
#include <mutex>

#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_select.h"
#include "moe_stack.h"

namespace moe {

constexpr int kPollWaves = 4;   // waves 0..3 poll and load the routed gate/up rows
// Copies of each exchange area: the producer of a word writes it into every
// copy and workgroup b reads copy b % R, so the 256 readers of one word are
// spread over R areas (4-KiB-aligned regions) instead of all polling the same
// few cache lines.  Eight copies shorten the logits and h exchanges (2 and 4
// copies of h helped less, 16 did worse); for t the extra stores cost more
// than they save.
// t: eight copies in the workspace, one per XCC for the XCD-slot path (each
// XCC builds all of t in its own copy); the other path writes and reads copy
// 0 only (measured: more copies of t cost more stores than they save)
constexpr int kRepT = 8, kRepLg = 8, kRepH = 8;
constexpr uint32_t rep_bytes(int n_words) { return (8u * (uint32_t)n_words + 4095u) & ~4095u; }
constexpr int kAuxSC1 = 16;     // agent-coherent (bypasses the XCD L2)
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

constexpr int kXcc = 8;   // accelerator complex dies (XCCs) of the MI355X, each with its own L2
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xfu;
}

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load of the wave (its workgroup-scope fence covers global
// memory), which would stall a wave at the first barrier after it has queued
// weight rows for a later phase.  Nothing in this kernel passes data between
// the waves of a workgroup through global memory; the rows streamed into LDS
// are waited for explicitly by the waves that queued them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void ll_store(const __amdgpu_buffer_rsrc_t& r, uint32_t word, uint32_t payload, uint32_t epoch,
                                         int aux) {
  v2u v = {payload, epoch};
  if (aux == kAuxSC1) __builtin_amdgcn_raw_buffer_store_b64(v, r, word * 8, 0, kAuxSC1);
  else __builtin_amdgcn_raw_buffer_store_b64(v, r, word * 8, 0, 0);
}
// the same word into each of R copies spaced rep bytes apart, the first at
// byte soff of the resource
template <int R>
__device__ __forceinline__ void ll_store_rep(const __amdgpu_buffer_rsrc_t& r, uint32_t soff, uint32_t rep, uint32_t word,
                                             uint32_t payload, uint32_t epoch) {
  v2u v = {payload, epoch};
#pragma unroll
  for (int c = 0; c < R; ++c) __builtin_amdgcn_raw_buffer_store_b64(v, r, c * rep + word * 8, soff, kAuxSC1);
}

// Poll n LL words until every epoch equals `epoch`, handing each current pair
// of words (2p, 2p+1) to sink(p, payload 2p, payload 2p+1) once.  Waves
// [w0, w0+nw) split the words; every lane issues all of its loads of a round
// (up to kPollMax 16-byte word pairs) before checking any, so one memory round
// trip covers up to 64*nw*kPollMax pairs.  Returns false on the spin limit.
constexpr int kPollMax = 6;
template <int AUX, class Sink>
__device__ __forceinline__ bool poll_ll_sink(const __amdgpu_buffer_rsrc_t& r, uint32_t soff, uint32_t n, uint32_t epoch,
                                             int nw, int w0, Sink sink) {
  const int wave = (threadIdx.x >> 6) - w0, lane = threadIdx.x & 63;
  if (wave < 0 || wave >= nw) return true;
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
          v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (first + m * stride) * 16, soff, AUX));
#pragma unroll
      for (int m = 0; m < kPollMax; ++m) {
        if ((want & ~done) & (1u << m)) {
          const uint32_t p = first + m * stride;
          const bool second = (2 * p + 1 < n);
          if (v[m].y == epoch && (!second || v[m].w == epoch)) {
            sink(p, v[m].x, v[m].z);
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

// the same, copying the payloads to dst[0..n)
template <int AUX>
__device__ __forceinline__ bool poll_ll(const __amdgpu_buffer_rsrc_t& r, uint32_t soff, uint32_t n, uint32_t epoch,
                                        uint32_t* dst, int nw, int w0 = 0) {
  return poll_ll_sink<AUX>(r, soff, n, epoch, nw, w0, [&](uint32_t p, uint32_t x, uint32_t z) {
    dst[2 * p] = x;
    if (2 * p + 1 < n) dst[2 * p + 1] = z;
  });
}

// Poll the M word pairs of this lane, pair[m] (< 0: none), until each is
// current (one epoch per pair: the words 2p and 2p+1 < n), leaving their
// payloads in lo[m], hi[m].  All loads of a round go out before any check.
// Returns false on the spin limit.
template <int AUX, int M>
__device__ __forceinline__ bool poll_lane_pairs(const __amdgpu_buffer_rsrc_t& r, uint32_t soff, const int (&pair)[M],
                                                uint32_t n, uint32_t epoch, uint32_t (&lo)[M], uint32_t (&hi)[M]) {
  uint32_t want = 0, done = 0;
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (pair[m] >= 0) want |= 1u << m;
  uint32_t spins = 0;
  for (;;) {
    uint4 v[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
      if ((want & ~done) & (1u << m))
        v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)pair[m] * 16u, soff, AUX));
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if ((want & ~done) & (1u << m)) {
        const bool second = (2u * (uint32_t)pair[m] + 1u < n);
        if (v[m].y == epoch && (!second || v[m].w == epoch)) {
          lo[m] = v[m].x;
          hi[m] = v[m].z;
          done |= 1u << m;
        }
      }
    }
    if (__all(done == want)) return true;
    if (++spins > kSpinLimit) return false;
  }
}

// R3: the Q8_1 blocks of the routed h, 16 blocks per wave per round.  Block
// j is block jb = j % nb_r of slot s = j / nb_r and covers words
// s*F + 32jb .. +31 (F % 32 == 0); blocks past F are the zero padding.  s
// comes from a float product: (j + 1/2)/nb_r lies at least 1/(2 nb_r) from an
// integer and the product is within 2^-23 relative of it, so truncation is
// exact for j < 2^22.  The wave polls its 16 blocks' words (load m of lane L
// is word pair (64m + L) % 16 of block 4m + L/16: 1 KiB of consecutive words
// per load where the blocks are), lands them in `land` at their word index
// and quantises its blocks from there without waiting for the other waves.
// Codes go to hqc + 32j, d and s to hqd[j], hqs[j].  Returns false on the
// spin limit.
__device__ __forceinline__ int h_block_word(int j, int nb_r, float inv_nbr, int F) {
  const int s = (int)(((float)j + 0.5f) * inv_nbr);
  const int jb = j - s * nb_r;
  return (32 * jb < F) ? s * F + 32 * jb : -1;
}
__device__ __forceinline__ bool poll_quantize_h(const __amdgpu_buffer_rsrc_t& r, uint32_t soff, int nblk, int nb_r,
                                                float inv_nbr, int F, uint32_t n, uint32_t epoch, uint32_t* land,
                                                uint8_t* hqc, float* hqd, float* hqs, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  bool ok = true;
  for (int j0 = wave * 16; j0 < nblk; j0 += nw * 16) {
    int pair[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int j = j0 + 4 * m + (lane >> 4);
      const int w0 = (j < nblk) ? h_block_word(j, nb_r, inv_nbr, F) : -1;
      pair[m] = (w0 >= 0) ? (w0 >> 1) + (lane & 15) : -1;
    }
    uint32_t lo[4] = {0u, 0u, 0u, 0u}, hi[4] = {0u, 0u, 0u, 0u};
    if (!poll_lane_pairs<kAuxSC1, 4>(r, soff, pair, n, epoch, lo, hi)) ok = false;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (pair[m] >= 0) *reinterpret_cast<uint2*>(land + 2 * pair[m]) = make_uint2(lo[m], hi[m]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    const int nb = min(16, nblk - j0);
    quantize_q81_groups<4, 1>(nb, reinterpret_cast<const float*>(land),
                              [&](int j) { return h_block_word(j0 + j, nb_r, inv_nbr, F); },
                              [&](int j) { return hqc + 32L * (j0 + j); }, hqd + j0, hqs + j0, lane, 64);
  }
  return ok;
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

// block-wide fp64 sum (all threads get the result); red needs kStackThreads/64
// doubles.  The caller keeps red unwritten until a later barrier (every wave
// reads it after this returns).
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kStackThreads / 64; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ double sq4_f64(float4 r) {
  return ((double)r.x * (double)r.x + (double)r.y * (double)r.y) + ((double)r.z * (double)r.z + (double)r.w * (double)r.w);
}

// A layer's weight pointers, wave-uniform.  Read once per layer at a moment
// when this wave has no row transfer in flight: a later read of the table
// would make the wave wait (in order) for every transfer queued before it.
struct LayerPtrs {
  const float* norm_w;
  const float* router_w;
  const float* shared_gate_w;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const uint8_t* shared_gate;
  const uint8_t* shared_up;
  const uint8_t* shared_down;
};

template <class T>
__device__ __forceinline__ const T* uniform_ptr(const void* p) {
  const unsigned long long a = (unsigned long long)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return reinterpret_cast<const T*>(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ LayerPtrs load_layer(const moe_layer_weights* table, int l) {
  const moe_layer_weights w = table[l];
  LayerPtrs p;
  p.norm_w = uniform_ptr<float>(w.norm_w);
  p.router_w = uniform_ptr<float>(w.router_w);
  p.shared_gate_w = uniform_ptr<float>(w.shared_gate_w);
  p.gate = uniform_ptr<uint8_t>(w.gate);
  p.up = uniform_ptr<uint8_t>(w.up);
  p.down = uniform_ptr<uint8_t>(w.down);
  p.shared_gate = uniform_ptr<uint8_t>(w.shared_gate);
  p.shared_up = uniform_ptr<uint8_t>(w.shared_up);
  p.shared_down = uniform_ptr<uint8_t>(w.shared_down);
  return p;
}

// Per-workgroup shares, LDS layout and exchange sizes of the persistent
// kernel for G workgroups (constexpr: also evaluated at compile time for the
// shape the kernel is specialised for).  The workspace offsets w_* are set by
// stack_ws_layout.
constexpr int up1k(long x) { return (int)((x + 1023) & ~1023L); }
constexpr int up16(long x) { return (int)((x + 15) & ~15L); }

constexpr int stack_geometry_core(int H, int E, int k, int F, int Fs, int down_type, int st, int G, StackGeom* out) {
  StackGeom g = {};
  const bool has_sg = Fs > 0;
  g.G = G;
  g.Kp = pad_k(down_type, F);
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
  const long rb_dn = row_bytes(down_type, g.Kp);
  const long rb_sdn = has_sg ? row_bytes(st, g.Kps) : 0;
  g.n_t = H / 2;
  g.n_lg = E + (has_sg ? 1 : 0);
  g.n_h = k * F + Fs;
  g.n_sel = 2 * k + 1;
  g.n_y = (k + 1) * H;   // the slots' down row values, then the shared expert's
  const int nblk = k * (g.Kp / 32) + g.Kps / 32;
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
  // the XCD-slot path (k = 8 on 256 workgroups) combines H/32 rows per
  // workgroup: as many row values
  const bool xs = (k == 8 && G == 256);
  const int rdx = xs ? H / (G / 8) : 0;
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
  np = np > 2L * rdx ? np : 2L * rdx;
  g.o_part = take(8L * np);
  long xb = g.n_h;                                   // words landing from an exchange
  xb = xb > g.n_t ? xb : g.n_t;
  xb = xb > g.n_lg ? xb : g.n_lg;
  // the exchange landing area is only written while the routed gate/up rows are
  // not in use (before they are staged, after they are consumed): share it
  if (4L * (xb + 2) <= 2L * g.rgu_half) g.o_xbuf = g.o_rgu;
  else g.o_xbuf = take(4L * (xb + 2));
  g.o_attn = take(up1k(2L * H));   // an attention-block output (bf16) of the layer
  g.o_sel = take(4L * (g.n_sel + 1));
  g.o_red = take(8L * (kStackThreads / 64));
  g.o_y = take(4L * (k + 1) * g.RD);
  g.o_cand = take(8L * 64);
  g.o_keys = take(8L * 256);
  g.o_lgsel = take(4L * (MOE_MAX_TOPK + 1));
  g.o_candlg = take(4L * 65);   // the candidates' logits and the shared-gate logit
  g.o_hs = take(4L * (g.Kps > 0 ? g.Kps : 1));
  g.lds = (int)o;
  if (g.lds < kStackMinLds) g.lds = kStackMinLds;   // keeps one workgroup per CU
  // workspace (exchange buffers after the per-layer region)
  out[0] = g;
  return MOE_OK;
}

// The shapes the kernel is also compiled for with every size a constant, on
// 256 workgroups: shape 1 = hidden 2048, 256 experts, top-8, expert and
// shared FFN 512 (down/shared types Q4_K/Q4_K and Q5_K/Q8_0); shape 2 =
// hidden 2048, 128 experts, top-8, expert FFN 768, no shared expert (Q4_K).
// Loop bounds, LDS offsets and quotients fold into the code, and the scalar
// registers that would hold them stay free.  Shape 0 takes every size from
// the arguments.
struct FixShape {
  int H, E, k, F, Fs, G;
};
constexpr FixShape kFixShapes[3] = {{0, 0, 0, 0, 0, 0}, {2048, 256, 8, 512, 512, 256}, {2048, 128, 8, 768, 0, 256}};
template <int DT, int ST, int S>
constexpr StackGeom fixed_geom() {
  StackGeom g = {};
  if (S != 0) {
    constexpr FixShape f = kFixShapes[S];
    stack_geometry_core(f.H, f.E, f.k, f.F, f.Fs, DT, ST, f.G, &g);
  }
  return g;
}
template <int DT, int ST, int S>
constexpr StackGeom kFixGeom = fixed_geom<DT, ST, S>();

// ---------------------------------------------------------------- the kernel
template <int DT, int ST, int S>
__global__ __launch_bounds__(kStackThreads) void k_stack(StackArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // S != 0: the geometry and sizes are the compile-time ones of shape S (the
  // launch checks that they equal the runtime ones); the workspace offsets
  // always come from the arguments
  constexpr bool FIX = S != 0;
  constexpr FixShape fs = kFixShapes[S];
  // XCD slots: with 8 selected experts on 256 workgroups, slot s is taken by
  // the 32 workgroups that run on die (XCC) s: their h exchange stays in that
  // die's L2
  constexpr bool XS = FIX && fs.k == kXcc && fs.G == 256;
  // XCD slots with the one-barrier selection (each polling wave finds its
  // slot's expert itself): measured faster for the Q5_K/Q8_0 stack (518.2 ->
  // 509.7 us per token) and slower for the Q4_K/Q4_K one (497.4 -> 501.2), so
  // that instance keeps the barrier
  constexpr bool OB = XS && !(DT == MOE_TYPE_Q4_K && ST == MOE_TYPE_Q4_K && S == 1);
  // router rows per workgroup of a fixed shape (E rows and the shared-gate row over G)
  constexpr int kRRFix = FIX ? (fs.E + (fs.Fs > 0 ? 1 : 0) + fs.G - 1) / fs.G : 0;
  const StackGeom g = FIX ? kFixGeom<DT, ST, S> : a.g;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const int H = FIX ? fs.H : a.H, E = FIX ? fs.E : a.E, k = FIX ? fs.k : a.k, F = FIX ? fs.F : a.F,
            Fs = FIX ? fs.Fs : a.Fs;
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
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(smem + g.o_cand);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(smem + g.o_keys);
  float* lgsel = reinterpret_cast<float*>(smem + g.o_lgsel);
  float* cand_lg = reinterpret_cast<float*>(smem + g.o_candlg);
  float* hsf = reinterpret_cast<float*>(smem + g.o_hs);   // the shared h, landed in phase B

  __shared__ uint32_t s_gen;
  __shared__ int s_fail;
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(a.ws + a.g.w_ctrl);
  const __amdgpu_buffer_rsrc_t r_ctrl = make_rsrc(ctrl, kStackCtrlBytes);
  if (tid == 0) {
    // the table bound in the workspace must be the caller's (the whole table's
    // hash), and no earlier launch may have stopped or been refused: a stopped
    // launch leaves exchange words of its generation behind, which a launch
    // of the same generation would take as current
    const bool bound = a.bound[0] == kBoundMagic && a.bound[1] == (uint32_t)a.L &&
                       a.bound[2] == (uint32_t)a.table_hash && a.bound[3] == (uint32_t)(a.table_hash >> 32);
    const uint32_t err = __builtin_amdgcn_raw_buffer_load_b32(r_ctrl, kErrWord * 4, 0, kAuxSC1);
    s_fail = !bound ? 2 : (err != 0u ? 3 : 0);
    // the XCD-slot exchanges pair each workgroup with the die it runs on
    if (XS && s_fail == 0 && xcc_id() >= (uint32_t)kXcc) {
      __builtin_amdgcn_raw_buffer_store_b32(3u, r_ctrl, kErrWord * 4, 0, kAuxSC1);
      s_fail = 3;
    }
    v2u gv = __builtin_amdgcn_raw_buffer_load_b64(r_ctrl, 0, 0, kAuxSC1);
    s_gen = gv.x;
  }
  lds_barrier();
  if (s_fail) {
    // refused: workgroup 0 sets the output to NaN; an unbound table is
    // recorded in the status word, an earlier failure stays as it is
    if (b == 0) {
      for (int i = tid; i < H; i += kStackThreads) a.output[i] = 0x7fc0u;
      if (tid == 0 && s_fail == 2) __builtin_amdgcn_raw_buffer_store_b32(2u, r_ctrl, kErrWord * 4, 0, kAuxSC1);
    }
    return;
  }
  const uint32_t base = s_gen * (uint32_t)(3 * a.L + 2) + 1u;

  // writers see every copy; this workgroup reads copy b % R
  const uint32_t rb_t = rep_bytes(g.n_t), rb_lg = rep_bytes(g.n_lg), rb_h = rep_bytes(g.n_h);
  // one resource over the three exchange areas (t, logits, h: consecutive in
  // the workspace); an area and a copy are picked by the instruction's
  // scalar offset, which keeps one descriptor in scalar registers instead of
  // one per area and copy
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.ws + a.g.w_t, (uint32_t)(a.g.w_trace - a.g.w_t));
  const uint32_t x_lg = (uint32_t)(a.g.w_lg - a.g.w_t), x_h = (uint32_t)(a.g.w_h - a.g.w_t),
                 x_y = (uint32_t)(a.g.w_y - a.g.w_t);
  // XS: the die this workgroup runs on.  A launch spreads its workgroups over
  // the 8 dies in rotation (workgroup b on die (b + r) % 8, r fixed for the
  // launch but not always 0), so each die holds exactly one workgroup of
  // every index j = b / 8: (die, j) names the workgroup's part of the XCD-slot
  // phases.  (Were a launch ever placed otherwise, some part would go
  // missing and the waits for it would stop the launch at their bound.)
  const uint32_t xcc = XS ? xcc_id() : 0u;
  const uint32_t rd_t = XS ? xcc * rb_t : 0u,
                 rd_h = x_h + (b % kRepH) * rb_h;

  const long rb_gu = row_bytes(MOE_TYPE_Q4_K, H);
  const long rb_sgu = has_sg ? row_bytes(ST, H) : 0;
  const long rb_dn = row_bytes(DT, g.Kp);
  const long rb_sdn = has_sg ? row_bytes(ST, g.Kps) : 0;
  const int row0 = b * g.RD;
  const int nrd = max(0, min(g.RD, H - row0));
  // reciprocals for quotients taken as float products (see their uses)
  const float inv_nrd = 1.0f / (float)max(nrd, 1);
  const float inv_nbr = 1.0f / (float)(g.Kp / 32);
  const int sf0 = b * g.SR;
  const int nsr = has_sg ? max(0, min(g.SR, Fs - sf0)) : 0;

  // XS: this workgroup's down rows (and combine rows) [dr0, dr0 + RDX)
  constexpr int RDX = XS ? fs.H / (fs.G / kXcc) : 0;
  const int dr0 = (b / kXcc) * RDX;
  // PD (XS with at most 4 router rows per workgroup): the router per die.
  // The 32 workgroups of die x compute all E logits (workgroup (x, j) rows j,
  // j + 32, ...; the shared-gate row too when j == 0) and exchange them within
  // the die, in its copy of the logits area, instead of across the dies.  The
  // rows stream into the router row area, then the routed gate/up and down
  // areas, which are idle from the end of a layer to the next one's
  // selection.  Each die then reads the whole router matrix: measured, this
  // pays at 4 rows per workgroup (128 experts: 698 -> 666 us per 48-layer
  // token) and not at 8 (256 experts: 525 -> 837 us per 40-layer token, the
  // 18 MB of router rows per layer stalling the row streams).
  constexpr int kRowsPD = XS ? fs.E / (fs.G / kXcc) : 0;
  constexpr bool PD = XS && kRowsPD <= 4;
  // FR: router dots fused into the norm (every router row already landed when
  // the norm runs, one float4 of xn per thread); kRRFused rows per workgroup
  constexpr bool FR = FIX && !PD && fs.H == 4 * kStackThreads && kRRFix <= 2;
  constexpr int kRRFused = FR ? kRRFix : 1;
  static_assert(!FR || kRRFused * kStackWaves <= (fs.k + 1) * kFixGeom<DT, ST, S>.RD,
                "the wave partials fit the row-value area (at least (k + 1) * RD doubles)");
  constexpr StackGeom gx = kFixGeom<DT, ST, S>;
  constexpr int kRowB = PD ? fs.H * 4 : 1;
  constexpr int kCapR = PD ? (gx.o_sgu - gx.o_rrow) / kRowB : 0, kCapG = PD ? (gx.o_rdn - gx.o_rgu) / kRowB : 0,
                kCapD = PD ? (gx.o_hqc - gx.o_rdn) / kRowB : 0;
  static_assert(!PD || (gx.o_sgu > gx.o_rrow && gx.o_rdn > gx.o_rgu && gx.o_hqc > gx.o_rdn), "router row areas");
  static_assert(!PD || kCapR + kCapG + kCapD >= kRowsPD + 1, "the router rows of a die's workgroup fit");
  static_assert(!PD || (fs.E % (fs.G / kXcc) == 0 && kRepLg == kXcc), "router per die");
  const int jd = XS ? b / kXcc : 0;                          // the workgroup's index within its die
  const int nrows_pd = PD ? kRowsPD + ((jd == 0 && has_sg) ? 1 : 0) : 0;
  // the logits copy this workgroup reads: its die's (PD), else copy b % R
  const uint32_t rd_lg = x_lg + (PD ? xcc : (uint32_t)(b % kRepLg)) * rb_lg;
  auto router_slot = [&](int m) -> uint8_t* {
    return m < kCapR ? rrow + (long)m * kRowB
                     : (m < kCapR + kCapG ? rgu + (long)(m - kCapR) * kRowB : rdn + (long)(m - kCapR - kCapG) * kRowB);
  };
  // weights that do not depend on the routing decision, for layer `w`
  // The next layer's fixed weights, requested at the layer's end, except the
  // norm weight of the per-die form, requested as soon as this layer has sent
  // its shared h (it is not read again): there the norm waits on its router
  // rows, and the norm weight landing early shortens that wait (the
  // 128-expert stack: 666 -> 660 us per token).  In the 256-expert form any
  // load issued then runs into the cross-die logits exchange: requesting the
  // norm weight early cost 9 us per token, with the router rows 29 us.
  auto prefetch_early = [&](const LayerPtrs& w) {
    if (PD) stage_async(smem + g.o_nw, w.norm_w, (uint32_t)(H * 4), wave, kPollWaves, kStackWaves - kPollWaves);
  };
  auto prefetch_late = [&](const LayerPtrs& w) {
    if (!PD) stage_async(smem + g.o_nw, w.norm_w, (uint32_t)(H * 4), wave, kPollWaves, kStackWaves - kPollWaves);
    for (int j = 0; !PD && j < g.RR; ++j) {
      const int r = b + j * g.G;
      const float* src = (r < E) ? w.router_w + (long)r * H : ((r == E && has_sg) ? w.shared_gate_w : nullptr);
      if (src) stage_async(rrow + (long)j * H * 4, src, (uint32_t)(H * 4), wave, kPollWaves, kStackWaves - kPollWaves);
    }
    if (nsr > 0) {
      stage_async(sgu, w.shared_gate + sf0 * rb_sgu, (uint32_t)(nsr * rb_sgu), wave, kPollWaves,
                  kStackWaves - kPollWaves);
      stage_async(sgu + g.sgu_half, w.shared_up + sf0 * rb_sgu, (uint32_t)(nsr * rb_sgu), wave,
                  kPollWaves, kStackWaves - kPollWaves);
    }
    if (has_sg && nrd > 0)
      stage_async(sdn, w.shared_down + row0 * rb_sdn, (uint32_t)(nrd * rb_sdn), wave, kPollWaves,
                  kStackWaves - kPollWaves);
    // PD: the router rows last, so that the norm can wait for the rest alone
    for (int m = 0; PD && m < nrows_pd; ++m) {
      const float* src = (m < kRowsPD) ? w.router_w + (long)(jd + (fs.G / kXcc) * m) * H : w.shared_gate_w;
      stage_async(router_slot(m), src, (uint32_t)(H * 4), wave, kPollWaves, kStackWaves - kPollWaves);
    }
  };

  uint64_t* trace = reinterpret_cast<uint64_t*>(a.ws + a.g.w_trace);
  auto stamp = [&](int l, int i) {
    if (b == 0 && tid == 0 && l < kTraceLayers) {
      trace[l * kTraceSlots + i] = wall_clock64();
      if (i == 0) trace[l * kTraceSlots + 10] = clock64();
      if (i == 9) trace[l * kTraceSlots + 11] = clock64();
    }
  };
  uint64_t* btrace = trace + kTraceLayers * kTraceSlots;
  auto bstamp = [&](int l, int i) {
    if (a.trace_blocks && tid == 0 && l < kTraceLayers && b < kTraceMaxG)
      btrace[((long)l * kTraceMaxG + b) * kBlockEvents + i] = wall_clock64();
  };

  // a stopped launch: status 1, and beside it the layer and the check that
  // stopped it (s_fail: 1 the t words, 2 the logits, 3 an incomplete
  // selection, 4 the shared h, 5 the routed h, 6 the down rows' values, 7 the
  // last t for the output)
  auto fail_out = [&](int l) {
    if (tid == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(((uint32_t)l << 8) | (uint32_t)s_fail, r_ctrl, (kErrWord + 1) * 4, 0,
                                            kAuxSC1);
      __builtin_amdgcn_raw_buffer_store_b32(1u, r_ctrl, kErrWord * 4, 0, kAuxSC1);
    }
  };

  // ---- layer-0 inputs: the token's residual, no previous outputs
  for (int i = tid; i < H; i += kStackThreads) res[i] = bf16_to_f32(a.input[i]);
  LayerPtrs w = load_layer(a.layers, 0);
  prefetch_early(w);
  prefetch_late(w);
  LayerPtrs w_next = w;

  for (int l = 0; l < a.L; ++l) {
    const uint32_t ep0 = base + 3u * l, ep1 = ep0 + 1u, ep2 = ep0 + 2u;
    stamp(l, 0);
    bstamp(l, 0);
    // this layer's attention-block output, if any, streamed into LDS by the
    // polling waves now, so that the t exchange hides the transfer
    if (a.attn) stage_async(smem + g.o_attn, a.attn + (long)l * H, (uint32_t)(2 * H), wave, 0, kPollWaves);
    // ================= R1: t of the previous layer, read by every workgroup.
    // Word pair p holds t rows 4p..4p+3 (bf16 pairs); the polling lane adds
    // them to its residual float4 as soon as they are current and takes the
    // sum of squares of the new residual on the way
    double ss = 0.0;
    float4* res4 = reinterpret_cast<float4*>(res);
    if (l > 0) {
      const bool ok = poll_ll_sink<kAuxSC1>(rx, rd_t, g.n_t, ep2 - 3u, kPollWaves, 0,
                                            [&](uint32_t p, uint32_t x, uint32_t z) {
        float4 r = res4[p];
        r.x = bf16_to_f32(f32_to_bf16(r.x + bf16_to_f32((uint16_t)(x & 0xffffu))));
        r.y = bf16_to_f32(f32_to_bf16(r.y + bf16_to_f32((uint16_t)(x >> 16))));
        r.z = bf16_to_f32(f32_to_bf16(r.z + bf16_to_f32((uint16_t)(z & 0xffffu))));
        r.w = bf16_to_f32(f32_to_bf16(r.w + bf16_to_f32((uint16_t)(z >> 16))));
        res4[p] = r;
        ss += sq4_f64(r);
      });
      if (!ok) s_fail = 1;
    } else {
      for (int c = tid; c < H / 4; c += kStackThreads) ss += sq4_f64(res4[c]);
    }
    // ================= phase A: norm, router rows, shared gate/up rows
    stamp(l, 1);
    bstamp(l, 1);
    if (wave >= kPollWaves) {
      if constexpr (PD) {
        // everything but the router rows (the last requests: two KiB per row
        // from each of the four issuing waves) has landed
        static_assert(fs.H * 4 == 1024 * (kStackWaves - kPollWaves) * 2, "two KiB per router row and wave");
        if (nrows_pd > kRowsPD) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (kRowsPD + 1)) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kRowsPD) : "memory");
      } else {
        wait_vmem();
      }
    }
    if (a.attn) {
      // the post-attention add: u2 = bf16(u1 + attn), once every t word and
      // the attention output are in
      if (wave < kPollWaves) wait_vmem();
      lds_barrier();
      ss = 0.0;
      const uint2* av = reinterpret_cast<const uint2*>(smem + g.o_attn);
      for (int c = tid; c < H / 4; c += kStackThreads) {
        float4 r = res4[c];
        const uint2 v = av[c];
        r.x = bf16_to_f32(f32_to_bf16(r.x + bf16_to_f32((uint16_t)(v.x & 0xffffu))));
        r.y = bf16_to_f32(f32_to_bf16(r.y + bf16_to_f32((uint16_t)(v.x >> 16))));
        r.z = bf16_to_f32(f32_to_bf16(r.z + bf16_to_f32((uint16_t)(v.y & 0xffffu))));
        r.w = bf16_to_f32(f32_to_bf16(r.w + bf16_to_f32((uint16_t)(v.y >> 16))));
        res4[c] = r;
        ss += sq4_f64(r);
      }
    }
    // the barrier inside also publishes s_fail and the new residual
    ss = block_sum_f64(ss, red);
    if (s_fail) { fail_out(l); return; }
    stamp(l, 2);
    bstamp(l, 2);
    if (b == 0 && a.resid_out)
      for (int i = tid; i < H; i += kStackThreads) a.resid_out[(long)l * H + i] = f32_to_bf16(res[i]);
    const double rinv = 1.0 / sqrt(ss / (double)H + (double)a.eps);
    // FR (a fixed shape with one float4 of xn per thread and the router rows
    // already landed): each thread also takes its four products with each of
    // the workgroup's router rows, and the rows' sums travel through the
    // barrier below instead of a pass over xn after it
    double rp[kRRFused];
    for (int c = tid; c < H / 4; c += kStackThreads) {
      const float4 r = res4[c];
      const float4 wv = reinterpret_cast<const float4*>(nw)[c];
      float4 o;
      o.x = (float)(((double)r.x * rinv) * (double)wv.x);
      o.y = (float)(((double)r.y * rinv) * (double)wv.y);
      o.z = (float)(((double)r.z * rinv) * (double)wv.z);
      o.w = (float)(((double)r.w * rinv) * (double)wv.w);
      reinterpret_cast<float4*>(xn)[c] = o;
      if constexpr (FR) {
#pragma unroll
        for (int j = 0; j < kRRFused; ++j) {
          const float4 rw = reinterpret_cast<const float4*>(rrow + (long)j * H * 4)[c];
          rp[j] = ((double)rw.x * (double)o.x + (double)rw.y * (double)o.y) +
                  ((double)rw.z * (double)o.z + (double)rw.w * (double)o.w);
        }
      }
    }
    if constexpr (FR) {
#pragma unroll
      for (int j = 0; j < kRRFused; ++j) {
        const double s = wave_sum_f64(rp[j]);
        if ((tid & 63) == 0) part[j * kStackWaves + wave] = s;
      }
    }
    if (PD && wave >= kPollWaves) wait_vmem();   // the router rows
    lds_barrier();
    bstamp(l, 11);
    // xq on waves 0..3 while waves 4.. take the router rows, which need xn only
    if (wave < kPollWaves)
      quantize_q81_groups<4, 1>(H / 32, xn, [](int j) { return 32 * j; }, [&](int j) { return xqc + 32 * j; }, xqd,
                                xqs, tid, 64 * kPollWaves);
    bstamp(l, 12);
    // PD: this workgroup's router rows of its die (fp64 dot of fp32 products),
    // one wave per row; the logits go to the die's copy with plain stores
    for (int m = wave - kPollWaves; PD && m >= 0 && m < nrows_pd; m += kStackWaves - kPollWaves) {
      const float* wr = reinterpret_cast<const float*>(router_slot(m));
      double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 4
      for (int i = (tid & 63) * 4; i < H; i += 256) {
        const float4 wv = *reinterpret_cast<const float4*>(wr + i);
        const float4 xv = *reinterpret_cast<const float4*>(xn + i);
        a0 += (double)wv.x * (double)xv.x;
        a1 += (double)wv.y * (double)xv.y;
        a2 += (double)wv.z * (double)xv.z;
        a3 += (double)wv.w * (double)xv.w;
      }
      const double acc = wave_sum_f64((a0 + a1) + (a2 + a3));
      const int r = (m < kRowsPD) ? jd + (fs.G / kXcc) * m : E;
      if ((tid & 63) == 0) {
        const v2u v = {__float_as_uint((float)acc), ep0};
        __builtin_amdgcn_raw_buffer_store_b64(v, rx, 8u * (uint32_t)r, x_lg + xcc * rb_lg, 0);
      }
    }
    // FR: the router rows' sums of the wave partials, in wave order, by the
    // first lanes of wave kPollWaves
    if constexpr (FR) {
      const int j = tid - 64 * kPollWaves;
      if (j >= 0 && j < kRRFused) {
        const int r = b + j * g.G;
        if ((r < E) || (r == E && has_sg)) {
          double acc = 0.0;
#pragma unroll
          for (int w2 = 0; w2 < kStackWaves; ++w2) acc += part[j * kStackWaves + w2];
          ll_store_rep<kRepLg>(rx, x_lg, rb_lg, r, __float_as_uint((float)acc), ep0);
        }
      }
    }
    // router rows (fp64 dot of fp32 products), one wave per row
    for (int j = wave - kPollWaves; !PD && !FR && j >= 0 && j < g.RR; j += kStackWaves - kPollWaves) {
      const int r = b + j * g.G;
      const bool real = (r < E) || (r == E && has_sg);
      if (!real) break;
      const float* wr = reinterpret_cast<const float*>(rrow + (long)j * H * 4);
      // four independent fp64 partial sums per lane (fp64 keeps the fp32 result
      // of the sum independent of its order but for rare last-bit cases)
      double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 4
      for (int i = (tid & 63) * 4; i < H; i += 256) {
        const float4 wv = *reinterpret_cast<const float4*>(wr + i);
        const float4 xv = *reinterpret_cast<const float4*>(xn + i);
        a0 += (double)wv.x * (double)xv.x;
        a1 += (double)wv.y * (double)xv.y;
        a2 += (double)wv.z * (double)xv.z;
        a3 += (double)wv.w * (double)xv.w;
      }
      const double acc = wave_sum_f64((a0 + a1) + (a2 + a3));
      if ((tid & 63) == 0) ll_store_rep<kRepLg>(rx, x_lg, rb_lg, r, __float_as_uint((float)acc), ep0);
    }
    bstamp(l, 3);
    lds_barrier();
    // shared gate/up rows -> hs (word k*F + f of the h exchange)
    if (nsr > 0) {
      const ActLds act{xqc, xqd, xqs};
      rows_dot<ST>(2 * nsr, tasks_per_row(ST, H), [&](int r) {
        return RowRef{(r < nsr) ? sgu + (long)r * rb_sgu : sgu + g.sgu_half + (long)(r - nsr) * rb_sgu, act};
      }, part, wave, kStackWaves);
      lds_barrier();
      if (tid < nsr) {
        const float gg = (float)part[tid];
        const float uu = (float)part[nsr + tid];
        const float hv = (float)(silu_f64((double)gg) * (double)uu);
        ll_store_rep<kRepH>(rx, x_h, rb_h, k * F + sf0 + tid, __float_as_uint(hv), ep1);
      }
    }
    // the next layer's early weights (per-die form): this layer has read its own
    if constexpr (PD) {
      if (l + 1 < a.L) {
        w_next = load_layer(a.layers, l + 1);
        prefetch_early(w_next);
      }
    }
    // ================= R2: logits -> selection, in every workgroup
    stamp(l, 3);
    bstamp(l, 4);
    uint32_t e_slot = 0;   // OB: this slot's expert, found by each polling wave
    bool sel_ok = true;
    {
      if (E <= 256) {
        // wave w < 4 polls the logits of its own 64 experts (word pairs
        // 32w .. 32w+31; pair 128, the shared-gate logit after 256 experts,
        // on lane 32 of wave 0), lands them and ranks them right away
        if (wave < kPollWaves) {
          const int lane = tid & 63;
          const int p = 32 * wave + (lane & 31) + 128 * (lane >> 5);
          const int pair[1] = {(uint32_t)p < ((g.n_lg + 1u) >> 1) ? p : -1};
          uint32_t lo[1] = {0u}, hi[1] = {0u};
          if (!poll_lane_pairs<kAuxSC1, 1>(rx, rd_lg, pair, g.n_lg, ep0, lo, hi)) s_fail = 2;
          if (pair[0] >= 0) {
            xbuf[2 * p] = lo[0];
            if (2 * p + 1 < g.n_lg) xbuf[2 * p + 1] = hi[0];
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
          bstamp(l, 13);
          // OB: the candidates' logits (and the shared-gate logit, landed by
          // wave 0) are copied beside them, as the landing area takes the
          // routed rows once the selection is known
          if (OB && wave == 0 && lane == 0) cand_lg[64] = has_sg ? reinterpret_cast<const float*>(xbuf)[E] : 0.0f;
          topk_candidates(reinterpret_cast<const float*>(xbuf), E, k, wave, keys, cand, OB ? cand_lg : nullptr);
        }
        lds_barrier();
        if (s_fail) { fail_out(l); return; }
      } else {
        const bool ok = poll_ll<kAuxSC1>(rx, rd_lg, g.n_lg, ep0, xbuf, kPollWaves);
        if (!ok) s_fail = 2;
        lds_barrier();
        if (s_fail) { fail_out(l); return; }
        bstamp(l, 13);
        topk_candidates(reinterpret_cast<const float*>(xbuf), E, k, wave, keys, cand);
        lds_barrier();
      }
      if constexpr (OB) {
        // no second barrier: each polling wave finds its slot's expert in
        // the candidates itself, and wave 0 writes the selection for the
        // combine from the candidates and their copied logits (a later
        // barrier publishes it; a failed selection stops the layer there)
        if (wave < kPollWaves) {
          bool ok = true;
          e_slot = candidate_of_rank(cand, k, (int)xcc, ok);
          sel_ok = ok;
          if (!ok) s_fail = 3;
        }
        if (wave == 0) {
          if (rank_candidates(reinterpret_cast<const float*>(xbuf), E, k, has_sg, cand, sel, lgsel, cand_lg))
            s_fail = 3;
          if (b == 0 && a.ids_out) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
            if (tid < k) a.ids_out[(long)l * k + tid] = (int32_t)sel[tid];
          }
        }
      } else {
        if (wave == 0 && rank_candidates(reinterpret_cast<const float*>(xbuf), E, k, has_sg, cand, sel, lgsel))
          s_fail = 3;
        lds_barrier();
        if (s_fail) { fail_out(l); return; }
        if (b == 0 && a.ids_out)
          for (int s = tid; s < k; s += kStackThreads) a.ids_out[(long)l * k + s] = (int32_t)sel[s];
      }
    }
    stamp(l, 4);
    bstamp(l, 5);
    // ================= phase B: routed gate/up rows (this workgroup's slot and rows)
    // XS: slot = the die, h rows [f0, f0 + F/32) and down rows [dr0, dr0 + H/32)
    // of that slot's expert; else consecutive workgroups share a slot
    const int p0 = b * g.RP;
    const int slot = XS ? (int)xcc : p0 / F;
    const int f0 = XS ? (b / kXcc) * (F / (fs.G / kXcc)) : p0 - slot * F;
    const int nrp = XS ? F / (fs.G / kXcc) : ((slot < k) ? min(g.RP, F - f0) : 0);

    if (nrp > 0 && wave < kPollWaves && sel_ok) {
      const long e = OB ? (long)e_slot : (long)sel[slot];
      stage_async(rgu, w.gate + (e * F + f0) * rb_gu, (uint32_t)(nrp * rb_gu), wave, 0, kPollWaves);
      stage_async(rgu + g.rgu_half, w.up + (e * F + f0) * rb_gu, (uint32_t)(nrp * rb_gu), wave, 0,
                  kPollWaves);
    }
    // the routing weights are first needed by the combine: computed while the rows land
    // (OB: scratch in the keys, as slower polling waves may still read the candidates)
    if (wave == 0) routing_weights(k, has_sg, lgsel, sel, reinterpret_cast<double*>(OB ? keys : cand));
    // meanwhile wave 4 reads the shared h (sent in phase A, so long arrived)
    // and quantises it: h blocks k*nb_r .. k*nb_r + nb_s - 1
    if (has_sg && wave == kPollWaves) {
      // the shared h words follow the k*F routed words
      if (!poll_ll<kAuxSC1>(rx, rd_h + 8u * k * F, Fs, ep1, reinterpret_cast<uint32_t*>(hsf), 1, kPollWaves)) s_fail = 4;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      const int nb_r = g.Kp / 32;
      quantize_q81_groups<4, 1>(g.Kps / 32, hsf, [&](int j) { return (32 * j < Fs) ? 32 * j : -1; },
                                [&](int j) { return hqc + (long)k * g.Kp + 32 * j; }, hqd + k * nb_r, hqs + k * nb_r,
                                tid & 63, 64);
    }
    if (wave < kPollWaves) wait_vmem();
    lds_barrier();
    if (s_fail) { fail_out(l); return; }
    stamp(l, 5);
    bstamp(l, 6);
    // the down rows are needed only after the h exchange: requested once the
    // gate/up rows have landed, so they do not share the memory system with
    // them (requested together, the gate/up rows land later by more than the
    // request time saved)
    if (XS && wave >= kPollWaves) {
      // this slot's down rows [dr0, dr0 + RDX): one contiguous stream, queued
      // once the gate/up rows have landed (queued beside them, they delay the
      // gate/up rows by more than the down rows gain)
      const long e = sel[slot];
      stage_async(rdn, w.down + (e * H + dr0) * rb_dn, (uint32_t)(RDX * rb_dn), wave, kPollWaves,
                  kStackWaves - kPollWaves);
    } else if (!XS && nrd > 0 && wave >= kPollWaves) {
      // wave 4+j queues slots j, j+4, j+8, j+12: their ids are read first, so
      // the requests go out back to back instead of each after an LDS round trip
      const int j = wave - kPollWaves;
      constexpr int kSlotsPerWave = (MOE_MAX_TOPK + kStackWaves - kPollWaves - 1) / (kStackWaves - kPollWaves);
      uint32_t ex[kSlotsPerWave];
#pragma unroll
      for (int i = 0; i < kSlotsPerWave; ++i) {
        const int s = j + (kStackWaves - kPollWaves) * i;
        ex[i] = (s < k) ? sel[s] : 0u;
      }
#pragma unroll
      for (int i = 0; i < kSlotsPerWave; ++i) {
        const int s = j + (kStackWaves - kPollWaves) * i;
        if (s < k)
          stage_async(rdn + (long)s * g.rdn_slot, w.down + ((long)ex[i] * H + row0) * rb_dn, (uint32_t)(nrd * rb_dn),
                      0, 0, 1);
      }
    }
    if (a.trace_blocks && tid == 256 && l < kTraceLayers && b < kTraceMaxG)
      btrace[((long)l * kTraceMaxG + b) * kBlockEvents + 15] = wall_clock64();
    if (nrp > 0) {
      const ActLds act{xqc, xqd, xqs};
      rows_dot<MOE_TYPE_Q4_K>(2 * nrp, tasks_per_row(MOE_TYPE_Q4_K, H), [&](int r) {
        return RowRef{(r < nrp) ? rgu + (long)r * rb_gu : rgu + g.rgu_half + (long)(r - nrp) * rb_gu, act};
      }, part, wave, kStackWaves);
      lds_barrier();
      if (tid < nrp) {
        const float gg = (float)part[tid];
        const float uu = (float)part[nrp + tid];
        const float hv = (float)(silu_f64((double)gg) * (double)uu);
        if (XS) {   // this XCC's copy of the h area, word f; a plain store stays in the XCC's L2
          const v2u v = {__float_as_uint(hv), ep1};
          __builtin_amdgcn_raw_buffer_store_b64(v, rx, 8u * (f0 + tid), x_h + slot * rb_h, 0);
        }
        else
          ll_store_rep<kRepH>(rx, x_h, rb_h, slot * F + f0 + tid, __float_as_uint(hv), ep1);
      }
    }
    // ================= R3: every routed h, read and quantised to Q8_1 by every workgroup
    // (the shared h was done in phase B)
    stamp(l, 6);
    bstamp(l, 7);
    if constexpr (XS) {
      // the shared expert's rows of the combine rows [row0, row0 + nrd): its
      // h was quantised in phase B, so this runs while the slot's h travels
      if (has_sg) {
        // computed once: rows [row0, row0 + nrd), sent as fp32 row values
        // (words H*k + row0 + r of the y area) to the workgroups that combine them
        const ActLds acts{hqc + (long)k * g.Kp, hqd + k * (g.Kp / 32), hqs + k * (g.Kp / 32)};
        rows_dot<ST>(nrd, tasks_per_row(ST, g.Kps), [&](int r) { return RowRef{sdn + (long)r * rb_sdn, acts}; },
                     part + RDX, wave, kStackWaves);
        lds_barrier();
        if (tid < nrd)
          ll_store(rx, (x_y >> 3) + (uint32_t)(k * H + row0 + tid), __float_as_uint((float)part[RDX + tid]), ep1,
                   kAuxSC1);
      }
      // this slot's h only, from this XCC's copy of the h area (its L2)
      if (!poll_quantize_h(rx, x_h + slot * rb_h, g.Kp / 32, g.Kp / 32, inv_nbr, F, (uint32_t)F, ep1, xbuf, hqc, hqd,
                           hqs, wave, kStackWaves))
        s_fail = 5;
      bstamp(l, 14);
    } else {
      // the down rows waves 4..7 requested in phase B have had the whole of
      // phase B to land, so every wave polls; each wave quantises its own
      // blocks as soon as they are current
      if (!poll_quantize_h(rx, rd_h, k * (g.Kp / 32), g.Kp / 32, inv_nbr, F, (uint32_t)(k * F), ep1, xbuf, hqc, hqd,
                           hqs, wave, kStackWaves))
        s_fail = 5;
      bstamp(l, 14);
    }
    // ================= phase C: down rows of all slots + shared, combine
    stamp(l, 7);
    bstamp(l, 8);
    if (wave >= kPollWaves) wait_vmem();
    lds_barrier();
    if (s_fail) { fail_out(l); return; }
    stamp(l, 8);
    bstamp(l, 9);
    if constexpr (XS) {
      // this slot's down rows [dr0, dr0 + RDX) -> y (fp32 row values), and
      // the shared expert's rows of the combine rows [row0, row0 + nrd)
      const ActLds actr{hqc, hqd, hqs};
      rows_dot<DT>(RDX, tasks_per_row(DT, g.Kp), [&](int r) { return RowRef{rdn + (long)r * rb_dn, actr}; }, part,
                   wave, kStackWaves);
      lds_barrier();
      // y of row i of slot s travels as word s*H + i (read by the one
      // workgroup that combines row i)
      if (tid < RDX) ll_store(rx, (x_y >> 3) + (uint32_t)(slot * H + dr0 + tid), __float_as_uint((float)part[tid]), ep1,
                              kAuxSC1);
      // the k slots' y of this workgroup's rows [dr0, dr0 + RDX): slot s's
      // words s*H + dr0 .. are RDX/2 pairs; waves 0..3 poll one pair per lane
      // (and, on wave 4, the shared expert's row values of the same rows:
      // words k*H + dr0 .., landed as "slot" k)
      if (wave <= kPollWaves) {
        constexpr int PPS = XS ? RDX / 2 : 1;   // word pairs per slot
        const int ps = tid / PPS, q = tid - ps * PPS;
        const bool live = ps < k || (ps == k && has_sg);
        const int pair[1] = {live ? (int)((x_y >> 4) + ((uint32_t)(ps * H + dr0) >> 1) + q) : -1};
        uint32_t lo[1] = {0u}, hi[1] = {0u};
        if (!poll_lane_pairs<kAuxSC1, 1>(rx, 0u, pair, 0xffffffffu, ep1, lo, hi)) s_fail = 6;
        if (live) {
          xbuf[ps * RDX + 2 * q] = lo[0];
          xbuf[ps * RDX + 2 * q + 1] = hi[0];
        }
      }
      lds_barrier();
      if (s_fail) { fail_out(l); return; }
      // combine: one lane per (row, slot), the k slots of a row in k adjacent
      // lanes summed by a DPP tree (fp64; y_s is the fp32 row value); the
      // per-layer outputs come from XCC 0's workgroups
      const float sgv = __uint_as_float(sel[2 * k]);
      uint16_t* tb = reinterpret_cast<uint16_t*>(yv);
      for (int i = tid; i < RDX * kXcc; i += kStackThreads) {
        const int r = i / kXcc, sl = i - r * kXcc;
        double v = (double)__uint_as_float(sel[k + sl]) * (double)__uint_as_float(xbuf[sl * RDX + r]);
        v = group_sum_f64(v, kXcc);
        if (sl == 0) {
          const uint16_t routed = f32_to_bf16((float)v);
          float t = bf16_to_f32(routed);
          if (a.routed_out && slot == 0) a.routed_out[(long)l * H + dr0 + r] = routed;
          if (has_sg) {
            const uint16_t shared = f32_to_bf16((float)((double)sgv * (double)__uint_as_float(xbuf[k * RDX + r])));
            t = bf16_to_f32(f32_to_bf16(bf16_to_f32(routed) + bf16_to_f32(shared)));
            if (a.shared_out && slot == 0) a.shared_out[(long)l * H + dr0 + r] = shared;
          }
          tb[r] = f32_to_bf16(t);
        }
      }
      lds_barrier();
      // t rows [dr0, dr0 + RDX) into this XCC's copy of t: plain stores, its L2
      for (int r2 = tid; 2 * r2 < RDX; r2 += kStackThreads) {
        const v2u v = {(uint32_t)tb[2 * r2] | ((uint32_t)tb[2 * r2 + 1] << 16), ep2};
        __builtin_amdgcn_raw_buffer_store_b64(v, rx, 8u * ((dr0 >> 1) + r2), rd_t, 0);
      }
    } else if (nrd > 0) {
      // row r < k*nrd is row r % nrd of slot r / nrd (the quotient from a
      // float product, exact as for the h blocks above); with the shared
      // expert's rows of the same type, its nrd rows follow as one more slot
      // in the same pass (they then run alongside the slot rows of one wave)
      const ActLds acts{hqc + (long)k * g.Kp, hqd + k * (g.Kp / 32), hqs + k * (g.Kp / 32)};
      const bool one_pass = has_sg && DT == ST && g.Kps == g.Kp;
      rows_dot<DT>((k + (one_pass ? 1 : 0)) * nrd, tasks_per_row(DT, g.Kp), [&](int r) {
        const int s = (int)(((float)r + 0.5f) * inv_nrd), rr = r - s * nrd;
        if (s == k) return RowRef{sdn + (long)rr * rb_sdn, acts};
        return RowRef{rdn + (long)s * g.rdn_slot + (long)rr * rb_dn,
                      ActLds{hqc + (long)s * g.Kp, hqd + s * (g.Kp / 32), hqs + s * (g.Kp / 32)}};
      }, part, wave, kStackWaves);
      if (has_sg && !one_pass)
        rows_dot<ST>(nrd, tasks_per_row(ST, g.Kps), [&](int r) { return RowRef{sdn + (long)r * rb_sdn, acts}; },
                     part + k * nrd, wave, kStackWaves);
      lds_barrier();
      // combine: one lane per (row, slot), the slots of a row in GS adjacent
      // lanes summed by a DPP tree (fp64; y_s is the fp32 row value)
      const float sgv = __uint_as_float(sel[2 * k]);
      const int GS = (k <= 8) ? 8 : 16;
      uint16_t* tb = reinterpret_cast<uint16_t*>(yv);
      for (int i = tid; i < nrd * GS; i += kStackThreads) {
        const int r = i / GS, sl = i - r * GS;
        double v = 0.0;
        if (sl < k) v = (double)__uint_as_float(sel[k + sl]) * (double)(float)part[sl * nrd + r];
        v = group_sum_f64(v, GS);
        if (sl == 0) {
          const uint16_t routed = f32_to_bf16((float)v);
          float t = bf16_to_f32(routed);
          if (a.routed_out) a.routed_out[(long)l * H + row0 + r] = routed;
          if (has_sg) {
            const uint16_t shared = f32_to_bf16((float)((double)sgv * (double)(float)part[k * nrd + r]));
            t = bf16_to_f32(f32_to_bf16(bf16_to_f32(routed) + bf16_to_f32(shared)));
            if (a.shared_out) a.shared_out[(long)l * H + row0 + r] = shared;
          }
          tb[r] = f32_to_bf16(t);
        }
      }
      lds_barrier();
      for (int r2 = tid; 2 * r2 < nrd; r2 += kStackThreads)
        ll_store_rep<1>(rx, 0u, rb_t, (row0 >> 1) + r2, (uint32_t)tb[2 * r2] | ((uint32_t)tb[2 * r2 + 1] << 16), ep2);
    }
    lds_barrier();
    stamp(l, 9);
    bstamp(l, 10);
    if (l + 1 < a.L) {
      w = PD ? w_next : load_layer(a.layers, l + 1);
      prefetch_late(w);
    }
  }
  // ================= the fold a next layer would do: output = bf16(res + t)
  if (b == 0) {
    const uint32_t epl = base + 3u * (a.L - 1) + 2u;
    const bool ok = poll_ll<kAuxSC1>(rx, rd_t, g.n_t, epl, xbuf, kPollWaves);
    if (!ok) s_fail = 7;
    lds_barrier();
    if (s_fail) { fail_out(a.L); return; }
    for (int i = tid; i < H; i += kStackThreads) {
      const uint32_t pr = xbuf[i >> 1];
      const float t = bf16_to_f32((uint16_t)((i & 1) ? (pr >> 16) : (pr & 0xffffu)));
      a.output[i] = f32_to_bf16(res[i] + t);
    }
    lds_barrier();
    if (tid == 0) {
      v2u nv = {s_gen + 1u, 0u};
      __builtin_amdgcn_raw_buffer_store_b64(nv, r_ctrl, 0, 0, kAuxSC1);
    }
  }
}

// ---------------------------------------------------------------- test export of the selection
// One workgroup per logit set runs the stack kernel's selection exactly as a
// layer does: topk_candidates on waves 0..3, rank_candidates and
// routing_weights on wave 0, with the same LDS arrays and barriers.  For
// E <= 256 and k <= 8 it also runs the one-barrier form (candidate_of_rank
// on waves 0..3, the merge from the copied candidate logits on wave 1) and
// reports ids of -1 unless both forms agree bit for bit.
__global__ __launch_bounds__(kStackThreads) void k_test_stack_select(const float* lg_in, int E, int k, int with_gate,
                                                                     int32_t* ids, float* wts, float* gate) {
  __shared__ float lg[MOE_MAX_EXPERTS + 1];
  __shared__ unsigned long long keys[256];
  __shared__ unsigned long long cand[64];
  __shared__ uint32_t sel[2 * MOE_MAX_TOPK + 2];
  __shared__ float lgsel[MOE_MAX_TOPK + 1];
  __shared__ float cand_lg[65];
  __shared__ float lgsel2[MOE_MAX_TOPK + 1];
  __shared__ uint32_t sel2[MOE_MAX_TOPK], sel3[MOE_MAX_TOPK];
  __shared__ int s_fail;
  const int set = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  const bool has_sg = with_gate != 0;
  const float* src = lg_in + (long)set * (E + 1);
  for (int i = tid; i < E + 1; i += kStackThreads) lg[i] = src[i];
  if (tid == 0) s_fail = 0;
  lds_barrier();
  // the one-barrier form's inputs beside the candidates (E <= 256, k <= 8):
  // the candidates' logits, and the shared-gate logit
  const bool ob = E <= 256 && k <= 8;
  if (ob && tid == 0) cand_lg[64] = has_sg ? lg[E] : 0.0f;
  topk_candidates(lg, E, k, wave, keys, cand, ob ? cand_lg : nullptr);
  lds_barrier();
  if (wave == 0 && rank_candidates(lg, E, k, has_sg, cand, sel, lgsel)) s_fail = 1;
  if (ob && wave == 1) rank_candidates(lg, E, k, has_sg, cand, sel2, lgsel2, cand_lg);
  if (ob && wave < 4) {   // each of these waves finds the experts of ranks wave, wave + 4, ...
    for (int r = wave; r < k; r += 4) {
      bool ok = true;
      const uint32_t id = candidate_of_rank(cand, k, r, ok);
      if (ok && (tid & 63) == 0) sel3[r] = id;
      if (!ok) s_fail = 2;
    }
  }
  lds_barrier();
  // the one-barrier form must agree with the two-barrier one bit for bit
  if (ob && tid < k + 1 && !s_fail) {
    if (tid < k && (sel2[tid] != sel[tid] || sel3[tid] != sel[tid])) s_fail = 3;
    if (__float_as_uint(lgsel2[tid]) != __float_as_uint(lgsel[tid])) s_fail = 3;
  }
  lds_barrier();
  if (wave == 0) routing_weights(k, has_sg, lgsel, sel, reinterpret_cast<double*>(cand));
  lds_barrier();
  for (int s = tid; s < k; s += kStackThreads) {
    ids[(long)set * k + s] = s_fail ? -1 : (int32_t)sel[s];
    wts[(long)set * k + s] = __uint_as_float(sel[k + s]);
  }
  if (tid == 0 && gate) gate[set] = __uint_as_float(sel[2 * k]);
}

int launch_test_stack_select(const float* logits, int n_sets, int E, int k, int with_gate, int32_t* ids, float* wts,
                             float* gate, hipStream_t st) {
  hipLaunchKernelGGL(k_test_stack_select, dim3(n_sets), dim3(kStackThreads), 0, st, logits, E, k, with_gate, ids, wts,
                     gate);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------- host side
int stack_geometry(const moe_layer_desc* d, int G, StackGeom* out) {
  const int st = d->shared_ffn > 0 ? d->shared_type : MOE_TYPE_Q4_K;
  return stack_geometry_core(d->hidden, d->n_experts, d->top_k, d->ffn, d->shared_ffn, d->down_type, st, G, out);
}

void stack_ws_layout(StackGeom* g, size_t base) {
  size_t o = base;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~(size_t)255; return r; };
  g->w_ctrl = take(kStackCtrlBytes);
  g->w_t = take((size_t)kRepT * rep_bytes(g->n_t));
  g->w_lg = take((size_t)kRepLg * rep_bytes(g->n_lg));
  g->w_h = take((size_t)kRepH * rep_bytes(g->n_h));
  g->w_y = take(8u * (size_t)g->n_y);
  g->w_trace = take(8u * kTraceLayers * kTraceSlots + 8u * kTraceLayers * kTraceMaxG * kBlockEvents);
  g->w_end = o;
}

int device_cu_count(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

uint64_t layer_table_hash(const moe_layer_weights* layers, int n) {
  // FNV-1a over 8-byte words of the table
  uint64_t h = 0xcbf29ce484222325ull;
  const size_t words = sizeof(moe_layer_weights) * (size_t)n / 8;
  for (size_t i = 0; i < words; ++i) {
    uint64_t w;
    memcpy(&w, reinterpret_cast<const uint8_t*>(layers) + 8 * i, 8);
    h = (h ^ w) * 0x100000001b3ull;
  }
  return h;
}

// The kernel instances: one per (down type, shared type) with every size from
// the arguments, and the compile-time shapes of kFixShapes with each weight
// variant the workloads use -- shape 1 (hidden 2048, 256 experts, top-8, FFN
// 512, shared 512) with Q4_K or Q5_K down and Q4_K or Q8_0 shared, shape 2
// (hidden 2048, 128 experts, top-8, FFN 768, no shared expert) with Q4_K or
// Q5_K down.  A description takes a compile-time instance when its sizes and
// its whole geometry are that instance's.
struct StackInst {
  int S, DT, ST;
  const void* fn;
  const StackGeom* geom;
};
#define MOE_STACK_INST(S, DT, ST) {S, DT, ST, (const void*)k_stack<DT, ST, S>, &kFixGeom<DT, ST, S>}
static const StackInst kStackInst[] = {
    MOE_STACK_INST(1, MOE_TYPE_Q4_K, MOE_TYPE_Q4_K), MOE_STACK_INST(1, MOE_TYPE_Q5_K, MOE_TYPE_Q8_0),
    MOE_STACK_INST(1, MOE_TYPE_Q4_K, MOE_TYPE_Q8_0), MOE_STACK_INST(1, MOE_TYPE_Q5_K, MOE_TYPE_Q4_K),
    MOE_STACK_INST(2, MOE_TYPE_Q4_K, MOE_TYPE_Q4_K), MOE_STACK_INST(2, MOE_TYPE_Q5_K, MOE_TYPE_Q4_K),
    MOE_STACK_INST(0, MOE_TYPE_Q4_K, MOE_TYPE_Q4_K), MOE_STACK_INST(0, MOE_TYPE_Q5_K, MOE_TYPE_Q8_0),
    MOE_STACK_INST(0, MOE_TYPE_Q4_K, MOE_TYPE_Q8_0), MOE_STACK_INST(0, MOE_TYPE_Q5_K, MOE_TYPE_Q4_K),
};
#undef MOE_STACK_INST

const void* stack_kernel_for(const moe_layer_desc* d, const StackGeom& g, int* shape) {
  const int dt = d->down_type;
  const int st = d->shared_ffn > 0 ? d->shared_type : MOE_TYPE_Q4_K;
  for (const StackInst& in : kStackInst) {
    if (in.DT != dt || in.ST != st) continue;
    if (in.S != 0) {
      const FixShape& f = kFixShapes[in.S];
      const bool sizes = d->hidden == f.H && d->n_experts == f.E && d->top_k == f.k && d->ffn == f.F &&
                         d->shared_ffn == f.Fs;
      if (!sizes || memcmp(&g, in.geom, offsetof(StackGeom, w_ctrl)) != 0) continue;
    }
    if (shape) *shape = in.S;
    return in.fn;
  }
  return nullptr;
}

// whether one workgroup of kernel fn with lds bytes fits a CU (the occupancy
// query, remembered per kernel and size: the answer does not change)
static bool fits_cu(const void* fn, size_t lds) {
  struct Entry {
    const void* fn;
    size_t lds;
    bool fits;
  };
  static std::mutex m;
  static Entry seen[32];
  static int n = 0;
  std::lock_guard<std::mutex> lock(m);
  for (int i = 0; i < n; ++i)
    if (seen[i].fn == fn && seen[i].lds == lds) return seen[i].fits;
  int per_cu = 0;
  const bool fits = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kStackThreads, lds) == hipSuccess &&
                    per_cu >= 1;
  if (!fits) (void)hipGetLastError();
  if (n < 32) seen[n++] = Entry{fn, lds, fits};
  return fits;
}

int launch_stack(const moe_layer_desc* d, int L, const moe_layer_weights* table_dev, const uint32_t* bound,
                 uint64_t table_hash, const moe_stack_io* io, uint8_t* ws, const StackGeom& g, hipStream_t st,
                 bool cooperative) {
  static_assert(sizeof(moe_layer_weights) % 8 == 0, "the table hashes in 8-byte words");
  StackArgs a;
  a.g = g;
  a.layers = table_dev;
  a.bound = bound;
  a.table_hash = table_hash;
  a.input = io->input;
  a.output = io->output;
  a.ids_out = io->ids;
  a.resid_out = io->resid;
  a.routed_out = io->routed;
  a.shared_out = io->shared;
  a.attn = io->attn;
  a.ws = ws;
  a.L = L;
  a.H = d->hidden;
  a.E = d->n_experts;
  a.k = d->top_k;
  a.F = d->ffn;
  a.Fs = d->shared_ffn;
  a.eps = d->eps;
  a.trace_blocks = io->trace ? 1 : 0;
  const void* fn = stack_kernel_for(d, g, nullptr);
  if (!fn) return MOE_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, g.lds) != hipSuccess) return MOE_ERR_HIP;
  void* args[] = {&a};
  // The grid is one workgroup per CU (g.G is the CU count).  A plain launch
  // places all of them at once when the kernel fits a CU and no other kernel
  // holds CUs; the cooperative launch has the runtime guarantee it, at about
  // 18 us more per launch.  A plain launch is used only when the occupancy
  // query confirms that a workgroup fits a CU.
  if (!cooperative && !fits_cu(fn, g.lds)) cooperative = true;
  const hipError_t e = cooperative ? hipLaunchCooperativeKernel(fn, dim3(g.G), dim3(kStackThreads), args, g.lds, st)
                                   : hipLaunchKernel(fn, dim3(g.G), dim3(kStackThreads), args, g.lds, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace moe
