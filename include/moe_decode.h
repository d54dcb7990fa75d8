/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) batch-1 decode MoE FFN stage.
 *
 * One MoE layer of a Qwen3.6-35B-A3B-shaped decoder, per token:
 *   a1  residual add folded into RMSNorm, Q8_1 of the normed vector
 *   a2  fp32 router GEMV over the experts (+ the shared-expert gate row)
 *   a3  top-k by (value descending, index ascending) + softmax over the selected logits
 *   a4  routed gate/up GEMVs (Q4_K x Q8_1) + SwiGLU + Q8_1 of the product
 *   a5  routed down GEMV (Q4_K or Q5_K x Q8_1) + weighted combine
 *   a6  sigmoid-gated shared expert (Q4_K or Q8_0 x Q8_1)
 * and the 40-layer stack of such layers without launch gaps (a7).
 *
 * Source pages (cited by short name in the comments below):
 *   [P273] "perf(qwen3.6): fused router GEMV+top-k + folded residual-norm (decode)"
 *   [P239] "perf(qwen3.6): fuse decode kernel launches -- shared-expert + GDN conv/L2-norm"
 *   [P359] "perf(qwen36): Q4_K shared-expert FFN kernels + Q8_0/Q5_K->Q4_K requant of the MoE FFN stage"
 *
 * Conventions (every entry point):
 *  - Pointers named "device" are HIP device pointers; descriptor structs and
 *    the layer-weights array of moe_stack_bind live in host memory and are
 *    read only during the call.
 *  - The caller allocates and owns every buffer, the workspace included.  The
 *    library keeps no mutable state between calls apart from what the caller's
 *    workspace holds and the host-side record of bound stacks (moe_stack_bind);
 *    it never allocates device memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  No call synchronises the host, reads device data back or
 *    issues a memset, so every call can be captured in a HIP graph.
 *  - Every argument is validated on the host before anything is enqueued.  An
 *    invalid argument returns a negative MOE_ERR_* code and enqueues nothing.
 *    A launch failure returns MOE_ERR_HIP.  There is no fallback path: an
 *    unsupported shape or type is an error.
 *  - bf16 values are passed as uint16_t bit patterns.  Quantised blocks are
 *    bytes in the GGUF layouts (see MOE_TYPE_*), rows of a matrix back to
 *    back, experts of a stacked matrix back to back; every weight pointer must
 *    be 16-byte aligned and every row a whole number of blocks.
 *  - Calls that share one workspace must not overlap in time (they are
 *    ordered when issued on one stream).
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)          /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)         /* a size is out of range or not a whole number of blocks */
#define MOE_ERR_TYPE (-3)          /* unsupported block type for that operand */
#define MOE_ERR_ALIGN (-4)         /* a pointer is not aligned as required */
#define MOE_ERR_WORKSPACE (-5)     /* workspace NULL or smaller than moe_workspace_size() */
#define MOE_ERR_HIP (-6)           /* a HIP launch or runtime call failed */
#define MOE_ERR_UNSUPPORTED (-7)   /* valid arguments, combination not implemented */
#define MOE_ERR_NOT_BOUND (-8)     /* moe_decode_stack before moe_stack_bind */

/* ---- block types: GGUF type ids ([P359] Summary: type id 12 is Q4_K) ----
 *  Q4_K 144 B / 256 elements: d f16 | dmin f16 | scales[12] (6-bit scale and min of
 *       8 sub-blocks of 32) | qs[128] (4-bit codes); element = d*sc*q - dmin*m.
 *  Q5_K 176 B / 256 elements: as Q4_K with qh[32] (fifth code bit) before qs[128].
 *  Q8_0  34 B / 32 elements: d f16 | q int8[32]  ([P359] Summary: 34 bytes per block).
 *  Q8_1  36 B / 32 elements: d f16 | s f16 | q int8[32], s = d * sum(q) (activations). */
#define MOE_TYPE_F32 0
#define MOE_TYPE_Q8_0 8
#define MOE_TYPE_Q8_1 9
#define MOE_TYPE_Q4_K 12
#define MOE_TYPE_Q5_K 13

/* ---- limits ---- */
#define MOE_MAX_HIDDEN 8192
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_MAX_FFN 4096
#define MOE_MAX_LAYERS 256
#define MOE_MAX_BATCH 64      /* tokens of one grouped (batch > 1) call */
#define MOE_MAX_GROUP_MIN 16  /* largest group size threshold */

typedef struct moe_layer_desc {
    int hidden;        /* H: multiple of 256, <= MOE_MAX_HIDDEN */
    int n_experts;     /* E: 1..MOE_MAX_EXPERTS */
    int top_k;         /* k: 1..min(E, MOE_MAX_TOPK) */
    int ffn;           /* F: routed intermediate size, multiple of 32, <= MOE_MAX_FFN */
    int shared_ffn;    /* Fs: 0 = no shared expert, else multiple of 32, <= MOE_MAX_FFN */
    int gate_up_type;  /* MOE_TYPE_Q4_K */
    int down_type;     /* MOE_TYPE_Q4_K or MOE_TYPE_Q5_K */
    int shared_type;   /* MOE_TYPE_Q4_K or MOE_TYPE_Q8_0 (all three shared matrices) */
    int norm;          /* 1: the layer input is folded and RMS-normed (a1);
                          0: the layer input is an fp32 vector used as the normed vector */
    float eps;         /* RMSNorm epsilon */
} moe_layer_desc;

/* Device pointers of one layer's weights.  Down rows have K = F rounded up to a
 * whole block of down_type (the padding is part of every row). */
typedef struct moe_layer_weights {
    const float* norm_w;        /* [H] fp32 (norm = 1) */
    const float* router_w;      /* [E][H] fp32 */
    const float* shared_gate_w; /* [H] fp32 (Fs > 0) */
    const void* gate;           /* [E][F] rows of H, gate_up_type */
    const void* up;             /* [E][F] rows of H, gate_up_type */
    const void* down;           /* [E][H] rows of pad(F), down_type */
    const void* shared_gate;    /* [Fs] rows of H, shared_type (Fs > 0) */
    const void* shared_up;      /* [Fs] rows of H, shared_type (Fs > 0) */
    const void* shared_down;    /* [H] rows of pad(Fs), shared_type (Fs > 0) */
} moe_layer_weights;

/* Per-call device buffers of moe_decode_layer (one token). */
typedef struct moe_layer_io {
    const uint16_t* residual;   /* [H] bf16 residual stream (norm = 1) */
    const uint16_t* routed_in;  /* [H] bf16 previous layer's routed output, or NULL (= 0) */
    const uint16_t* shared_in;  /* [H] bf16 previous layer's shared output, or NULL (2-input form) */
    const float* x;             /* [H] fp32 input (norm = 0) */
    uint16_t* out_sum;          /* [H] bf16 new residual = bf16(residual + bf16(routed_in + shared_in)) (norm = 1);
                                   may be the residual buffer itself (updated in place) */
    uint16_t* routed_out;       /* [H] bf16 */
    uint16_t* shared_out;       /* [H] bf16 (Fs > 0) */
    /* optional intermediates, NULL = not written */
    float* xn;                  /* [H] fp32 normed vector */
    void* xq;                   /* [H/32] Q8_1 blocks */
    float* logits;              /* [E] fp32 */
    int32_t* ids;               /* [k] selected experts, slot order */
    float* weights;             /* [k] routing weights */
    float* shared_gate;         /* [1] sigmoid of the shared-gate logit */
    float* h;                   /* [k][F] SwiGLU outputs */
    float* hs;                  /* [Fs] shared SwiGLU output */
} moe_layer_io;

/* ------------------------------------------------------------------------
 * Workspace.  moe_workspace_size gives the bytes one token of `desc` needs
 * (n_layers >= 1: the bound stack of moe_stack_bind included).  The
 * workspace must be 256-byte aligned and initialised once by
 * moe_workspace_init before its first use; the library returns every
 * counter in it to its initial value, so graph replays need no reset.
 * ---------------------------------------------------------------------- */
size_t moe_workspace_size(const moe_layer_desc* desc, int n_layers);
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Human-readable text of a status code (static storage). */
const char* moe_status_string(int status);

/* ------------------------------------------------------------------------
 * a1: residual add folded into RMSNorm ([P273] Summary item 2: the
 * routed+shared residual add is folded into a 3-input add_rmsnorm3 that is
 * bit-identical to the add followed by the 2-input norm; [P273] Relation to
 * open PRs: add_rmsnorm3_q8 keeps the reload of the stored sum).
 *   t = shared ? bf16(routed + shared) : (routed ? routed : 0)
 *   u = bf16(residual + t)              -> out_sum (bf16), the new residual
 *   xn = u * (1/sqrt(mean(u^2) + eps)) * norm_w   (fp32; mean over H)
 *   xq = Q8_1(xn): per 32 values d = amax/127, codes rounded half away from
 *        zero, d and s = d*sum(q) stored as fp16; an all-zero block is zero.
 * residual: [n_tok][H] bf16; routed, shared: [n_tok][H] bf16 or NULL;
 * norm_w [H] fp32; out_sum [n_tok][H] bf16; xn [n_tok][H] fp32 or NULL;
 * xq [n_tok][H/32] Q8_1 or NULL.  All device.  n_tok 1..4096.
 * ---------------------------------------------------------------------- */
int add_rmsnorm3(const uint16_t* residual, const uint16_t* routed, const uint16_t* shared,
                 const float* norm_w, int hidden, int n_tok, float eps,
                 uint16_t* out_sum, float* xn, void* xq, void* stream);

/* ------------------------------------------------------------------------
 * The post-attention add-norm ([P273] Relation to open PRs: add_rmsnorm2_q8,
 * after the attention block; the 3-input fold precedes the attention):
 *   u = bf16(residual + attn_out) -> out_sum; xn = u * (1/sqrt(mean(u^2) + eps))
 *   * norm_w; xq = Q8_1(xn).  The 2-input form of add_rmsnorm3, with the same
 * layouts, limits and error codes.
 * ---------------------------------------------------------------------- */
int add_rmsnorm2_q8(const uint16_t* residual, const uint16_t* attn_out, const float* norm_w, int hidden, int n_tok,
                    float eps, uint16_t* out_sum, float* xn, void* xq, void* stream);

/* ------------------------------------------------------------------------
 * a2 + a3: router GEMV + in-kernel top-k + routing weights ([P273] Summary
 * item 1: the split-K fp32 GEMV's logits and the top-k select in one kernel,
 * selection by value descending with ties to the lower expert index, the
 * last workgroup selecting after a grid-completion handshake that returns to
 * zero by itself).  Routing weights: softmax over the k selected logits.
 *   logits[e] = sum_i W[e][i] * xn[i]           (fp32 result)
 *   ids       = top-k of logits                 (slot order = rank order)
 *   weights   = softmax(logits[ids])
 *   shared_gate_out = sigmoid(sum_i g[i] * xn[i]) if w_shared_gate != NULL
 * xn [n_tok][H] fp32; w_router [E][H] fp32; w_shared_gate [H] fp32 or NULL;
 * logits [n_tok][E] or NULL; ids [n_tok][k] int32; weights [n_tok][k] fp32;
 * shared_gate_out [n_tok] or NULL.  All device.  Needs the workspace for the
 * handshake counter and, when logits == NULL, the logit buffer.
 * ---------------------------------------------------------------------- */
int router_topk(const float* xn, const float* w_router, const float* w_shared_gate,
                int n_tok, int hidden, int n_experts, int top_k,
                float* logits, int32_t* ids, float* weights, float* shared_gate_out,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * a4 + a5 (+ a6): expert FFN for one token ([P359] Summary: Q8_1 activations
 * -> gate/up with SiLU -> Q8_1 of the product -> down, with an int8 dot of the
 * weight codes against the Q8_1 codes; [P239] Summary item 1: gate and up of
 * the shared expert in one pass over the activations).
 *   for slot s (expert e = ids[s]): g = G_e xq, u = U_e xq (fp32 rows),
 *     h = silu(g) * u (fp32), y_e = D_e Q8_1(h) (fp32 rows; Q8_1 padding blocks
 *     of zeros up to the down row length)
 *   routed_out = bf16(sum_s weights[s] * y_e)       (slot order)
 *   shared (desc->shared_ffn > 0): same FFN with the shared matrices,
 *     shared_out = bf16(shared_gate[0] * ys)
 * xq [H/32] Q8_1; ids [k]; weights [k]; shared_gate [1] fp32 (device, read
 * when Fs > 0); routed_out, shared_out [H] bf16; h [k][F], hs [Fs] fp32 or
 * NULL.  All device.  n_tok must be 1.  An id outside [0, E) is not read
 * through: its slot's h and the routed/shared outputs become NaN.
 * ---------------------------------------------------------------------- */
int expert_ffn_q4k(const moe_layer_desc* desc, const moe_layer_weights* w,
                   const void* xq, const int32_t* ids, const float* weights, const float* shared_gate,
                   int n_tok, uint16_t* routed_out, uint16_t* shared_out, float* h, float* hs,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * a1..a6: one MoE layer for one token, composed on the device (no host
 * synchronisation, ids never leave the device).
 * ---------------------------------------------------------------------- */
int moe_decode_layer(const moe_layer_desc* desc, const moe_layer_weights* w,
                     const moe_layer_io* io, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_decode_layer without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation).  Same arguments, kernels and results as
 * moe_decode_layer; the layer's intermediates (router counters, xn, xq,
 * logits, ids, weights, gate, h, hs) live in a static device array of the
 * library of 256 KiB, one per GPU, held until the process ends.  A shape whose
 * intermediates need more returns MOE_ERR_WORKSPACE and enqueues nothing
 * (every shape of up to 8 selected experts of FFN 2048 at hidden 8192 fits).
 * No allocation happens: the first call on a device looks the array up and
 * queues the clearing of its router counters on `stream`; every completed
 * call leaves them at zero again.  All calls on one GPU share the array and
 * see what the last call left there: calls that may overlap in time on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * ---------------------------------------------------------------------- */
int moe_decode_layer_noalloc(const moe_layer_desc* desc, const moe_layer_weights* w,
                             const moe_layer_io* io, void* stream);

/* ------------------------------------------------------------------------
 * a8: several tokens at once, experts grouped by the tokens that selected
 * them (the pages describe batch 1 only; this is the batch > 1 reading).
 * Per token the norm, router, top-k and weights are the batch-1 steps.  The
 * group of expert e is the set of tokens whose ids contain e (token order).
 * A group of >= group_min tokens reads the expert's rows once and runs on the
 * int8 matrix cores: the weight codes against the tokens' Q8_1 codes (xq for
 * gate/up, Q8_1 of h for down), each 32-element block's exact integer dot
 * scaled and summed in fp64 as the batch-1 integer path does.  A smaller
 * group runs that integer path for all its tokens at once.  Either way each
 * token's h, y, routed_out and shared_out are bit-identical to what the
 * batch-1 calls give it (the grouped path is batch-invariant; group_min only
 * moves work between the two code paths).  The matrix-core tile holds 16
 * tokens, so a group of fewer than 9 leaves most of it empty: on one layer
 * of the 40-layer shape group_min 9 was the fastest at batch 8 and 32.  The shared expert is one group of
 * all n_tok tokens.  routed_out[t] = bf16(sum_s weights[t][s] * y[t][s]) in
 * slot order; shared_out[t] = bf16(shared_gate[t] * ys[t]).  When a call has
 * groups of both kinds, the matrix-core groups run on a second stream of the
 * device (made by the first such call that is not under graph capture; a
 * captured call before then keeps to `stream`), forked from `stream` after
 * the grouping and joined back before the combine, so every kernel of the
 * call is ordered before later work on `stream`.  Calls from several host
 * threads share that stream and serialise the fork and join under a lock.
 *
 * moe_batch_workspace_size: bytes of workspace for n_tok tokens (0 on a bad
 * description or n_tok outside 1..MOE_MAX_BATCH).
 *
 * expert_ffn_grouped (a4..a6 + a8): xn [n_tok][H] fp32 (16-byte aligned);
 * xq [n_tok][H/32] Q8_1; ids, weights [n_tok][k]; shared_gate [n_tok] (read
 * when Fs > 0); routed_out, shared_out [n_tok][H] bf16; h [n_tok][k][F] and
 * hs [n_tok][Fs] fp32 or NULL (then kept in the workspace).  group_min in
 * 1..MOE_MAX_GROUP_MIN.  All device.  An id outside [0, E) is never read
 * through: every output of the call becomes NaN.
 *
 * moe_decode_layer_batch (a1..a6 + a8): io fields hold [n_tok][...] arrays
 * (residual, routed_in, shared_in, x, out_sum, routed_out, shared_out, xn,
 * xq, logits, ids, weights, shared_gate); optional ones may be NULL; io->h and
 * io->hs, when given, are [n_tok][k][F] and [n_tok][Fs].
 * ---------------------------------------------------------------------- */
size_t moe_batch_workspace_size(const moe_layer_desc* desc, int n_tok);
int expert_ffn_grouped(const moe_layer_desc* desc, const moe_layer_weights* w, const float* xn, const void* xq,
                       const int32_t* ids, const float* weights, const float* shared_gate, int n_tok,
                       int group_min, uint16_t* routed_out, uint16_t* shared_out, float* h, float* hs,
                       void* ws, size_t ws_bytes, void* stream);
int moe_decode_layer_batch(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io,
                           int n_tok, int group_min, void* ws, size_t ws_bytes, void* stream);

/* moe_tune_group_min: the group_min for this description, batch size and
 * device, chosen by measurement ([P273] "Relation to open PRs": the router's
 * split factor and the F = 512 dispatch were retuned per shape by measuring
 * them; here the threshold between the two grouped code paths is).  Each of
 * the n_candidates values (each 1..MOE_MAX_GROUP_MIN) runs
 * moe_decode_layer_batch on `io` once to warm up and then `reps` times
 * (1..100), timed with events on `stream`; *best receives the candidate with
 * the lowest mean time, *best_us that mean (may be NULL).  group_min changes
 * no bit of any output, so the choice is a speed setting only.  io's outputs
 * are overwritten.  The call synchronises `stream`: it returns
 * MOE_ERR_UNSUPPORTED under graph capture and enqueues nothing then.  Other
 * errors as for moe_decode_layer_batch; candidates and best are host memory.
 */
int moe_tune_group_min(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io, int n_tok,
                       const int* candidates, int n_candidates, int reps, void* ws, size_t ws_bytes, void* stream,
                       int* best, float* best_us);

/* ------------------------------------------------------------------------
 * a7: the L-layer stack for one token ([P239] Summary: decode is graph- and
 * launch-bound; [P273] Summary item 2: one graph node per layer matters).
 *   res_0 = input, previous outputs 0; layer l folds the previous layer's
 *   routed/shared outputs into its norm; output = bf16(res_L + t_L) with
 *   t_L = bf16(routed_{L-1} + shared_{L-1}) (the fold the next norm would do).
 * layers: host array of n_layers structs of device pointers.
 *
 * mode MOE_STACK_KERNELS enqueues 4 kernels per layer plus the final fold on
 * `stream` (capture them in a HIP graph to remove launch overhead).
 * MOE_STACK_PERSISTENT runs every layer in one launch of one workgroup per
 * CU, whose workgroups exchange data through bounded waits and so must all
 * be resident at once.  It is a plain launch: on a device that runs nothing
 * else, every CU takes one of its workgroups.  When other streams' kernels
 * hold CUs, a workgroup may start only after others have waited past their
 * bound, and the launch then stops with status 1 (moe_stack_status_offset).
 * MOE_STACK_COOPERATIVE is the same kernel in a cooperative launch, for which
 * the runtime places the whole grid at once (about 18 us more per token on
 * one MI355X).  Both need a prior moe_stack_bind of the same layers into
 * the same workspace, else it returns MOE_ERR_NOT_BOUND and enqueues nothing;
 * bind copies the pointer table to the device, clears the stack's exchange
 * buffers and synchronises `stream` once (do not call it during graph
 * capture).  The library keeps a host-side record of the workspaces that
 * hold a bound stack (workspace address, size, layer count and a hash of the
 * whole pointer table), the only state it keeps outside the caller's
 * buffers; moe_workspace_init of an overlapping range drops the record.  Each
 * launch also checks on the device that the table bound in the workspace
 * hashes to the caller's (see moe_stack_status_offset for the outcome).
 * MOE_STACK_AUTO uses the persistent kernel when the layers are bound in this
 * workspace and the shape fits in LDS, else the per-layer kernels.
 * desc->norm must be 1.
 * ---------------------------------------------------------------------- */
#define MOE_STACK_AUTO 0
#define MOE_STACK_KERNELS 1
#define MOE_STACK_PERSISTENT 2
#define MOE_STACK_COOPERATIVE 3

/* Device buffers of one moe_decode_stack call.  The per-layer outputs are
 * optional (NULL = not written). */
typedef struct moe_stack_io {
    const uint16_t* input;   /* [H] bf16 token input (the residual of layer 0) */
    uint16_t* output;        /* [H] bf16 stack output */
    int32_t* ids;            /* [L][k] experts selected per layer, slot order */
    uint16_t* resid;         /* [L][H] bf16 out_sum of each layer (the residual after its fold) */
    uint16_t* routed;        /* [L][H] bf16 routed output of each layer */
    uint16_t* shared;        /* [L][H] bf16 shared output of each layer (Fs > 0) */
    const uint16_t* attn;    /* [L][H] bf16 attention-block output per layer, or NULL: layer l then
                                folds the previous outputs, u1 = bf16(res + t), and normalises
                                u2 = bf16(u1 + attn_l), its out_sum (the add_rmsnorm2_q8 step) */
    int trace;               /* persistent mode: 1 = every workgroup stamps its phase events
                                (moe_stack_trace_offset); 0 = only workgroup 0's phase table */
} moe_stack_io;

int moe_stack_bind(const moe_layer_desc* desc, const moe_layer_weights* layers, int n_layers,
                   void* ws, size_t ws_bytes, void* stream);
int moe_decode_stack(const moe_layer_desc* desc, const moe_layer_weights* layers, int n_layers,
                     const moe_stack_io* io, int mode, void* ws, size_t ws_bytes, void* stream);

/* Byte offset, in a workspace sized for (desc, n_layers), of a uint32 status
 * word of the persistent stack: 0 while every launch completed; 1 after a
 * launch stopped (a bounded wait ran out, or a selection came out
 * incomplete); 2 after a launch found that the table
 * bound in the workspace is not the caller's; 3 after a launch of an instance
 * that pairs each workgroup with the accelerator die (XCC) it runs on read a
 * die number outside 0..7 (it stops before any exchange).  After a stop (1)
 * the next uint32 word holds (layer << 8) | check, the check being 1 the previous
 * layer's outputs, 2 the logits, 3 an incomplete selection, 4 the shared
 * expert's h, 5 the routed h, 6 the down rows' values, 7 the last layer's
 * outputs for the final fold.  A launch that starts with a
 * nonzero word does no work: it sets its output to NaN and leaves the word as
 * it is.  So after a stopped or refused launch every later persistent launch
 * on that workspace is refused too (their outputs are NaN), until
 * moe_stack_bind (or moe_workspace_init) clears the word.  Returns 0 if the
 * shape has no persistent stack. */
size_t moe_stack_status_offset(const moe_layer_desc* desc, int n_layers);

/* Which persistent-kernel instance the current device would run for desc:
 * 0 = the instance that takes every size at run time, n >= 1 = a compile-time
 * shape (hidden 2048 with 256 experts top-8, FFN 512, shared 512 = 1; with
 * 128 experts top-8, FFN 768, no shared expert = 2), each for Q4_K or Q5_K
 * down and Q4_K or Q8_0 shared matrices; -1 = no persistent kernel for desc
 * (the per-layer kernels then run).  Queries the device's compute-unit
 * count; enqueues nothing. */
int moe_stack_kernel_shape(const moe_layer_desc* desc);

/* Byte offset, in the same workspace, of the persistent stack's phase
 * timestamps: uint64 [64 layers][12 slots], written by the last launch for each
 * of its first 64 layers.  Slots 0..9: the 100 MHz device wall clock seen by
 * workgroup 0 at its phase boundaries (0 layer start, 1 previous outputs
 * received, 2 fixed weights landed, 3 router rows done, 4 experts selected,
 * 5 routed gate/up rows landed, 6 gate/up done, 7 every h quantised, 8 down rows
 * landed, 9 layer done); slots 10/11: its shader cycle counter at the layer's
 * start and end.  Right after them, uint64 [64 layers][256 workgroups][16
 * events]: the wall clock of every workgroup at its own events (0 layer start,
 * 1 previous outputs received, 2 fixed weights landed, 3 router rows stored,
 * 4 shared h stored, 5 experts known, 6 routed gate/up rows landed, 7 routed h
 * stored, 8 down inputs quantised, 9 down rows landed, 10 layer outputs stored,
 * 11 input normalised, 12 input quantised, 13 logits received, 14 every h
 * received, 15 down rows queued), written only by launches with io->trace = 1.
 * Returns 0 if the shape has no persistent stack. */
size_t moe_stack_trace_offset(const moe_layer_desc* desc, int n_layers);

/* ------------------------------------------------------------------------
 * Test export: the integer sub-block dots of weight rows against Q8_1
 * activations, the bit-exact quantity of the int8 dot path ([P359] Summary).
 * rows: [n_rows] rows of K elements of `type` (Q4_K, Q5_K or Q8_0); xq [K/32]
 * Q8_1; out [n_rows][K/32] int32: out[r][j] = sum over the 32 elements of
 * sub-block j of weight code * activation code.  All device.
 * ---------------------------------------------------------------------- */
int moe_test_subblock_dots(const void* rows, int type, int K, int n_rows, const void* xq,
                           int32_t* out, void* stream);

/* ------------------------------------------------------------------------
 * Load-time requantisation to Q4_K ([P359] Summary: the shared expert's
 * Q8_0 matrices and the routed down projection's Q5_K matrices are
 * re-quantised to Q4_K once at model load, so the per-token reads shrink).
 * The pages do not give the quantiser; this one, per 256-value superblock,
 * decodes the source values exactly and rounds them once to fp32, then:
 *   per 32-value sub-block lo = min(0, min x), hi = max x,
 *     step = (hi - lo)/15, off = -lo;
 *   d = f16(max step / 63), dmin = f16(max off / 63);
 *   sc, m = nearest integer (ties to even) to step/d, off/dmin, in 0..63
 *     (0 when d, dmin = 0);
 *   q = nearest integer to (x + dmin*m)/(d*sc) in 0..15 (0 when d*sc = 0);
 * each step one fp32 operation rounded to nearest, written in the GGUF Q4_K
 * layout.  src: n_rows rows of K elements (K % 256 == 0) of src_type
 * (MOE_TYPE_Q8_0, MOE_TYPE_Q5_K or MOE_TYPE_Q4_K), 16-byte aligned; dst:
 * n_rows rows of K/256 Q4_K blocks (144 B), 2-byte aligned; the two must not
 * overlap.  All device, asynchronous on stream.  Source values that are not
 * finite give unspecified blocks.
 * ---------------------------------------------------------------------- */
int moe_requant_q4k(const void* src, int src_type, int n_rows, int K, void* dst, void* stream);

/* ------------------------------------------------------------------------
 * Measurement helper: a plain streaming read of `bytes` (a multiple of 16)
 * from device memory p (16-byte aligned) by `blocks` workgroups of 256
 * threads, each lane folding its 16-byte words; out [blocks] uint32 (device)
 * receives one fold per workgroup.  It gives the achievable HBM read rate the
 * stage's weight streaming is compared with (not a step of the method).
 * ---------------------------------------------------------------------- */
int moe_stream_read(const void* p, size_t bytes, uint32_t* out, int blocks, void* stream);

/* ------------------------------------------------------------------------
 * Test export: the persistent kernel's Q8_1 quantiser ([P359] Summary: the
 * activations and the gate/up product are quantised to Q8_1 blocks of 32
 * before the int8 dots), run over n/32 independent blocks.  Same definition
 * as in add_rmsnorm3: d = amax/127, codes rounded half away from zero, d and
 * s = d*sum(q) as fp16, an all-zero block all zero.  The codes of a block
 * holding a NaN or an infinity, or whose d or 1/d leaves the fp32 range,
 * are unspecified.
 * x [n] fp32 (16-byte aligned), n a multiple of 32 up to 2^26; xq [n/32]
 * Q8_1 blocks of 36 bytes (d, s, 32 codes).  All device.
 * ---------------------------------------------------------------------- */
int moe_test_quantize_q81(const float* x, int n, void* xq, void* stream);

/* ------------------------------------------------------------------------
 * Test export: the persistent stack kernel's own expert selection ([P273]
 * Summary item 1: top-k by value with ties to the lower expert index, checked
 * over tie-heavy cases), run on n_sets independent logit sets, one workgroup
 * each, with the same device functions and barriers a layer uses.
 * logits [n_sets][E+1] fp32 (element E of a set is the shared-gate logit,
 * read when with_gate != 0); ids [n_sets][k] int32 (slot order; -1 for every
 * slot of a set where fewer than k candidates ranked, which valid input never
 * gives); weights [n_sets][k] fp32 = softmax over the selected logits;
 * gate [n_sets] fp32 = sigmoid of the shared-gate logit (with_gate != 0).
 * NaN ranks as -inf and -0 equals +0.  All device.  E 1..MOE_MAX_EXPERTS,
 * k 1..min(E, MOE_MAX_TOPK), n_sets 1..65535.
 * ---------------------------------------------------------------------- */
int moe_test_stack_select(const float* logits, int n_sets, int n_experts, int top_k, int with_gate, int32_t* ids,
                          float* weights, float* gate, void* stream);

#ifdef __cplusplus
}
#endif
#endif
