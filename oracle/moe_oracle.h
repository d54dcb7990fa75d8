/*
 * moe_oracle.h -- plain CPU oracle for the batch-1 decode MoE FFN stage.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this library: only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Every real value is computed in fp64 and rounded only at the storage points
 * the method defines (first to fp32, then to the storage type).  Loops are
 * plain and sequential in the order the definitions are written; the only
 * parallelism is an optional OpenMP split over independent output rows, each
 * row computed by one thread in the same order.
 *
 * Sources (the three web pages the method is described on):
 *   [P273] "perf(qwen3.6): fused router GEMV+top-k + folded residual-norm (decode)"
 *   [P239] "perf(qwen3.6): fuse decode kernel launches -- shared-expert + GDN conv/L2-norm"
 *   [P359] "perf(qwen36): Q4_K shared-expert FFN kernels + Q8_0/Q5_K->Q4_K requant of the MoE FFN stage"
 * The pages name the formats and fusions but never write the MoE arithmetic
 * or any block bit layout.  Where they are silent the plainest reading is
 * taken and marked "reading:" next to the code.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF type ids ([P359] Summary, routed down: type id 12 is Q4_K). */
enum { ORC_F32 = 0, ORC_Q8_0 = 8, ORC_Q8_1 = 9, ORC_Q4_K = 12, ORC_Q5_K = 13 };

/* Longest row (elements) the oracle accepts. */
enum { ORC_MAX_K = 32768 };

/* Byte sizes of one block. */
enum { ORC_Q4K_BYTES = 144, ORC_Q5K_BYTES = 176, ORC_Q80_BYTES = 34, ORC_Q81_BYTES = 36 };

/* ---- scalar conversions, written from the IEEE-754 definitions ---- */
uint16_t orc_f32_to_bf16(float x);   /* round to nearest, ties to even */
uint16_t orc_f32_to_f16(float x);    /* round to nearest, ties to even, subnormals kept */
double orc_bf16_to_f64(uint16_t h);
double orc_f16_to_f64(uint16_t h);

/* ---- block decoders (exact in fp64) ---- */
void orc_decode_q4k(const uint8_t* blk, double out[256]);
void orc_decode_q5k(const uint8_t* blk, double out[256]);
void orc_decode_q8_0(const uint8_t* blk, double out[32]);
/* Q8_1 block: out[i] = d*q[i]; *sum_out = the stored s field. */
void orc_decode_q8_1(const uint8_t* blk, double out[32], double* sum_out);
/* Unpacked 6-bit scales/mins of a Q4_K/Q5_K block (sc[8], m[8]). */
void orc_kquant_scales(const uint8_t* blk, int sc[8], int m[8]);

/* ---- Q8_1 activation quantiser, n a multiple of 32 ---- */
void orc_quantize_q8_1(const float* x, int n, uint8_t* out);

/* Load-time requantisation to Q4_K ([P359] Summary), quantiser reading in
 * moe_oracle.c.  orc_quantize_q4k: 256 fp32 values -> one 144-byte block.
 * orc_requant_q4k: n_rows rows of K elements (K % 256 == 0) of src_type
 * (ORC_Q8_0, ORC_Q5_K or ORC_Q4_K) -> n_rows rows of K/256 Q4_K blocks.
 * Returns 0, or -1 for an unsupported type or K. */
void orc_quantize_q4k(const float x[256], uint8_t blk[144]);
int orc_requant_q4k(const uint8_t* src, int src_type, int n_rows, int K, uint8_t* dst);

/* ---- integer sub-block dots: out[j] = sum_{32} qw*qa for each 32-element
 *      sub-block j of one weight row against Q8_1 activations ----
 * type: ORC_Q4_K, ORC_Q5_K or ORC_Q8_0; K multiple of 256 (K-quants) or 32 (Q8_0).
 * Returns 0, or -1 on a bad type/size. */
int orc_subblock_dots(const uint8_t* row, int type, int K, const uint8_t* xq, int32_t* out);

/* ---- one weight row against Q8_1 activations, unrounded fp64 value ---- */
double orc_row_dot(const uint8_t* row, int type, int K, const uint8_t* xq);

/* ---- residual add + RMSNorm + Q8_1 ----
 * routed/shared may be NULL (2-input form: shared == NULL; no previous
 * output: both NULL).  xn, xq may be NULL. */
void orc_add_rmsnorm(const uint16_t* residual, const uint16_t* routed, const uint16_t* shared,
                     const float* w, int H, float eps,
                     uint16_t* out_sum, float* xn, uint8_t* xq);

/* ---- router GEMV: logits[e] = f32(sum_i W[e][i]*xn[i]) ---- */
void orc_router(const float* xn, const float* W, int E, int H, float* logits);

/* ---- top-k by (value descending, index ascending) ---- */
void orc_topk(const float* logits, int E, int k, int32_t* ids);

/* ---- routing weights: softmax over the selected logits ---- */
void orc_softmax_selected(const float* logits, const int32_t* ids, int k, float* w);

/* ---- layer description ---- */
typedef struct {
    int H;            /* hidden size (multiple of 256) */
    int E;            /* routed experts */
    int k;            /* experts per token */
    int F;            /* routed intermediate size (multiple of 32) */
    int Fs;           /* shared intermediate size; 0 = no shared expert */
    int gate_up_type; /* ORC_Q4_K */
    int down_type;    /* ORC_Q4_K or ORC_Q5_K */
    int shared_type;  /* ORC_Q4_K or ORC_Q8_0 (all three shared matrices) */
    int norm;         /* 1: residual-add + RMSNorm; 0: the fp32 input is xn itself */
    float eps;
} orc_desc;

typedef struct {
    const float* norm_w;        /* [H] */
    const float* router_w;      /* [E][H] */
    const float* shared_gate_w; /* [H], only if Fs > 0 */
    const uint8_t* gate;        /* [E][F] rows of K=H */
    const uint8_t* up;          /* [E][F] rows of K=H */
    const uint8_t* down;        /* [E][H] rows of K=pad(F) */
    const uint8_t* sgate;       /* [Fs] rows of K=H */
    const uint8_t* sup;         /* [Fs] rows of K=H */
    const uint8_t* sdown;       /* [H] rows of K=pad(Fs) */
} orc_weights;

/* Everything one layer produces.  Any pointer may be NULL except the ones
 * a later step reads (the oracle keeps its own scratch for those). */
typedef struct {
    uint16_t* out_sum;       /* [H] bf16: the new residual */
    float* xn;               /* [H] */
    uint8_t* xq;             /* [H/32] Q8_1 blocks */
    float* logits;           /* [E] */
    float* z;                /* [1] shared-gate logit */
    float* shared_gate;      /* [1] f32(sigmoid(z)) */
    int32_t* ids;            /* [k] */
    float* weights;          /* [k] */
    float* h;                /* [k][F] */
    float* hs;               /* [Fs] */
    float* y;                /* [k][H] */
    float* ys;               /* [H] */
    uint16_t* routed;        /* [H] bf16 */
    uint16_t* shared;        /* [H] bf16 */
    double* routed_exact;    /* [H] fp64 value before the final roundings */
    double* shared_exact;    /* [H] */
} orc_layer_out;

/* Row byte size of a weight row of K elements of the given type (0 on error). */
long orc_row_bytes(int type, int K);
/* K of the down rows: F rounded up to a whole superblock for K-quants. */
int orc_pad_k(int type, int K);

/* Router + top-k + weights + shared gate for one token (steps a2, a3). */
void orc_router_topk(const orc_desc* d, const orc_weights* w, const float* xn,
                     float* logits, float* z, int32_t* ids, float* weights, float* shared_gate);

/* Expert FFN for one token (steps a4, a5, a6) given xq, ids, weights, gate. */
void orc_expert_ffn(const orc_desc* d, const orc_weights* w, const uint8_t* xq,
                    const int32_t* ids, const float* weights, float shared_gate,
                    orc_layer_out* o);

/* One full layer (a1..a6) for one token.
 * norm=1: residual (bf16) + routed_prev/shared_prev (bf16, nullable) are folded and normed.
 * norm=0: x (fp32 [H]) is used directly as xn. */
int orc_moe_layer(const orc_desc* d, const orc_weights* w,
                  const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                  const float* x, orc_layer_out* o);

/* orc_moe_layer with the selection given: ids_in[0..k) (distinct, in
 * [0, E)) are the experts in slot order and the routing weights are the
 * softmax over their logits; everything else as defined.  For chained
 * comparisons that hit a near tie (two logits closer than the other side's
 * rounding can separate): the oracle continues with the other side's
 * selection.  Returns -1 on an invalid selection. */
int orc_moe_layer_sel(const orc_desc* d, const orc_weights* w,
                      const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                      const float* x, const int32_t* ids_in, orc_layer_out* o);

/* L-layer stack for one token: res_0 = input, previous outputs zero at layer 0;
 * layer l folds the previous layer's routed/shared into its norm; the result
 * is the fold a virtual layer L would do.  With attn_per_layer ([L][H] bf16,
 * an attention block's output per layer) layer l first folds the previous
 * outputs, u1 = bf16(res + bf16(routed + shared)), then normalises
 * u2 = bf16(u1 + attn_l) (which becomes its out_sum).  Per-layer outputs are
 * optional (arrays of L entries each, or NULL). */
int orc_moe_stack(const orc_desc* d, const orc_weights* layers, int L,
                  const uint16_t* input, const uint16_t* attn_per_layer, uint16_t* output,
                  int32_t* ids_per_layer /* [L][k] or NULL */,
                  uint16_t* routed_per_layer /* [L][H] or NULL */,
                  uint16_t* shared_per_layer /* [L][H] or NULL */,
                  uint16_t* resid_per_layer /* [L][H] or NULL: out_sum of each layer */);

/* ---- several tokens at once, grouped by expert ----
 * Per token: a1..a3.  The tokens whose ids contain expert e form its group
 * and the shared expert is one group of all n_tok tokens; each member of a
 * group gets exactly the batch-1 integer path's result (a4..a6), so nothing
 * depends on the batch.  Arrays are [n_tok][...] versions of the
 * single-token ones; every output pointer may be NULL. */
typedef struct {
    uint16_t* out_sum;       /* [n][H] */
    float* xn;               /* [n][H] */
    uint8_t* xq;             /* [n][H/32] Q8_1 */
    int32_t* ids;            /* [n][k] */
    float* weights;          /* [n][k] */
    float* shared_gate;      /* [n] */
    int32_t* group_size;     /* [n][k]: tokens in the group of that slot's expert */
    float* h;                /* [n][k][F] */
    float* hs;               /* [n][Fs] */
    float* y;                /* [n][k][H] */
    float* ys;               /* [n][H] */
    uint16_t* routed;        /* [n][H] */
    uint16_t* shared;        /* [n][H] */
    double* routed_exact;    /* [n][H] */
    double* shared_exact;    /* [n][H] */
} orc_batch_out;

int orc_moe_layer_batch(const orc_desc* d, const orc_weights* w, int n_tok,
                        const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                        const float* x, orc_batch_out* o);

/* Threads the OpenMP loops use (1 when built without OpenMP). */
int orc_num_threads(void);
/* OpenMP threads for the calls that follow (n > 0) */
void orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
