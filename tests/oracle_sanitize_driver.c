/*
 * oracle_sanitize_driver.c -- runs the CPU oracle, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer, over inputs a test wrote to a directory, and
 * writes the results back there for comparison with the normal build.
 *
 * Test infrastructure only (compiled and run by tests/test_oracle_sanitize.py).
 *
 * Inputs (raw little-endian files in argv[1]):
 *   desc.i32      H E k F Fs gate_up_type down_type shared_type L n_tok n_sets
 *   norm_w.f32    [L][H]           router.f32 [L][E][H]    sgw.f32 [L][H]
 *   gate.u8 up.u8 down.u8 sgate.u8 sup.u8 sdown.u8   (L layers back to back)
 *   input.u16     [H]              batch_res.u16 batch_rp.u16 batch_sp.u16 [n_tok][H]
 *   logits.f32    [n_sets][E]      q81_x.f32 [n] (n % 32 == 0)
 *   attn.u16      [L][H]           (an attention block's output per layer)
 * Outputs: stack_out.u16 [H], stack_ids.i32 [L][k], stack_attn_out.u16 [H], batch_routed.u16
 * [n_tok][H], batch_shared.u16 [n_tok][H], topk.i32 [n_sets][k], q81.u8,
 * requant_down.u8, requant_sgate.u8.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/moe_oracle.h"

static const char* g_dir;

static void* read_file(const char* name, size_t* size)
{
    char path[4096];
    snprintf(path, sizeof(path), "%s/%s", g_dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(2);
    }
    fseek(f, 0, SEEK_END);
    long n = ftell(f);
    fseek(f, 0, SEEK_SET);
    void* p = malloc(n > 0 ? (size_t)n : 1);
    if (!p || fread(p, 1, (size_t)n, f) != (size_t)n) {
        fprintf(stderr, "cannot read %s\n", path);
        exit(2);
    }
    fclose(f);
    if (size) *size = (size_t)n;
    return p;
}

static void write_file(const char* name, const void* p, size_t n)
{
    char path[4096];
    snprintf(path, sizeof(path), "%s/%s", g_dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, n, f) != n) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(2);
    }
    fclose(f);
}

int main(int argc, char** argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s <dir>\n", argv[0]);
        return 2;
    }
    g_dir = argv[1];
    int32_t* dv = (int32_t*)read_file("desc.i32", NULL);
    orc_desc d = {dv[0], dv[1], dv[2], dv[3], dv[4], dv[5], dv[6], dv[7], 1, 1e-6f};
    const int L = dv[8], n_tok = dv[9], n_sets = dv[10];
    const int H = d.H, E = d.E, k = d.k, F = d.F, Fs = d.Fs;
    const long rb_gu = orc_row_bytes(d.gate_up_type, H);
    const int Kp = orc_pad_k(d.down_type, F), Kps = orc_pad_k(d.shared_type, Fs);
    const long rb_dn = orc_row_bytes(d.down_type, Kp);
    const long rb_s = orc_row_bytes(d.shared_type, H), rb_sd = orc_row_bytes(d.shared_type, Kps);
    float* norm_w = (float*)read_file("norm_w.f32", NULL);
    float* router = (float*)read_file("router.f32", NULL);
    float* sgw = (float*)read_file("sgw.f32", NULL);
    uint8_t* gate = (uint8_t*)read_file("gate.u8", NULL);
    uint8_t* up = (uint8_t*)read_file("up.u8", NULL);
    uint8_t* down = (uint8_t*)read_file("down.u8", NULL);
    uint8_t* sgate = (uint8_t*)read_file("sgate.u8", NULL);
    uint8_t* sup = (uint8_t*)read_file("sup.u8", NULL);
    uint8_t* sdown = (uint8_t*)read_file("sdown.u8", NULL);
    orc_weights* W = (orc_weights*)malloc(sizeof(orc_weights) * (size_t)L);
    for (int l = 0; l < L; ++l) {
        W[l].norm_w = norm_w + (long)l * H;
        W[l].router_w = router + (long)l * E * H;
        W[l].shared_gate_w = sgw + (long)l * H;
        W[l].gate = gate + (long)l * E * F * rb_gu;
        W[l].up = up + (long)l * E * F * rb_gu;
        W[l].down = down + (long)l * E * H * rb_dn;
        W[l].sgate = sgate + (long)l * Fs * rb_s;
        W[l].sup = sup + (long)l * Fs * rb_s;
        W[l].sdown = sdown + (long)l * H * rb_sd;
    }

    /* the stack */
    uint16_t* input = (uint16_t*)read_file("input.u16", NULL);
    uint16_t* out = (uint16_t*)calloc((size_t)H, sizeof(uint16_t));
    int32_t* ids = (int32_t*)calloc((size_t)L * k, sizeof(int32_t));
    if (orc_moe_stack(&d, W, L, input, NULL, out, ids, NULL, NULL, NULL) != 0) return 3;
    write_file("stack_out.u16", out, sizeof(uint16_t) * (size_t)H);
    write_file("stack_ids.i32", ids, sizeof(int32_t) * (size_t)L * k);
    /* the stack behind an attention block's outputs */
    uint16_t* attn = (uint16_t*)read_file("attn.u16", NULL);
    if (orc_moe_stack(&d, W, L, input, attn, out, ids, NULL, NULL, NULL) != 0) return 7;
    write_file("stack_attn_out.u16", out, sizeof(uint16_t) * (size_t)H);
    free(attn);

    /* the grouped batch on layer 0 */
    uint16_t* br = (uint16_t*)read_file("batch_res.u16", NULL);
    uint16_t* brp = (uint16_t*)read_file("batch_rp.u16", NULL);
    uint16_t* bsp = (uint16_t*)read_file("batch_sp.u16", NULL);
    orc_batch_out bo;
    memset(&bo, 0, sizeof(bo));
    bo.routed = (uint16_t*)calloc((size_t)n_tok * H, sizeof(uint16_t));
    bo.shared = (uint16_t*)calloc((size_t)n_tok * H, sizeof(uint16_t));
    if (orc_moe_layer_batch(&d, &W[0], n_tok, br, brp, bsp, NULL, &bo) != 0) return 4;
    write_file("batch_routed.u16", bo.routed, sizeof(uint16_t) * (size_t)n_tok * H);
    write_file("batch_shared.u16", bo.shared, sizeof(uint16_t) * (size_t)n_tok * H);

    /* top-k of tie-heavy logit sets */
    float* lg = (float*)read_file("logits.f32", NULL);
    int32_t* tk = (int32_t*)calloc((size_t)n_sets * k, sizeof(int32_t));
    for (int s = 0; s < n_sets; ++s) orc_topk(lg + (long)s * E, E, k, tk + (long)s * k);
    write_file("topk.i32", tk, sizeof(int32_t) * (size_t)n_sets * k);

    /* the Q8_1 quantiser */
    size_t nx = 0;
    float* qx = (float*)read_file("q81_x.f32", &nx);
    nx /= sizeof(float);
    uint8_t* q81 = (uint8_t*)calloc(nx / 32 * 36, 1);
    orc_quantize_q8_1(qx, (int)nx, q81);
    write_file("q81.u8", q81, nx / 32 * 36);

    /* load-time requantisation of layer 0's routed down and shared gate rows */
    const long rq_down = (long)E * H * (Kp / 256) * 144, rq_sg = (long)Fs * (H / 256) * 144;
    uint8_t* rd = (uint8_t*)calloc((size_t)rq_down, 1);
    uint8_t* rs = (uint8_t*)calloc((size_t)rq_sg, 1);
    if (orc_requant_q4k(W[0].down, d.down_type, E * H, Kp, rd) != 0) return 5;
    if (orc_requant_q4k(W[0].sgate, d.shared_type, Fs, H, rs) != 0) return 6;
    write_file("requant_down.u8", rd, (size_t)rq_down);
    write_file("requant_sgate.u8", rs, (size_t)rq_sg);

    free(rs); free(rd); free(q81); free(qx); free(tk); free(lg);
    free(bo.shared); free(bo.routed); free(bsp); free(brp); free(br);
    free(ids); free(out); free(input); free(W);
    free(sdown); free(sup); free(sgate); free(down); free(up); free(gate);
    free(sgw); free(router); free(norm_w); free(dv);
    return 0;
}
