// moe_stack.h -- geometry and arguments of the persistent L-layer stack kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

constexpr int kStackThreads = 512;
constexpr int kStackWaves = kStackThreads / 64;
constexpr int kStackMinLds = 84 * 1024;     // above half of a CU's LDS: one workgroup per CU
constexpr int kStackMaxLds = 160 * 1024;
// control block: word 0 = generation, word kErrWord = error
constexpr uint32_t kErrWord = 16;
constexpr uint32_t kStackCtrlBytes = 256;
// phase timestamps of workgroup 0: [layer][slot], 100 MHz wall clock
constexpr int kTraceLayers = 64;
constexpr int kTraceSlots = 12;   // 0..9 wall clock at phase boundaries, 10/11 shader cycles at layer start/end
// per-workgroup event times [layer][workgroup][event], written only when asked for
constexpr int kBlockEvents = 16;
constexpr int kTraceMaxG = 256;

struct StackGeom {
  int G;
  int RR, SR, RD, RP;                 // per-workgroup rows: router, shared gate/up, down outputs, routed gate/up pairs
  int Kp, Kps;
  int n_t, n_lg, n_h, n_sel, n_y;     // exchange sizes in 8-byte words (n_sel: selection words in LDS)
  // LDS byte offsets
  int o_res, o_xn, o_xqc, o_xqd, o_xqs, o_nw, o_rrow, o_sgu, o_sdn, o_rgu, o_rdn, o_hqc, o_hqd, o_hqs, o_part, o_xbuf,
      o_sel, o_red, o_y, o_cand, o_keys, o_lgsel, o_hs, o_attn, o_candlg;
  int sgu_half, rgu_half, rdn_slot;
  int lds;
  // workspace byte offsets
  size_t w_ctrl, w_t, w_lg, w_h, w_y, w_trace, w_end;
};

constexpr uint32_t kBoundMagic = 0x4d6f4553u;

// 64-bit hash of a layer-pointer table (its bytes, 8 at a time): moe_stack_bind
// stores it beside the device copy of the table, and every launch compares it
// with the caller's.
uint64_t layer_table_hash(const moe_layer_weights* layers, int n);

struct StackArgs {
  StackGeom g;
  const moe_layer_weights* layers;   // device copy of the per-layer pointer table
  const uint32_t* bound;             // {magic, n_layers, hash lo, hash hi} written by moe_stack_bind
  uint64_t table_hash;               // hash of the caller's table
  const uint16_t* input;
  uint16_t* output;
  int32_t* ids_out;
  uint16_t* resid_out;
  uint16_t* routed_out;
  uint16_t* shared_out;
  const uint16_t* attn;              // [L][H] attention-block outputs, or nullptr
  uint8_t* ws;
  int L, H, E, k, F, Fs;
  float eps;
  int trace_blocks;                  // nonzero: every workgroup stamps its events
};

int stack_geometry(const moe_layer_desc* d, int G, StackGeom* out);
void stack_ws_layout(StackGeom* g, size_t base);
// cooperative: a cooperative launch (the runtime places the whole grid at
// once); else a plain one, resident as a whole when no other kernel holds CUs
int launch_stack(const moe_layer_desc* d, int L, const moe_layer_weights* table_dev, const uint32_t* bound,
                 uint64_t table_hash, const moe_stack_io* io, uint8_t* ws, const StackGeom& g, hipStream_t st,
                 bool cooperative);
int device_cu_count(int* n);
// the persistent kernel instance for a description and its geometry; *shape
// (if given) gets the compile-time shape index (0 = sizes at run time)
const void* stack_kernel_for(const moe_layer_desc* d, const StackGeom& g, int* shape);
int launch_test_stack_select(const float* logits, int n_sets, int E, int k, int with_gate, int32_t* ids, float* wts,
                             float* gate, hipStream_t st);

}  // namespace moe
