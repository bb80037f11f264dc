// Types shared by the host scheduler and the device interpreter.
//
// The static schedule follows the Hazy Research "Megakernel" article (section
// "Megakernel: a fusion design from scratch"): each compute unit gets an ordered
// list of instructions, each one a structural unit of the transformer, laid out
// once on the host and reused for every token.
#pragma once
#include <stdint.h>

// Work-group shape, one work-group per CU: MK_NC compute waves that only read LDS,
// MK_NL loader waves that only stream pages HBM -> LDS, and one leader wave that
// waits on dependencies and stages the activation vector.
#define MK_NC 4
#define MK_NL 2
#define MK_NWAVES (MK_NC + MK_NL + 1)
#define MK_THREADS (64 * MK_NWAVES)
#define MK_MAX_SLOTS 32

// LDS budget (gfx950 has 160 KiB per work-group).
#define MK_ACT_FLOATS 4096                // activation vector staged per instruction
#define MK_PAGES_BYTES (128 * 1024)       // page ring shared by the loaders and compute waves
#define MK_MAX_RES_ROWS 64                // rows of x one CU owns in a residual op
#define MK_GATE_SCRATCH 16                // gate results held per wave until the up row
#define MK_MAX_HPG 8                      // query heads per KV head
#define MK_PART_OFF 1024                  // offset (floats) of per-wave attention partials in act
#define MK_GATHER_MAXW 32                 // words per lane one gather batch holds
// The activation-word arena is padded by one gather batch, so a batch may load past the
// end of the vector it polls without a bounds test per word.
#define MK_LL_PAD (64 * MK_GATHER_MAXW)

// Instruction opcodes — the article's six fused instructions.
enum {
  MK_OP_QKV = 1,    // RMSNorm + QKV projection (RoPE is applied where q/k are consumed)
  MK_OP_ATTN = 2,   // split-KV GQA attention partial (+ merge of the splits)
  MK_OP_O = 3,      // O-projection + residual
  MK_OP_GATEUP = 4, // RMSNorm + SiLU(gate) * up
  MK_OP_DOWN = 5,   // one K-chunk of the down projection (+ residual on the last chunk)
  MK_OP_LMHEAD = 6  // final RMSNorm + LM head + argmax
};

// One instruction record (12 x int32).
struct MkInstr {
  int32_t op, layer;
  int32_t r0, n;          // output rows [r0, r0 + n): QKV rows, O/DOWN rows of x, GATEUP
                          // intermediate features, LM-head vocabulary rows
  int32_t k0, kn;         // input columns [k0, k0 + kn) of every row (a DOWN chunk); else 0, K
  int32_t a, b;           // ATTN: kv head, split index; DOWN: chunk index, chunk count
  int32_t res_r0, res_n;  // QKV / GATEUP: rows of x kept for the residual of the next O / DOWN
  int32_t pad0, pad1;
};
#define MK_INSTR_WORDS 12

struct MkLayerPtrs {
  const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *wg, *wu, *wd;
};

// Device control block.
struct MkCtrl {
  uint32_t epoch;      // tag of the step in flight; advanced by the step's last CU
  uint32_t ticket;     // arrivals at the final argmax
  int32_t error;       // 0 or an MK_E* code set by a device-side check
  int32_t bad_token;   // a device-side token was outside [0, vocab) and was clamped
  uint32_t pad[4];
};

// Kernel argument block (passed by value).
struct MkParams {
  // shape
  int32_t n_layers, d, hq, hkv, hd, F, V, max_ctx;
  int32_t nq, nkv, nqkv, hpg;
  float eps, attn_scale;
  // schedule
  int32_t n_cus, page_bytes, nslot, lpp, s_max, min_chunk;   // nslot: pages in the LDS ring
  // weights (bf16)
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  const MkLayerPtrs* layers;      // [n_layers + 1]; entry n_layers: attn_norm = final norm
  const float* rope;              // [max_ctx][hd/2][2]: cos, sin
  // static plan
  const int32_t* plan_off;        // [n_cus + 1]
  const MkInstr* plan;
  // communication words: low 32 bits value, high 32 bits producing step's epoch
  unsigned long long* ll_x;       // [2L + 1][d]      (x after each residual; index 0 unused)
  unsigned long long* ll_qkv;     // [L][hkv][q heads of the group | k | v][hd] (raw)
  unsigned long long* ll_part;    // [L][hkv][hpg][s_max][hd + 2]  (m, l, o of a split)
  unsigned long long* ll_o;       // [L][hq * hd]     (attention output)
  unsigned long long* ll_a;       // [L][F]           (SiLU(gate) * up)
  unsigned long long* amax;       // [n_cus]          (per-CU argmax keys)
  MkCtrl* ctrl;
  // per step
  uint16_t* kv;                   // [L][2][hkv][max_ctx][hd]
  float* logits;                  // [V]
  int32_t* next_token;            // [1] or null
  const int32_t* token_dev;       // [1] or null
  int32_t token, pos;
  long long watchdog_ticks;       // s_memrealtime ticks (100 MHz)
  // optional timestamp trace [n_cus][trace_len][MK_TRACE_SLOTS] (s_memrealtime ticks)
  unsigned long long* trace;
  int32_t trace_len;
};

// Trace slots per instruction: leader start, inputs ready, activation staged, leader
// done (after attention merge / argmax), then the finish time of each compute wave.
#define MK_TRACE_SLOTS 8
