// Types shared by the host scheduler and the device interpreter.
//
// The static schedule follows the Hazy Research "Megakernel" article (section
// "Megakernel: a fusion design from scratch"): each compute unit gets an ordered
// list of instructions, each one a structural unit of the transformer, laid out
// once on the host and reused for every token.
#pragma once
#include <stdint.h>

// Work-group shape, one work-group per CU: MK_NC compute waves that only read LDS,
// MK_NL loader waves that only stream pages HBM -> LDS, and one leader wave that waits on
// dependencies and stages activation vectors.
#define MK_NC 4
#define MK_NL 2
#define MK_NWAVES (MK_NC + MK_NL + 1)
#define MK_THREADS (64 * MK_NWAVES)
#define MK_MAX_SLOTS 16
#define MK_PAGE_BYTES 16384               // one LDS page: 16 units of 1 KiB
#define MK_NACT 2                         // staged activation vectors (ring)
#ifndef MK_HOLD_PAGES
#define MK_HOLD_PAGES 1                   // compute waves hold weight pages in registers (0: off)
#endif
#define MK_MAX_RES_ROWS 64                // rows of x one CU owns in a residual op
#define MK_MAX_NCH 4                      // K-chunks of the down projection
#ifndef MK_SPLIT_PAGES
#define MK_SPLIT_PAGES 1                  // two-page O / down instructions: two waves per page
#endif

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
  int32_t pad0, pad1;     // reserved (zero)
  int32_t rs;             // row stride: the instruction's rows are r0, r0 + rs, ...; GATEUP:
                          // features come in page groups of FPP, feature q = r0 + (q / FPP) * rs + q % FPP
  int32_t pad2;
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

// Kernel argument block (passed by value).  The model's widths are template
// parameters of the kernel; only what varies per call or per model depth is here.
struct MkParams {
  int32_t n_layers, V, max_ctx, n_cus;
  int32_t nslot, s_max, min_chunk;   // nslot: pages in the LDS ring
  int32_t demand_depth;              // pages in flight per loader for an instruction already staged
  float eps, attn_scale;
  // weights (bf16)
  const uint16_t* embed;
  const uint16_t* lm_head;
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

// Trace slots per instruction: [0] leader starts, [1] leader starts polling its
// inputs, [2] inputs all present, [3] slot free, [4] activation staged, [5] compute
// wave 0 starts, [6] last compute wave done, [7] leader done (attention merge /
// argmax), [8] leader saw every compute wave done (attention / LM head), [9] ticks the
// compute waves waited for the instruction's pages (a sum over waves).
#define MK_TRACE_SLOTS 12
#define MK_TRACE_MAX 272                  // instructions of a CU's list the trace covers
