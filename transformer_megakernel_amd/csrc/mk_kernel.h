// Persistent decode-step interpreter for gfx950 (one work-group per CU).
//
// Design after the Hazy Research "Megakernel" article on Llama-3.2-1B, section
// "Megakernel: a fusion design from scratch", re-thought for CDNA4:
//
//  * Instruction interpreter.  Every CU walks its own ordered instruction list
//    (QKV, ATTN, O, GATEUP, DOWN x4 per layer, then LMHEAD) laid out by the host.
//  * Paged LDS with early weight loads.  The article pages shared memory so that the
//    next instruction's weights load while the current one computes.  Here MK_NL
//    loader waves stream every page of the CU's list into one LDS ring with
//    global_load_lds_dwordx4 (HBM -> LDS, no registers, non-temporal), across
//    instruction boundaries and before the data an instruction depends on exists:
//    weights and cached keys never depend on this step's activations.  A loader
//    knows a page is complete from its own vmcnt and raises the slot's LDS flag;
//    compute waves never issue loads, so a wait for data never stalls behind the
//    weight stream.
//  * Dependencies without grid barriers.  The article uses integer counters in
//    global memory; on gfx950 the eight XCDs have separate L2s, so a counter costs a
//    store-acknowledge, an atomic and a second round trip for the data.  Instead each
//    produced value travels with its own completion flag: a 64-bit word holding the
//    fp32 value and the step's epoch, stored and polled with device-scope accesses.
//    A consumer is ready when every word it needs carries the current epoch.  The
//    step's last CU (an atomic ticket, the one counter kept) advances the epoch.
//  * A leader wave per CU does the waiting: it polls the inputs of the next
//    instruction, applies RMSNorm / RoPE and stages the fp32 activation vector into
//    one of MK_NACT LDS slots, so it can prepare instruction i+1 while the compute
//    waves still work on instruction i.
//  * The model's widths are template parameters: indices are compile-time arithmetic
//    and loops have fixed trip counts.
//  * The article's 4-chunk MLP intermediate: the down projection is issued as K-chunks,
//    each waiting only for its part of SiLU(gate)*up.
//
// Every wait is bounded (watchdog); on expiry the wave records MK_ETIMEOUT, drains
// its outstanding loads and exits, and the other waves follow.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/mk.h"
#include "mk_types.h"

namespace mkdev {

typedef __attribute__((address_space(3))) char lds_char;
typedef unsigned long long u64;
// Read-only tables are read through the constant address space so that the compiler
// uses scalar loads.
#if defined(__HIP_DEVICE_COMPILE__)
typedef const __attribute__((address_space(4))) MkInstr* cinstr_t;
typedef const __attribute__((address_space(4))) MkLayerPtrs* clayers_t;
typedef const __attribute__((address_space(4))) int32_t* cint_t;
#else
typedef const MkInstr* cinstr_t;   // host pass: the kernel body is only parsed
typedef const MkLayerPtrs* clayers_t;
typedef const int32_t* cint_t;
#endif

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// ------------------------------------------------------------------ model shape
// Widths of one Llama-style decoder.  NCH: K-chunks of the down projection.
template <int D_, int HQ_, int HKV_, int HD_, int F_, int NCH_>
struct Shape {
  static constexpr int D = D_, HQ = HQ_, HKV = HKV_, HD = HD_, F = F_, NCH = NCH_;
  static constexpr int HPG = HQ / HKV, NQ = HQ * HD, NKV = HKV * HD, NQKV = NQ + 2 * NKV;
  static constexpr int KC = F / NCH;                  // width of one down chunk
  static constexpr int GRP = (HPG + 2) * HD;          // q heads | k | v of one KV group
  static constexpr int ACT = cmax(cmax(D, NQ), cmax(KC, GRP));   // floats of one staged vector
  static constexpr int PPP = MK_PAGE_BYTES / (4 * HD);           // cached positions per page
  static_assert(D % 128 == 0 && NQ % 64 == 0 && KC % 64 == 0 && GRP % 64 == 0, "widths");
  static_assert(HD == 64 || HD == 128, "head_dim");
  static_assert(NCH >= 1 && NCH <= MK_MAX_NCH, "down chunks");
  static constexpr bool TRACE = false;
};
// The same widths, built with the per-instruction trace (a separate kernel, so that the
// untraced one carries no trace code: it measured 1.5-2 % slower when the loader's
// instrumentation was merely compiled in, from instruction-cache misses).
template <class B>
struct Traced : B {
  static constexpr bool TRACE = true;
};

// Attention items with several splits.  On the matrix units (head_dim 64 or 128), every
// compute wave taking 16 keys of its pages for all of the group's query heads (KS = 4 key
// subsets); otherwise one query head per wave (KS = MK_NC / HPG subsets per head).
// The subsets' partials (m, l, o) per head go to the activation slot, after q|k|v, where
// there is room, else to their own LDS array.
template <class S>
struct AttnGeo {
  static constexpr bool MMA = (S::HD == 64 || S::HD == 128) && S::HPG <= 4 && S::PPP % 16 == 0 &&
                              MK_NC % (S::PPP / 16) == 0;
  static constexpr int KS = MMA ? MK_NC : MK_NC / S::HPG;
  static constexpr int PART = KS * S::HPG * (S::HD + 2);     // floats of partials
  static constexpr int OFF = (S::GRP + 63) / 64 * 64;        // their offset in the slot
  static constexpr bool IN_ACT = OFF + PART <= S::ACT;
  static constexpr int OWN = IN_ACT ? 0 : PART;              // floats of the LDS array
  // q-head mode keeps one (m, l, o) per compute wave in the array
  static constexpr int LDS = cmax(MK_NC * (S::HD + 2), OWN);
};

// LDS of one work-group (the page ring is a separate array).
template <class S>
struct __align__(16) MkShared {
  float act[MK_NACT][S::ACT];               // staged activation vectors (ring)
  float part[AttnGeo<S>::LDS];              // attention partials (m, l, o): q-head mode, key subsets
  static_assert(MK_NC % S::HPG == 0, "query heads per KV head must divide the compute waves");
  int acnt[MK_MAX_SLOTS];                   // readers done with the attention page in a slot
  float xres[2][MK_MAX_RES_ROWS];           // x rows for the residual of O (0) and DOWN (1)
  float dpart[MK_MAX_NCH][MK_MAX_RES_ROWS]; // down-projection partial sums per chunk
  u64 amax[MK_NC];                          // per-wave argmax keys (LM head)
  alignas(16) int done[MK_NC];              // instructions finished, per compute wave
  int full[MK_MAX_SLOTS];                   // ring slot holds page k once full == k + 1
  int freed[MK_MAX_SLOTS];                  // ring slot's page k consumed once freed == k + 1
  uint32_t tr[S::TRACE ? MK_TRACE_MAX : 1][MK_TRACE_SLOTS];   // the trace: ticks after t0 (slots 9, 11: durations)
  unsigned long long t0;                    // s_memrealtime at the work-group's start
  int act_seq;                              // instructions staged by the leader
  int pcnt;                                 // matrix-unit attention partials written (per wave)
  int abort_flag;
  uint32_t epoch;                           // tag of this step's words
  int token;                                // input token (validated)
};

// Pages in the LDS ring: what is left of 160 KiB, a multiple of MK_NL.
template <class S>
struct Ring {
  static constexpr int FIXED = (int)sizeof(MkShared<S>) + 256;
  static constexpr int NSLOT_RAW = (160 * 1024 - FIXED) / MK_PAGE_BYTES;
  static constexpr int NSLOT = (NSLOT_RAW > MK_MAX_SLOTS ? MK_MAX_SLOTS : NSLOT_RAW) / MK_NL * MK_NL;
  static_assert(NSLOT >= 2 * MK_NL, "LDS");
};

// ------------------------------------------------------------------ small helpers
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// HBM -> LDS, 16 bytes per lane: lane i lands at lds + 16*i.  Issued through inline
// assembly so that the compiler does not add a wait for it before later LDS accesses.
// Non-temporal: each weight byte is read once per step and should not displace
// anything in L2.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(g), "s"(l) : "memory", "m0");
}

#define MK_VMCNT_CASE(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
// Wait until at most n vector-memory operations of this wave are outstanding (n is a
// multiple of 16 below 64: pages are 16 loads).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    MK_VMCNT_CASE(16) MK_VMCNT_CASE(32) MK_VMCNT_CASE(48)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
#undef MK_VMCNT_CASE

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// A copy of v the compiler cannot see through: per-lane addresses derived from it are
// recomputed in each loop iteration instead of being hoisted and kept live all kernel.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
// Ties a loaded value to this point of the program, so that the compiler cannot sink
// the load into the branch that uses it (which would make one round trip per load).
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ int lds_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Device-scope (cross-XCD coherent) 64-bit words: value in the low half, epoch above.
__device__ __forceinline__ u64 ll_load(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ll_store(u64* p, float v, uint32_t epoch) {
  __hip_atomic_store(p, ((u64)epoch << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ll_val(u64 w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ bool ll_ok(u64 w, uint32_t epoch) { return (uint32_t)(w >> 32) == epoch; }

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (quiet NaN kept).
// bf16 bits of a finite float, rounded to nearest even (no NaN case: no branches)
__device__ __forceinline__ uint16_t f2bf_finite(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float dot8(uint4 w, const float* a, float acc) {
  acc = fmaf(bf_lo(w.x), a[0], acc);
  acc = fmaf(bf_hi(w.x), a[1], acc);
  acc = fmaf(bf_lo(w.y), a[2], acc);
  acc = fmaf(bf_hi(w.y), a[3], acc);
  acc = fmaf(bf_lo(w.z), a[4], acc);
  acc = fmaf(bf_hi(w.z), a[5], acc);
  acc = fmaf(bf_lo(w.w), a[6], acc);
  acc = fmaf(bf_hi(w.w), a[7], acc);
  return acc;
}

// ------------------------------------------------------------------ reductions
// Cross-lane sums through DPP moves (no LDS round trip).  sumN leaves the sum of each
// aligned group of N lanes in every lane of the group.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v, float old) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<0xB1>(v, 0.f);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v, 0.f);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v, 0.f);   // row_half_mirror
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp_f<0x140>(v, 0.f);   // row_mirror
  return v;
}
// Sum over the wave, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  v += dpp_f<0x142, 0xa>(v, 0.f);   // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(v, 0.f);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x4E>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x141>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x140>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x142, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x143, 0xc>(v, -INFINITY));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// gfx950 lane swaps (VALU, no LDS round trip).  For a, b per lane, swap32 returns
// {a[l] | b[l - 32], a[l + 32] | b[l]} (lanes below | from 32), swap16 the same within
// each 32-lane half with 16-lane rows.  So for the pair (lo, hi) the sum of the two
// results is lo(l) + lo(partner) in the lower lanes and hi(l) + hi(partner) in the upper
// ones: one halving step of a cross-lane reduction.
__device__ __forceinline__ float swap_sum32(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v of lane l ^ 32, lane l ^ 16.
__device__ __forceinline__ float xor32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}
__device__ __forceinline__ float xor16(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
// v of lane l ^ OFF for OFF in {8, 16, 32}; other distances through LDS permutes.
template <int OFF>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  if constexpr (OFF == 32) return xor32(v, lane);
  else if constexpr (OFF == 16) return xor16(v, lane);
  else if constexpr (OFF == 8) return dpp_f<0x128>(v, 0.f);   // row_ror:8 within 16-lane rows
  else return __shfl_xor(v, OFF);
}
// Sum within aligned groups of G lanes (G a power of two <= 64), in every lane.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 16) v = sum16(v);
  else if constexpr (G == 8) v = sum8(v);
  else {
    if constexpr (G >= 2) v += dpp_f<0xB1>(v, 0.f);
    if constexpr (G >= 4) v += dpp_f<0x4E>(v, 0.f);
  }
  if constexpr (G >= 32) v = swap_sum16(v, v);
  if constexpr (G >= 64) v = swap_sum32(v, v);
  return v;
}

// N values per lane, each to be summed over aligned groups of G lanes (N <= G, both
// powers of two).  Halving steps hand half of the values to the partner lane, so that
// after log2(N) steps each lane holds one partial; the rest of the group is then summed.
// Value n ends in the lanes l with (l % G) / (G / N) == n.
template <int N, int G>
__device__ __forceinline__ float reduce_rows(float (&v)[N], int lane) {
  static_assert(N <= G, "reduce_rows");
#pragma unroll
  for (int s = 0; s < ilog2(N); ++s) {
    const int dist = G >> (s + 1);
    const int n = N >> s;
    if (dist == 32 || dist == 16) {   // lane swaps: lo kept in the lower lanes, hi in the upper
#pragma unroll
      for (int i = 0; i < n / 2; ++i) v[i] = dist == 32 ? swap_sum32(v[i], v[i + n / 2]) : swap_sum16(v[i], v[i + n / 2]);
      continue;
    }
    // Selects through a bit mask: a lane-dependent choice between two array elements
    // must not become an indexed (private memory) access.
    const uint32_t m = (lane & dist) ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + n / 2]);
      const float keep = __uint_as_float((hi & m) | (lo & ~m));
      const float send = __uint_as_float((lo & m) | (hi & ~m));
      v[i] = keep + __shfl_xor(send, dist);
    }
  }
  return group_sum<G / N>(v[0]);
}

__device__ __forceinline__ u64 wave_max_u64(u64 v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    u64 o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// Argmax key: larger value wins, then the lower index.
__device__ __forceinline__ u64 amax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((u64)u << 32) | (u64)(0xffffffffu - idx);
}

// The trace is kept in LDS during the step and written out once at its end (a global
// store per mark would queue behind the weight stream and hold up the next poll's wait).
template <class S>
__device__ __forceinline__ void trace_mark(const MkParams& p, MkShared<S>& sh, int i, int slot, int lane) {
  if constexpr (S::TRACE) {
    if (lane == 0 && i < p.trace_len)
      sh.tr[i][slot] = (uint32_t)(__builtin_amdgcn_s_memrealtime() - sh.t0) + 1u;   // 0: not marked
  }
}
// Latest of several waves' marks.
template <class S>
__device__ __forceinline__ void trace_max(const MkParams& p, MkShared<S>& sh, int i, int slot, int lane) {
  if constexpr (S::TRACE) {
    if (lane == 0 && i < p.trace_len)
      atomicMax(&sh.tr[i][slot], (uint32_t)(__builtin_amdgcn_s_memrealtime() - sh.t0) + 1u);
  }
}

// ------------------------------------------------------------------ step geometry
struct StepGeo {
  int pos, s_eff, chunk;   // attention split of the cached keys 0..pos-1
  int qh;                  // one split: item (g, b < HPG) computes query head g * HPG + b
};

// Attention items in a step.  With one split (short contexts) the first HPG items of a
// KV group each take one query head over all keys, its four compute waves splitting the
// keys, so a head's scores are spread over four waves instead of one; with several
// splits, item (g, s) takes split s of group g for all of the group's heads.
__device__ __forceinline__ bool attn_active(const StepGeo& g, int b, int hpg) {
  return g.qh ? b < hpg : b < g.s_eff;
}

template <class S>
__device__ __forceinline__ StepGeo step_geo(const MkParams& p, int pos) {
  StepGeo g;
  g.pos = pos;
  // The splits cover the cached keys 0..pos-1; the current key joins the last split.
  // (Splitting keys 0..pos instead left a split holding the current key alone whenever
  // pos was a multiple of the split size, and at pos 8192 forced 320-key splits, 26 of
  // them instead of 32 of 256: 687.6 vs 680.0 us per step.)
  const int nk = pos > 1 ? pos : 1;
  int chunk = (nk + p.s_max - 1) / p.s_max;
  if (chunk < p.min_chunk) chunk = p.min_chunk;
  chunk = (chunk + S::PPP - 1) / S::PPP * S::PPP;
  g.chunk = chunk;
  g.s_eff = (nk + chunk - 1) / chunk;
  g.qh = g.s_eff == 1;
  return g;
}

// ------------------------------------------------------------------ page geometry
// Rows of SEG bytes in a 16 KiB page.  Wide rows (>= 1 KiB) are KU whole units of
// 1 KiB, lane l holding bytes 16l.. of each unit; narrow rows share a unit, LPR lanes
// per row.
template <int SEG>
struct RowGeo {
  static constexpr bool WIDE = SEG >= 1024;
  static constexpr int KU = WIDE ? SEG / 1024 : 1;        // units per row
  static constexpr int LPR = WIDE ? 64 : SEG / 16;        // lanes per row within a unit
  static constexpr int RPU = WIDE ? 1 : 64 / LPR;         // rows per unit
  static constexpr int RPP = WIDE ? 16 / KU : 16 * RPU;   // rows per page
  static constexpr int USED = WIDE ? RPP * KU : 16;       // units carrying payload
  static constexpr int NV = WIDE ? RPP : 16;              // partial sums per lane per page
  static constexpr int G = WIDE ? 64 : LPR;               // lanes a partial is summed over
  static_assert(WIDE ? (SEG % 1024 == 0 && SEG <= 8192) : (SEG == 256 || SEG == 512), "row length");
};

// An instruction decoded once: everything its pages need, wave-uniform.
struct Dec {
  int op, layer, r0, n, k0, a, b;
  int rs;            // row stride of the instruction's rows
  int np;            // pages of the instruction on this CU
  int rpp;           // rows per page (GATEUP: gate and up rows, two per feature)
  const char* m0;    // row 0 of each source matrix, input column k0 applied (bytes)
  const char* m1;
  const char* m2;
  int j0, ce;        // ATTN: cached keys [j0, ce); m0 / m1 = K / V of (layer, kv head) at key 0
  int rp, rw;        // leading pages held in compute-wave registers: page j by wave rw + j;
                     // np counts the ring pages that follow them
};

// Held pages (see compute_wave) take 64 VGPRs per compute wave: used where the kernel has
// that room (hidden <= 2048; the 4096-wide instance spills registers already, and holding
// pages there measured 1.2 % slower).  Down pages can be held when they are whole 16-unit
// pages and there are at least two chunks.
template <class S>
__device__ constexpr bool hold_pages() { return MK_HOLD_PAGES && S::D <= 2048; }
template <class S>
__device__ constexpr bool hold_down() { return hold_pages<S>() && S::NCH >= 2 && RowGeo<2 * S::KC>::USED == 16; }

template <class S>
__device__ __forceinline__ Dec decode(const MkParams& p, const MkInstr& in, const StepGeo& g) {
  Dec d;
  d.op = in.op; d.layer = in.layer; d.r0 = in.r0; d.n = in.n; d.k0 = in.k0; d.a = in.a; d.b = in.b;
  d.rs = in.rs;
  d.m0 = d.m1 = d.m2 = nullptr;
  d.j0 = d.ce = 0;
  d.rpp = 0;
  d.rp = d.rw = 0;
  if (in.op == MK_OP_ATTN) {
    d.np = 0;
    if (attn_active(g, in.b, S::HPG)) {
      const int sb = g.qh ? 0 : in.b;
      d.j0 = sb * g.chunk;
      d.ce = min(min(g.pos + 1, (sb + 1) * g.chunk), g.pos);   // the current key is not in the cache yet
      const int cached = d.ce - d.j0;
      d.np = cached > 0 ? (cached + S::PPP - 1) / S::PPP : 0;
    }
    const size_t head = ((size_t)(in.layer * 2) * S::HKV + in.a) * p.max_ctx;
    d.m0 = (const char*)(p.kv + head * S::HD);
    d.m1 = (const char*)(p.kv + (head + (size_t)S::HKV * p.max_ctx) * S::HD);
    return d;
  }
  const int seg = in.op == MK_OP_O ? 2 * S::NQ : in.op == MK_OP_DOWN ? 2 * S::KC : 2 * S::D;
  d.rpp = MK_PAGE_BYTES / seg;
  const int rows = in.op == MK_OP_GATEUP ? 2 * in.n : in.n;
  d.np = (rows + d.rpp - 1) / d.rpp;
  // Held pages (see compute_wave): gate/up page w by wave w, and the pages of the last two
  // down chunks, chunk NCH-2 by waves 0, 1 and chunk NCH-1 by waves 2, 3.
  if (hold_pages<S>() && in.op == MK_OP_GATEUP) {
    d.rp = min(MK_NC, d.np);
  } else if (in.op == MK_OP_DOWN && hold_down<S>() && in.a >= S::NCH - 2) {
    d.rp = min(2, d.np);
    d.rw = 2 * (in.a - (S::NCH - 2));
  }
  d.np -= d.rp;
  // Plain selects, not a switch: a switch over runtime values becomes a table in
  // private memory.
  const MkLayerPtrs L = ((clayers_t)p.layers)[in.layer < p.n_layers ? in.layer : 0];
  const bool qkv = in.op == MK_OP_QKV, gu = in.op == MK_OP_GATEUP, o = in.op == MK_OP_O,
             dn = in.op == MK_OP_DOWN;
  const uint16_t* a0 = qkv ? L.wq : gu ? L.wg : o ? L.wo : dn ? L.wd + in.k0 : p.lm_head;
  d.m0 = (const char*)a0;
  d.m1 = (const char*)(qkv ? L.wk : gu ? L.wu : a0);
  d.m2 = (const char*)(qkv ? L.wv : a0);
  return d;
}

// Feature of the GATEUP instruction's q-th feature: the features come in blocks of 2^a
// (a page's features, or eight: one 64-byte line of link words), one block per rs
// features of the intermediate.
template <class S>
__device__ __forceinline__ int gu_feature(const Dec& d, int q) {
  return d.r0 + (q >> d.a) * d.rs + (q & ((1 << d.a) - 1));   // blocks of 2^a features
}

// Address of row pr of the instruction, for one opcode.  GATEUP rows interleave gate(f),
// up(f), gate(f+1), up(f+1), ...; QKV rows run through Wq, then Wk, then Wv.
template <class S, int OP>
__device__ __forceinline__ const char* row_addr(const Dec& d, int pr) {
  if constexpr (OP == MK_OP_GATEUP) {
    const long long f = gu_feature<S>(d, pr >> 1);
    return ((pr & 1) ? d.m1 : d.m0) + f * (2LL * S::D);
  } else if constexpr (OP == MK_OP_QKV) {
    const int gr = d.r0 + pr * d.rs;
    if (gr >= S::NQ + S::NKV) return d.m2 + (long long)(gr - S::NQ - S::NKV) * (2 * S::D);
    if (gr >= S::NQ) return d.m1 + (long long)(gr - S::NQ) * (2 * S::D);
    return d.m0 + (long long)gr * (2 * S::D);
  } else {
    constexpr long long RB = OP == MK_OP_O ? 2 * S::NQ : OP == MK_OP_DOWN ? 2 * S::F : 2 * S::D;
    return d.m0 + (long long)(d.r0 + pr * d.rs) * RB;
  }
}

// Row j (page-relative) of page pg, any GEMV opcode.
template <class S>
__device__ __forceinline__ const char* row_ptr(const Dec& d, int pg, int j) {
  const int pr = pg * d.rpp + j;
  if (d.op == MK_OP_GATEUP) return row_addr<S, MK_OP_GATEUP>(d, pr);
  if (d.op == MK_OP_QKV) return row_addr<S, MK_OP_QKV>(d, pr);
  if (d.op == MK_OP_O) return row_addr<S, MK_OP_O>(d, pr);
  if (d.op == MK_OP_DOWN) return row_addr<S, MK_OP_DOWN>(d, pr);
  return row_addr<S, MK_OP_LMHEAD>(d, pr);
}

// Issue the DMA of page pg into the LDS page at `slot`: always 16 loads of 1 KiB so the
// wave's vmcnt moves in steps of 16; loads past the payload re-read valid bytes.  The
// opcode is a template parameter so that each row's address is formed once per page with
// no branching between the loads (the vector-memory issue slot is the loader's critical
// resource).
template <class S, int OP, int SEG>
__device__ __forceinline__ void issue_rows(const Dec& d, int pg, uint32_t slot, int lane) {
  using R = RowGeo<SEG>;
  const int rows = (OP == MK_OP_GATEUP ? 2 * d.n : d.n) - pg * d.rpp;   // rows from this page on
  if constexpr (R::WIDE) {
    const char* rb[R::RPP];
#pragma unroll
    for (int j = 0; j < R::RPP; ++j) rb[j] = row_addr<S, OP>(d, pg * R::RPP + (j < rows ? j : 0));
    const int lo = lane * 16;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = u / R::KU, c = u % R::KU;
      const bool real = u < R::USED;
      dma16(real ? rb[j] + c * 1024 + lo : rb[0] + lo, slot + u * 1024);
    }
  } else {
    const int jl = lane / R::LPR, cl = lane % R::LPR;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = u * R::RPU + jl;
      dma16(row_addr<S, OP>(d, pg * R::RPP + (j < rows ? j : 0)) + cl * 16, slot + u * 1024);
    }
  }
}
template <class S>
__device__ __forceinline__ void issue_page(const Dec& d, int pg, uint32_t slot, int lane) {
  if (d.op == MK_OP_ATTN) {
    constexpr int ROWB = 2 * S::HD;
    const int q0 = d.j0 + pg * S::PPP;
    const int np = min(S::PPP, d.ce - q0);
    const int kbytes = np * ROWB;
    const char* kb = d.m0 + (size_t)q0 * ROWB;
    const char* vb = d.m1 + (size_t)q0 * ROWB;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int o = u * 1024 + lane * 16;
      const char* a = o < kbytes ? kb + o : (o < 2 * kbytes ? vb + (o - kbytes) : kb);
      dma16(a, slot + u * 1024);
    }
    return;
  }
  if (d.op == MK_OP_GATEUP) issue_rows<S, MK_OP_GATEUP, 2 * S::D>(d, pg, slot, lane);
  else if (d.op == MK_OP_DOWN) issue_rows<S, MK_OP_DOWN, 2 * S::KC>(d, pg, slot, lane);
  else if (d.op == MK_OP_QKV) issue_rows<S, MK_OP_QKV, 2 * S::D>(d, pg, slot, lane);
  else if (d.op == MK_OP_O) issue_rows<S, MK_OP_O, 2 * S::NQ>(d, pg, slot, lane);
  else issue_rows<S, MK_OP_LMHEAD, 2 * S::D>(d, pg, slot, lane);
}

// ------------------------------------------------------------------ waits and aborts
template <class S>
__device__ __forceinline__ void raise_error(const MkParams& p, MkShared<S>& sh, int code) {
  atomicCAS(&p.ctrl->error, 0, code);
  lds_store(&sh.abort_flag, 1);
}

// Compute waves never read the global error word; they follow the LDS abort flag and
// their own clock.
template <class S>
struct Waiter {
  long long t0;
  int n;
  bool global_check;
  __device__ __forceinline__ Waiter(bool leader) : t0(__builtin_amdgcn_s_memrealtime()), n(0), global_check(leader) {}
  // true when the wait must be abandoned
  // nosleep: spin without s_sleep (LDS waits of the compute and loader waves, which
  // measured faster that way; the leader's waits, which poll global memory, keep it).
  __device__ __forceinline__ bool tick(const MkParams& p, MkShared<S>& sh, bool nosleep = false) {
    if (!nosleep) __builtin_amdgcn_s_sleep(1);
    if (__builtin_expect(lds_load(&sh.abort_flag) != 0, 0)) return true;
    // A zero budget gives up at the first round of waiting (the host's way to exercise the
    // abandon path); otherwise the clock is read every 64 rounds.  The rare paths are
    // marked unlikely so that the compiler lays them out away from the wait loops.
    if (__builtin_expect((++n & 63) == 0 || p.watchdog_ticks == 0, 0)) {
      if (__builtin_expect(global_check &&
                           __hip_atomic_load(&p.ctrl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0, 0)) {
        lds_store(&sh.abort_flag, 1);
        return true;
      }
      if (__builtin_expect((long long)__builtin_amdgcn_s_memrealtime() - t0 > p.watchdog_ticks, 0)) {
        raise_error(p, sh, MK_ETIMEOUT);
        return true;
      }
    }
    return false;
  }
};

// Wait until *flag >= target (LDS).  False if abandoned.  No wave reads the global
// error word here: the leader learns of other CUs' failures in its global polls (every
// wait also has its own time budget), and a global load issued from an LDS wait queues
// behind the CU's page loads (about 1 us), delaying the wait's end by as much when the
// flag flips meanwhile (1.3 us per step).
template <class S>
__device__ __forceinline__ bool wait_flag(const MkParams& p, MkShared<S>& sh, const int* flag, int target,
                                          bool leader) {
  if (lds_load(flag) >= target) { compiler_fence(); return true; }
  Waiter<S> wt(false);
  while (lds_load(flag) < target)
    if (wt.tick(p, sh, !leader)) return false;
  compiler_fence();
  return true;
}

template <class S>
__device__ __forceinline__ bool wait_all_done(const MkParams& p, MkShared<S>& sh, int target, bool leader) {
  static_assert(MK_NC == 4, "two 8-byte reads of the flags");
  // Usually all done already: two LDS reads instead of four round trips.
  const u64 d01 = __hip_atomic_load((const u64*)&sh.done[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const u64 d23 = __hip_atomic_load((const u64*)&sh.done[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int m = min(min((int)(uint32_t)d01, (int)(uint32_t)(d01 >> 32)), min((int)(uint32_t)d23, (int)(uint32_t)(d23 >> 32)));
  if (m >= target) {
    compiler_fence();
    return true;
  }
  for (int w = 0; w < MK_NC; ++w)
    if (!wait_flag(p, sh, &sh.done[w], target, leader)) return false;
  return true;
}

// 16 bytes from global memory, marked non-temporal (streamed weights).
__device__ __forceinline__ uint4 ld_nt16(const char* a) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)a);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads gate/up page ipg of the instruction straight into registers, laid out as the
// loaders lay a page out in LDS (unit u of the page in hold[u]).
template <class S, int OP, int SEG>
__device__ __forceinline__ void load_hold(const Dec& d, int ipg, int lane, uint4 (&hold)[16]) {
  using R = RowGeo<SEG>;
  static_assert(R::USED == 16, "held pages are whole");
  const int rows = (OP == MK_OP_GATEUP ? 2 * d.n : d.n) - ipg * R::RPP;
  if constexpr (R::WIDE) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = u / R::KU, c = u % R::KU;
      const char* a = row_addr<S, OP>(d, ipg * R::RPP + (j < rows ? j : 0)) + c * 1024 + lane * 16;
      hold[u] = ld_nt16(a);
    }
  } else {
    const int jl = lane / R::LPR, cl = lane % R::LPR;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = u * R::RPU + jl;
      const char* a = row_addr<S, OP>(d, ipg * R::RPP + (j < rows ? j : 0)) + cl * 16;
      hold[u] = ld_nt16(a);
    }
  }
}



// ------------------------------------------------------------------ page ring
// The pages of the CU's whole list, in list order, are numbered k = 0, 1, ...; page k
// lives in ring slot k % NSLOT, is issued by loader wave k % MK_NL and consumed by
// compute wave k % MK_NC.  LDS flags: full[slot] = k + 1 once page k has landed,
// freed[slot] = k + 1 once its compute wave has read it.  NSLOT is a multiple of
// MK_NL, so the page a loader waits to be freed is one it issued itself.
__device__ __forceinline__ int first_of(int who, int base, int period) {
  return ((who - base) % period + period) % period;
}

// Loader wave l.  It publishes its pages in order, each once vmcnt shows it complete.
// Two pacing modes, chosen per page:
//  - demand: the page's instruction is staged, or about to be, so compute waves are (or
//    soon will be) waiting for it; keep up to DEPTH of the wave's pages in flight for
//    bandwidth.  A down chunk's pages count as such from the layer's gate/up staging on
//    (its chunks follow back to back; 538.4 vs 543.1 us per step, against from the
//    chunk's own staging), those of QKV, attention and O from the previous instruction's
//    staging (a further 0.9 us).
//  - prefetch: the page is for a later instruction; keep a single page in flight for the
//    whole CU (the two loaders take turns).  A CU's vector-memory requests are served in
//    order, so every poll of a dependency and every result store queues behind the bytes
//    this CU has in flight; while the CU is on the critical path (polling, publishing)
//    its queue must stay short.
// While it waits for a slot still in use it keeps publishing what it has in flight: a
// compute wave may be waiting for one of them.
template <class S>
__device__ __forceinline__ void loader_wave(const MkParams& p, MkShared<S>& sh, char* ring_base, cinstr_t list,
                                            int nins, const StepGeo& g, int l, int lane) {
  constexpr int NSLOT = Ring<S>::NSLOT;
  constexpr int MAXD = NSLOT / MK_NL < 4 ? NSLOT / MK_NL : 4;   // 16 loads per page, vmcnt <= 63
  const int DEPTH = p.demand_depth < 1 ? 1 : p.demand_depth > MAXD ? MAXD : p.demand_depth;
  const uint32_t ring = lds_addr(ring_base);
  int oldest = 0, pend = 0;   // own pages issued and not yet published: oldest, then every MK_NL-th
  int base = 0;
  auto publish_oldest = [&]() {
    if (lane == 0) lds_store(&sh.full[oldest % NSLOT], oldest + 1);
    oldest += MK_NL;
    --pend;
  };
  for (int i = 0; i < nins; ++i) {
    const Dec d = decode<S>(p, list[i], g);
    lane = opaque(lane);
    for (int pg = first_of(l, base, MK_NL); pg < d.np; pg += MK_NL) {
      const int k = base + pg;
      const int slot = k % NSLOT;
      // Slot still in use: publish own pages as they land (oldest first) while waiting.
      while (lds_load(&sh.freed[slot]) < k - NSLOT + 1) {
        if (pend == 0) {
          // nothing of this loader's in flight: the ring is full (traced: for how long)
          u64 t_idle = 0;
          if constexpr (S::TRACE) t_idle = __builtin_amdgcn_s_memrealtime();
          if (!wait_flag(p, sh, &sh.freed[slot], k - NSLOT + 1, false)) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // nothing may land in LDS after the wave has left
            return;
          }
          if constexpr (S::TRACE) {
            if (lane == 0 && i < p.trace_len)
              atomicAdd(&sh.tr[i][11], (uint32_t)(__builtin_amdgcn_s_memrealtime() - t_idle));
          }
          break;
        }
        wait_vmcnt((pend - 1) * 16);
        publish_oldest();
      }
      // Demand from: the layer's gate/up staged (down chunks), the previous instruction
      // staged (QKV, attention, O), the instruction itself staged (gate/up, LM head).  Where
      // pages are not held in registers (the 4096-wide shape, six ring pages) the earlier
      // points measured slower (3320 vs 3262 us per step): there, from its own staging.
      const int from = !hold_pages<S>() ? i + 1
                       : d.op == MK_OP_DOWN ? i - d.a
                       : (d.op == MK_OP_QKV || d.op == MK_OP_ATTN || d.op == MK_OP_O) ? i : i + 1;
      const bool demand = lds_load(&sh.act_seq) >= from;
      if (!demand && k > 0) {
        // Prefetch: own pages first (the other loader may be waiting for one), then the other
        // loader's page k - 1 must have landed (one page in flight per CU; two per CU measured
        // slower, 576-585 against 574 us).
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        while (pend > 0) publish_oldest();
        if (!wait_flag(p, sh, &sh.full[(k - 1) % NSLOT], k, false)) return;
      }
      if (pg == 0) trace_mark<S>(p, sh, i, 10, lane);   // the instruction's first ring page
      issue_page<S>(d, d.rp + pg, ring + (uint32_t)(slot * MK_PAGE_BYTES), lane);
      if (pend == 0) oldest = k;
      ++pend;
      const int depth = demand ? DEPTH : 1;
      while (pend >= depth) {   // the oldest is complete once at most (pend - 1) pages are outstanding
        wait_vmcnt((pend - 1) * 16);
        publish_oldest();
      }
    }
    base += d.np;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  while (pend > 0) publish_oldest();
}

// Page k for a compute wave, once it has landed (nullptr if the wait was abandoned).
// When tracing, the ticks spent waiting are added to `waited` (the wave's total for the
// instruction, recorded once at its end).
template <class S>
__device__ __forceinline__ const char* page_wait(const MkParams& p, MkShared<S>& sh, const char* ring_base, int k,
                                                 u64& waited) {
  const int slot = k % Ring<S>::NSLOT;
  if (S::TRACE && lds_load(&sh.full[slot]) < k + 1) {
    const u64 t0 = __builtin_amdgcn_s_memrealtime();
    if (!wait_flag(p, sh, &sh.full[slot], k + 1, false)) return nullptr;
    waited += (u64)__builtin_amdgcn_s_memrealtime() - t0;
  } else if (!wait_flag(p, sh, &sh.full[slot], k + 1, false)) {
    return nullptr;
  }
  return ring_base + slot * MK_PAGE_BYTES;
}
// The wave has finished reading page k: once its LDS reads have returned the loader
// may overwrite the slot.
template <class S>
__device__ __forceinline__ void page_free(MkShared<S>& sh, int k, int lane) {
  lds_fence();
  if (lane == 0) lds_store(&sh.freed[k % Ring<S>::NSLOT], k + 1);
}

// ------------------------------------------------------------------ compute waves
// Group-major index of a raw q/k/v row: [kv head][q heads of the group | k | v][hd].
template <class S>
__device__ __forceinline__ int qkv_index(int row) {
  if (row < S::NQ) {
    const int h = row / S::HD;
    return (h / S::HPG) * S::GRP + (h % S::HPG) * S::HD + (row % S::HD);
  }
  if (row < S::NQ + S::NKV) {
    const int r = row - S::NQ;
    return (r / S::HD) * S::GRP + S::HPG * S::HD + (r % S::HD);
  }
  const int r = row - S::NQ - S::NKV;
  return (r / S::HD) * S::GRP + (S::HPG + 1) * S::HD + (r % S::HD);
}

// The down chunk before the held ones: at its start waves 0 and 1 issue the loads of
// their held pages of the next chunk (16 per wave, which wait behind the CU's page
// stream), so its two ring pages go whole to waves 2 and 3 instead of being shared by the
// four waves (2 us per step faster).
template <class S>
__device__ __forceinline__ bool whole_pages_23(const Dec& d) {
  return hold_down<S>() && S::NCH >= 3 && MK_NC == 4 && d.op == MK_OP_DOWN && d.a == S::NCH - 3 && d.np == 2;
}

// One GEMV instruction on the wave's pages.  The lane's slice of the activation stays in
// registers for the whole instruction.  Per page: every row's partial dot product, one
// combined cross-lane reduction for all rows of the page, then the rows' epilogues run
// in parallel in the lanes that hold them.
template <class S, int SEG>
__device__ __forceinline__ bool gemv(const MkParams& p, MkShared<S>& sh, const char* ring_base, const Dec& d,
                                     const float* act, int base, int w, int lane, uint32_t epoch, u64* best,
                                     const uint4 (&hold)[16], int mode, u64& waited) {
  using R = RowGeo<SEG>;
  // The activation slice is kept in registers for rows of up to 4 KiB; longer rows read
  // it from LDS per unit (it would otherwise take 64 registers).
  constexpr bool AREG = R::KU <= 4;
  constexpr int AU = AREG ? R::KU : 1;
  float av[AU][8];
  if constexpr (AREG) {
#pragma unroll
    for (int u = 0; u < R::KU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        av[u][e] = act[(R::WIDE ? u * 512 + lane * 8 : (lane % R::LPR) * 8) + e];
  }
  const int rows_total = d.op == MK_OP_GATEUP ? 2 * d.n : d.n;
  const int l = d.layer;
  // Output row pr of the instruction (not gate/up), value v: store it (with the residual
  // or the earlier chunks' partial sums where the instruction has them).
  auto emit_row = [&](float v, int pr) {
    const int gr = d.r0 + pr * d.rs;
    if (d.op == MK_OP_QKV) {
      ll_store(p.ll_qkv + (size_t)l * S::NQKV + qkv_index<S>(gr), v, epoch);
    } else if (d.op == MK_OP_O) {
      ll_store(p.ll_x + (size_t)(2 * l + 1) * S::D + gr, sh.xres[0][pr] + v, epoch);
    } else if (d.op == MK_OP_DOWN) {
      if (d.a + 1 < S::NCH) {
        sh.dpart[d.a][pr] = v;
      } else {
        float acc2 = 0.f;
#pragma unroll
        for (int c = 0; c + 1 < S::NCH; ++c) acc2 += sh.dpart[c][pr];
        ll_store(p.ll_x + (size_t)(2 * l + 2) * S::D + gr, sh.xres[1][pr] + (acc2 + v), epoch);
      }
    } else {   // MK_OP_LMHEAD
      p.logits[gr] = v;
      const u64 key = amax_key(v, (uint32_t)gr);
      if (key > *best) *best = key;
    }
  };
  // Two ring pages and four compute waves (the O projection, the first down chunks): each
  // page is shared by two waves, one per pair of its rows, halving the time the
  // instruction spends on its critical path.
  if constexpr (MK_SPLIT_PAGES && AREG && R::WIDE && R::RPP == 4 && MK_NC == 4) {
    if ((d.op == MK_OP_O || (d.op == MK_OP_DOWN && !whole_pages_23<S>(d))) && d.np == 2 && d.rp == 0 && mode == 0) {
      constexpr int NSLOT = Ring<S>::NSLOT;
      const int pgi = w >> 1, h = w & 1, k = base + pgi;
      const char* page = page_wait<S>(p, sh, ring_base, k, waited);
      if (!page) return false;
      uint4 wv[2 * R::KU];
#pragma unroll
      for (int u = 0; u < 2 * R::KU; ++u) wv[u] = *(const uint4*)(page + (2 * h * R::KU + u) * 1024 + lane * 16);
      float acc[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < R::KU; ++u) a = dot8(wv[jj * R::KU + u], av[u], a);
        acc[jj] = a;
      }
      // the page's second reader frees it (the count is taken once this wave's reads of
      // the page have returned)
      lds_fence();
      int old = 0;
      if (lane == 0) old = atomicAdd(&sh.acnt[k % NSLOT], 1);
      const float v = reduce_rows<2, 64>(acc, lane);
      old = __builtin_amdgcn_readlane(old, 0);
      if (old == 1 && lane == 0) {
        sh.acnt[k % NSLOT] = 0;
        lds_store(&sh.freed[k % NSLOT], k + 1);
      }
      const int pr = pgi * d.rpp + 2 * h + (lane >> 5);
      if ((lane & 31) == 0 && pr < rows_total) emit_row(v, pr);
      return true;
    }
  }
  // One page: wv holds its units; ipg is its page in the instruction; kfree the ring page
  // to release once read (-1: a page held in registers).
  auto page_body = [&](const uint4 (&wv)[R::USED], int ipg, int kfree) {
    float acc[R::NV];
    if constexpr (R::WIDE && AREG) {
#pragma unroll
      for (int j = 0; j < R::RPP; ++j) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < R::KU; ++u)
          a = dot8(wv[j * R::KU + u], av[u], a);
        acc[j] = a;
      }
    } else if constexpr (R::WIDE) {
#pragma unroll
      for (int j = 0; j < R::RPP; ++j) acc[j] = 0.f;
#pragma unroll
      for (int u = 0; u < R::KU; ++u) {
        const float4 x0 = *(const float4*)(act + u * 512 + lane * 8);
        const float4 x1 = *(const float4*)(act + u * 512 + lane * 8 + 4);
        const float a[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int j = 0; j < R::RPP; ++j) acc[j] = dot8(wv[j * R::KU + u], a, acc[j]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u] = dot8(wv[u], av[0], 0.f);
    }
    if (kfree >= 0) page_free<S>(sh, kfree, lane);
    const float v = reduce_rows<R::NV, R::G>(acc, lane);
    // The row this lane holds, relative to the page, and whether the lane stores it.
    constexpr int SPAN = R::G / R::NV;                        // lanes holding one value
    const int vi = (lane % R::G) / SPAN;                      // value index
    const int j = R::WIDE ? vi : vi * R::RPU + lane / R::LPR;  // row in the page
    const bool owner = (lane % SPAN) == 0;
    const int pr = ipg * d.rpp + j;                            // row of the instruction
    const bool valid = owner && pr < rows_total;
    if (d.op == MK_OP_GATEUP) {
      constexpr int UP = R::WIDE ? SPAN : R::LPR;             // lane distance gate row -> up row
      float up;
      if constexpr (UP == 16) up = xor16(v, lane);   // gate rows sit in the lanes below their up row
      else if constexpr (UP == 32) up = xor32(v, lane);
      else up = __shfl_down(v, UP);
      if (valid && (pr & 1) == 0) {
        const float a = (v / (1.0f + __expf(-v))) * up;
        ll_store(p.ll_a + (size_t)l * S::F + gu_feature<S>(d, pr >> 1), a, epoch);
      }
    } else if (valid) {
      emit_row(v, pr);
    }
  };
  // mode 0: the held page (if this wave holds one) and the ring pages; 1: only the held
  // page; 2: only the ring pages.
  if constexpr (R::USED == 16) {
    if (mode != 2 && w >= d.rw && w < d.rw + d.rp) page_body(hold, w - d.rw, -1);
  }
  if (mode == 1) return true;
  for (int pg = whole_pages_23<S>(d) ? (w >= 2 ? w - 2 : d.np) : first_of(w, base, MK_NC); pg < d.np; pg += MK_NC) {
    const char* page = page_wait<S>(p, sh, ring_base, base + pg, waited);
    if (!page) return false;
    uint4 wv[R::USED];
#pragma unroll
    for (int u = 0; u < R::USED; ++u) wv[u] = *(const uint4*)(page + u * 1024 + lane * 16);
    page_body(wv, d.rp + pg, base + pg);
  }
  return true;
}

template <class S>
__device__ __forceinline__ size_t part_index(const MkParams& p, int l, int g, int h, int s) {
  return ((((size_t)l * S::HKV + g) * S::HPG + h) * p.s_max + s) * (size_t)(S::HD + 2);
}

// ------------------------------------------------------------------ attention
// Short contexts (one split, q-head mode): item (g, b) is query head b of KV group g and
// the four compute waves split the keys.  Several splits: the matrix units (attn_run_mma:
// each wave 16 keys of its pages for all heads).  Shapes the matrix-unit form does not
// cover keep the VALU one: compute wave w handles query head h = w % HPG of the item's KV group over the key
// subset t = w / HPG (pages t, t + NSUB, ... of the split; NSUB = MK_NC / HPG): with four
// query heads per KV head every wave sees every page and owns its head outright, so no
// cross-wave merge is needed.  Each page is read by HPG waves and freed by the last.
template <int HD>
struct HeadState {
  float q[8];        // dims 8c.. of the head, c = lane % (HD / 8)
  float m, l;        // running max and denominator over the lane's positions
  float o[8];        // running numerator for the lane's dims
};

// One page of cached keys/values: [npos][HD] keys, then [npos][HD] values.  Lane l holds
// 8 dims (chunk l % LPP) of position l / LPP of each 1 KiB unit.  Every byte of a page
// is a copy of an attended cache row (the loader re-reads valid rows past the payload),
// so all key and value units are read unconditionally and positions past npos only get
// a zero weight: no branches, and the value reads overlap the score arithmetic.
//
// The wave takes units u0, u0 + USTEP, ... of the page (USTEP = 1: all of them); with
// NP > 1, of each of NP pages at once (one running-max update for all of them).
template <int HD, int USTEP, int NP = 1>
__device__ __forceinline__ void head_page(HeadState<HD>& st, const char* const (&pages)[NP], const int (&nposv)[NP],
                                          float scale, int lane, int u0) {
  constexpr int LPP = HD / 8;          // lanes per position
  constexpr int PPU = 64 / LPP;        // positions per 1 KiB unit
  constexpr int MAXU = 8 / USTEP;      // units per key block (16 KiB page) for this wave
  constexpr int NU = NP * MAXU;
  const int jl = lane / LPP;
  uint4 kw[NU], vw[NU];
#pragma unroll
  for (int pi = 0; pi < NP; ++pi)
#pragma unroll
    for (int u = 0; u < MAXU; ++u) kw[pi * MAXU + u] = *(const uint4*)(pages[pi] + (u0 + u * USTEP) * 1024 + lane * 16);
#pragma unroll
  for (int pi = 0; pi < NP; ++pi)
#pragma unroll
    for (int u = 0; u < MAXU; ++u)
      vw[pi * MAXU + u] = *(const uint4*)(pages[pi] + nposv[pi] * HD * 2 + (u0 + u * USTEP) * 1024 + lane * 16);
  float s[NU];
#pragma unroll
  for (int pi = 0; pi < NP; ++pi)
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
      float part = dot8(kw[pi * MAXU + u], st.q, 0.f);
      part = LPP == 8 ? sum8(part) : sum16(part);
      s[pi * MAXU + u] = (u0 + u * USTEP) * PPU + jl < nposv[pi] ? part * scale : -INFINITY;
    }
  float pm = s[0];
#pragma unroll
  for (int u = 1; u < NU; ++u) pm = fmaxf(pm, s[u]);
  pm = wave_max(pm);
  const float mn = fmaxf(st.m, pm);
  const float alpha = st.m == -INFINITY ? 0.f : __expf(st.m - mn);
  // -inf only while the wave has seen no position at all (a unit subset past npos)
  const float mref = mn == -INFINITY ? 0.f : mn;
  st.m = mn;
  st.l *= alpha;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] *= alpha;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const float pr = __expf(s[u] - mref);   // exactly 0 for positions past npos
    st.l += pr;
    st.o[0] = fmaf(pr, bf_lo(vw[u].x), st.o[0]);
    st.o[1] = fmaf(pr, bf_hi(vw[u].x), st.o[1]);
    st.o[2] = fmaf(pr, bf_lo(vw[u].y), st.o[2]);
    st.o[3] = fmaf(pr, bf_hi(vw[u].y), st.o[3]);
    st.o[4] = fmaf(pr, bf_lo(vw[u].z), st.o[4]);
    st.o[5] = fmaf(pr, bf_hi(vw[u].z), st.o[5]);
    st.o[6] = fmaf(pr, bf_lo(vw[u].w), st.o[6]);
    st.o[7] = fmaf(pr, bf_hi(vw[u].w), st.o[7]);
  }
}

// Where the key subsets' partials of an attention item live (the item's activation slot
// or the LDS array): [subset][head][m, l, o[HD]].
template <class S>
__device__ __forceinline__ float* part_base(MkShared<S>& sh, const float* act) {
  if constexpr (AttnGeo<S>::IN_ACT) return const_cast<float*>(act) + AttnGeo<S>::OFF;
  else return sh.part;
}

// Attention over the item's cached keys on the matrix units (several splits): a wave takes
// 16 keys of a page for all of the group's query heads, so each K/V element is unpacked
// once per CU instead of once per head (head_dim 64: 64 keys per page, wave w keys 16w..
// of every page; head_dim 128: 32 keys per page, waves 0-1 the even pages and 2-3 the
// odd ones, 16 keys each).  Per page:
//   S = K q   (16 keys x 16 head columns, 16x16x32 bf16 products; q is split into three
//              bf16 parts hi + mid + lo, exact to ~2^-24, so the scores keep fp32
//              accuracy: with two parts (~16 bits), errors the score's size amplifies
//              let the 32-layer 8B shape's appended K/V drift past the fp32 bound),
//   an online softmax per head over the wave's keys (its running max is shared by the
//   four lanes of a column),
//   O += P V  (16 heads x hd dims as hd/16 16x16x16 bf16 products; P in [0, 1] is split
//              into bf16 hi + lo, ~2^-17, which keeps that bound; a third part cost
//              ~3 us per step at context 8192).
// Operand layouts (lane l, c = l % 16, g = l / 16): A[row c][k 8g..] (16x16x32) or
// [row c][k 4g..] (16x16x16); B[k ...][column c]; C/D[rows 4g..4g+3][column c].  The
// scores' C layout (key 4g + i, head c) is exactly the A layout P needs (head c, key
// 4g + j), so P goes from softmax to the product without moving.  Columns c >= HPG are
// padding (q = 0, P = 0).  The waves' partials meet in LDS; then wave h folds head h's
// with the current key and publishes the split's (m, l, o) for that head.
template <class S>
__device__ __forceinline__ bool attn_run_mma(const MkParams& p, MkShared<S>& sh, const char* ring_base, const Dec& d,
                                             const StepGeo& sg, const float* act, int base, int w, int lane,
                                             uint32_t epoch, int& nmma, u64& waited) {
  constexpr int HD = S::HD, HPG = S::HPG, NSLOT = Ring<S>::NSLOT;
  constexpr int KB = HD / 32, NT = HD / 16;                 // 32-dim blocks of S, 16-dim tiles of O
  constexpr int WPP = S::PPP / 16, STR = MK_NC / WPP;       // waves per page, page stride per wave
  static_assert(AttnGeo<S>::MMA && MK_NC == 4, "matrix-unit attention shape");
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int c = lane & 15, g = lane >> 4;
  // q as B: column c = head, k = dims 8g + 32kk + e (padding columns read head 0's q and
  // take zeros)
  bf16x8 qh[KB], qm[KB], ql[KB];
  const float* qc = act + (c < HPG ? c : 0) * HD + 8 * g;
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
    const float4 x0 = *(const float4*)(qc + 32 * kk), x1 = *(const float4*)(qc + 32 * kk + 4);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = c < HPG ? xs[e] : 0.f;
      const uint32_t xb = __float_as_uint(x);
      const float r1 = x - __uint_as_float(xb & 0xffff0000u);
      const uint32_t rb = __float_as_uint(r1);
      qh[kk][e] = __builtin_bit_cast(__bf16, (uint16_t)(xb >> 16));
      qm[kk][e] = __builtin_bit_cast(__bf16, (uint16_t)(rb >> 16));
      ql[kk][e] = __builtin_bit_cast(__bf16, f2bf_finite(r1 - __uint_as_float(rb & 0xffff0000u)));
    }
  }
  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;   // running max of head c; this lane's part of its denominator
  int prev_k = -1, prev_old = 0;
  auto release_prev = [&]() {
    if (prev_k >= 0) {
      const int old = __builtin_amdgcn_readlane(prev_old, 0);   // lane 0's count, no LDS trip
      if (old == WPP - 1 && lane == 0) {
        sh.acnt[prev_k % NSLOT] = 0;
        lds_store(&sh.freed[prev_k % NSLOT], prev_k + 1);
      }
      prev_k = -1;
    }
  };
  const int kw = 16 * (w % WPP);        // the wave's first key in each of its pages
  const int kr = kw + c;                // the key row this lane loads for A = K
  const int vr = kw + 4 * g;            // first of the four key rows it loads for B = V
  for (int pg = w / WPP; pg < d.np; pg += STR) {
    const int k = base + pg;
    const char* page = page_wait<S>(p, sh, ring_base, k, waited);
    if (!page) return false;
    const int npos = min(S::PPP, d.ce - (d.j0 + pg * S::PPP));
    // keys [npos][HD], then values [npos][HD]; rows past npos hold copies of cached rows
    bf16x8 kb[KB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) kb[kk] = *(const bf16x8*)(page + kr * (HD * 2) + g * 16 + kk * 64);
    const char* vb = page + npos * (HD * 2) + vr * (HD * 2) + c * 2;
    i16x4 vv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) vv[nt][j] = *(const short*)(vb + j * (HD * 2) + nt * 32);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qh[kk], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qm[kk], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], ql[kk], sc, 0, 0, 0);
    }
    float sv[4], pm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = vr + i < npos ? sc[i] * p.attn_scale : -INFINITY;
      pm = fmaxf(pm, sv[i]);
    }
    pm = fmaxf(pm, xor16(pm, lane));
    pm = fmaxf(pm, xor32(pm, lane));
    const float mn = fmaxf(m, pm);
    const float alpha = m == -INFINITY ? 0.f : __expf(m - mn);
    const float mref = mn == -INFINITY ? 0.f : mn;   // -inf only while no key has been seen
    m = mn;
    i16x4 ph, pl;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pr = c < HPG ? __expf(sv[j] - mref) : 0.f;   // 0 for keys past npos
      ps += pr;
      const uint32_t pb = __float_as_uint(pr);
      ph[j] = (short)(pb >> 16);
      pl[j] = (short)f2bf_finite(pr - __uint_as_float(pb & 0xffff0000u));
    }
    lsum = fmaf(lsum, alpha, ps);
    // O's rows 4g + i are heads; heads 0..3 sit in lanes 0..15 (g = 0), and head h's
    // factor is alpha of column h
    float ah[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ah[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= ah[i];
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vv[nt], o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vv[nt], o[nt], 0, 0, 0);
    }
    // the page's last reader frees it (its count examined one page later)
    release_prev();
    int old = 0;
    if (lane == 0) old = atomicAdd(&sh.acnt[k % NSLOT], 1);
    prev_k = k;
    prev_old = old;
  }
  release_prev();
  // head c's denominator: the four lanes of column c
  float L = lsum + xor16(lsum, lane);
  L += xor32(L, lane);
  float* part = part_base<S>(sh, act) + w * HPG * (HD + 2);
  if (g == 0 && c < HPG) {
    part[c * (HD + 2)] = m;
    part[c * (HD + 2) + 1] = L;
  }
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < HPG; ++i) part[i * (HD + 2) + 2 + 16 * nt + c] = o[nt][i];
  }
  // Once every wave's partials are in, wave h folds head h's four with the current key
  // and publishes the split's (m, l, o) of that head (the heads in parallel, not one
  // after another on the leader).
  lds_fence();
  if (lane == 0) __hip_atomic_fetch_add(&sh.pcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  ++nmma;
  if (!wait_flag(p, sh, &sh.pcnt, MK_NC * nmma, false)) return false;
  if (w < HPG) {
    constexpr int E = HD / 64, STRIDE = HD + 2;
    const int h = w;
    const float* pb = part_base<S>(sh, act);
    float mw[MK_NC], lw[MK_NC], ow[MK_NC][E];
#pragma unroll
    for (int t = 0; t < MK_NC; ++t) {
      const float* q = pb + (t * HPG + h) * STRIDE;
      mw[t] = q[0];
      lw[t] = q[1];
#pragma unroll
      for (int cc = 0; cc < E; ++cc) ow[t][cc] = q[2 + cc * 64 + lane];
    }
    const bool has_pos = d.b == sg.s_eff - 1;
    float sp = -INFINITY;
    if (has_pos) {
      float a = 0.f;
#pragma unroll
      for (int cc = 0; cc < E; ++cc) a = fmaf(act[h * HD + cc * 64 + lane], act[HPG * HD + cc * 64 + lane], a);
      sp = wave_sum(a) * p.attn_scale;
    }
    float M = sp;
#pragma unroll
    for (int t = 0; t < MK_NC; ++t) M = fmaxf(M, mw[t]);
    float Lt = 0.f, wt[MK_NC];
#pragma unroll
    for (int t = 0; t < MK_NC; ++t) {
      wt[t] = mw[t] == -INFINITY ? 0.f : __expf(mw[t] - M);
      Lt = fmaf(lw[t], wt[t], Lt);
    }
    const float wp = has_pos ? __expf(sp - M) : 0.f;
    Lt += wp;
    u64* dst = p.ll_part + part_index<S>(p, d.layer, d.a, h, d.b);
#pragma unroll
    for (int cc = 0; cc < E; ++cc) {
      float oo = wp * act[(HPG + 1) * HD + cc * 64 + lane];
#pragma unroll
      for (int t = 0; t < MK_NC; ++t) oo = fmaf(ow[t][cc], wt[t], oo);
      ll_store(dst + 2 + cc * 64 + lane, oo, epoch);
    }
    if (lane < 2) ll_store(dst + lane, lane ? Lt : M, epoch);
  }
  return true;
}

// The item's cached keys for one head, then (one head per wave) the current position's
// key and value, and the result: o / l into the attention output (one split) or the
// split's (m, l, o) words; with several waves per head the partial goes to LDS and the
// leader combines it.
template <class S>
__device__ __forceinline__ bool attn_run(const MkParams& p, MkShared<S>& sh, const char* ring_base, const Dec& d,
                                         const StepGeo& g, const float* act, int base, int w, int lane,
                                         uint32_t epoch, int& nmma, u64& waited) {
  constexpr int HD = S::HD, HPG = S::HPG, LPP = HD / 8, NSUB = MK_NC / HPG, NSLOT = Ring<S>::NSLOT;
  if constexpr (AttnGeo<S>::MMA) {
    if (!g.qh) return attn_run_mma<S>(p, sh, ring_base, d, g, act, base, w, lane, epoch, nmma, waited);
  }
  // q-head mode: head d.b of the group; every wave reads every page and takes units
  // w, w + MK_NC of it.  Otherwise one head per wave (w % HPG) over pages t, t + NSUB, ...
  const bool qh = g.qh;
  const int h = qh ? d.b : w % HPG, t = w / HPG, c = lane % LPP;
  const int readers = qh ? MK_NC : HPG;
  HeadState<HD> st;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    st.q[e] = act[h * HD + c * 8 + e];
    st.o[e] = 0.f;
  }
  st.m = -INFINITY;
  st.l = 0.f;
  // The page's last reader frees it.  The count's returned value is examined one page
  // later (or after the loop), so the wave does not wait for the LDS atomic's round trip
  // on every page; LDS operations of a wave complete in order, so the count is taken
  // after this wave's reads of the page.
  int prev_k = -1, prev_old = 0;
  auto release_prev = [&]() {
    if (prev_k >= 0) {
      const int old = __builtin_amdgcn_readlane(prev_old, 0);   // lane 0's count, no LDS trip
      if (old == readers - 1 && lane == 0) {
        sh.acnt[prev_k % NSLOT] = 0;
        lds_store(&sh.freed[prev_k % NSLOT], prev_k + 1);
      }
      prev_k = -1;
    }
  };
  for (int pg = qh ? 0 : t; pg < d.np;) {
    const int k = base + pg;
    const char* page = page_wait<S>(p, sh, ring_base, k, waited);
    if (!page) return false;
    const int npos = min(S::PPP, d.ce - (d.j0 + pg * S::PPP));
    if (qh && pg + 1 < d.np) {
      // q-head mode: two pages at a time (one running-max update for both)
      const char* page2 = page_wait<S>(p, sh, ring_base, k + 1, waited);
      if (!page2) return false;
      const char* const pp[2] = {page, page2};
      const int nn[2] = {npos, min(S::PPP, d.ce - (d.j0 + (pg + 1) * S::PPP))};
      head_page<HD, MK_NC, 2>(st, pp, nn, p.attn_scale, lane, w);
      release_prev();
      int old = 0, old2 = 0;
      if (lane == 0) {
        old = atomicAdd(&sh.acnt[k % NSLOT], 1);
        old2 = atomicAdd(&sh.acnt[(k + 1) % NSLOT], 1);
      }
      prev_k = k;
      prev_old = old;
      release_prev();
      prev_k = k + 1;
      prev_old = old2;
      pg += 2;
      continue;
    }
    const char* const pp[1] = {page};
    const int nn[1] = {npos};
    if (qh)
      head_page<HD, MK_NC>(st, pp, nn, p.attn_scale, lane, w);
    else
      head_page<HD, 1>(st, pp, nn, p.attn_scale, lane, 0);
    release_prev();
    int old = 0;
    if (lane == 0) old = atomicAdd(&sh.acnt[k % NSLOT], 1);
    prev_k = k;
    prev_old = old;
    pg += qh ? 1 : NSUB;
  }
  release_prev();
  // Sum over the lanes holding other positions (same dims), halving the values at each
  // step: the lanes at distance 32, then 16 (then 8, hd 64) trade half of their dims and
  // add (lane swaps and one DPP move, instead of all nine values at every step).  Lane l
  // then holds the NE = 8 / (positions per unit) dims dim(l) + j, j < NE.
  constexpr int NE = LPP == 8 ? 1 : 2;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = st.o[e];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = swap_sum32(v[e], v[e + 4]);   // dim e + 4 * b5
#pragma unroll
  for (int e = 0; e < 2; ++e) v[e] = swap_sum16(v[e], v[e + 2]);   // dim e + 2 * b4 + 4 * b5
  float L = st.l;
  if constexpr (LPP == 8) {
    const uint32_t m8 = (lane & 8) ? 0xffffffffu : 0u;
    const uint32_t a = __float_as_uint(v[0]), b = __float_as_uint(v[1]);
    v[0] = __uint_as_float((b & m8) | (a & ~m8)) + xor_lane<8>(__uint_as_float((a & m8) | (b & ~m8)), lane);
    L += xor_lane<8>(L, lane);
  }
  L = swap_sum16(L, L);
  L = swap_sum32(L, L);
  const int dim = LPP == 8 ? c * 8 + (lane >> 3) : c * 8 + 2 * (lane >> 4);
  if (qh || NSUB > 1) {
    // partial (m, l, o) for the leader; q-head mode: one slot per wave
    float* part = qh ? sh.part + w * (HD + 2) : part_base<S>(sh, act) + (t * HPG + h) * (HD + 2);
#pragma unroll
    for (int j = 0; j < NE; ++j) part[2 + dim + j] = v[j];
    if (lane == 0) {
      part[0] = st.m;
      part[1] = L;
    }
    return true;
  }
  // One head per wave: fold in the current position (its key is not in the cache yet).
  const int s = d.b;
  const bool has_pos = s == g.s_eff - 1;
  float M = st.m;
  if (has_pos) {
    float sc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sc = fmaf(st.q[e], act[HPG * HD + c * 8 + e], sc);
    sc = (LPP == 8 ? sum8(sc) : sum16(sc)) * p.attn_scale;
    const float Mn = fmaxf(M, sc);
    const float a = M == -INFINITY ? 0.f : __expf(M - Mn);
    const float b = __expf(sc - Mn);
    L = L * a + b;
#pragma unroll
    for (int j = 0; j < NE; ++j) v[j] = fmaf(v[j], a, b * act[(HPG + 1) * HD + dim + j]);
    M = Mn;
  }
  // every lane stores its dims: one full line per store instruction
  const int l = d.layer, gi = d.a;
  if (g.s_eff == 1) {
    u64* dst = p.ll_o + (size_t)l * S::NQ + (gi * HPG + h) * HD + dim;
#pragma unroll
    for (int j = 0; j < NE; ++j) ll_store(dst + j, v[j] / L, epoch);
  } else {
    u64* dst = p.ll_part + part_index<S>(p, l, gi, h, s);
#pragma unroll
    for (int j = 0; j < NE; ++j) ll_store(dst + 2 + dim + j, v[j], epoch);
    if (lane == 0) {
      ll_store(dst, M, epoch);
      ll_store(dst + 1, L, epoch);
    }
  }
  return true;
}

template <class S>
__device__ __forceinline__ void compute_wave(const MkParams& p, MkShared<S>& sh, const char* ring_base, cinstr_t list,
                                             int nins, const StepGeo& g, int w, int lane, uint32_t epoch) {
  int base = 0;   // ring number of the instruction's first page
  u64 best = 0;
  int nmma = 0;   // matrix-unit attention items done (their partial count in LDS)
  // Held pages.  Each compute wave keeps one weight page in registers (64 VGPRs), loaded
  // ahead of its instruction with plain non-temporal loads; the loaders skip those pages,
  // so the LDS ring reaches that much further ahead.  Per layer a wave holds its gate/up
  // page, loaded when it reaches the layer's O projection (the ring is full while the CU
  // waits for attention and the O inputs, so four more pages per CU stream during that
  // wait), and then a page of one of the last two down chunks, loaded when it reaches the
  // chunk before that one (those pages would otherwise stream only after the first chunks').
  // hold_for: the instruction whose page `hold` holds.
  uint4 hold[16];
  int hold_for = -1;
  auto holds = [&](const Dec& x) { return x.rp > 0 && w >= x.rw && w < x.rw + x.rp; };
  auto load_held = [&](const Dec& x, int j) {
    if (x.op == MK_OP_GATEUP)
      load_hold<S, MK_OP_GATEUP, 2 * S::D>(x, w - x.rw, lane, hold);
    else if constexpr (hold_down<S>())
      load_hold<S, MK_OP_DOWN, 2 * S::KC>(x, w - x.rw, lane, hold);
    hold_for = j;
  };
  for (int i = 0; i < nins; ++i) {
    const Dec d = decode<S>(p, list[i], g);
    lane = opaque(lane);
    if (hold_pages<S>() && d.op == MK_OP_O) {
      // the wave has reached the layer's O projection; its GATEUP follows.  (Issued at the
      // layer's start, while the CU polls for x, the loads slowed that poll; issued after
      // QKV, they were 4 us per step slower than here.)
      for (int j = i; j < i + 3 && j < nins; ++j) {
        const MkInstr r = list[j];
        if (r.op == MK_OP_GATEUP) {
          const Dec dg = decode<S>(p, r, g);
          if (holds(dg)) load_held(dg, j);
          break;
        }
      }
    }
    if constexpr (hold_down<S>()) {
      if (d.op == MK_OP_DOWN) {
        // a held page of the next down chunk, loaded one chunk ahead: loaded at the first
        // chunk, the 64 KiB per CU were in flight while the CU polled the next two chunks'
        // inputs, and those polls queued behind them (14 us per step slower)
        for (int j = i + 1; j < i + 2 && j < nins; ++j) {
          const MkInstr r = list[j];
          if (r.op != MK_OP_DOWN) break;
          const Dec dd = decode<S>(p, r, g);
          if (holds(dd)) {
            load_held(dd, j);
            break;
          }
        }
      }
    }
    if (hold_pages<S>() && holds(d) && hold_for != i) load_held(d, i);   // not loaded ahead
    if (!wait_flag(p, sh, &sh.act_seq, i + 1, false)) return;
    // The last down chunk adds the partial sums of the earlier chunks, which any wave
    // may have produced: wait until every wave has finished the previous instruction.
    if (S::NCH > 1 && d.op == MK_OP_DOWN && d.a + 1 == S::NCH && !wait_all_done(p, sh, i, false)) return;
    if (w == 0) trace_mark<S>(p, sh, i, 5, lane);
    const float* act = sh.act[i % MK_NACT];
    bool ok = true;
    u64 waited = 0;
    if (d.op == MK_OP_ATTN) {
      if (attn_active(g, d.b, S::HPG)) ok = attn_run<S>(p, sh, ring_base, d, g, act, base, w, lane, epoch, nmma, waited);
    } else if constexpr (S::NQ == S::D && S::KC == S::D) {
      // every matrix-vector instruction has rows of the same length: one copy of the code
      // (the instruction cache holds the kernel's hot code better that way)
      ok = gemv<S, 2 * S::D>(p, sh, ring_base, d, act, base, w, lane, epoch, &best, hold, 0, waited);
    } else if (d.op == MK_OP_O) {
      ok = gemv<S, 2 * S::NQ>(p, sh, ring_base, d, act, base, w, lane, epoch, &best, hold, 0, waited);
    } else if (d.op == MK_OP_DOWN) {
      ok = gemv<S, 2 * S::KC>(p, sh, ring_base, d, act, base, w, lane, epoch, &best, hold, 0, waited);
    } else {
      ok = gemv<S, 2 * S::D>(p, sh, ring_base, d, act, base, w, lane, epoch, &best, hold, 0, waited);
    }
    if (!ok) return;
    if constexpr (S::TRACE) {
      if (waited && lane == 0 && i < p.trace_len) atomicAdd(&sh.tr[i][9], (uint32_t)waited);
    }
    if (d.op == MK_OP_LMHEAD) {
      const u64 b = wave_max_u64(best);
      if (lane == 0) sh.amax[w] = b;
    }
    base += d.np;
    trace_max<S>(p, sh, i, 6, lane);   // before the done flag: the leader writes the trace out after it
    lds_fence();
    if (lane == 0) lds_store(&sh.done[w], i + 1);
  }
}

// ------------------------------------------------------------------ leader wave
// Poll NW words per lane (word k*64 + lane of src lands in wv[k]) until all carry this
// step's epoch.  The first pass loads every word; while words are missing, a single
// lane re-polls one missing word (one load per wave per round trip) and the wave
// reloads the whole batch once it has arrived, up to five times back to back (the
// other producers' words usually land within those round trips; 2 % faster per step
// than a single reload).  Every CU polls the same few words, so probe traffic is kept
// to a minimum: re-polling every missing word each round was measured 25 % slower per
// step, one word per lane (64 per wave) 4.5 % slower than this, eight lanes 2.5 %.
// A later load of a location never returns an older value than an earlier one, and each
// word is written once per step.
template <class S, int NW>
__device__ __forceinline__ bool poll(const MkParams& p, MkShared<S>& sh, const u64* src, u64 (&wv)[NW],
                                     uint32_t epoch, int lane) {
  const u64* q = src + lane;
#pragma unroll
  for (int k = 0; k < NW; ++k) wv[k] = ll_load(q + k * 64);
  bool all = true;
#pragma unroll
  for (int k = 0; k < NW; ++k) all = all && ll_ok(wv[k], epoch);
  if (__ballot(!all) == 0) return true;
  Waiter<S> wt(true);
  for (;;) {
    if (wt.tick(p, sh)) return false;
    int first_bad = NW;
#pragma unroll
    for (int k = NW - 1; k >= 0; --k) first_bad = ll_ok(wv[k], epoch) ? first_bad : k;
    // One probing lane per wave: the lowest lane still missing a word.
    const u64 bal = __ballot(first_bad < NW);
    const int pl = bal ? __builtin_ctzll(bal) : 0;
    u64 s = 0;
    if (lane == pl) s = ll_load(q + first_bad * 64);
    if (__ballot(lane == pl && ll_ok(s, epoch)) != 0) {
      // The producers' words land within a short window: reload the batch back to back
      // a few times before going back to a single probe.
      for (int rep = 0; rep < 5; ++rep) {
#pragma unroll
        for (int k = 0; k < NW; ++k) wv[k] = ll_load(q + k * 64);
        all = true;
#pragma unroll
        for (int k = 0; k < NW; ++k) all = all && ll_ok(wv[k], epoch);
        if (__ballot(!all) == 0) return true;
      }
    }
  }
}

// Wait until slot i % MK_NACT of the activation ring may be overwritten: every compute
// wave has finished instruction i - MK_NACT.
template <class S>
__device__ __forceinline__ bool slot_free(const MkParams& p, MkShared<S>& sh, int i) {
  return i < MK_NACT || wait_all_done(p, sh, i - MK_NACT + 1, true);
}

// RMSNorm staging: act = x * (1 / sqrt(mean(x^2) + eps)) * g, with x the residual
// stream (the embedding row for the first layer).  Up to 2048 values stay in registers
// between the sum of squares and the scaled write; longer vectors are written raw in
// batches and normalised in place.
template <class S>
__device__ __forceinline__ bool stage_norm(const MkParams& p, MkShared<S>& sh, const u64* src, const uint16_t* gain,
                                           int i, uint32_t epoch, int lane) {
  constexpr int NW = S::D / 64;
  constexpr int BW = NW < 32 ? NW : 32;   // words per lane per batch
  // Gain of element k*64 + lane, loaded into this lane before the poll (one 16-bit load
  // per element, so no cross-lane exchange afterwards).  Rows wider than one batch load
  // their gains in the normalising pass instead (registers).
  constexpr int NGV = NW > BW ? 1 : NW;
  uint32_t gv[NGV];
  if constexpr (NW <= BW) {
#pragma unroll
    for (int k = 0; k < NW; ++k) gv[k] = gain[k * 64 + lane];
#pragma unroll
    for (int k = 0; k < NW; ++k) pin(gv[k]);
  }
  trace_mark<S>(p, sh, i, 1, lane);
  float* act = sh.act[i % MK_NACT];
  float ss = 0.f;
  float xv[BW];
  for (int b = 0; b < NW; b += BW) {
    if (src == nullptr) {
      const uint16_t* e = p.embed + (size_t)sh.token * S::D + b * 64;
      uint32_t eb[BW];
#pragma unroll
      for (int k = 0; k < BW; ++k) eb[k] = e[k * 64 + lane];
#pragma unroll
      for (int k = 0; k < BW; ++k) pin(eb[k]);
#pragma unroll
      for (int k = 0; k < BW; ++k) xv[k] = bf16f((uint16_t)eb[k]);
    } else {
      u64 wv[BW];
      if (!poll<S, BW>(p, sh, src + b * 64, wv, epoch, lane)) return false;
#pragma unroll
      for (int k = 0; k < BW; ++k) xv[k] = ll_val(wv[k]);
    }
#pragma unroll
    for (int k = 0; k < BW; ++k) ss = fmaf(xv[k], xv[k], ss);
    if constexpr (NW > BW) {   // raw batch into the slot; normalised below
      if (b == 0 && !slot_free(p, sh, i)) return false;
#pragma unroll
      for (int k = 0; k < BW; ++k) act[(b + k) * 64 + lane] = xv[k];
    }
  }
  trace_mark<S>(p, sh, i, 2, lane);
  const float rinv = 1.0f / sqrtf(wave_sum(ss) / (float)S::D + p.eps);
  if constexpr (NW > BW) {
    lds_fence();
    trace_mark<S>(p, sh, i, 3, lane);
#pragma unroll
    for (int k = 0; k < NW; ++k) act[k * 64 + lane] = (act[k * 64 + lane] * rinv) * bf16f(gain[k * 64 + lane]);
  } else {
    if (!slot_free(p, sh, i)) return false;
    trace_mark<S>(p, sh, i, 3, lane);
#pragma unroll
    for (int k = 0; k < NW; ++k) act[k * 64 + lane] = (xv[k] * rinv) * bf16f((uint16_t)gv[k]);
  }
  return true;
}

template <class S, int N>
__device__ __forceinline__ bool stage_raw(const MkParams& p, MkShared<S>& sh, const u64* src, int i, uint32_t epoch,
                                          int lane, const u64* xrow = nullptr, const uint16_t* erow = nullptr,
                                          int xn = 0, int which = 0) {
  constexpr int NW = N / 64;
  // Residual rows of x for the instruction's epilogue (xres[which]), when it has one:
  // from the link words (produced long before this instruction's inputs) or from the
  // embedding row; loaded alongside the poll so that they cost no extra round trip.
  const bool has_x = lane < xn;
  u64 xr = 0;
  float ev = 0.f;
  if (xrow && has_x) xr = ll_load(xrow + lane);
  if (erow && has_x) ev = bf16f(erow[lane]);
  u64 wv[NW];
  trace_mark<S>(p, sh, i, 1, lane);
  if (!poll<S, NW>(p, sh, src, wv, epoch, lane)) return false;
  trace_mark<S>(p, sh, i, 2, lane);
  if (xrow) {
    Waiter<S> wt(true);
    while (__ballot(has_x && !ll_ok(xr, epoch)) != 0) {
      if (wt.tick(p, sh)) return false;
      if (has_x && !ll_ok(xr, epoch)) xr = ll_load(xrow + lane);
    }
  }
  if (!slot_free(p, sh, i)) return false;
  trace_mark<S>(p, sh, i, 3, lane);
  float* act = sh.act[i % MK_NACT];
#pragma unroll
  for (int k = 0; k < NW; ++k) act[k * 64 + lane] = ll_val(wv[k]);
  if (has_x) sh.xres[which][lane] = xrow ? ll_val(xr) : ev;
  return true;
}

// Attention staging for item (kv head g, split s): q of the group's heads, the new k
// and v; RoPE on q and k; k, v rounded to bf16 (what the cache holds).  The split that
// contains the current position writes k, v into cache slot pos.  Word j of the group
// (elements 64j + lane) lies in one head; element e's rotation partner e +- hd/2 is in
// lane ^ 32 of the same word (hd 64) or the same lane of word j ^ 1 (hd 128).
template <class S>
__device__ __forceinline__ bool stage_attn(const MkParams& p, MkShared<S>& sh, const MkInstr& in, const StepGeo& g,
                                           int i, uint32_t epoch, int lane) {
  constexpr int HD = S::HD, HALF = HD / 2, NW = S::GRP / 64;
  constexpr int KB = S::HPG * HD, VB = (S::HPG + 1) * HD;   // offsets of k and v in the group
  const int l = in.layer, gi = in.a;
  const u64* src = p.ll_qkv + (size_t)l * S::NQKV + (size_t)gi * S::GRP;
  const float* cs = p.rope + (size_t)g.pos * HD + 2 * (lane & (HALF - 1));   // [half][2]
  const float c = cs[0], sn = cs[1];
  u64 wv[NW];
  trace_mark<S>(p, sh, i, 1, lane);
  if (!poll<S, NW>(p, sh, src, wv, epoch, lane)) return false;
  trace_mark<S>(p, sh, i, 2, lane);
  float v[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) v[j] = ll_val(wv[j]);
  float pr[NW];   // rotation partners
#pragma unroll
  for (int j = 0; j < NW; ++j) pr[j] = HD == 64 ? xor32(v[j], lane) : v[j ^ 1];
  // one writer of the new key and value: the split holding pos (q-head mode: head 0's item)
  const bool has_pos = g.qh ? in.b == 0 : in.b == g.s_eff - 1;
  uint16_t* kslot = p.kv + ((((size_t)l * 2) * S::HKV + gi) * p.max_ctx + g.pos) * HD;
  uint16_t* vslot = kslot + (size_t)S::HKV * p.max_ctx * HD;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int idx = j * 64 + lane;
    const bool first = HD == 64 ? lane < 32 : (j & 1) == 0;   // e < half
    if (j * 64 < VB) {   // q heads and k: rotate
      v[j] = first ? __fsub_rn(__fmul_rn(v[j], c), __fmul_rn(pr[j], sn))
                   : __fadd_rn(__fmul_rn(v[j], c), __fmul_rn(pr[j], sn));
    }
    if (j * 64 >= KB) {   // k and v: what the cache holds
      const uint16_t b = f2bf(v[j]);
      v[j] = bf16f(b);
      if (has_pos) (idx < VB ? kslot : vslot)[idx - (idx < VB ? KB : VB)] = b;
    }
  }
  if (!slot_free(p, sh, i)) return false;
  trace_mark<S>(p, sh, i, 3, lane);
  float* act = sh.act[i % MK_NACT];
#pragma unroll
  for (int j = 0; j < NW; ++j) act[j * 64 + lane] = v[j];
  return true;
}

// After the compute waves.  With fewer query heads per KV head than compute waves (and
// not the matrix-unit form, whose waves do this themselves), the waves of one head covered
// disjoint key subsets: combine their partials (and the current position's key) into this
// split's (m, l, o), then write o (single split) or publish the split.  Then, with several splits, CUs whose split index is below the
// heads per group merge one head each over all splits.  Lane `lane` handles elements
// lane + 64c of each head.
template <class S>
__device__ __forceinline__ bool attn_finalize(const MkParams& p, MkShared<S>& sh, const MkInstr& in,
                                              const StepGeo& g, int i, uint32_t epoch, int lane) {
  constexpr int HD = S::HD, HPG = S::HPG, E = HD / 64, STRIDE = HD + 2, NSUB = AttnGeo<S>::KS;
  const int l = in.layer, gi = in.a, s = in.b;
  const float* act = sh.act[i % MK_NACT];
  if (g.qh) {
    // q-head mode: combine the compute waves' partials of head s with the current key.
    // The current key's score is formed while the compute waves still work; the leader
    // then waits for them (the caller does not).
    if (s >= HPG) return wait_all_done(p, sh, i + 1, true);
    const float* pb = sh.part;
    float mw[MK_NC], lw[MK_NC], ow[MK_NC][E], kn[E], vn[E];
    float sp = 0.f;
#pragma unroll
    for (int c = 0; c < E; ++c) {
      kn[c] = act[HPG * HD + c * 64 + lane];
      vn[c] = act[(HPG + 1) * HD + c * 64 + lane];
      sp = fmaf(act[s * HD + c * 64 + lane], kn[c], sp);
    }
    sp = wave_sum(sp) * p.attn_scale;
    if (!wait_all_done(p, sh, i + 1, true)) return false;
    trace_mark<S>(p, sh, i, 8, lane);
#pragma unroll
    for (int w = 0; w < MK_NC; ++w) {
      mw[w] = pb[w * STRIDE];
      lw[w] = pb[w * STRIDE + 1];
#pragma unroll
      for (int c = 0; c < E; ++c) ow[w][c] = pb[w * STRIDE + 2 + c * 64 + lane];
    }
    float M = sp;
#pragma unroll
    for (int w = 0; w < MK_NC; ++w) M = fmaxf(M, mw[w]);
    const float wp = __expf(sp - M);
    float L = wp, wt[MK_NC];
#pragma unroll
    for (int w = 0; w < MK_NC; ++w) {
      wt[w] = mw[w] == -INFINITY ? 0.f : __expf(mw[w] - M);
      L = fmaf(lw[w], wt[w], L);
    }
#pragma unroll
    for (int c = 0; c < E; ++c) {
      float o = wp * vn[c];
#pragma unroll
      for (int w = 0; w < MK_NC; ++w) o = fmaf(ow[w][c], wt[w], o);
      ll_store(p.ll_o + (size_t)l * S::NQ + (gi * HPG + s) * HD + c * 64 + lane, o / L, epoch);
    }
    return true;
  }
  if (NSUB > 1 && !AttnGeo<S>::MMA && s < g.s_eff) {
    const bool has_pos = s == g.s_eff - 1;
    const float* pb = part_base<S>(sh, act);
    float mw[NSUB][HPG], lw[NSUB][HPG], ow[NSUB][HPG][E], qv[HPG][E], kn[E], vn[E];
#pragma unroll
    for (int w = 0; w < NSUB; ++w)
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float* q = pb + (w * HPG + h) * STRIDE;
        mw[w][h] = q[0];
        lw[w][h] = q[1];
#pragma unroll
        for (int c = 0; c < E; ++c) ow[w][h][c] = q[2 + c * 64 + lane];
      }
#pragma unroll
    for (int c = 0; c < E; ++c) {
#pragma unroll
      for (int h = 0; h < HPG; ++h) qv[h][c] = act[h * HD + c * 64 + lane];
      kn[c] = act[HPG * HD + c * 64 + lane];
      vn[c] = act[(HPG + 1) * HD + c * 64 + lane];
    }
    float sp[HPG];   // score of the current position (the key that is not in the cache yet)
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < E; ++c) acc = fmaf(qv[h][c], kn[c], acc);
      sp[h] = acc;
    }
#pragma unroll
    for (int h = 0; h < HPG; ++h) sp[h] = has_pos ? wave_sum(sp[h]) * p.attn_scale : -INFINITY;
    float Mh[HPG], Lh[HPG];
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      float M = sp[h];
#pragma unroll
      for (int w = 0; w < NSUB; ++w) M = fmaxf(M, mw[w][h]);
      float L = 0.f, wt[NSUB];
#pragma unroll
      for (int w = 0; w < NSUB; ++w) {
        wt[w] = mw[w][h] == -INFINITY ? 0.f : __expf(mw[w][h] - M);
        L = fmaf(lw[w][h], wt[w], L);
      }
      const float wp = has_pos ? __expf(sp[h] - M) : 0.f;
      L += wp;
#pragma unroll
      for (int c = 0; c < E; ++c) {
        float o = wp * vn[c];
#pragma unroll
        for (int w = 0; w < NSUB; ++w) o = fmaf(ow[w][h][c], wt[w], o);
        const int e = c * 64 + lane;
        if (g.s_eff == 1)
          ll_store(p.ll_o + (size_t)l * S::NQ + (gi * HPG + h) * HD + e, o / L, epoch);
        else
          ll_store(p.ll_part + part_index<S>(p, l, gi, h, s) + 2 + e, o, epoch);
      }
      Mh[h] = M;
      Lh[h] = L;
    }
    if (g.s_eff > 1) {
      // every head's (m, l) in one store instruction: lane 2h + j writes word j of head h
      // (the CU's store queue sits behind its page loads; fewer instructions wait less)
      const int hh = lane >> 1;
      float ml = 0.f;
#pragma unroll
      for (int h = 0; h < HPG; ++h) ml = hh == h ? ((lane & 1) ? Lh[h] : Mh[h]) : ml;
      if (lane < 2 * HPG) ll_store(p.ll_part + part_index<S>(p, l, gi, hh, s) + (lane & 1), ml, epoch);
    }
  }
  if (g.s_eff > 1 && s < HPG) {
    // Merge head s of this group over all splits; split t's words are [t*STRIDE, +STRIDE):
    // (m, l, o[HD]).  Splits are polled MB at a time and folded in split order.
    const int h = s;
    const u64* src = p.ll_part + part_index<S>(p, l, gi, h, 0);
    float M = -INFINITY, L = 0.f, o[E];
#pragma unroll
    for (int c = 0; c < E; ++c) o[c] = 0.f;
    Waiter<S> wt(true);
    constexpr int MB = 16 / E;
    for (int t0 = 0; t0 < g.s_eff; t0 += MB) {
      u64 ml, ow[MB][E];
      const int tl = t0 + (lane & 15);
      for (;;) {
        // lanes 0-15: m of split t0 + lane; lanes 16-31: its l (lanes 32-63 repeat them)
        ml = ll_load(src + (size_t)(tl < g.s_eff ? tl : t0) * STRIDE + ((lane >> 4) & 1));
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int c = 0; c < E; ++c)
            ow[j][c] = ll_load(src + (size_t)(t0 + j < g.s_eff ? t0 + j : t0) * STRIDE + 2 + c * 64 + lane);
        bool ok = ll_ok(ml, epoch);
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int c = 0; c < E; ++c) ok = ok && ll_ok(ow[j][c], epoch);
        if (__ballot(!ok) == 0) break;
        if (wt.tick(p, sh)) return false;
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float mt = __shfl(ll_val(ml), j), lt = __shfl(ll_val(ml), 16 + j);
        if (t0 + j < g.s_eff) {
          const float Mn = fmaxf(M, mt);
          const float a = M == -INFINITY ? 0.f : __expf(M - Mn);
          const float b = mt == -INFINITY ? 0.f : __expf(mt - Mn);
          L = L * a + lt * b;
#pragma unroll
          for (int c = 0; c < E; ++c) o[c] = o[c] * a + ll_val(ow[j][c]) * b;
          M = Mn;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < E; ++c)
      ll_store(p.ll_o + (size_t)l * S::NQ + (gi * HPG + h) * HD + c * 64 + lane, o[c] / L, epoch);
  }
  return true;
}

// Final argmax: combine the waves, publish the CU's key, take a ticket; the last CU
// reduces all keys, writes the next token and advances the epoch for the next step.
template <class S>
__device__ __forceinline__ void lm_finalize(const MkParams& p, MkShared<S>& sh, uint32_t epoch, int lane) {
  const int cu = blockIdx.x;
  u64 key = 0;
  for (int w = 0; w < MK_NC; ++w) key = sh.amax[w] > key ? sh.amax[w] : key;
  uint32_t old = 0;
  if (lane == 0) {
    // The key goes to memory (device-scope store) and has landed before the ticket counts
    // it; the last CU reads the keys with device-scope loads after its own ticket.  No
    // release or acquire of the XCD's L2 is needed (nothing else read in this step depends
    // on the order), and it would write back and invalidate the whole L2.
    __hip_atomic_store(p.amax + cu, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    old = __hip_atomic_fetch_add(&p.ctrl->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  old = __shfl(old, 0);
  if (old != (uint32_t)(p.n_cus - 1)) return;
  u64 best = 0;
  for (int c0 = 0; c0 < p.n_cus; c0 += 256) {
    u64 k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      k[j] = __hip_atomic_load(p.amax + min(c0 + 64 * j + lane, p.n_cus - 1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < 4; ++j) best = k[j] > best ? k[j] : best;   // a repeated key changes nothing
  }
  best = wave_max_u64(best);
  if (lane == 0) {
    if (p.next_token) p.next_token[0] = (int32_t)(0xffffffffu - (uint32_t)best);
    __hip_atomic_store(&p.ctrl->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // read by the next step, after the kernel boundary
    __hip_atomic_store(&p.ctrl->epoch, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class S>
__device__ __forceinline__ void leader_wave(const MkParams& p, MkShared<S>& sh, cinstr_t list, int nins,
                                            const StepGeo& g, int lane, uint32_t epoch) {
  for (int i = 0; i < nins; ++i) {
    const MkInstr in = list[i];
    const int l = in.layer;
    lane = opaque(lane);
    trace_mark<S>(p, sh, i, 0, lane);
    // One call site per staging routine: each is inlined once (the instruction cache holds
    // the kernel's hot code better than with a copy per instruction type).
    bool ok = true;
    if (in.op == MK_OP_ATTN) {
      if (attn_active(g, in.b, S::HPG)) ok = stage_attn<S>(p, sh, in, g, i, epoch, lane);
    } else if (in.op == MK_OP_O || in.op == MK_OP_DOWN) {
      // O: the residual is x entering the layer (the embedding row for the first layer);
      // the last down chunk adds x after attention
      const bool o = in.op == MK_OP_O, last = !o && in.a + 1 == S::NCH;
      const u64* src = o ? p.ll_o + (size_t)l * S::NQ : p.ll_a + (size_t)l * S::F + in.k0;
      const u64* xrow = o ? (l == 0 ? nullptr : p.ll_x + (size_t)(2 * l) * S::D + in.r0)
                          : (last ? p.ll_x + (size_t)(2 * l + 1) * S::D + in.r0 : nullptr);
      const uint16_t* erow = o && l == 0 ? p.embed + (size_t)sh.token * S::D + in.r0 : nullptr;
      const int xn = o || last ? in.n : 0;
      if constexpr (S::NQ == S::KC)
        ok = stage_raw<S, S::NQ>(p, sh, src, i, epoch, lane, xrow, erow, xn, o ? 0 : 1);
      else if (o)
        ok = stage_raw<S, S::NQ>(p, sh, src, i, epoch, lane, xrow, erow, xn, 0);
      else
        ok = stage_raw<S, S::KC>(p, sh, src, i, epoch, lane, xrow, erow, xn, 1);
    } else {
      // RMSNorm staging: QKV (x entering the layer, the embedding row for the first layer),
      // gate/up (x after attention), LM head (its record carries layer = n_layers: the last
      // residual version, and the final norm's gain)
      const bool gu = in.op == MK_OP_GATEUP;
      const u64* src = gu ? p.ll_x + (size_t)(2 * l + 1) * S::D
                          : (in.op == MK_OP_QKV && l == 0 ? nullptr : p.ll_x + (size_t)(2 * l) * S::D);
      const MkLayerPtrs& L = ((clayers_t)p.layers)[l];
      ok = stage_norm<S>(p, sh, src, gu ? L.mlp_norm : L.attn_norm, i, epoch, lane);
    }
    if (!ok) return;
    lds_fence();
    if (lane == 0) lds_store(&sh.act_seq, i + 1);
    trace_mark<S>(p, sh, i, 4, lane);
    if (in.op == MK_OP_ATTN) {
      // Partials in LDS only when several waves share a head (the matrix-unit form folds
      // them in the compute waves themselves); a merge polls global words.  (In q-head
      // mode attn_finalize waits itself, after the current key's score.)
      if (!g.qh) {
        if (AttnGeo<S>::KS > 1 && !AttnGeo<S>::MMA && !wait_all_done(p, sh, i + 1, true)) return;
        trace_mark<S>(p, sh, i, 8, lane);
      }
      if (!attn_finalize<S>(p, sh, in, g, i, epoch, lane)) return;
    } else if (in.op == MK_OP_LMHEAD) {
      if (!wait_all_done(p, sh, i + 1, true)) return;
      trace_mark<S>(p, sh, i, 8, lane);
      lm_finalize<S>(p, sh, epoch, lane);
    }
    trace_mark<S>(p, sh, i, 7, lane);
  }
  if constexpr (S::TRACE) {
    // every compute wave has finished the last instruction (the LM head waits for them)
    const int n = min(nins, p.trace_len);
    u64* dst = p.trace + (size_t)blockIdx.x * p.trace_len * MK_TRACE_SLOTS;
    for (int k = lane; k < n * MK_TRACE_SLOTS; k += 64) {
      const uint32_t v = sh.tr[k / MK_TRACE_SLOTS][k % MK_TRACE_SLOTS];
      const int slot = k % MK_TRACE_SLOTS;
      dst[k] = v == 0 ? 0ull : (slot == 9 || slot == 11) ? (u64)v : sh.t0 + v - 1u;
    }
  }
}

}  // namespace mkdev

// One decode step.  Grid: one work-group per CU, all resident at once (one fits per CU).
template <class S>
__global__ void __launch_bounds__(MK_THREADS) mk_step_kernel(MkParams p) {
  using namespace mkdev;
  __shared__ MkShared<S> sh;
  __shared__ __align__(16) char ring[Ring<S>::NSLOT * MK_PAGE_BYTES];
  // the wave index is uniform per wave; saying so keeps everything derived from it scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, cu = blockIdx.x;
  if constexpr (S::TRACE) {
    for (int k = threadIdx.x; k < MK_TRACE_MAX * MK_TRACE_SLOTS; k += MK_THREADS) (&sh.tr[0][0])[k] = 0;
  }
  if (threadIdx.x == 0) {
    sh.t0 = __builtin_amdgcn_s_memrealtime();
    sh.act_seq = 0;
    sh.pcnt = 0;
    // A step launched after an earlier one was abandoned (device error not yet reported
    // and reset by the host) does nothing: the communication words and the ticket may
    // still hold that step's partial state, and its words carry the current epoch.
    sh.abort_flag = __hip_atomic_load(&p.ctrl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    for (int w = 0; w < MK_NC; ++w) {
      sh.done[w] = 0;
      sh.amax[w] = 0;
    }
    for (int k = 0; k < MK_MAX_SLOTS; ++k) {
      sh.full[k] = 0;
      sh.freed[k] = 0;
      sh.acnt[k] = 0;
    }
    sh.epoch = __hip_atomic_load(&p.ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int t = p.token_dev ? p.token_dev[0] : p.token;
    if (t < 0 || t >= p.V) {
      if (cu == 0) __hip_atomic_store(&p.ctrl->bad_token, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      t = t < 0 ? 0 : p.V - 1;
    }
    sh.token = t;
  }
  __syncthreads();
  if (sh.abort_flag) return;
  const uint32_t epoch = sh.epoch;
  const int o0 = ((cint_t)p.plan_off)[cu];
  const int nins = ((cint_t)p.plan_off)[cu + 1] - o0;
  cinstr_t list = (cinstr_t)p.plan + o0;
  const StepGeo g = step_geo<S>(p, p.pos);
  // Issue priority within a SIMD (each SIMD runs a compute wave and one other wave): the
  // leader, which is on the critical path between instructions, first, then the loaders,
  // which keep the DMA queue full; measured 2-3 us per step faster than equal priorities.
  if (wave < MK_NC) {
    compute_wave<S>(p, sh, ring, list, nins, g, wave, lane, epoch);
  } else if (wave < MK_NC + MK_NL) {
    __builtin_amdgcn_s_setprio(2);
    loader_wave<S>(p, sh, ring, list, nins, g, wave - MK_NC, lane);
  } else {
    __builtin_amdgcn_s_setprio(3);
    leader_wave<S>(p, sh, list, nins, g, lane, epoch);
  }
}
