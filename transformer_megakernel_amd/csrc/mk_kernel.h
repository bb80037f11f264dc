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
//    global_load_lds_dwordx4 (HBM -> LDS, no registers), across instruction
//    boundaries and before the data an instruction depends on exists: weights and
//    cached keys never depend on this step's activations.  A loader knows a page is
//    complete from its own vmcnt and raises the slot's LDS flag; compute waves never
//    issue loads, so a wait for data never stalls behind the weight stream.  The
//    compiler is kept out of the DMA accounting (it would otherwise wait for every
//    load before any LDS access).
//  * Dependencies without grid barriers.  The article uses integer counters in
//    global memory; on gfx950 the eight XCDs have separate L2s, so a counter costs a
//    store-acknowledge, an atomic and a second round trip for the data.  Instead each
//    produced value travels with its own completion flag: a 64-bit word holding the
//    fp32 value and the step's epoch, stored and polled with device-scope (sc1)
//    accesses.  A consumer is ready when every word it needs carries the current
//    epoch, so one store and one poll cover data and signal.  The step's last CU
//    (an atomic ticket, the one counter kept) advances the epoch for the next step.
//  * A leader wave per CU does the waiting: it polls the inputs of the next
//    instruction, applies RMSNorm / RoPE, stages the fp32 activation vector in LDS
//    and releases the compute waves, which then only touch LDS and store results.
//  * The article's 4-chunk MLP intermediate: the down projection is issued as 4
//    K-chunks, each waiting only for its quarter of SiLU(gate)*up.
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
// uses scalar loads: a vector load in a compute wave would make the compiler wait
// for every page load in flight before using it.
#if defined(__HIP_DEVICE_COMPILE__)
typedef const __attribute__((address_space(4))) MkInstr* cinstr_t;
typedef const __attribute__((address_space(4))) MkLayerPtrs* clayers_t;
typedef const __attribute__((address_space(4))) int32_t* cint_t;
#else
typedef const MkInstr* cinstr_t;   // host pass: the kernel body is only parsed
typedef const MkLayerPtrs* clayers_t;
typedef const int32_t* cint_t;
#endif

struct __align__(16) MkShared {
  float act[MK_ACT_FLOATS];                 // staged activation vector of the instruction
  char pages[MK_PAGES_BYTES];               // page ring (nslot pages)
  float xres[MK_MAX_RES_ROWS];              // x rows this CU's next residual adds to
  float rowacc[MK_MAX_RES_ROWS];            // DOWN partial sums over the K-chunks
  float rowres[MK_NC][64];                  // row results of the page being finished
  u64 amax[MK_NC];                          // per-wave argmax keys (LM head)
  int done[MK_NC];                          // instructions finished, per compute wave
  uint16_t gain[MK_ACT_FLOATS];             // RMSNorm gains of the instruction being staged
  int full[MK_MAX_SLOTS];                   // ring slot holds page k once full == k + 1
  int freed[MK_MAX_SLOTS];                  // ring slot's page k consumed once freed == k + 1
  int act_seq;                              // instructions staged by the leader
  int abort_flag;
  uint32_t epoch;                           // tag of this step's words
  int token;                                // input token (validated)
};

// ------------------------------------------------------------------ small helpers
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// HBM -> LDS, 16 bytes per lane: lane i lands at lds + 16*i.  Issued through inline
// assembly so that the compiler does not add a wait for it before later LDS accesses.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(l) : "memory", "m0");
}

#define MK_VMCNT_CASE(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
// Wait until at most n vector-memory operations of this wave are outstanding.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    MK_VMCNT_CASE(0) MK_VMCNT_CASE(1) MK_VMCNT_CASE(2) MK_VMCNT_CASE(3) MK_VMCNT_CASE(4)
    MK_VMCNT_CASE(5) MK_VMCNT_CASE(6) MK_VMCNT_CASE(7) MK_VMCNT_CASE(8) MK_VMCNT_CASE(9)
    MK_VMCNT_CASE(10) MK_VMCNT_CASE(11) MK_VMCNT_CASE(12) MK_VMCNT_CASE(13) MK_VMCNT_CASE(14)
    MK_VMCNT_CASE(15) MK_VMCNT_CASE(16) MK_VMCNT_CASE(17) MK_VMCNT_CASE(18) MK_VMCNT_CASE(19)
    MK_VMCNT_CASE(20) MK_VMCNT_CASE(21) MK_VMCNT_CASE(22) MK_VMCNT_CASE(23) MK_VMCNT_CASE(24)
    MK_VMCNT_CASE(25) MK_VMCNT_CASE(26) MK_VMCNT_CASE(27) MK_VMCNT_CASE(28) MK_VMCNT_CASE(29)
    MK_VMCNT_CASE(30) MK_VMCNT_CASE(31) MK_VMCNT_CASE(32) MK_VMCNT_CASE(33) MK_VMCNT_CASE(34)
    MK_VMCNT_CASE(35) MK_VMCNT_CASE(36) MK_VMCNT_CASE(37) MK_VMCNT_CASE(38) MK_VMCNT_CASE(39)
    MK_VMCNT_CASE(40) MK_VMCNT_CASE(41) MK_VMCNT_CASE(42) MK_VMCNT_CASE(43) MK_VMCNT_CASE(44)
    MK_VMCNT_CASE(45) MK_VMCNT_CASE(46) MK_VMCNT_CASE(47) MK_VMCNT_CASE(48) MK_VMCNT_CASE(49)
    MK_VMCNT_CASE(50) MK_VMCNT_CASE(51) MK_VMCNT_CASE(52) MK_VMCNT_CASE(53) MK_VMCNT_CASE(54)
    MK_VMCNT_CASE(55) MK_VMCNT_CASE(56) MK_VMCNT_CASE(57) MK_VMCNT_CASE(58) MK_VMCNT_CASE(59)
    MK_VMCNT_CASE(60) MK_VMCNT_CASE(61) MK_VMCNT_CASE(62)
    default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
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

// ------------------------------------------------------------------ reductions (DPP)
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
// Sum within aligned groups of g lanes (g a power of two <= 64), by lane swaps.
__device__ __forceinline__ float group_sum(float v, int g) {
  for (int off = g >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
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

__device__ __forceinline__ void trace_mark(const MkParams& p, int cu, int i, int slot, int lane) {
  if (p.trace && lane == 0 && i < p.trace_len)
    p.trace[((size_t)cu * p.trace_len + i) * MK_TRACE_SLOTS + slot] = __builtin_amdgcn_s_memrealtime();
}

// ------------------------------------------------------------------ step geometry
struct StepGeo {
  int pos, s_eff, chunk, ppp;   // attention split of keys 0..pos
};

__device__ __forceinline__ StepGeo step_geo(const MkParams& p, int pos) {
  StepGeo g;
  g.pos = pos;
  g.ppp = p.page_bytes / (4 * p.hd);       // key+value positions per page
  const int nk = pos + 1;
  int chunk = (nk + p.s_max - 1) / p.s_max;
  if (chunk < p.min_chunk) chunk = p.min_chunk;
  chunk = (chunk + g.ppp - 1) / g.ppp * g.ppp;
  g.chunk = chunk;
  g.s_eff = (nk + chunk - 1) / chunk;
  return g;
}

// Keys [j0, j1) of split s; the cached part (read from the cache) is [j0, min(j1, pos)).
__device__ __forceinline__ void attn_range(const StepGeo& g, int s, int* j0, int* j1, int* cached_end) {
  const int nk = g.pos + 1;
  *j0 = s * g.chunk;
  *j1 = min(nk, (s + 1) * g.chunk);
  *cached_end = min(*j1, g.pos);
}

// An instruction decoded once: everything its pages need, wave-uniform.
struct Dec {
  int op, layer, r0, n, k0, kn, a, b;
  int np;            // pages of the instruction on this CU
  int seg;           // bytes of one row segment
  int rpp;           // rows per page (GATEUP: gate/up pairs per page)
  int upr;           // 1 KiB units per row, or 0 when a row is shorter than 1 KiB
  int lpr_sh;        // log2(lanes per row) when a row is shorter than 1 KiB
  int s1, s2;        // QKV: rows below s1 come from m0, below s2 from m1, the rest from m2
  const char* m0;    // row 0 of each source matrix, input column k0 applied (bytes)
  const char* m1;
  const char* m2;
  long long stride;  // bytes between rows
  int j0, ce;        // ATTN: cached keys [j0, ce); m0 / m1 = K / V of (layer, kv head) at key 0
};

__device__ __forceinline__ Dec decode(const MkParams& p, const MkInstr& in, const StepGeo& g) {
  Dec d;
  d.op = in.op; d.layer = in.layer; d.r0 = in.r0; d.n = in.n; d.k0 = in.k0; d.kn = in.kn; d.a = in.a; d.b = in.b;
  d.s1 = d.s2 = 0;
  d.m0 = d.m1 = d.m2 = nullptr;
  d.upr = d.lpr_sh = 0;
  d.seg = d.rpp = 0;
  d.j0 = d.ce = 0;
  d.stride = 0;
  if (in.op == MK_OP_ATTN) {
    d.np = 0;
    if (in.b < g.s_eff) {
      int j1;
      attn_range(g, in.b, &d.j0, &j1, &d.ce);
      const int cached = d.ce - d.j0;
      d.np = cached > 0 ? (cached + g.ppp - 1) / g.ppp : 0;
    }
    const size_t head = ((size_t)(in.layer * 2) * p.hkv + in.a) * p.max_ctx;
    d.m0 = (const char*)(p.kv + head * p.hd);
    d.m1 = (const char*)(p.kv + (head + (size_t)p.hkv * p.max_ctx) * p.hd);
    return d;
  }
  d.seg = 2 * in.kn;
  d.rpp = in.op == MK_OP_GATEUP ? p.page_bytes / (2 * d.seg) : p.page_bytes / d.seg;
  d.np = (in.n + d.rpp - 1) / d.rpp;
  if (d.seg >= 1024) d.upr = d.seg >> 10;
  else d.lpr_sh = 31 - __builtin_clz((unsigned)(d.seg >> 4));
  const MkLayerPtrs L = ((clayers_t)p.layers)[in.layer < p.n_layers ? in.layer : 0];
  // Plain selects, not a switch: a switch over runtime values becomes a table in
  // private memory, read with vector loads.
  const bool qkv = in.op == MK_OP_QKV, gu = in.op == MK_OP_GATEUP, o = in.op == MK_OP_O,
             dn = in.op == MK_OP_DOWN;
  const uint16_t* a0 = qkv ? L.wq : gu ? L.wg : o ? L.wo : dn ? L.wd : p.lm_head;
  const uint16_t* a1 = qkv ? L.wk : gu ? L.wu : nullptr;
  const uint16_t* a2 = qkv ? L.wv : nullptr;
  d.stride = 2LL * (o ? p.nq : dn ? p.F : p.d);
  if (qkv) {
    d.s1 = p.nq;
    d.s2 = p.nq + p.nkv;
  }
  d.m0 = (const char*)(a0 + in.k0);
  d.m1 = a1 ? (const char*)(a1 + in.k0) : d.m0;
  d.m2 = a2 ? (const char*)(a2 + in.k0) : d.m0;
  return d;
}

// Row j of page `first`: the page holds rows first.. of the instruction, or for GATEUP the
// interleaved pairs gate(f), up(f), gate(f+1), up(f+1), ... with f = r0 + first.
__device__ __forceinline__ const char* page_row(const Dec& d, int first, int j) {
  if (d.op == MK_OP_GATEUP) {
    const long long f = d.r0 + first + (j >> 1);
    return ((j & 1) ? d.m1 : d.m0) + f * d.stride;
  }
  const int gr = d.r0 + first + j;
  if (d.op == MK_OP_QKV) {
    if (gr >= d.s2) return d.m2 + (long long)(gr - d.s2) * d.stride;
    if (gr >= d.s1) return d.m1 + (long long)(gr - d.s1) * d.stride;
  }
  return d.m0 + (long long)gr * d.stride;
}

// Issue the DMA of page pg into the LDS page at `slot`: always `lpp` loads of 1 KiB so
// the wave's vmcnt moves in multiples of lpp; loads past the payload re-read valid bytes.
__device__ __forceinline__ void issue_page(const Dec& d, int pg, int ppp, int hd, int lpp, uint32_t slot,
                                           int lane) {
  if (d.op == MK_OP_ATTN) {
    const int q0 = d.j0 + pg * ppp;
    const int np = min(ppp, d.ce - q0);
    const int rowb = 2 * hd;
    const int kbytes = np * rowb;
    const char* kb = d.m0 + (size_t)q0 * rowb;
    const char* vb = d.m1 + (size_t)q0 * rowb;
    for (int u = 0; u < lpp; ++u) {
      const int o = u * 1024 + lane * 16;
      const char* a = o < kbytes ? kb + o : (o < 2 * kbytes ? vb + (o - kbytes) : kb);
      dma16(a, slot + u * 1024);
    }
    return;
  }
  const int first = pg * d.rpp;
  const int m = min(d.rpp, d.n - first);
  const int rows = d.op == MK_OP_GATEUP ? 2 * m : m;
  if (d.upr) {
    // One row base per row (a few scalar ops), then its 1 KiB units by plain adds.
    uint32_t dst = slot;
    int u = 0;
    for (int j = 0; j < rows; ++j) {
      const char* rb = page_row(d, first, j) + lane * 16;
      for (int c = 0; c < d.upr; ++c, ++u, dst += 1024) dma16(rb + c * 1024, dst);
    }
    const char* dummy = d.m0 + lane * 16;   // keeps the load count at lpp
    for (; u < lpp; ++u, dst += 1024) dma16(dummy, dst);
  } else {
    const int rpu = 64 >> d.lpr_sh;
    const int cl = lane & ((1 << d.lpr_sh) - 1);
    for (int u = 0; u < lpp; ++u) {
      const int jl = u * rpu + (lane >> d.lpr_sh);
      dma16(page_row(d, first, jl < rows ? jl : 0) + cl * 16, slot + u * 1024);
    }
  }
}

// ------------------------------------------------------------------ waits and aborts
__device__ __forceinline__ void raise_error(const MkParams& p, MkShared& sh, int code) {
  atomicCAS(&p.ctrl->error, 0, code);
  lds_store(&sh.abort_flag, 1);
}

// Compute waves never read the global error word (a vector load would wait for their
// page loads); they follow the LDS abort flag and their own clock.
struct Waiter {
  long long t0;
  int n;
  bool global_check;
  __device__ __forceinline__ Waiter(bool leader) : t0(__builtin_amdgcn_s_memrealtime()), n(0), global_check(leader) {}
  // true when the wait must be abandoned
  __device__ __forceinline__ bool tick(const MkParams& p, MkShared& sh) {
    __builtin_amdgcn_s_sleep(1);
    if (lds_load(&sh.abort_flag)) return true;
    if ((++n & 63) == 0) {
      if (global_check &&
          __hip_atomic_load(&p.ctrl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        lds_store(&sh.abort_flag, 1);
        return true;
      }
      if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > p.watchdog_ticks) {
        raise_error(p, sh, MK_ETIMEOUT);
        return true;
      }
    }
    return false;
  }
};

// Wait until *flag >= target (LDS).  False if abandoned.
__device__ __forceinline__ bool wait_flag(const MkParams& p, MkShared& sh, const int* flag, int target,
                                          bool leader) {
  if (lds_load(flag) >= target) { compiler_fence(); return true; }
  Waiter wt(leader);
  while (lds_load(flag) < target)
    if (wt.tick(p, sh)) return false;
  compiler_fence();
  return true;
}

__device__ __forceinline__ bool wait_all_done(const MkParams& p, MkShared& sh, int target) {
  for (int w = 0; w < MK_NC; ++w)
    if (!wait_flag(p, sh, &sh.done[w], target, true)) return false;
  return true;
}

// ------------------------------------------------------------------ page ring
// The pages of the CU's whole list, in list order, are numbered k = 0, 1, ...; page k
// lives in ring slot k % nslot, is issued by loader wave k % MK_NL and consumed by
// compute wave k % MK_NC.  LDS flags: full[slot] = k + 1 once page k has landed,
// freed[slot] = k + 1 once its compute wave has read it.  nslot is a multiple of
// MK_NL, so the page a loader waits to be freed is one it issued itself.
__device__ __forceinline__ int first_of(int who, int base, int period) {
  return ((who - base) % period + period) % period;
}

// Loader wave l.  It publishes its pages in order, each once vmcnt shows it complete,
// keeping at most D of them unpublished (vmcnt counts to 63).  While it waits for a
// slot still in use it keeps publishing what it has in flight: a compute wave may be
// waiting for one of those pages.
__device__ __forceinline__ void loader_wave(const MkParams& p, MkShared& sh, cinstr_t list, int nins,
                                            const StepGeo& g, int l, int lane) {
  const int nslot = p.nslot, lpp = p.lpp, pb = p.page_bytes;
  const uint32_t ring = lds_addr(sh.pages);
  const int D = min(8, min(nslot / MK_NL, 63 / lpp + 1));
  int oldest = 0, pend = 0;   // own pages issued and not yet published: oldest, then every MK_NL-th
  int base = 0;
  for (int i = 0; i < nins; ++i) {
    const Dec d = decode(p, list[i], g);
    lane = opaque(lane);
    for (int pg = first_of(l, base, MK_NL); pg < d.np; pg += MK_NL) {
      const int k = base + pg;
      const int slot = k % nslot;
      // Slot still in use: publish own pages as they land (oldest first) while waiting.
      while (lds_load(&sh.freed[slot]) < k - nslot + 1) {
        if (pend == 0) {
          if (!wait_flag(p, sh, &sh.freed[slot], k - nslot + 1, false)) {
            wait_vmcnt(0);   // nothing may land in LDS after the wave has left
            return;
          }
          break;
        }
        wait_vmcnt((pend - 1) * lpp);
        if (lane == 0) lds_store(&sh.full[oldest % nslot], oldest + 1);
        oldest += MK_NL;
        --pend;
      }
      issue_page(d, pg, g.ppp, p.hd, lpp, ring + (uint32_t)(slot * pb), lane);
      if (pend == 0) oldest = k;
      ++pend;
      if (pend == D) {   // the oldest is complete once at most (D - 1) pages are outstanding
        wait_vmcnt((D - 1) * lpp);
        if (lane == 0) lds_store(&sh.full[oldest % nslot], oldest + 1);
        oldest += MK_NL;
        --pend;
      }
    }
    base += d.np;
  }
  wait_vmcnt(0);
  for (; pend > 0; --pend, oldest += MK_NL)
    if (lane == 0) lds_store(&sh.full[oldest % nslot], oldest + 1);
}

// Page k for a compute wave, once it has landed (nullptr if the wait was abandoned).
__device__ __forceinline__ const char* page_wait(const MkParams& p, MkShared& sh, int k) {
  const int slot = k % p.nslot;
  if (!wait_flag(p, sh, &sh.full[slot], k + 1, false)) return nullptr;
  return sh.pages + slot * p.page_bytes;
}
// The wave has finished reading page k: once its LDS reads have returned the loader
// may overwrite the slot.
__device__ __forceinline__ void page_free(const MkParams& p, MkShared& sh, int k, int lane) {
  lds_fence();
  if (lane == 0) lds_store(&sh.freed[k % p.nslot], k + 1);
}

// ------------------------------------------------------------------ compute waves
// Group-major index of a raw q/k/v row: [kv head][q heads of the group | k | v][hd].
__device__ __forceinline__ int qkv_index(const MkParams& p, int row) {
  const int grp = (p.hpg + 2) * p.hd;
  if (row < p.nq) {
    const int h = row / p.hd;
    return (h / p.hpg) * grp + (h % p.hpg) * p.hd + (row - h * p.hd);
  }
  if (row < p.nq + p.nkv) {
    const int r = row - p.nq;
    return (r / p.hd) * grp + p.hpg * p.hd + (r % p.hd);
  }
  const int r = row - p.nq - p.nkv;
  return (r / p.hd) * grp + (p.hpg + 1) * p.hd + (r % p.hd);
}

// Finish one output row (value v, uniform over the wave; lane 0 stores).
__device__ __forceinline__ void row_epilogue(const MkParams& p, MkShared& sh, const Dec& d, int gr, float v,
                                             int lane, uint32_t epoch, u64* best) {
  const int l = d.layer;
  switch (d.op) {
    case MK_OP_QKV:
      if (lane == 0) ll_store(p.ll_qkv + (size_t)l * p.nqkv + qkv_index(p, gr), v, epoch);
      break;
    case MK_OP_O:
      if (lane == 0) ll_store(p.ll_x + (size_t)(2 * l + 1) * p.d + gr, sh.xres[gr - d.r0] + v, epoch);
      break;
    case MK_OP_DOWN: {
      const int k = gr - d.r0;
      const float acc = (d.a == 0 ? 0.f : sh.rowacc[k]) + v;
      if (d.a + 1 < d.b) {
        if (lane == 0) sh.rowacc[k] = acc;
      } else if (lane == 0) {
        ll_store(p.ll_x + (size_t)(2 * l + 2) * p.d + gr, sh.xres[k] + acc, epoch);
      }
      break;
    }
    default: {  // MK_OP_LMHEAD
      if (lane == 0) p.logits[gr] = v;
      const u64 key = amax_key(v, (uint32_t)gr);
      if (key > *best) *best = key;
      break;
    }
  }
}

__device__ __forceinline__ void gateup_epilogue(const MkParams& p, const Dec& d, int f, float gt, float up,
                                                int lane, uint32_t epoch) {
  const float a = (gt / (1.0f + __expf(-gt))) * up;
  if (lane == 0) ll_store(p.ll_a + (size_t)d.layer * p.F + f, a, epoch);
}

// Rows of at least 1 KiB: the lane's slice of the activation stays in registers for the
// whole instruction; each row is UPR units of 1 KiB, lane l holding bytes 16l.. of each.
template <int UPR>
__device__ __forceinline__ float row_dot(const char* page, int j, const float (&av)[UPR][8], int lane) {
  uint4 wv[UPR];   // all units' LDS reads first, so their latency overlaps
#pragma unroll
  for (int u = 0; u < UPR; ++u) wv[u] = *(const uint4*)(page + (j * UPR + u) * 1024 + lane * 16);
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < UPR; ++u) acc = dot8(wv[u], av[u], acc);
  return acc;
}

template <int UPR>
__device__ __forceinline__ bool gemv_wide(const MkParams& p, MkShared& sh, const Dec& d, int base, int w, int lane,
                                          uint32_t epoch, u64* best) {
  float av[UPR][8];
#pragma unroll
  for (int u = 0; u < UPR; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) av[u][e] = sh.act[u * 512 + lane * 8 + e];
  for (int pg = first_of(w, base, MK_NC); pg < d.np; pg += MK_NC) {
    const char* page = page_wait(p, sh, base + pg);
    if (!page) return false;
    const int first = pg * d.rpp;
    const int m = min(d.rpp, d.n - first);
    if (d.op == MK_OP_GATEUP) {
      for (int j = 0; j < m; ++j) {
        const float g = wave_sum(row_dot<UPR>(page, 2 * j, av, lane));
        const float u = wave_sum(row_dot<UPR>(page, 2 * j + 1, av, lane));
        gateup_epilogue(p, d, d.r0 + first + j, g, u, lane, epoch);
      }
    } else {
      int j = 0;
      for (; j + 1 < m; j += 2) {
        const float v0 = wave_sum(row_dot<UPR>(page, j, av, lane));
        const float v1 = wave_sum(row_dot<UPR>(page, j + 1, av, lane));
        row_epilogue(p, sh, d, d.r0 + first + j, v0, lane, epoch, best);
        row_epilogue(p, sh, d, d.r0 + first + j + 1, v1, lane, epoch, best);
      }
      if (j < m) row_epilogue(p, sh, d, d.r0 + first + j, wave_sum(row_dot<UPR>(page, j, av, lane)), lane, epoch, best);
    }
    page_free(p, sh, base + pg, lane);
  }
  return true;
}

// Rows shorter than 1 KiB (small models): several rows per 1 KiB unit, lpr lanes per row;
// results go through LDS so that lane j can finish row j.
__device__ __forceinline__ bool gemv_narrow(const MkParams& p, MkShared& sh, const Dec& d, int base, int w,
                                            int lane, uint32_t epoch, u64* best) {
  const int lpr = 1 << d.lpr_sh, rpu = 64 >> d.lpr_sh, c = lane & (lpr - 1);
  float av[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) av[e] = sh.act[c * 8 + e];
  float* res = sh.rowres[w];
  for (int pg = first_of(w, base, MK_NC); pg < d.np; pg += MK_NC) {
    const char* page = page_wait(p, sh, base + pg);
    if (!page) return false;
    const int first = pg * d.rpp;
    const int m = min(d.rpp, d.n - first);
    const int rows = d.op == MK_OP_GATEUP ? 2 * m : m;
    for (int u = 0; u * rpu < rows; ++u) {
      float acc = dot8(*(const uint4*)(page + u * 1024 + lane * 16), av, 0.f);
      acc = group_sum(acc, lpr);
      const int j = u * rpu + (lane >> d.lpr_sh);
      if (c == 0 && j < rows) res[j] = acc;
    }
    page_free(p, sh, base + pg, lane);
    for (int j = 0; j < m; ++j) {
      if (d.op == MK_OP_GATEUP) gateup_epilogue(p, d, d.r0 + first + j, res[2 * j], res[2 * j + 1], lane, epoch);
      else row_epilogue(p, sh, d, d.r0 + first + j, res[j], lane, epoch, best);
    }
  }
  return true;
}

template <int HD, int HPG>
struct AttnState {
  float q[HPG][8];
  float m[HPG], l[HPG];
  float o[HPG][8];
};

template <int HD, int HPG>
__device__ __forceinline__ void attn_init(AttnState<HD, HPG>& st, const MkShared& sh, int lane) {
  constexpr int LPP = HD / 8;
  const int c = lane % LPP;
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st.q[h][e] = sh.act[h * HD + c * 8 + e];
      st.o[h][e] = 0.f;
    }
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
  }
}

// One page of cached keys/values: [npos][HD] keys, then [npos][HD] values.  Lane l holds
// 8 dims (chunk l % LPP) of position l / LPP of each 1 KiB unit.
template <int HD, int HPG>
__device__ __forceinline__ void attn_page(AttnState<HD, HPG>& st, const char* page, int npos, float scale,
                                          int lane) {
  constexpr int LPP = HD / 8;        // lanes per position
  constexpr int PPU = 64 / LPP;      // positions per 1 KiB unit
  constexpr int MAXU = 8;            // units per key block (16 KiB page)
  const int nu = (npos + PPU - 1) / PPU;
  const int kbytes = npos * HD * 2;
  const int jl = lane / LPP;
  float s[MAXU][HPG];
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) s[u][h] = -INFINITY;
    if (u < nu) {
      const uint4 kw = *(const uint4*)(page + u * 1024 + lane * 16);
      const bool valid = u * PPU + jl < npos;
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        float part = dot8(kw, st.q[h], 0.f);
        part = LPP == 8 ? sum8(part) : sum16(part);
        s[u][h] = valid ? part * scale : -INFINITY;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    float pm = s[0][h];
#pragma unroll
    for (int u = 1; u < MAXU; ++u) pm = fmaxf(pm, s[u][h]);
    pm = wave_max(pm);
    const float mn = fmaxf(st.m[h], pm);
    const float alpha = __expf(st.m[h] - mn);
    st.m[h] = mn;
    st.l[h] *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[h][e] *= alpha;
  }
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    if (u < nu && u * PPU + jl < npos) {
      const uint4 vw = *(const uint4*)(page + kbytes + u * 1024 + lane * 16);
      float vf[8] = {bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y),
                     bf_lo(vw.z), bf_hi(vw.z), bf_lo(vw.w), bf_hi(vw.w)};
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float pr = __expf(s[u][h] - st.m[h]);
        st.l[h] += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[h][e] = fmaf(pr, vf[e], st.o[h][e]);
      }
    }
  }
}

// Reduce the wave's state over its position groups and leave (m, l, o) in LDS.  The
// HPG * 9 sums are independent: each swap step is applied to all of them before the
// next, so their LDS round trips overlap instead of forming one long chain.
template <int HD, int HPG>
__device__ __forceinline__ void attn_publish(AttnState<HD, HPG>& st, MkShared& sh, int w, int lane) {
  constexpr int LPP = HD / 8;
  float* part = sh.act + MK_PART_OFF + w * HPG * (HD + 2);
#pragma unroll
  for (int off = LPP; off < 64; off <<= 1) {
    float t[HPG][9];
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      t[h][8] = __shfl_xor(st.l[h], off);
#pragma unroll
      for (int e = 0; e < 8; ++e) t[h][e] = __shfl_xor(st.o[h][e], off);
    }
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      st.l[h] += t[h][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[h][e] += t[h][e];
    }
  }
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    if (lane < LPP) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[h * (HD + 2) + 2 + lane * 8 + e] = st.o[h][e];
    }
    if (lane == 0) {
      part[h * (HD + 2)] = st.m[h];
      part[h * (HD + 2) + 1] = st.l[h];
    }
  }
}

template <int HD, int HPG>
__device__ __forceinline__ bool attn_run(const MkParams& p, MkShared& sh, const Dec& d, const StepGeo& g, int base,
                                         int w, int lane) {
  AttnState<HD, HPG> st;
  attn_init<HD, HPG>(st, sh, lane);
  for (int pg = first_of(w, base, MK_NC); pg < d.np; pg += MK_NC) {
    const char* page = page_wait(p, sh, base + pg);
    if (!page) return false;
    const int npos = min(g.ppp, d.ce - (d.j0 + pg * g.ppp));
    attn_page<HD, HPG>(st, page, npos, p.attn_scale, lane);
    page_free(p, sh, base + pg, lane);
  }
  attn_publish<HD, HPG>(st, sh, w, lane);
  return true;
}

__device__ __forceinline__ void compute_wave(const MkParams& p, MkShared& sh, cinstr_t list, int nins,
                                             const StepGeo& g, int w, int lane, uint32_t epoch) {
  int base = 0;   // ring number of the instruction's first page
  for (int i = 0; i < nins; ++i) {
    const Dec d = decode(p, list[i], g);
    lane = opaque(lane);
    if (!wait_flag(p, sh, &sh.act_seq, i + 1, false)) return;
    bool ok = true;
    if (d.op == MK_OP_ATTN) {
      // A split that is inactive at this position does nothing: in particular it must not
      // write partials into act, which other waves may still read for the previous
      // instruction (the leader releases inactive splits without waiting for them).
      if (d.b >= g.s_eff) {
      } else if (p.hd == 64) {
        if (p.hpg == 4) ok = attn_run<64, 4>(p, sh, d, g, base, w, lane);
        else if (p.hpg == 2) ok = attn_run<64, 2>(p, sh, d, g, base, w, lane);
        else ok = attn_run<64, 1>(p, sh, d, g, base, w, lane);
      } else {
        if (p.hpg == 4) ok = attn_run<128, 4>(p, sh, d, g, base, w, lane);
        else if (p.hpg == 2) ok = attn_run<128, 2>(p, sh, d, g, base, w, lane);
        else ok = attn_run<128, 1>(p, sh, d, g, base, w, lane);
      }
    } else {
      u64 best = 0;
      switch (d.upr) {
        case 0: ok = gemv_narrow(p, sh, d, base, w, lane, epoch, &best); break;
        case 1: ok = gemv_wide<1>(p, sh, d, base, w, lane, epoch, &best); break;
        case 2: ok = gemv_wide<2>(p, sh, d, base, w, lane, epoch, &best); break;
        case 4: ok = gemv_wide<4>(p, sh, d, base, w, lane, epoch, &best); break;
        case 7: ok = gemv_wide<7>(p, sh, d, base, w, lane, epoch, &best); break;
        default: ok = gemv_wide<8>(p, sh, d, base, w, lane, epoch, &best); break;
      }
      if (d.op == MK_OP_LMHEAD) {
        best = wave_max_u64(best);
        if (lane == 0) sh.amax[w] = best;
      }
    }
    if (!ok) return;
    base += d.np;
    lds_fence();
    if (lane == 0) lds_store(&sh.done[w], i + 1);
    trace_mark(p, blockIdx.x, i, 4 + w, lane);
  }
}

// ------------------------------------------------------------------ leader wave
// Loads in the leader are issued in batches with no branch between them: a load under
// a per-lane condition gets its own block, and the compiler then waits for each one
// before the next (a full round trip per load).  Out-of-range lanes load a valid
// address and discard the value.

// Poll words [base, base + 64*NW) of src until all carry this step's epoch.  Word base + 64k + lane lands in wv[k]; words past `total` are loaded (the
// arena is padded by MK_LL_PAD words) but not waited for.
// The first pass loads every word; while words are missing, each lane re-polls only its
// first missing word (one load per lane per round trip) and the wave reloads the whole
// batch once one has arrived: re-polling whole vectors from every CU would compete with
// the weight stream for HBM.  Reloading a word that already carries the epoch is
// harmless: each word is written once per step, and a later load of a location never
// returns an older value than an earlier one.
template <int NW = MK_GATHER_MAXW>
__device__ __forceinline__ bool poll_batch(const MkParams& p, MkShared& sh, const u64* src, int total, int base,
                                           u64 (&wv)[NW], uint32_t epoch, int lane) {
  const u64* q = src + base + lane;
  const int lim = total - base - lane;      // word k is in range when 64k < lim
#pragma unroll
  for (int k = 0; k < NW; ++k) wv[k] = ll_load(q + k * 64);
  Waiter wt(true);
  for (;;) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < NW; ++k) all = all && (ll_ok(wv[k], epoch) || k * 64 >= lim);
    if (__ballot(!all) == 0) return true;
    int first_bad = -1;
#pragma unroll
    for (int k = NW - 1; k >= 0; --k)
      first_bad = (k * 64 >= lim || ll_ok(wv[k], epoch)) ? first_bad : k;
    if (wt.tick(p, sh)) return false;
    const u64 s = ll_load(q + (first_bad >= 0 ? first_bad * 64 : 0));
    if (__ballot(first_bad >= 0 && ll_ok(s, epoch)) != 0) {
#pragma unroll
      for (int k = 0; k < NW; ++k) wv[k] = ll_load(q + k * 64);
    }
  }
}

// Gather `total` words of src into dst (LDS floats), waiting for the compute waves to
// have finished instruction `prev_done` before the first LDS write.  The lane's sum of
// squares of what it wrote goes to *ss when ss is not null.
__device__ __forceinline__ bool gather(const MkParams& p, MkShared& sh, const u64* src, int total, float* dst,
                                       int prev_done, uint32_t epoch, int lane, float* ss) {
  bool waited = false;
  float acc = 0.f;
  for (int base = 0; base < total; base += 64 * MK_GATHER_MAXW) {
    u64 wv[MK_GATHER_MAXW];
    if (!poll_batch(p, sh, src, total, base, wv, epoch, lane)) return false;
    if (base + 64 * MK_GATHER_MAXW >= total) trace_mark(p, blockIdx.x, prev_done, 1, lane);
    if (!waited) {
      if (!wait_all_done(p, sh, prev_done)) return false;
      waited = true;
    }
    if (total - base >= 64 * MK_GATHER_MAXW) {   // a full batch: no per-word test
#pragma unroll
      for (int k = 0; k < MK_GATHER_MAXW; ++k) {
        const float v = ll_val(wv[k]);
        dst[base + k * 64 + lane] = v;
        acc = fmaf(v, v, acc);
      }
    } else {
#pragma unroll
      for (int k = 0; k < MK_GATHER_MAXW; ++k) {
        const int idx = base + k * 64 + lane;
        if (idx < total) {
          const float v = ll_val(wv[k]);
          dst[idx] = v;
          acc = fmaf(v, v, acc);
        }
      }
    }
  }
  if (!waited && !wait_all_done(p, sh, prev_done)) return false;
  if (ss) *ss = acc;
  return true;
}

// RMSNorm staging: act = x * (1 / sqrt(mean(x^2) + eps)) * g, with x the residual
// stream (the embedding row for the first layer).  Rows [res_r0, res_r0 + res_n) of the
// raw x are kept for the residual add of the next O / DOWN instruction.  The gains go
// to LDS before any wait.  Vectors of up to 64 * MK_GATHER_MAXW values stay in
// registers between the sum of squares and the scaled write (one LDS pass); longer ones
// are normalised in place in a second pass.
__device__ __forceinline__ bool stage_norm(const MkParams& p, MkShared& sh, const u64* src, const uint16_t* gain,
                                           int res_r0, int res_n, int i, uint32_t epoch, int lane) {
  const int d = p.d, npair = d >> 1;
  for (int b0 = 0; b0 < npair; b0 += 64 * 16) {   // gain pairs, 16 loads per lane per batch
    uint32_t gp[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) gp[k] = ((const uint32_t*)gain)[min(b0 + k * 64 + lane, npair - 1)];
#pragma unroll
    for (int k = 0; k < 16; ++k) pin(gp[k]);
#pragma unroll
    for (int k = 0; k < 16; ++k)   // lanes past the end rewrite the last pair with its own value
      ((uint32_t*)sh.gain)[min(b0 + k * 64 + lane, npair - 1)] = gp[k];
  }
  if (d <= 64 * MK_GATHER_MAXW) {
    const int kmax = d >> 6;   // hidden is a multiple of 64: word k is in range iff k < kmax
    float xv[MK_GATHER_MAXW];
    if (src == nullptr) {
      const uint16_t* e = p.embed + (size_t)sh.token * d;
      uint32_t eb[MK_GATHER_MAXW];
#pragma unroll
      for (int k = 0; k < MK_GATHER_MAXW; ++k) eb[k] = e[min(k * 64 + lane, d - 1)];
#pragma unroll
      for (int k = 0; k < MK_GATHER_MAXW; ++k) pin(eb[k]);
#pragma unroll
      for (int k = 0; k < MK_GATHER_MAXW; ++k) xv[k] = k * 64 + lane < d ? bf16f((uint16_t)eb[k]) : 0.f;
    } else {
      u64 wv[MK_GATHER_MAXW];
      if (!poll_batch(p, sh, src, d, 0, wv, epoch, lane)) return false;
      trace_mark(p, blockIdx.x, i, 1, lane);
#pragma unroll
      for (int k = 0; k < MK_GATHER_MAXW; ++k) xv[k] = k < kmax ? ll_val(wv[k]) : 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k) ss = fmaf(xv[k], xv[k], ss);
    const float rinv = 1.0f / sqrtf(wave_sum(ss) / (float)d + p.eps);
    // All LDS reads first, then all writes: a read issued after a write waits for it.
    uint32_t gl[MK_GATHER_MAXW];
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k) gl[k] = sh.gain[(k < kmax ? k * 64 : 0) + lane];
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k) pin(gl[k]);
    float nv[MK_GATHER_MAXW];
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k) nv[k] = (xv[k] * rinv) * bf16f((uint16_t)gl[k]);
    // Residual rows res_r0 + j (j < res_n <= 64) lie in words k0 and k0 + 1: pick those two
    // words with uniform selects, then fetch each row's value from the lane that holds it.
    const int k0 = res_r0 >> 6;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k) {
      a0 = k == k0 ? xv[k] : a0;
      a1 = k == k0 + 1 ? xv[k] : a1;
    }
    const int ridx = res_r0 + lane;
    const float b0 = __shfl(a0, ridx & 63), b1 = __shfl(a1, ridx & 63);
    if (!wait_all_done(p, sh, i)) return false;
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k)
      if (k < kmax) sh.act[k * 64 + lane] = nv[k];
    if (lane < res_n) sh.xres[lane] = (ridx >> 6) == k0 ? b0 : b1;
    return true;
  }
  float ss = 0.f;
  if (src == nullptr) {
    const uint16_t* e = p.embed + (size_t)sh.token * d;
    if (!wait_all_done(p, sh, i)) return false;
    for (int b0 = 0; b0 < d; b0 += 64 * 16) {
      uint32_t eb[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) eb[k] = e[min(b0 + k * 64 + lane, d - 1)];
#pragma unroll
      for (int k = 0; k < 16; ++k) pin(eb[k]);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int idx = b0 + k * 64 + lane;
        const float v = idx < d ? bf16f((uint16_t)eb[k]) : 0.f;
        if (idx < d) sh.act[idx] = v;
        ss = fmaf(v, v, ss);
      }
    }
  } else {
    if (!gather(p, sh, src, d, sh.act, i, epoch, lane, &ss)) return false;
  }
  const float rinv = 1.0f / sqrtf(wave_sum(ss) / (float)d + p.eps);
  lds_fence();
  for (int j = lane; j < res_n; j += 64) sh.xres[j] = sh.act[res_r0 + j];
  for (int idx = lane; idx < d; idx += 64) sh.act[idx] = (sh.act[idx] * rinv) * bf16f(sh.gain[idx]);
  return true;
}

__device__ __forceinline__ bool stage_raw(const MkParams& p, MkShared& sh, const u64* src, int n, int i,
                                          uint32_t epoch, int lane) {
  return gather(p, sh, src, n, sh.act, i, epoch, lane, nullptr);
}

// Attention staging for item (kv head g, split s): q of the group's heads, the new k
// and v; RoPE on q and k; k, v rounded to bf16 (what the cache holds).  The split that
// contains the current position writes k, v into cache slot pos.  Everything happens in
// registers between the poll and one batch of LDS writes.  Word idx = 64j + lane of the
// group holds element e = idx % hd of head idx / hd; its rotation partner e +- hd/2 is
// in lane ^ 32 of the same word (hd 64) or in the same lane of word j ^ 1 (hd 128).
constexpr int MK_ATTN_NW = 12;   // (4 + 2) heads x 128 / 64: words per lane of the largest group
__device__ __forceinline__ bool stage_attn(const MkParams& p, MkShared& sh, const MkInstr& in, const StepGeo& g,
                                           int i, uint32_t epoch, int lane) {
  const int hd = p.hd, hpg = p.hpg, half = hd >> 1, l = in.layer, gi = in.a;
  const int total = (hpg + 2) * hd;
  const u64* src = p.ll_qkv + (size_t)l * p.nqkv + (size_t)gi * total;   // group-major q | k | v
  const float* cs = p.rope + (size_t)g.pos * hd + 2 * (lane & (half - 1));  // [half][2], e % half == lane % half
  const float c = cs[0], sn = cs[1];
  u64 wv[MK_ATTN_NW];
  if (!poll_batch<MK_ATTN_NW>(p, sh, src, total, 0, wv, epoch, lane)) return false;
  trace_mark(p, blockIdx.x, i, 1, lane);
  float v[MK_ATTN_NW];
#pragma unroll
  for (int j = 0; j < MK_ATTN_NW; ++j) v[j] = ll_val(wv[j]);
  float pr[MK_ATTN_NW];   // rotation partners
  const bool hd64 = hd == 64;
#pragma unroll
  for (int j = 0; j < MK_ATTN_NW; ++j) {
    const float x = __shfl_xor(v[j], 32);
    pr[j] = hd64 ? x : v[j ^ 1];
  }
  const int kbase = hpg * hd, vbase = (hpg + 1) * hd;   // offsets of k and v in the group
  const bool has_pos = in.b == g.s_eff - 1;
  uint16_t* kslot = p.kv + ((((size_t)l * 2) * p.hkv + gi) * p.max_ctx + g.pos) * hd;
  uint16_t* vslot = kslot + (size_t)p.hkv * p.max_ctx * hd;
#pragma unroll
  for (int j = 0; j < MK_ATTN_NW; ++j) {
    const int idx = j * 64 + lane;
    const bool first = hd64 ? lane < 32 : (j & 1) == 0;   // e < half
    if (idx < vbase) {   // q heads and k: rotate
      v[j] = first ? __fsub_rn(__fmul_rn(v[j], c), __fmul_rn(pr[j], sn))
                   : __fadd_rn(__fmul_rn(v[j], c), __fmul_rn(pr[j], sn));
    }
    if (idx >= kbase && idx < total) {   // k and v: what the cache holds
      const uint16_t b = f2bf(v[j]);
      v[j] = bf16f(b);
      if (has_pos) (idx < vbase ? kslot : vslot)[idx - (idx < vbase ? kbase : vbase)] = b;
    }
  }
  if (!wait_all_done(p, sh, i)) return false;
#pragma unroll
  for (int j = 0; j < MK_ATTN_NW; ++j)
    if (j * 64 + lane < total) sh.act[j * 64 + lane] = v[j];
  return true;
}

__device__ __forceinline__ size_t part_index(const MkParams& p, int l, int g, int h, int s) {
  return ((((size_t)l * p.hkv + g) * p.hpg + h) * p.s_max + s) * (size_t)(p.hd + 2);
}

// After the compute waves: combine their partials (and the current position's key)
// into this split's (m, l, o), then either write o (single split), publish the split,
// and/or merge all splits of one head (CUs with split index < heads per group).  Lane
// `lane` handles elements lane + 64c of each head.  LDS reads are batched ahead of use.
template <int HD, int HPG>
__device__ __forceinline__ bool attn_finalize(const MkParams& p, MkShared& sh, const MkInstr& in, const StepGeo& g,
                                              int i, uint32_t epoch, int lane) {
  constexpr int E = HD / 64, STRIDE = HD + 2;
  const int l = in.layer, gi = in.a, s = in.b;
  if (s < g.s_eff) {
    const bool has_pos = s == g.s_eff - 1;
    const float* part = sh.act + MK_PART_OFF;
    float mw[MK_NC][HPG], lw[MK_NC][HPG], ow[MK_NC][HPG][E], qv[HPG][E], kn[E], vn[E];
#pragma unroll
    for (int w = 0; w < MK_NC; ++w)
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        mw[w][h] = part[(w * HPG + h) * STRIDE];
        lw[w][h] = part[(w * HPG + h) * STRIDE + 1];
#pragma unroll
        for (int c = 0; c < E; ++c) ow[w][h][c] = part[(w * HPG + h) * STRIDE + 2 + c * 64 + lane];
      }
#pragma unroll
    for (int c = 0; c < E; ++c) {
#pragma unroll
      for (int h = 0; h < HPG; ++h) qv[h][c] = sh.act[h * HD + c * 64 + lane];
      kn[c] = sh.act[HPG * HD + c * 64 + lane];
      vn[c] = sh.act[(HPG + 1) * HD + c * 64 + lane];
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
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      float M = sp[h];
#pragma unroll
      for (int w = 0; w < MK_NC; ++w) M = fmaxf(M, mw[w][h]);
      float L = 0.f, wt[MK_NC];
#pragma unroll
      for (int w = 0; w < MK_NC; ++w) {
        wt[w] = mw[w][h] == -INFINITY ? 0.f : __expf(mw[w][h] - M);
        L = fmaf(lw[w][h], wt[w], L);
      }
      const float wp = has_pos ? __expf(sp[h] - M) : 0.f;
      L += wp;
#pragma unroll
      for (int c = 0; c < E; ++c) {
        float o = wp * vn[c];
#pragma unroll
        for (int w = 0; w < MK_NC; ++w) o = fmaf(ow[w][h][c], wt[w], o);
        const int e = c * 64 + lane;
        if (g.s_eff == 1)
          ll_store(p.ll_o + (size_t)l * p.nq + (gi * HPG + h) * HD + e, o / L, epoch);
        else
          ll_store(p.ll_part + part_index(p, l, gi, h, s) + 2 + e, o, epoch);
      }
      if (g.s_eff > 1 && lane == 0) {
        ll_store(p.ll_part + part_index(p, l, gi, h, s), M, epoch);
        ll_store(p.ll_part + part_index(p, l, gi, h, s) + 1, L, epoch);
      }
    }
  }
  if (g.s_eff > 1 && s < HPG) {
    // Merge head s of this group over all splits.
    const int h = s;
    lds_fence();
    if (!gather(p, sh, p.ll_part + part_index(p, l, gi, h, 0), g.s_eff * STRIDE, sh.act, i + 1, epoch, lane,
                nullptr))
      return false;
    lds_fence();
    float M = -INFINITY;
    for (int t = 0; t < g.s_eff; ++t) M = fmaxf(M, sh.act[t * STRIDE]);
    float L = 0.f, o[E];
#pragma unroll
    for (int c = 0; c < E; ++c) o[c] = 0.f;
    for (int t = 0; t < g.s_eff; ++t) {
      const float mt = sh.act[t * STRIDE];
      const float wt = mt == -INFINITY ? 0.f : __expf(mt - M);
      L = fmaf(sh.act[t * STRIDE + 1], wt, L);
#pragma unroll
      for (int c = 0; c < E; ++c) o[c] = fmaf(sh.act[t * STRIDE + 2 + c * 64 + lane], wt, o[c]);
    }
#pragma unroll
    for (int c = 0; c < E; ++c)
      ll_store(p.ll_o + (size_t)l * p.nq + (gi * HPG + h) * HD + c * 64 + lane, o[c] / L, epoch);
  }
  return true;
}

// Final argmax: combine the waves, publish the CU's key, take a ticket; the last CU
// reduces all keys, writes the next token and advances the epoch for the next step.
__device__ __forceinline__ void lm_finalize(const MkParams& p, MkShared& sh, uint32_t epoch, int cu, int lane) {
  u64 key = 0;
  for (int w = 0; w < MK_NC; ++w) key = sh.amax[w] > key ? sh.amax[w] : key;
  uint32_t old = 0;
  if (lane == 0) {
    __hip_atomic_store(p.amax + cu, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __hip_atomic_fetch_add(&p.ctrl->ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
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
    __hip_atomic_store(&p.ctrl->epoch, epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void leader_wave(const MkParams& p, MkShared& sh, cinstr_t list, int nins, const StepGeo& g,
                            int lane, uint32_t epoch, int cu) {
  for (int i = 0; i < nins; ++i) {
    const MkInstr in = list[i];
    const int l = in.layer;
    lane = opaque(lane);
    trace_mark(p, cu, i, 0, lane);
    bool ok = true;
    switch (in.op) {
      case MK_OP_QKV:
        ok = stage_norm(p, sh, l == 0 ? nullptr : p.ll_x + (size_t)(2 * l) * p.d, ((clayers_t)p.layers)[l].attn_norm,
                        in.res_r0, in.res_n, i, epoch, lane);
        break;
      case MK_OP_ATTN:
        if (in.b < g.s_eff) ok = stage_attn(p, sh, in, g, i, epoch, lane);
        break;
      case MK_OP_O:
        ok = stage_raw(p, sh, p.ll_o + (size_t)l * p.nq, p.nq, i, epoch, lane);
        break;
      case MK_OP_GATEUP:
        ok = stage_norm(p, sh, p.ll_x + (size_t)(2 * l + 1) * p.d, ((clayers_t)p.layers)[l].mlp_norm, in.res_r0, in.res_n, i,
                        epoch, lane);
        break;
      case MK_OP_DOWN:
        ok = stage_raw(p, sh, p.ll_a + (size_t)l * p.F + in.k0, in.kn, i, epoch, lane);
        break;
      default:  // MK_OP_LMHEAD (its record carries layer = n_layers: the last residual version)
        ok = stage_norm(p, sh, p.ll_x + (size_t)(2 * l) * p.d, ((clayers_t)p.layers)[l].attn_norm, 0, 0, i,
                        epoch, lane);
        break;
    }
    if (!ok) return;
    lds_fence();
    if (lane == 0) lds_store(&sh.act_seq, i + 1);
    trace_mark(p, cu, i, 2, lane);
    if (in.op == MK_OP_ATTN) {
      if (!wait_all_done(p, sh, i + 1)) return;
      bool fin;
      if (p.hd == 64) {
        fin = p.hpg == 4 ? attn_finalize<64, 4>(p, sh, in, g, i, epoch, lane)
            : p.hpg == 2 ? attn_finalize<64, 2>(p, sh, in, g, i, epoch, lane)
                         : attn_finalize<64, 1>(p, sh, in, g, i, epoch, lane);
      } else {
        fin = p.hpg == 4 ? attn_finalize<128, 4>(p, sh, in, g, i, epoch, lane)
            : p.hpg == 2 ? attn_finalize<128, 2>(p, sh, in, g, i, epoch, lane)
                         : attn_finalize<128, 1>(p, sh, in, g, i, epoch, lane);
      }
      if (!fin) return;
    } else if (in.op == MK_OP_LMHEAD) {
      if (!wait_all_done(p, sh, i + 1)) return;
      lm_finalize(p, sh, epoch, cu, lane);
    }
    trace_mark(p, cu, i, 3, lane);
  }
}

}  // namespace mkdev

// One decode step.  Grid: one work-group per CU (all resident: cooperative launch).
__global__ void __launch_bounds__(MK_THREADS) mk_step_kernel(MkParams p) {
  using namespace mkdev;
  __shared__ MkShared sh;
  // the wave index is uniform per wave; saying so keeps everything derived from it scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, cu = blockIdx.x;
  if (threadIdx.x == 0) {
    sh.act_seq = 0;
    sh.abort_flag = 0;
    for (int w = 0; w < MK_NC; ++w) {
      sh.done[w] = 0;
      sh.amax[w] = 0;
    }
    for (int k = 0; k < MK_MAX_SLOTS; ++k) {
      sh.full[k] = 0;
      sh.freed[k] = 0;
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
  const uint32_t epoch = sh.epoch;
  const int o0 = ((cint_t)p.plan_off)[cu];
  const int nins = ((cint_t)p.plan_off)[cu + 1] - o0;
  cinstr_t list = (cinstr_t)p.plan + o0;
  const StepGeo g = step_geo(p, p.pos);
  if (wave < MK_NC) compute_wave(p, sh, list, nins, g, wave, lane, epoch);
  else if (wave < MK_NC + MK_NL) loader_wave(p, sh, list, nins, g, wave - MK_NC, lane);
  else leader_wave(p, sh, list, nins, g, lane, epoch, cu);
}
