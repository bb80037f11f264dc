// Persistent decode-step interpreter for gfx950 (one work-group per CU).
//
// Design after the Hazy Research "Megakernel" article on Llama-3.2-1B, section
// "Megakernel: a fusion design from scratch", re-thought for CDNA4:
//
//  * Instruction interpreter.  Every CU walks its own ordered instruction list
//    (QKV, ATTN, O, GATEUP, DOWN x4 per layer, then LMHEAD) laid out by the host.
//  * Paged LDS with early weight loads.  The article pages shared memory so that the
//    next instruction's weights load while the current one computes.  Here each of
//    the MK_NC compute waves owns a ring of LDS pages and fills them with
//    global_load_lds_dwordx4 (HBM -> LDS, no registers) for its future pages, across
//    instruction boundaries and before the data an instruction depends on exists:
//    weights and cached keys never depend on this step's activations.  A page is
//    complete when the wave's vmcnt says so; the compiler is kept out of that
//    accounting (it would otherwise wait for every DMA before any LDS access).
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
//    and releases the compute waves, which then only touch LDS.
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
  char pages[MK_PAGES_BYTES];               // page rings, MK_NC x npw pages
  float xres[MK_MAX_RES_ROWS];              // x rows this CU's next residual adds to
  float rowacc[MK_MAX_RES_ROWS];            // DOWN partial sums over the K-chunks
  float rowres[MK_NC][64];                  // row results of the page being finished
  u64 amax[MK_NC];                          // per-wave argmax keys (LM head)
  int done[MK_NC];                          // instructions finished, per compute wave
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
// Sum within aligned groups of g lanes (g a power of two <= 64).
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

__device__ __forceinline__ int rows_per_page(const MkParams& p, const MkInstr& in) {
  const int seg = 2 * in.kn;
  return in.op == MK_OP_GATEUP ? p.page_bytes / (2 * seg) : p.page_bytes / seg;
}

__device__ __forceinline__ int instr_pages(const MkParams& p, const MkInstr& in, const StepGeo& g) {
  if (in.op == MK_OP_ATTN) {
    if (in.b >= g.s_eff) return 0;
    int j0, j1, ce;
    attn_range(g, in.b, &j0, &j1, &ce);
    const int cached = ce - j0;
    return cached > 0 ? (cached + g.ppp - 1) / g.ppp : 0;
  }
  const int rpp = rows_per_page(p, in);
  return (in.n + rpp - 1) / rpp;
}

__device__ __forceinline__ const uint16_t* row_ptr(const MkParams& p, const MkInstr& in, int row) {
  const MkLayerPtrs L = ((clayers_t)p.layers)[in.layer < p.n_layers ? in.layer : 0];
  switch (in.op) {
    case MK_OP_QKV:
      if (row < p.nq) return L.wq + (size_t)row * p.d;
      if (row < p.nq + p.nkv) return L.wk + (size_t)(row - p.nq) * p.d;
      return L.wv + (size_t)(row - p.nq - p.nkv) * p.d;
    case MK_OP_O: return L.wo + (size_t)row * p.nq;
    case MK_OP_DOWN: return L.wd + (size_t)row * p.F;
    default: return p.lm_head + (size_t)row * p.d;   // MK_OP_LMHEAD
  }
}

// Issue the DMA of page `pg` of instruction `in` into the LDS page at `slot`: always
// p.lpp load instructions of 1 KiB, so that vmcnt accounting is a multiple of lpp.
// Lanes beyond the page payload re-read the page's first 16 bytes (always valid).
__device__ __forceinline__ void issue_page(const MkParams& p, const MkInstr& in, int pg,
                                           const StepGeo& g, uint32_t slot, int lane) {
  if (in.op == MK_OP_ATTN) {
    int j0, j1, ce;
    attn_range(g, in.b, &j0, &j1, &ce);
    const int q0 = j0 + pg * g.ppp;
    const int np = min(g.ppp, ce - q0);
    const int rowb = 2 * p.hd;
    const int kbytes = np * rowb;
    const size_t head = ((size_t)(in.layer * 2) * p.hkv + in.a) * p.max_ctx;
    const char* kb = (const char*)(p.kv + (head + q0) * p.hd);
    const char* vb = (const char*)(p.kv + (head + (size_t)p.hkv * p.max_ctx + q0) * p.hd);
    for (int u = 0; u < p.lpp; ++u) {
      const int o = u * 1024 + lane * 16;
      const char* a = o < kbytes ? kb + o : (o < 2 * kbytes ? vb + (o - kbytes) : kb);
      dma16(a, slot + u * 1024);
    }
    return;
  }
  const int seg = 2 * in.kn;
  const int rpp = rows_per_page(p, in);
  const int first = pg * rpp;
  const int m = min(rpp, in.n - first);                 // rows (GATEUP: pairs) in the page
  const int payload = (in.op == MK_OP_GATEUP ? 2 * m : m) * seg;
  const MkLayerPtrs L = ((clayers_t)p.layers)[in.layer < p.n_layers ? in.layer : 0];
  for (int u = 0; u < p.lpp; ++u) {
    int o = u * 1024 + lane * 16;
    if (o >= payload) o = 0;
    const int j = o / seg;
    const int cb = o - j * seg;
    const uint16_t* rp;
    if (in.op == MK_OP_GATEUP)
      rp = j < m ? L.wg + (size_t)(in.r0 + first + j) * p.d : L.wu + (size_t)(in.r0 + first + j - m) * p.d;
    else
      rp = row_ptr(p, in, in.r0 + first + j);
    dma16((const char*)(rp + in.k0) + cb, slot + u * 1024);
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

// ------------------------------------------------------------------ compute waves
// Finish one GEMV page: dot every row of the page with the staged activation.
__device__ __forceinline__ void gemv_page(const MkParams& p, MkShared& sh, const MkInstr& in, int pg,
                                          const char* page, int w, int lane, uint32_t epoch,
                                          u64* best) {
  const int seg = 2 * in.kn;
  const int rpp = rows_per_page(p, in);
  const int first = pg * rpp;
  const int m = min(rpp, in.n - first);
  const int nrows = in.op == MK_OP_GATEUP ? 2 * m : m;
  float* res = sh.rowres[w];
  if (seg >= 1024) {
    const int upr = seg >> 10;
    for (int r = 0; r < nrows; ++r) {
      float acc = 0.f;
      for (int u = 0; u < upr; ++u) {
        const uint4 wv = *(const uint4*)(page + (r * upr + u) * 1024 + lane * 16);
        acc = dot8(wv, sh.act + u * 512 + lane * 8, acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) res[r] = acc;
    }
  } else {
    const int lpr = seg >> 4;             // lanes per row
    const int rpu = 64 / lpr;             // rows per 1 KiB unit
    const int c = lane & (lpr - 1);
    for (int u = 0; u * rpu < nrows; ++u) {
      const uint4 wv = *(const uint4*)(page + u * 1024 + lane * 16);
      float acc = dot8(wv, sh.act + c * 8, 0.f);
      acc = group_sum(acc, lpr);
      const int r = u * rpu + lane / lpr;
      if (c == 0 && r < nrows) res[r] = acc;
    }
  }
  lds_fence();
  // Epilogue: lane j finishes row (or gate/up pair) j of the page.
  const int l = in.layer;
  const int j = lane;
  if (j >= m) return;
  const int row = in.r0 + first + j;
  switch (in.op) {
    case MK_OP_QKV: {
      // group-major: [kv head g][q heads of g | k_g | v_g][hd]
      const int grp = (p.hpg + 2) * p.hd;
      int idx;
      if (row < p.nq) {
        const int h = row / p.hd;
        idx = (h / p.hpg) * grp + (h % p.hpg) * p.hd + (row - h * p.hd);
      } else if (row < p.nq + p.nkv) {
        const int r = row - p.nq;
        idx = (r / p.hd) * grp + p.hpg * p.hd + (r % p.hd);
      } else {
        const int r = row - p.nq - p.nkv;
        idx = (r / p.hd) * grp + (p.hpg + 1) * p.hd + (r % p.hd);
      }
      ll_store(p.ll_qkv + (size_t)l * p.nqkv + idx, res[j], epoch);
      break;
    }
    case MK_OP_O:
      ll_store(p.ll_x + (size_t)(2 * l + 1) * p.d + row, sh.xres[row - in.r0] + res[j], epoch);
      break;
    case MK_OP_GATEUP: {
      const float gt = res[j], up = res[m + j];
      const float a = (gt / (1.0f + __expf(-gt))) * up;
      ll_store(p.ll_a + (size_t)l * p.F + row, a, epoch);
      break;
    }
    case MK_OP_DOWN: {
      const int k = row - in.r0;
      const float acc = (in.a == 0 ? 0.f : sh.rowacc[k]) + res[j];
      if (in.a + 1 < in.b) sh.rowacc[k] = acc;
      else ll_store(p.ll_x + (size_t)(2 * l + 2) * p.d + row, sh.xres[k] + acc, epoch);
      break;
    }
    default: {  // MK_OP_LMHEAD
      p.logits[row] = res[j];
      const u64 key = amax_key(res[j], (uint32_t)row);
      if (key > *best) *best = key;
      break;
    }
  }
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

// One page of cached keys/values: [npos][HD] keys, then [npos][HD] values.
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
        part = group_sum(part, LPP);
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

// Reduce the wave's state over its position groups and leave (m, l, o) in LDS.
template <int HD, int HPG>
__device__ __forceinline__ void attn_publish(AttnState<HD, HPG>& st, MkShared& sh, int w, int lane) {
  constexpr int LPP = HD / 8;
  float* part = sh.act + MK_PART_OFF + w * HPG * (HD + 2);
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    float l = st.l[h];
#pragma unroll
    for (int off = LPP; off < 64; off <<= 1) l += __shfl_xor(l, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = st.o[h][e];
#pragma unroll
      for (int off = LPP; off < 64; off <<= 1) v += __shfl_xor(v, off);
      if (lane < LPP) part[h * (HD + 2) + 2 + lane * 8 + e] = v;
    }
    if (lane == 0) {
      part[h * (HD + 2)] = st.m[h];
      part[h * (HD + 2) + 1] = l;
    }
  }
}


// ------------------------------------------------------------------ page ring
// The stream of pages one compute wave consumes, in consumption order.  Page pg of
// instruction i goes to wave (base_i + pg) % MK_NC, base_i = pages of instructions
// before i, so successive instructions start on successive waves.
__device__ __forceinline__ int first_page(int w, int base) { return ((w - base) % MK_NC + MK_NC) % MK_NC; }

struct Ring {
  const MkParams* p;
  cinstr_t list;
  int nins;
  StepGeo g;
  int w, lane;
  const char* base;       // this wave's pages (LDS)
  uint32_t base_lds;
  int issued, consumed;
  int si, spg, sbase, snp;  // issue cursor: instruction, page, pages before it, its pages

  __device__ __forceinline__ void settle() {
    while (si < nins && spg >= snp) {
      sbase += snp;
      ++si;
      if (si < nins) {
        snp = instr_pages(*p, list[si], g);
        spg = first_page(w, sbase);
      }
    }
  }
  __device__ __forceinline__ void init() {
    issued = consumed = 0;
    si = 0;
    sbase = 0;
    snp = nins > 0 ? instr_pages(*p, list[0], g) : 0;
    spg = first_page(w, 0);
    settle();
    for (int k = 0; k < p->npw; ++k) issue();
  }
  __device__ __forceinline__ void issue() {
    if (si >= nins) return;
    issue_page(*p, list[si], spg, g, base_lds + (uint32_t)((issued % p->npw) * p->page_bytes), lane);
    ++issued;
    spg += MK_NC;
    settle();
  }
  // Oldest page in flight, once it has landed.
  __device__ __forceinline__ const char* front() {
    wait_vmcnt((issued - consumed - 1) * p->lpp);
    return base + (consumed % p->npw) * p->page_bytes;
  }
  __device__ __forceinline__ void pop() {
    ++consumed;
    issue();
  }
};

template <int HD, int HPG>
__device__ __forceinline__ void attn_run(const MkParams& p, MkShared& sh, const MkInstr& in, int np, int p0,
                                         Ring& r, int w, int lane) {
  AttnState<HD, HPG> st;
  attn_init<HD, HPG>(st, sh, lane);
  int j0, j1, ce;
  attn_range(r.g, in.b, &j0, &j1, &ce);
  for (int pg = p0; pg < np; pg += MK_NC) {
    const char* page = r.front();
    const int npos = min(r.g.ppp, ce - (j0 + pg * r.g.ppp));
    attn_page<HD, HPG>(st, page, npos, p.attn_scale, lane);
    r.pop();
  }
  attn_publish<HD, HPG>(st, sh, w, lane);
}

__device__ __forceinline__ void compute_wave(const MkParams& p, MkShared& sh, cinstr_t list, int nins,
                             const StepGeo& g, int w, int lane, uint32_t epoch) {
  Ring r;
  r.p = &p;
  r.list = list;
  r.nins = nins;
  r.g = g;
  r.w = w;
  r.lane = lane;
  r.base = sh.pages + w * p.npw * p.page_bytes;
  r.base_lds = lds_addr(r.base);
  r.init();
  int cbase = 0;
  for (int i = 0; i < nins; ++i) {
    const MkInstr in = list[i];
    lane = opaque(lane);
    r.lane = lane;
    const int np = instr_pages(p, in, g);
    const int p0 = first_page(w, cbase);
    cbase += np;
    if (!wait_flag(p, sh, &sh.act_seq, i + 1, false)) break;
    if (in.op == MK_OP_ATTN) {
      // A split that is inactive at this position does nothing: in particular it must not
      // write partials into act, which other waves may still read for the previous
      // instruction (the leader releases inactive splits without waiting for them).
      if (in.b >= g.s_eff) {
      } else if (p.hd == 64) {
        if (p.hpg == 4) attn_run<64, 4>(p, sh, in, np, p0, r, w, lane);
        else if (p.hpg == 2) attn_run<64, 2>(p, sh, in, np, p0, r, w, lane);
        else attn_run<64, 1>(p, sh, in, np, p0, r, w, lane);
      } else {
        if (p.hpg == 4) attn_run<128, 4>(p, sh, in, np, p0, r, w, lane);
        else if (p.hpg == 2) attn_run<128, 2>(p, sh, in, np, p0, r, w, lane);
        else attn_run<128, 1>(p, sh, in, np, p0, r, w, lane);
      }
    } else {
      u64 best = 0;
      for (int pg = p0; pg < np; pg += MK_NC) {
        const char* page = r.front();
        gemv_page(p, sh, in, pg, page, w, lane, epoch, &best);
        r.pop();
      }
      if (in.op == MK_OP_LMHEAD) {
        best = wave_max_u64(best);
        if (lane == 0) sh.amax[w] = best;
      }
    }
    lds_fence();
    if (lane == 0) lds_store(&sh.done[w], i + 1);
  }
  wait_vmcnt(0);   // no page load may land after the wave has left
}

// ------------------------------------------------------------------ leader wave
// Poll words [base, base + 64*MK_GATHER_MAXW) of src until all carry this step's
// epoch.  Word base + 64k + lane lands in wv[k].
__device__ __forceinline__ bool poll_batch(const MkParams& p, MkShared& sh, const u64* src, int total, int base,
                                           u64 (&wv)[MK_GATHER_MAXW], uint32_t epoch, int lane) {
  const u64* q = src + base + lane;
  const int lim = total - base - lane;      // word k is in range when 64k < lim
#pragma unroll
  for (int k = 0; k < MK_GATHER_MAXW; ++k) {
    wv[k] = (u64)epoch << 32;
    if (k * 64 < lim) wv[k] = ll_load(q + k * 64);
  }
  Waiter wt(true);
  for (;;) {
    bool bad = false;
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k) bad |= !ll_ok(wv[k], epoch);
    if (__ballot(bad) == 0) return true;
    if (wt.tick(p, sh)) return false;
#pragma unroll
    for (int k = 0; k < MK_GATHER_MAXW; ++k)
      if (!ll_ok(wv[k], epoch)) wv[k] = ll_load(q + k * 64);
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
    if (!waited) {
      if (!wait_all_done(p, sh, prev_done)) return false;
      waited = true;
    }
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
  if (!waited && !wait_all_done(p, sh, prev_done)) return false;
  if (ss) *ss = acc;
  return true;
}

// RMSNorm staging: act = x / sqrt(mean(x^2) + eps) * g, with x the residual stream
// (the embedding row for the first layer).  Rows [res_r0, res_r0 + res_n) of the raw x
// are kept for the residual add of the next O / DOWN instruction.
__device__ __forceinline__ bool stage_norm(const MkParams& p, MkShared& sh, const u64* src, const uint16_t* gain,
                           int res_r0, int res_n, int i, uint32_t epoch, int lane) {
  const int d = p.d;
  const int npair = d >> 1;
  uint32_t gw[MK_ACT_FLOATS / 128];                 // gain pairs, prefetched
#pragma unroll
  for (int k = 0; k < MK_ACT_FLOATS / 128; ++k) {
    const int q = k * 64 + lane;
    gw[k] = q < npair ? ((const uint32_t*)gain)[q] : 0u;
  }
  float ss = 0.f;
  if (src == nullptr) {
    const uint16_t* e = p.embed + (size_t)sh.token * d;
    if (!wait_all_done(p, sh, i)) return false;
    for (int idx = lane; idx < d; idx += 64) {
      const float v = bf16f(e[idx]);
      sh.act[idx] = v;
      ss = fmaf(v, v, ss);
    }
  } else {
    if (!gather(p, sh, src, d, sh.act, i, epoch, lane, &ss)) return false;
  }
  ss = wave_sum(ss);
  const float rms = sqrtf(ss / (float)d + p.eps);
  lds_fence();
  for (int j = lane; j < res_n; j += 64) sh.xres[j] = sh.act[res_r0 + j];
#pragma unroll
  for (int k = 0; k < MK_ACT_FLOATS / 128; ++k) {
    const int q = k * 64 + lane;
    if (q < npair) {
      const float a0 = sh.act[2 * q], a1 = sh.act[2 * q + 1];
      sh.act[2 * q] = (a0 / rms) * bf_lo(gw[k]);
      sh.act[2 * q + 1] = (a1 / rms) * bf_hi(gw[k]);
    }
  }
  return true;
}

__device__ __forceinline__ bool stage_raw(const MkParams& p, MkShared& sh, const u64* src, int n, int i,
                                          uint32_t epoch, int lane) {
  return gather(p, sh, src, n, sh.act, i, epoch, lane, nullptr);
}

// Attention staging for item (kv head g, split s): q of the group's heads, the new k
// and v; RoPE on q and k; k, v rounded to bf16 (what the cache holds).  The split that
// contains the current position writes k, v into cache slot pos.
__device__ __forceinline__ bool stage_attn(const MkParams& p, MkShared& sh, const MkInstr& in, const StepGeo& g, int i,
                           uint32_t epoch, int lane) {
  const int hd = p.hd, hpg = p.hpg, half = hd >> 1, l = in.layer, gi = in.a;
  const int total = (hpg + 2) * hd;
  const u64* src = p.ll_qkv + (size_t)l * p.nqkv + (size_t)gi * total;   // group-major q | k | v
  if (!gather(p, sh, src, total, sh.act, i, epoch, lane, nullptr)) return false;
  lds_fence();
  const float* cs = p.rope + (size_t)g.pos * hd;   // [half][2]
  for (int t = lane; t < (hpg + 1) * half; t += 64) {
    const int hh = t / half, e = t - hh * half;
    float* v = sh.act + hh * hd;
    const float c = cs[2 * e], sn = cs[2 * e + 1];
    const float a = v[e], b = v[e + half];
    v[e] = __fsub_rn(__fmul_rn(a, c), __fmul_rn(b, sn));
    v[e + half] = __fadd_rn(__fmul_rn(b, c), __fmul_rn(a, sn));
  }
  lds_fence();
  const bool has_pos = in.b == g.s_eff - 1;
  uint16_t* kslot = p.kv + ((((size_t)l * 2) * p.hkv + gi) * p.max_ctx + g.pos) * hd;
  uint16_t* vslot = kslot + (size_t)p.hkv * p.max_ctx * hd;
  for (int e = lane; e < hd; e += 64) {
    const uint16_t kb = f2bf(sh.act[hpg * hd + e]);
    const uint16_t vb = f2bf(sh.act[(hpg + 1) * hd + e]);
    sh.act[hpg * hd + e] = bf16f(kb);
    sh.act[(hpg + 1) * hd + e] = bf16f(vb);
    if (has_pos) {
      kslot[e] = kb;
      vslot[e] = vb;
    }
  }
  return true;
}

__device__ __forceinline__ size_t part_index(const MkParams& p, int l, int g, int h, int s) {
  return ((((size_t)l * p.hkv + g) * p.hpg + h) * p.s_max + s) * (size_t)(p.hd + 2);
}

// After the compute waves: combine their partials (and the current position's key)
// into this split's (m, l, o), then either write o (single split), publish the split,
// and/or merge all splits of one head (CUs with split index < heads per group).
__device__ __forceinline__ bool attn_finalize(const MkParams& p, MkShared& sh, const MkInstr& in, const StepGeo& g, int i,
                              uint32_t epoch, int lane) {
  const int hd = p.hd, hpg = p.hpg, l = in.layer, gi = in.a, s = in.b;
  const int stride = hd + 2;
  if (s < g.s_eff) {
    const bool has_pos = s == g.s_eff - 1;
    for (int h = 0; h < hpg; ++h) {
      float M = -INFINITY;
      for (int w = 0; w < MK_NC; ++w) M = fmaxf(M, sh.act[MK_PART_OFF + (w * hpg + h) * stride]);
      float sp = -INFINITY;
      if (has_pos) {
        float acc = 0.f;
        for (int e = lane; e < hd; e += 64) acc = fmaf(sh.act[h * hd + e], sh.act[hpg * hd + e], acc);
        sp = wave_sum(acc) * p.attn_scale;
        M = fmaxf(M, sp);
      }
      float L = 0.f;
      float wgt[MK_NC];
      for (int w = 0; w < MK_NC; ++w) {
        const float mw = sh.act[MK_PART_OFF + (w * hpg + h) * stride];
        wgt[w] = mw == -INFINITY ? 0.f : __expf(mw - M);
        L = fmaf(sh.act[MK_PART_OFF + (w * hpg + h) * stride + 1], wgt[w], L);
      }
      const float wp = has_pos ? __expf(sp - M) : 0.f;
      L += wp;
      for (int e = lane; e < hd; e += 64) {
        float o = 0.f;
        for (int w = 0; w < MK_NC; ++w) o = fmaf(sh.act[MK_PART_OFF + (w * hpg + h) * stride + 2 + e], wgt[w], o);
        if (has_pos) o = fmaf(wp, sh.act[(hpg + 1) * hd + e], o);
        if (g.s_eff == 1)
          ll_store(p.ll_o + (size_t)l * p.nq + (gi * hpg + h) * hd + e, o / L, epoch);
        else
          ll_store(p.ll_part + part_index(p, l, gi, h, s) + 2 + e, o, epoch);
      }
      if (g.s_eff > 1 && lane == 0) {
        ll_store(p.ll_part + part_index(p, l, gi, h, s), M, epoch);
        ll_store(p.ll_part + part_index(p, l, gi, h, s) + 1, L, epoch);
      }
    }
  }
  if (g.s_eff > 1 && s < hpg) {
    // Merge head s of this group over all splits.
    const int h = s;
    lds_fence();
    if (!gather(p, sh, p.ll_part + part_index(p, l, gi, h, 0), g.s_eff * stride, sh.act, i + 1, epoch, lane,
                nullptr))
      return false;
    lds_fence();
    float M = -INFINITY;
    for (int t = 0; t < g.s_eff; ++t) M = fmaxf(M, sh.act[t * stride]);
    float L = 0.f;
    for (int t = 0; t < g.s_eff; ++t) {
      const float mt = sh.act[t * stride];
      if (mt != -INFINITY) L = fmaf(sh.act[t * stride + 1], __expf(mt - M), L);
    }
    for (int e = lane; e < hd; e += 64) {
      float o = 0.f;
      for (int t = 0; t < g.s_eff; ++t) {
        const float mt = sh.act[t * stride];
        if (mt != -INFINITY) o = fmaf(sh.act[t * stride + 2 + e], __expf(mt - M), o);
      }
      ll_store(p.ll_o + (size_t)l * p.nq + (gi * hpg + h) * hd + e, o / L, epoch);
    }
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
  for (int c = lane; c < p.n_cus; c += 64) {
    const u64 k = __hip_atomic_load(p.amax + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    best = k > best ? k : best;
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
    if (in.op == MK_OP_ATTN) {
      if (!wait_all_done(p, sh, i + 1)) return;
      if (!attn_finalize(p, sh, in, g, i, epoch, lane)) return;
    } else if (in.op == MK_OP_LMHEAD) {
      if (!wait_all_done(p, sh, i + 1)) return;
      lm_finalize(p, sh, epoch, cu, lane);
    }
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
  else leader_wave(p, sh, list, nins, g, lane, epoch, cu);
}
