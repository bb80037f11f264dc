// C ABI of the decode megakernel library: context, static schedule upload, launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_kernel.h"
#include "mk_plan.h"
#include "mk_shapes.h"

struct mk_ctx {
  mk_config cfg{};
  int device = -1;
  int n_cus = 0;
  bool plan_only = false;
  bool loaded = false;
  bool needs_reset = false;
  long long watchdog_us = 2000000;
  // Loader pages in flight per loader for staged instructions.  Two (four per CU) keep HBM
  // streaming at full rate while polls queue behind fewer loads: 556.3 vs 557.9 us per
  // step at the Llama-3.2-1B shape and 3258 vs 3293 us at the Llama-3.1-8B shape against
  // four, once the kernel's code fit the instruction cache.
  int demand_depth = 2;
  bool ll_uncached = true;   // communication words in uncached memory (else cached)
  MkPlan plan;
  const void* kernel = nullptr;   // the step kernel compiled for this shape
  const void* kernel_traced = nullptr;   // the same, with the per-instruction trace
  // borrowed weights
  const uint16_t* embed = nullptr;
  const uint16_t* lm_head = nullptr;
  const uint16_t* final_norm = nullptr;
  // owned device memory
  MkLayerPtrs* d_layers = nullptr;
  int32_t* d_off = nullptr;
  MkInstr* d_plan = nullptr;
  float* d_rope = nullptr;
  unsigned long long* d_ll = nullptr;
  size_t ll_words = 0;
  size_t off_x = 0, off_qkv = 0, off_part = 0, off_o = 0, off_a = 0;
  unsigned long long* d_amax = nullptr;
  MkCtrl* d_ctrl = nullptr;
  int32_t* d_next = nullptr;   // argmax sink when the caller passes none
  unsigned long long* trace = nullptr;   // borrowed device buffer, or null
  int trace_len = 0;
  bool used_static = false;              // has run steps on the device's static scratch
};

// Scratch of the allocation-free step (mk_decode_step_noalloc): the communication words,
// argmax keys, control block and token sink, held statically on every device the library
// runs on.  In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress (kept per device) and only that address is ever passed on.
#define MK_STATIC_SCRATCH_BYTES (16u << 20)
#define MK_MAX_DEVICES 64
static __device__ __align__(256) unsigned long long scratch[MK_STATIC_SCRATCH_BYTES / 8];

namespace {

thread_local char g_hip_msg[512] = "";

// One step-kernel instance per compiled shape, with its LDS ring size.
struct ShapeKernel {
  int D, HQ, HKV, HD, F;
  const void* kernel;
  const void* kernel_traced;   // the same step with the per-instruction trace
  int nslot;       // pages in the LDS ring
  int lds_bytes;   // LDS of one work-group
};
#define MK_KERNEL_ENTRY(D, HQ, HKV, HD, F, NCH)                                                    \
  {D, HQ, HKV, HD, F, (const void*)mk_step_kernel<mkdev::Shape<D, HQ, HKV, HD, F, NCH>>,          \
   (const void*)mk_step_kernel<mkdev::Traced<mkdev::Shape<D, HQ, HKV, HD, F, NCH>>>,              \
   mkdev::Ring<mkdev::Shape<D, HQ, HKV, HD, F, NCH>>::NSLOT,                                     \
   (int)sizeof(mkdev::MkShared<mkdev::Shape<D, HQ, HKV, HD, F, NCH>>) +                          \
       mkdev::Ring<mkdev::Shape<D, HQ, HKV, HD, F, NCH>>::NSLOT * MK_PAGE_BYTES},
const ShapeKernel kShapeKernels[] = {MK_SHAPES(MK_KERNEL_ENTRY)};
#undef MK_KERNEL_ENTRY
// The ring sizes the shapes were tuned with (the LDS trace and the rest of the shared
// state leave this much of the 160 KiB).
static_assert(mkdev::Ring<mkdev::Shape<2048, 32, 8, 64, 8192, 4>>::NSLOT == 8, "Llama-3.2-1B ring");
static_assert(mkdev::Ring<mkdev::Shape<4096, 32, 8, 128, 14336, 4>>::NSLOT == 6, "Llama-3.1-8B ring");
// a traced step runs with the same ring as an untraced one
static_assert(mkdev::Ring<mkdev::Traced<mkdev::Shape<2048, 32, 8, 64, 8192, 4>>>::NSLOT == 8, "traced 1B ring");
static_assert(mkdev::Ring<mkdev::Traced<mkdev::Shape<4096, 32, 8, 128, 14336, 4>>>::NSLOT == 6, "traced 8B ring");

const ShapeKernel* shape_kernel(const mk_config& c) {
  for (const ShapeKernel& k : kShapeKernels)
    if (k.D == c.hidden && k.HQ == c.n_q_heads && k.HKV == c.n_kv_heads && k.HD == c.head_dim && k.F == c.ffn)
      return &k;
  return nullptr;
}

// Every ABI call starts with a clean message, so that mk_strerror never reports a detail
// left behind by an earlier, unrelated failure.
void abi_enter() { g_hip_msg[0] = 0; }

int einval(const char* why) {
  snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", why);
  return MK_EINVAL;
}

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_hip_msg, sizeof(g_hip_msg), "%s: %s", what, hipGetErrorString(e));
  return MK_EHIP;
}

#define HIPCHK(call)                                  \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

// ---- uncached arenas for the communication words ------------------------------------
// Every word the step exchanges between CUs is stored and polled with device-scope
// accesses, which on this part go past the XCD's L2 anyway; in uncached device memory the
// step measured 578 against 586 us per step with the same words cached (Llama-3.2-1B
// shape, one GPU call).  Memory of that kind is never freed once a kernel has read it (on
// these GPUs a later allocation can then alias it wrongly): contexts take arenas from a
// per-process pool and give them back on destroy or reload.
struct UcArena {
  void* p;
  size_t bytes;
  int device;
  bool in_use;
  bool uncached;
};
std::mutex g_uc_mu;
std::vector<UcArena> g_uc_pool;

void* uc_acquire(int device, size_t bytes, bool uncached) {
  std::lock_guard<std::mutex> lock(g_uc_mu);
  for (UcArena& a : g_uc_pool)
    if (!a.in_use && a.device == device && a.bytes >= bytes && a.uncached == uncached) {
      a.in_use = true;
      return a.p;
    }
  void* p = nullptr;
  const hipError_t e = uncached ? hipExtMallocWithFlags(&p, bytes, hipDeviceMallocUncached) : hipMalloc(&p, bytes);
  if (e != hipSuccess) return nullptr;
  g_uc_pool.push_back(UcArena{p, bytes, device, true, uncached});
  return p;
}

void uc_release(void* p) {
  std::lock_guard<std::mutex> lock(g_uc_mu);
  for (UcArena& a : g_uc_pool)
    if (a.p == p) a.in_use = false;
}

void free_device(mk_ctx* c) {
  if (c->plan_only) return;
  if (c->d_ll) uc_release(c->d_ll);
  void* ptrs[] = {c->d_layers, c->d_off, c->d_plan, c->d_rope, c->d_amax, c->d_ctrl, c->d_next};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  c->d_layers = nullptr;
  c->d_off = nullptr;
  c->d_plan = nullptr;
  c->d_rope = nullptr;
  c->d_ll = nullptr;
  c->d_amax = nullptr;
  c->d_ctrl = nullptr;
  c->d_next = nullptr;
  c->loaded = false;
}

// ---- the static scratch, per device ------------------------------------------------
// Layout in 64-bit words: control block at 0, argmax keys at 8, the token sink after
// them, then the communication words (at a 256-byte boundary) with the context's layout.
std::mutex g_static_mu;
unsigned long long* g_static_ptr[MK_MAX_DEVICES];     // device address of `scratch`
std::atomic<bool> g_static_rearm[MK_MAX_DEVICES];      // re-arm the control block first
constexpr size_t ST_CTRL = 0, ST_AMAX = 8;
size_t st_next(int n_cus) { return ST_AMAX + (((size_t)n_cus + 7) & ~(size_t)7); }
size_t st_ll(int n_cus) { return (st_next(n_cus) + 8 + 31) & ~(size_t)31; }

// After an abandoned step: advance the epoch (no word that step or any earlier one wrote
// carries the new one, whichever context wrote it) and clear the ticket and error.
__global__ void static_rearm_kernel(MkCtrl* ctrl) {
  ctrl->epoch = ctrl->epoch + 1u;
  ctrl->ticket = 0u;
  ctrl->error = 0;
  ctrl->bad_token = 0;
}

// Once per device, with that device current (from mk_create): look up the array's device
// address and clear it, epoch 1.
int static_scratch_setup(int device) {
  if (device < 0 || device >= MK_MAX_DEVICES) return MK_OK;   // such devices use no static scratch
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_ptr[device]) return MK_OK;
  void* p = nullptr;
  HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
  HIPCHK(hipMemset(p, 0, MK_STATIC_SCRATCH_BYTES));
  MkCtrl ctrl{};
  ctrl.epoch = 1;
  HIPCHK(hipMemcpy(p, &ctrl, sizeof(ctrl), hipMemcpyHostToDevice));
  g_static_ptr[device] = (unsigned long long*)p;
  g_static_rearm[device] = false;
  return MK_OK;
}

int reset_device_state(mk_ctx* c, hipStream_t s) {
  HIPCHK(hipMemsetAsync(c->d_ll, 0, c->ll_words * sizeof(unsigned long long), s));
  MkCtrl ctrl{};
  ctrl.epoch = 1;
  HIPCHK(hipMemcpyAsync(c->d_ctrl, &ctrl, sizeof(ctrl), hipMemcpyHostToDevice, s));
  HIPCHK(hipStreamSynchronize(s));
  c->needs_reset = false;
  return MK_OK;
}

int launch(mk_ctx* c, int32_t token, const int32_t* token_dev, int32_t pos, void* kv, float* logits,
           int32_t* next_token, hipStream_t s, bool use_static = false) {
  abi_enter();
  if (!c) return MK_EINVAL;
  if (!c->loaded || c->plan_only) return MK_ESTATE;
  if (!kv || !logits) return einval("kv_cache and logits_out must not be null");
  // Cache rows are streamed with 16-byte loads; logits, tokens are 4-byte words.
  if ((uintptr_t)kv & 15) return einval("kv_cache must be 16-byte aligned");
  if ((uintptr_t)logits & 3) return einval("logits_out must be 4-byte aligned");
  if (((uintptr_t)next_token & 3) || ((uintptr_t)token_dev & 3)) return einval("token buffers must be 4-byte aligned");
  if (pos < 0 || pos >= c->cfg.max_ctx) return MK_ERANGE;
  if (!token_dev && (token < 0 || token >= c->cfg.vocab)) return MK_ERANGE;
  unsigned long long* st = nullptr;
  if (use_static) {
    st = c->device < MK_MAX_DEVICES ? g_static_ptr[c->device] : nullptr;
    if (!st) return MK_ESTATE;
    const size_t need = (st_ll(c->plan.n_cus) + c->ll_words) * sizeof(unsigned long long);
    if (need > MK_STATIC_SCRATCH_BYTES) {
      snprintf(g_hip_msg, sizeof(g_hip_msg),
               "the allocation-free step needs %zu bytes of scratch for this shape; the static scratch "
               "holds %u bytes",
               need, (unsigned)MK_STATIC_SCRATCH_BYTES);
      return MK_EINVAL;
    }
  }
  HIPCHK(hipSetDevice(c->device));
  if (use_static) {
    if (g_static_rearm[c->device].exchange(false)) {
      hipLaunchKernelGGL(static_rearm_kernel, dim3(1), dim3(1), 0, s, (MkCtrl*)(st + ST_CTRL));
      HIPCHK(hipGetLastError());
    }
    c->used_static = true;
  } else if (c->needs_reset) {
    int rc = reset_device_state(c, s);
    if (rc) return rc;
  }
  const mk_config& g = c->cfg;
  MkParams p{};
  p.n_layers = g.n_layers;
  p.V = g.vocab;
  p.max_ctx = g.max_ctx;
  p.n_cus = c->plan.n_cus;
  p.nslot = c->plan.slots;
  p.s_max = c->plan.s_max;
  p.min_chunk = c->plan.min_chunk;
  p.demand_depth = c->demand_depth;
  p.eps = g.rms_eps;
  p.attn_scale = (float)(1.0 / std::sqrt((double)g.head_dim));
  p.embed = c->embed;
  p.lm_head = c->lm_head;
  p.layers = c->d_layers;
  p.rope = c->d_rope;
  p.plan_off = c->d_off;
  p.plan = c->d_plan;
  p.ll_x = c->d_ll + c->off_x;
  p.ll_qkv = c->d_ll + c->off_qkv;
  p.ll_part = c->d_ll + c->off_part;
  p.ll_o = c->d_ll + c->off_o;
  p.ll_a = c->d_ll + c->off_a;
  p.amax = c->d_amax;
  p.ctrl = c->d_ctrl;
  p.next_token = next_token ? next_token : c->d_next;
  if (use_static) {   // the same words, in the device's static scratch
    unsigned long long* ll = st + st_ll(c->plan.n_cus);
    p.ll_x = ll + c->off_x;
    p.ll_qkv = ll + c->off_qkv;
    p.ll_part = ll + c->off_part;
    p.ll_o = ll + c->off_o;
    p.ll_a = ll + c->off_a;
    p.amax = st + ST_AMAX;
    p.ctrl = (MkCtrl*)(st + ST_CTRL);
    p.next_token = next_token ? next_token : (int32_t*)(st + st_next(c->plan.n_cus));
  }
  p.kv = (uint16_t*)kv;
  p.logits = logits;
  p.token_dev = token_dev;
  p.token = token;
  p.pos = pos;
  p.watchdog_ticks = c->watchdog_us * 100;   // s_memrealtime runs at 100 MHz
  p.trace = c->trace;
  p.trace_len = c->trace_len;
  void* args[] = {&p};
  // One work-group per CU, all resident at once: mk_create checked that a CU holds one
  // (the work-group takes most of the LDS, so it never holds two).  A plain launch of
  // exactly that many work-groups puts one on every CU; should another kernel hold some
  // CUs, the remaining work-groups start as those CUs free up.  (A cooperative launch
  // gives the same guarantee formally, but cost ~14 us more per step, measured.)
  HIPCHK(hipLaunchKernel(c->trace ? c->kernel_traced : c->kernel, dim3(c->plan.n_cus), dim3(MK_THREADS), args, 0, s));
  return MK_OK;
}

}  // namespace

extern "C" {

int mk_create(const mk_config* cfg, int hip_device, mk_ctx** out) {
  abi_enter();
  if (!cfg || !out) return MK_EINVAL;
  *out = nullptr;
  std::string why;
  if (mk_check_config(*cfg, &why)) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", why.c_str());
    return MK_EINVAL;
  }
  int n = 0;
  HIPCHK(hipGetDeviceCount(&n));
  if (hip_device < 0 || hip_device >= n) return MK_EINVAL;
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, hip_device));
  const void* kernel = shape_kernel(*cfg)->kernel;
  const void* kernel_traced = shape_kernel(*cfg)->kernel_traced;
  int per_cu = 0, per_cu_traced = 0, prev = 0;
  HIPCHK(hipGetDevice(&prev));
  HIPCHK(hipSetDevice(hip_device));
  hipError_t occ = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, MK_THREADS, 0);
  if (occ == hipSuccess)
    occ = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_traced, kernel_traced, MK_THREADS, 0);
  per_cu = std::min(per_cu, per_cu_traced);
  HIPCHK(hipSetDevice(prev));
  HIPCHK(occ);
  if (per_cu < 1) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "the decode kernel does not fit on a CU of device %d", hip_device);
    return MK_EHIP;
  }
  {   // the allocation-free step's scratch on this device, set up once
    HIPCHK(hipSetDevice(hip_device));
    const int rc = static_scratch_setup(hip_device);
    HIPCHK(hipSetDevice(prev));
    if (rc) return rc;
  }
  mk_ctx* c = new mk_ctx();
  c->cfg = *cfg;
  c->device = hip_device;
  c->n_cus = prop.multiProcessorCount;
  c->kernel = kernel;
  c->kernel_traced = kernel_traced;
  // Tuning overrides, for measurement: loader pages in flight per loader for staged
  // instructions (MK_DEMAND_DEPTH, 1-4) and cached instead of uncached communication words
  // (MK_LL_UNCACHED=0).
  if (const char* e = getenv("MK_LL_UNCACHED")) c->ll_uncached = atoi(e) != 0;
  if (const char* e = getenv("MK_DEMAND_DEPTH")) c->demand_depth = std::max(1, std::min(4, atoi(e)));
  *out = c;
  return MK_OK;
}

int mk_plan_only(const mk_config* cfg, int n_cus, mk_ctx** out) {
  abi_enter();
  if (!cfg || !out) return MK_EINVAL;
  *out = nullptr;
  mk_ctx* c = new mk_ctx();
  c->cfg = *cfg;
  c->plan_only = true;
  c->n_cus = n_cus;
  std::string why;
  int rc = mk_build_plan(*cfg, n_cus, &c->plan, &why);
  if (rc) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", why.c_str());
    delete c;
    return rc;
  }
  c->plan.slots = shape_kernel(*cfg)->nslot;
  *out = c;
  return MK_OK;
}

int mk_load_weights(mk_ctx* c, const mk_weights* w) {
  abi_enter();
  if (!c || !w) return MK_EINVAL;
  if (c->plan_only) return MK_ESTATE;
  const mk_config& g = c->cfg;
  if (!w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down)
    return MK_EINVAL;
  // n_layers + 1 entries: the extra one carries the final norm gain for the LM head.
  std::vector<MkLayerPtrs> layers(g.n_layers + 1);
  for (int l = 0; l < g.n_layers; ++l) {
    MkLayerPtrs& L = layers[l];
    L.attn_norm = (const uint16_t*)w->attn_norm[l];
    L.wq = (const uint16_t*)w->wq[l];
    L.wk = (const uint16_t*)w->wk[l];
    L.wv = (const uint16_t*)w->wv[l];
    L.wo = (const uint16_t*)w->wo[l];
    L.mlp_norm = (const uint16_t*)w->mlp_norm[l];
    L.wg = (const uint16_t*)w->w_gate[l];
    L.wu = (const uint16_t*)w->w_up[l];
    L.wd = (const uint16_t*)w->w_down[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.mlp_norm || !L.wg || !L.wu || !L.wd)
      return MK_EINVAL;
    // 16-byte alignment: rows are streamed with 16-byte loads
    const void* ps[] = {L.wq, L.wk, L.wv, L.wo, L.wg, L.wu, L.wd};
    for (const void* q : ps)
      if ((uintptr_t)q & 15) return MK_EINVAL;
    if (((uintptr_t)L.attn_norm & 3) || ((uintptr_t)L.mlp_norm & 3)) return MK_EINVAL;
  }
  if (((uintptr_t)w->lm_head & 15) || ((uintptr_t)w->final_norm & 3)) return MK_EINVAL;
  layers[g.n_layers] = MkLayerPtrs{};
  layers[g.n_layers].attn_norm = (const uint16_t*)w->final_norm;
  std::string why;
  MkPlan plan;
  int rc = mk_build_plan(g, c->n_cus, &plan, &why);
  if (rc) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", why.c_str());
    return rc;
  }
  plan.slots = shape_kernel(g)->nslot;
  HIPCHK(hipSetDevice(c->device));
  free_device(c);
  c->plan = std::move(plan);
  c->embed = (const uint16_t*)w->embed;
  c->lm_head = (const uint16_t*)w->lm_head;
  c->final_norm = (const uint16_t*)w->final_norm;

  // RoPE table [max_ctx][hd/2][cos, sin], angles in double, rounded to fp32.
  const int half = g.head_dim / 2;
  std::vector<float> rope((size_t)g.max_ctx * half * 2);
  for (int pos = 0; pos < g.max_ctx; ++pos)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)g.rope_theta, -2.0 * i / g.head_dim);
      const double ang = (double)pos * inv;
      rope[((size_t)pos * half + i) * 2] = (float)std::cos(ang);
      rope[((size_t)pos * half + i) * 2 + 1] = (float)std::sin(ang);
    }

  const int hpg = g.n_q_heads / g.n_kv_heads;
  const size_t nq = (size_t)g.n_q_heads * g.head_dim, nqkv = nq + 2 * (size_t)g.n_kv_heads * g.head_dim;
  c->off_x = 0;
  c->off_qkv = c->off_x + (size_t)(2 * g.n_layers + 1) * g.hidden;
  c->off_part = c->off_qkv + (size_t)g.n_layers * nqkv;
  c->off_o = c->off_part + (size_t)g.n_layers * g.n_kv_heads * hpg * c->plan.s_max * (g.head_dim + 2);
  c->off_a = c->off_o + (size_t)g.n_layers * nq;
  c->ll_words = c->off_a + (size_t)g.n_layers * g.ffn;

  auto alloc = [&](void** p, size_t bytes) -> int {
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
      hip_fail(e, "hipMalloc");
      return MK_ENOMEM;
    }
    return MK_OK;
  };
  if ((rc = alloc((void**)&c->d_layers, layers.size() * sizeof(MkLayerPtrs))) ||
      (rc = alloc((void**)&c->d_off, c->plan.off.size() * sizeof(int32_t))) ||
      (rc = alloc((void**)&c->d_plan, c->plan.rec.size() * sizeof(MkInstr))) ||
      (rc = alloc((void**)&c->d_rope, rope.size() * sizeof(float))) ||
      !(c->d_ll = (unsigned long long*)uc_acquire(c->device, c->ll_words * sizeof(unsigned long long),
                                                  c->ll_uncached)) ||
      (rc = alloc((void**)&c->d_amax, c->plan.n_cus * sizeof(unsigned long long))) ||
      (rc = alloc((void**)&c->d_ctrl, sizeof(MkCtrl))) || (rc = alloc((void**)&c->d_next, 64))) {
    if (!rc) {
      snprintf(g_hip_msg, sizeof(g_hip_msg), "uncached allocation of the communication words failed");
      rc = MK_ENOMEM;
    }
    free_device(c);
    return rc;
  }
  HIPCHK(hipMemcpy(c->d_layers, layers.data(), layers.size() * sizeof(MkLayerPtrs), hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(c->d_off, c->plan.off.data(), c->plan.off.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(c->d_plan, c->plan.rec.data(), c->plan.rec.size() * sizeof(MkInstr), hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(c->d_rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice));
  HIPCHK(hipMemset(c->d_amax, 0, c->plan.n_cus * sizeof(unsigned long long)));
  HIPCHK(hipMemset(c->d_next, 0, 64));
  c->loaded = true;
  rc = reset_device_state(c, nullptr);
  if (rc) return rc;
  return MK_OK;
}

int mk_decode_step(mk_ctx* c, int32_t token, int32_t pos, void* kv_cache, float* logits_out,
                   int32_t* next_token, void* stream) {
  return launch(c, token, nullptr, pos, kv_cache, logits_out, next_token, (hipStream_t)stream);
}

int mk_decode_step_dev(mk_ctx* c, const int32_t* token_dev, int32_t pos, void* kv_cache, float* logits_out,
                       int32_t* next_token, void* stream) {
  abi_enter();
  if (!token_dev) return einval("token_dev must not be null");
  return launch(c, 0, token_dev, pos, kv_cache, logits_out, next_token, (hipStream_t)stream);
}

int mk_sync(mk_ctx* c, void* stream) {
  abi_enter();
  if (!c) return MK_EINVAL;
  if (!c->loaded) return MK_ESTATE;
  HIPCHK(hipSetDevice(c->device));
  HIPCHK(hipStreamSynchronize((hipStream_t)stream));
  MkCtrl ctrl{};
  HIPCHK(hipMemcpy(&ctrl, c->d_ctrl, sizeof(ctrl), hipMemcpyDeviceToHost));
  int rc = MK_OK;
  if (ctrl.error != 0 || ctrl.bad_token) {
    c->needs_reset = true;
    rc = ctrl.error != 0 ? ctrl.error : MK_ERANGE;
  }
  if (c->used_static) {   // steps this context ran on the device's static scratch
    MkCtrl sc{};
    HIPCHK(hipMemcpy(&sc, g_static_ptr[c->device] + ST_CTRL, sizeof(sc), hipMemcpyDeviceToHost));
    if (sc.error != 0 || sc.bad_token) {
      g_static_rearm[c->device] = true;
      if (rc == MK_OK) rc = sc.error != 0 ? sc.error : MK_ERANGE;
    }
  }
  return rc;
}

int mk_decode_step_noalloc(mk_ctx* c, int32_t token, int32_t pos, void* kv_cache, float* logits_out,
                           int32_t* next_token, void* stream) {
  return launch(c, token, nullptr, pos, kv_cache, logits_out, next_token, (hipStream_t)stream, true);
}

int mk_set_watchdog_us(mk_ctx* c, int64_t us) {
  abi_enter();
  if (!c || us < 0) return MK_EINVAL;
  c->watchdog_us = us;
  return MK_OK;
}

int mk_plan_info(const mk_ctx* c, int32_t info[8]) {
  abi_enter();
  if (!c || !info) return MK_EINVAL;
  if (c->plan.off.empty()) return MK_ESTATE;
  info[0] = c->plan.n_cus;
  info[1] = MK_INSTR_WORDS;
  info[2] = (int32_t)c->plan.rec.size();
  info[3] = c->plan.page_bytes;
  info[4] = c->plan.slots;
  info[5] = MK_NC;
  info[6] = c->plan.s_max;
  info[7] = shape_kernel(c->cfg)->lds_bytes;
  return MK_OK;
}

int mk_plan_copy(const mk_ctx* c, int32_t* offsets, int32_t* records, int64_t cap_words) {
  abi_enter();
  if (!c || !offsets || !records) return MK_EINVAL;
  if (c->plan.off.empty()) return MK_ESTATE;
  if (cap_words < (int64_t)c->plan.rec.size() * MK_INSTR_WORDS) return MK_EINVAL;
  memcpy(offsets, c->plan.off.data(), c->plan.off.size() * sizeof(int32_t));
  memcpy(records, c->plan.rec.data(), c->plan.rec.size() * sizeof(MkInstr));
  return MK_OK;
}

int mk_debug_dump(const mk_ctx* c, uint64_t* host, int64_t cap, int64_t offsets[6]) {
  abi_enter();
  if (!c || !offsets) return MK_EINVAL;
  if (!c->loaded) return MK_ESTATE;
  offsets[0] = (int64_t)c->off_x;
  offsets[1] = (int64_t)c->off_qkv;
  offsets[2] = (int64_t)c->off_part;
  offsets[3] = (int64_t)c->off_o;
  offsets[4] = (int64_t)c->off_a;
  offsets[5] = (int64_t)c->ll_words;
  if (!host) return MK_OK;
  if (cap < (int64_t)c->ll_words) return MK_EINVAL;
  HIPCHK(hipSetDevice(c->device));
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(host, c->d_ll, c->ll_words * sizeof(uint64_t), hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_set_trace(mk_ctx* c, uint64_t* dev_buf, int64_t capacity_words, int64_t* required_words) {
  abi_enter();
  if (!c) return MK_EINVAL;
  if (c->plan.off.empty()) return MK_ESTATE;
  int len = 0;
  for (size_t i = 0; i + 1 < c->plan.off.size(); ++i) len = std::max(len, c->plan.off[i + 1] - c->plan.off[i]);
  len = std::min(len, MK_TRACE_MAX);   // the kernel keeps this many instructions' marks
  const int64_t need = (int64_t)c->plan.n_cus * len * MK_TRACE_SLOTS;
  if (required_words) *required_words = need;
  if (!dev_buf) {
    c->trace = nullptr;
    c->trace_len = 0;
    return MK_OK;
  }
  if (capacity_words < need || ((uintptr_t)dev_buf & 7)) return MK_EINVAL;
  c->trace = (unsigned long long*)dev_buf;
  c->trace_len = len;
  return MK_OK;
}

void mk_destroy(mk_ctx* c) {
  if (!c) return;
  if (!c->plan_only && c->device >= 0) {
    (void)hipSetDevice(c->device);
    free_device(c);
  }
  delete c;
}

const char* mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_EINVAL: return g_hip_msg[0] ? g_hip_msg : "invalid argument";
    case MK_ERANGE: return "position or token out of range";
    case MK_ESTATE: return "weights not loaded / wrong state";
    case MK_EHIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
    case MK_ETIMEOUT: return "device-side wait expired (step abandoned)";
    case MK_ENOMEM: return "device allocation failed";
    default: return "unknown error";
  }
}

const char* mk_version(void) { return "mk 0.1.0 (gfx950)"; }

}  // extern "C"

#include "mk_plan.cpp"
