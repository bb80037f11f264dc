// Measurement kernels of the library: the practical ceilings the decode step is compared
// against.  Nothing in the decode path calls them.
//
//  * mk_stream_read: a plain streaming read of a device buffer (16-byte non-temporal loads,
//    coalesced per wave, several loads in flight per lane): the HBM read rate a simple
//    kernel reaches on this part, the figure the step's algorithmic bandwidth stands
//    against (the pages' own bandwidth model divides a forward's bytes by the part's
//    bandwidth: Megakernel article, section "Why are traditional inference methods so
//    inefficient?", bandwidth paragraph).
//  * mk_bench_gemv_page: the per-page cost of the decode step's matrix-vector work on
//    the compute units, one variant at a time: the article finds the best unit for its
//    matrix-vector products differs between GPU generations (section "Megakernel: a
//    fusion design from scratch", matrix-vector paragraph), so the choice for gfx950 is
//    measured, page by page, with the operands already in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"
#include "mk_kernel.h"

namespace {

// ---------------------------------------------------------------- GEMV page variants
// One page = 16 KiB of bf16 weights = 4 rows of 2048 (the Llama-3.2-1B hidden width),
// times an fp32 activation of 2048.  Each variant computes the 4 row sums; every wave of
// the work-group walks `pages` pages of its own 16 KiB LDS region.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int PB_ROWS = 4, PB_K = 2048, PB_WAVES = 4;

// Deterministic weights and activation (the page content does not matter for the timing;
// the variants are compared with each other on it).
__device__ __forceinline__ float pb_w(int row, int k) {
  uint32_t h = (uint32_t)(row * 2654435761u) ^ (uint32_t)(k * 2246822519u);
  h ^= h >> 15; h *= 2654435761u; h ^= h >> 13;
  return ((int)(h & 1023) - 512) * (0.05f / 512.f);
}
__device__ __forceinline__ float pb_x(int k) { return __sinf(0.37f * k) * 1.3f + 0.01f * (k & 7); }
__device__ __forceinline__ uint16_t pb_bf(float f) { return (uint16_t)(__float_as_uint(f) >> 16); }

__device__ __forceinline__ int pb_opaque(int v) { asm volatile("" : "+v"(v)); return v; }


// variant 0: fp32 FMA on the widened bf16 (the decode kernel's path): lane l holds 16
// bytes of each 1 KiB unit, the activation slice in registers; unit u = row u / 4,
// columns 512 * (u % 4) + 8 l ...
// variant 1: v_dot2 on bf16 pairs against the activation split in two bf16 terms
// (hi = x truncated, lo = x - hi truncated; ~2^-16 relative).
// variant 2: the 16x16x32 bf16 matrix instruction against the activation split in three
// bf16 terms (hi, mid, lo: fp32-exact up to the last bit): 16 instructions per page.
// Matrix row m = 4 j + b is weight row j over columns 512 b + 32 s + (0..31) in step s;
// matrix column n = 4 b' + t carries term t of the activation over the same columns of
// block b' (t = 3: zero), so row j's sum is the sum of D[4 j + b][4 b + t] over b, t.
// The page is laid out for it: unit s holds step s, lane l its row l % 16, 8 columns at
// 8 * (l / 16), so every step reads one contiguous 1 KiB.
// variant 3: the LDS reads of variant 0 alone.
template <int V>
__global__ void __launch_bounds__(256) gemv_page_kernel(int pages, unsigned long long* ticks, float* out) {
  __shared__ __align__(16) char lds[PB_WAVES * 16384];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  char* page = lds + wave * 16384;
  // fill this wave's page in the variant's layout
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int row, k;
      if (V == 2) {
        const int m = lane % 16, g = lane / 16;
        row = m / 4;
        k = 512 * (m % 4) + 32 * u + 8 * g + e;
      } else {
        row = u / 4;
        k = 512 * (u % 4) + 8 * lane + e;
      }
      v[e] = pb_bf(pb_w(row, k));
    }
    uint4 q;
    q.x = v[0] | ((uint32_t)v[1] << 16); q.y = v[2] | ((uint32_t)v[3] << 16);
    q.z = v[4] | ((uint32_t)v[5] << 16); q.w = v[6] | ((uint32_t)v[7] << 16);
    *(uint4*)(page + u * 1024 + lane * 16) = q;
  }
  __syncthreads();
  float acc_out = 0.f;
  // activation operands, kept in registers for all pages
  float av[4][8];
  uint32_t xhi[4][4], xlo[4][4];
  bf16x8_t xb[16];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) av[c][e] = pb_x(512 * c + 8 * lane + e);
  if (V == 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t a0 = __float_as_uint(av[c][e]), a1 = __float_as_uint(av[c][e + 1]);
        const float r0 = av[c][e] - __uint_as_float(a0 & 0xffff0000u);
        const float r1 = av[c][e + 1] - __uint_as_float(a1 & 0xffff0000u);
        xhi[c][e / 2] = (a0 >> 16) | (a1 & 0xffff0000u);
        xlo[c][e / 2] = (__float_as_uint(r0) >> 16) | (__float_as_uint(r1) & 0xffff0000u);
      }
  }
  if (V == 2) {
    const int n = lane % 16, g = lane / 16, bb = n / 4, t = n % 4;
#pragma unroll
    for (int st = 0; st < 16; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = pb_x(512 * bb + 32 * st + 8 * g + e);
        const float hi = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
        const float r1 = x - hi;
        const float mid = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
        const float lo = r1 - mid;
        const float term = t == 0 ? hi : t == 1 ? mid : t == 2 ? lo : 0.f;
        xb[st][e] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(term) >> 16));
      }
  }
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < pages; ++it) {
    const char* pg = page + pb_opaque(0);
    float y = 0.f;
    if constexpr (V == 0 || V == 1 || V == 3) {
      float r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 w = *(const uint4*)(pg + (4 * j + c) * 1024 + lane * 16);
          if constexpr (V == 0) {
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              a = fmaf(__uint_as_float(ws[q] << 16), av[c][2 * q], a);
              a = fmaf(__uint_as_float(ws[q] & 0xffff0000u), av[c][2 * q + 1], a);
            }
          } else if constexpr (V == 1) {
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ws[q]),
                                                  __builtin_bit_cast(bf16x2_t, xhi[c][q]), a, false);
              a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ws[q]),
                                                  __builtin_bit_cast(bf16x2_t, xlo[c][q]), a, false);
            }
          } else {
            a += __uint_as_float(w.x ^ w.y ^ w.z ^ w.w);
          }
        }
        r[j] = a;
      }
      // the decode kernel's per-page reduction: row j ends in the lanes of 16-lane group j
      y = mkdev::reduce_rows<4, 64>(r, lane);
    } else {
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const bf16x8_t a = *(const bf16x8_t*)(pg + st * 1024 + lane * 16);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[st], d, 0, 0, 0);
      }
      // lane l holds D[4 (l / 16) + i][l % 16]; keep i = b' = (l % 16) / 4, sum the row's 16 lanes
      const int sel = (lane % 16) / 4;
      const float v = sel == 0 ? d[0] : sel == 1 ? d[1] : sel == 2 ? d[2] : d[3];
      y = mkdev::sum16(v);
    }
    acc_out += y;
    if (it == 0 && (lane % 16) == 0) out[(blockIdx.x * PB_WAVES + wave) * 8 + 4 + lane / 16] = y;
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) ticks[blockIdx.x * PB_WAVES + wave] = t1 - t0;
  if (lane < 4) out[(blockIdx.x * PB_WAVES + wave) * 8 + lane] = acc_out;
}

// Grid-stride read of n16 16-byte words, U loads in flight per lane.  The loaded bits are
// folded into one word per thread, which is stored only if it matches a value no input
// here produces, so the loads cannot be dropped and almost nothing is written.
template <int U, bool NT = true>
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j)
      v[j] = NT ? __builtin_nontemporal_load((const u32x4*)(src + i + j * stride)) : *(const u32x4*)(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < U; ++j) acc += v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(src + i));
    acc += v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// ---------------------------------------------------------------- poll latency
// The round trip of one dependency poll while the CU streams weights: wave 0 times
// `probes` single-word loads (a vector agent-scope load, or a scalar load that bypasses
// the scalar cache), each of a word no other probe touches, ~1 us apart; waves 1-2 stream
// their CU's region of `stream` into a 128 KiB LDS ring with 1 KiB LDS-direct loads, the
// way the decode kernel's loaders do, keeping `depth` pages of 16 KiB in flight each.
__device__ __forceinline__ void pl_wait_vmcnt(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
  }
}

template <int SCALAR>
__global__ void __launch_bounds__(192) poll_latency_kernel(const char* stream, long long region_bytes,
                                                           const unsigned long long* words, int depth, int probes,
                                                           unsigned long long* out) {
  __shared__ __align__(16) char ring[8 * 16384];
  __shared__ int stop;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x == 0) stop = 0;
  __syncthreads();
  if (wave == 0) {
    unsigned long long fold = 0;
    for (int i = 0; i < probes; ++i) {
      for (int k = 0; k < 20; ++k) __builtin_amdgcn_s_sleep(127);   // ~1 us between probes
      const unsigned long long* w = words + ((size_t)blockIdx.x * probes + i) * 16;   // 128 B apart
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      unsigned long long v;
      if constexpr (SCALAR) {
        asm volatile("s_load_dwordx2 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(w) : "memory");
      } else {
        v = 0;
        if (lane == 0) v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = __shfl(v, 0);
      }
      asm volatile("" ::"v"(v) : "memory");   // the stamp below waits for the probe
      const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
      fold += v;
      if (lane == 0) out[(size_t)blockIdx.x * probes + i] = t1 - t0;
    }
    if (lane == 0) {
      if (fold == 0x5bd1e995ull) out[0] = 0;
      __hip_atomic_store(&stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // the span the loaders streamed over: from the first probe to now
    if (lane == 0) out[(size_t)gridDim.x * probes + blockIdx.x] = __builtin_amdgcn_s_memrealtime();
  } else if (depth > 0) {
    const int L = wave - 1;
    const char* base = stream + (size_t)blockIdx.x * region_bytes;
    const uint32_t ring_l = mkdev::lds_addr(ring) + L * 4 * 16384;
    int pend = 0;
    long long k = 0;
    const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();
    for (;; ++k) {
      if (__hip_atomic_load(&stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
      const char* pg = base + ((2 * k + L) * 16384) % region_bytes;
      const uint32_t slot = ring_l + (uint32_t)(k % 4) * 16384;
#pragma unroll
      for (int u = 0; u < 16; ++u) mkdev::dma16(pg + u * 1024 + lane * 16, slot + u * 1024);
      if (++pend >= depth) {
        pl_wait_vmcnt((depth - 1) * 16);
        --pend;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // pages streamed and the loader's start, for the achieved rate
    if (lane == 0) {
      out[(size_t)gridDim.x * (probes + 1) + blockIdx.x * 2 + L] = (unsigned long long)k;
      if (L == 0) out[(size_t)gridDim.x * (probes + 3) + blockIdx.x] = t_start;
    }
  }
}

// Broadcast read of a 16 KiB vector of 64-bit words by every CU at once (agent-scope loads,
// as the decode kernel's activation polls), against each CU reading its own 16 KiB.
template <int SHARED>
__global__ void __launch_bounds__(64) bcast_read_kernel(const unsigned long long* buf, int reps,
                                                        unsigned long long* out) {
  const int lane = threadIdx.x;
  const unsigned long long* src = SHARED ? buf : buf + (size_t)blockIdx.x * 2048;
  unsigned long long fold = 0;
  for (int r = 0; r < reps; ++r) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long w[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) w[k] = __hip_atomic_load(src + k * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < 32; ++k) fold += w[k];
    fold = __shfl(fold, 0);   // every load has returned
    asm volatile("" ::"v"(fold) : "memory");
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) out[(size_t)blockIdx.x * reps + r] = t1 - t0;
    for (int k = 0; k < 10; ++k) __builtin_amdgcn_s_sleep(127);
  }
  if (fold == 0x5bd1e995ull && lane == 0) out[0] = 0;
}

}  // namespace

extern "C" {

int mk_bench_poll_latency(const void* stream_buf, int64_t region_bytes, const uint64_t* probe_words, int32_t depth,
                          int32_t scalar, int32_t probes, int32_t blocks, unsigned long long* out, void* stream) {
  if (!stream_buf || !probe_words || !out || region_bytes < (1 << 20) || (region_bytes & 16383) || depth < 0 ||
      depth > 4 || probes < 1 || blocks < 1 || blocks > 4096)
    return MK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (scalar)
    hipLaunchKernelGGL(poll_latency_kernel<1>, dim3(blocks), dim3(192), 0, s, (const char*)stream_buf,
                       (long long)region_bytes, (const unsigned long long*)probe_words, depth, probes, out);
  else
    hipLaunchKernelGGL(poll_latency_kernel<0>, dim3(blocks), dim3(192), 0, s, (const char*)stream_buf,
                       (long long)region_bytes, (const unsigned long long*)probe_words, depth, probes, out);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

int mk_bench_bcast_read(const uint64_t* buf, int32_t shared, int32_t reps, int32_t blocks, unsigned long long* out,
                        void* stream) {
  if (!buf || !out || reps < 1 || blocks < 1 || blocks > 4096) return MK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (shared)
    hipLaunchKernelGGL(bcast_read_kernel<1>, dim3(blocks), dim3(64), 0, s, (const unsigned long long*)buf, reps, out);
  else
    hipLaunchKernelGGL(bcast_read_kernel<0>, dim3(blocks), dim3(64), 0, s, (const unsigned long long*)buf, reps, out);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

int mk_bench_gemv_page(int32_t variant, int32_t pages, int32_t blocks, unsigned long long* ticks, float* out,
                       void* stream) {
  if (!ticks || !out || pages < 1 || blocks < 1 || blocks > 4096) return MK_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  switch (variant) {
    case 0: hipLaunchKernelGGL(gemv_page_kernel<0>, dim3(blocks), dim3(256), 0, s, pages, ticks, out); break;
    case 1: hipLaunchKernelGGL(gemv_page_kernel<1>, dim3(blocks), dim3(256), 0, s, pages, ticks, out); break;
    case 2: hipLaunchKernelGGL(gemv_page_kernel<2>, dim3(blocks), dim3(256), 0, s, pages, ticks, out); break;
    case 3: hipLaunchKernelGGL(gemv_page_kernel<3>, dim3(blocks), dim3(256), 0, s, pages, ticks, out); break;
    default: return MK_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

int mk_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll, void* stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || ((uintptr_t)sink & 3) ||
      blocks < 1 || blocks > (1 << 20))
    return MK_EINVAL;
  const size_t n16 = (size_t)bytes / 16;
  hipStream_t s = (hipStream_t)stream;
  const uint4* src = (const uint4*)buf;
  if (unroll == -8) {   // plain (temporal) loads, 8 in flight
    hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(blocks), dim3(256), 0, s, src, n16, sink);
    return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
  }
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, s, src, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, src, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, src, n16, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(256), 0, s, src, n16, sink); break;
    default: return MK_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? MK_OK : MK_EHIP;
}

}  // extern "C"
