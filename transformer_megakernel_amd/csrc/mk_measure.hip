// Measurement kernels of the library: the practical ceilings the decode step is compared
// against.  Nothing in the decode path calls them.
//
//  * mk_stream_read: a plain streaming read of a device buffer (16-byte non-temporal loads,
//    coalesced per wave, several loads in flight per lane): the HBM read rate a simple
//    kernel reaches on this part, the figure the step's algorithmic bandwidth stands
//    against (the pages' own bandwidth model divides a forward's bytes by the part's
//    bandwidth: Megakernel article, section "Why are traditional inference methods so
//    inefficient?", bandwidth paragraph).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace {

// Grid-stride read of n16 16-byte words, U loads in flight per lane.  The loaded bits are
// folded into one word per thread, which is stored only if it matches a value no input
// here produces, so the loads cannot be dropped and almost nothing is written.
template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load((const u32x4*)(src + i + j * stride));
#pragma unroll
    for (int j = 0; j < U; ++j) acc += v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(src + i));
    acc += v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

int mk_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll, void* stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || ((uintptr_t)sink & 3) ||
      blocks < 1 || blocks > (1 << 20))
    return MK_EINVAL;
  const size_t n16 = (size_t)bytes / 16;
  hipStream_t s = (hipStream_t)stream;
  const uint4* src = (const uint4*)buf;
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
