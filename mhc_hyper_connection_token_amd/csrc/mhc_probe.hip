// mhc_probe.hip -- pure-stream bandwidth probes, a measurement aid beside the
// site kernels: the HBM rate this part sustains for a plain read and a plain
// copy, against which the site kernels' rates are read.  (The hc_fused_gate.rs
// page's gate carries a bandwidth probe of its own, a pure streamer reporting
// read and read + write GB/s.)
//
// Both kernels move one 16-byte quad per thread with streaming (non-temporal)
// loads over a grid that covers the buffer, consecutive threads on consecutive
// quads: on this part that layout streams faster than grid-stride loops, whose
// quads in flight per thread lie far apart.  The read probe folds each block's
// quads into one float so that no load can be dropped.
#include "mhc_device.h"
#include "mhc_kernels.h"

namespace mhc {

__global__ __launch_bounds__(256) void probe_copy_kernel(const float* __restrict__ src,
                                                         float* __restrict__ dst, long nq) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < nq) nt_store4(dst + 4 * i, nt_load4(src + 4 * i));
}

__global__ __launch_bounds__(256) void probe_read_kernel(const float* __restrict__ src, long nq,
                                                         float* __restrict__ sink) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const float4 v = i < nq ? nt_load4(src + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
  float acc = sum_wave((v.x + v.y) + (v.z + v.w));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

long probe_blocks(long nq) { return (nq + 255) / 256; }

hipError_t launch_probe(const float* src, float* dst, long nq, bool copy, hipStream_t st) {
  const long blocks = probe_blocks(nq);
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (copy)
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, nq);
  else
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, nq, dst);
  return hipGetLastError();
}

}  // namespace mhc
