// mhc_post.hip -- the post mix of one site (hyper.rs page, doc comment of `post`):
//   x_out[t,k,i] = post[t,k] * f[t,i] + sum_j comb[t,j,k] * x[t,j,i]
//
// A pure stream: every thread owns one hidden quad (16 bytes) of one token,
// reads the S source quads and the branch quad once (non-temporal: they are
// not read again by this kernel), and writes the S target quads once.  The
// token's gates are block-uniform (one token per block row), so they come
// through scalar loads.  HBM-bound: the bytes per token are
// 4*(2*S*H + H) plus the gates.
#include "mhc_device.h"
#include "mhc_kernels.h"

namespace mhc {

template <int S>
__global__ __launch_bounds__(256) void post_kernel(const float* __restrict__ x,
                                                   const float* __restrict__ f,
                                                   const float* __restrict__ post,
                                                   const float* __restrict__ comb, int H,
                                                   int QB, float* __restrict__ out) {
  const int t = blockIdx.x / QB;
  const int HQ = H >> 2;
  const int q = (blockIdx.x - t * QB) * 256 + threadIdx.x;
  if (q >= HQ) return;
  float pk[S], ck[S][S];
#pragma unroll
  for (int k = 0; k < S; ++k) pk[k] = post[(size_t)t * S + k];
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int k = 0; k < S; ++k) ck[j][k] = comb[(size_t)t * S * S + j * S + k];

  const float4* xt = reinterpret_cast<const float4*>(x) + (size_t)t * S * HQ + q;
  float4 xv[S];
#pragma unroll
  for (int j = 0; j < S; ++j) xv[j] = nt_load4(reinterpret_cast<const float*>(xt + (size_t)j * HQ));
  const float4 fv = nt_load4(f + ((size_t)t * HQ + q) * 4);
  float4* ot = reinterpret_cast<float4*>(out) + (size_t)t * S * HQ + q;
#pragma unroll
  for (int k = 0; k < S; ++k) ot[(size_t)k * HQ] = post_mix4<S>(pk[k], &ck[0][k], S, xv, fv, S);
}

hipError_t launch_post(const float* x, const float* f, const float* post, const float* comb,
                       int T, int S, int H, float* x_out, hipStream_t st) {
  const int HQ = H / 4;
  const int QB = (HQ + 255) / 256;
  dim3 grid((unsigned)T * QB);
  switch (S) {
#define MHC_S(SS)                                                                         \
  case SS:                                                                                \
    hipLaunchKernelGGL((post_kernel<SS>), grid, dim3(256), 0, st, x, f, post, comb, H, QB, \
                       x_out);                                                             \
    break;
    MHC_S(1) MHC_S(2) MHC_S(3) MHC_S(4) MHC_S(5) MHC_S(6) MHC_S(7) MHC_S(8)
#undef MHC_S
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mhc
