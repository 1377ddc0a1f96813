// mhc_trunk.hip -- the trunk's entry and exit around the sites (hyper.rs page:
// doc comments of `expand`, `contract_mean` and `collapse`; the HyperHead
// loader sizes the head's weight [S][S*H], bias [S] and single scale).
//
//   expand: x[t,k,:] = e[t,:] for every stream k
//   mean:   y[t,:]   = (sum_k x[t,k,:]) / S, streams in ascending order
//   head:   the pre half of a site with the head's own S rows, one scale and S
//           biases: rinv = 1/sqrt(mean x[t]^2 + eps) over the slab,
//           g_c = sigmoid(scale * rinv * (fn_h[c] . x[t]) + base_c),
//           y[t,:] = sum_c g_c x[t,c,:]
//
// expand and mean are pure streams (one hidden quad per thread, 16-byte
// non-temporal loads and stores).  The head reuses the small-batch split-K
// partials (with R = S rows) and this file's finish kernel, which adds the
// partials in the fixed order of the site's finish kernel and collapses.
#include "mhc_device.h"
#include "mhc_kernels.h"
#include "mhc_split.h"

namespace mhc {

__global__ __launch_bounds__(256) void expand_kernel(const float* __restrict__ e, int S, int HQ,
                                                     long total, float* __restrict__ x) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long t = i / HQ, q = i - t * HQ;
  const float4 v = nt_load4(e + 4 * i);
  float* xt = x + (t * S * HQ + q) * 4;
  for (int k = 0; k < S; ++k) nt_store4(xt + (long)k * HQ * 4, v);
}

__global__ __launch_bounds__(256) void mean_kernel(const float* __restrict__ x, int S, int HQ,
                                                   long total, float* __restrict__ y) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long t = i / HQ, q = i - t * HQ;
  const float* xt = x + (t * S * HQ + q) * 4;
  float4 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < S) v[k] = nt_load4(xt + (long)k * HQ * 4);
  float4 s = v[0];
#pragma unroll
  for (int k = 1; k < 8; ++k)
    if (k < S) {
      s.x += v[k].x;
      s.y += v[k].y;
      s.z += v[k].z;
      s.w += v[k].w;
    }
  const float d = (float)S;
  nt_store4(y + 4 * i, make_float4(s.x / d, s.y / d, s.z / d, s.w / d));
}

// Per token: add the G partials (R = S rows and the sum of squares) in the
// fixed order, gate, collapse.  Grid (T, HB) as the site's finish kernel: every
// block of a token recomputes the gates, block 0 writes them.
__global__ __launch_bounds__(256) void head_finish_kernel(
    const float* __restrict__ x, const float* __restrict__ part, int G, int T, int S, int H,
    const float* __restrict__ scale_h, const float* __restrict__ base_h, float eps,
    float* __restrict__ gates, float* __restrict__ y, int quads_per_block) {
  const int RP = S + 1;
  const int t = blockIdx.x;
  const int hb = blockIdx.y;
  const int HQ = H >> 2;
  __shared__ float red[256];
  __shared__ float m_raw[16];
  // the pre gate's parameter layout: scale at 0, the biases from 3 on
  __shared__ float params[3 + 8];
  if (threadIdx.x == 0)
    params[0] = scale_h[0];
  else if (threadIdx.x >= 3 && threadIdx.x < 3 + S)
    params[threadIdx.x] = base_h[threadIdx.x - 3];

  const int q0 = hb * quads_per_block;
  const int q1 = min(HQ, q0 + quads_per_block);
  const float4* xt = reinterpret_cast<const float4*>(x + (size_t)t * S * H);
  float4 xq[8];
  const int qa = q0 + threadIdx.x;
  if (qa < q1) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < S) xq[c] = xt[(size_t)c * HQ + qa];
  }

  reduce_token_partials<16>(part, G, T, t, RP, red, m_raw);  // ends with a barrier

  float pc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) pc[c] = c < S ? pre_gate(m_raw, c, S, S * H, eps, params) : 0.f;
  if (hb == 0 && threadIdx.x < S) gates[(size_t)t * S + threadIdx.x] = pc[threadIdx.x];

  float4* yt = reinterpret_cast<float4*>(y + (size_t)t * H);
  if (qa < q1) yt[qa] = collapse4<8>(pc, xq, S);
  for (int q = qa + 256; q < q1; q += 256) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < S) xq[c] = xt[(size_t)c * HQ + q];
    yt[q] = collapse4<8>(pc, xq, S);
  }
}

hipError_t launch_expand(const float* e, int T, int S, int H, float* x, hipStream_t st) {
  const long total = (long)T * (H / 4);
  const long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)blocks), dim3(256), 0, st, e, S, H / 4, total,
                     x);
  return hipGetLastError();
}

hipError_t launch_mean(const float* x, int T, int S, int H, float* y, hipStream_t st) {
  if (S > 8) return hipErrorInvalidValue;
  const long total = (long)T * (H / 4);
  const long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mean_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, S, H / 4, total, y);
  return hipGetLastError();
}

hipError_t launch_head_finish(const float* x, const float* part, int G, int T, int S, int H,
                              const float* scale_h, const float* base_h, float eps, float* gates,
                              float* y, hipStream_t st) {
  if (S > 8) return hipErrorInvalidValue;
  const int HQ = H / 4;
  int HB = 1;
  if (T < 512) {
    HB = (1024 + T - 1) / T;
    HB = min(HB, (HQ + 63) / 64);
    HB = max(HB, 1);
  }
  const int qpb = (HQ + HB - 1) / HB;
  hipLaunchKernelGGL(head_finish_kernel, dim3(T, HB), dim3(256), 0, st, x, part, G, T, S, H,
                     scale_h, base_h, eps, gates, y, qpb);
  return hipGetLastError();
}

}  // namespace mhc
