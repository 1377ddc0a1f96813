// mhc_finish.hip -- per-token finish of the pre chain from split-K partials.
//
// Steps (hyper.rs page, module doc: arithmetic contract, lines two to four):
// add the G partial mixes / sums of squares of a token in fixed order, apply
// the RMS rescale, the three gate groups and the Sinkhorn (one wavefront, no
// block barrier inside the iteration loop), then collapse the streams:
// y[t,i] = sum_c pre[t,c] * x[t,c,i].
//
// Grid: (T, HB).  Block y-index hb covers a contiguous range of hidden quads
// for the collapse; every block of a token recomputes the (cheap) gates so that
// no cross-block wait is needed, and only hb == 0 writes pre/post/comb.
#include "mhc_device.h"
#include "mhc_kernels.h"

namespace mhc {

template <int P>
__global__ __launch_bounds__(256) void finish_kernel(
    const float* __restrict__ x, const float* __restrict__ part, int G, int T, int S, int H,
    const float* __restrict__ scale, const float* __restrict__ base, int iters, float eps,
    float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb,
    float* __restrict__ y, int quads_per_block) {
  const int R = (2 + S) * S;
  const int RP = R + 1;
  const int t = blockIdx.x;
  const int hb = blockIdx.y;
  __shared__ float red[256];
  __shared__ float m_raw[96];  // R + 1 <= 81
  __shared__ float pre_lds[8];

  // 1. fixed-order reduction of the G partials: thread (r, q) with q < Q adds
  //    g = q, q + Q, ... ; then thread r adds the Q results in order.
  const int Q = 256 / RP;
  {
    const int r = threadIdx.x % RP, q = threadIdx.x / RP;
    float s = 0.f;
    if (q < Q) {
      const float* p = part + (size_t)t * RP + r;
      for (int g = q; g < G; g += Q) s += p[(size_t)g * T * RP];
    }
    red[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x < RP) {
    float s = 0.f;
    for (int q = 0; q < Q; ++q) s += red[q * RP + threadIdx.x];
    m_raw[threadIdx.x] = s;
  }
  __syncthreads();

  // 2. gates + Sinkhorn in wave 0
  if (threadIdx.x < kWave) {
    gates_wave<P>(m_raw, m_raw[R], S, S * H, scale, base, iters, eps, hb == 0,
                  pre + (size_t)t * S, post + (size_t)t * S, comb + (size_t)t * S * S, pre_lds);
  }
  __syncthreads();

  // 3. collapse from x (float4 over hidden)
  const int HQ = H >> 2;
  const int q0 = hb * quads_per_block;
  const int q1 = min(HQ, q0 + quads_per_block);
  float pc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) pc[c] = c < S ? pre_lds[c] : 0.f;
  const float4* xt = reinterpret_cast<const float4*>(x + (size_t)t * S * H);
  float4* yt = reinterpret_cast<float4*>(y + (size_t)t * H);
  for (int q = q0 + threadIdx.x; q < q1; q += 256) {
    float4 v = xt[q];
    float4 o = make_float4(pc[0] * v.x, pc[0] * v.y, pc[0] * v.z, pc[0] * v.w);
    for (int c = 1; c < S; ++c) {
      v = xt[(size_t)c * HQ + q];
      o.x = fmaf(pc[c], v.x, o.x);
      o.y = fmaf(pc[c], v.y, o.y);
      o.z = fmaf(pc[c], v.z, o.z);
      o.w = fmaf(pc[c], v.w, o.w);
    }
    yt[q] = o;
  }
}

hipError_t launch_finish(const float* x, const float* part, int G, int T, int S, int H,
                         const float* scale, const float* base, int iters, float eps,
                         float* pre, float* post, float* comb, float* y, hipStream_t st) {
  const int HQ = H / 4;
  // Enough blocks to fill the chip at small T; one block per token at large T.
  int HB = 1;
  if (T < 512) {
    HB = (1024 + T - 1) / T;
    HB = min(HB, (HQ + 63) / 64);
    HB = max(HB, 1);
  }
  const int qpb = (HQ + HB - 1) / HB;
  dim3 grid(T, HB);
#define MHC_F(PP)                                                                             \
  hipLaunchKernelGGL((finish_kernel<PP>), grid, dim3(256), 0, st, x, part, G, T, S, H, scale, \
                     base, iters, eps, pre, post, comb, y, qpb);                              \
  return hipGetLastError();
  if (S == 1) { MHC_F(1) }
  if (S == 2) { MHC_F(2) }
  if (S <= 4) { MHC_F(4) }
  if (S <= 8) { MHC_F(8) }
#undef MHC_F
  return hipErrorInvalidValue;
}

}  // namespace mhc
