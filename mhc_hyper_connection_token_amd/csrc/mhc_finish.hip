// mhc_finish.hip -- per-token finish of the pre chain from split-K partials.
//
// Steps (hyper.rs page, module doc: arithmetic contract, lines two to four):
// add the G partial mixes / sums of squares of a token in fixed order, apply
// the RMS rescale, the three gate groups and the Sinkhorn (one wavefront, lane
// exchanges on DPP / permlane, no barrier inside the iteration loop), then
// collapse the streams: y[t,i] = sum_c pre[t,c] * x[t,c,i].
//
// Grid: (T, HB).  Block y-index hb covers a contiguous range of hidden quads
// for the collapse; every block of a token recomputes the (cheap) pre gates so
// that no cross-block wait is needed, and only hb == 0 runs the Sinkhorn and
// writes pre/post/comb.  The
// first x quads of the collapse are loaded before the gates are computed, so
// their latency hides behind the reduction and the Sinkhorn.
#include "mhc_kernels.h"
#include "mhc_split.h"

namespace mhc {

template <int L>
__global__ __launch_bounds__(256) void finish_kernel(
    const float* __restrict__ x, const float* __restrict__ part, int G, int T, int S, int H,
    const float* __restrict__ scale, const float* __restrict__ base, int iters, float eps,
    float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb,
    float* __restrict__ y, int quads_per_block) {
  const int R = (2 + S) * S;
  const int RP = R + 1;
  const int t = blockIdx.x;
  const int hb = blockIdx.y;
  const int HQ = H >> 2;
  __shared__ float red[256];
  __shared__ float m_raw[96];
  __shared__ float params[3 + 80];
  stage_site_params(scale, base, R, params);

  // 0. first collapse quad of this thread, loaded early
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

  // 1. fixed-order reduction of the G partials
  reduce_token_partials<false, 16>(part, G, T, t, RP, red, m_raw);

  // 2. pre gates, computed by every thread (uniform); only block hb == 0 runs
  // the Sinkhorn (wave 0, post and comb) and writes the gates.  No barrier
  // follows, so the other waves collapse while wave 0 iterates.
  float pc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) pc[c] = c < S ? pre_gate(m_raw, c, R, S * H, eps, params) : 0.f;
  if (hb == 0) {
    if (threadIdx.x < S)
      pre[(size_t)t * S + threadIdx.x] = pre_gate(m_raw, threadIdx.x, R, S * H, eps, params);
    if (threadIdx.x < kWave)
      gates_wave<L, false>(m_raw, 0, 1, S, S * H, params, iters, eps, true, nullptr,
                           post + (size_t)t * S, comb + (size_t)t * S * S, nullptr);
  }

  // 3. collapse
  float4* yt = reinterpret_cast<float4*>(y + (size_t)t * H);
  if (qa < q1) yt[qa] = collapse4<8>(pc, xq, S);
  for (int q = qa + 256; q < q1; q += 256) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < S) xq[c] = xt[(size_t)c * HQ + q];
    yt[q] = collapse4<8>(pc, xq, S);
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
  if (S <= 4)
    hipLaunchKernelGGL((finish_kernel<4>), grid, dim3(256), 0, st, x, part, G, T, S, H, scale,
                       base, iters, eps, pre, post, comb, y, qpb);
  else
    hipLaunchKernelGGL((finish_kernel<8>), grid, dim3(256), 0, st, x, part, G, T, S, H, scale,
                       base, iters, eps, pre, post, comb, y, qpb);
  return hipGetLastError();
}

}  // namespace mhc
