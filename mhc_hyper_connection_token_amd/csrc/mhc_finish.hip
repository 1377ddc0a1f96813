// mhc_finish.hip -- per-token finish of the pre chain from split-K partials.
//
// Steps (hyper.rs page, module doc: arithmetic contract, lines two to four):
// add the G partial mixes / sums of squares of a token in fixed order, apply
// the RMS rescale, the three gate groups and the Sinkhorn (one wavefront, lane
// exchanges on DPP / permlane, no barrier inside the iteration loop), then
// collapse the streams: y[t,i] = sum_c pre[t,c] * x[t,c,i].
//
// Grid: (T, HB).  Block y-index hb covers a contiguous range of hidden quads
// for the collapse; every thread that collapses computes the (cheap) pre gates
// itself, so that no cross-block wait is needed.  In block hb == 0, wave 0
// runs the comb gates and the Sinkhorn while wave 3 writes pre and post.  Wave 0
// takes the last quads of each 256, so that where a block has at most 192
// quads (small T) the Sinkhorn wave does no collapse work.  Blocks with more
// than one pass of quads request their first collapse operands before the
// reduction, to hide that latency; single-pass blocks request them after it,
// so that the reduction does not wait behind them (loads complete in order).
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
  __shared__ float pre_lds[8];
  stage_site_params(scale, base, R, params);

  const int q0 = hb * quads_per_block;
  const int q1 = min(HQ, q0 + quads_per_block);
  const bool early = q1 - q0 > 256;  // block-uniform
  const float4* xt = reinterpret_cast<const float4*>(x + (size_t)t * S * H);
  const int qa = q0 + ((threadIdx.x + 192) & 255);
  float4 xq[8];
  auto load_quads = [&](int q) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < S) xq[c] = xt[(size_t)c * HQ + q];
  };
  if (early && qa < q1) load_quads(qa);

  // 1. fixed-order reduction of the G partials
  reduce_token_partials<false, 16>(part, G, T, t, RP, red, m_raw);

  // 2. block 0: comb (gates and Sinkhorn) on wave 0, pre and post on wave 3
  if (hb == 0) {
    if (threadIdx.x < kWave)
      gates_comb<L>(m_raw, 0, 1, S, S * H, params, iters, eps, true, comb + (size_t)t * S * S);
    else if (threadIdx.x >= 3 * kWave)
      gates_pre_post<L>(m_raw, 0, 1, S, S * H, params, eps, true, pre + (size_t)t * S,
                        post + (size_t)t * S, pre_lds);
  }

  // 3. collapse
  if (qa < q1) {
    if (!early) load_quads(qa);
    float pc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) pc[c] = c < S ? pre_gate(m_raw, c, R, S * H, eps, params) : 0.f;
    float4* yt = reinterpret_cast<float4*>(y + (size_t)t * H);
    yt[qa] = collapse4<8>(pc, xq, S);
    for (int q = qa + 256; q < q1; q += 256) {
      load_quads(q);
      yt[q] = collapse4<8>(pc, xq, S);
    }
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
