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
  reduce_token_partials<16>(part, G, T, t, RP, red, m_raw);

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

// One decode token (T = 1, S <= 4) with the branch-input epilogue (hc_fused_gate.rs
// page, the v4z timing block: RMS norm of y with nw, q8 codes and block scales).
// Two blocks that each add the partials in the fixed order above:
//   block 0: comb (gates and Sinkhorn) on wave 0, pre and post on wave 3;
//   block 1: the collapse of every hidden quad (quads tid + 256k, y kept in
//            registers), then the epilogue exactly as the standalone epilogue
//            kernel computes it (the same per-thread sums, the same block tree),
//            so that z, q and d equal the two-launch result bit for bit.
// The epilogue block never waits for the Sinkhorn.  Block 1 requests its x
// and nw quads right behind the partials (block 0 requests the same offsets
// out of range, so that both blocks run the same wait sequence).
template <int KQ>
__global__ __launch_bounds__(256) void finish_zq8_kernel(
    const float* __restrict__ x, const float* __restrict__ part, int G, int S, int H,
    const float* __restrict__ scale, const float* __restrict__ base, int iters, float eps,
    float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb,
    float* __restrict__ y, Zq8Out zq) {
  const int R = (2 + S) * S;
  const int RP = R + 1;
  const int n = S * H;
  const int HQ = H >> 2;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  __shared__ float red[256];
  __shared__ float m_raw[32];
  __shared__ float params[3 + 24];
  __shared__ float pre_lds[8];
  stage_site_params(scale, base, R, params);
  const bool gates = blockIdx.x == 0;  // block-uniform

  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x), (short)0, n * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(zq.nw), (short)0, H * 4, 0x00020000);
  float4 xq[KQ][4], wq[KQ];
  auto ld = [](__amdgpu_buffer_rsrc_t rs, unsigned off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
  };
  auto request = [&]() {
#pragma unroll
    for (int k = 0; k < KQ; ++k) {
      const int q = tid + 256 * k;
      // streams past S, quads past H / 4 and block 0's requests fall past the
      // end of their buffer and read zero (offsets are unsigned to the unit)
      unsigned off = (!gates && q < HQ) ? 16u * q : 0x7FFFFFF0u;
      asm volatile("" : "+v"(off));  // a plain offset, not a branch per load
#pragma unroll
      for (int c = 0; c < 4; ++c) xq[k][c] = ld(xrs, off + (unsigned)c * (unsigned)H * 4u);
      wq[k] = ld(wrs, off);
    }
  };
  reduce_token_partials<16>(part, G, 1, 0, RP, red, m_raw, request);

  if (gates) {
    if (wave == 0)
      gates_comb<4>(m_raw, 0, 1, S, n, params, iters, eps, true, comb);
    else if (wave == 3)
      gates_pre_post<4>(m_raw, 0, 1, S, n, params, eps, true, pre, post, pre_lds);
    return;
  }

  float pc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) pc[c] = c < S ? pre_gate(m_raw, c, R, n, eps, params) : 0.f;
  float4 yk[KQ];
  float ss = 0.f;
  float4* y4 = reinterpret_cast<float4*>(y);
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const int q = tid + 256 * k;
    yk[k] = q < HQ ? collapse4<4>(pc, xq[k], S) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (q < HQ) y4[q] = yk[k];
    ss = sq4(yk[k], ss);
  }
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float r = zq8_rinv(red[0], H, zq.norm_eps);
  float4* zt = reinterpret_cast<float4*>(zq.z);
  char4* qt = reinterpret_cast<char4*>(zq.q);
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const int q = tid + 256 * k;
    const bool in = q < HQ;  // HQ % 8 == 0: a 32-entry block is all in or all out
    const float4 o = zq8_norm(yk[k], r, wq[k]);
    float db;
    const char4 cq = zq8_codes(o, &db);
    if (in) {
      zt[q] = o;
      qt[q] = cq;
      if ((tid & 7) == 0) zq.d[q >> 3] = db;
    }
  }
}

bool finish_zq8_supported(int T, int S, int H) {
  return T == 1 && S >= 1 && S <= 4 && H % 32 == 0 && H / 4 <= 8 * 256;
}

hipError_t launch_finish_zq8(const float* x, const float* part, int G, int S, int H,
                             const float* scale, const float* base, int iters, float eps,
                             float* pre, float* post, float* comb, float* y, const Zq8Out& zq,
                             hipStream_t st) {
  if (!finish_zq8_supported(1, S, H)) return hipErrorInvalidValue;
  if (H / 4 <= 4 * 256)
    hipLaunchKernelGGL((finish_zq8_kernel<4>), dim3(2), dim3(256), 0, st, x, part, G, S, H, scale,
                       base, iters, eps, pre, post, comb, y, zq);
  else
    hipLaunchKernelGGL((finish_zq8_kernel<8>), dim3(2), dim3(256), 0, st, x, part, G, S, H, scale,
                       base, iters, eps, pre, post, comb, y, zq);
  return hipGetLastError();
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
