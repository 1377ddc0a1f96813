// mhc_decode.hip -- one decode token's pre chain and branch-input epilogue in a
// single launch.
//
// Steps (hyper.rs page, module doc: arithmetic contract, lines one to four;
// the epilogue: hc_fused_gate.rs page, the v4z timing block).  At decode sizes
// the weight (1.5 MiB at 4 x 4096) is the only real traffic, so it is spread
// over G blocks that each produce split-K partials exactly as the small-batch
// partials kernel does (vector ALU, same per-token order).  Which block
// finishes is decided by a ticket counter, without any block waiting for
// another, so the kernel cannot stall on scheduling.  The block that draws the
// last ticket requests every partial and, right behind them, the collapse
// operands and the norm weight, adds the partials in the finish kernel's fixed
// order, and splits: wave 0 runs the gates and the Sinkhorn while the other
// waves compute the pre gates themselves and collapse, keeping y in registers;
// after one more barrier they run the epilogue (z = RMS-norm(y) * nw, q8 codes
// and scales).  It resets the counter for the next call.  Results are
// bit-identical to the two-kernel path (small-batch partials, finish kernel,
// epilogue kernel) for the same G.
//
// Without the epilogue the two-kernel path is as fast at one token and faster
// at two, so only the call with the epilogue uses this kernel, at T = 1; the
// kernel itself handles T <= 2.
#include "mhc_kernels.h"
#include "mhc_split.h"

namespace mhc {

constexpr int kD4Batch = 6;  // collapse quads in flight per collapse thread
constexpr int kD4ZqBatches = 2;  // collapse batches whose y the epilogue keeps in registers

template <int RPT>
__global__ __launch_bounds__(256) void decode_zq8_kernel(
    const float* __restrict__ x, const float* __restrict__ fn_w, const float* __restrict__ scale,
    const float* __restrict__ base, int T, int S, int H, int iters, float eps,
    int chunks_per_range, float* __restrict__ part, unsigned int* __restrict__ counter,
    float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb,
    float* __restrict__ y, Zq8Out zq) {
  constexpr int KB = kD4Batch;
  __shared__ float red256[2][256];
  __shared__ float zred[4][2];
  __shared__ float m_raw[2][32];
  __shared__ float params[3 + 24];
  __shared__ int is_last;

  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = S * H, R = (2 + S) * S, RP = R + 1;
  const int nchunks = (n + 15) >> 4;
  const int c_beg = g * chunks_per_range;
  const int c_end = min(nchunks, c_beg + chunks_per_range);
  stage_site_params(scale, base, R, params);

  float* pg = part + (size_t)g * T * RP;
  small_partials<2, RPT>(x, fn_w, T, n, R, c_beg * 16, min(n, c_end * 16),
                         [=](size_t i, float v) { store_partial<true>(pg + i, v); });
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are complete ...
  __syncthreads();                // ... and so are those of the whole block
  // The ticket: a release of the block's partials (ordered before it by the
  // barrier) and, for the block that draws the last ticket, an acquire of
  // everyone else's, both at agent scope, so that the last block's loads below
  // see every partial under the memory model and not only on this hardware.
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(G - 1);
  __syncthreads();
  if (!is_last) return;
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // The last block.  First every partial is requested (thread (r, q) takes
  // blocks q, q + Q, ... of row r, the order in which the finish kernel adds
  // them), then the first collapse operands, so that the reduction waits only
  // for its own loads while the operands stream in behind them.
  const int Q = 256 / RP;
  const int r = tid % RP, q = tid / RP;
  const bool rq = q < Q;
  const int qc = rq ? q : 0;
  float v[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int gg = qc + u * Q;
      v[t][u] = load_partial<true>(part + ((size_t)(gg < G ? gg : 0) * T + (t < T ? t : 0)) * RP + r);
    }
  __builtin_amdgcn_sched_barrier(0);

  const int wave = tid >> 6;
  const int ct = tid - kWave, nct = 3 * kWave;
  const int HQ = H >> 2;
  const int total = T * HQ;
  float4 xq[KB][4];
  float4 wk[kD4ZqBatches][KB];  // epilogue weight quads of the kept batches
  const float4* nw4 = reinterpret_cast<const float4*>(zq.nw);
  auto load_batch = [&](int i0, int bb) {
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int idx = i0 + k * nct;
      const int ic = idx < total ? idx : 0;  // past the end: re-read quad 0, never stored
      const int t = ic / HQ, qq = ic - t * HQ;
      const float4* xt = reinterpret_cast<const float4*>(x + (size_t)t * S * H) + qq;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < S) xq[k][c] = xt[(size_t)c * HQ];
    }
    // the norm weight behind the x quads, so the collapse does not wait for it
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int idx = i0 + k * nct;
      const int ic = idx < total ? idx : 0;
      wk[bb][k] = nw4[ic - (ic / HQ) * HQ];
    }
  };
  if (wave >= 1) load_batch(ct, 0);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (rq && qc + u * Q < G) s += v[t][u];
    red256[t][tid] = s;
  }
  __syncthreads();
  if (tid < RP)
    for (int t = 0; t < T; ++t) {
      float s = 0.f;
      for (int qi = 0; qi < Q; ++qi) s += red256[t][qi * RP + tid];
      m_raw[t][tid] = s;
    }
  __syncthreads();

  if (wave == 0) {
    gates_wave<4, false>(&m_raw[0][0], 32, T, S, n, params, iters, eps, true, pre, post, comb,
                         nullptr);
    // wave 0 then meets the collapse waves at the epilogue's barrier
  }

  // collapse: y[t, i] = sum_c pre[t, c] * x[t, c, i]
  float pc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      pc[t][c] = (t < T && c < S) ? pre_gate(m_raw[t], c, R, n, eps, params) : 0.f;
  if (wave != 0 && ct < T * S) pre[ct] = pre_gate(m_raw[ct / S], ct % S, R, n, eps, params);
  // Collapse with y kept in registers (T*H/4 <= kD4ZqBatches*KB*192 quads),
  // then the branch-input epilogue.  [T][H] outputs are indexed by the
  // flattened quad idx = t*H/4 + quad; H % 32 == 0 puts the 8 quads of a
  // 32-entry block in 8 neighbouring lanes (idx = ct mod 8) of one token,
  // wholly before or past the end.
  float4 yk[kD4ZqBatches][KB];
  float ys[2] = {0.f, 0.f};
  if (wave != 0) {
#pragma unroll
    for (int bb = 0; bb < kD4ZqBatches; ++bb) {
      if (bb * KB * nct < total) {  // the same in every thread
        const int i0 = ct + bb * KB * nct;
        if (bb != 0) load_batch(i0, bb);
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int idx = i0 + k * nct;
          const int ic = idx < total ? idx : 0;
          const int t = ic / HQ;
          yk[bb][k] = collapse4<4>(t == 0 ? pc[0] : pc[1], xq[k], S);
          if (idx < total) {
            reinterpret_cast<float4*>(y)[idx] = yk[bb][k];
            if (t == 0)
              ys[0] = sq4(yk[bb][k], ys[0]);
            else
              ys[1] = sq4(yk[bb][k], ys[1]);
          }
        }
      }
    }
    // sums of squares of y per token: each wave, then waves 1, 2, 3 in order
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float sw = sum_wave(ys[t]);
      if ((tid & (kWave - 1)) == 0) zred[wave][t] = sw;
    }
  }
  __syncthreads();  // all four waves (wave 0 once its Sinkhorn is done)
  if (wave == 0) return;
  const float r0 = zq8_rinv(zred[1][0] + zred[2][0] + zred[3][0], H, zq.norm_eps);
  const float r1 = zq8_rinv(zred[1][1] + zred[2][1] + zred[3][1], H, zq.norm_eps);
#pragma unroll
  for (int bb = 0; bb < kD4ZqBatches; ++bb) {
    if (bb * KB * nct < total) {
      const int i0 = ct + bb * KB * nct;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int idx = i0 + k * nct;
        const int ic = idx < total ? idx : 0;
        const float4 o = zq8_norm(yk[bb][k], ic < HQ ? r0 : r1, wk[bb][k]);
        float db;
        const char4 cq = zq8_codes(o, &db);
        if (idx < total) {
          reinterpret_cast<float4*>(zq.z)[idx] = o;
          reinterpret_cast<char4*>(zq.q)[idx] = cq;
          if ((idx & 7) == 0) zq.d[idx >> 3] = db;
        }
      }
    }
  }
}

bool decode_zq8_supported(int T, int S, int H, int G) {
  const int RP = (2 + S) * S + 1;
  return T == 1 && S >= 1 && S <= 4 && G >= 1 && G <= 16 * (256 / RP) && H % 32 == 0 &&
         (long)T * (H / 4) <= (long)kD4ZqBatches * kD4Batch * 3 * kWave;
}

hipError_t launch_decode_zq8(const float* x, const float* fn_w, const float* scale,
                             const float* base, int T, int S, int H, int iters, float eps, int G,
                             int chunks_per_range, float* part, unsigned int* counter, float* pre,
                             float* post, float* comb, float* y, const Zq8Out& zq,
                             hipStream_t st) {
  if (!decode_zq8_supported(T, S, H, G)) return hipErrorInvalidValue;
  const int rpt = small_rows_per_thread(S);
#define MHC_DZ(RP_)                                                                            \
  if (rpt == RP_) {                                                                            \
    hipLaunchKernelGGL((decode_zq8_kernel<RP_>), dim3(G), dim3(256), 0, st, x, fn_w, scale,     \
                       base, T, S, H, iters, eps, chunks_per_range, part, counter, pre, post,   \
                       comb, y, zq);                                                            \
    return hipGetLastError();                                                                  \
  }
  MHC_DZ(1) MHC_DZ(2) MHC_DZ(4)
#undef MHC_DZ
  return hipErrorInvalidValue;
}

}  // namespace mhc
