// mhc_partials.hip -- split-K partial mixes and sums of squares on MFMA.
//
// Step: the mixes projection raw[t,r] = sum_i fn_w[r,i] * x[t,i] over each
// token's contiguous S*H slab, plus ss[t] = sum_i x[t,i]^2 (hyper.rs page,
// module doc: arithmetic contract, first two lines).  This kernel produces
// PARTIAL sums over one K-range of the slab:
//
//   part[g][t][r]  for r < R   : partial raw over the g-th K-range
//   part[g][t][R]              : partial ss over the g-th K-range
//
// The contraction runs on v_mfma_f32_16x16x4_f32 (fp32 operands, exact fp32
// products, fp32 accumulation): A = fn_w rows (16 per tile), B = token slabs
// (16 tokens per tile), K along the slab.  Each lane loads 16 bytes of one
// weight row and 16 bytes of one token slab per 16-element K chunk; the four
// floats feed four MFMAs, the k-index of each MFMA block being whatever the
// lanes hold (A and B agree by construction).  Sums of squares ride along on
// the VALU from the same B registers.
//
// Grid: (token tiles of 16*NTT tokens, G K-ranges).  Block: 256 threads = four
// waves, each wave taking every fourth K chunk of the block's K-range; the four
// wave partials are added in fixed wave order through LDS, so the result does
// not depend on T or on scheduling.
#include "mhc_kernels.h"
#include "mhc_split.h"

namespace mhc {

template <int NRT, int NTT>
__global__ __launch_bounds__(256) void partials_kernel(const float* __restrict__ x,
                                                       const float* __restrict__ fn_w, int T,
                                                       int n, int R, int chunks_per_range,
                                                       float* __restrict__ part) {
  constexpr int kVals = NRT * NTT * 4 + NTT;
  __shared__ float red[4 * kVals * kWave];
  const int g = blockIdx.y;
  const int nchunks = (n + 15) >> 4;
  const int c_beg = g * chunks_per_range;
  const int c_end = min(nchunks, c_beg + chunks_per_range);
  float* pg = part + (size_t)g * T * (R + 1);
  block_partials<NRT, NTT>(x, fn_w, T, n, R, blockIdx.x * (16 * NTT), c_beg, c_end, red,
                           [=](size_t i, float v) { pg[i] = v; });
}

template <int NRT, int NTT>
static hipError_t launch_partials_t(const float* x, const float* fn_w, int T, int n, int R,
                                    int G, int chunks_per_range, float* part, hipStream_t st) {
  dim3 grid((T + 16 * NTT - 1) / (16 * NTT), G);
  hipLaunchKernelGGL((partials_kernel<NRT, NTT>), grid, dim3(256), 0, st, x, fn_w, T, n, R,
                     chunks_per_range, part);
  return hipGetLastError();
}

// Vector-ALU partials (S <= 4), one token at a time in the same order as the
// single-launch decode kernel, so a token's result does not depend on the
// batch it is in.  Grid: (G K-ranges, groups of 16 tokens).
template <int RPT>
__global__ __launch_bounds__(256) void small_partials_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ fn_w,
                                                             int T, int n, int R,
                                                             int chunks_per_range,
                                                             float* __restrict__ part) {
  const int g = blockIdx.x;
  const int t0 = blockIdx.y * 16;
  const int k_beg = g * chunks_per_range * 16;
  const int k_end = min(n, k_beg + chunks_per_range * 16);
  float* pg = part + ((size_t)g * T + t0) * (R + 1);
  small_partials<16, RPT>(x + (size_t)t0 * n, fn_w, min(16, T - t0), n, R, k_beg, k_end,
                          [=](size_t i, float v) { pg[i] = v; });
}

int small_rows_per_thread(int S) {
  const int rows = (2 + S) * S + 1;  // R rows and the sum of squares
  const int rpt = (rows + 7) / 8;
  return rpt <= 1 ? 1 : (rpt <= 2 ? 2 : (rpt <= 4 ? 4 : 0));
}

hipError_t launch_small_partials(const float* x, const float* fn_w, int T, int S, int H, int G,
                                 int chunks_per_range, float* part, hipStream_t st) {
  if (T < 1 || T > 65535 * 16) return hipErrorInvalidValue;
  const int n = S * H, R = (2 + S) * S;
  const dim3 grid(G, (T + 15) / 16);
  switch (small_rows_per_thread(S)) {
    case 1:
      hipLaunchKernelGGL((small_partials_kernel<1>), grid, dim3(256), 0, st, x, fn_w, T, n, R,
                         chunks_per_range, part);
      break;
    case 2:
      hipLaunchKernelGGL((small_partials_kernel<2>), grid, dim3(256), 0, st, x, fn_w, T, n, R,
                         chunks_per_range, part);
      break;
    case 4:
      hipLaunchKernelGGL((small_partials_kernel<4>), grid, dim3(256), 0, st, x, fn_w, T, n, R,
                         chunks_per_range, part);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_partials(const float* x, const float* fn_w, int T, int n, int R, int ntt,
                           int G, int chunks_per_range, float* part, hipStream_t st) {
  const int nrt = (R + 15) / 16;
#define MHC_P(NR, NT)                                                                     \
  if (nrt == NR && ntt == NT)                                                              \
    return launch_partials_t<NR, NT>(x, fn_w, T, n, R, G, chunks_per_range, part, st);
  MHC_P(1, 1) MHC_P(1, 4) MHC_P(2, 1) MHC_P(2, 4) MHC_P(3, 1) MHC_P(3, 4)
  MHC_P(4, 1) MHC_P(4, 2) MHC_P(5, 1) MHC_P(5, 2)
#undef MHC_P
  return hipErrorInvalidValue;
}

}  // namespace mhc
