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
#include "mhc_device.h"
#include "mhc_kernels.h"

namespace mhc {

template <int NRT, int NTT>
__global__ __launch_bounds__(256) void partials_kernel(const float* __restrict__ x,
                                                       const float* __restrict__ fn_w, int T,
                                                       int n, int R, int chunks_per_range,
                                                       float* __restrict__ part) {
  constexpr int kVals = NRT * NTT * 4 + NTT;  // per lane, per wave
  __shared__ float red[4][kVals][kWave];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * (16 * NTT);
  const int g = blockIdx.y;
  const int nchunks = (n + 15) >> 4;
  const int c_beg = g * chunks_per_range;
  const int c_end = min(nchunks, c_beg + chunks_per_range);
  const int RP = R + 1;

  floatx4 acc[NRT][NTT];
  float ss[NTT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) ss[tt] = 0.f;

  const int sub = lane & 15;   // row within a row tile / token within a token tile
  const int kq = (lane >> 4) * 4;  // this lane's 4-float offset inside a 16-float chunk

  // Row and token pointers (clamped to a valid row so that masked lanes never
  // form an out-of-range address; their loads are skipped anyway).
  const float* wrow[NRT];
  bool wvalid[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rt * 16 + sub;
    wvalid[rt] = r < R;
    wrow[rt] = fn_w + (size_t)(wvalid[rt] ? r : 0) * n;
  }
  const float* xrow[NTT];
  bool xvalid[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int t = tok0 + tt * 16 + sub;
    xvalid[tt] = t < T;
    xrow[tt] = x + (size_t)(xvalid[tt] ? t : 0) * n;
  }

  for (int c = c_beg + wave; c < c_end; c += 4) {
    const int k = c * 16 + kq;
    const bool kin = k < n;  // n % 4 == 0, so a float4 is fully in or fully out
    float4 a[NRT], b[NTT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
      a[rt] = (kin && wvalid[rt]) ? *reinterpret_cast<const float4*>(wrow[rt] + k)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
      b[tt] = (kin && xvalid[tt]) ? *reinterpret_cast<const float4*>(xrow[tt] + k)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      ss[tt] = fmaf(b[tt].x, b[tt].x, ss[tt]);
      ss[tt] = fmaf(b[tt].y, b[tt].y, ss[tt]);
      ss[tt] = fmaf(b[tt].z, b[tt].z, ss[tt]);
      ss[tt] = fmaf(b[tt].w, b[tt].w, ss[tt]);
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].x, b[tt].x, acc[rt][tt], 0, 0, 0);
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].y, b[tt].y, acc[rt][tt], 0, 0, 0);
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].z, b[tt].z, acc[rt][tt], 0, 0, 0);
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].w, b[tt].w, acc[rt][tt], 0, 0, 0);
      }
  }

  // Sum of squares: lanes l, l^16, l^32, l^48 hold the same token's partials.
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) ss[tt] = xor_sum<16, 64>(ss[tt]);

  // Stage the wave's partials, then add the four waves in fixed order.
  {
    int v = 0;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][v++][lane] = acc[rt][tt][e];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) red[wave][v++][lane] = ss[tt];
  }
  __syncthreads();

  float* pg = part + (size_t)g * T * RP;
  for (int idx = threadIdx.x; idx < kVals * kWave; idx += 256) {
    const int v = idx / kWave, l = idx % kWave;
    const float s = ((red[0][v][l] + red[1][v][l]) + red[2][v][l]) + red[3][v][l];
    if (v < NRT * NTT * 4) {
      // MFMA D layout: row = 4*(l/16) + e within the row tile, token = l % 16.
      const int rt = v / (NTT * 4), tt = (v / 4) % NTT, e = v % 4;
      const int r = rt * 16 + 4 * (l >> 4) + e;
      const int t = tok0 + tt * 16 + (l & 15);
      if (r < R && t < T) pg[(size_t)t * RP + r] = s;
    } else {
      const int tt = v - NRT * NTT * 4;
      const int t = tok0 + tt * 16 + (l & 15);
      if (l < 16 && t < T) pg[(size_t)t * RP + R] = s;
    }
  }
}

template <int NRT, int NTT>
static hipError_t launch_partials_t(const float* x, const float* fn_w, int T, int n, int R,
                                    int G, int chunks_per_range, float* part, hipStream_t st) {
  dim3 grid((T + 16 * NTT - 1) / (16 * NTT), G);
  hipLaunchKernelGGL((partials_kernel<NRT, NTT>), grid, dim3(256), 0, st, x, fn_w, T, n, R,
                     chunks_per_range, part);
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
