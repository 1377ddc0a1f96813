// mhc_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Wavefront-level helpers (64 lanes), the gate epilogue and the one-wavefront
// Sinkhorn.  The gate forms and Sinkhorn semantics are the ones stated in
// include/mhc.h (hyper.rs page, module doc: arithmetic contract).
#pragma once
#include <hip/hip_runtime.h>

namespace mhc {

constexpr int kWave = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));

// Butterfly sum over the lanes whose index differs only in the bits of
// [lo, hi) (both powers of two).  Every participating lane ends with the same
// bits: at each level the two partners add the same pair of values.
template <int LO, int HI>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int o = LO; o < HI; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float sigmoidf_exact_ends(float z) {
  // 1/(1+exp(-z)): z -> -inf gives exactly 0, z -> +inf exactly 1.
  return 1.0f / (1.0f + expf(-z));
}

// Sinkhorn-Knopp on an S x S block held one entry per lane of one wavefront.
// Lane l holds entry (j = l / P, k = l % P) where P = S rounded up to a power
// of two (P*P <= 64); entries with j >= S or k >= S, and lanes >= P*P, hold 0
// and stay 0, so the padded sums equal the true sums.  One iteration = a row
// pass (sum over k, divide by sum + eps) then a column pass (sum over j).
template <int P>
__device__ __forceinline__ float sinkhorn_wave(float c, bool valid, int iters, float eps) {
  for (int it = 0; it < iters; ++it) {
    float s = xor_sum<1, P>(c);
    c = valid ? c / (s + eps) : 0.0f;
    s = xor_sum<P, P * P>(c);
    c = valid ? c / (s + eps) : 0.0f;
  }
  return c;
}

// Gate epilogue for one token, executed by ONE full wavefront (all 64 lanes
// must call it together).  m_raw[r] = fn_w[r,:] . x[t,:] (unscaled dots) and
// ss = sum x^2 live in LDS (or any memory visible to the wave).  Writes pre/post
// (S floats each) and comb (S*S floats, [j][k]) when `write_out` is set, and
// pre into pre_lds (for the collapse) when pre_lds is non-null.
template <int P>
__device__ __forceinline__ void gates_wave(const float* m_raw, float ss, int S, int n,
                                           const float* __restrict__ scale,
                                           const float* __restrict__ base, int iters,
                                           float eps, bool write_out,
                                           float* __restrict__ pre_out,
                                           float* __restrict__ post_out,
                                           float* __restrict__ comb_out, float* pre_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const float rinv = 1.0f / sqrtf(ss / (float)n + eps);
  const float s_pre = scale[0], s_post = scale[1], s_comb = scale[2];
  // pre / post gates: lanes [0, S) and [S, 2S)
  if (lane < 2 * S) {
    const float m = m_raw[lane] * rinv;
    if (lane < S) {
      const float g = sigmoidf_exact_ends(fmaf(s_pre, m, base[lane]));
      if (write_out) pre_out[lane] = g;
      if (pre_lds) pre_lds[lane] = g;
    } else {
      const float g = 2.0f * sigmoidf_exact_ends(fmaf(s_post, m, base[lane]));
      if (write_out) post_out[lane - S] = g;
    }
  }
  // comb: lane (j, k) with j = lane / P, k = lane % P
  const int j = lane / P, k = lane % P;
  const bool valid = (lane < P * P) && (j < S) && (k < S);
  float c = 0.0f;
  if (valid) {
    const int r = 2 * S + j * S + k;
    c = expf(fmaf(s_comb, m_raw[r] * rinv, base[r]));
  }
  c = sinkhorn_wave<P>(c, valid, iters, eps);
  if (valid && write_out) comb_out[j * S + k] = c;
}

}  // namespace mhc
