// mhc_zq8.hip -- branch-input epilogue of a pre site: the RMS norm of y with a
// weight nw and its int8 q8 encoding (hc_fused_gate.rs page, the v4z timing
// block: the norm-and-q8 step that feeds the branch, epsilon 1e-5, int8 codes
// q[H] and fp32 scales d[H/32]).  Per token t:
//   z[t,i] = y[t,i] * nw[i] * r,   r = 1/sqrt(mean_i y[t,i]^2 + norm_eps)
//   per block of 32 consecutive i: d = max|z| / 127; q = z * (1/d) rounded to
//   nearest with ties away from zero (d = 0 and q = 0 for an all-zero block).
// (The arithmetic of one entry and one block is in mhc_device.h, shared with
// the pre kernels that run this epilogue in their own tail.)
//
// Standalone form, for the shapes whose pre kernel does not: one block of 256
// threads per token; each thread owns hidden quads
// q4 = tid, tid + 256, ...; the eight threads of a 32-entry block are eight
// neighbouring lanes, so the block maximum is a three-step lane butterfly.
#include "mhc_device.h"
#include "mhc_kernels.h"

namespace mhc {

constexpr int kZq8MaxQuads = 8;  // hidden up to 8 * 256 * 4 = 8192 per token

__global__ __launch_bounds__(256) void zq8_kernel(const float* __restrict__ y,
                                                  const float* __restrict__ nw, int H,
                                                  float norm_eps, float* __restrict__ z,
                                                  signed char* __restrict__ q,
                                                  float* __restrict__ d) {
  __shared__ float red[256];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int HQ = H >> 2;
  const float4* yt = reinterpret_cast<const float4*>(y + (size_t)t * H);
  float4 v[kZq8MaxQuads];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kZq8MaxQuads; ++k) {
    const int i = tid + 256 * k;
    v[k] = i < HQ ? yt[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss = sq4(v[k], ss);
  }
  // fixed-order block sum of the squares
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float r = zq8_rinv(red[0], H, norm_eps);
  const float4* w4 = reinterpret_cast<const float4*>(nw);
  float4* zt = reinterpret_cast<float4*>(z + (size_t)t * H);
  char4* qt = reinterpret_cast<char4*>(q + (size_t)t * H);
  float* dt = d + (size_t)t * (H >> 5);
#pragma unroll
  for (int k = 0; k < kZq8MaxQuads; ++k) {
    const int i = tid + 256 * k;
    const bool in = i < HQ;  // HQ % 8 == 0: a 32-entry block is all in or all out
    const float4 w = in ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 o = zq8_norm(v[k], r, w);
    float db;
    const char4 c = zq8_codes(o, &db);
    if (in) {
      zt[i] = o;
      qt[i] = c;
      if ((tid & 7) == 0) dt[i >> 3] = db;
    }
  }
}

bool zq8_supported(int H) { return H % 32 == 0 && H / 4 <= kZq8MaxQuads * 256; }

hipError_t launch_zq8(const float* y, const float* nw, int T, int H, float norm_eps, float* z,
                      signed char* q, float* d, hipStream_t st) {
  if (!zq8_supported(H)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zq8_kernel, dim3(T), dim3(256), 0, st, y, nw, H, norm_eps, z, q, d);
  return hipGetLastError();
}

}  // namespace mhc
