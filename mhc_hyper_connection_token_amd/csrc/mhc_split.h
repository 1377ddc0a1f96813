// mhc_split.h -- device routines of the split-K pre path, shared by the
// partials, finish and single-launch decode kernels so that all of them add
// the same numbers in the same order.
#pragma once
#include "mhc_device.h"

namespace mhc {

// Per-block split-K partials (hyper.rs page, module doc: arithmetic contract,
// first two lines): for tokens [tok0, tok0 + 16*NTT) and the 16-float K chunks
// [c_beg, c_end) of the slab, the partial dots with the R weight rows and the
// partial sum of squares, handed to sink(t*(R+1) + r, value) (r == R: sum of
// squares; t is the token's index in the batch).
// 256 threads = four waves; wave w takes chunks c_beg + w, c_beg + w + 4, ...;
// the four wave partials are added in wave order through `red`
// (4 * (NRT*NTT*4 + NTT) * 64 floats of LDS).
//
// The contraction runs on v_mfma_f32_16x16x4_f32 (fp32 operands, exact fp32
// products, fp32 accumulation): A = weight rows (16 per tile), B = token slabs
// (16 tokens per tile).  Each lane loads 16 bytes of one weight row and 16
// bytes of one token slab per chunk; the four floats feed four MFMAs whose
// k-index is whatever the lanes hold (A and B agree by construction).
// Plain store, or (COHERENT) an agent-scope relaxed atomic store that is
// written through to the device-coherent level, for partials that another
// block reads in the same launch.
template <bool COHERENT>
__device__ __forceinline__ void store_partial(float* p, float v) {
  if (COHERENT)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COHERENT>
__device__ __forceinline__ float load_partial(const float* p) {
  if (COHERENT) return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

template <int NRT, int NTT, class Sink>
__device__ __forceinline__ void block_partials(const float* __restrict__ x,
                                               const float* __restrict__ fn_w, int T, int n,
                                               int R, int tok0, int c_beg, int c_end,
                                               float* red, Sink sink) {
  constexpr int kVals = NRT * NTT * 4 + NTT;  // per lane, per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int RP = R + 1;

  floatx4 acc[NRT][NTT];
  float ss[NTT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) ss[tt] = 0.f;

  const int sub = lane & 15;       // row within a row tile / token within a token tile
  const int kq = (lane >> 4) * 4;  // this lane's 4-float offset inside a 16-float chunk

  // Row and token pointers, clamped to a valid row / token: out-of-range lanes
  // read valid memory and are zeroed before use.
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

  // Double-buffered chunk loop: the loads of chunk c + 4 are issued before the
  // MFMAs of chunk c.  Loads are branch-free (clamped addresses) and the
  // out-of-range lanes are zeroed by a select when the chunk is consumed.
  auto load_chunk = [&](int c, float4* a, float4* b) {
    const int k = c * 16 + kq;
    const int kc = k < n ? k : 0;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) a[rt] = *reinterpret_cast<const float4*>(wrow[rt] + kc);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) b[tt] = *reinterpret_cast<const float4*>(xrow[tt] + kc);
  };
  auto sel = [](bool ok, float4 v) {
    return make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
  };
  float4 a0[NRT], b0[NTT], a1[NRT], b1[NTT];
  int c = c_beg + wave;
  if (c < c_end) load_chunk(c, a0, b0);
  while (c < c_end) {
    const int cn = c + 4;
    if (cn < c_end) load_chunk(cn, a1, b1);
    const bool kin = c * 16 + kq < n;  // n % 4 == 0: a float4 is fully in or fully out
    float4 a[NRT], b[NTT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) a[rt] = sel(kin && wvalid[rt], a0[rt]);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) b[tt] = sel(kin && xvalid[tt], b0[tt]);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      ss[tt] = fmaf(b[tt].x, b[tt].x, ss[tt]);
      ss[tt] = fmaf(b[tt].y, b[tt].y, ss[tt]);
      ss[tt] = fmaf(b[tt].z, b[tt].z, ss[tt]);
      ss[tt] = fmaf(b[tt].w, b[tt].w, ss[tt]);
    }
    // Component-major issue: consecutive MFMAs go to different accumulators, so
    // none waits for the previous one (each accumulator still adds x, y, z, w
    // in that order).
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].x, b[tt].x, acc[rt][tt], 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].y, b[tt].y, acc[rt][tt], 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].z, b[tt].z, acc[rt][tt], 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt].w, b[tt].w, acc[rt][tt], 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) a0[rt] = a1[rt];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) b0[tt] = b1[tt];
    c = cn;
  }

  // Sum of squares: lanes l, l^16, l^32, l^48 hold the same token's partials.
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) ss[tt] = swap32_sum(swap16_sum(ss[tt]));

  // Stage the wave's partials, then add the four waves in fixed order.
  {
    int v = 0;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(wave * kVals + v++) * kWave + lane] = acc[rt][tt][e];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) red[(wave * kVals + v++) * kWave + lane] = ss[tt];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kVals * kWave; idx += 256) {
    const int v = idx / kWave, l = idx % kWave;
    const float s = ((red[(0 * kVals + v) * kWave + l] + red[(1 * kVals + v) * kWave + l]) +
                     red[(2 * kVals + v) * kWave + l]) +
                    red[(3 * kVals + v) * kWave + l];
    if (v < NRT * NTT * 4) {
      // MFMA D layout: row = 4*(l/16) + e within the row tile, token = l % 16.
      const int rt = v / (NTT * 4), tt = (v / 4) % NTT, e = v % 4;
      const int r = rt * 16 + 4 * (l >> 4) + e;
      const int t = tok0 + tt * 16 + (l & 15);
      if (r < R && t < T) sink((size_t)t * RP + r, s);
    } else {
      const int tt = v - NRT * NTT * 4;
      const int t = tok0 + tt * 16 + (l & 15);
      if (l < 16 && t < T) sink((size_t)t * RP + R, s);
    }
  }
}

// Split-K partials of a small batch (T <= TMAX tokens) on the vector ALU: for
// every token t and row r < R the dot of fn_w[r, k_beg:k_end] with
// x[t, k_beg:k_end], and at r == R the sum of squares of that slice, handed to
// sink(t*(R+1) + r, value).  256 threads = 8 row slots x 32 lanes: lane l of
// slot s takes the column quads l, l + 32, ... and rows s, s + 8, s + 16, ...
// (RPT of them), so every weight load is a coalesced run of one row.  A
// token's arithmetic (the order of its products and of the 32-lane butterfly
// sum) does not depend on T or TMAX: a token's partials are the same in any
// small batch.  k_beg and k_end are multiples of 4.
template <int TMAX, int RPT, class Sink>
__device__ __forceinline__ void small_partials(const float* __restrict__ x,
                                               const float* __restrict__ fn_w, int T, int n,
                                               int R, int k_beg, int k_end, Sink sink) {
  const int tid = threadIdx.x;
  const int l = tid & 31, slot = tid >> 5;
  const int nq = (k_end - k_beg) >> 2;
  float acc[RPT][TMAX];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[i][t] = 0.f;
  for (int q = l; q < nq; q += 32) {
    const int col = k_beg + 4 * q;
    // all loads of this column quad first (branch-free: clamped rows / tokens)
    float4 w[RPT], xv[TMAX];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = slot + 8 * i;
      w[i] = *reinterpret_cast<const float4*>(fn_w + (size_t)(r < R ? r : 0) * n + col);
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      xv[t] = *reinterpret_cast<const float4*>(x + (size_t)(t < T ? t : 0) * n + col);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = slot + 8 * i;
      const float4 wi = r == R ? make_float4(1.f, 1.f, 1.f, 1.f) : w[i];
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        // the sum-of-squares row multiplies x by itself
        const float4 a = r == R ? xv[t] : wi;
        float v = acc[i][t];
        v = fmaf(a.x, xv[t].x, v);
        v = fmaf(a.y, xv[t].y, v);
        v = fmaf(a.z, xv[t].z, v);
        v = fmaf(a.w, xv[t].w, v);
        acc[i][t] = v;
      }
    }
  }
  const int RP = R + 1;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = slot + 8 * i;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      float v = acc[i][t];
      v = sum_xor1_2(v);
      v = sum_xor4_in8(v);
      v = sum_xor8_in16(v);
      v = swap16_sum(v);
      if (l == 0 && t < T && r <= R) sink((size_t)t * RP + r, v);
    }
  }
}

// Fixed-order sum of the G partials of token t into m_out[0..R] (256 threads):
// thread (r, q), q < Q = 256 / (R+1), adds g = q, q + Q, q + 2Q, ... in that
// order (eight independent loads in flight per batch); then thread r adds the Q
// sums in q order.  The order depends only on G and R, not on T.  Ends with a
// block barrier; m_out is in LDS.
template <bool COHERENT = false, int BATCH = 8>
__device__ __forceinline__ void reduce_token_partials(const float* __restrict__ part, int G, int T,
                                                      int t, int RP, float* red256,
                                                      float* m_out) {
  const int Q = 256 / RP;
  {
    const int r = threadIdx.x % RP, q = threadIdx.x / RP;
    float s = 0.f;
    if (q < Q) {
      const float* p = part + (size_t)t * RP + r;
      const size_t gstride = (size_t)T * RP;
      for (int g0 = q; g0 < G; g0 += BATCH * Q) {
        float v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int g = g0 + u * Q;
          v[u] = load_partial<COHERENT>(p + (size_t)(g < G ? g : q) * gstride);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (g0 + u * Q < G) s += v[u];
      }
    }
    red256[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x < RP) {
    float s = 0.f;
    for (int q = 0; q < Q; ++q) s += red256[q * RP + threadIdx.x];
    m_out[threadIdx.x] = s;
  }
  __syncthreads();
}

// The same fixed-order sum as reduce_token_partials (bit-identical result), done
// by ONE wavefront: lane l plays threads l, l + 64, l + 128 and l + 192 of the
// 256-thread version, with all of their loads of a batch in flight together.
// LDS accesses of one wavefront complete in order, so no barrier is needed;
// only m_out (in LDS) is written for the rest of the block, which must
// synchronise before reading it.
template <bool COHERENT = false, int BATCH = 16>
__device__ __forceinline__ void reduce_token_partials_wave(const float* __restrict__ part, int G,
                                                           int T, int t, int RP, float* red256,
                                                           float* m_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int Q = 256 / RP;
  const int QR = Q * RP;
  const float* p = part + (size_t)t * RP;
  const size_t gstride = (size_t)T * RP;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < G; g0 += BATCH * Q) {
    float v[4][BATCH];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tid = lane + kWave * i;
      const int tc = tid < QR ? tid : lane;  // lane < 64 <= QR is always valid
      const int r = tc % RP, q = tc / RP;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int g = g0 + q + u * Q;
        v[i][u] = load_partial<COHERENT>(p + r + (size_t)(g < G ? g : q) * gstride);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tid = lane + kWave * i;
      const int q = (tid < QR ? tid : lane) / RP;
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (g0 + q + u * Q < G) s[i] += v[i][u];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tid = lane + kWave * i;
    if (tid < QR) red256[tid] = s[i];
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < RP) {
    float sum = 0.f;
    for (int q = 0; q < Q; ++q) sum += red256[q * RP + lane];
    m_out[lane] = sum;
  }
}

}  // namespace mhc
