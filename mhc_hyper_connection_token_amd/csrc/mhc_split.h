// mhc_split.h -- device routines of the split-K pre path, shared by the
// partials and finish kernels so that all of them add the same numbers in the
// same order.
#pragma once
#include <type_traits>

#include "mhc_device.h"

namespace mhc {

// Values each lane of a wave hands to the cross-wave sum, and the number of
// slices that sum is staged in (the caller's `red` holds 4 * block_slice * 64
// floats).
template <int NRT, int NTT>
constexpr int block_vals() { return NRT * NTT * 4 + NTT; }
template <int NRT, int NTT>
constexpr int block_passes() { return block_vals<NRT, NTT>() > 48 ? 2 : 1; }
template <int NRT, int NTT>
constexpr int block_slice() {
  return (block_vals<NRT, NTT>() + block_passes<NRT, NTT>() - 1) / block_passes<NRT, NTT>();
}

// Per-block split-K partials (hyper.rs page, module doc: arithmetic contract,
// first two lines): for tokens [tok0, tok0 + 16*NTT) and the 16-float K chunks
// [c_beg, c_end) of the slab, the partial dots with the R weight rows and the
// partial sum of squares, handed to sink(t*(R+1) + r, value) (r == R: sum of
// squares; t is the token's index in the batch).
// 256 threads = four waves; wave w takes chunks c_beg + w, c_beg + w + 4, ...;
// the four wave partials are added in wave order through `red`
// (4 * block_slice<NRT, NTT>() * 64 floats of LDS).
//
// The contraction runs on v_mfma_f32_16x16x4_f32 (fp32 operands, exact fp32
// products, fp32 accumulation): A = weight rows (16 per tile), B = token slabs
// (16 tokens per tile).  Each lane loads 16 bytes of one weight row and 16
// bytes of one token slab per chunk; the four floats feed four MFMAs whose
// k-index is whatever the lanes hold (A and B agree by construction).
template <int NRT, int NTT, bool BUF, class Sink>
__device__ __forceinline__ void block_partials(const float* __restrict__ x,
                                               const float* __restrict__ fn_w, int T, int n,
                                               int R, int tok0, int c_beg, int c_end,
                                               float* red, Sink sink) {
  constexpr int kVals = block_vals<NRT, NTT>();  // per lane, per wave
  constexpr int kPasses = block_passes<NRT, NTT>();
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

  // BUF: operands through buffer loads, one resource over the R weight rows
  // and one over the block's tokens in range, so lanes of rows past R or
  // tokens past T read zero (out of range), and a chunk past the slab takes an
  // out-of-range offset: no select in the chunk loop.  The launch takes this
  // form when every byte offset fits in 31 bits.  Otherwise row and token
  // pointers are clamped to a valid row / token, and the out-of-range lanes
  // are zeroed by a select when the chunk is consumed.
  const float* wrow[NRT];
  bool wvalid[NRT];
  const float* xrow[NTT];
  bool xvalid[NTT];
  int woff[NRT], xoff[NTT];  // byte offsets of this lane's rows and tokens (BUF)
  __amdgpu_buffer_rsrc_t wrs, xrs;
  if constexpr (BUF) {
    wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(fn_w), (short)0, R * n * 4,
                                            0x00020000);
    const int tv = T - tok0 < 16 * NTT ? T - tok0 : 16 * NTT;  // the block's tokens in range
    xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x + (size_t)tok0 * n), (short)0,
                                            tv * n * 4, 0x00020000);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) woff[rt] = (rt * 16 + sub) * n * 4;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) xoff[tt] = (tt * 16 + sub) * n * 4;
  } else {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int r = rt * 16 + sub;
      wvalid[rt] = r < R;
      wrow[rt] = fn_w + (size_t)(wvalid[rt] ? r : 0) * n;
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int t = tok0 + tt * 16 + sub;
      xvalid[tt] = t < T;
      xrow[tt] = x + (size_t)(xvalid[tt] ? t : 0) * n;
    }
  }

  // Chunk loop over three operand sets: the loads of chunk c + 8 are issued
  // before the MFMAs of chunk c, so two chunks are in flight behind the one
  // being consumed.  Loads are branch-free.
  auto ld = [](__amdgpu_buffer_rsrc_t rs, int off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                       __uint_as_float(v[3]));
  };
  auto load_chunk = [&](int c, float4* a, float4* b) {
    const int k = c * 16 + kq;
    if constexpr (BUF) {
      const bool kin = k < n;  // n % 4 == 0: a float4 is fully in or fully out
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) a[rt] = ld(wrs, kin ? woff[rt] + 4 * k : 0x7FFFFFF0);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) b[tt] = ld(xrs, kin ? xoff[tt] + 4 * k : 0x7FFFFFF0);
    } else {
      const int kc = k < n ? k : 0;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) a[rt] = *reinterpret_cast<const float4*>(wrow[rt] + kc);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) b[tt] = *reinterpret_cast<const float4*>(xrow[tt] + kc);
    }
  };
  auto sel = [](bool ok, float4 v) {
    return make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
  };
  // The MFMAs of one chunk, on operands a0 / b0 (zero outside the valid rows,
  // tokens and K).
  auto consume = [&](int c, const float4* a0, const float4* b0) {
    float4 a[NRT], b[NTT];
    if constexpr (BUF) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) a[rt] = a0[rt];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) b[tt] = b0[tt];
    } else {
      const bool kin = c * 16 + kq < n;  // n % 4 == 0: a float4 is fully in or fully out
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) a[rt] = sel(kin && wvalid[rt], a0[rt]);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) b[tt] = sel(kin && xvalid[tt], b0[tt]);
    }
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
  };
  // three operand sets in a ring: chunk c + 8 is requested while chunk c is
  // consumed (the ring is unrolled so every set stays in named registers; a
  // fourth set measured slower in the buffer form)
  float4 a0[NRT], b0[NTT], a1[NRT], b1[NTT], a2[NRT], b2[NTT];
  int c = c_beg + wave;
  if (c < c_end) load_chunk(c, a0, b0);
  if (c + 4 < c_end) load_chunk(c + 4, a1, b1);
  while (c < c_end) {
    if (c + 8 < c_end) load_chunk(c + 8, a2, b2);
    consume(c, a0, b0);
    c += 4;
    if (c >= c_end) break;
    if (c + 8 < c_end) load_chunk(c + 8, a0, b0);
    consume(c, a1, b1);
    c += 4;
    if (c >= c_end) break;
    if (c + 8 < c_end) load_chunk(c + 8, a1, b1);
    consume(c, a2, b2);
    c += 4;
  }

  // Sum of squares: lanes l, l^16, l^32, l^48 hold the same token's partials.
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) ss[tt] = swap32_sum(swap16_sum(ss[tt]));

  // Stage the wave's partials, then add the four waves in fixed order, in
  // kPasses slices of the values (bounds the LDS; the order of every sum is the
  // same for any slicing).
  constexpr int kSlice = (kVals + kPasses - 1) / kPasses;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int v0 = pass * kSlice;
    {
      int v = 0;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e, ++v)
            if (v >= v0 && v < v0 + kSlice)
              red[(wave * kSlice + v - v0) * kWave + lane] = acc[rt][tt][e];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt, ++v)
        if (v >= v0 && v < v0 + kSlice) red[(wave * kSlice + v - v0) * kWave + lane] = ss[tt];
    }
    __syncthreads();
    const int nv = kVals - v0 < kSlice ? kVals - v0 : kSlice;
    for (int idx = threadIdx.x; idx < nv * kWave; idx += 256) {
      const int vs = idx / kWave, l = idx % kWave;
      const int v = v0 + vs;
      const float s = ((red[(0 * kSlice + vs) * kWave + l] + red[(1 * kSlice + vs) * kWave + l]) +
                       red[(2 * kSlice + vs) * kWave + l]) +
                      red[(3 * kSlice + vs) * kWave + l];
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
    if (pass + 1 < kPasses) __syncthreads();
  }
}

// ---------------------------------------------------------------- 32-lane tree sums
// The value of the lane whose index (within its 32-lane half) differs in bit B.
template <int B>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(B >= 0 && B <= 3, "bit 4 goes through permlane16_swap");
  if constexpr (B == 0) return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  if constexpr (B == 1) return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (B == 2)                       // ds_swizzle, bit mode: xor mask 4
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
  return dpp<0x128>(v);  // row_ror:8 == lane ^ 8 within a row of 16
}

// One level of tree32: the pairs of lanes that differ in bit B add their values.
// With NV >= 2 values left the level is transposed: each lane hands half of its
// values to the partner, the lane with bit B clear keeping the lower half of the
// index range and its partner the upper half, so every add does useful work.
template <int B, int NV>
__device__ __forceinline__ void tree32_level(float* v, int lane) {
  if constexpr (NV >= 2) {
    constexpr int H = NV / 2;
    if constexpr (B == 4) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        // swaps row 1 of v[j] with row 0 of v[j + H]: both rows then hold
        // (row 0 value) and (row 1 value) of their own index
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j + H]),
                                                  false, false);
        v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    } else {
      const bool hi = (lane >> B) & 1;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float send = hi ? v[j] : v[j + H];
        const float keep = hi ? v[j + H] : v[j];
        v[j] = keep + lane_xor<B>(send);
      }
    }
  } else {
    if constexpr (B == 4)
      v[0] = swap16_sum(v[0]);
    else
      v[0] = v[0] + lane_xor<B>(v[0]);
  }
}

// Sums over the 32 lanes of each half-wave of V (a power of two) values per
// lane.  Every sum is the balanced binary tree over lanes 0..31 in lane order
// (pairs differing in bit 0 first, then bit 1, ..., bit 4), exactly the tree of
// a plain five-step butterfly on one value, so the bits do not depend on V or on
// where the value sits.  On return the lane holds max(V/32, 1) sums in v[0..):
// sum j of lane l is original index tree32_index<V>(l, j); with V < 32 the lanes
// that differ only in bits log2(V) and up hold the same sums.
template <int V>
__device__ __forceinline__ void tree32(float (&v)[V], int lane) {
  tree32_level<0, V>(v, lane);
  tree32_level<1, (V >= 2 ? V / 2 : 1)>(v, lane);
  tree32_level<2, (V >= 4 ? V / 4 : 1)>(v, lane);
  tree32_level<3, (V >= 8 ? V / 8 : 1)>(v, lane);
  tree32_level<4, (V >= 16 ? V / 16 : 1)>(v, lane);
}
template <int V>
__device__ __forceinline__ constexpr int tree32_log2() {
  return V <= 1 ? 0 : 1 + tree32_log2<V / 2>();
}
template <int V>
__device__ __forceinline__ int tree32_index(int lane, int j) {
  constexpr int m = tree32_log2<V>();
  constexpr int lv = m < 5 ? m : 5;  // transposed levels
  int o = 0;
#pragma unroll
  for (int b = 0; b < lv; ++b) o |= ((lane >> b) & 1) << (m - 1 - b);
  return o + j;
}

// Split-K partials of a small batch (T <= TMAX tokens) on the vector ALU: for
// every token t and row r < R the dot of fn_w[r, k_beg:k_end] with
// x[t, k_beg:k_end], and at r == R the sum of squares of that slice, handed to
// sink(t*(R+1) + r, value).  256 threads = 8 row slots x 32 lanes: lane l of
// slot s takes the column quads l, l + 32, ... and rows s, s + 8, s + 16, ...
// (RPT of them), so every weight load is a coalesced run of one row.  A
// token's arithmetic (the order of its products and the 32-lane tree of tree32)
// does not depend on T or TMAX: a token's partials are the same in any small
// batch.  k_beg and k_end are multiples of 4.
// One column quad of small_partials: acc[i][t] += fn_w[r_i, quad] . x[t, quad]
// (row R: x . x), four fused multiply-adds in element order.
template <int TMAX, int RPT>
__device__ __forceinline__ void small_quad(float (&acc)[RPT][TMAX], const float4 (&w)[RPT],
                                           const float4 (&xv)[TMAX], int slot, int R) {
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

// The 32-lane tree of every (row, token) lane partial, handed to sink(t*(R+1) + r).
template <int TMAX, int RPT, class Sink>
__device__ __forceinline__ void small_tree_out(float (&acc)[RPT][TMAX], int l, int slot, int T,
                                               int R, Sink sink) {
  const int RP = R + 1;
  constexpr int V = RPT * TMAX;
  float v[V];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int t = 0; t < TMAX; ++t) v[i * TMAX + t] = acc[i][t];
  tree32<V>(v, l);
  constexpr int m = tree32_log2<V>();
  if (m >= 5 || (l >> m) == 0) {
#pragma unroll
    for (int j = 0; j < (V >= 32 ? V / 32 : 1); ++j) {
      const int o = tree32_index<V>(l, j);
      const int i = o / TMAX, t = o % TMAX;
      const int r = slot + 8 * i;
      if (t < T && r <= R) sink((size_t)t * RP + r, v[j]);
    }
  }
}

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
    small_quad<TMAX, RPT>(acc, w, xv, slot, R);
  }
  small_tree_out<TMAX, RPT>(acc, l, slot, T, R, sink);
}

// small_partials over many groups of TMAX tokens of one K-range (at most 32*QL
// column quads): the weight quads are loaded once, and each group's x quads are
// requested while the previous group is being reduced.  Group tg covers tokens
// [tg*TMAX, tg*TMAX + TMAX); this thread takes groups tg0, tg0 + step, ...
// Every token gets exactly the arithmetic of small_partials.  sink(t, r, v)
// receives the partial of token t (global index) and row r <= R.
template <int TMAX, int RPT, int QL, class Sink>
__device__ __forceinline__ void small_partials_groups(const float* __restrict__ x,
                                                      const float* __restrict__ fn_w, int T,
                                                      int n, int R, int k_beg, int k_end,
                                                      int tg0, int step, Sink sink) {
  const int tid = threadIdx.x;
  const int l = tid & 31, slot = tid >> 5;
  const int nq = (k_end - k_beg) >> 2;
  const int groups = (T + TMAX - 1) / TMAX;
  if (tg0 >= groups) return;
  float4 w[QL][RPT];
#pragma unroll
  for (int u = 0; u < QL; ++u) {
    const int q = l + 32 * u;
    const int col = k_beg + 4 * (q < nq ? q : 0);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = slot + 8 * i;
      w[u][i] = *reinterpret_cast<const float4*>(fn_w + (size_t)(r < R ? r : 0) * n + col);
    }
  }
  auto load_x = [&](int tg, float4 (&xv)[QL][TMAX]) {
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int q = l + 32 * u;
      const int col = k_beg + 4 * (q < nq ? q : 0);
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        const int tok = tg * TMAX + t;
        xv[u][t] = *reinterpret_cast<const float4*>(x + (size_t)(tok < T ? tok : 0) * n + col);
      }
    }
  };
  float4 xa[QL][TMAX], xb[QL][TMAX];
  load_x(tg0, xa);
  for (int tg = tg0; tg < groups; tg += step) {
    const bool more = tg + step < groups;  // the same in every thread
    if (more) load_x(tg + step, xb);
    float acc[RPT][TMAX];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int t = 0; t < TMAX; ++t) acc[i][t] = 0.f;
#pragma unroll
    for (int u = 0; u < QL; ++u)
      if (l + 32 * u < nq) small_quad<TMAX, RPT>(acc, w[u], xa[u], slot, R);
    const int t0 = tg * TMAX;
    small_tree_out<TMAX, RPT>(acc, l, slot, min(TMAX, T - t0), R, [&](size_t i, float v) {
      const int RP = R + 1;
      sink(t0 + (int)(i / RP), (int)(i % RP), v);
    });
#pragma unroll
    for (int u = 0; u < QL; ++u)
#pragma unroll
      for (int t = 0; t < TMAX; ++t) xa[u][t] = xb[u][t];
  }
}

// Fixed-order sum of the G partials of token t into m_out[0..R] (256 threads):
// thread (r, q), q < Q = 256 / (R+1), adds g = q, q + Q, q + 2Q, ... in that
// order (BATCH independent loads in flight per batch); then thread r adds the Q
// sums in q order.  The order depends only on G and R, not on T.  Ends with a
// block barrier; m_out is in LDS.  issue() runs in every thread right after
// the first batch of loads is requested: loads it requests complete after the
// partials (a wave's loads complete in order), so the reduction does not wait
// for them.
struct NoIssue {
  __device__ __forceinline__ void operator()() const {}
};
template <int BATCH = 8, class Issue = NoIssue>
__device__ __forceinline__ void reduce_token_partials(const float* __restrict__ part, int G, int T,
                                                      int t, int RP, float* red256,
                                                      float* m_out, Issue issue = Issue()) {
  const int Q = 256 / RP;
  {
    const int r = threadIdx.x % RP, q = threadIdx.x / RP;
    const float* p = part + (size_t)t * RP + r;
    const size_t gstride = (size_t)T * RP;
    float s = 0.f;
    if constexpr (std::is_same_v<Issue, NoIssue>) {
      if (q < Q) {
        for (int g0 = q; g0 < G; g0 += BATCH * Q) {
          float v[BATCH];
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int g = g0 + u * Q;
            v[u] = p[(size_t)(g < G ? g : q) * gstride];
          }
#pragma unroll
          for (int u = 0; u < BATCH; ++u)
            if (g0 + u * Q < G) s += v[u];
        }
      }
    } else {
      // the same sums, with the first batch peeled so that issue() follows it
      float v[BATCH];
      if (q < Q) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
          const int g = q + u * Q;
          v[u] = p[(size_t)(g < G ? g : q) * gstride];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      issue();
      __builtin_amdgcn_sched_barrier(0);
      if (q < Q) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (q + u * Q < G) s += v[u];
        for (int g0 = q + BATCH * Q; g0 < G; g0 += BATCH * Q) {
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int g = g0 + u * Q;
            v[u] = p[(size_t)(g < G ? g : q) * gstride];
          }
#pragma unroll
          for (int u = 0; u < BATCH; ++u)
            if (g0 + u * Q < G) s += v[u];
        }
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

}  // namespace mhc
