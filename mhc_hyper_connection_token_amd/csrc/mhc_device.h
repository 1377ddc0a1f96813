// mhc_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Cross-lane sums on DPP and the gfx950 permlane swaps (plain VALU, no LDS),
// the one-wavefront Sinkhorn, and the gate epilogue.  Gate forms and Sinkhorn
// semantics are the ones stated in include/mhc.h (hyper.rs page, module doc:
// arithmetic contract).
#pragma once
#include <hip/hip_runtime.h>

namespace mhc {

constexpr int kWave = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- lane exchange
// DPP move within rows of 16 lanes; CTRL is the DPP control word
// (quad_perm 0x00-0xFF, row_ror:n 0x120+n, row_half_mirror 0x141).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v + (the same register of the lane 16 apart within each 32-lane half).  Both
// lanes of a pair add the same two values in the same order, so they agree to
// the bit.
__device__ __forceinline__ float swap16_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v + (the same register of the lane 32 apart).
__device__ __forceinline__ float swap32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Butterfly sums: all lanes of a group end with bit-identical totals.
__device__ __forceinline__ float sum_xor1_2(float v) {  // over lane bits 0-1
  v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  return v;
}
__device__ __forceinline__ float sum_xor4_in8(float v) {  // quads of a half-row (bit 2)
  return v + dpp<0x141>(v);  // row_half_mirror: the other quad of the 8-lane half-row
}
__device__ __forceinline__ float sum_xor8_in16(float v) {  // bit 3
  return v + dpp<0x128>(v);  // row_ror:8 == lane ^ 8 within a row of 16
}

// Sum over the 16 blocks of a v_mfma_f32_4x4x1_16b_f32 accumulator register
// (lane 4b + j, b = 0..15): every lane ends with the total of its column j.  The
// association order differs between lanes, so only one lane per column should
// be read; it is the same on every run.
__device__ __forceinline__ float sum_mfma4_blocks(float v) {
  v += dpp<0x124>(v);  // row_ror:4   (the four quads of a 16-lane row)
  v += dpp<0x128>(v);  // row_ror:8
  v = swap16_sum(v);
  return swap32_sum(v);
}
// Sum over each 16-lane row (lane bits 0-3); read one lane per row.
__device__ __forceinline__ float sum_row16(float v) {
  v = sum_xor1_2(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return v;
}

// Sum over the whole wavefront; read one lane (lane 0).
__device__ __forceinline__ float sum_wave(float v) {
  return swap32_sum(swap16_sum(sum_row16(v)));
}

// ---------------------------------------------------------------- Sinkhorn
// Two lane layouts for the S x S block (entries outside S x S hold 0 and stay 0,
// so padded sums equal the true sums):
//   L = 4 (S <= 4): four tokens u per wavefront, u = lane bits 4-5; row j =
//                   lane bits 2-3; column k = lane bits 0-1 for even j and
//                   3 - (bits 0-1) for odd j.  A row is one quad (sums by quad
//                   permutes); the four entries of a column sit at lanes
//                   {k, 7-k, 8+k, 15-k} of the token's 16-lane row, paired by
//                   the half-row mirror and then by rotation by 8, so both
//                   passes are two DPP adds.
//   L = 8 (S <= 8): lane = 8*j + k, one token per wavefront;
//                   row sums over bits 0-2, column sums over bits 3-5.
// Every reduction is a butterfly: all lanes of a row (column) end with the
// same bits.
template <int L>
__device__ __forceinline__ void sinkhorn_lane_entry(int lane, int& u, int& j, int& k) {
  if (L == 4) {
    u = lane >> 4;
    j = (lane >> 2) & 3;
    k = (j & 1) ? 3 - (lane & 3) : (lane & 3);
  } else {
    u = 0;
    j = lane >> 3;
    k = lane & 7;
  }
}
template <int L>
__device__ __forceinline__ float row_sum(float v) {
  v = sum_xor1_2(v);
  if (L == 8) v = sum_xor4_in8(v);
  return v;
}
template <int L>
__device__ __forceinline__ float col_sum(float v) {
  if (L == 4) {
    v += dpp<0x141>(v);  // row_half_mirror: lane k <-> 7-k (rows 0 and 1, 2 and 3)
    return v + dpp<0x128>(v);  // row_ror:8: rows 0+1 <-> 2+3
  }
  v = sum_xor8_in16(v);
  v = swap16_sum(v);
  return swap32_sum(v);
}

// iters rounds of: row pass C /= (row sum + eps), then column pass
// C /= (column sum + eps).  The division is a hardware reciprocal (1 ulp) and a
// multiply; zero entries stay zero.  Every sum runs over L lanes (padding
// included), so each lane adds eps / L (exact: L is a power of two) to the
// value it hands to the sum, in the same fused multiply-add that scales it;
// the sum then carries the eps with no add of its own on the dependent chain.
// The scaled entry itself is a plain rounded product.
template <int L>
__device__ __forceinline__ float sinkhorn_lanes(float c, int iters, float eps) {
  const float el = eps * (1.0f / L);
  float ce = c + el;
  for (int it = 0; it < iters; ++it) {
    const float r = __builtin_amdgcn_rcpf(row_sum<L>(ce));
    ce = fmaf(c, r, el);
    c = __fmul_rn(c, r);
    const float k = __builtin_amdgcn_rcpf(col_sum<L>(ce));
    ce = fmaf(c, k, el);
    c = __fmul_rn(c, k);
  }
  return c;
}

// Streaming (non-temporal) 16-byte load / store for data touched exactly once,
// so that it does not displace reused data (the mixes weight) from L2.
__device__ __forceinline__ float4 nt_load4(const float* p) {
  const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_store4(float* p, float4 v) {
  __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, reinterpret_cast<floatx4*>(p));
}

__device__ __forceinline__ float sigmoid_exact_ends(float z) {
  // 1/(1+exp(-z)) with a hardware reciprocal (1 ulp): z -> -inf gives exactly
  // 0 (rcp(inf) = 0), z -> +inf exactly 1 (rcp(1) = 1), z = 0 exactly 1/2.
  return __builtin_amdgcn_rcpf(1.0f + expf(-z));
}

// 1/sqrt(ss/n + eps) with the hardware reciprocal square root (1 ulp).  The
// fused multiply-add is explicit so that every caller rounds identically.
__device__ __forceinline__ float rms_inverse(float ss, int n, float eps) {
  return __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / (float)n, eps));
}

// The pre gate of stream c of one token: sigmoid(scale_pre * raw_c * rinv + base_c)
// from the token's unscaled dots mr[0..R) and sum of squares mr[R], with the site
// parameters as staged by stage_site_params.  Every path that needs a pre gate
// (the gate epilogue and the collapse) calls this, so they agree to the bit.
__device__ __forceinline__ float pre_gate(const float* mr, int c, int R, int n, float eps,
                                          const float* params) {
  const float rinv = rms_inverse(mr[R], n, eps);
  return sigmoid_exact_ends(fmaf(params[0], mr[c] * rinv, params[3 + c]));
}

// ---------------------------------------------------------------- gate epilogue
// The site parameters (scale[3] then base[R]) staged in LDS at kernel start, so
// that their memory latency is off the path of the gates.  Threads 0 .. R+2 of
// the block each load one value; a block barrier must follow before use.
__device__ __forceinline__ void stage_site_params(const float* __restrict__ scale,
                                                  const float* __restrict__ base, int R,
                                                  float* params) {
  const int i = threadIdx.x;
  if (i < 3)
    params[i] = scale[i];
  else if (i < 3 + R)
    params[i] = base[i - 3];
}

// Gates of up to NT tokens (NT = 4 for L = 4, 1 for L = 8) in ONE wavefront;
// all 64 lanes must call it together.  With PRE = false the pre gates are left
// to the caller (pre_gate), and pre / pre_lds are not touched.  With POST_NT the
// post gates are non-temporal stores: a kernel with requests into LDS in flight
// uses it, because the compiler otherwise merges the post store with the
// pre_lds store into one flat store, which would wait for those requests.
//   mraw + u*ldm : the unscaled dots fn_w[r,:].x[t,:] (r < R) of token slot u,
//                  followed at index R by the token's sum of squares.
//   params       : scale[0..2] then base[0..R-1] (see stage_site_params).
//   ntok         : valid token slots (the rest are padding).
//   pre/post/comb: outputs of slot 0 (slot u at + u*S, + u*S, + u*S*S);
//                  written only when write_out.
//   pre_lds      : pre gates for the collapse, slot u at + u*8.
// Per token: rinv = 1/sqrt(ss/n + eps); m = raw*rinv; z = fma(scale_g, m, base);
// pre = sigmoid(z), post = 2 sigmoid(z), comb = Sinkhorn(exp(z)).
// The two halves, gates_pre_post and gates_comb, may also run on two different
// wavefronts (same arguments); gates_comb needs all 64 lanes of its wave.
template <int L, bool PRE = true, bool POST_NT = false>
__device__ __forceinline__ void gates_pre_post(const float* mraw, int ldm, int ntok, int S,
                                               int n, const float* params, float eps,
                                               bool write_out, float* __restrict__ pre,
                                               float* __restrict__ post, float* pre_lds) {
  // The lane index through an opaque copy: in a kernel that loops over tiles,
  // the per-lane output offsets derived from it would otherwise be hoisted out
  // of the loop and held (or spilled) across it.
  int lane = threadIdx.x & (kWave - 1);
  asm volatile("" : "+v"(lane));
  const int R = (2 + S) * S;
  const float s_post = params[1];
  const float* base = params + 3;
  // lane = 8*u + g (g < 2S) for L = 4; lane = g for L = 8
  const int u = (L == 4) ? (lane >> 3) : 0;
  const int g = (L == 4) ? (lane & 7) : lane;
  if (u < ntok && g < 2 * S && (L == 8 || lane < 32)) {
    const float* mr = mraw + u * ldm;
    if (g < S) {
      if (PRE) {
        const float v = pre_gate(mr, g, R, n, eps, params);
        if (write_out) pre[u * S + g] = v;
        pre_lds[u * 8 + g] = v;
      }
    } else {
      const float rinv = rms_inverse(mr[R], n, eps);
      const float v = 2.0f * sigmoid_exact_ends(fmaf(s_post, mr[g] * rinv, base[g]));
      if (write_out) {
        if (POST_NT)
          __builtin_nontemporal_store(v, post + u * S + g - S);
        else
          post[u * S + g - S] = v;
      }
    }
  }
}

template <int L>
__device__ __forceinline__ void gates_comb(const float* mraw, int ldm, int ntok, int S, int n,
                                           const float* params, int iters, float eps,
                                           bool write_out, float* __restrict__ comb) {
  int lane = threadIdx.x & (kWave - 1);  // opaque, as in gates_pre_post
  asm volatile("" : "+v"(lane));
  const int R = (2 + S) * S;
  const float s_comb = params[2];
  const float* base = params + 3;
  int j, k, u;
  sinkhorn_lane_entry<L>(lane, u, j, k);
  const bool valid = (j < S) && (k < S) && (u < ntok);
  float c = 0.0f;
  if (valid) {
    const float* mr = mraw + u * ldm;
    const float rinv = rms_inverse(mr[R], n, eps);
    const int r = 2 * S + j * S + k;
    c = expf(fmaf(s_comb, mr[r] * rinv, base[r]));
  }
  c = sinkhorn_lanes<L>(c, iters, eps);
  if (valid && write_out) comb[u * S * S + j * S + k] = c;
}

template <int L, bool PRE = true, bool POST_NT = false>
__device__ __forceinline__ void gates_wave(const float* mraw, int ldm, int ntok, int S, int n,
                                           const float* params, int iters, float eps,
                                           bool write_out, float* __restrict__ pre,
                                           float* __restrict__ post, float* __restrict__ comb,
                                           float* pre_lds) {
  gates_pre_post<L, PRE, POST_NT>(mraw, ldm, ntok, S, n, params, eps, write_out, pre, post,
                                  pre_lds);
  gates_comb<L>(mraw, ldm, ntok, S, n, params, iters, eps, write_out, comb);
}

// y = sum_c pre[c] * x_c, streams in ascending order, first term a product.
// Shared by every collapse so that all paths agree bit for bit given pre.
// SMAX is a compile-time bound on S so that xs stays in registers.
template <int SMAX>
__device__ __forceinline__ float4 collapse4(const float* pre, const float4* xs, int S) {
  float4 o = make_float4(pre[0] * xs[0].x, pre[0] * xs[0].y, pre[0] * xs[0].z, pre[0] * xs[0].w);
#pragma unroll
  for (int c = 1; c < SMAX; ++c) {
    if (c < S) {
      o.x = fmaf(pre[c], xs[c].x, o.x);
      o.y = fmaf(pre[c], xs[c].y, o.y);
      o.z = fmaf(pre[c], xs[c].z, o.z);
      o.w = fmaf(pre[c], xs[c].w, o.w);
    }
  }
  return o;
}

// The post mix of one hidden quad of target stream k (hyper.rs page, doc comment
// of `post`): post_k * f + sum_j comb[j][k] * x_j, the first term a product and
// the sources added in ascending order by fused multiply-adds.  comb[j][k] is
// cj[j * cstride].  Shared by the post kernel and the fused post-then-pre
// kernel, so both write the same bits.
template <int SMAX>
__device__ __forceinline__ float4 post_mix4(float pk, const float* cj, int cstride,
                                            const float4* xv, float4 fv, int S) {
  float4 o = make_float4(pk * fv.x, pk * fv.y, pk * fv.z, pk * fv.w);
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    if (j < S) {
      const float c = cj[j * cstride];
      o.x = fmaf(c, xv[j].x, o.x);
      o.y = fmaf(c, xv[j].y, o.y);
      o.z = fmaf(c, xv[j].z, o.z);
      o.w = fmaf(c, xv[j].w, o.w);
    }
  }
  return o;
}

// ---------------------------------------------------------------- branch-input epilogue
// (hc_fused_gate.rs page, the v4z timing block: the norm and the q8 encoding of
// the branch input.)  z = y * r * w per entry, r = 1/sqrt(mean y^2 + norm_eps);
// per block of 32 consecutive entries d = max|z| / 127 and codes round(z * (1/d))
// with ties away from zero (d = 0, codes 0 for an all-zero block).  The division
// and the reciprocal are IEEE fp32 and the rounding is roundf, so codes and scale
// are a pure function of the fp32 z that is written.
__device__ __forceinline__ float zq8_rinv(float ss, int H, float norm_eps) {
  return __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / (float)H, norm_eps));
}
__device__ __forceinline__ float4 zq8_norm(float4 y, float r, float4 w) {
  return make_float4(y.x * r * w.x, y.y * r * w.y, y.z * r * w.z, y.w * r * w.w);
}
__device__ __forceinline__ float sq4(float4 v, float acc) {
  acc = fmaf(v.x, v.x, acc);
  acc = fmaf(v.y, v.y, acc);
  acc = fmaf(v.z, v.z, acc);
  return fmaf(v.w, v.w, acc);
}
// q8 of one quad of z whose 32-entry block is held by the eight neighbouring
// lanes of an aligned 8-lane group (lane bits 0-2), all eight calling together.
// Returns the codes; *db receives the block scale (the same in all 8 lanes).
__device__ __forceinline__ char4 zq8_codes(float4 o, float* db) {
  float a = fmaxf(fmaxf(fabsf(o.x), fabsf(o.y)), fmaxf(fabsf(o.z), fabsf(o.w)));
  a = fmaxf(a, dpp<0xB1>(a));   // quad_perm [1,0,3,2]
  a = fmaxf(a, dpp<0x4E>(a));   // quad_perm [2,3,0,1]
  a = fmaxf(a, dpp<0x141>(a));  // half-row mirror: the other quad
  const float d = a / 127.0f;
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
  *db = d;
  return make_char4((signed char)roundf(o.x * id), (signed char)roundf(o.y * id),
                    (signed char)roundf(o.z * id), (signed char)roundf(o.w * id));
}

}  // namespace mhc
