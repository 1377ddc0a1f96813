// mhc_fused.hip -- token-tiled fused pre chain for S <= 4 with the slab held
// on chip: x is read from HBM exactly once per token.
//
// Steps (hyper.rs page, module doc: arithmetic contract, lines one to four):
// mixes = fn_w . x[t] over the contiguous S*H slab, the sum of squares, the RMS
// rescale, gates + Sinkhorn, and the collapse y[t,:] = sum_c pre[t,c] x[t,c,:].
//
// One block = 512 threads (8 waves) = a tile of 4 consecutive tokens.  Wave w
// owns the hidden columns [64*w*CPW, 64*(w+1)*CPW) of EVERY stream, so once the
// gates are known each lane collapses its own registers.
//
// Operand traffic.  The contraction runs on v_mfma_f32_4x4x1_16b_f32 (A = 4
// tokens, B = 4 weight rows, 16 independent blocks = 16 k-streams).  MFMA lane
// layouts put different rows in neighbouring lanes, which defeats coalescing,
// so (1) the weight is re-packed once per call into exactly the order the
// kernel consumes it (every fetch is one contiguous KiB per wave; see
// pack_weight_kernel), and (2) x is loaded coalesced (16 lanes per token) and
// moved into the A-operand lanes with ds_bpermute.  Every tile streams the whole
// packed weight from L2 (1.5 MiB at 4 x 4096), which bounds the kernel by the
// CU's L1 fill rate; one weight chunk is prefetched ahead of the MFMAs.
//
// With ZQ the tail also runs the branch-input epilogue (z = RMS-norm(y) * nw,
// its q8 codes and scales) from the y still in registers: one more barrier for
// the per-token sum of squares, and y is never read back.
//
// With POST the kernel first finishes the previous site: it reads that site's
// input state, branch output and gates, computes the post mix in registers,
// writes it out as the new state, and runs this site's pre chain on it, so the
// new state is never read back from memory.
#include <atomic>

#include "mhc_device.h"
#include "mhc_kernels.h"

namespace mhc {

// Weight packing: the operand order the fused kernel consumes.  Entry
// ((w*NCH + ci)*RG + rg)*64 + lane (a float4) holds, for lane = 4b + j,
// fn_w[4rg + j][c*H + 64*(w*CPW + u) + 4b .. +3] with c = ci / CPW, u = ci % CPW
// (zero past the last row or column), so that every weight fetch of the fused
// kernel is one contiguous kilobyte per wavefront.
template <int S, int R, int CPW>
__global__ __launch_bounds__(256) void pack_weight_kernel(const float* __restrict__ fn_w, int H,
                                                          float4* __restrict__ packed) {
  constexpr int RG = (R + 3) / 4;
  constexpr int NCH = S * CPW;
  constexpr int TOTAL = 8 * NCH * RG * 64;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= TOTAL) return;
  const int lane = e & 63;
  const int rg = (e >> 6) % RG;
  const int ci = (e / (64 * RG)) % NCH;
  const int w = e / (64 * RG * NCH);
  const int b = lane >> 2, j = lane & 3;
  const int c = ci / CPW, u = ci % CPW;
  const int row = 4 * rg + j;
  const int h = 64 * (w * CPW + u) + 4 * b;
  packed[e] = (row < R && h < H)
                  ? *reinterpret_cast<const float4*>(fn_w + (size_t)row * S * H + c * H + h)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int S, int CPW, int WD, bool ZQ, bool POST, bool HEAD = false>
__global__ __launch_bounds__(512) void fused_pre_kernel(
    const float* __restrict__ x, const float4* __restrict__ wpack,
    const float* __restrict__ scale, const float* __restrict__ base, int T, int H, int iters,
    float eps, float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb,
    float* __restrict__ y, Zq8Out zq, PostIn pin) {
  static_assert(!HEAD || (!ZQ && !POST), "the head has no epilogue and no post half");
  constexpr int R = HEAD ? S : (2 + S) * S;
  constexpr int RG = (R + 3) / 4;  // weight-row groups of 4
  constexpr int NW = 8;
  constexpr int NOUT = 4 * (R + 1);
  constexpr int NCH = S * CPW;     // chunks per wave: chunk ci = stream ci / CPW, column block ci % CPW
  __shared__ float red[NW][NOUT];  // per-wave totals, [token][row], row R = sum of squares
  __shared__ float mr[4][R + 1];
  __shared__ float pre_lds[4 * 8];
  __shared__ float params[3 + R];
  __shared__ float zred[ZQ ? NW : 1][4];
  __shared__ float gpc[POST ? 4 : 1][POST ? S * (S + 1) : 1];  // post gates, then comb [j][k]

  if constexpr (HEAD) {
    // the head's single scale at 0 and its S biases from 3 on (pre_gate's layout)
    if (threadIdx.x == 0)
      params[0] = scale[0];
    else if (threadIdx.x >= 3 && threadIdx.x < 3 + S)
      params[threadIdx.x] = base[threadIdx.x - 3];
  } else {
    stage_site_params(scale, base, R, params);
  }
  if constexpr (POST) {
    // the previous site's gates of the tile's tokens (a barrier follows below)
    constexpr int G1 = S * (S + 1);
    for (int i = threadIdx.x; i < 4 * G1; i += 512) {
      const int u = i / G1, e = i - u * G1;
      const int tk = min((int)blockIdx.x * 4 + u, T - 1);
      gpc[u][e] = e < S ? pin.post[(size_t)tk * S + e] : pin.comb[(size_t)tk * S * S + (e - S)];
    }
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 4;
  const int n = S * H;
  // Memory layout of a lane: token tq = lane / 16, column offset 4 * (lane % 16),
  // so 16 neighbouring lanes read 256 contiguous bytes of one token.
  const int tq = lane >> 4, bq = lane & 15;
  const int tok = t0 + tq;
  const bool tok_ok = tok < T;
  const float* xt = x + (size_t)(tok_ok ? tok : 0) * n;
  // MFMA layout of a lane: block b = lane / 4, token (A row) q = lane % 4.  Its
  // operand lives in lane 16*q + b of the memory layout.
  const int src_lane4 = 4 * (16 * (lane & 3) + (lane >> 2));

  float4 xr[NCH];
  float4 wb[WD + 1][RG];
  // x is read exactly once: non-temporal, so it does not displace the weight.
  // The loads are branch-free, which keeps them in issue order so that chunk ci
  // waits only for itself: a lane past the hidden size reads column 0 instead
  // (its MFMA terms vanish against the zero-padded packed weight, its square is
  // masked below, and it stores nothing); lanes of tokens past T read token 0
  // and are never written out.
  auto load_x = [&](int ci) {
    const int c = ci / CPW, u = ci % CPW;
    const int h = 64 * (wave * CPW + u) + 4 * bq;
    xr[ci] = nt_load4(xt + c * H + (h < H ? h : 0));
  };
  const float4* wp = wpack + (size_t)wave * NCH * RG * 64 + lane;
  auto load_w = [&](int ci, float4* dst) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) dst[rg] = wp[(ci * RG + rg) * 64];
  };

  floatx4 acc[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) acc[rg] = floatx4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
#pragma unroll
  for (int ci = 0; ci < NCH; ++ci) load_x(ci);
  if constexpr (POST) {
    // The previous site's post mix, in registers: x' = post * f + comb^T x for
    // every column block, kept as this site's input (and written out as the new
    // state after the MFMA loop: a wave's memory operations retire in order, so
    // stores issued here would hold up every weight load behind them).  A lane
    // holds all S streams of its columns.  f comes in batches of 4 to 8
    // column blocks, which bounds its registers.
    constexpr int FB = CPW < 8 ? CPW : (CPW < 16 ? 8 : 4);
    const float* ft = pin.f + (size_t)(tok_ok ? tok : 0) * H;
    __syncthreads();  // gpc staged
    const float* g = &gpc[tq][0];
#pragma unroll
    for (int u0 = 0; u0 < CPW; u0 += FB) {
      float4 fq[FB];
#pragma unroll
      for (int i = 0; i < FB; ++i) {
        const int h = 64 * (wave * CPW + u0 + i) + 4 * bq;
        fq[i] = nt_load4(ft + (h < H ? h : 0));
      }
#pragma unroll
      for (int i = 0; i < FB; ++i) {
        const int u = u0 + i;
        float4 xs[S];
#pragma unroll
        for (int c = 0; c < S; ++c) xs[c] = xr[c * CPW + u];
#pragma unroll
        for (int k = 0; k < S; ++k)
          xr[k * CPW + u] = post_mix4<S>(g[k], g + S + k, S, xs, fq[i], S);
      }
    }
  }
#pragma unroll
  for (int ci = 0; ci < WD && ci < NCH; ++ci) load_w(ci, wb[ci]);
#pragma unroll
  for (int ci = 0; ci < NCH; ++ci) {
    if (ci + WD < NCH) load_w(ci + WD, wb[(ci + WD) % (WD + 1)]);
    // keep the prefetch above the compute of this chunk
    __builtin_amdgcn_sched_barrier(0);
    const float4 v = xr[ci];
    if (64 * (wave * CPW + ci % CPW) + 4 * bq < H) {
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
    // re-lay the chunk into the MFMA A-operand lanes (an opaque copy of the
    // address keeps each permute inside its own chunk)
    int sl = src_lane4;
    asm volatile("" : "+v"(sl));
    const float ax = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.x)));
    const float ay = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.y)));
    const float az = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.z)));
    const float aw = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.w)));
    const float4* w = wb[ci % (WD + 1)];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(ax, w[rg].x, acc[rg], 0, 0, 0);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(ay, w[rg].y, acc[rg], 0, 0, 0);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(az, w[rg].z, acc[rg], 0, 0, 0);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(aw, w[rg].w, acc[rg], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (POST) {
    // the new state, written while the partial sums are being reduced
    if (tok_ok) {
#pragma unroll
      for (int ci = 0; ci < NCH; ++ci) {
        const int c = ci / CPW, u = ci % CPW;
        const int h = 64 * (wave * CPW + u) + 4 * bq;
        if (h < H) nt_store4(pin.x_out + ((size_t)tok * S + c) * H + h, xr[ci]);
      }
    }
  }

  // ---- fixed-order reduction: the 16 MFMA blocks in registers (DPP / permlane),
  // then the 8 waves in wave order through LDS.
  // acc[rg][v] at lane (b, j) = partial of (token v, row 4rg + j) over block b;
  // ss at lane (tq, bq) = partial sum of squares of token tq.
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float t = sum_mfma4_blocks(acc[rg][v]);
      if (lane < 4 && 4 * rg + lane < R) red[wave][v * (R + 1) + 4 * rg + lane] = t;
    }
  {
    const float t = sum_row16(ss);
    if ((lane & 15) == 0) red[wave][tq * (R + 1) + R] = t;
  }
  __syncthreads();
  if (threadIdx.x < NOUT) {
    const int o = threadIdx.x;
    float sum = red[0][o];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww][o];
    mr[o / (R + 1)][o % (R + 1)] = sum;
  }
  __syncthreads();

  // ---- gates + Sinkhorn of the four tokens in wave 0 (the head: its sigmoid
  // gates alone, lane 4u + c for token u, stream c)
  if (HEAD) {
    if (wave == 0 && lane < 16) {
      const int u = lane >> 2, c = lane & 3;
      if (c < S && t0 + u < T) {
        const float g = pre_gate(&mr[u][0], c, R, n, eps, params);
        pre[(size_t)(t0 + u) * S + c] = g;
        pre_lds[u * 8 + c] = g;
      }
    }
  } else if (wave == 0) {
    const int ntok = min(4, T - t0);
    gates_wave<4>(&mr[0][0], R + 1, ntok, S, n, params, iters, eps, true,
                  pre + (size_t)t0 * S, post + (size_t)t0 * S, comb + (size_t)t0 * S * S,
                  pre_lds);
  }
  __syncthreads();

  // ---- collapse from registers (memory layout: token tq, columns 4*bq..)
  if constexpr (ZQ) {
    // Collapse and branch-input epilogue.  Every lane computes (lanes of tokens
    // past T on token 0's data, never stored), because the block maximum of a
    // 32-entry block is a butterfly over the 8 lanes holding it (bq bits 0-2;
    // H % 32 == 0, so a block is wholly inside or outside the hidden size).
    float pc[S];
#pragma unroll
    for (int c = 0; c < S; ++c) pc[c] = pre_lds[tq * 8 + c];
    float4 yv[CPW];
    float ys = 0.f;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int h = 64 * (wave * CPW + u) + 4 * bq;
      float4 xs[S];
#pragma unroll
      for (int c = 0; c < S; ++c) xs[c] = xr[c * CPW + u];
      yv[u] = collapse4<S>(pc, xs, S);
      if (h < H) {
        ys = sq4(yv[u], ys);
        if (tok_ok) nt_store4(y + (size_t)tok * H + h, yv[u]);
      }
    }
    // sum of squares of the token's y: its 16 lanes, then the 8 waves in order
    ys = sum_row16(ys);
    if ((lane & 15) == 0) zred[wave][tq] = ys;
    __syncthreads();
    float ssy = zred[0][tq];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) ssy += zred[ww][tq];
    const float r = zq8_rinv(ssy, H, zq.norm_eps);
    const size_t row = (size_t)(tok_ok ? tok : 0) * H;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int h = 64 * (wave * CPW + u) + 4 * bq;
      const bool hin = h < H;
      const float4 w = *reinterpret_cast<const float4*>(zq.nw + (hin ? h : 0));
      const float4 o = zq8_norm(yv[u], r, w);
      float db;
      const char4 cq = zq8_codes(o, &db);
      if (tok_ok && hin) {
        nt_store4(zq.z + row + h, o);
        *reinterpret_cast<char4*>(zq.q + row + h) = cq;
        if ((bq & 7) == 0) zq.d[(row + h) >> 5] = db;
      }
    }
  } else if (tok_ok) {
    float pc[S];
#pragma unroll
    for (int c = 0; c < S; ++c) pc[c] = pre_lds[tq * 8 + c];
    float* yt = y + (size_t)tok * H;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int h = 64 * (wave * CPW + u) + 4 * bq;
      if (h < H) {
        float4 xs[S];
#pragma unroll
        for (int c = 0; c < S; ++c) xs[c] = xr[c * CPW + u];
        nt_store4(yt + h, collapse4<S>(pc, xs, S));
      }
    }
  }
}

// ---------------------------------------------------------------- persistent tiles
// The same token-tiled pre chain (fused_pre_kernel without the epilogue, the
// post half or the head) on a persistent grid, for batches of two tiles or
// more per compute unit: block b takes tiles b, b + G, b + 2G, ..., and after
// a tile's last MFMA it requests tokens 2 and 3 of its next tile into LDS, so
// that half of the next slab streams in while this tile reduces its partial
// sums, runs the gates and the Sinkhorn and collapses.  On the next tile
// those lanes take their slab from LDS, and their global loads are buffer
// loads out of range, which fetch nothing; tokens 0 and 1 come from HBM as
// in the fused kernel.  Every value a tile computes with is the one the fused
// kernel loads, and every operation the same, so the outputs are
// bit-identical to it.
//
// The request cannot start earlier.  A wave's memory operations complete in
// issue order, and the compiler turns the first wait that follows a request
// into LDS into a wait for every outstanding load (vmcnt(0)), so a request
// issued inside the weight stream would stall it until the request lands.
//
// LDS: wave w's request for chunks 2p and 2p + 1 is one 1 KiB record p (lane
// 32 (ci & 1) + 16 (token - 2) + bq), NCH / 2 records per wave, 128 KiB per
// block at NCH = 32.

// A block barrier for LDS hand-offs alone: the wave's LDS operations complete
// (lgkmcnt(0)), then s_barrier.  __syncthreads() would also wait for the
// next tile's LDS requests (its fence counts them in vmcnt), which have to
// stay in flight through the tile's epilogue.  The empty asm statements keep
// the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int S, int CPW>
__global__ __launch_bounds__(512) void fused_pf_kernel(
    const float* __restrict__ x, const float4* __restrict__ wpack,
    const float* __restrict__ scale, const float* __restrict__ base, int T, int H, int iters,
    float eps, float* __restrict__ pre, float* __restrict__ post, float* __restrict__ comb,
    float* __restrict__ y) {
  constexpr int R = (2 + S) * S;
  constexpr int RG = (R + 3) / 4;
  constexpr int NW = 8;
  constexpr int NOUT = 4 * (R + 1);
  constexpr int NCH = S * CPW;
  constexpr int WD = 1;
  static_assert(NCH % 2 == 0 && NCH <= 32, "two chunks per request record, 16 KiB per wave");
  __shared__ float4 nxt[NW][NCH * 32];
  __shared__ float red[NW][NOUT];
  __shared__ float mr[4][R + 1];
  __shared__ float pre_lds[4 * 8];
  __shared__ float params[3 + R];

  stage_site_params(scale, base, R, params);
  const int n = S * H;
  const int ntiles = (T + 3) / 4;

  float4 xr[NCH];
  float4 wb[WD + 1][RG];
  // A tile's slab (buffer loads straight into xr: lanes whose slab is in LDS,
  // and tokens past T, are out of range and fetch nothing) and its first
  // weight chunk.  Lane values come from an opaque copy of the thread index,
  // as everywhere in the tile loop: they are the same in every tile, and kept
  // across it they would hold registers the slab needs.
  auto request_tile = [&](int tile, bool in_lds) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int tq = lane >> 4, bq = lane & 15;
    const int hb = 64 * wave * CPW + 4 * bq, tb = tq * n;
    const int wo = wave * NCH * RG * 64 + lane;
    const int t0 = tile * 4;
    const bool skip = in_lds && tq >= 2;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(x + (size_t)t0 * n), (short)0, min(4, T - t0) * n * 4, 0x00020000);
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
      const int c = ci / CPW, u = ci % CPW;
      const int h = hb + 64 * u;
      const int off = skip ? 0x7FFFFFF0 : 4 * (tb + c * H + (h < H ? h : 0));
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2);
      xr[ci] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                           __uint_as_float(v[3]));
    }
#pragma unroll
    for (int ci = 0; ci < WD && ci < NCH; ++ci)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) wb[ci][rg] = wpack[wo + (ci * RG + rg) * 64];
  };

  bool have = false;  // tokens 2 and 3 of this tile are in LDS (the same in every lane)
  if (blockIdx.x < ntiles) request_tile(blockIdx.x, false);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int tq = lane >> 4, bq = lane & 15;
    const int src_lane4 = 4 * (16 * (lane & 3) + (lane >> 2));
    const int wo = wave * NCH * RG * 64 + lane;  // this lane's first packed-weight entry
    float4* mine = &nxt[wave][0];
    // this lane's record entry for chunk ci (lanes of tokens 0 and 1 read an
    // entry of token 2, which they discard)
    const int rec_lane = 16 * ((tq - 2) & 1) + bq;
    const int hb = 64 * wave * CPW + 4 * bq;
    const int t0 = tile * 4;
    const int tok = t0 + tq;
    const bool tok_ok = tok < T;
    const int next = tile + gridDim.x;
    const bool want = next < ntiles;  // the same in every lane
    const bool use_lds = have && tq >= 2;

    // The slab and the first weight chunk, requested at the end of the
    // previous tile (or above), and the request into LDS issued before them
    // have landed before any record is read.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- weight stream and MFMAs, as in fused_pre_kernel; the record entries
    // replace the slab values of lanes whose slab is in LDS as each chunk is
    // consumed
    floatx4 acc[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[rg] = floatx4{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    auto load_w = [&](int ci, float4* dst) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) dst[rg] = wpack[wo + (ci * RG + rg) * 64];
    };
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
      if (ci + WD < NCH) load_w(ci + WD, wb[(ci + WD) % (WD + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      const float4 lv = mine[(ci >> 1) * 64 + 32 * (ci & 1) + rec_lane];
      const float4 v = use_lds ? lv : xr[ci];
      xr[ci] = v;
      if (64 * (wave * CPW + ci % CPW) + 4 * bq < H) {
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
      }
      int sl = src_lane4;
      asm volatile("" : "+v"(sl));
      const float ax = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.x)));
      const float ay = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.y)));
      const float az = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.z)));
      const float aw = __int_as_float(__builtin_amdgcn_ds_bpermute(sl, __float_as_int(v.w)));
      const float4* w = wb[ci % (WD + 1)];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(ax, w[rg].x, acc[rg], 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(ay, w[rg].y, acc[rg], 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(az, w[rg].z, acc[rg], 0, 0, 0);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        acc[rg] = __builtin_amdgcn_mfma_f32_4x4x1f32(aw, w[rg].w, acc[rg], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      // Tokens 2 and 3 of the next tile, behind the tile's last weight load,
      // its last read of the records and its last MFMA.  Issued on every tile,
      // so that no wait depends on a branch; past the last tile every lane
      // re-reads one small region of token 0, which stays in cache.
      const int pc = (lane >> 5) & 1;
      const int ptok = min(next * 4 + 2 + ((lane >> 4) & 1), T - 1);
      const float* pt = want ? x + (size_t)ptok * n : x;
      const int on = want ? 1 : 0;
#pragma unroll
      for (int p = 0; p < NCH / 2; ++p) {
        const int cj = 2 * p + pc;
        const int c = cj / CPW, u = cj % CPW;
        const int h = hb + 64 * u;
        __builtin_amdgcn_global_load_lds(pt + on * (c * H + (h < H ? h : 0)) + (1 - on) * 4 * bq,
                                         &mine[p * 64], 16, 0, 2);
      }
    }

    // ---- fixed-order reduction (as in fused_pre_kernel)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float t = sum_mfma4_blocks(acc[rg][v]);
        if (lane < 4 && 4 * rg + lane < R) red[wave][v * (R + 1) + 4 * rg + lane] = t;
      }
    {
      const float t = sum_row16(ss);
      if ((lane & 15) == 0) red[wave][tq * (R + 1) + R] = t;
    }
    lds_barrier();
    if (threadIdx.x < NOUT) {
      const int o = threadIdx.x;
      float sum = red[0][o];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) sum += red[ww][o];
      mr[o / (R + 1)][o % (R + 1)] = sum;
    }
    lds_barrier();

    // ---- collapse from registers, each lane taking its token's pre gates
    // from the sums with the pre-gate routine gates_wave uses (so the two
    // agree to the bit); the Sinkhorn is not on this path
    if (tok_ok) {
      float pc[S];
#pragma unroll
      for (int c = 0; c < S; ++c) pc[c] = pre_gate(&mr[tq][0], c, R, n, eps, params);
      float* yt = y + (size_t)tok * H;
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const int h = 64 * (wave * CPW + u) + 4 * bq;
        if (h < H) {
          float4 xs[S];
#pragma unroll
          for (int c = 0; c < S; ++c) xs[c] = xr[c * CPW + u];
          nt_store4(yt + h, collapse4<S>(pc, xs, S));
        }
      }
    }
    // ---- the next tile's slab (its tokens 2 and 3 are on their way into
    // LDS) streams in while wave 0 runs the gates and the Sinkhorn
    if (want) request_tile(next, true);
    if (wave == 0) {
      const int ntok = min(4, T - t0);
      gates_wave<4, true, true>(&mr[0][0], R + 1, ntok, S, n, params, iters, eps, true,
                                pre + (size_t)t0 * S, post + (size_t)t0 * S,
                                comb + (size_t)t0 * S * S, pre_lds);
    }
    // the next tile's reduction reuses red and mr
    lds_barrier();
    have = want;
  }
}

// Chunks per wave for a hidden size: ceil(H / 64 / 8), rounded up to a supported value.
static int fused_cpw(int H) {
  const int need = (H + 64 * 8 - 1) / (64 * 8);
  int cpw = 1;
  while (cpw < need) cpw *= 2;
  return cpw;
}

bool fused_supported(int S, int H) {
  if (S < 1 || S > 4) return false;
  const int cpw = fused_cpw(H);
  return cpw <= 16 && S * cpw <= 32;
}

static size_t pack_bytes_rows(int S, int R, int H) {
  return (size_t)8 * S * fused_cpw(H) * ((R + 3) / 4) * 64 * sizeof(float4);
}

size_t fused_pack_bytes(int S, int H) { return pack_bytes_rows(S, (2 + S) * S, H); }

size_t fused_head_pack_bytes(int S, int H) { return pack_bytes_rows(S, S, H); }

hipError_t launch_pack_weight(const float* fn_w, int S, int H, float* wpack, hipStream_t st) {
  if (!fused_supported(S, H)) return hipErrorInvalidValue;
  const int cpw = fused_cpw(H);
  const int total = (int)(fused_pack_bytes(S, H) / sizeof(float4));
  float4* pk = reinterpret_cast<float4*>(wpack);
#define MHC_PK(SS, CC)                                                                        \
  if (S == SS && cpw == CC) {                                                                 \
    hipLaunchKernelGGL((pack_weight_kernel<SS, (2 + SS) * SS, CC>), dim3((total + 255) / 256), \
                       dim3(256), 0, st, fn_w, H, pk);                                        \
    return hipGetLastError();                                                                 \
  }
  MHC_PK(1, 1) MHC_PK(1, 2) MHC_PK(1, 4) MHC_PK(1, 8) MHC_PK(1, 16)
  MHC_PK(2, 1) MHC_PK(2, 2) MHC_PK(2, 4) MHC_PK(2, 8) MHC_PK(2, 16)
  MHC_PK(3, 1) MHC_PK(3, 2) MHC_PK(3, 4) MHC_PK(3, 8)
  MHC_PK(4, 1) MHC_PK(4, 2) MHC_PK(4, 4) MHC_PK(4, 8)
#undef MHC_PK
  return hipErrorInvalidValue;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

hipError_t launch_fused_pre(const float* x, const float* fn_w, const float* scale,
                            const float* base, int T, int S, int H, int iters, float eps,
                            float* pre, float* post, float* comb, float* y, float* wpack,
                            const Zq8Out* zq, const PostIn* pin, hipStream_t st,
                            bool prepacked) {
  if (!fused_supported(S, H) || (zq && H % 32 != 0)) return hipErrorInvalidValue;
  const Zq8Out zv = zq ? *zq : Zq8Out{nullptr, 0.f, nullptr, nullptr, nullptr};
  const PostIn pv = pin ? *pin : PostIn{nullptr, nullptr, nullptr, nullptr};
  const int cpw = fused_cpw(H);
  const int total = (int)(fused_pack_bytes(S, H) / sizeof(float4));
  float4* pk = reinterpret_cast<float4*>(wpack);
  dim3 grid((T + 3) / 4);
#define MHC_FK(SS, CC, Z, P)                                                                  \
  hipLaunchKernelGGL((fused_pre_kernel<SS, CC, 1, Z, P>), grid, dim3(512), 0, st, x, pk, scale, \
                     base, T, H, iters, eps, pre, post, comb, y, zv, pv)
#define MHC_FU(SS, CC)                                                                        \
  if (S == SS && cpw == CC) {                                                                 \
    if (!prepacked)                                                                           \
      hipLaunchKernelGGL((pack_weight_kernel<SS, (2 + SS) * SS, CC>),                         \
                         dim3((total + 255) / 256), dim3(256), 0, st, fn_w, H, pk);           \
    if constexpr ((SS * CC) % 2 == 0 && SS * CC <= 32) {                                      \
      const int cus = device_cus();                                                           \
      if (!pin && !zq && cus > 0 && (T + 3) / 4 >= 2 * cus) {                                 \
        hipLaunchKernelGGL((fused_pf_kernel<SS, CC>), dim3(cus), dim3(512), 0, st, x, pk,     \
                           scale, base, T, H, iters, eps, pre, post, comb, y);                \
        return hipGetLastError();                                                             \
      }                                                                                       \
    }                                                                                         \
    if (pin) {                                                                                \
      if (zq)                                                                                 \
        MHC_FK(SS, CC, true, true);                                                           \
      else                                                                                    \
        MHC_FK(SS, CC, false, true);                                                          \
    } else {                                                                                  \
      if (zq)                                                                                 \
        MHC_FK(SS, CC, true, false);                                                          \
      else                                                                                    \
        MHC_FK(SS, CC, false, false);                                                         \
    }                                                                                         \
    return hipGetLastError();                                                                 \
  }
  MHC_FU(1, 1) MHC_FU(1, 2) MHC_FU(1, 4) MHC_FU(1, 8) MHC_FU(1, 16)
  MHC_FU(2, 1) MHC_FU(2, 2) MHC_FU(2, 4) MHC_FU(2, 8) MHC_FU(2, 16)
  MHC_FU(3, 1) MHC_FU(3, 2) MHC_FU(3, 4) MHC_FU(3, 8)
  MHC_FU(4, 1) MHC_FU(4, 2) MHC_FU(4, 4) MHC_FU(4, 8)
#undef MHC_FU
#undef MHC_FK
  return hipErrorInvalidValue;
}

hipError_t launch_fused_head(const float* x, const float* fn_h, const float* scale_h,
                             const float* base_h, int T, int S, int H, float eps, float* gates,
                             float* y, float* wpack, hipStream_t st) {
  if (!fused_supported(S, H)) return hipErrorInvalidValue;
  const int cpw = fused_cpw(H);
  const int total = (int)(fused_head_pack_bytes(S, H) / sizeof(float4));
  float4* pk = reinterpret_cast<float4*>(wpack);
  const Zq8Out zv{nullptr, 0.f, nullptr, nullptr, nullptr};
  const PostIn pv{nullptr, nullptr, nullptr, nullptr};
  dim3 grid((T + 3) / 4);
#define MHC_FH(SS, CC)                                                                        \
  if (S == SS && cpw == CC) {                                                                 \
    hipLaunchKernelGGL((pack_weight_kernel<SS, SS, CC>), dim3((total + 255) / 256), dim3(256), \
                       0, st, fn_h, H, pk);                                                   \
    hipLaunchKernelGGL((fused_pre_kernel<SS, CC, 1, false, false, true>), grid, dim3(512), 0,  \
                       st, x, pk, scale_h, base_h, T, H, 1, eps, gates, nullptr, nullptr, y,  \
                       zv, pv);                                                               \
    return hipGetLastError();                                                                 \
  }
  MHC_FH(1, 1) MHC_FH(1, 2) MHC_FH(1, 4) MHC_FH(1, 8) MHC_FH(1, 16)
  MHC_FH(2, 1) MHC_FH(2, 2) MHC_FH(2, 4) MHC_FH(2, 8) MHC_FH(2, 16)
  MHC_FH(3, 1) MHC_FH(3, 2) MHC_FH(3, 4) MHC_FH(3, 8)
  MHC_FH(4, 1) MHC_FH(4, 2) MHC_FH(4, 4) MHC_FH(4, 8)
#undef MHC_FH
  return hipErrorInvalidValue;
}

}  // namespace mhc
