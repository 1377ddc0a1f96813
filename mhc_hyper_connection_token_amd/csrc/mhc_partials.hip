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

// Two waves per SIMD at least: the register bound keeps the three operand sets
// of the chunk loop from dropping the kernel to one wave per SIMD.
template <int NRT, int NTT, bool BUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void partials_kernel(const float* __restrict__ x,
                                                       const float* __restrict__ fn_w, int T,
                                                       int n, int R, int chunks_per_range,
                                                       float* __restrict__ part) {
  __shared__ float red[4 * block_slice<NRT, NTT>() * kWave];
  // Workgroups go to the eight XCDs in turn, by linear index.  When the
  // K-range count is a multiple of eight, block L takes K-range
  // g = L % 8 + 8 * ((L / 8) % (G / 8)) and token tile (L / 8) / (G / 8): each
  // XCD then serves G / 8 K-ranges for every token tile, and its L2 fetches
  // only those ranges of the weight.  A block's work does not depend on which
  // block does it, so the results are the same either way.
  int tile = blockIdx.x, g = blockIdx.y;
  if ((gridDim.y & 7) == 0) {
    const int L = blockIdx.y * gridDim.x + blockIdx.x;
    const int gpx = gridDim.y >> 3;
    const int r = L >> 3;
    g = (L & 7) + 8 * (r % gpx);
    tile = r / gpx;
  }
  const int nchunks = (n + 15) >> 4;
  const int c_beg = g * chunks_per_range;
  const int c_end = min(nchunks, c_beg + chunks_per_range);
  float* pg = part + (size_t)g * T * (R + 1);
  block_partials<NRT, NTT, BUF>(x, fn_w, T, n, R, tile * (16 * NTT), c_beg, c_end, red,
                           [=](size_t i, float v) { pg[i] = v; });
}

template <int NRT, int NTT>
static hipError_t launch_partials_t(const float* x, const float* fn_w, int T, int n, int R,
                                    int G, int chunks_per_range, float* part, hipStream_t st) {
  dim3 grid((T + 16 * NTT - 1) / (16 * NTT), G);
  // buffer loads where every byte offset of a block's rows and tokens fits in
  // 31 bits
  const long rows = 16L * (NRT > NTT ? NRT : NTT);
  if (rows * n * 4 + 64 < (1L << 31))
    hipLaunchKernelGGL((partials_kernel<NRT, NTT, true>), grid, dim3(256), 0, st, x, fn_w, T, n,
                       R, chunks_per_range, part);
  else
    hipLaunchKernelGGL((partials_kernel<NRT, NTT, false>), grid, dim3(256), 0, st, x, fn_w, T,
                       n, R, chunks_per_range, part);
  return hipGetLastError();
}

// Vector-ALU partials (S <= 4), every token's sums in the same order whatever
// the group size, so a token's result does not depend on the batch it is in.
// Grid: (G K-ranges, Y); block (g, y) takes the groups of kSmallGroup tokens
// (one token at T = 1) y, y + Y, ..., with the weight quads of its K-range
// held in registers and the next group's x requested while the current one is
// reduced.  QL = column quads per lane (a K-range of at most 128*QL floats).
constexpr int kSmallGroup = 4;
constexpr int kSmallBlocks = 2048;  // target grid size at large T

// The finish kernel that follows needs the site parameters (scale[3], base[R])
// right after its reduction.  Block (0, 0) reads them first thing, so that the
// finish finds them in the memory-side cache rather than in HBM.  The value is
// consumed just before each partial is stored: by then every later load has
// been waited for, so the wait costs nothing (loads complete in order), and no
// store is waited for, as a wait at the end of the kernel would.  pa / pb may
// be null.
struct ParamTouch {
  float v = 0.f;
  __device__ __forceinline__ void issue(const float* __restrict__ pa, int na,
                                        const float* __restrict__ pb, int nb) {
    const int i = threadIdx.x;
    if (pa != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && i < na + nb)
      v = i < na ? pa[i] : pb[i - na];
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void consume() const { asm volatile("" ::"v"(v)); }
};

// TG tokens per group: kSmallGroup, or 1 for a single token (the same sums,
// since every partial is its own lane tree, with a quarter of the work).
template <int RPT, int QL, int TG>
__global__ __launch_bounds__(256) void small_partials_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ fn_w,
                                                             int T, int n, int R,
                                                             int chunks_per_range,
                                                             float* __restrict__ part,
                                                             const float* __restrict__ pa,
                                                             const float* __restrict__ pb) {
  ParamTouch touch;
  touch.issue(pa, 3, pb, R);
  const int g = blockIdx.x;
  const int k_beg = g * chunks_per_range * 16;
  const int k_end = min(n, k_beg + chunks_per_range * 16);
  float* pg = part + (size_t)g * T * (R + 1);
  small_partials_groups<TG, RPT, QL>(
      x, fn_w, T, n, R, k_beg, k_end, blockIdx.y, gridDim.y,
      [=](int t, int r, float v) {
        touch.consume();
        pg[(size_t)t * (R + 1) + r] = v;
      });
}

// The same partials for K-ranges longer than 512 floats: the plain per-group
// loop of small_partials, without holding the weight quads.
template <int RPT>
__global__ __launch_bounds__(256) void small_partials_long_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ fn_w,
                                                                  int T, int n, int R,
                                                                  int chunks_per_range,
                                                                  float* __restrict__ part,
                                                                  const float* __restrict__ pa,
                                                                  const float* __restrict__ pb) {
  ParamTouch touch;
  touch.issue(pa, 3, pb, R);
  const int g = blockIdx.x;
  const int groups = (T + kSmallGroup - 1) / kSmallGroup;
  const int k_beg = g * chunks_per_range * 16;
  const int k_end = min(n, k_beg + chunks_per_range * 16);
  float* pg = part + (size_t)g * T * (R + 1);
  for (int tg = blockIdx.y; tg < groups; tg += gridDim.y) {
    const int t0 = tg * kSmallGroup;
    float* pt = pg + (size_t)t0 * (R + 1);
    small_partials<kSmallGroup, RPT>(x + (size_t)t0 * n, fn_w, min(kSmallGroup, T - t0), n, R,
                                     k_beg, k_end, [=](size_t i, float v) {
                                       touch.consume();
                                       pt[i] = v;
                                     });
  }
}

// Rows per thread for R weight rows and the sum of squares over 8 row slots.
static int rows_per_thread(int R) {
  const int rpt = (R + 1 + 7) / 8;
  return rpt <= 1 ? 1 : (rpt <= 2 ? 2 : (rpt <= 4 ? 4 : 0));
}

int small_rows_per_thread(int S) { return rows_per_thread((2 + S) * S); }

hipError_t launch_small_partials_rows(const float* x, const float* fn_w, int T, int n, int R,
                                      int G, int chunks_per_range, float* part, hipStream_t st,
                                      const float* scale, const float* base) {
  if (T < 1 || G < 1 || R < 1) return hipErrorInvalidValue;
  const int groups = (T + kSmallGroup - 1) / kSmallGroup;
  const int ymax = kSmallBlocks / G > 1 ? kSmallBlocks / G : 1;
  const dim3 grid(G, groups < ymax ? groups : ymax);
  const int ql = (chunks_per_range * 4 + 31) / 32;  // column quads per lane
  const int rpt = rows_per_thread(R);
#define MHC_SP(RP_, QL_)                                                                       \
  if (rpt == RP_ && ql <= QL_) {                                                               \
    if (T == 1)                                                                                \
      hipLaunchKernelGGL((small_partials_kernel<RP_, QL_, 1>), grid, dim3(256), 0, st, x, fn_w, \
                         T, n, R, chunks_per_range, part, scale, base);                        \
    else                                                                                       \
      hipLaunchKernelGGL((small_partials_kernel<RP_, QL_, kSmallGroup>), grid, dim3(256), 0, st, \
                         x, fn_w, T, n, R, chunks_per_range, part, scale, base);               \
    return hipGetLastError();                                                                  \
  }
  MHC_SP(1, 1) MHC_SP(1, 2) MHC_SP(1, 4)
  MHC_SP(2, 1) MHC_SP(2, 2) MHC_SP(2, 4)
  MHC_SP(4, 1) MHC_SP(4, 2) MHC_SP(4, 4)
#undef MHC_SP
#define MHC_SL(RP_)                                                                            \
  if (rpt == RP_) {                                                                            \
    hipLaunchKernelGGL((small_partials_long_kernel<RP_>), grid, dim3(256), 0, st, x, fn_w, T,   \
                       n, R, chunks_per_range, part, scale, base);                             \
    return hipGetLastError();                                                                  \
  }
  MHC_SL(1) MHC_SL(2) MHC_SL(4)
#undef MHC_SL
  return hipErrorInvalidValue;
}

hipError_t launch_small_partials(const float* x, const float* fn_w, int T, int S, int H, int G,
                                 int chunks_per_range, float* part, hipStream_t st,
                                 const float* scale, const float* base) {
  return launch_small_partials_rows(x, fn_w, T, S * H, (2 + S) * S, G, chunks_per_range, part,
                                    st, scale, base);
}

hipError_t launch_partials(const float* x, const float* fn_w, int T, int n, int R, int ntt,
                           int G, int chunks_per_range, float* part, hipStream_t st) {
  const int nrt = (R + 15) / 16;
#define MHC_P(NR, NT)                                                                     \
  if (nrt == NR && ntt == NT)                                                              \
    return launch_partials_t<NR, NT>(x, fn_w, T, n, R, G, chunks_per_range, part, st);
  MHC_P(1, 1) MHC_P(1, 4) MHC_P(2, 1) MHC_P(2, 4) MHC_P(3, 1) MHC_P(3, 4)
  MHC_P(4, 1) MHC_P(4, 2) MHC_P(4, 4) MHC_P(5, 1) MHC_P(5, 2) MHC_P(5, 4)
#undef MHC_P
  return hipErrorInvalidValue;
}

}  // namespace mhc
