// mhc_kernels.h -- host-side launchers of the gfx950 kernels (internal to libmhc).
#pragma once
#include <hip/hip_runtime.h>

namespace mhc {

// Operands of the branch-input epilogue run in a pre kernel's tail: z = RMS-norm
// of y times nw, its int8 codes q and per-32 scales d (token-major, like y).
struct Zq8Out {
  const float* nw;
  float norm_eps;
  float* z;
  signed char* q;
  float* d;
};

// Split-K partial mixes + sums of squares: part[G][T][R+1].
// ntt = token tiles of 16 per block (1, 2 or 4, by the row-tile count and T).
hipError_t launch_partials(const float* x, const float* fn_w, int T, int n, int R, int ntt,
                           int G, int chunks_per_range, float* part, hipStream_t st);

// Vector-ALU split-K partials (S <= 4, any T in groups of 4 tokens, or one
// token), every token's sums in one fixed order; same part layout.  With
// scale / base given, one block also reads the site parameters first thing, so
// that the finish kernel finds them in the memory-side cache.
int small_rows_per_thread(int S);
hipError_t launch_small_partials(const float* x, const float* fn_w, int T, int S, int H, int G,
                                 int chunks_per_range, float* part, hipStream_t st,
                                 const float* scale = nullptr, const float* base = nullptr);
// The same for any R <= 31 rows of a weight [R][n] (the head's R = S).
hipError_t launch_small_partials_rows(const float* x, const float* fn_w, int T, int n, int R,
                                      int G, int chunks_per_range, float* part, hipStream_t st,
                                      const float* scale = nullptr, const float* base = nullptr);

// Reduce partials, gates, Sinkhorn, collapse.
hipError_t launch_finish(const float* x, const float* part, int G, int T, int S, int H,
                         const float* scale, const float* base, int iters, float eps,
                         float* pre, float* post, float* comb, float* y, hipStream_t st);

// The previous site's post half, run in front of a pre chain: its input state
// x (the pre chain's x argument), branch output f [T][H] and gates post [T][S],
// comb [T][S][S]; the post mix is written to x_out and feeds the pre chain.
struct PostIn {
  const float* f;
  const float* post;
  const float* comb;
  float* x_out;
};

// Token-tiled fused pre chain (slab held on chip), for S <= 4 and H up to a
// register budget; fused_supported() says whether a shape qualifies.
// wpack: scratch of fused_pack_bytes(S, H) bytes for the weight in operand order,
// filled by the call; with prepacked, wpack already holds launch_pack_weight's
// output for fn_w and is only read.
// With zq non-null (H % 32 == 0) the kernel also writes the branch-input epilogue;
// with pin non-null it first runs the previous site's post mix on x.
bool fused_supported(int S, int H);
size_t fused_pack_bytes(int S, int H);
hipError_t launch_pack_weight(const float* fn_w, int S, int H, float* wpack, hipStream_t st);
hipError_t launch_fused_pre(const float* x, const float* fn_w, const float* scale,
                            const float* base, int T, int S, int H, int iters, float eps,
                            float* pre, float* post, float* comb, float* y, float* wpack,
                            const Zq8Out* zq, const PostIn* pin, hipStream_t st,
                            bool prepacked = false);

// The gated head (R = S rows, one scale, S biases, sigmoid gates, collapse) on
// the same token tiles, for the shapes fused_supported() accepts; wpack holds
// fused_head_pack_bytes(S, H) bytes.
size_t fused_head_pack_bytes(int S, int H);
hipError_t launch_fused_head(const float* x, const float* fn_h, const float* scale_h,
                             const float* base_h, int T, int S, int H, float eps, float* gates,
                             float* y, float* wpack, hipStream_t st);

// One decode token's finish with the branch-input epilogue (T = 1, S <= 4,
// H % 32 == 0, H <= 8192): the partials as launch_finish takes them.
bool finish_zq8_supported(int T, int S, int H);
hipError_t launch_finish_zq8(const float* x, const float* part, int G, int S, int H,
                             const float* scale, const float* base, int iters, float eps,
                             float* pre, float* post, float* comb, float* y, const Zq8Out& zq,
                             hipStream_t st);

// Branch-input epilogue: z = RMS-norm(y) * nw and its q8 codes / block scales,
// one block per token; H % 32 == 0 and H <= 8192 (zq8_supported).
bool zq8_supported(int H);
hipError_t launch_zq8(const float* y, const float* nw, int T, int H, float norm_eps, float* z,
                      signed char* q, float* d, hipStream_t st);

// Trunk entry and exit: expand e [T][H] -> x [T][S][H]; mean x -> y [T][H];
// the gated head's finish (partials of its S rows, from launch_small_partials_rows,
// then gates [T][S] and y [T][H]).
hipError_t launch_expand(const float* e, int T, int S, int H, float* x, hipStream_t st);
hipError_t launch_mean(const float* x, int T, int S, int H, float* y, hipStream_t st);
hipError_t launch_head_finish(const float* x, const float* part, int G, int T, int S, int H,
                              const float* scale_h, const float* base_h, float eps, float* gates,
                              float* y, hipStream_t st);

// Bandwidth probes: copy nq 16-byte quads from src to dst, or (copy false)
// read them and write probe_blocks(nq) block sums to dst.
long probe_blocks(long nq);
hipError_t launch_probe(const float* src, float* dst, long nq, bool copy, hipStream_t st);

// Post mix.
hipError_t launch_post(const float* x, const float* f, const float* post, const float* comb,
                       int T, int S, int H, float* x_out, hipStream_t st);

}  // namespace mhc
