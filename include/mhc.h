/*
 * mhc.h -- C ABI of the MI355X (gfx950) mHC site library (libmhc.so).
 *
 * The library runs the per-token, per-site mHC (manifold-constrained
 * hyper-connections) residual program on one GPU, as two calls:
 *
 *   mhc_site_pre   mixes GEMV + RMS rescale + gates + Sinkhorn + collapse
 *   mhc_site_post  post mix of the branch output back into the streams
 *
 * The operation is the one described on the docs.rs page "memra_engine
 * 0.125.0 src/memra_engine/hyper.rs", module documentation ("ARITHMETIC
 * CONTRACT" and "MEMORY LAYOUT"), with the row order of the mixes given by the
 * doc comment of HyperTopology::rows and the post mix by the doc comment of the
 * page's `post` function.  The gate forms the page leaves open are fixed here:
 * pre = sigmoid, post = 2*sigmoid, comb = Sinkhorn-Knopp of exp(.), one
 * iteration being a row pass then a column pass, each dividing by (sum + eps).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers to dense fp32 arrays owned by the
 *    caller; each must be 16-byte aligned.  Outputs are fully overwritten (no
 *    zeroing needed, prior contents never read).  The library keeps no pointer
 *    after a call returns.
 *  - Layout is token-major: x[T][S][H], element (t,k,i) at (t*S+k)*H+i, so one
 *    token's S*H slab is contiguous.  S = streams, H = hidden, R = (2+S)*S.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work and do not wait for the device, except that a call which must grow
 *    the library scratch (below) allocates device memory with hipMalloc.
 *    Results are ready once the stream reaches the enqueued work.
 *  - Every argument check happens on the host BEFORE any GPU work is enqueued;
 *    a call that returns an error has enqueued nothing.
 *  - Calls on the same device share one library-owned scratch area (partial
 *    sums of the split reduction, the packed weight of the large-batch
 *    kernel).  Two calls enqueued on DIFFERENT streams of the same device must
 *    not run concurrently; calls on one stream are always safe.  The first
 *    call on a device that needs scratch allocates it, and a later call that
 *    needs more allocates a larger area.  No scratch area is ever freed
 *    before the process ends, so HIP graphs captured earlier stay valid.  A
 *    call that would have to grow the scratch while its stream is being
 *    captured returns MHC_ECAPTURE: make one call of the largest size before
 *    capturing (or use a workspace, which never allocates).
 *  - Supported shapes: 1 <= S <= 8, H >= 4 with H % 4 == 0, T >= 0
 *    (T == 0 is a no-op), iters >= 1, eps > 0 and finite, T*S*H < 2^31.
 *  - Numeric domain: finite inputs with |scale*m + base| below about 80, so
 *    that exp() stays finite in fp32; outside it results are unspecified.
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  MHC_OK = 0,
  MHC_EINVAL = 1,      /* bad size, count, eps, iteration count or NULL pointer */
  MHC_EALIGN = 2,      /* H % 4 != 0 or a pointer not 16-byte aligned            */
  MHC_EUNSUPPORTED = 3,/* valid arguments the library does not handle (S > 8, sizes too large) */
  MHC_EHIP = 4,        /* the HIP runtime reported an error (launch, allocation) */
  MHC_EOVERLAP = 5,    /* an output buffer overlaps an input buffer              */
  MHC_ECAPTURE = 6     /* the scratch would have to grow while the stream is captured */
};

/*
 * mhc_site_pre -- the pre half of one site, for T tokens.
 *
 * Per token t (hyper.rs module doc, arithmetic contract, first four lines):
 *   ss      = sum_i x[t,i]^2 over the whole S*H slab;  rinv = 1/sqrt(ss/(S*H) + eps)
 *   m[r]    = rinv * sum_i fn_w[r,i] * x[t,i]                         r < R
 *   z[r]    = scale[g] * m[r] + base[r]   g = 0 for rows [0,S), 1 for [S,2S),
 *                                         2 for the S*S comb rows [2S,R)
 *   pre[t,c]   = 1/(1+exp(-z[c]))
 *   post[t,k]  = 2/(1+exp(-z[S+k]))
 *   comb[t,j,k]= Sinkhorn of exp(z[2S + j*S + k]) over `iters` rounds
 *                (j = source stream, k = target stream)
 *   y[t,i]     = sum_c pre[t,c] * x[t,c,i]
 *
 * Arguments:
 *   x      [T][S][H]  stream state (read only)
 *   fn_w   [R][S*H]   mixes weight, row-major (read only)
 *   scale  [3]        pre, post and comb scales (read only)
 *   base   [R]        per-row bias (read only)
 *   T, streams (=S), hidden (=H), iters, eps   as above
 *   pre    [T][S]     out
 *   post   [T][S]     out
 *   comb   [T][S][S]  out
 *   y      [T][H]     out (the branch input)
 *   stream            hipStream_t or NULL
 * Outputs must not overlap x, fn_w, scale, base or each other (MHC_EOVERLAP).
 * Returns MHC_OK or an error code above.
 */
int mhc_site_pre(const float* x, const float* fn_w, const float* scale, const float* base,
                 int T, int streams, int hidden, int iters, float eps,
                 float* pre, float* post, float* comb, float* y, void* stream);

/*
 * mhc_site_pre_scratch_bytes -- bytes of library scratch that
 * mhc_site_pre needs for T tokens of this shape: the packed weight where the
 * large-batch kernel runs, else the split reduction's partial sums.  0 for
 * T < 1 or a shape the call rejects.  Host only: no HIP call, safe without a
 * GPU.  A caller that captures HIP graphs can make one eager call at its
 * largest T first, or compare this figure across the shapes it will capture.
 */
size_t mhc_site_pre_scratch_bytes(int T, int streams, int hidden);

/*
 * mhc_site_pre_static -- mhc_site_pre for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks, kernels and results, but the kernel
 * scratch is a fixed device array inside the library, 16 MiB on each GPU the
 * process uses, held until the process ends.  The call allocates, frees and
 * clears nothing.  A shape whose scratch (mhc_site_pre_scratch_bytes) exceeds
 * 16 MiB returns MHC_EUNSUPPORTED before anything is enqueued (large batches
 * of short slabs can need more; the decode, verify, prefill and wide sites
 * need at most 10.7 MB).  Every call on a GPU shares that GPU's array
 * (the last call's contents stay in it): two calls that overlap in time on one
 * GPU (different streams, or concurrent graph replays) race on it and must be
 * ordered by the caller.
 */
int mhc_site_pre_static(const float* x, const float* fn_w, const float* scale, const float* base,
                        int T, int streams, int hidden, int iters, float eps, float* pre,
                        float* post, float* comb, float* y, void* stream);

/*
 * mhc_site_post -- the post half of one site (hyper.rs, doc comment of `post`):
 *   x_out[t,k,i] = post[t,k] * f[t,i] + sum_j comb[t,j,k] * x[t,j,i]
 * where x is the SITE's input state (the same x given to mhc_site_pre) and f the
 * branch output for the site.
 *
 * Arguments:
 *   x      [T][S][H]  site input state (read only)
 *   f      [T][H]     branch output (read only)
 *   post   [T][S]     post gates (read only)
 *   comb   [T][S][S]  combination matrices, comb[t][j][k] (read only)
 *   T, streams (=S), hidden (=H)
 *   x_out  [T][S][H]  out; must not overlap any input (MHC_EOVERLAP)
 *   stream            hipStream_t or NULL
 * Returns MHC_OK or an error code above.
 */
int mhc_site_post(const float* x, const float* f, const float* post, const float* comb,
                  int T, int streams, int hidden, float* x_out, void* stream);

/*
 * Pre-packed mixes weight.  A site's weight fn_w is a fixed parameter (the
 * hyper.rs page's module doc: the mixes weight of a site, [R][S*H]), while the
 * large-batch pre kernel reads it in its own MFMA operand order, which
 * mhc_site_pre produces by packing fn_w into the library scratch on every
 * call.  A caller that keeps a site's weight can pack it once instead:
 *
 * mhc_packed_weight_bytes(streams, hidden): bytes of the packed form, or 0 for
 *   a shape the large-batch kernel does not serve (then no packed form exists
 *   and mhc_site_pre_packed takes packed == NULL).
 * mhc_pack_weight(fn_w, streams, hidden, packed, stream): writes the packed
 *   form of fn_w [R][S*H] into packed (mhc_packed_weight_bytes bytes, caller
 *   owned, 16-byte aligned, not overlapping fn_w).  MHC_EUNSUPPORTED for a
 *   shape with no packed form; asynchronous on `stream`.
 * mhc_site_pre_packed(x, fn_w, packed, scale, base, ...): mhc_site_pre with
 *   the weight read from `packed` wherever the large-batch kernel runs (fn_w
 *   is still read on the small-batch path).  packed must hold
 *   mhc_pack_weight's output for this fn_w and shape, and must not overlap the
 *   outputs (MHC_EOVERLAP); NULL is MHC_EINVAL for a shape with a packed form.
 *   The results are bit-identical to mhc_site_pre's.  Nothing is written to
 *   the library scratch on the large-batch path.
 */
size_t mhc_packed_weight_bytes(int streams, int hidden);
int mhc_pack_weight(const float* fn_w, int streams, int hidden, float* packed, void* stream);
int mhc_site_pre_packed(const float* x, const float* fn_w, const float* packed,
                        const float* scale, const float* base, int T, int streams, int hidden,
                        int iters, float eps, float* pre, float* post, float* comb, float* y,
                        void* stream);
/* mhc_site_post_pre with the next site's weight read from `packed` wherever the
 * fused kernel runs: same arguments as mhc_site_post_pre plus `packed`, with the
 * conditions of mhc_site_pre_packed (packed must not overlap x_out or the
 * outputs either); bit-identical results. */
int mhc_site_post_pre_packed(const float* x, const float* f, const float* post_in,
                             const float* comb_in, const float* fn_w, const float* packed,
                             const float* scale, const float* base, int T, int streams,
                             int hidden, int iters, float eps, float* x_out, float* pre,
                             float* post, float* comb, float* y, void* stream);

/*
 * mhc_site_pre_exact -- mhc_site_pre with decode-exact batching: every token's
 * pre, post, comb and y are bit-identical to those of a call of mhc_site_pre on
 * that token alone (T = 1), whatever T is and whatever else is in the batch
 * (the hyper.rs page, doc comment of pre_exact: a batched decode row must equal
 * the session's solo step, so the mixes of every row are reduced in the order
 * of a solo token).  Same arguments, checks and return codes as mhc_site_pre.
 * mhc_site_pre itself already has this property for T < 256 when S <= 4 and
 * for T <= 64 when S > 4 (there the two calls run the same kernels); above
 * that this call keeps the solo K-split instead of the faster large-batch
 * schedules, and reads x twice.
 */
int mhc_site_pre_exact(const float* x, const float* fn_w, const float* scale, const float* base,
                       int T, int streams, int hidden, int iters, float eps, float* pre,
                       float* post, float* comb, float* y, void* stream);

/*
 * mhc_site_pre_zq8 -- mhc_site_pre followed by the branch-input epilogue: the
 * RMS norm of y with weight nw and its int8 q8 encoding (the norm-and-q8 step
 * that the fused "v4z" pre kernel of the hc_fused_gate.rs page folds into the
 * pre chain; epsilon 1e-5 there).  Per token t, after y[t,:] as above:
 *   z[t,i] = y[t,i] * nw[i] / sqrt(mean_i(y[t,i]^2) + norm_eps)
 *   per block of 32 consecutive i:  d[t,b] = max|z| / 127,
 *   q[t,i] = z[t,i] * (1/d[t,b]) rounded to nearest, ties away from zero
 *   (an all-zero block gives d = 0 and q = 0).  d and 1/d are IEEE fp32
 *   divisions, so q and d are a function of the fp32 z written.
 *
 * Arguments: as mhc_site_pre, plus
 *   nw        [H]         norm weight (read only)
 *   norm_eps              > 0 and finite
 *   z         [T][H]      out (fp32)
 *   q         [T][H]      out (int8)
 *   d         [T][H/32]   out (fp32)
 * hidden must be a multiple of 32 and at most 8192 (MHC_EALIGN / MHC_EUNSUPPORTED).
 * Outputs must not overlap any input or each other (MHC_EOVERLAP).
 */
int mhc_site_pre_zq8(const float* x, const float* fn_w, const float* scale, const float* base,
                     const float* nw, int T, int streams, int hidden, int iters, float eps,
                     float norm_eps, float* pre, float* post, float* comb, float* y, float* z,
                     signed char* q, float* d, void* stream);

/*
 * mhc_site_post_pre -- the post half of one site followed by the pre half of the
 * next site on its output, the order in which a trunk runs them (hyper.rs page,
 * module doc: per site, attention then MLP, each site's output state is the
 * next site's input).  Equivalent to
 *     mhc_site_post(x, f, post_in, comb_in, ..., x_out);
 *     mhc_site_pre(x_out, fn_w, scale, base, ..., pre, post, comb, y);
 * and bit-identical to that pair.  Where the token-tiled pre kernel serves the
 * shape (S <= 4, T >= 256) one kernel does both and the new state is not read
 * back from memory.  The _zq8 form adds the branch-input epilogue of the second
 * site, as mhc_site_pre_zq8.
 *
 * Arguments: x, f, post_in, comb_in as mhc_site_post (the first site);
 * fn_w, scale, base, iters, eps as mhc_site_pre (the second site); x_out is the
 * first site's output and the second site's input; pre, post, comb, y (and
 * z, q, d) the second site's outputs.  An output that overlaps an input or
 * another output is MHC_EOVERLAP (a walk alternates two sets of gate buffers).
 */
int mhc_site_post_pre(const float* x, const float* f, const float* post_in, const float* comb_in,
                      const float* fn_w, const float* scale, const float* base, int T,
                      int streams, int hidden, int iters, float eps, float* x_out, float* pre,
                      float* post, float* comb, float* y, void* stream);
int mhc_site_post_pre_zq8(const float* x, const float* f, const float* post_in,
                          const float* comb_in, const float* fn_w, const float* scale,
                          const float* base, const float* nw, int T, int streams, int hidden,
                          int iters, float eps, float norm_eps, float* x_out, float* pre,
                          float* post, float* comb, float* y, float* z, signed char* q, float* d,
                          void* stream);
int mhc_site_post_pre_check(const float* x, const float* f, const float* post_in,
                            const float* comb_in, const float* fn_w, const float* scale,
                            const float* base, int T, int streams, int hidden, int iters,
                            float eps, const float* x_out, const float* pre, const float* post,
                            const float* comb, const float* y);

/*
 * Trunk entry and exit (hyper.rs page: doc comments of `expand`,
 * `contract_mean` and `collapse`; the HyperHead loader sizes the head).
 *
 * mhc_expand: x_out[t,k,i] = e[t,i] for every stream k.
 *   e [T][H] (read only) -> x_out [T][S][H]; x_out must not overlap e.
 * mhc_mean: y_out[t,i] = (sum_k x[t,k,i]) / S, streams summed in ascending
 *   order in fp32, then one IEEE division.  x [T][S][H] -> y_out [T][H].
 * mhc_head: the gated-head exit, the pre half of a site with the head's own
 *   weight fn_w [S][S*H], one scale [1] and biases base [S]:
 *     rinv = 1/sqrt(sum_i x[t,i]^2 / (S*H) + eps)         (over the slab)
 *     gates[t,c] = 1/(1+exp(-(scale * rinv * (fn_w[c,:] . x[t,:]) + base[c])))
 *     y[t,i] = sum_c gates[t,c] * x[t,c,i]
 *   gates [T][S] and y [T][H] are outputs; they must not overlap the inputs or
 *   each other.  Uses the library's per-device scratch (as mhc_site_pre).
 * Same size, pointer and return-code conventions as the site calls (hidden % 4
 * == 0, 16-byte aligned pointers, 1 <= streams <= 8, eps > 0 and finite;
 * T = 0 does nothing).  mhc_head_check is the host-side check alone.
 */
int mhc_expand(const float* e, int T, int streams, int hidden, float* x_out, void* stream);
int mhc_mean(const float* x, int T, int streams, int hidden, float* y_out, void* stream);
int mhc_head(const float* x, const float* fn_w, const float* scale, const float* base, int T,
             int streams, int hidden, float eps, float* gates, float* y, void* stream);
int mhc_head_check(const float* x, const float* fn_w, const float* scale, const float* base,
                   int T, int streams, int hidden, float eps, const float* gates,
                   const float* y);

/*
 * Persistent site workspace (the hyper.rs page, doc comment of HyperDecodeWs:
 * one set of buffers per engine, every buffer fully overwritten before it is
 * read, the stream state ping-ponged with one spare slot, so that a decode
 * token makes no allocation).  Here the caller provides the memory and the
 * library never allocates on the workspace path, so a walk over sites can be
 * captured in a HIP graph.
 *
 * mhc_workspace_bytes(max_tokens, streams, hidden) is the device memory a
 * workspace needs (0 for an invalid shape; 1 <= max_tokens <= 8192).
 * mhc_workspace_init carves `mem` (device memory, 256-byte aligned, at least
 * that many bytes, owned by the caller and kept alive while the workspace is
 * used) into the regions below and fills *ws (host memory of the caller); it
 * makes no HIP call and enqueues nothing.  Returns MHC_EINVAL / MHC_EALIGN /
 * MHC_EUNSUPPORTED.
 *
 * The fields are read-only for the caller except that the current stream state
 * state[cur] may be written (e.g. the trunk's entry state) and read at any
 * time.  All outputs have max_tokens rows; a call with T tokens writes the
 * first T.  z, q and d are meaningful only when hidden % 32 == 0.
 *
 * mhc_ws_site_pre / mhc_ws_site_pre_zq8: mhc_site_pre / mhc_site_pre_zq8 on
 * x = state[cur] with the workspace's outputs and its own scratch (so two
 * workspaces may run concurrently on different streams; one workspace must not).
 * mhc_ws_site_post: mhc_site_post from state[cur] with the workspace's post and
 * comb into state[cur ^ 1], then flips cur on the host.  A captured graph bakes
 * the slots in: capture an even number of posts (the two sites of a layer) so
 * that every replay starts and ends in the same slot.  0 <= T <= max_tokens; a
 * call with T = 0 does nothing and does not flip.  Errors as the plain calls.
 */
typedef struct mhc_workspace {
  int max_tokens, streams, hidden;
  int cur;              /* index of the current stream state: 0 or 1 */
  float* state[2];      /* [max_tokens][S][H] each */
  float* pre;           /* [max_tokens][S] */
  float* post;          /* [max_tokens][S] */
  float* comb;          /* [max_tokens][S][S] */
  float* y;             /* [max_tokens][H] */
  float* z;             /* [max_tokens][H] */
  signed char* q;       /* [max_tokens][H] */
  float* d;             /* [max_tokens][ceil(H/32)] */
  void* scratch;        /* kernel scratch: partials / packed weight */
  size_t scratch_bytes; /* bytes of scratch */
} mhc_workspace;

size_t mhc_workspace_bytes(int max_tokens, int streams, int hidden);
size_t mhc_workspace_struct_bytes(void); /* sizeof(mhc_workspace), for bindings */
int mhc_workspace_init(mhc_workspace* ws, void* mem, size_t bytes, int max_tokens, int streams,
                       int hidden);
int mhc_ws_site_pre(mhc_workspace* ws, const float* fn_w, const float* scale, const float* base,
                    int T, int iters, float eps, void* stream);
int mhc_ws_site_pre_zq8(mhc_workspace* ws, const float* fn_w, const float* scale,
                        const float* base, const float* nw, int T, int iters, float eps,
                        float norm_eps, void* stream);
int mhc_ws_site_post(mhc_workspace* ws, const float* f, int T, void* stream);

/*
 * Argument checks alone: return exactly the code mhc_site_pre / mhc_site_post
 * would return for these arguments before enqueuing any work (MHC_OK if the
 * call would go ahead).  They make no HIP call and are safe without a GPU.
 */
int mhc_site_pre_check(const float* x, const float* fn_w, const float* scale, const float* base,
                       int T, int streams, int hidden, int iters, float eps,
                       const float* pre, const float* post, const float* comb, const float* y);
int mhc_site_post_check(const float* x, const float* f, const float* post, const float* comb,
                        int T, int streams, int hidden, const float* x_out);
int mhc_site_pre_zq8_check(const float* x, const float* fn_w, const float* scale,
                           const float* base, const float* nw, int T, int streams, int hidden,
                           int iters, float eps, float norm_eps, const float* pre,
                           const float* post, const float* comb, const float* y, const float* z,
                           const signed char* q, const float* d);

/* Static text for a return code (never NULL). */
const char* mhc_status_string(int status);

/*
 * Bandwidth probe (a measurement aid, not part of the site program).  The
 * hc_fused_gate.rs page's gate carries a bandwidth probe of its own, a pure
 * streamer reporting read and read + write GB/s; this one gives the same two
 * rates on this part, and the site kernels' rates are read against them.
 *
 * mhc_bandwidth_probe: with copy != 0, copies `bytes` from src to dst (both
 *   `bytes` long, not overlapping); with copy == 0, reads `bytes` from src and
 *   writes mhc_probe_sink_floats(bytes) block sums (one per 4 KiB of src) to
 *   dst.  Streaming 16-byte loads (and stores), one quad per thread.
 *   bytes % 16 == 0 and 16-byte aligned pointers (MHC_EALIGN otherwise); NULL
 *   pointers are MHC_EINVAL; overlapping buffers MHC_EOVERLAP; more than 2^43
 *   bytes MHC_EUNSUPPORTED; bytes == 0 does nothing.  Asynchronous on
 *   `stream` like the site calls.
 */
size_t mhc_probe_sink_floats(size_t bytes);
int mhc_bandwidth_probe(const float* src, float* dst, size_t bytes, int copy, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MHC_H */
