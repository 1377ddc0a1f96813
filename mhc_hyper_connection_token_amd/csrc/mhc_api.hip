// mhc_api.hip -- the C ABI of libmhc (declared in include/mhc.h): argument
// checks, the per-device scratch area, and the choice of kernels per shape.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "mhc.h"
#include "mhc_kernels.h"

namespace {

constexpr long kMaxElems = 1L << 31;  // T*S*H must stay below this (int indexing)
constexpr int kMaxTokens = 1 << 23;   // bounds the flattened launch grids
constexpr int kFusedMinTokens = 256;  // below this the split-K path fills the chip better
constexpr int kSoloPlanMaxWide = 64;  // S > 4: up to this T the solo K-split with 16-token tiles
constexpr int kExactChunk = 8192;     // tokens per pass of mhc_site_pre_exact

int check_ptr(const void* p) {
  if (!p) return MHC_EINVAL;
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return MHC_EALIGN;
  return MHC_OK;
}

struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int check_shape(int T, int S, int H) {
  if (T < 0 || S < 1 || H < 1) return MHC_EINVAL;
  if (S > 8) return MHC_EUNSUPPORTED;
  if (H % 4 != 0) return MHC_EALIGN;
  if ((long)T * S * H >= kMaxElems || T >= kMaxTokens) return MHC_EUNSUPPORTED;
  return MHC_OK;
}

// Library-owned scratch, one current buffer per device (split-K partials,
// packed weight).
//
// A call that needs more than the current buffer allocates a larger one and
// makes it current.  The smaller one is never freed: work already enqueued on
// it, and HIP graphs captured while it was current, keep pointing at valid
// memory until the process ends (the buffers grow by a quarter each time, so
// the retired ones add up to a bounded multiple of the largest).  Growth is a
// hipMalloc, which HIP graph capture does not allow, so a call that would grow
// the buffer while its stream is being captured returns MHC_ECAPTURE and
// enqueues nothing; one call of the same size outside the capture sizes it.
struct DeviceScratch {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_scratch_mu;
DeviceScratch g_scratch[64];

struct Scratch {
  float* general = nullptr;
};

// Bytes of the next buffer when `need` bytes are wanted and
// `have` are current: 1 MiB at least, then a quarter more than asked for.
size_t scratch_grow_bytes(size_t need, size_t have) {
  if (need <= have) return have;
  return need < (size_t(1) << 20) ? (size_t(1) << 20) : need + need / 4;
}

int get_scratch(size_t bytes, hipStream_t st, Scratch* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MHC_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  DeviceScratch& s = g_scratch[dev];
  const size_t need = bytes;
  if (s.bytes < need) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess) return MHC_EHIP;
    if (cap != hipStreamCaptureStatusNone) return MHC_ECAPTURE;
    const size_t want = scratch_grow_bytes(need, s.bytes);
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) return MHC_EHIP;
    s.ptr = p;  // the previous buffer stays allocated (see above)
    s.bytes = want;
  }
  out->general = static_cast<float*>(s.ptr);
  return MHC_OK;
}

// Scratch for one call: a workspace's own area when the caller brings one (it
// was sized for the largest request of its shape), else the library's
// per-device area.
struct ScratchSource {
  const Scratch* fixed = nullptr;
  size_t bytes = 0;
};

int acquire_scratch(const ScratchSource& src, size_t bytes, hipStream_t st, Scratch* out) {
  if (src.fixed) {
    if (bytes > src.bytes) return MHC_EINVAL;
    *out = *src.fixed;
    return MHC_OK;
  }
  return get_scratch(bytes, st, out);
}

// Split-K plan for the pre chain: token tiles of 16*ntt tokens, G K-ranges of
// cpr 16-float chunks each.  G and the tile width depend only on (T <= 16) and
// the shape, never on which tokens a block holds, so a token's result is the
// same whatever else is in the batch as long as T stays on the same side of 16.
struct PrePlan {
  int ntt, G, cpr;
  size_t part_floats;
};

PrePlan plan_pre(int T, int S, int H);

// The plan the pre chain uses at T tokens on the split path.  Where the solo
// token's K-split is also the faster schedule (S <= 4 below the fused kernel's
// threshold, S > 4 up to 64 tokens) it is kept, which makes those rows
// bit-identical to solo calls; larger batches take wider ranges and tiles.
PrePlan plan_split(int T, int S, int H) {
  const bool solo = S <= 4 ? T < kFusedMinTokens : T <= kSoloPlanMaxWide;
  if (!solo) return plan_pre(T, S, H);
  PrePlan p = plan_pre(1, S, H);
  p.part_floats = (size_t)p.G * T * ((2 + S) * S + 1);
  return p;
}

PrePlan plan_pre(int T, int S, int H) {
  const int n = S * H, R = (2 + S) * S, nrt = (R + 15) / 16;
  const int nchunks = (n + 15) / 16;
  PrePlan p;
  // 64-token blocks where the grid stays at 512 blocks or more (every weight
  // fetch then serves 64 tokens); 32-token blocks for 4-5 row tiles below that
  p.ntt = T <= 16 ? 1 : ((nrt <= 3 || T >= 512) ? 4 : 2);
  const int tiles = (T + 16 * p.ntt - 1) / (16 * p.ntt);
  int G;
  if (tiles == 1) {
    G = nchunks / 8;
    if (G > 128) G = 128;
  } else {
    G = (512 + tiles - 1) / tiles;
    if (G > 64) G = 64;
    if (G > nchunks / 32) G = nchunks / 32;
  }
  if (G < 1) G = 1;
  p.cpr = (nchunks + G - 1) / G;
  p.G = (nchunks + p.cpr - 1) / p.cpr;
  p.part_floats = (size_t)p.G * T * (R + 1);
  return p;
}

// Scratch bytes of the pre chain at T tokens (the kernel choice of site_pre_run).
size_t pre_scratch_bytes(int T, int S, int H) {
  if (T >= kFusedMinTokens && mhc::fused_supported(S, H)) return mhc::fused_pack_bytes(S, H);
  return plan_split(T, S, H).part_floats * sizeof(float);
}

}  // namespace

extern "C" {

const char* mhc_status_string(int status) {
  switch (status) {
    case MHC_OK: return "ok";
    case MHC_EINVAL: return "invalid argument (size, count, eps, iterations or NULL pointer)";
    case MHC_EALIGN: return "misaligned: hidden must be a multiple of 4 and pointers 16-byte aligned";
    case MHC_EUNSUPPORTED:
      return "unsupported size (streams > 8, T*streams*hidden >= 2^31, or a larger buffer than "
             "the call handles)";
    case MHC_EHIP: return "HIP runtime error";
    case MHC_EOVERLAP: return "an output buffer overlaps an input or another output";
    case MHC_ECAPTURE:
      return "the call needs a larger library scratch area while its stream is being captured "
             "(make one call of this size before the capture)";
    default: return "unknown status";
  }
}

size_t mhc_site_pre_scratch_bytes(int T, int streams, int hidden) {
  if (T < 1 || check_shape(T, streams, hidden) != MHC_OK) return 0;
  return pre_scratch_bytes(T, streams, hidden);
}

int mhc_site_pre_check(const float* x, const float* fn_w, const float* scale, const float* base,
                       int T, int streams, int hidden, int iters, float eps, const float* pre,
                       const float* post, const float* comb, const float* y) {
  int rc = check_shape(T, streams, hidden);
  if (rc) return rc;
  if (iters < 1 || !(eps > 0.0f) || !std::isfinite(eps)) return MHC_EINVAL;
  if (T == 0) return MHC_OK;
  const void* ptrs[] = {x, fn_w, scale, base, pre, post, comb, y};
  for (const void* p : ptrs)
    if (!p) return MHC_EINVAL;
  for (const void* p : ptrs)
    if ((rc = check_ptr(p))) return rc;
  const size_t S = streams, H = hidden, Tz = T, R = (2 + S) * S;
  const Span in[] = {span(x, Tz * S * H * 4), span(fn_w, R * S * H * 4), span(scale, 12),
                     span(base, R * 4)};
  const Span out[] = {span(pre, Tz * S * 4), span(post, Tz * S * 4), span(comb, Tz * S * S * 4),
                      span(y, Tz * H * 4)};
  for (int o = 0; o < 4; ++o) {
    for (const Span& i : in)
      if (overlaps(out[o], i)) return MHC_EOVERLAP;
    for (int p = o + 1; p < 4; ++p)
      if (overlaps(out[o], out[p])) return MHC_EOVERLAP;
  }
  return MHC_OK;
}

int mhc_site_post_check(const float* x, const float* f, const float* post, const float* comb,
                        int T, int streams, int hidden, const float* x_out) {
  int rc = check_shape(T, streams, hidden);
  if (rc) return rc;
  if (T == 0) return MHC_OK;
  const void* ptrs[] = {x, f, post, comb, x_out};
  for (const void* p : ptrs)
    if (!p) return MHC_EINVAL;
  for (const void* p : ptrs)
    if ((rc = check_ptr(p))) return rc;
  const size_t S = streams, H = hidden, Tz = T;
  const Span o = span(x_out, Tz * S * H * 4);
  const Span in[] = {span(x, Tz * S * H * 4), span(f, Tz * H * 4), span(post, Tz * S * 4),
                     span(comb, Tz * S * S * 4)};
  for (const Span& i : in)
    if (overlaps(o, i)) return MHC_EOVERLAP;
  return MHC_OK;
}

}  // extern "C"

namespace {

// The pre chain for checked arguments.  With zq, the branch-input epilogue runs
// in the tail of the fused kernels and in the one-token finish where they
// support it, otherwise as its own launch after the chain.
int site_pre_run(const float* x, const float* fn_w, const float* scale, const float* base, int T,
                 int S, int H, int iters, float eps, float* pre, float* post, float* comb,
                 float* y, const mhc::Zq8Out* zq, hipStream_t st,
                 const ScratchSource& src = ScratchSource(), const float* packed = nullptr) {
  int rc;
  const int n = S * H, R = (2 + S) * S;
  bool zq_done = false;
  if (T >= kFusedMinTokens && mhc::fused_supported(S, H)) {
    // Large batches with a slab that fits on chip: x read once.  A weight the
    // caller packed beforehand is read as it is; otherwise it is packed into
    // the scratch first.
    hipError_t e;
    if (packed) {
      e = mhc::launch_fused_pre(x, fn_w, scale, base, T, S, H, iters, eps, pre, post, comb, y,
                                const_cast<float*>(packed), zq, nullptr, st, true);
    } else {
      Scratch sc;
      if ((rc = acquire_scratch(src, mhc::fused_pack_bytes(S, H), st, &sc))) return rc;
      e = mhc::launch_fused_pre(x, fn_w, scale, base, T, S, H, iters, eps, pre, post, comb, y,
                                sc.general, zq, nullptr, st);
    }
    if (e != hipSuccess) return MHC_EHIP;
    zq_done = true;
  } else {
    const PrePlan p = plan_split(T, S, H);
    Scratch sc;
    if ((rc = acquire_scratch(src, p.part_floats * sizeof(float), st, &sc))) return rc;
    float* part = sc.general;
    hipError_t e;
    if (zq && mhc::finish_zq8_supported(T, S, H)) {
      // one decode token with the epilogue: the partials, then two blocks that
      // finish (one runs the Sinkhorn, the other the collapse and epilogue)
      e = mhc::launch_small_partials(x, fn_w, T, S, H, p.G, p.cpr, part, st, scale, base);
      if (e == hipSuccess)
        e = mhc::launch_finish_zq8(x, part, p.G, S, H, scale, base, iters, eps, pre, post, comb,
                                   y, *zq, st);
      zq_done = true;
    } else {
      // S <= 4 below the fused threshold: the vector-ALU partials
      e = (S <= 4 && T < kFusedMinTokens)
              ? mhc::launch_small_partials(x, fn_w, T, S, H, p.G, p.cpr, part, st, scale, base)
              : mhc::launch_partials(x, fn_w, T, n, R, p.ntt, p.G, p.cpr, part, st);
      if (e == hipSuccess)
        e = mhc::launch_finish(x, part, p.G, T, S, H, scale, base, iters, eps, pre, post, comb,
                               y, st);
    }
    if (e != hipSuccess) return MHC_EHIP;
  }
  if (zq && !zq_done &&
      mhc::launch_zq8(y, zq->nw, T, H, zq->norm_eps, zq->z, zq->q, zq->d, st) != hipSuccess)
    return MHC_EHIP;
  return MHC_OK;
}

// The post half of one site followed by the pre half of the next on its output.
// Where the fused kernel serves the shape, one launch (plus the weight pack)
// does both and the new state is never read back; elsewhere the post kernel
// and then the pre chain.
int site_post_pre_run(const float* x, const float* f, const float* post_in, const float* comb_in,
                      const float* fn_w, const float* scale, const float* base, int T, int S,
                      int H, int iters, float eps, float* x_out, float* pre, float* post,
                      float* comb, float* y, const mhc::Zq8Out* zq, hipStream_t st,
                      const float* packed = nullptr) {
  if (T >= kFusedMinTokens && mhc::fused_supported(S, H)) {
    const mhc::PostIn pin{f, post_in, comb_in, x_out};
    hipError_t e;
    if (packed) {
      e = mhc::launch_fused_pre(x, fn_w, scale, base, T, S, H, iters, eps, pre, post, comb, y,
                                const_cast<float*>(packed), zq, &pin, st, true);
    } else {
      Scratch sc;
      int rc;
      if ((rc = get_scratch(mhc::fused_pack_bytes(S, H), st, &sc))) return rc;
      e = mhc::launch_fused_pre(x, fn_w, scale, base, T, S, H, iters, eps, pre, post, comb, y,
                                sc.general, zq, &pin, st);
    }
    return e == hipSuccess ? MHC_OK : MHC_EHIP;
  }
  // size the scratch of the pre chain first, so that a refusal (MHC_ECAPTURE)
  // comes before anything is enqueued
  Scratch sc;
  int rc;
  if ((rc = get_scratch(pre_scratch_bytes(T, S, H), st, &sc))) return rc;
  if (mhc::launch_post(x, f, post_in, comb_in, T, S, H, x_out, st) != hipSuccess) return MHC_EHIP;
  return site_pre_run(x_out, fn_w, scale, base, T, S, H, iters, eps, pre, post, comb, y, zq, st,
                      ScratchSource(), packed);
}

// A packed weight given with a call: checked against the shape and the outputs.
int check_packed(const float* packed, int S, int H, const Span* outs, int nout, size_t* pb) {
  *pb = mhc_packed_weight_bytes(S, H);
  if (*pb == 0) return MHC_OK;
  if (!packed) return MHC_EINVAL;
  int rc;
  if ((rc = check_ptr(packed))) return rc;
  const Span p = span(packed, *pb);
  for (int i = 0; i < nout; ++i)
    if (overlaps(outs[i], p)) return MHC_EOVERLAP;
  return MHC_OK;
}

}  // namespace

extern "C" {

int mhc_site_pre(const float* x, const float* fn_w, const float* scale, const float* base, int T,
                 int streams, int hidden, int iters, float eps, float* pre, float* post,
                 float* comb, float* y, void* stream) {
  int rc = mhc_site_pre_check(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post,
                              comb, y);
  if (rc || T == 0) return rc;
  return site_pre_run(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post, comb, y,
                      nullptr, static_cast<hipStream_t>(stream));
}

size_t mhc_packed_weight_bytes(int streams, int hidden) {
  if (streams < 1 || hidden < 1 || hidden % 4 != 0 || !mhc::fused_supported(streams, hidden))
    return 0;
  return mhc::fused_pack_bytes(streams, hidden);
}

int mhc_pack_weight(const float* fn_w, int streams, int hidden, float* packed, void* stream) {
  int rc = check_shape(1, streams, hidden);
  if (rc) return rc;
  const size_t pb = mhc_packed_weight_bytes(streams, hidden);
  if (pb == 0) return MHC_EUNSUPPORTED;
  if (!fn_w || !packed) return MHC_EINVAL;
  if ((rc = check_ptr(fn_w)) || (rc = check_ptr(packed))) return rc;
  const size_t R = (2 + streams) * streams, n = (size_t)streams * hidden;
  if (overlaps(span(packed, pb), span(fn_w, R * n * 4))) return MHC_EOVERLAP;
  return mhc::launch_pack_weight(fn_w, streams, hidden, packed,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? MHC_OK
             : MHC_EHIP;
}

int mhc_site_pre_packed(const float* x, const float* fn_w, const float* packed,
                        const float* scale, const float* base, int T, int streams, int hidden,
                        int iters, float eps, float* pre, float* post, float* comb, float* y,
                        void* stream) {
  int rc = mhc_site_pre_check(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post,
                              comb, y);
  if (rc || T == 0) return rc;
  const size_t S = streams, H = hidden, Tz = T;
  const Span out[] = {span(pre, Tz * S * 4), span(post, Tz * S * 4), span(comb, Tz * S * S * 4),
                      span(y, Tz * H * 4)};
  size_t pb;
  if ((rc = check_packed(packed, streams, hidden, out, 4, &pb))) return rc;
  return site_pre_run(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post, comb, y,
                      nullptr, static_cast<hipStream_t>(stream), ScratchSource(),
                      pb ? packed : nullptr);
}

int mhc_site_pre_exact(const float* x, const float* fn_w, const float* scale, const float* base,
                       int T, int streams, int hidden, int iters, float eps, float* pre,
                       float* post, float* comb, float* y, void* stream) {
  int rc = mhc_site_pre_check(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post,
                              comb, y);
  if (rc || T == 0) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int S = streams, H = hidden, n = S * H, R = (2 + S) * S;
  // Where the plain call keeps the solo K-split it is already exact.
  if (S <= 4 ? T < kFusedMinTokens : T <= kSoloPlanMaxWide)
    return site_pre_run(x, fn_w, scale, base, T, S, H, iters, eps, pre, post, comb, y, nullptr,
                        st);
  // Otherwise the same split path with the solo K-split at any T: partials in
  // the per-token order of a solo call (vector ALU for S <= 4, 16-token MFMA
  // tiles above), then the finish kernel.  Tokens go in chunks so that the
  // partials stay bounded.
  const PrePlan p1 = plan_pre(1, S, H);
  const int chunk = T < kExactChunk ? T : kExactChunk;
  Scratch sc;
  if ((rc = get_scratch((size_t)p1.G * chunk * (R + 1) * sizeof(float), st, &sc))) return rc;
  for (int t0 = 0; t0 < T; t0 += chunk) {
    const int tc = T - t0 < chunk ? T - t0 : chunk;
    const float* xc = x + (size_t)t0 * n;
    hipError_t e = S <= 4 ? mhc::launch_small_partials(xc, fn_w, tc, S, H, p1.G, p1.cpr,
                                                       sc.general, st)
                          : mhc::launch_partials(xc, fn_w, tc, n, R, 1, p1.G, p1.cpr, sc.general,
                                                 st);
    if (e == hipSuccess)
      e = mhc::launch_finish(xc, sc.general, p1.G, tc, S, H, scale, base, iters, eps,
                             pre + (size_t)t0 * S, post + (size_t)t0 * S,
                             comb + (size_t)t0 * S * S, y + (size_t)t0 * H, st);
    if (e != hipSuccess) return MHC_EHIP;
  }
  return MHC_OK;
}

int mhc_site_pre_zq8_check(const float* x, const float* fn_w, const float* scale,
                           const float* base, const float* nw, int T, int streams, int hidden,
                           int iters, float eps, float norm_eps, const float* pre,
                           const float* post, const float* comb, const float* y, const float* z,
                           const signed char* q, const float* d) {
  // size checks first (as in mhc_site_pre_check), then pointers
  int rc = check_shape(T, streams, hidden);
  if (rc) return rc;
  if (iters < 1 || !(eps > 0.0f) || !std::isfinite(eps)) return MHC_EINVAL;
  if (!(norm_eps > 0.0f) || !std::isfinite(norm_eps)) return MHC_EINVAL;
  if (hidden % 32 != 0) return MHC_EALIGN;
  if (!mhc::zq8_supported(hidden)) return MHC_EUNSUPPORTED;
  if ((rc = mhc_site_pre_check(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post,
                               comb, y)))
    return rc;
  if (T == 0) return MHC_OK;
  const void* ptrs[] = {nw, z, q, d};
  for (const void* p : ptrs)
    if (!p) return MHC_EINVAL;
  for (const void* p : ptrs)
    if ((rc = check_ptr(p))) return rc;
  const size_t S = streams, H = hidden, Tz = T, R = (2 + S) * S;
  const Span in[] = {span(x, Tz * S * H * 4), span(fn_w, R * S * H * 4), span(scale, 12),
                     span(base, R * 4), span(nw, H * 4)};
  const Span out[] = {span(pre, Tz * S * 4), span(post, Tz * S * 4), span(comb, Tz * S * S * 4),
                      span(y, Tz * H * 4), span(z, Tz * H * 4), span(q, Tz * H),
                      span(d, Tz * (H / 32) * 4)};
  for (int o = 0; o < 7; ++o) {
    for (const Span& i : in)
      if (overlaps(out[o], i)) return MHC_EOVERLAP;
    for (int p = o + 1; p < 7; ++p)
      if (overlaps(out[o], out[p])) return MHC_EOVERLAP;
  }
  return MHC_OK;
}

int mhc_site_pre_zq8(const float* x, const float* fn_w, const float* scale, const float* base,
                     const float* nw, int T, int streams, int hidden, int iters, float eps,
                     float norm_eps, float* pre, float* post, float* comb, float* y, float* z,
                     signed char* q, float* d, void* stream) {
  int rc = mhc_site_pre_zq8_check(x, fn_w, scale, base, nw, T, streams, hidden, iters, eps,
                                  norm_eps, pre, post, comb, y, z, q, d);
  if (rc || T == 0) return rc;
  const mhc::Zq8Out zq{nw, norm_eps, z, q, d};
  return site_pre_run(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post, comb, y,
                      &zq, static_cast<hipStream_t>(stream));
}

int mhc_site_post_pre_check(const float* x, const float* f, const float* post_in,
                            const float* comb_in, const float* fn_w, const float* scale,
                            const float* base, int T, int streams, int hidden, int iters,
                            float eps, const float* x_out, const float* pre, const float* post,
                            const float* comb, const float* y) {
  int rc = mhc_site_post_check(x, f, post_in, comb_in, T, streams, hidden, x_out);
  if (rc) return rc;
  if ((rc = mhc_site_pre_check(x_out, fn_w, scale, base, T, streams, hidden, iters, eps, pre,
                               post, comb, y)))
    return rc;
  if (T == 0) return MHC_OK;
  // the next site's outputs against the previous site's inputs
  const size_t S = streams, H = hidden, Tz = T;
  const Span old_in[] = {span(x, Tz * S * H * 4), span(f, Tz * H * 4),
                         span(post_in, Tz * S * 4), span(comb_in, Tz * S * S * 4)};
  const Span out[] = {span(pre, Tz * S * 4), span(post, Tz * S * 4), span(comb, Tz * S * S * 4),
                      span(y, Tz * H * 4)};
  for (const Span& o : out)
    for (const Span& i : old_in)
      if (overlaps(o, i)) return MHC_EOVERLAP;
  return MHC_OK;
}

int mhc_site_post_pre(const float* x, const float* f, const float* post_in, const float* comb_in,
                      const float* fn_w, const float* scale, const float* base, int T,
                      int streams, int hidden, int iters, float eps, float* x_out, float* pre,
                      float* post, float* comb, float* y, void* stream) {
  int rc = mhc_site_post_pre_check(x, f, post_in, comb_in, fn_w, scale, base, T, streams, hidden,
                                   iters, eps, x_out, pre, post, comb, y);
  if (rc || T == 0) return rc;
  return site_post_pre_run(x, f, post_in, comb_in, fn_w, scale, base, T, streams, hidden, iters,
                           eps, x_out, pre, post, comb, y, nullptr,
                           static_cast<hipStream_t>(stream));
}

int mhc_site_post_pre_packed(const float* x, const float* f, const float* post_in,
                             const float* comb_in, const float* fn_w, const float* packed,
                             const float* scale, const float* base, int T, int streams,
                             int hidden, int iters, float eps, float* x_out, float* pre,
                             float* post, float* comb, float* y, void* stream) {
  int rc = mhc_site_post_pre_check(x, f, post_in, comb_in, fn_w, scale, base, T, streams, hidden,
                                   iters, eps, x_out, pre, post, comb, y);
  if (rc || T == 0) return rc;
  const size_t S = streams, H = hidden, Tz = T;
  const Span out[] = {span(x_out, Tz * S * H * 4), span(pre, Tz * S * 4),
                      span(post, Tz * S * 4), span(comb, Tz * S * S * 4), span(y, Tz * H * 4)};
  size_t pb;
  if ((rc = check_packed(packed, streams, hidden, out, 5, &pb))) return rc;
  return site_post_pre_run(x, f, post_in, comb_in, fn_w, scale, base, T, streams, hidden, iters,
                           eps, x_out, pre, post, comb, y, nullptr,
                           static_cast<hipStream_t>(stream), pb ? packed : nullptr);
}

int mhc_site_post_pre_zq8(const float* x, const float* f, const float* post_in,
                          const float* comb_in, const float* fn_w, const float* scale,
                          const float* base, const float* nw, int T, int streams, int hidden,
                          int iters, float eps, float norm_eps, float* x_out, float* pre,
                          float* post, float* comb, float* y, float* z, signed char* q, float* d,
                          void* stream) {
  int rc = mhc_site_post_pre_check(x, f, post_in, comb_in, fn_w, scale, base, T, streams, hidden,
                                   iters, eps, x_out, pre, post, comb, y);
  if (rc) return rc;
  if ((rc = mhc_site_pre_zq8_check(x_out, fn_w, scale, base, nw, T, streams, hidden, iters, eps,
                                   norm_eps, pre, post, comb, y, z, q, d)))
    return rc;
  if (T == 0) return MHC_OK;
  const size_t S = streams, H = hidden, Tz = T;
  const Span old_in[] = {span(x, Tz * S * H * 4), span(f, Tz * H * 4),
                         span(post_in, Tz * S * 4), span(comb_in, Tz * S * S * 4)};
  const Span out[] = {span(z, Tz * H * 4), span(q, Tz * H), span(d, Tz * (H / 32) * 4)};
  for (const Span& o : out)
    for (const Span& i : old_in)
      if (overlaps(o, i)) return MHC_EOVERLAP;
  const mhc::Zq8Out zq{nw, norm_eps, z, q, d};
  return site_post_pre_run(x, f, post_in, comb_in, fn_w, scale, base, T, streams, hidden, iters,
                           eps, x_out, pre, post, comb, y, &zq,
                           static_cast<hipStream_t>(stream));
}

int mhc_site_post(const float* x, const float* f, const float* post, const float* comb, int T,
                  int streams, int hidden, float* x_out, void* stream) {
  int rc = mhc_site_post_check(x, f, post, comb, T, streams, hidden, x_out);
  if (rc || T == 0) return rc;
  if (mhc::launch_post(x, f, post, comb, T, streams, hidden, x_out,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return MHC_EHIP;
  return MHC_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- bandwidth probe
extern "C" {

size_t mhc_probe_sink_floats(size_t bytes) {
  return (size_t)mhc::probe_blocks((long)(bytes / 16));
}

int mhc_bandwidth_probe(const float* src, float* dst, size_t bytes, int copy, void* stream) {
  if (bytes == 0) return MHC_OK;
  int rc;
  if ((rc = check_ptr(src)) || (rc = check_ptr(dst))) return rc;
  if (bytes % 16 != 0) return MHC_EALIGN;
  if (bytes / 16 / 256 >= 0x7fffffffUL) return MHC_EUNSUPPORTED;
  const size_t dst_bytes = copy ? bytes : mhc_probe_sink_floats(bytes) * sizeof(float);
  if (overlaps(span(src, bytes), span(dst, dst_bytes))) return MHC_EOVERLAP;
  return mhc::launch_probe(src, dst, (long)(bytes / 16), copy != 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
             ? MHC_OK
             : MHC_EHIP;
}

}  // extern "C"

// ---------------------------------------------------------------- trunk ends
extern "C" {

int mhc_expand(const float* e, int T, int streams, int hidden, float* x_out, void* stream) {
  int rc = check_shape(T, streams, hidden);
  if (rc || T == 0) return rc;
  if ((rc = check_ptr(e)) || (rc = check_ptr(x_out))) return rc;
  const size_t Tz = T, S = streams, H = hidden;
  if (overlaps(span(x_out, Tz * S * H * 4), span(e, Tz * H * 4))) return MHC_EOVERLAP;
  return mhc::launch_expand(e, T, streams, hidden, x_out, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MHC_OK
             : MHC_EHIP;
}

int mhc_mean(const float* x, int T, int streams, int hidden, float* y_out, void* stream) {
  int rc = check_shape(T, streams, hidden);
  if (rc || T == 0) return rc;
  if ((rc = check_ptr(x)) || (rc = check_ptr(y_out))) return rc;
  const size_t Tz = T, S = streams, H = hidden;
  if (overlaps(span(y_out, Tz * H * 4), span(x, Tz * S * H * 4))) return MHC_EOVERLAP;
  return mhc::launch_mean(x, T, streams, hidden, y_out, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MHC_OK
             : MHC_EHIP;
}

int mhc_head_check(const float* x, const float* fn_w, const float* scale, const float* base,
                   int T, int streams, int hidden, float eps, const float* gates,
                   const float* y) {
  int rc = check_shape(T, streams, hidden);
  if (rc) return rc;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return MHC_EINVAL;
  if (T == 0) return MHC_OK;
  const void* ptrs[] = {x, fn_w, scale, base, gates, y};
  for (const void* p : ptrs)
    if (!p) return MHC_EINVAL;
  for (const void* p : ptrs)
    if ((rc = check_ptr(p))) return rc;
  const size_t S = streams, H = hidden, Tz = T;
  const Span in[] = {span(x, Tz * S * H * 4), span(fn_w, S * S * H * 4), span(scale, 4),
                     span(base, S * 4)};
  const Span out[] = {span(gates, Tz * S * 4), span(y, Tz * H * 4)};
  for (const Span& o : out)
    for (const Span& i : in)
      if (overlaps(o, i)) return MHC_EOVERLAP;
  if (overlaps(out[0], out[1])) return MHC_EOVERLAP;
  return MHC_OK;
}

int mhc_head(const float* x, const float* fn_w, const float* scale, const float* base, int T,
             int streams, int hidden, float eps, float* gates, float* y, void* stream) {
  int rc = mhc_head_check(x, fn_w, scale, base, T, streams, hidden, eps, gates, y);
  if (rc || T == 0) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int S = streams, H = hidden, n = S * H;
  if (T >= kFusedMinTokens && mhc::fused_supported(S, H)) {
    // Large batches with a slab that fits on chip: the site's token tiles with the
    // head's S rows, x read once.
    Scratch sc;
    if ((rc = get_scratch(mhc::fused_head_pack_bytes(S, H), st, &sc))) return rc;
    return mhc::launch_fused_head(x, fn_w, scale, base, T, S, H, eps, gates, y, sc.general,
                                  st) == hipSuccess
               ? MHC_OK
               : MHC_EHIP;
  }
  // Otherwise the site's solo K-split over the same slab, S rows, in passes of at
  // most kExactChunk tokens so that the partials stay bounded.
  const PrePlan p1 = plan_pre(1, S, H);
  const int chunk = T < kExactChunk ? T : kExactChunk;
  Scratch sc;
  if ((rc = get_scratch((size_t)p1.G * chunk * (S + 1) * sizeof(float), st, &sc))) return rc;
  for (int t0 = 0; t0 < T; t0 += chunk) {
    const int tc = T - t0 < chunk ? T - t0 : chunk;
    const float* xc = x + (size_t)t0 * n;
    hipError_t e = mhc::launch_small_partials_rows(xc, fn_w, tc, n, S, p1.G, p1.cpr, sc.general,
                                                   st);
    if (e == hipSuccess)
      e = mhc::launch_head_finish(xc, sc.general, p1.G, tc, S, H, scale, base, eps,
                                  gates + (size_t)t0 * S, y + (size_t)t0 * H, st);
    if (e != hipSuccess) return MHC_EHIP;
  }
  return MHC_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- workspace
// Caller memory carved into 256-byte aligned regions, in this order: the kernel
// scratch (the largest partials / packed weight of any T <= max_tokens), the two stream states, pre, post, comb, y, z, q, d.
namespace {
constexpr size_t kWsAlign = 256;
size_t ws_round(size_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct WsLayout {
  size_t scratch_general, off[10], total;
};

bool ws_layout(int max_tokens, int S, int H, WsLayout* L) {
  if (max_tokens < 1 || max_tokens > kExactChunk || check_shape(max_tokens, S, H) != MHC_OK)
    return false;
  size_t general = 0;
  for (int t = 1; t <= max_tokens; ++t) {
    const size_t b = pre_scratch_bytes(t, S, H);
    if (b > general) general = b;
  }
  const size_t T = max_tokens;
  const size_t sizes[10] = {general, T * S * H * 4, T * S * H * 4, T * S * 4,
                            T * S * 4, T * S * S * 4, T * H * 4, T * H * 4, T * H,
                            T * ((H + 31) / 32) * 4};
  size_t o = 0;
  for (int i = 0; i < 10; ++i) {
    L->off[i] = o;
    o += ws_round(sizes[i]);
  }
  L->scratch_general = general;
  L->total = o;
  return true;
}

int ws_ok(const mhc_workspace* ws, int T) {
  if (!ws || !ws->scratch || (ws->cur != 0 && ws->cur != 1)) return MHC_EINVAL;
  if (T < 0 || T > ws->max_tokens) return MHC_EINVAL;
  return MHC_OK;
}

ScratchSource ws_scratch(const mhc_workspace* ws, Scratch* holder) {
  holder->general = static_cast<float*>(ws->scratch);
  ScratchSource src;
  src.fixed = holder;
  src.bytes = ws->scratch_bytes;
  return src;
}
}  // namespace

extern "C" {

size_t mhc_workspace_bytes(int max_tokens, int streams, int hidden) {
  WsLayout L;
  return ws_layout(max_tokens, streams, hidden, &L) ? L.total : 0;
}

size_t mhc_workspace_struct_bytes(void) { return sizeof(mhc_workspace); }

int mhc_workspace_init(mhc_workspace* ws, void* mem, size_t bytes, int max_tokens, int streams,
                       int hidden) {
  if (!ws || !mem) return MHC_EINVAL;
  WsLayout L;
  if (!ws_layout(max_tokens, streams, hidden, &L)) {
    const int rc = check_shape(max_tokens, streams, hidden);
    return rc ? rc : MHC_EINVAL;
  }
  if (reinterpret_cast<uintptr_t>(mem) % kWsAlign != 0) return MHC_EALIGN;
  if (bytes < L.total) return MHC_EINVAL;
  char* b = static_cast<char*>(mem);
  ws->max_tokens = max_tokens;
  ws->streams = streams;
  ws->hidden = hidden;
  ws->cur = 0;
  ws->scratch = b + L.off[0];
  ws->scratch_bytes = L.scratch_general;
  ws->state[0] = reinterpret_cast<float*>(b + L.off[1]);
  ws->state[1] = reinterpret_cast<float*>(b + L.off[2]);
  ws->pre = reinterpret_cast<float*>(b + L.off[3]);
  ws->post = reinterpret_cast<float*>(b + L.off[4]);
  ws->comb = reinterpret_cast<float*>(b + L.off[5]);
  ws->y = reinterpret_cast<float*>(b + L.off[6]);
  ws->z = reinterpret_cast<float*>(b + L.off[7]);
  ws->q = reinterpret_cast<signed char*>(b + L.off[8]);
  ws->d = reinterpret_cast<float*>(b + L.off[9]);
  return MHC_OK;
}

int mhc_ws_site_pre(mhc_workspace* ws, const float* fn_w, const float* scale, const float* base,
                    int T, int iters, float eps, void* stream) {
  int rc = ws_ok(ws, T);
  if (rc) return rc;
  const float* x = ws->state[ws->cur];
  if ((rc = mhc_site_pre_check(x, fn_w, scale, base, T, ws->streams, ws->hidden, iters, eps,
                               ws->pre, ws->post, ws->comb, ws->y)) ||
      T == 0)
    return rc;
  Scratch holder;
  return site_pre_run(x, fn_w, scale, base, T, ws->streams, ws->hidden, iters, eps, ws->pre,
                      ws->post, ws->comb, ws->y, nullptr, static_cast<hipStream_t>(stream),
                      ws_scratch(ws, &holder));
}

int mhc_ws_site_pre_zq8(mhc_workspace* ws, const float* fn_w, const float* scale,
                        const float* base, const float* nw, int T, int iters, float eps,
                        float norm_eps, void* stream) {
  int rc = ws_ok(ws, T);
  if (rc) return rc;
  const float* x = ws->state[ws->cur];
  if ((rc = mhc_site_pre_zq8_check(x, fn_w, scale, base, nw, T, ws->streams, ws->hidden, iters,
                                   eps, norm_eps, ws->pre, ws->post, ws->comb, ws->y, ws->z,
                                   ws->q, ws->d)) ||
      T == 0)
    return rc;
  const mhc::Zq8Out zq{nw, norm_eps, ws->z, ws->q, ws->d};
  Scratch holder;
  return site_pre_run(x, fn_w, scale, base, T, ws->streams, ws->hidden, iters, eps, ws->pre,
                      ws->post, ws->comb, ws->y, &zq, static_cast<hipStream_t>(stream),
                      ws_scratch(ws, &holder));
}

int mhc_ws_site_post(mhc_workspace* ws, const float* f, int T, void* stream) {
  int rc = ws_ok(ws, T);
  if (rc) return rc;
  const float* x = ws->state[ws->cur];
  float* x_out = ws->state[ws->cur ^ 1];
  if ((rc = mhc_site_post_check(x, f, ws->post, ws->comb, T, ws->streams, ws->hidden, x_out)) ||
      T == 0)
    return rc;  // nothing written: the state stays where it is
  if (mhc::launch_post(x, f, ws->post, ws->comb, T, ws->streams, ws->hidden, x_out,
                       static_cast<hipStream_t>(stream)) != hipSuccess)
    return MHC_EHIP;
  ws->cur ^= 1;
  return MHC_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation pre call
// mhc_site_pre_static: mhc_site_pre with its kernel scratch (the packed weight
// of the token-tiled kernel, or the split reduction's partial sums) in a
// fixed device array of this library instead of the growable library scratch,
// so that the call never allocates, frees or clears device memory.  Every
// process that loads the library holds kStaticScratchBytes of it on each GPU
// it runs on, until the process ends.  The array's host-side name is not a
// device address: its address on each device comes from hipGetSymbolAddress,
// taken once per device (with that device current) and kept.  Nothing in the
// array has to start at zero: the pre chain writes every scratch value before
// reading it.
namespace {
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_static_mu;
void* g_static_ptr[64];

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MHC_EHIP;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MHC_EHIP;
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return MHC_OK;
}
}  // namespace

extern "C" {

int mhc_site_pre_static(const float* x, const float* fn_w, const float* scale, const float* base,
                        int T, int streams, int hidden, int iters, float eps, float* pre,
                        float* post, float* comb, float* y, void* stream) {
  int rc = mhc_site_pre_check(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post,
                              comb, y);
  if (rc || T == 0) return rc;
  const size_t need = pre_scratch_bytes(T, streams, hidden);
  if (need > kStaticScratchBytes) return MHC_EUNSUPPORTED;
  void* p = nullptr;
  if ((rc = static_scratch(&p))) return rc;
  Scratch holder;
  holder.general = static_cast<float*>(p);
  ScratchSource src;
  src.fixed = &holder;
  src.bytes = kStaticScratchBytes;
  return site_pre_run(x, fn_w, scale, base, T, streams, hidden, iters, eps, pre, post, comb, y,
                      nullptr, static_cast<hipStream_t>(stream), src);
}

}  // extern "C"
