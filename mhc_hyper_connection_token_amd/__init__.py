"""MI355X (gfx950) mHC site library: Python binding of libmhc.so.

The two calls mirror the C ABI in ``include/mhc.h``:

* :func:`site_pre`  -> ``mhc_site_pre``  (mixes GEMV, RMS rescale, gates, Sinkhorn, collapse)
* :func:`site_post` -> ``mhc_site_post`` (post mix)

This module only marshals arguments: it checks that the operands are contiguous
float32 CUDA (HIP) tensors of matching shapes, allocates outputs with
``torch.empty`` when none are given, and passes raw device pointers and the
current HIP stream to the library.  Every step of the computation runs in the
library's kernels.  There is no fallback: if ``libmhc.so`` is missing the calls
raise.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["site_pre", "site_post", "site_pre_zq8", "site_pre_check", "site_post_check",
           "site_pre_zq8_check", "site_post_pre", "site_post_pre_check", "expand", "mean",
           "head", "head_check", "bandwidth_probe", "packed_weight_bytes", "pack_weight",
           "site_pre_scratch_bytes",
           "Workspace",
           "workspace_bytes", "load_library", "MhcError", "LIB_PATH", "EXPORTED_SYMBOLS",
           "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmhc.so")

EXPORTED_SYMBOLS = ("mhc_site_pre", "mhc_site_post", "mhc_site_pre_exact", "mhc_site_pre_zq8",
                    "mhc_site_pre_check", "mhc_site_post_check", "mhc_site_pre_zq8_check",
                    "mhc_workspace_bytes", "mhc_workspace_struct_bytes", "mhc_workspace_init",
                    "mhc_ws_site_pre", "mhc_ws_site_pre_zq8", "mhc_ws_site_post",
                    "mhc_expand", "mhc_mean", "mhc_head", "mhc_head_check",
                    "mhc_site_post_pre", "mhc_site_post_pre_zq8", "mhc_site_post_pre_check",
                    "mhc_status_string", "mhc_probe_sink_floats", "mhc_bandwidth_probe",
                    "mhc_packed_weight_bytes", "mhc_pack_weight", "mhc_site_pre_packed",
                    "mhc_site_post_pre_packed", "mhc_site_pre_scratch_bytes",
                    "mhc_site_pre_static")

STATUS = {0: "MHC_OK", 1: "MHC_EINVAL", 2: "MHC_EALIGN", 3: "MHC_EUNSUPPORTED",
          4: "MHC_EHIP", 5: "MHC_EOVERLAP", 6: "MHC_ECAPTURE"}

_lib = None


class MhcError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libmhc.so from this package directory (built by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first "
                           "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fl, i = ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.mhc_site_pre.argtypes = [vp, vp, vp, vp, i, i, i, i, fl, vp, vp, vp, vp, vp]
    lib.mhc_site_pre.restype = i
    lib.mhc_site_pre_exact.argtypes = [vp, vp, vp, vp, i, i, i, i, fl, vp, vp, vp, vp, vp]
    lib.mhc_site_pre_exact.restype = i
    lib.mhc_site_post.argtypes = [vp, vp, vp, vp, i, i, i, vp, vp]
    lib.mhc_site_post.restype = i
    lib.mhc_site_pre_check.argtypes = [vp, vp, vp, vp, i, i, i, i, fl, vp, vp, vp, vp]
    lib.mhc_site_pre_check.restype = i
    lib.mhc_site_post_check.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.mhc_site_post_check.restype = i
    lib.mhc_site_pre_zq8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, fl, fl, vp, vp, vp, vp,
                                     vp, vp, vp, vp]
    lib.mhc_site_pre_zq8.restype = i
    lib.mhc_site_pre_zq8_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, fl, fl, vp, vp, vp,
                                           vp, vp, vp, vp]
    lib.mhc_site_pre_zq8_check.restype = i
    lib.mhc_status_string.argtypes = [i]
    lib.mhc_status_string.restype = ctypes.c_char_p
    sz, wsp = ctypes.c_size_t, ctypes.POINTER(_WsStruct)
    lib.mhc_workspace_bytes.argtypes = [i, i, i]
    lib.mhc_workspace_bytes.restype = sz
    lib.mhc_workspace_struct_bytes.argtypes = []
    lib.mhc_workspace_struct_bytes.restype = sz
    lib.mhc_workspace_init.argtypes = [wsp, vp, sz, i, i, i]
    lib.mhc_workspace_init.restype = i
    lib.mhc_ws_site_pre.argtypes = [wsp, vp, vp, vp, i, i, fl, vp]
    lib.mhc_ws_site_pre.restype = i
    lib.mhc_ws_site_pre_zq8.argtypes = [wsp, vp, vp, vp, vp, i, i, fl, fl, vp]
    lib.mhc_ws_site_pre_zq8.restype = i
    lib.mhc_ws_site_post.argtypes = [wsp, vp, i, vp]
    lib.mhc_ws_site_post.restype = i
    lib.mhc_site_post_pre.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, fl, vp, vp, vp,
                                      vp, vp, vp]
    lib.mhc_site_post_pre.restype = i
    lib.mhc_site_post_pre_zq8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, fl, fl,
                                          vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mhc_site_post_pre_zq8.restype = i
    lib.mhc_site_post_pre_check.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, fl, vp, vp,
                                            vp, vp, vp]
    lib.mhc_site_post_pre_check.restype = i
    lib.mhc_expand.argtypes = [vp, i, i, i, vp, vp]
    lib.mhc_expand.restype = i
    lib.mhc_mean.argtypes = [vp, i, i, i, vp, vp]
    lib.mhc_mean.restype = i
    lib.mhc_head.argtypes = [vp, vp, vp, vp, i, i, i, fl, vp, vp, vp]
    lib.mhc_head.restype = i
    lib.mhc_head_check.argtypes = [vp, vp, vp, vp, i, i, i, fl, vp, vp]
    lib.mhc_head_check.restype = i
    lib.mhc_packed_weight_bytes.argtypes = [i, i]
    lib.mhc_packed_weight_bytes.restype = sz
    lib.mhc_pack_weight.argtypes = [vp, i, i, vp, vp]
    lib.mhc_pack_weight.restype = i
    lib.mhc_site_pre_packed.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, fl, vp, vp, vp, vp, vp]
    lib.mhc_site_pre_packed.restype = i
    lib.mhc_site_post_pre_packed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, fl, vp,
                                             vp, vp, vp, vp, vp]
    lib.mhc_site_post_pre_packed.restype = i
    lib.mhc_site_pre_static.argtypes = [vp, vp, vp, vp, i, i, i, i, fl, vp, vp, vp, vp, vp]
    lib.mhc_site_pre_static.restype = i
    lib.mhc_site_pre_scratch_bytes.argtypes = [i, i, i]
    lib.mhc_site_pre_scratch_bytes.restype = sz
    lib.mhc_probe_sink_floats.argtypes = [sz]
    lib.mhc_probe_sink_floats.restype = sz
    lib.mhc_bandwidth_probe.argtypes = [vp, vp, sz, i, vp]
    lib.mhc_bandwidth_probe.restype = i
    if lib.mhc_workspace_struct_bytes() != ctypes.sizeof(_WsStruct):
        raise RuntimeError("mhc_workspace layout of the library and the binding differ")
    _lib = lib
    return lib


class _WsStruct(ctypes.Structure):
    """Mirror of struct mhc_workspace (include/mhc.h)."""
    _fields_ = [("max_tokens", ctypes.c_int), ("streams", ctypes.c_int),
                ("hidden", ctypes.c_int), ("cur", ctypes.c_int),
                ("state", ctypes.c_void_p * 2), ("pre", ctypes.c_void_p),
                ("post", ctypes.c_void_p), ("comb", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("z", ctypes.c_void_p), ("q", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("scratch", ctypes.c_void_p), ("scratch_bytes", ctypes.c_size_t)]


def _status_text(lib, rc: int) -> str:
    return lib.mhc_status_string(rc).decode()


def _dev(t, name, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def site_pre(x, fn_w, scale, base, iters: int, eps: float, *, out=None, stream=None,
             exact: bool = False, packed=None, static_scratch: bool = False):
    """Pre half of a site.  x: [T,S,H]; fn_w: [(2+S)*S, S*H]; scale: [3]; base: [(2+S)*S].
    Returns (pre [T,S], post [T,S], comb [T,S,S], y [T,H]); `out` may supply that tuple.
    exact=True calls mhc_site_pre_exact (every row bit-identical to a solo T=1 call);
    packed (from pack_weight) calls mhc_site_pre_packed (same results, no per-call pack);
    static_scratch=True calls mhc_site_pre_static (the library's fixed scratch array,
    no device allocation by the library; pass `out` to allocate nothing at all)."""
    if (exact, packed is not None, static_scratch).count(True) > 1:
        raise ValueError("exact, packed and static_scratch are separate calls")
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    R = (2 + S) * S
    px = _dev(x, "x")
    pw = _dev(fn_w, "fn_w", (R, S * H))
    ps = _dev(scale, "scale", (3,))
    pb = _dev(base, "base", (R,))
    if out is None:
        out = (torch.empty((T, S), device=x.device, dtype=torch.float32),
               torch.empty((T, S), device=x.device, dtype=torch.float32),
               torch.empty((T, S, S), device=x.device, dtype=torch.float32),
               torch.empty((T, H), device=x.device, dtype=torch.float32))
    pre, post, comb, y = out
    ptrs = (_dev(pre, "pre", (T, S)), _dev(post, "post", (T, S)),
            _dev(comb, "comb", (T, S, S)), _dev(y, "y", (T, H)))
    if packed is not None:
        nbytes = int(lib.mhc_packed_weight_bytes(S, H))
        pk = _dev(packed, "packed", (nbytes // 4,)) if nbytes else None
        rc = lib.mhc_site_pre_packed(px, pw, pk, ps, pb, T, S, H, int(iters), float(eps), *ptrs,
                                     _stream_handle(stream))
        if rc != 0:
            raise MhcError("mhc_site_pre_packed", rc, _status_text(lib, rc))
        return out
    if exact:
        fn, name = lib.mhc_site_pre_exact, "mhc_site_pre_exact"
    elif static_scratch:
        fn, name = lib.mhc_site_pre_static, "mhc_site_pre_static"
    else:
        fn, name = lib.mhc_site_pre, "mhc_site_pre"
    rc = fn(px, pw, ps, pb, T, S, H, int(iters), float(eps), *ptrs, _stream_handle(stream))
    if rc != 0:
        raise MhcError(name, rc, _status_text(lib, rc))
    return out


def site_pre_scratch_bytes(T: int, streams: int, hidden: int) -> int:
    """Bytes of library scratch a site_pre call of this shape needs (0: rejected shape)."""
    return int(load_library().mhc_site_pre_scratch_bytes(T, streams, hidden))


def packed_weight_bytes(streams: int, hidden: int) -> int:
    """Bytes of a site weight's packed form (0: the shape has none)."""
    return int(load_library().mhc_packed_weight_bytes(streams, hidden))


def pack_weight(fn_w, streams: int, hidden: int, *, out=None, stream=None):
    """Pack a site weight fn_w [(2+S)*S, S*H] once for site_pre(..., packed=...).
    Returns a float32 GPU tensor of packed_weight_bytes(S, H) / 4 floats."""
    import torch
    lib = load_library()
    S, H = int(streams), int(hidden)
    R = (2 + S) * S
    nbytes = int(lib.mhc_packed_weight_bytes(S, H))
    if nbytes == 0:
        raise MhcError("mhc_pack_weight", 3, _status_text(lib, 3))
    pw = _dev(fn_w, "fn_w", (R, S * H))
    if out is None:
        out = torch.empty(nbytes // 4, device=fn_w.device, dtype=torch.float32)
    rc = lib.mhc_pack_weight(pw, S, H, _dev(out, "packed", (nbytes // 4,)), _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_pack_weight", rc, _status_text(lib, rc))
    return out


def site_pre_zq8(x, fn_w, scale, base, nw, iters: int, eps: float, norm_eps: float = 1e-5, *,
                 out=None, stream=None):
    """Pre half of a site plus the branch-input epilogue (RMS norm of y with weight nw,
    then q8 codes).  Returns (pre, post, comb, y, z [T,H] f32, q [T,H] int8, d [T,H/32] f32);
    `out` may supply that tuple."""
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    R = (2 + S) * S
    px = _dev(x, "x")
    pw = _dev(fn_w, "fn_w", (R, S * H))
    ps = _dev(scale, "scale", (3,))
    pb = _dev(base, "base", (R,))
    pn = _dev(nw, "nw", (H,))
    if out is None:
        e = lambda s, dt=torch.float32: torch.empty(s, device=x.device, dtype=dt)  # noqa: E731
        out = (e((T, S)), e((T, S)), e((T, S, S)), e((T, H)), e((T, H)), e((T, H), torch.int8),
               e((T, H // 32)))
    pre, post, comb, y, z, q, d = out
    if q.dtype != torch.int8 or not q.is_cuda or not q.is_contiguous() or tuple(q.shape) != (T, H):
        raise ValueError("q must be a contiguous int8 GPU tensor of shape [T, H]")
    ptrs = (_dev(pre, "pre", (T, S)), _dev(post, "post", (T, S)), _dev(comb, "comb", (T, S, S)),
            _dev(y, "y", (T, H)), _dev(z, "z", (T, H)), q.data_ptr(), _dev(d, "d", (T, H // 32)))
    rc = lib.mhc_site_pre_zq8(px, pw, ps, pb, pn, T, S, H, int(iters), float(eps),
                              float(norm_eps), *ptrs, _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_site_pre_zq8", rc, _status_text(lib, rc))
    return out


def site_post(x, f, post, comb, *, out=None, stream=None):
    """Post half of a site: x' [T,S,H] from x [T,S,H], f [T,H], post [T,S], comb [T,S,S]."""
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    px = _dev(x, "x")
    pf = _dev(f, "f", (T, H))
    pp = _dev(post, "post", (T, S))
    pc = _dev(comb, "comb", (T, S, S))
    if out is None:
        out = torch.empty((T, S, H), device=x.device, dtype=torch.float32)
    po = _dev(out, "out", (T, S, H))
    rc = lib.mhc_site_post(px, pf, pp, pc, T, S, H, po, _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_site_post", rc, _status_text(lib, rc))
    return out


def site_pre_check(x_ptr, fn_w_ptr, scale_ptr, base_ptr, T, S, H, iters, eps,
                   pre_ptr, post_ptr, comb_ptr, y_ptr) -> int:
    """The library's host-side argument check on raw addresses (no HIP call)."""
    lib = load_library()
    return lib.mhc_site_pre_check(x_ptr, fn_w_ptr, scale_ptr, base_ptr, T, S, H, iters,
                                  float(eps), pre_ptr, post_ptr, comb_ptr, y_ptr)


def site_post_check(x_ptr, f_ptr, post_ptr, comb_ptr, T, S, H, out_ptr) -> int:
    lib = load_library()
    return lib.mhc_site_post_check(x_ptr, f_ptr, post_ptr, comb_ptr, T, S, H, out_ptr)


def site_pre_zq8_check(x_ptr, fn_w_ptr, scale_ptr, base_ptr, nw_ptr, T, S, H, iters, eps,
                       norm_eps, pre_ptr, post_ptr, comb_ptr, y_ptr, z_ptr, q_ptr, d_ptr) -> int:
    lib = load_library()
    return lib.mhc_site_pre_zq8_check(x_ptr, fn_w_ptr, scale_ptr, base_ptr, nw_ptr, T, S, H,
                                      iters, float(eps), float(norm_eps), pre_ptr, post_ptr,
                                      comb_ptr, y_ptr, z_ptr, q_ptr, d_ptr)


def site_post_pre(x, f, post, comb, fn_w, scale, base, iters: int, eps: float, *, nw=None,
                  norm_eps: float = 1e-5, out=None, stream=None, packed=None):
    """The post half of a site (x, f, post, comb) followed by the pre half of the
    next site (fn_w, scale, base) on its output.  Returns (x_out, pre, post, comb, y),
    plus (z, q, d) when the norm weight nw of the next site's epilogue is given;
    `out` may supply that tuple.  packed (from pack_weight, without nw) calls
    mhc_site_post_pre_packed."""
    if packed is not None and nw is not None:
        raise ValueError("the packed call has no epilogue")
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    R = (2 + S) * S
    px = _dev(x, "x")
    pf = _dev(f, "f", (T, H))
    ppi = _dev(post, "post", (T, S))
    pci = _dev(comb, "comb", (T, S, S))
    pw = _dev(fn_w, "fn_w", (R, S * H))
    ps = _dev(scale, "scale", (3,))
    pb = _dev(base, "base", (R,))
    if out is None:
        e = lambda s, dt=torch.float32: torch.empty(s, device=x.device, dtype=dt)  # noqa: E731
        out = (e((T, S, H)), e((T, S)), e((T, S)), e((T, S, S)), e((T, H)))
        if nw is not None:
            out = out + (e((T, H)), e((T, H), torch.int8), e((T, H // 32)))
    ptrs = [_dev(out[0], "x_out", (T, S, H)), _dev(out[1], "pre", (T, S)),
            _dev(out[2], "post", (T, S)), _dev(out[3], "comb", (T, S, S)),
            _dev(out[4], "y", (T, H))]
    st = _stream_handle(stream)
    if packed is not None:
        nbytes = int(lib.mhc_packed_weight_bytes(S, H))
        pk = _dev(packed, "packed", (nbytes // 4,)) if nbytes else None
        rc = lib.mhc_site_post_pre_packed(px, pf, ppi, pci, pw, pk, ps, pb, T, S, H, int(iters),
                                          float(eps), *ptrs, st)
        name = "mhc_site_post_pre_packed"
    elif nw is None:
        rc = lib.mhc_site_post_pre(px, pf, ppi, pci, pw, ps, pb, T, S, H, int(iters),
                                   float(eps), *ptrs, st)
        name = "mhc_site_post_pre"
    else:
        z, q, d = out[5], out[6], out[7]
        if q.dtype != torch.int8 or not q.is_cuda or not q.is_contiguous():
            raise ValueError("q must be a contiguous int8 GPU tensor")
        rc = lib.mhc_site_post_pre_zq8(px, pf, ppi, pci, pw, ps, pb, _dev(nw, "nw", (H,)), T, S,
                                       H, int(iters), float(eps), float(norm_eps), *ptrs,
                                       _dev(z, "z", (T, H)), q.data_ptr(),
                                       _dev(d, "d", (T, H // 32)), st)
        name = "mhc_site_post_pre_zq8"
    if rc != 0:
        raise MhcError(name, rc, _status_text(lib, rc))
    return out


def site_post_pre_check(x_ptr, f_ptr, post_ptr, comb_ptr, fn_w_ptr, scale_ptr, base_ptr, T, S,
                        H, iters, eps, x_out_ptr, pre2_ptr, post2_ptr, comb2_ptr, y2_ptr) -> int:
    """The library's host-side argument check of mhc_site_post_pre on raw addresses."""
    lib = load_library()
    return lib.mhc_site_post_pre_check(x_ptr, f_ptr, post_ptr, comb_ptr, fn_w_ptr, scale_ptr,
                                       base_ptr, T, S, H, iters, float(eps), x_out_ptr, pre2_ptr,
                                       post2_ptr, comb2_ptr, y2_ptr)


def expand(e, streams: int, *, out=None, stream=None):
    """Trunk entry: e [T, H] -> x [T, S, H] (a copy of e in every stream)."""
    import torch
    lib = load_library()
    if e.dim() != 2:
        raise ValueError("e must be [T, H]")
    T, H = e.shape
    pe = _dev(e, "e")
    if out is None:
        out = torch.empty((T, streams, H), device=e.device, dtype=torch.float32)
    po = _dev(out, "out", (T, streams, H))
    rc = lib.mhc_expand(pe, T, streams, H, po, _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_expand", rc, _status_text(lib, rc))
    return out


def mean(x, *, out=None, stream=None):
    """Trunk exit (unweighted): x [T, S, H] -> y [T, H], the mean over the streams."""
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    px = _dev(x, "x")
    if out is None:
        out = torch.empty((T, H), device=x.device, dtype=torch.float32)
    po = _dev(out, "out", (T, H))
    rc = lib.mhc_mean(px, T, S, H, po, _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_mean", rc, _status_text(lib, rc))
    return out


def head(x, fn_w, scale, base, eps: float, *, out=None, stream=None):
    """Trunk exit (gated head): x [T, S, H], fn_w [S, S*H], scale [1], base [S] ->
    (gates [T, S], y [T, H]); `out` may supply that pair."""
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    px = _dev(x, "x")
    pw = _dev(fn_w, "fn_w", (S, S * H))
    ps = _dev(scale, "scale", (1,))
    pb = _dev(base, "base", (S,))
    if out is None:
        out = (torch.empty((T, S), device=x.device, dtype=torch.float32),
               torch.empty((T, H), device=x.device, dtype=torch.float32))
    g, y = out
    rc = lib.mhc_head(px, pw, ps, pb, T, S, H, float(eps), _dev(g, "gates", (T, S)),
                      _dev(y, "y", (T, H)), _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_head", rc, _status_text(lib, rc))
    return out


def bandwidth_probe(src, dst, copy: bool, *, stream=None):
    """Pure-stream probe (mhc_bandwidth_probe): copy src into dst (same size), or
    read src and write block sums into dst (probe_sink_floats(src) floats)."""
    lib = load_library()
    ps = _dev(src, "src")
    want = src.numel() if copy else int(lib.mhc_probe_sink_floats(src.numel() * 4))
    if dst.numel() != want:
        raise ValueError(f"dst must hold {want} floats")
    pd = _dev(dst, "dst")
    rc = lib.mhc_bandwidth_probe(ps, pd, src.numel() * 4, int(bool(copy)), _stream_handle(stream))
    if rc != 0:
        raise MhcError("mhc_bandwidth_probe", rc, _status_text(lib, rc))
    return dst


def head_check(x_ptr, fn_w_ptr, scale_ptr, base_ptr, T, S, H, eps, gates_ptr, y_ptr) -> int:
    """The library's host-side argument check of mhc_head on raw addresses."""
    lib = load_library()
    return lib.mhc_head_check(x_ptr, fn_w_ptr, scale_ptr, base_ptr, T, S, H, float(eps),
                              gates_ptr, y_ptr)


def workspace_bytes(max_tokens: int, streams: int, hidden: int) -> int:
    """Device bytes a workspace of this shape needs (0 for an invalid shape)."""
    return int(load_library().mhc_workspace_bytes(max_tokens, streams, hidden))


class Workspace:
    """A persistent site workspace (mhc_workspace_init and the mhc_ws_* calls).

    The device memory is one torch uint8 buffer owned by this object; the library
    carves it and never allocates on the workspace path.  Tensor views of the
    regions: ``state`` (the current stream state, [max_tokens, S, H], writable),
    ``pre``, ``post``, ``comb``, ``y``, ``z``, ``q``, ``d`` (max_tokens rows; a call
    with T tokens writes the first T)."""

    def __init__(self, max_tokens: int, streams: int, hidden: int, device=None):
        import torch
        lib = load_library()
        nbytes = int(lib.mhc_workspace_bytes(max_tokens, streams, hidden))
        if nbytes == 0:
            raise ValueError(f"invalid workspace shape ({max_tokens}, {streams}, {hidden})")
        self._mem = torch.empty(nbytes + 256, dtype=torch.uint8,
                                device=device if device is not None else "cuda")
        base = self._mem.data_ptr()
        self._base = base
        off = (-base) % 256
        self._ws = _WsStruct()
        rc = lib.mhc_workspace_init(ctypes.byref(self._ws), base + off, nbytes, max_tokens,
                                    streams, hidden)
        if rc != 0:
            raise MhcError("mhc_workspace_init", rc, _status_text(lib, rc))
        self.max_tokens, self.streams, self.hidden = max_tokens, streams, hidden
        T, S, H = max_tokens, streams, hidden
        f32, i8 = torch.float32, torch.int8
        w = self._ws
        self._states = (self._view(w.state[0], (T, S, H), f32),
                        self._view(w.state[1], (T, S, H), f32))
        self.pre = self._view(w.pre, (T, S), f32)
        self.post = self._view(w.post, (T, S), f32)
        self.comb = self._view(w.comb, (T, S, S), f32)
        self.y = self._view(w.y, (T, H), f32)
        self.z = self._view(w.z, (T, H), f32)
        self.q = self._view(w.q, (T, H), i8)
        self.d = self._view(w.d, (T, (H + 31) // 32), f32)

    def _view(self, ptr, shape, dtype):
        import torch
        itemsize = torch.empty((), dtype=dtype).element_size()
        count = 1
        for s in shape:
            count *= s
        o = ptr - self._base
        return self._mem[o:o + count * itemsize].view(dtype).view(shape)

    @property
    def cur(self) -> int:
        return int(self._ws.cur)

    @property
    def state(self):
        """The current stream state [max_tokens, S, H] (state[cur])."""
        return self._states[self._ws.cur]

    def site_pre(self, fn_w, scale, base, iters: int, eps: float, T: int = None, stream=None):
        lib = load_library()
        T = self.max_tokens if T is None else T
        S, H = self.streams, self.hidden
        R = (2 + S) * S
        rc = lib.mhc_ws_site_pre(ctypes.byref(self._ws), _dev(fn_w, "fn_w", (R, S * H)),
                                 _dev(scale, "scale", (3,)), _dev(base, "base", (R,)), T,
                                 int(iters), float(eps), _stream_handle(stream))
        if rc != 0:
            raise MhcError("mhc_ws_site_pre", rc, _status_text(lib, rc))

    def site_pre_zq8(self, fn_w, scale, base, nw, iters: int, eps: float,
                     norm_eps: float = 1e-5, T: int = None, stream=None):
        lib = load_library()
        T = self.max_tokens if T is None else T
        S, H = self.streams, self.hidden
        R = (2 + S) * S
        rc = lib.mhc_ws_site_pre_zq8(ctypes.byref(self._ws), _dev(fn_w, "fn_w", (R, S * H)),
                                     _dev(scale, "scale", (3,)), _dev(base, "base", (R,)),
                                     _dev(nw, "nw", (H,)), T, int(iters), float(eps),
                                     float(norm_eps), _stream_handle(stream))
        if rc != 0:
            raise MhcError("mhc_ws_site_pre_zq8", rc, _status_text(lib, rc))

    def site_post(self, f, T: int = None, stream=None):
        lib = load_library()
        T = self.max_tokens if T is None else T
        if not (f.is_cuda and f.dtype.is_floating_point and f.is_contiguous()):
            raise ValueError("f must be a contiguous float32 GPU tensor")
        if f.dim() != 2 or f.shape[0] < T or f.shape[1] != self.hidden:
            raise ValueError(f"f must be [>= {T}, {self.hidden}]")
        rc = lib.mhc_ws_site_post(ctypes.byref(self._ws), _dev(f, "f"), T,
                                  _stream_handle(stream))
        if rc != 0:
            raise MhcError("mhc_ws_site_post", rc, _status_text(lib, rc))
