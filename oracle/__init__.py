"""fp64 CPU oracle for the mHC site program -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never calls it, and it shares no code with that path.

The arithmetic lives in ``mhc_oracle.c`` (plain C, double precision, sequential
ascending-index sums); this module only compiles it with gcc and marshals numpy
arrays.  What it computes follows the docs.rs page "memra_engine 0.125.0
src/memra_engine/hyper.rs": module documentation (arithmetic contract, memory
layout), the HyperTopology::rows doc comment (row order) and the doc comment of
``post`` (the post mix).  Gate forms and Sinkhorn iteration semantics the page
leaves open are the readings stated in ``mhc_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.c")
_LIB = os.path.join(_HERE, "libmhc_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # A test may point the loader at a deliberately broken build of this
        # same source (the pin-strength check); everything else uses _LIB.
        path = os.environ.get("MHC_ORACLE_TEST_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        lib.mhc_oracle_pre.argtypes = [fp, fp, fp, fp, ctypes.c_long, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                       dp, dp, dp, dp, dp, ctypes.c_int]
        lib.mhc_oracle_pre.restype = ctypes.c_int
        lib.mhc_oracle_post.argtypes = [fp, fp, fp, fp, ctypes.c_long, ctypes.c_int,
                                        ctypes.c_int, dp, ctypes.c_int]
        lib.mhc_oracle_post.restype = ctypes.c_int
        lib.mhc_oracle_sinkhorn.argtypes = [dp, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_double, dp]
        lib.mhc_oracle_sinkhorn.restype = ctypes.c_int
        lib.mhc_oracle_rmsnorm.argtypes = [fp, fp, ctypes.c_long, ctypes.c_int,
                                           ctypes.c_double, dp]
        lib.mhc_oracle_rmsnorm.restype = ctypes.c_int
        lib.mhc_oracle_q8.argtypes = [fp, ctypes.c_long, ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_int8), fp]
        lib.mhc_oracle_q8.restype = ctypes.c_int
        lib.mhc_oracle_expand.argtypes = [fp, ctypes.c_long, ctypes.c_int, ctypes.c_int, fp]
        lib.mhc_oracle_expand.restype = ctypes.c_int
        lib.mhc_oracle_mean.argtypes = [fp, ctypes.c_long, ctypes.c_int, ctypes.c_int, dp]
        lib.mhc_oracle_mean.restype = ctypes.c_int
        lib.mhc_oracle_head.argtypes = [fp, fp, fp, fp, ctypes.c_long, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_double, dp, dp]
        lib.mhc_oracle_head.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def site_pre(x, fn_w, scale, base, iters: int, eps: float, nthreads: int | None = None,
             want_y: bool = True):
    """Oracle pre chain.

    x: float32 [T, S, H]; fn_w: float32 [R, S*H]; scale: float32 [3]; base: float32 [R].
    eps is used exactly as given (pass the float32 value the GPU receives).
    Returns a dict of float64 arrays: mixes [T,R], pre [T,S], post [T,S],
    comb [T,S,S] (comb[t,j,k], j = source stream), y [T,H].
    """
    x, xp = _f32(x)
    if x.ndim != 3:
        raise ValueError("x must be [T, S, H]")
    T, S, H = x.shape
    R = (2 + S) * S
    fn_w, wp = _f32(fn_w)
    scale, sp = _f32(scale)
    base, bp = _f32(base)
    if fn_w.shape != (R, S * H) or scale.shape != (3,) or base.shape != (R,):
        raise ValueError("operand shapes do not match x")
    mixes, mp = _f64(np.empty((T, R)))
    pre, pp = _f64(np.empty((T, S)))
    post, qp = _f64(np.empty((T, S)))
    comb, cp = _f64(np.empty((T, S, S)))
    if want_y:
        y, yp = _f64(np.empty((T, H)))
    else:
        y, yp = None, None
    rc = _load().mhc_oracle_pre(xp, wp, sp, bp, T, S, H, int(iters), float(eps),
                                mp, pp, qp, cp, yp, int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"mhc_oracle_pre rejected its arguments (rc={rc})")
    return {"mixes": mixes, "pre": pre, "post": post, "comb": comb, "y": y}


def site_post(x, f, post, comb, nthreads: int | None = None):
    """Oracle post mix: x' [T,S,H] float64 from x [T,S,H], f [T,H], post [T,S], comb [T,S,S]
    (all float32, taken as given)."""
    x, xp = _f32(x)
    T, S, H = x.shape
    f, fp = _f32(f)
    post, pp = _f32(post)
    comb, cp = _f32(comb)
    if f.shape != (T, H) or post.shape != (T, S) or comb.shape != (T, S, S):
        raise ValueError("operand shapes do not match x")
    out, op = _f64(np.empty((T, S, H)))
    rc = _load().mhc_oracle_post(xp, fp, pp, cp, T, S, H, op,
                                 int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"mhc_oracle_post rejected its arguments (rc={rc})")
    return out


def sinkhorn(z, iters: int, eps: float):
    """comb = Sinkhorn(exp(z)) for one S x S logit block (float64)."""
    z, zp = _f64(z)
    S = z.shape[0]
    if z.shape != (S, S):
        raise ValueError("z must be square")
    out, op = _f64(np.empty((S, S)))
    rc = _load().mhc_oracle_sinkhorn(zp, S, int(iters), float(eps), op)
    if rc != 0:
        raise ValueError(f"mhc_oracle_sinkhorn rejected its arguments (rc={rc})")
    return out


def rmsnorm(y, nw, norm_eps):
    """O8: z = y * nw / sqrt(mean(y^2) + norm_eps) per token, in double precision.
    y [T, H] float32, nw [H] float32 -> z [T, H] float64."""
    lib = _load()
    y, py = _f32(y)
    nw, pn = _f32(nw)
    T, H = y.shape
    z, pz = _f64(np.empty((T, H)))
    if lib.mhc_oracle_rmsnorm(py, pn, T, H, float(norm_eps), pz) != 0:
        raise ValueError("mhc_oracle_rmsnorm rejected its arguments")
    return z


def q8(z):
    """O9: the int8 codes and fp32 block scales of z [T, H] (float32, H % 32 == 0),
    decided in fp32.  Returns (q [T, H] int8, d [T, H/32] float32)."""
    lib = _load()
    z, pz = _f32(z)
    T, H = z.shape
    q = np.empty((T, H), dtype=np.int8)
    d, pd = _f32(np.empty((T, H // 32), dtype=np.float32))
    if lib.mhc_oracle_q8(pz, T, H, q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), pd) != 0:
        raise ValueError("mhc_oracle_q8 rejected its arguments")
    return q, d


def expand(e, S: int):
    """O10: the trunk entry, e [T, H] float32 -> x [T, S, H] float32 (a copy into
    every stream)."""
    lib = _load()
    e, pe = _f32(e)
    T, H = e.shape
    x, px = _f32(np.empty((T, S, H), dtype=np.float32))
    if lib.mhc_oracle_expand(pe, T, S, H, px) != 0:
        raise ValueError("mhc_oracle_expand rejected its arguments")
    return x


def mean(x):
    """O11: the unweighted stream mean, x [T, S, H] float32 -> y [T, H] float64."""
    lib = _load()
    x, px = _f32(x)
    T, S, H = x.shape
    y, py = _f64(np.empty((T, H)))
    if lib.mhc_oracle_mean(px, T, S, H, py) != 0:
        raise ValueError("mhc_oracle_mean rejected its arguments")
    return y


def head(x, fn_h, scale_h, base_h, eps: float):
    """O12: the gated-head exit.  x [T, S, H], fn_h [S, S*H], scale_h [1], base_h [S]
    (float32) -> {"gates": [T, S], "y": [T, H]} in float64."""
    lib = _load()
    x, px = _f32(x)
    T, S, H = x.shape
    fn_h, pw = _f32(fn_h)
    scale_h, ps = _f32(np.asarray(scale_h).reshape(1))
    base_h, pb = _f32(base_h)
    if fn_h.shape != (S, S * H) or base_h.shape != (S,):
        raise ValueError("head weight must be [S, S*H] and bias [S]")
    g, pg = _f64(np.empty((T, S)))
    y, py = _f64(np.empty((T, H)))
    if lib.mhc_oracle_head(px, pw, ps, pb, T, S, H, float(eps), pg, py) != 0:
        raise ValueError("mhc_oracle_head rejected its arguments")
    return {"gates": g, "y": y}
