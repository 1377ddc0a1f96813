"""Seeded synthetic inputs for the mHC site program.

This module is shared by the oracle-side tests and the GPU-side tests/bench and
therefore holds none of the method's arithmetic: only shapes, seeds and random
draws.  Shapes follow the production site of the pages (streams=4,
n_embd=4096, 20 Sinkhorn iterations, eps=1e-6; hc_fused_gate.rs module
constants), their 128-wide mini fixture, and a wider 8-stream site.  There is
no public dataset behind the pages' timings (they were taken while serving a
model whose weights are not available), so these draws stand in for it.

Draw recipe: numpy PCG64 seeded with SeedSequence([20261202, cfg, T]); five
children spawned in the order x, fn_w, scale, base, f; draws in float64 cast
to float32; U[a,b) is ``uniform(a, b)``; N(0, v) is ``standard_normal() *
sqrt(v)`` (the second parameter is the variance).
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED = 20261202


@dataclasses.dataclass(frozen=True)
class SiteConfig:
    name: str
    cfg: int          # index used in the seed
    T: int
    S: int
    H: int
    iters: int = 20
    eps: float = 1e-6

    @property
    def R(self) -> int:
        return (2 + self.S) * self.S

    @property
    def n(self) -> int:
        return self.S * self.H


CONFIGS = {
    # tiny: T=4, 4 streams, hidden 128 (the pages' 128-wide mini fixture)
    "tiny": SiteConfig("tiny", 0, 4, 4, 128),
    # decode site at the production shape
    "decode": SiteConfig("decode", 1, 1, 4, 4096),
    # verify-batch sites
    "verify4": SiteConfig("verify4", 2, 4, 4, 4096),
    "verify8": SiteConfig("verify8", 2, 8, 4, 4096),
    # prefill chunk, 256 MiB of stream state
    "prefill": SiteConfig("prefill", 3, 4096, 4, 4096),
    # wider site: 8 streams (80 mixes rows, 8x8 comb), hidden 7168
    "wide": SiteConfig("wide", 4, 1024, 8, 7168),
}


def make_site(cfg: SiteConfig, T: int | None = None, seed: int = SEED):
    """Draw one site's operands.  Returns a dict of float32 numpy arrays:
    x [T,S,H], fn_w [R, S*H], scale [3], base [R], f [T,H]."""
    T = cfg.T if T is None else T
    S, H = cfg.S, cfg.H
    R, n = cfg.R, cfg.n
    ss = np.random.SeedSequence([seed, cfg.cfg, T])
    gx, gw, gs, gb, gf = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(5)]
    x = gx.uniform(-1.0, 1.0, size=(T, S, H)).astype(np.float32)
    fn_w = (gw.standard_normal(size=(R, n)) * np.sqrt(1.0 / n)).astype(np.float32)
    scale = gs.uniform(0.5, 1.5, size=3).astype(np.float32)
    base = (gb.standard_normal(size=R) * np.sqrt(0.1)).astype(np.float32)
    f = gf.uniform(-1.0, 1.0, size=(T, H)).astype(np.float32)
    return {"x": x, "fn_w": fn_w, "scale": scale, "base": base, "f": f}


def make_random_shape(T: int, S: int, H: int, seed: int):
    """Same distributions as the configs, for an arbitrary (T, S, H)."""
    cfg = SiteConfig("adhoc", 1000 + S * 131 + H, T, S, H)
    return make_site(cfg, T=T, seed=seed)


def make_norm_weight(H: int, seed: int = SEED):
    """The branch-input norm weight nw [H] (float32): 1 + U[-0.5, 0.5), seeded by
    SeedSequence([seed, 77, H]); the pages' gate draws it as one plus a small
    random vector."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77, H])))
    return (1.0 + g.uniform(-0.5, 0.5, size=H)).astype(np.float32)
