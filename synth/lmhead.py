"""Seeded synthetic inputs for verification fed by the output projections:
hidden states and projection weights of a target and a draft model that share
a vocabulary (no verification arithmetic here).

The pages pair a target with a smaller model of the same family (page
www.2kiu.com/news/5895634 §4.1, e.g. an 8B target with a 1B draft, both of
vocabulary 128256, widths 4096 and 2048).  No weights are available, so each
projection row j is built from three parts:

* a prior: four coordinates carry a per-token log-frequency bias
  -3 log10(rank_j) / 4 each, rank a seeded permutation of 1..V shared by both
  models, and every hidden state holds 1 there (the Zipf-like shape of the
  streaming workloads);
* a shared part: ``shared`` coordinates where the draft's weights equal the
  target's and the draft's hidden state is the target's plus a little noise
  (what makes the draft a useful predictor of the target);
* a private part: every other coordinate, independent between the models
  (small weights: the noise that makes the draft disagree).

``grid=True`` puts every value on a coarse grid (hidden: multiples of 2^-3
in [-1, 1]; weights: multiples of 2^-6 of magnitude below 4).  Every product
is then an integer multiple of 2^-9 and every partial sum of d <= 8192 of
them is below 2^24 such units, so a float32 accumulation in any order is
exact: device and oracle logits agree bit for bit.  ``grid=False`` draws
plain bfloat16-rounded normals (accumulation rounding then differs).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import f32_to_bf16_bits

NPRIOR = 4
GRID_H = 8.0      # hidden values are multiples of 1 / GRID_H
GRID_W = 64.0     # weight values are multiples of 1 / GRID_W
MAX_WQ = 255      # |weight| * GRID_W <= MAX_WQ (exact in bfloat16)
MAX_HQ = 8        # |hidden| * GRID_H <= MAX_HQ


@dataclass(frozen=True)
class LmWorkload:
    name: str
    B: int
    K: int
    V: int
    d_t: int
    d_d: int
    temperature: float
    top_k: int
    top_p: float
    seed: int
    grid: bool = True
    shared: int = 256        # coordinates shared by the two models
    sigma_h: float = 0.35    # hidden state spread (shared and private parts)
    sigma_s: float = 0.27    # shared weight spread
    sigma_dh: float = 0.1    # draft's deviation from the target's shared hidden part


LM_WORKLOADS: dict[str, LmWorkload] = {}


def _lw(*a, **k):
    w = LmWorkload(*a, **k)
    LM_WORKLOADS[w.name] = w
    return w


# the headline verification shape fed by 8B-class / 1B-class projections
LM_HEADLINE = _lw("lm-b64-k6-v128256-d4096-dd2048-t0.7-topp0.9", 64, 6, 128256, 4096, 2048, 0.7, 0, 0.9, 21)
_lw("lm-b8-k5-v32000-d1024-dd512-t1.0", 8, 5, 32000, 1024, 512, 1.0, 0, 1.0, 22)
_lw("lm-b8-k5-v32000-d1024-dd512-t1.0-normal", 8, 5, 32000, 1024, 512, 1.0, 0, 1.0, 23, grid=False)
_lw("lm-b16-k4-v50001-d512-dd256-topk50", 16, 4, 50001, 512, 256, 1.0, 50, 1.0, 24, shared=128)
_lw("lm-b32-k6-v128256-d4096-dd2048-greedy", 32, 6, 128256, 4096, 2048, 0.0, 0, 1.0, 25)
_lw("lm-b3-k2-v3001-d128-dd64-t0.8-topp0.95", 3, 2, 3001, 128, 64, 0.8, 0, 0.95, 26, shared=32)
_lw("lm-b12-k3-v20000-d256-dd128-t0.9-topk40-topp0.8", 12, 3, 20000, 256, 128, 0.9, 40, 0.8, 27, shared=64)


def _q(x: np.ndarray, scale: float, lim: int) -> np.ndarray:
    """Round to the grid 1/scale and clip to |x| <= lim/scale (float32)."""
    return (np.clip(np.rint(x * scale), -lim, lim) / scale).astype(np.float32)


def _bits(x: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32))


# bfloat16 bit patterns of the private weight codes -PRIV_Q..PRIV_Q (grid)
PRIV_Q = 2
_PRIV_LUT = _bits(np.arange(-PRIV_Q, PRIV_Q + 1, dtype=np.float32) / GRID_W)


def make_lm_inputs(w: LmWorkload) -> dict:
    """Draw one batch.  Returns bfloat16 bit patterns (uint16) hidden_t
    [B, K+1, d_t], weight_t [V, d_t], hidden_d [B, K, d_d], weight_d
    [V, d_d], and float32 uniforms [B, K+1] and draft_u [B, K] (the draft
    sampling uniforms).  Private weights: uniform on the codes
    -PRIV_Q..PRIV_Q of the grid (grid inputs), or normal with the same spread
    (std sqrt(2) / 64)."""
    if w.grid and max(w.d_t, w.d_d) > 8192:
        raise ValueError("grid inputs are exact only up to d = 8192")
    B, K, V = w.B, w.K, w.V
    r = w.shared
    ss = np.random.SeedSequence(w.seed)
    g_w, g_h, g_dw, g_dh, g_u = [np.random.default_rng(s) for s in ss.spawn(5)]
    q = (lambda x, sc, lim: _q(x, sc, lim)) if w.grid else (lambda x, sc, lim: x)

    rank = g_w.permutation(V).astype(np.float64) + 1.0
    prior = _bits(q((-3.0 * np.log10(rank) / NPRIOR).astype(np.float32), GRID_W, MAX_WQ))
    S = _bits(q(g_w.standard_normal((V, r), dtype=np.float32) * w.sigma_s, GRID_W, MAX_WQ))

    def weights(g, d):
        Wm = np.empty((V, d), dtype=np.uint16)
        Wm[:, :NPRIOR] = prior[:, None]
        Wm[:, NPRIOR:NPRIOR + r] = S
        n = d - NPRIOR - r
        if w.grid:
            Wm[:, NPRIOR + r:] = _PRIV_LUT[g.integers(0, 2 * PRIV_Q + 1, (V, n), dtype=np.int8)]
        else:
            Wm[:, NPRIOR + r:] = _bits(g.standard_normal((V, n), dtype=np.float32) * (np.sqrt(2.0) / GRID_W))
        return Wm

    Wt = weights(g_w, w.d_t)
    Wd = weights(g_dw, w.d_d)

    Gh = g_h.standard_normal((B, K + 1, r), dtype=np.float32) * w.sigma_h
    Ht = np.empty((B, K + 1, w.d_t), dtype=np.float32)
    Ht[..., :NPRIOR] = 1.0
    Ht[..., NPRIOR:NPRIOR + r] = Gh
    Ht[..., NPRIOR + r:] = g_h.standard_normal((B, K + 1, w.d_t - NPRIOR - r), dtype=np.float32) * w.sigma_h
    Hd = np.empty((B, K, w.d_d), dtype=np.float32)
    Hd[..., :NPRIOR] = 1.0
    Hd[..., NPRIOR:NPRIOR + r] = Gh[:, :K] + g_dh.standard_normal((B, K, r), dtype=np.float32) * w.sigma_dh
    Hd[..., NPRIOR + r:] = g_dh.standard_normal((B, K, w.d_d - NPRIOR - r), dtype=np.float32) * w.sigma_h
    return dict(
        hidden_t=_bits(q(Ht, GRID_H, MAX_HQ)), weight_t=Wt,
        hidden_d=_bits(q(Hd, GRID_H, MAX_HQ)), weight_d=Wd,
        uniforms=g_u.random((B, K + 1), dtype=np.float32),
        draft_u=g_u.random((B, K), dtype=np.float32),
    )


def grid_hidden_weight(g: np.random.Generator, M: int, V: int, d: int, grid: bool = True):
    """Plain hidden [M, d] and weight [V, d] bit patterns for projection-only
    cases (normal values, on the exact grid when ``grid``)."""
    H = g.standard_normal((M, d), dtype=np.float32) * 0.35
    W = g.standard_normal((V, d), dtype=np.float32) * 0.05
    if grid:
        H, W = _q(H, GRID_H, MAX_HQ), _q(W, GRID_W, MAX_WQ)
    return f32_to_bf16_bits(H), f32_to_bf16_bits(W)
