"""Seeded synthetic inputs for the verification step.

This module only draws random numbers and lays them out; it holds none of the
verification arithmetic.  Both the fp64 oracle (through the tests) and the
device path (through the tests and the benchmark) are fed from here.

No trained model is involved: the logits are synthetic rows whose shapes,
vocabulary sizes and acceptance rates follow the workloads the pages discuss
(Llama-2 vocabulary 32000 for the Llama-2-7B / 68M draft pairing on page
www.gsyq.cn/news/428210 §3.3; Llama-3 128256 and Qwen2.5 152064 for the
same-family pairings on page www.2kiu.com/news/5895634 §4.1; K between 4 and 8
as both pages advise).

Row shapes
----------
normal   target logit ~ N(0, s_t^2) i.i.d.
zipf     sorted N(0,1) draws minus 3*log10(rank), scattered through a
         per-row random permutation of the vocabulary
peaked   N(0, s_t^2) plus 8 on exactly round(0.01 V) entries per row, chosen
         uniformly without replacement
draft    target[:, :K] + N(0, s_d^2), in float32; bf16 workloads round the
         float32 target and draft independently to bfloat16 (nearest-even)

Random streams: ``SeedSequence(seed, spawn_key)`` spawns four generators,
for the target, the draft noise, the draft-sampling uniforms and the
verification uniforms, in that order.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    dtype: str            # "f32" or "bf16"
    shape: str            # "normal", "zipf" or "peaked"
    target_sigma: float
    draft_sigma: float
    temperature: float
    top_k: int
    top_p: float
    seed: int
    spawn_key: tuple = ()

    @property
    def rows(self) -> int:
        return self.B * (2 * self.K + 1)

    @property
    def logit_bytes(self) -> int:
        """Bytes of logits one verification pass must read: every target and
        draft logit once (only the target rows at temperature 0)."""
        esz = 2 if self.dtype == "bf16" else 4
        rows = self.B * (self.K + 1) if self.temperature == 0.0 else self.rows
        return rows * self.V * esz

    def with_batch(self, B: int, seed: int | None = None) -> "Workload":
        return replace(self, B=B, seed=self.seed if seed is None else seed)


def _w(name, B, K, V, dtype, shape, ts, ds, T, top_k, top_p, seed, key=()):
    return Workload(name, B, K, V, dtype, shape, ts, ds, T, top_k, top_p, seed, key)


WORKLOADS: dict[str, Workload] = {}
for _wl in [
    _w("b1-k4-v32000-f32-normal", 1, 4, 32000, "f32", "normal", 2.0, 0.5, 1.0, 0, 1.0, 0),
    _w("b8-k5-v32000-f32-zipf", 8, 5, 32000, "f32", "zipf", 1.0, 0.8, 1.0, 0, 1.0, 1),
    _w("b64-k6-v128256-bf16-zipf-t0.7-topp0.9", 64, 6, 128256, "bf16", "zipf", 1.0, 0.5, 0.7, 0, 0.9, 2),
    _w("b256-k8-v152064-f32-peaked-topk50", 256, 8, 152064, "f32", "peaked", 2.5, 0.6, 1.0, 50, 1.0, 3),
    _w("b32-k6-v128256-bf16-normal-s1.5", 32, 6, 128256, "bf16", "normal", 2.0, 1.5, 1.0, 0, 1.0, 4, (0,)),
    _w("b32-k6-v128256-bf16-normal-s1.0", 32, 6, 128256, "bf16", "normal", 2.0, 1.0, 1.0, 0, 1.0, 4, (1,)),
    _w("b32-k6-v128256-bf16-normal-s0.6", 32, 6, 128256, "bf16", "normal", 2.0, 0.6, 1.0, 0, 1.0, 4, (2,)),
    _w("b32-k6-v128256-bf16-normal-s0.4", 32, 6, 128256, "bf16", "normal", 2.0, 0.4, 1.0, 0, 1.0, 4, (3,)),
    _w("b32-k6-v128256-bf16-normal-greedy", 32, 6, 128256, "bf16", "normal", 2.0, 0.6, 0.0, 0, 1.0, 4, (4,)),
]:
    WORKLOADS[_wl.name] = _wl

# the workload the benchmark times by default
HEADLINE = "b64-k6-v128256-bf16-zipf-t0.7-topp0.9"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    uint16 bit patterns.  Inputs are finite here."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rows(g: np.random.Generator, n: int, V: int, shape: str, sigma: float) -> np.ndarray:
    out = np.empty((n, V), dtype=np.float32)
    if shape == "normal":
        for r in range(n):
            out[r] = sigma * g.standard_normal(V, dtype=np.float32)
    elif shape == "zipf":
        bias = (3.0 * np.log10(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
        for r in range(n):
            z = -np.sort(-g.standard_normal(V, dtype=np.float32))
            vals = z - bias
            perm = g.permutation(V)
            out[r, perm] = vals
    elif shape == "peaked":
        m = int(round(0.01 * V))
        for r in range(n):
            row = sigma * g.standard_normal(V, dtype=np.float32)
            hot = g.choice(V, size=m, replace=False)
            row[hot] += np.float32(8.0)
            out[r] = row
    else:
        raise ValueError(shape)
    return out


def make_inputs(w: Workload) -> dict:
    """Draw one batch.  Returns a dict of numpy arrays:

    target   [B, K+1, V] float32, or uint16 bf16 patterns
    draft    [B, K, V]   same dtype
    uniforms [B, K+1]    float32 in [0, 1): accept tests, then the sample
    draft_u  [B, K]      float64 in [0, 1): uniforms for drawing x ~ q
    """
    ss = np.random.SeedSequence(w.seed, spawn_key=w.spawn_key)
    g_t, g_d, g_x, g_u = [np.random.default_rng(s) for s in ss.spawn(4)]
    B, K, V = w.B, w.K, w.V
    tgt = _rows(g_t, B * (K + 1), V, w.shape, w.target_sigma).reshape(B, K + 1, V)
    drf = np.empty((B, K, V), dtype=np.float32)
    for b in range(B):
        for i in range(K):
            drf[b, i] = tgt[b, i] + np.float32(w.draft_sigma) * g_d.standard_normal(V, dtype=np.float32)
    draft_u = g_x.random((B, K))
    uniforms = g_u.random((B, K + 1), dtype=np.float32)
    if w.dtype == "bf16":
        tgt = f32_to_bf16_bits(tgt)
        drf = f32_to_bf16_bits(drf)
    return dict(target=tgt, draft=drf, uniforms=uniforms, draft_u=draft_u)


def ragged_lengths(B: int, k_lo: int, k_hi: int, seed: int) -> np.ndarray:
    """Per-sequence draft lengths, uniform on [k_lo, k_hi] (2 to 10 is the
    range a draft-length controller keeps K in on page
    www.2kiu.com/news/5895634 §4.4)."""
    g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(1000,)))
    return g.integers(k_lo, k_hi + 1, size=B).astype(np.int64)


def pack_ragged(d: dict, ks) -> dict:
    """A ragged batch cut from a rectangular one drawn at K >= max(ks):
    sequence b keeps its first K_b + 1 target rows, its first K_b draft rows
    and draft-sampling uniforms, and its first K_b + 1 uniforms (the last of
    them is its sampling uniform).  Returns

    target   [N + B, V]  sequence b's rows from row cu[b] + b
    draft    [N, V]      its draft rows from row cu[b]
    uniforms [N + B]     float32, from cu[b] + b
    draft_u  [N]         float64, from cu[b]
    cu       [B + 1]     int32 offsets, N = cu[B]
    """
    ks = np.asarray(ks, dtype=np.int64)
    B = ks.shape[0]
    if d["target"].shape[0] != B or np.any(ks < 0) or np.any(ks > d["draft"].shape[1]):
        raise ValueError("need one length in [0, K] per sequence")
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    V = d["target"].shape[2]
    tgt = np.concatenate([d["target"][b, :k + 1] for b, k in enumerate(ks)])
    drf = (np.concatenate([d["draft"][b, :k] for b, k in enumerate(ks)]) if cu[-1] > 0
           else np.zeros((0, V), dtype=d["draft"].dtype))
    uni = np.concatenate([d["uniforms"][b, :k + 1] for b, k in enumerate(ks)]).astype(np.float32)
    du = np.concatenate([d["draft_u"][b, :k] for b, k in enumerate(ks)]) if cu[-1] > 0 else np.zeros(0)
    return dict(target=np.ascontiguousarray(tgt), draft=np.ascontiguousarray(drf), uniforms=uni, draft_u=du, cu=cu)
