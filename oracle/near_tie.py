"""Classify a mismatch between a device result and the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/spec_verify.py``).

Every decision of the verification step compares a continuous quantity with
a uniform or with a threshold: the accept test compares u with p(x)/q(x), the
inverse CDF compares u*Z with the running sums C_j, and top-p compares a
running mass with top_p.  Two correct implementations that round differently
can only disagree when one of these comparisons is within rounding distance
of its boundary.  A sequence is *flagged* (an admissible near-tie) when the
device and the oracle disagree and the first disagreeing decision is one the
oracle itself would take if the uniform, or top_p, moved by at most
``eps`` (relative to Z for the sampling comparison).  Any other disagreement
is a *failure*.
"""
from __future__ import annotations

import numpy as np

from .spec_verify import filtered_probs, verify_one, widen

MATCH = "match"
FLAGGED = "flagged"
FAIL = "fail"


def _sample_interval(C, g):
    lo = 0.0 if g == 0 else float(C[g - 1])
    return lo, float(C[g])


def _token_reachable(w, u, g, eps):
    """True when token g's CDF interval [C_{g-1}, C_g) meets [uZ - eps Z, uZ + eps Z]."""
    if w is None or g < 0 or g >= w.shape[0] or w[g] <= 0.0:
        return False
    C = np.cumsum(w)
    Z = float(w.sum())
    t = u * Z
    lo, hi = _sample_interval(C, g)
    return hi > t - eps * Z and lo <= t + eps * Z


def _rows_with_top_p(target_b, draft_b, T, top_k, top_p, dtype, pos, Td=None, qprobs_b=None):
    t = widen(target_b[pos:pos + 1], dtype)
    P = filtered_probs(t, T, top_k, top_p)[0]
    if qprobs_b is not None:
        # a q given as probabilities does not depend on the filters
        Q = np.asarray(qprobs_b[pos], dtype=np.float64) if pos < qprobs_b.shape[0] else None
    elif pos < draft_b.shape[0]:
        Q = filtered_probs(widen(draft_b[pos:pos + 1], dtype), T if Td is None or T == 0.0 else Td, top_k, top_p)[0]
    else:
        Q = None
    return P, Q


def classify(target_b, draft_b, x_b, u_b, temperature, top_k, top_p, dtype,
             dev_tokens_b, dev_n_b, eps: float = 1e-5, draft_temperature=None, draft_probs_b=None):
    """Return (verdict, reason) for one sequence.  verdict in {match, flagged, fail}.
    draft_probs_b: the sequence's q given as probabilities [K, V] (draft_b unused)."""
    ref = verify_one(target_b, draft_b, x_b, u_b, temperature, top_k, top_p, dtype=dtype,
                     draft_temperature=draft_temperature, draft_probs_b=draft_probs_b)
    dev_tokens_b = np.asarray(dev_tokens_b).astype(np.int64)
    dev_n = int(dev_n_b)
    if dev_n == ref["n"] and np.array_equal(dev_tokens_b, ref["out_tokens"].astype(np.int64)):
        return MATCH, ""
    if ref["n"] < 0 or dev_n < 0:
        return FAIL, f"sentinel mismatch: oracle n={ref['n']} device n={dev_n}"
    K = np.asarray(x_b).shape[0]
    u = np.asarray(u_b, dtype=np.float32).astype(np.float64)
    # the accepted prefix must be the drafted tokens themselves
    m = min(ref["n"], dev_n)
    if not np.array_equal(dev_tokens_b[:m], np.asarray(x_b, dtype=np.int64)[:m]):
        return FAIL, "accepted prefix differs from the drafted tokens"
    if dev_n > K or np.any(dev_tokens_b[dev_n + 1:] != -1):
        return FAIL, "malformed device row"
    tp_perturb = [] if float(np.float32(top_p)) >= 1.0 else [top_p - eps, min(1.0, top_p + eps)]

    if ref["n"] != dev_n:
        i0 = m  # first position whose accept decision differs
        px, qx = float(ref["px"][i0]), float(ref["qx"][i0])
        if qx > 0.0 and abs(u[i0] - px / qx) <= eps:
            return FLAGGED, f"accept near-tie at position {i0}: u={u[i0]:.9g} p/q={px / qx:.9g}"
        for tp2 in tp_perturb:
            P, Q = _rows_with_top_p(target_b, draft_b, temperature, top_k, tp2, dtype, i0, draft_temperature,
                                    draft_probs_b)
            x = int(x_b[i0])
            if (u[i0] * Q[x] < P[x]) != bool(ref["accept"][i0]):
                return FLAGGED, f"top-p boundary near-tie at position {i0}"
        return FAIL, f"accept decision differs at position {i0}: u={u[i0]:.9g} p={px:.9g} q={qx:.9g}"

    n = dev_n
    g = int(dev_tokens_b[n])
    if _token_reachable(ref["w"], u[K], g, eps):
        return FLAGGED, f"sampling near-tie at position {n}: token {g} vs oracle {ref['token']}"
    for tp2 in tp_perturb:
        P, Q = _rows_with_top_p(target_b, draft_b, temperature, top_k, tp2, dtype, n, draft_temperature,
                                draft_probs_b)
        if n < K:
            w = np.maximum(0.0, P - Q)
            if w.sum() == 0.0:
                w = P
        else:
            w = P
        if _token_reachable(w, u[K], g, eps):
            return FLAGGED, f"top-p boundary near-tie in the sampled row {n}"
    return FAIL, f"sampled token differs at position {n}: device {g} oracle {ref['token']}"


def at_risk(ref: dict, u_b, eps: float = 1e-5) -> bool:
    """Informational: the oracle's own decisions for this sequence lie within
    eps of a boundary (accept tests up to n, or the sampling comparison)."""
    if ref["n"] < 0:
        return False
    u = np.asarray(u_b, dtype=np.float32).astype(np.float64)
    K = ref["qx"].shape[0]
    last = min(ref["n"], K - 1)
    for i in range(0, last + 1):
        qx = ref["qx"][i]
        if qx > 0 and abs(u[i] - ref["px"][i] / qx) <= eps:
            return True
    C, Z = ref["C"], ref["Z"]
    t = u[K] * Z
    j = int(np.searchsorted(C, t, side="right"))
    for jj in (j - 1, j):
        if 0 <= jj < C.shape[0] and abs(C[jj] - t) <= eps * Z:
            return True
    return False


def classify_sample(row: np.ndarray, temperature, top_k, top_p, u: float, got: int, ref: int,
                    eps: float = 1e-5) -> str:
    """Classify a device draw ``got`` against the oracle's ``ref`` for one row
    (widened logits [V]) drawn with uniform ``u``: flagged when the oracle
    itself could draw ``got`` with u moved by at most eps*Z, under top_p or
    top_p moved by a relative eps (a kept set at its boundary)."""
    if got == ref:
        return MATCH
    tps = [top_p]
    if top_p < 1.0:
        tps += [top_p * (1.0 - eps), min(1.0, top_p * (1.0 + eps))]
    for tp in tps:
        q = filtered_probs(np.asarray(row, dtype=np.float64)[None], temperature, top_k, tp)[0]
        if not np.isnan(q).any() and _token_reachable(q, float(u), int(got), eps):
            return FLAGGED
    return FAIL
