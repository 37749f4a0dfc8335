"""Classify a mismatch between a device result and the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/spec_verify.py``).

Every decision of the verification step compares a continuous quantity with
a uniform or with a threshold: the accept test compares u with p(x)/q(x), the
inverse CDF compares u*Z with the running sums C_j, and top-p compares a
running mass with top_p.  Two correct implementations that round differently
can only disagree when one of these comparisons is within rounding distance
of its boundary.  A sequence is *flagged* (an admissible near-tie) when the
device and the oracle disagree and every decision on the device's path that
differs from the oracle's is one the oracle itself would take if the
uniform, or top_p, moved by at most ``eps`` (absolute for u and top_p,
relative to Z for the sampling comparison); the draw on that path is then
held to the oracle's draw with the same uniform.  Any other disagreement is
a *failure*.  This is the gate's one reading: u within eps of p/q, u*Z within
eps*Z of a running sum, top_p within eps of the cumulative mass.
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


def _draw_weights(P, Q, n, K):
    """Weights of the draw that follows a first rejection at n (n < K: the
    residual, or p_n when it is empty) or the acceptance of all K drafts
    (n == K: p_K)."""
    if n < K:
        w = np.maximum(0.0, P[n] - Q[n])
        if w.sum() == 0.0:
            w = P[n].copy()
    else:
        w = P[K].copy()
    return np.where(np.isnan(w), 0.0, w)


def _perturbed_top_p(top_p, eps):
    """The top_p values within eps of top_p (absolute) that the classifier
    also admits: a kept set at the boundary of the mass cut."""
    tp = float(np.float32(top_p))
    return [] if tp >= 1.0 else [tp - eps, min(1.0, tp + eps)]


def classify(target_b, draft_b, x_b, u_b, temperature, top_k, top_p, dtype,
             dev_tokens_b, dev_n_b, eps: float = 1e-5, draft_temperature=None, draft_probs_b=None):
    """Return (verdict, reason) for one sequence.  verdict in {match, flagged, fail}.
    draft_probs_b: the sequence's q given as probabilities [K, V] (draft_b unused).

    The device's outputs fix the path it took: accepts at positions
    0..n-1, a rejection at n (n < K), and a draw at n.  Every accept decision
    on that path must be the oracle's own, or lie within eps of its boundary
    (|u_i - p_i(x_i)/q_i(x_i)| <= eps, or flipped by moving top_p by at most
    eps).  The drawn token must then be the oracle's draw on that path (the
    residual at n, or the bonus row), with the same uniform, or within eps*Z
    of it (its interval [C_{g-1}, C_g) meets [uZ - eps Z, uZ + eps Z]), with
    the rows at top_p or at top_p moved by eps.  Any near-tie taken makes the
    sequence flagged; anything else that differs is a failure.
    """
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
    if dev_n > K or np.any(dev_tokens_b[dev_n + 1:] != -1):
        return FAIL, "malformed device row"
    # the accepted prefix must be the drafted tokens themselves
    if not np.array_equal(dev_tokens_b[:dev_n], np.asarray(x_b, dtype=np.int64)[:dev_n]):
        return FAIL, "accepted prefix differs from the drafted tokens"
    tps = _perturbed_top_p(top_p, eps)
    reasons = []

    # accept decisions along the device's path
    for i in range(min(dev_n + 1, K)):
        dev_acc = i < dev_n
        if dev_acc == bool(ref["accept"][i]):
            continue
        px, qx = float(ref["px"][i]), float(ref["qx"][i])
        if qx > 0.0 and abs(u[i] - px / qx) <= eps:
            reasons.append(f"accept near-tie at position {i}: u={u[i]:.9g} p/q={px / qx:.9g}")
            continue
        flipped = False
        for tp2 in tps:
            P, Q = _rows_with_top_p(target_b, draft_b, temperature, top_k, tp2, dtype, i, draft_temperature,
                                    draft_probs_b)
            x = int(x_b[i])
            if bool(u[i] * Q[x] < P[x]) == dev_acc:
                flipped = True
                break
        if not flipped:
            return FAIL, f"accept decision differs at position {i}: u={u[i]:.9g} p={px:.9g} q={qx:.9g}"
        reasons.append(f"top-p boundary near-tie in the accept test at position {i}")

    # the draw at the device's n, with the oracle's rows
    n = dev_n
    g = int(dev_tokens_b[n])
    w = _draw_weights(ref["P"], ref["Q"], n, K)
    C = np.cumsum(w)
    tok_ref = int(np.searchsorted(C, u[K] * w.sum(), side="right"))
    if tok_ref >= w.shape[0]:
        tok_ref = int(np.flatnonzero(w > 0)[-1]) if (w > 0).any() else -1
    if g != tok_ref:
        if _token_reachable(w, u[K], g, eps):
            reasons.append(f"sampling near-tie at position {n}: token {g} vs oracle {tok_ref}")
        else:
            hit = False
            for tp2 in tps:
                P2, Q2 = _rows_with_top_p(target_b, draft_b, temperature, top_k, tp2, dtype, n, draft_temperature,
                                          draft_probs_b)
                # the draw's row at top_p moved: position 0 of a one-position path
                w2 = _draw_weights(P2[None], Q2[None], 0, 1) if n < K else _draw_weights(P2[None], None, 0, 0)
                if _token_reachable(w2, u[K], g, eps):
                    hit = True
                    break
            if not hit:
                return FAIL, f"sampled token differs at position {n}: device {g} oracle {tok_ref}"
            reasons.append(f"top-p boundary near-tie in the sampled row {n}")
    if not reasons:
        # same path and same token but some other entry differs
        return FAIL, "device row differs from the oracle's on the same path"
    return FLAGGED, "; ".join(reasons)


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
    top_p moved by eps (absolute, as in ``classify``: a kept set at its
    boundary)."""
    if got == ref:
        return MATCH
    tps = [top_p] + _perturbed_top_p(top_p, eps)
    for tp in tps:
        q = filtered_probs(np.asarray(row, dtype=np.float64)[None], temperature, top_k, tp)[0]
        if not np.isnan(q).any() and _token_reachable(q, float(u), int(got), eps):
            return FLAGGED
    return FAIL
