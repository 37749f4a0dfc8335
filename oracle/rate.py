"""Many verifications of the same rows: the oracle's decisions for large
numbers of (drafted tokens, uniforms) draws, for measuring near-tie rates.

TEST INFRASTRUCTURE ONLY (see ``oracle/spec_verify.py``).

A near-tie (a decision that two correct implementations can take
differently because its input lies within rounding distance of the boundary)
is a rare event, so its rate is measured over many sequences.  The rows a
sequence is verified on are fixed by its logits; only the drafted tokens and
the uniforms change from one verification to the next.  ``DrawTables`` forms,
once per batch, everything of ``decide`` (oracle/spec_verify.py) that depends
on the rows alone:

* the filtered distributions p_0..p_K and q_0..q_{K-1} (given);
* for each position j < K, the weights of the draw after a rejection at j:
  max(0, p_j - q_j), or p_j when that residual is empty (round-off only);
  for j = K the bonus weights p_K; NaN entries (rows with no distribution)
  count as 0;
* their running sums C and totals Z, formed by the same NumPy calls on the
  same rows as ``inverse_cdf``, so every value equals the one ``decide``
  would compute.

Each verification then takes the steps of ``decide`` in order: the accept
tests u_i * q_i(x_i) < p_i(x_i), the first rejection n, and the draw
token = min{j : u_K * Z < C_j} (``np.searchsorted(C, u_K * Z, "right")``,
the same index for a non-decreasing C), or the last token with positive
weight when round-off leaves none.  tests/test_oracle_rate.py checks the
results against ``verify_given`` element for element.
"""
from __future__ import annotations

import numpy as np


class DrawTables:
    """Precomputed draw tables of one batch.

    P [B, K+1, V] and Q [B, K, V]: float64 filtered probabilities (a row of
    NaN has no distribution), as ``filtered_probs`` returns them.
    """

    def __init__(self, P: np.ndarray, Q: np.ndarray):
        P = np.asarray(P, dtype=np.float64)
        Q = np.asarray(Q, dtype=np.float64)
        B, K1, V = P.shape
        K = K1 - 1
        if Q.shape != (B, K, V):
            raise ValueError("P must be [B, K+1, V] and Q [B, K, V]")
        self.P, self.Q = P, Q
        self.B, self.K, self.V = B, K, V
        self.bad_rows = np.isnan(P).any(axis=(1, 2))
        if K > 0:
            self.bad_rows |= np.isnan(Q).any(axis=(1, 2))
        self.C = np.empty((B, K1, V))
        self.Z = np.empty((B, K1))
        self.last = np.empty((B, K1), dtype=np.int64)
        for j in range(K1):
            if j < K:
                w = np.maximum(0.0, P[:, j] - Q[:, j])
                empty = w.sum(axis=1) == 0.0
                w[empty] = P[empty, j]
            else:
                w = P[:, K].copy()
            w = np.where(np.isnan(w), 0.0, w)
            self.Z[:, j] = w.sum(axis=1)
            self.C[:, j] = np.cumsum(w, axis=1)
            pos = w > 0
            self.last[:, j] = V - 1 - np.argmax(pos[:, ::-1], axis=1)

    def draw_drafts(self, u: np.ndarray) -> np.ndarray:
        """Drafted tokens x[r, b, i] ~ q_i of sequence b by the inverse CDF
        with uniforms u [R, B, K] (float64).  Rows with no distribution give
        token 0 (such sequences are sentinels whatever their drafts)."""
        R = u.shape[0]
        x = np.zeros((R, self.B, self.K), dtype=np.int64)
        for i in range(self.K):
            q = np.where(np.isnan(self.Q[:, i]), 0.0, self.Q[:, i])
            Cq = np.cumsum(q, axis=1)
            Zq = q.sum(axis=1)
            for b in range(self.B):
                if Zq[b] > 0:
                    x[:, b, i] = np.minimum(np.searchsorted(Cq[b], u[:, b, i] * Zq[b], side="right"), self.V - 1)
        return x

    def decide(self, x: np.ndarray, uniforms: np.ndarray, diag: bool = False):
        """The verification of every replica: x [R, B, K] drafted tokens,
        uniforms [R, B, K+1] float32.  Returns (tokens int32 [R, B, K+1],
        n int32 [R, B]) and, with ``diag``, px, qx [R, B, K] and the row n,
        the total Z and the scaled uniform t = u_K * Z of each draw."""
        B, K, V = self.B, self.K, self.V
        x = np.asarray(x).astype(np.int64)
        U = np.asarray(uniforms)
        if U.dtype != np.float32:
            raise TypeError("uniforms must be float32")
        R = x.shape[0]
        if x.shape != (R, B, K) or U.shape != (R, B, K + 1):
            raise ValueError("x must be [R, B, K] and uniforms [R, B, K+1]")
        u = U.astype(np.float64)
        bad = np.broadcast_to(self.bad_rows, (R, B)) | ((x < 0) | (x >= V)).any(axis=2)
        xs = np.clip(x, 0, V - 1)
        bb = np.arange(B)[None, :, None]
        kk = np.arange(K)[None, None, :]
        px = self.P[bb, kk, xs]
        qx = self.Q[bb, kk, xs]
        acc = u[:, :, :K] * qx < px
        n = np.where(acc.all(axis=2), K, np.argmin(acc, axis=2)) if K > 0 else np.zeros((R, B), np.int64)
        Z = self.Z[np.arange(B)[None, :], n]
        t = u[:, :, K] * Z
        tok = np.empty((R, B), dtype=np.int64)
        for b in range(B):
            for j in np.unique(n[:, b]):
                sel = n[:, b] == j
                tok[sel, b] = np.searchsorted(self.C[b, j], t[sel, b], side="right")
        none = tok >= V
        if none.any():
            tok[none] = self.last[np.broadcast_to(np.arange(B), (R, B))[none], n[none]]
        pos = np.arange(K + 1)[None, None, :]
        xp = np.concatenate([x, np.zeros((R, B, 1), np.int64)], axis=2)
        row = np.where(pos < n[..., None], xp, -1)
        row = np.where(pos == n[..., None], tok[..., None], row)
        row[bad] = -1
        out = (row.astype(np.int32), np.where(bad, -1, n).astype(np.int32))
        if diag:
            return out + (dict(px=px, qx=qx, n=n, Z=Z, t=t),)
        return out

    def at_risk(self, x: np.ndarray, uniforms: np.ndarray, eps: float = 1e-5) -> np.ndarray:
        """Informational: replicas whose own decisions lie within eps of a
        boundary (an accept test |u_i - p/q| <= eps up to the first
        rejection, or the draw's u_K * Z within eps * Z of a running sum).
        Returns a bool array [R, B]."""
        tok, n, dg = self.decide(x, uniforms, diag=True)
        u = np.asarray(uniforms).astype(np.float64)
        R, B, K = x.shape
        risk = np.zeros((R, B), dtype=bool)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(dg["qx"] > 0, dg["px"] / dg["qx"], np.inf)
        for i in range(K):
            reached = dg["n"] >= i
            risk |= reached & (np.abs(u[:, :, i] - ratio[:, :, i]) <= eps)
        t, Z, nn = dg["t"], dg["Z"], dg["n"]
        for b in range(B):
            for j in np.unique(nn[:, b]):
                sel = nn[:, b] == j
                C = self.C[b, j]
                idx = np.searchsorted(C, t[sel, b], side="right")
                lo = C[np.clip(idx - 1, 0, self.V - 1)]
                hi = C[np.clip(idx, 0, self.V - 1)]
                tol = eps * Z[sel, b]
                near = ((idx >= 1) & (np.abs(t[sel, b] - lo) <= tol)) | ((idx < self.V) & (np.abs(hi - t[sel, b]) <= tol))
                risk[sel, b] |= near
        return risk & (n >= 0)
