"""Plain fp64 CPU oracle for the speculative-sampling verification step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path.

What it computes, step by step, in the pages' notation (p = target
distribution, q = draft distribution, x = drafted token, K = draft length):

* Each drafted token x_i is accepted with probability min(1, p_i(x_i)/q_i(x_i));
  on rejection a replacement is drawn from norm(max(0, p - q)).  Sources: page
  www.cf-1.com/news/5155685 §2.2 (the accept/reject rule and its losslessness)
  and page www.2kiu.com/news/5895634 §2.2 (same rule, residual written (p-q)_+).
* Verification walks the positions in order and stops at the first rejection
  (the first wrong position is rolled back and the target supplies that one
  token): page www.cf-1.com/news/5155685 §2.1, page www.gsyq.cn/news/428210
  §3.1 (steps 3 and 4), page www.2kiu.com/news/5895634 §2.
* When all K drafts are accepted the target's distribution at position K gives
  one more token.  The pages state this only through the expected count
  1 + a + ... + a^K of tokens per target forward (page www.gsyq.cn/news/428210
  §3.2, page www.2kiu.com/news/5895634 §3.1), whose last term is the
  all-accepted case.
* Temperature, top-k and top-p are applied identically to p and q: page
  www.gsyq.cn/news/428210 §3.3 (sampling parameters must be aligned).

Readings where the pages are silent (each is also listed in the design notes):

* Accept test is ``u * q(x) < p(x)`` with u ~ U[0,1): the division-free strict
  form of "accept with probability min(1, p/q)".  p(x) = 0 never accepts.
* Uniforms are one [B, K+1] array: column i < K drives the accept test at
  draft i, column K is the single sampling uniform (residual or bonus).
* Inverse-CDF sampling runs in ascending vocabulary order:
  token = min{j : u*Z < C_j}, C the running sum of the weights, Z their total;
  if round-off leaves no such j, the last token with positive weight is taken.
* An empty residual (Z == 0, reachable only through round-off) falls back to p.
* T == 0 means greedy: p and q are one-hot at their arg-max, ties to the
  lowest index.
* top-k keeps every token whose scaled logit is >= the k-th largest
  (duplicates counted, ties kept); top-p then keeps the smallest
  descending-probability prefix whose mass reaches top_p, again keeping ties
  of its last member; top-k is applied before top-p, both after temperature.
* T and top_p are used at the float32 value the C ABI receives.
* A sequence whose rows include one with every logit -inf (no distribution),
  or whose drafted token lies outside [0, V), yields the sentinel n = -1 and
  tokens all -1.  NaN and +inf logits are rejected with ValueError.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen",
    "filtered_probs",
    "inverse_cdf",
    "sample_tokens",
    "sample",
    "verify",
    "verify_given",
    "decide",
    "verify_ragged",
    "ragged_offsets_ok",
    "verify_one",
]

BF16 = "bf16"
F32 = "f32"
F64 = "f64"  # logits computed by the oracle itself (the language-model head)


# ---------------------------------------------------------------------------
# input widening (exact)
# ---------------------------------------------------------------------------
def widen(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen logits exactly to float64.

    ``dtype == "bf16"``: ``logits`` is a uint16 array of bfloat16 bit patterns;
    the pattern is the upper half of the float32 with the same value, so the
    widening is exact.  ``dtype == "f32"``: a float32 array.  ``dtype ==
    "f64"``: a float64 array, taken as it is.
    """
    if dtype == BF16:
        a = np.asarray(logits)
        if a.dtype != np.uint16:
            raise TypeError("bf16 logits must be given as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        a = np.asarray(logits)
        if a.dtype != np.float32:
            raise TypeError("f32 logits must be a float32 array")
        return a.astype(np.float64)
    if dtype == F64:
        a = np.asarray(logits)
        if a.dtype != np.float64:
            raise TypeError("f64 logits must be a float64 array")
        return a
    raise ValueError(f"unknown dtype {dtype!r}")


def _check_params(temperature, top_k, top_p):
    t = float(np.float32(temperature))
    if not (t >= 0.0):  # also rejects NaN
        raise ValueError("temperature must be >= 0")
    tp = float(np.float32(top_p))
    if not (0.0 < tp <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")
    k = int(top_k)
    if k < 0:
        raise ValueError("top_k must be >= 0")
    return t, k, tp


# ---------------------------------------------------------------------------
# the filtered distribution of one row (A1..A3 of the path)
# ---------------------------------------------------------------------------
def filtered_probs(logits: np.ndarray, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """Probabilities after temperature, top-k and top-p, for every row.

    ``logits``: float64 array [N, V] (exactly widened).  Returns float64 [N, V].
    Rows whose logits are all -inf come back as all-NaN (no distribution);
    callers treat them as bad rows.
    """
    T, k, tp = _check_params(temperature, top_k, top_p)
    z_in = np.asarray(logits, dtype=np.float64)
    if z_in.ndim != 2:
        raise ValueError("logits must be 2-D [rows, V]")
    N, V = z_in.shape
    out = np.zeros((N, V), dtype=np.float64)
    if N == 0:
        return out
    row_max = z_in.max(axis=1)
    dead = row_max == -np.inf
    out[dead] = np.nan
    live = ~dead
    if not live.any():
        return out
    z = z_in[live]
    n = z.shape[0]
    rows = np.arange(n)

    if T == 0.0:
        # greedy: one-hot at the first (lowest-index) maximum
        a = np.argmax(z, axis=1)
        p = np.zeros_like(z)
        p[rows, a] = 1.0
        out[live] = p
        return out

    z = z / T
    keep = np.ones_like(z, dtype=bool)

    if 0 < k < V:
        # k-th largest scaled logit, duplicates counted; every token >= it is kept
        kth = np.partition(z, V - k, axis=1)[:, V - k]
        keep &= z >= kth[:, None]

    if tp < 1.0:
        # softmax over the tokens kept so far
        zk = np.where(keep, z, -np.inf)
        m = zk.max(axis=1, keepdims=True)
        e = np.exp(zk - m)
        pi = e / e.sum(axis=1, keepdims=True)
        # probabilities in descending order and their running mass
        desc = -np.sort(-pi, axis=1)
        mass = np.cumsum(desc, axis=1)
        reach = mass >= tp
        # Some prefix always reaches top_p: the total mass is 1 up to
        # round-off, less than 2 V 2^-53 below it (the quotients e_j / sum e
        # and the two sums each lose at most V 2^-53), while a float32 top_p
        # below 1 is at most 1 - 2^-24; so for any V below 2^28 the whole row
        # reaches it.  The check makes a violation loud instead of silent.
        if not reach[:, -1].all():
            raise AssertionError("cumulative mass below top_p: round-off beyond its bound")
        # first prefix length whose mass reaches top_p
        nstar = np.argmax(reach, axis=1)
        tau = desc[rows, nstar]
        keep &= pi >= tau[:, None]

    zk = np.where(keep, z, -np.inf)
    m = zk.max(axis=1, keepdims=True)
    e = np.exp(zk - m)
    out[live] = e / e.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------------------
# inverse-CDF sampling in vocabulary order (A6)
# ---------------------------------------------------------------------------
def inverse_cdf(w: np.ndarray, u: np.ndarray):
    """Sample one index per row of non-negative weights ``w`` [N, V].

    token = min{j : u*Z < C_j} with C the running sum of w in index order and
    Z = sum(w); if round-off leaves no such j, the last j with w_j > 0.
    Returns (tokens int64 [N], Z float64 [N]).
    """
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    Z = w.sum(axis=1)
    C = np.cumsum(w, axis=1)
    t = u * Z
    hit = t[:, None] < C
    tok = np.argmax(hit, axis=1)
    none = ~hit.any(axis=1)
    if none.any():
        pos = w[none] > 0
        last = w.shape[1] - 1 - np.argmax(pos[:, ::-1], axis=1)
        tok[none] = last
    return tok.astype(np.int64), Z


def sample_tokens(logits: np.ndarray, temperature, top_k, top_p, u: np.ndarray) -> np.ndarray:
    """Draw one token per row from the filtered distribution (used to prepare
    drafted tokens x ~ q for test inputs).  ``u``: float64 uniforms [N]."""
    q = filtered_probs(logits, temperature, top_k, top_p)
    if np.isnan(q).any():
        raise ValueError("cannot sample from a row with no distribution")
    tok, _ = inverse_cdf(q, u)
    return tok


# ---------------------------------------------------------------------------
# the verification step (A4..A7)
# ---------------------------------------------------------------------------
def _check_finite(x: np.ndarray):
    if np.isnan(x).any() or np.isposinf(x).any():
        raise ValueError("NaN or +inf logits are outside the defined input range")


# ---------------------------------------------------------------------------
# the drafting draw: x ~ q, and q(x)
# ---------------------------------------------------------------------------
def sample(logits: np.ndarray, temperature, top_k, top_p, u: np.ndarray, dtype: str = F32):
    """Draw one token per row from the row's filtered distribution, as the
    draft model does for each drafted position (page www.gsyq.cn/news/428210
    section 3.1, step 1: the small model samples the tokens that the large
    model then scores), with the sampling parameters shared with the target
    (section 3.3).  The draw is ``inverse_cdf`` over ``filtered_probs``; the
    probability reported is q(x) of the token drawn, the value the accept
    test of ``verify`` divides by.

    logits [N, V] (float32, or uint16 bf16 patterns with dtype="bf16");
    u [N] uniforms (their float64 values).  Returns (tokens int64 [N],
    prob float64 [N]); a row whose logits are all -inf has no distribution
    and gives token -1 and prob NaN.
    """
    z = widen(logits, dtype)
    if z.ndim != 2:
        raise ValueError("logits must be [rows, V]")
    _check_finite(z)
    N = z.shape[0]
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    if u.shape[0] != N:
        raise ValueError("one uniform per row")
    q = filtered_probs(z, temperature, top_k, top_p)
    live = ~np.isnan(q).any(axis=1)
    tok = np.full(N, -1, dtype=np.int64)
    prob = np.full(N, np.nan)
    if live.any():
        t, _ = inverse_cdf(q[live], u[live])
        tok[live] = t
        prob[live] = q[live][np.arange(t.shape[0]), t]
    return tok, prob


def _draft_probs(draft, dtype, T, k, tp):
    nb, K, V = draft.shape
    if K == 0:
        return np.zeros((nb, 0, V))
    d64 = widen(draft, dtype)
    _check_finite(d64)
    Q = filtered_probs(d64.reshape(nb * K, V), T, k, tp).reshape(nb, K, V)
    if T == 0.0:
        # Greedy: the outcome does not depend on q.  With p one-hot at a and q
        # one-hot at b, x is accepted iff x == a, and a rejection's residual is
        # one-hot at a (or empty, falling back to p); so a draft row with no
        # distribution is given zero mass instead of making the sequence bad.
        Q = np.where(np.isnan(Q), 0.0, Q)
    return Q


def _draft_temperature(T, draft_temperature, k, tp):
    """The temperature of the draft rows: the target's unless the drafts were
    sampled at their own (page www.2kiu.com/news/5895634 section 7: a lower
    draft temperature such as 0.5).  The drafts are then verified against
    the q they were drawn from, which keeps the rule lossless.  Ignored in
    greedy mode; otherwise it must be a valid temperature above 0."""
    if draft_temperature is None or T == 0.0:
        return T
    Td = _check_params(draft_temperature, k, tp)[0]
    if not Td > 0.0:
        raise ValueError("the draft temperature must be > 0 when the target's is")
    return Td


def _given_draft_probs(q, dtype_ok=(np.float32, np.float64)):
    """A draft distribution supplied as probabilities (the q the drafts were
    actually drawn from), widened exactly to float64."""
    q = np.asarray(q)
    if q.dtype not in dtype_ok:
        raise TypeError("draft probabilities must be float32 (or float64)")
    q = q.astype(np.float64)
    if np.isnan(q).any() or np.isinf(q).any() or (q < 0).any():
        raise ValueError("draft probabilities must be finite and >= 0")
    return q


def decide(P: np.ndarray, Q: np.ndarray, x: np.ndarray, uniforms: np.ndarray):
    """The accept tests, the first rejection and the final draw (A4..A7) for
    sequences whose filtered distributions are already formed.

    P [nb, K+1, V] and Q [nb, K, V]: float64 probabilities (a row of NaN has
    no distribution); x [nb, K] drafted tokens; uniforms [nb, K+1] float32.
    Returns (tokens [nb, K+1], n [nb], px [nb, K], qx [nb, K], Z [nb]) with
    the sentinel rows (n = -1, tokens -1, Z NaN) of bad sequences: a row with
    no distribution, or a drafted token outside [0, V).
    """
    nb, K1, V = P.shape
    K = K1 - 1
    x = np.asarray(x).astype(np.int64)
    u = np.asarray(uniforms).astype(np.float64)
    # bad sequences: a row with no distribution, or a drafted token out of range
    bad = np.isnan(P).any(axis=(1, 2))
    if K > 0:
        bad |= np.isnan(Q).any(axis=(1, 2))
    bad |= ((x < 0) | (x >= V)).any(axis=1)
    xs = np.clip(x, 0, V - 1)
    ii = np.arange(nb)[:, None]
    kk = np.arange(K)[None, :]
    px = P[ii, kk, xs]
    qx = Q[ii, kk, xs]
    # accept test at each position
    acc = u[:, :K] * qx < px
    # first rejection
    n = np.where(acc.all(axis=1), K, np.argmin(acc, axis=1)) if K > 0 else np.zeros(nb, np.int64)
    # sampled row: residual at n < K, bonus at n == K
    rows_p = P[np.arange(nb), n]
    w = np.empty((nb, V))
    rej = n < K
    if rej.any():
        nr = n[rej]
        idx = np.flatnonzero(rej)
        res = np.maximum(0.0, P[idx, nr] - Q[idx, nr])
        empty = res.sum(axis=1) == 0.0
        res[empty] = P[idx[empty], nr[empty]]
        w[rej] = res
    w[~rej] = rows_p[~rej]
    w = np.where(np.isnan(w), 0.0, w)
    tok, Z = inverse_cdf(w, u[:, K])
    # emit: accepted drafts, then the sampled token, then -1 padding
    pos = np.arange(K + 1)[None, :]
    row = np.where(pos < n[:, None], np.pad(x, ((0, 0), (0, 1))), -1)
    row = np.where(pos == n[:, None], tok[:, None], row)
    row[bad] = -1
    return row, np.where(bad, -1, n), px, qx, np.where(bad, np.nan, Z)


def verify_given(P, Q, draft_tokens, uniforms, diag: bool = False):
    """Verification of a batch whose filtered distributions are given: P
    [B, K+1, V] (the target's p_0..p_K) and Q [B, K, V] (the draft's q_i, the
    distributions the drafts were drawn from), both float64 probabilities with
    a row of NaN for a row that has no distribution.  The rule is that of
    ``verify``, which is this function applied to the filtered rows of the
    logits.  uniforms: float32 [B, K+1].  Returns as ``verify``.
    """
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    X = np.asarray(draft_tokens).astype(np.int64)
    U = np.asarray(uniforms)
    if U.dtype != np.float32:
        raise TypeError("uniforms must be float32")
    if P.ndim != 3:
        raise ValueError("P must be [B, K+1, V]")
    B, K1, V = P.shape
    K = K1 - 1
    if Q.shape != (B, K, V) or X.shape != (B, K) or U.shape != (B, K + 1):
        raise ValueError("shape mismatch")
    if B == 0:
        e = (np.full((0, K + 1), -1, np.int32), np.full((0,), -1, np.int32))
        return e + (dict(px=np.zeros((0, K)), qx=np.zeros((0, K)), Z=np.zeros(0)),) if diag else e
    row, n, px, qx, Z = decide(P, Q, X, U)
    out = (row.astype(np.int32), n.astype(np.int32))
    return out + (dict(px=px, qx=qx, Z=Z),) if diag else out


def verify(target, draft, draft_tokens, uniforms, temperature, top_k, top_p,
           dtype: str = F32, block: int | None = None, diag: bool = False, draft_temperature=None,
           draft_probs=None):
    """Run verification for a batch.

    target: [B, K+1, V] logits (float32, or uint16 bf16 patterns when
    dtype == "bf16"); draft: [B, K, V]; draft_tokens: [B, K] ints;
    uniforms: float32 [B, K+1].  draft_temperature: the temperature the
    drafts were sampled at, when it differs from the target's.
    draft_probs: [B, K, V] float32 probabilities to use as q directly, in
    place of the draft logits (which are then not read and may be None);
    the rule is unchanged, and lossless for drafts drawn from that q.

    Returns (out_tokens int32 [B, K+1], out_num_accepted int32 [B]) and, when
    ``diag``, a dict with p(x_i), q(x_i) float64 [B, K] and Z float64 [B].
    """
    T, k, tp = _check_params(temperature, top_k, top_p)
    Td = _draft_temperature(T, draft_temperature, k, tp)
    target = np.asarray(target)
    X = np.asarray(draft_tokens).astype(np.int64)
    U = np.asarray(uniforms)
    if U.dtype != np.float32:
        raise TypeError("uniforms must be float32")
    B, K1, V = target.shape
    K = K1 - 1
    if draft_probs is not None:
        draft = _given_draft_probs(draft_probs)
    else:
        draft = np.asarray(draft)
    if draft.shape != (B, K, V) or X.shape != (B, K) or U.shape != (B, K + 1):
        raise ValueError("shape mismatch")
    out_tok = np.full((B, K + 1), -1, dtype=np.int32)
    out_n = np.full((B,), -1, dtype=np.int32)
    px_all = np.full((B, K), np.nan)
    qx_all = np.full((B, K), np.nan)
    Z_all = np.full((B,), np.nan)
    if B == 0:
        return (out_tok, out_n, dict(px=px_all, qx=qx_all, Z=Z_all)) if diag else (out_tok, out_n)
    if block is None:
        block = max(1, int(2**26 // max(1, (2 * K + 1) * V)))
    for s in range(0, B, block):
        e = min(B, s + block)
        nb = e - s
        t64 = widen(target[s:e], dtype)
        _check_finite(t64)
        P = filtered_probs(t64.reshape(nb * (K + 1), V), T, k, tp).reshape(nb, K + 1, V)
        del t64
        if draft_probs is not None:
            Q = draft[s:e]
        else:
            Q = _draft_probs(draft[s:e], dtype, Td, k, tp)
        row, n, px, qx, Z = decide(P, Q, X[s:e], U[s:e])
        out_tok[s:e] = row
        out_n[s:e] = n
        px_all[s:e] = px
        qx_all[s:e] = qx
        Z_all[s:e] = Z
    if diag:
        return out_tok, out_n, dict(px=px_all, qx=qx_all, Z=Z_all)
    return out_tok, out_n


def ragged_offsets_ok(cu, n_draft_rows: int, max_k: int) -> bool:
    """True when ``cu`` [B+1] describes B sequences of 0..max_k drafts that
    tile ``n_draft_rows`` packed draft rows in order: cu[0] = 0, each
    K_b = cu[b+1] - cu[b] in [0, max_k], cu[B] = n_draft_rows."""
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.shape[0] < 1 or cu[0] != 0 or cu[-1] != n_draft_rows:
        return False
    k = np.diff(cu)
    return bool(np.all((k >= 0) & (k <= max_k)))


def verify_ragged(target, draft, draft_tokens, uniforms, cu_num_draft, temperature, top_k, top_p,
                  dtype: str = F32, max_k: int | None = None, diag: bool = False, draft_temperature=None):
    """Verification of a batch whose sequences carry different numbers of drafts.

    The draft length varies from step to step and from input to input when it
    is tuned by the acceptance history (page www.cf-1.com/news/5155685 §2.4,
    page www.2kiu.com/news/5895634 §4.4); each sequence is still verified by
    the rule of ``verify`` with its own K_b = cu[b+1] - cu[b] (0 allowed:
    then the sequence only draws its bonus token).

    Packed layout: target [cu[B] + B, V] (sequence b's K_b + 1 rows from row
    cu[b] + b), draft [cu[B], V] (its K_b rows from row cu[b]), draft_tokens
    [cu[B]] (from cu[b]), uniforms float32 [cu[B] + B] (its K_b accept
    uniforms then its sampling uniform, from cu[b] + b).

    Returns (out_tokens int32 [B, max_k + 1] padded with -1, out_num_accepted
    int32 [B]); with ``diag`` also px, qx float64 [cu[B]] and Z float64 [B].
    max_k defaults to the largest K_b.  Offsets that do not describe such a
    packing (cu[0] != 0, a K_b outside [0, max_k], cu[B] != the number of
    draft rows) make every sequence a sentinel (n = -1, tokens -1), as a
    device that only sees the offsets at run time reports them.
    """
    target = np.asarray(target)
    draft = np.asarray(draft)
    X = np.asarray(draft_tokens).astype(np.int64).reshape(-1)
    U = np.asarray(uniforms)
    cu = np.asarray(cu_num_draft, dtype=np.int64).reshape(-1)
    if U.dtype != np.float32:
        raise TypeError("uniforms must be float32")
    if cu.shape[0] < 1:
        raise ValueError("cu_num_draft needs B + 1 entries")
    B = cu.shape[0] - 1
    ND = draft.shape[0]
    if target.ndim != 2 or draft.ndim != 2 or target.shape[0] != ND + B or draft.shape[1] != target.shape[1]:
        raise ValueError("target must be [n_draft + B, V] and draft [n_draft, V]")
    if X.shape[0] != ND or U.reshape(-1).shape[0] != ND + B:
        raise ValueError("draft_tokens must be [n_draft] and uniforms [n_draft + B]")
    U = U.reshape(-1)
    ks = np.diff(cu)
    if max_k is None:
        max_k = int(max(0, ks.max(initial=0)))
    if max_k < 0:
        raise ValueError("max_k must be >= 0")
    out_tok = np.full((B, max_k + 1), -1, dtype=np.int32)
    out_n = np.full((B,), -1, dtype=np.int32)
    px_all = np.full((ND,), np.nan)
    qx_all = np.full((ND,), np.nan)
    Z_all = np.full((B,), np.nan)
    if ragged_offsets_ok(cu, ND, max_k):
        # sequences of equal length verified together (the rule is per sequence)
        for K in np.unique(ks):
            K = int(K)
            bs = np.flatnonzero(ks == K)
            t_idx = (cu[bs] + bs)[:, None] + np.arange(K + 1)[None, :]
            d_idx = cu[bs][:, None] + np.arange(K)[None, :]
            tok, n, d = verify(target[t_idx], draft[d_idx], X[d_idx], U[t_idx], temperature, top_k, top_p,
                               dtype=dtype, diag=True, draft_temperature=draft_temperature)
            out_tok[bs, :K + 1] = tok
            out_n[bs] = n
            px_all[d_idx] = d["px"]
            qx_all[d_idx] = d["qx"]
            Z_all[bs] = d["Z"]
    if diag:
        return out_tok, out_n, dict(px=px_all, qx=qx_all, Z=Z_all)
    return out_tok, out_n


def verify_one(target_b, draft_b, x_b, u_b, temperature, top_k, top_p, dtype: str = F32, draft_temperature=None,
               draft_probs_b=None):
    """All intermediate values for one sequence (used to classify a mismatch).

    Returns a dict: P [K+1, V], Q [K, V], px, qx, accept [K], n, w [V],
    Z, C [V], token.  The arithmetic is exactly that of ``verify``.
    draft_probs_b: [K, V] probabilities used as q (draft_b is then ignored).
    """
    dp = None if draft_probs_b is None else np.asarray(draft_probs_b)[None]
    out_tok, out_n = verify(target_b[None], None if dp is not None else draft_b[None], np.asarray(x_b)[None],
                            np.asarray(u_b, dtype=np.float32)[None],
                            temperature, top_k, top_p, dtype=dtype, draft_temperature=draft_temperature,
                            draft_probs=dp)
    T, k, tp = _check_params(temperature, top_k, top_p)
    Td = _draft_temperature(T, draft_temperature, k, tp)
    K = np.asarray(x_b).shape[0]
    V = target_b.shape[-1]
    P = filtered_probs(widen(target_b, dtype), T, k, tp)
    if dp is not None:
        Q = _given_draft_probs(dp)[0]
    else:
        Q = _draft_probs(np.asarray(draft_b)[None], dtype, Td, k, tp)[0]
    x = np.clip(np.asarray(x_b, dtype=np.int64), 0, V - 1)
    u = np.asarray(u_b, dtype=np.float32).astype(np.float64)
    px = P[np.arange(K), x]
    qx = Q[np.arange(K), x]
    accept = u[:K] * qx < px
    n = int(out_n[0])
    if n < 0:
        return dict(P=P, Q=Q, px=px, qx=qx, accept=accept, n=n, w=None, Z=None, C=None,
                    token=-1, out_tokens=out_tok[0])
    if n < K:
        w = np.maximum(0.0, P[n] - Q[n])
        if w.sum() == 0.0:
            w = P[n].copy()
    else:
        w = P[K].copy()
    return dict(P=P, Q=Q, px=px, qx=qx, accept=accept, n=n, w=w, Z=w.sum(),
                C=np.cumsum(w), token=int(out_tok[0, n]), out_tokens=out_tok[0])
