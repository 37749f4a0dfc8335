"""Checks that pin the oracle to facts that do not come from the oracle itself.

Each ``check_*`` takes the oracle's verification module (``oracle.spec_verify``
or a deliberately broken copy of it) and raises AssertionError when the
module disagrees with the pinned fact.  The tests run them on the real oracle
(they must pass) and on planted-mistake copies (they must fail).

The facts:
* losslessness: the emitted token at every position is distributed as the
  target p (page www.cf-1.com/news/5155685 §2.2; page www.2kiu.com/news/5895634
  §2.2), by a chi-square test and by exact stratified integration;
* the number of accepted drafts is truncated-geometric with parameter
  alpha = sum_x min(p, q) when every position has the same alpha, so the mean
  emitted count is (1 - alpha^(K+1)) / (1 - alpha) (page www.gsyq.cn/news/428210
  §3.2; page www.2kiu.com/news/5895634 §3.1);
* reductions to textbook routines: softmax (scipy), inverse CDF
  (numpy searchsorted), greedy arg-max matching at T = 0, brute-force top-k and
  top-p sets on tiny vocabularies.
"""
from __future__ import annotations

import itertools

import numpy as np
from scipy import special, stats

CHI2_MIN_P = 1e-4


def closed_form(alpha: float, K: int) -> float:
    """Expected tokens emitted per target forward, 1 + alpha + ... + alpha^K."""
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def softmax_rows(logits32: np.ndarray, T: float = 1.0) -> np.ndarray:
    return special.softmax(logits32.astype(np.float64) / T, axis=-1)


def _chi2_pvalue(counts: np.ndarray, probs: np.ndarray) -> float:
    n = counts.sum()
    pos = probs > 0
    assert np.all(counts[~pos] == 0), "a token with zero target probability was emitted"
    if pos.sum() <= 1:
        return 1.0
    exp = probs[pos] * n
    stat = ((counts[pos] - exp) ** 2 / exp).sum()
    return float(stats.chi2.sf(stat, df=pos.sum() - 1))


def tile_rows(rows: np.ndarray, N: int) -> np.ndarray:
    return np.ascontiguousarray(np.broadcast_to(rows, (N,) + rows.shape))


# ---------------------------------------------------------------------------
# losslessness by chi-square
# ---------------------------------------------------------------------------
def lossless_case(case: str, V: int = 8, K: int = 3, seed: int = 11):
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 1.5, (K + 1, V)).astype(np.float32)
    if case == "random":
        dl = rng.normal(0, 1.5, (K, V)).astype(np.float32)
    elif case == "close":
        dl = (tl[:K] + rng.normal(0, 0.4, (K, V))).astype(np.float32)
    elif case == "equal":
        dl = tl[:K].copy()
    elif case == "disjoint":
        h = V // 2
        tl[:, h:] = -np.inf
        dl = rng.normal(0, 1.5, (K, V)).astype(np.float32)
        dl[:, :h] = -np.inf
    elif case == "masked":
        tl[:, ::3] = -np.inf
        dl = rng.normal(0, 1.5, (K, V)).astype(np.float32)
        dl[:, 1::4] = -np.inf
    else:
        raise ValueError(case)
    return tl, dl


def check_lossless(mod, case: str = "random", N: int = 400_000, seed: int = 11):
    V, K = 8, 3
    tl, dl = lossless_case(case, V, K, seed)
    P = softmax_rows(tl)
    Q = softmax_rows(dl)
    rng = np.random.default_rng(seed + 1)
    x = np.stack([rng.choice(V, size=N, p=Q[i]) for i in range(K)], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = mod.verify(tile_rows(tl, N), tile_rows(dl, N), x, u, 1.0, 0, 1.0)
    assert np.all((n >= 0) & (n <= K))
    for j in range(K + 1):
        sel = n >= j
        if sel.sum() < 1000:
            continue
        counts = np.bincount(tok[sel, j], minlength=V)
        pv = _chi2_pvalue(counts, P[j])
        assert pv > CHI2_MIN_P, f"{case}: position {j} emitted tokens differ from p (chi2 p={pv:.2e})"
    if case == "equal":
        assert np.all(n == K), "identical p and q must accept every draft"
    if case == "disjoint":
        assert np.all(n == 0), "disjoint supports must reject the first draft"


def check_lossless_draft_temperature(mod, T: float = 1.0, Td: float = 0.5, N: int = 300_000, seed: int = 21):
    """Drafts sampled from q at their own temperature Td and verified against
    that q: the emitted tokens follow p at T.  Verifying them against q at T
    instead (the draft temperature ignored) breaks the law, which the same
    chi-square detects: returns that p-value for the caller to assert on."""
    V, K = 8, 3
    tl, dl = lossless_case("close", V, K, seed)
    P = softmax_rows(tl, T)
    Qd = softmax_rows(dl, Td)
    rng = np.random.default_rng(seed + 1)
    x = np.stack([rng.choice(V, size=N, p=Qd[i]) for i in range(K)], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = mod.verify(tile_rows(tl, N), tile_rows(dl, N), x, u, T, 0, 1.0, draft_temperature=Td)
    counts = np.bincount(tok[:, 0], minlength=V)
    pv = _chi2_pvalue(counts, P[0])
    assert pv > CHI2_MIN_P, f"draft temperature {Td}: position 0 differs from p (chi2 p={pv:.2e})"
    tok_w, _ = mod.verify(tile_rows(tl, N), tile_rows(dl, N), x, u, T, 0, 1.0)
    return _chi2_pvalue(np.bincount(tok_w[:, 0], minlength=V), P[0])


# ---------------------------------------------------------------------------
# accepted-count distribution at a fixed alpha
# ---------------------------------------------------------------------------
def exact_alpha_rows(V: int, alpha: float, K: int, rng) -> tuple[np.ndarray, np.ndarray]:
    """Logits whose softmaxes satisfy sum_x min(p, q) = alpha at every position:
    p lives on the first half of the vocabulary, r on the second, q = a p + (1-a) r."""
    h = V // 2
    tl = np.full((K + 1, V), -np.inf, dtype=np.float32)
    dl = np.empty((K, V), dtype=np.float32)
    for i in range(K + 1):
        p = rng.dirichlet(np.ones(h))
        tl[i, :h] = np.log(p)
        if i < K:
            r = rng.dirichlet(np.ones(V - h))
            q = np.concatenate([alpha * p, (1 - alpha) * r])
            dl[i] = np.log(q)
    return tl, dl


def check_accept_count(mod, alpha: float, K: int, N: int = 200_000, V: int = 8, seed: int = 5):
    rng = np.random.default_rng(seed)
    tl, dl = exact_alpha_rows(V, alpha, K, rng)
    P = softmax_rows(tl)
    Q = softmax_rows(dl)
    a_true = np.minimum(P[:K], Q).sum(axis=1)  # per position, from the rounded logits
    x = np.stack([rng.choice(V, size=N, p=Q[i]) for i in range(K)], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = mod.verify(tile_rows(tl, N), tile_rows(dl, N), x, u, 1.0, 0, 1.0)
    # truncated geometric: P(n = j) = prod_{i<j} a_i * (1 - a_j), P(n = K) = prod a_i
    probs = np.empty(K + 1)
    run = 1.0
    for j in range(K):
        probs[j] = run * (1 - a_true[j])
        run *= a_true[j]
    probs[K] = run
    counts = np.bincount(n, minlength=K + 1)
    pv = _chi2_pvalue(counts, probs)
    assert pv > CHI2_MIN_P, f"accepted-count distribution is not truncated geometric (p={pv:.2e})"
    mean = (n + 1).mean()
    se = (n + 1).std() / np.sqrt(N)
    E = closed_form(float(a_true.mean()), K)
    assert abs(mean - E) < 4 * se + 1e-6, f"mean emitted {mean:.4f} vs closed form {E:.4f} (se {se:.4f})"
    return mean, se, E


# ---------------------------------------------------------------------------
# exact stratified integration over the uniforms (deterministic)
# ---------------------------------------------------------------------------
def check_exact_integration(mod, seed: int = 3, V: int = 8, N: int = 1 << 16):
    """K = 1.  P(emit j) = sum_x q(x) [A(x) [j = x] + (1 - A(x)) R(j)] where
    A(x) = P_u(accept x) and R the resampling law; both integrals are taken on
    a midpoint grid of N uniforms through the module itself."""
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 1.2, (2, V)).astype(np.float32)
    dl = rng.normal(0, 1.2, (1, V)).astype(np.float32)
    tl[0, 1] = -np.inf  # a token the target never emits at position 0
    P = softmax_rows(tl)
    Q = softmax_rows(dl)
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    below_one = np.float32(1.0) - np.float32(2.0 ** -24)
    phat = np.zeros(V)
    for x in range(V):
        X = np.full((N, 1), x)
        u = np.stack([grid, np.full(N, 0.5, np.float32)], axis=1)
        tok, n = mod.verify(tile_rows(tl, N), tile_rows(dl, N), X, u, 1.0, 0, 1.0)
        A = (n == 1).mean()
        assert abs(A - min(1.0, P[0, x] / Q[0, x])) <= 1.0 / N + 1e-12, "accept probability is not min(1, p/q)"
        phat[x] += Q[0, x] * A
        if A < 1.0:
            u2 = np.stack([np.full(N, below_one), grid], axis=1)
            tok2, n2 = mod.verify(tile_rows(tl, N), tile_rows(dl, N), X, u2, 1.0, 0, 1.0)
            assert np.all(n2 == 0)
            R = np.bincount(tok2[:, 0], minlength=V) / N
            phat += Q[0, x] * (1.0 - A) * R
    err = np.abs(phat - P[0]).max()
    assert err <= 2 * (V + 1) / N, f"emitted law differs from p by {err:.3e}"


# ---------------------------------------------------------------------------
# reductions to textbook routines
# ---------------------------------------------------------------------------
def check_softmax(mod, seed: int = 0):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 3, (16, 1000)).astype(np.float32)
    z[3, :500] = -np.inf
    for T in (1.0, 0.7, 2.5):
        got = mod.filtered_probs(z.astype(np.float64), T, 0, 1.0)
        ref = special.softmax(z.astype(np.float64) / np.float64(np.float32(T)), axis=1)
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-300), f"softmax differs at T={T}"
        lse = special.logsumexp(z.astype(np.float64) / np.float64(np.float32(T)), axis=1)
        j = 7
        assert np.allclose(np.log(got[:, j]), z[:, j] / np.float64(np.float32(T)) - lse, rtol=1e-12)


def check_inverse_cdf(mod, seed: int = 0):
    rng = np.random.default_rng(seed)
    w = rng.random((64, 50))
    w[:, ::4] = 0.0
    w[5] = 0.0
    w[5, 17] = 2.0
    u = rng.random(64)
    u[0] = 0.0
    u[1] = np.nextafter(1.0, 0.0)
    tok, Z = mod.inverse_cdf(w, u)
    C = np.cumsum(w, axis=1)
    for r in range(64):
        ref = np.searchsorted(C[r], u[r] * w[r].sum(), side="right")
        if ref >= w.shape[1]:
            ref = np.flatnonzero(w[r] > 0)[-1]
        assert tok[r] == ref, f"row {r}: inverse cdf {tok[r]} vs searchsorted {ref}"
        assert w[r, tok[r]] > 0, "a zero-weight token was sampled"


def check_greedy(mod, seed: int = 0, N: int = 2000, V: int = 64, K: int = 4):
    rng = np.random.default_rng(seed)
    # bf16-coarse values so that tied maxima are common
    tl = np.round(rng.normal(0, 1, (N, K + 1, V)) * 2).astype(np.float32)
    dl = np.round(rng.normal(0, 1, (N, K, V)) * 2).astype(np.float32)
    amax = np.argmax(tl, axis=2)  # numpy returns the first (lowest-index) maximum
    x = np.where(rng.random((N, K)) < 0.7, amax[:, :K], rng.integers(0, V, (N, K)))
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = mod.verify(tl, dl, x, u, 0.0, 0, 1.0)
    match = x == amax[:, :K]
    n_ref = np.where(match.all(axis=1), K, np.argmin(match, axis=1))
    assert np.array_equal(n, n_ref), "greedy acceptance is not arg-max matching"
    assert np.array_equal(tok[np.arange(N), n], amax[np.arange(N), n_ref]), "greedy token is not the arg-max"


def brute_topk_keep(z: np.ndarray, k: int) -> np.ndarray:
    """Tokens with fewer than k strictly larger values."""
    return np.array([(z > z[j]).sum() < k for j in range(z.shape[0])])


def brute_topp_keep(pi: np.ndarray, top_p: float) -> np.ndarray:
    """Smallest set with mass >= top_p, found by enumerating every subset; among
    the smallest, the one of largest mass; then every token tied with its
    least probable member is added."""
    V = pi.shape[0]
    best = None
    for size in range(1, V + 1):
        cands = []
        for S in itertools.combinations(range(V), size):
            m = sum(pi[list(S)])
            if m >= top_p:
                cands.append((m, S))
        if cands:
            best = max(cands)[1]
            break
    if best is None:
        best = tuple(range(V))
    tau = min(pi[list(best)])
    return pi >= tau


def check_filters(mod, seed: int = 0, trials: int = 300):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        V = int(rng.integers(2, 9))
        z = (np.round(rng.normal(0, 1.5, V) * 2) / 2).astype(np.float32)  # many ties
        if t % 5 == 0:
            z[rng.integers(0, V)] = -np.inf
        if not np.isfinite(z).any():
            z[0] = 0.0
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.integers(0, V + 2))
        tp = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95, 1.0]))
        zz = z.astype(np.float64) / np.float64(np.float32(T))
        keep = np.ones(V, bool)
        if 0 < k < V:
            keep &= brute_topk_keep(zz, k)
        if np.float32(tp) < 1.0:
            pi = np.where(keep, special.softmax(np.where(keep, zz, -np.inf)), 0.0)
            keep &= brute_topp_keep(pi, float(np.float32(tp))) & keep
        ref = np.where(keep, special.softmax(np.where(keep, zz, -np.inf)), 0.0)
        got = mod.filtered_probs(z[None].astype(np.float64), T, k, tp)[0]
        assert np.array_equal(got > 0, ref > 0), f"kept set differs: z={z} T={T} k={k} top_p={tp}"
        assert np.allclose(got, ref, rtol=1e-13, atol=0), "filtered probabilities differ"


def check_zero_weight_never_sampled(mod):
    """Deterministic: u = 0 must not pick a leading zero-probability token,
    and a token with p(x) = 0 is never accepted even at u = 0."""
    V, K = 6, 1
    tl = np.array([[-np.inf, -np.inf, 0.0, 1.0, -np.inf, 0.5]] * 2, dtype=np.float32)
    dl = np.array([[0.0, 0.2, 0.1, -1.0, 0.3, 0.0]], dtype=np.float32)
    u = np.zeros((1, 2), dtype=np.float32)
    tok, n = mod.verify(tl[None], dl[None], np.array([[0]]), u, 1.0, 0, 1.0)
    assert n[0] == 0, "a draft with p(x) = 0 was accepted"
    assert tok[0, 0] in (2, 3, 5), "a zero-weight token was sampled"
    tok, n = mod.verify(tl[None], tl[None, :1], np.array([[3]]), u, 1.0, 0, 1.0)
    assert n[0] == 1 and tok[0, 1] == 2, "bonus at u = 0 must be the first positive-weight token"


# ---------------------------------------------------------------------------
# q supplied as probabilities (the distribution the drafts were drawn from)
# ---------------------------------------------------------------------------
def check_lossless_draft_probs(mod, N: int = 300_000, seed: int = 31):
    """Drafts drawn from arbitrary given distributions q_i (Dirichlet draws,
    one token of each given zero mass), verified with q_i supplied as
    probabilities: every emitted token follows the target p (the same law as
    with logits, page www.cf-1.com/news/5155685 §2.2)."""
    V, K = 8, 3
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 1.5, (K + 1, V)).astype(np.float32)
    P = softmax_rows(tl)
    Q = rng.dirichlet(np.full(V, 0.7), size=K)
    Q[np.arange(K), rng.integers(0, V, K)] = 0.0
    Q = (Q / Q.sum(axis=1, keepdims=True)).astype(np.float32)
    Q64 = Q.astype(np.float64)
    x = np.stack([rng.choice(V, size=N, p=Q64[i] / Q64[i].sum()) for i in range(K)], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = mod.verify(tile_rows(tl, N), None, x, u, 1.0, 0, 1.0, draft_probs=tile_rows(Q, N))
    assert np.all((n >= 0) & (n <= K))
    for j in range(K + 1):
        sel = n >= j
        counts = np.bincount(tok[sel, j], minlength=V)
        pv = _chi2_pvalue(counts, P[j])
        assert pv > CHI2_MIN_P, f"given q: position {j} differs from p (chi2 p={pv:.2e})"


# ---------------------------------------------------------------------------
# the empty residual (reached through a given q at or above p everywhere)
# ---------------------------------------------------------------------------
def empty_residual_case(V: int = 8, K: int = 2, seed: int = 41):
    """Target logits and a given q with q >= p at every token, extra mass on
    one token per position (rows summing past 1): a rejection then leaves
    max(0, p - q) with no mass.  Returns (target logits [K+1, V] float32,
    q [K, V] float32, P [K+1, V] float64 from scipy's softmax, the bumped
    token of each position)."""
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 1.2, (K + 1, V)).astype(np.float32)
    P = softmax_rows(tl)
    bump = rng.integers(0, V, K)
    Q = P[:K] * (1.0 + 1e-6)
    Q[np.arange(K), bump] += 0.3
    Qf = Q.astype(np.float32)
    Qf = np.where(Qf.astype(np.float64) < Q, np.nextafter(Qf, np.float32(np.inf)), Qf)
    assert np.all(Qf.astype(np.float64) > P[:K])
    return tl, Qf, P, bump


def check_empty_residual(mod, N: int = 4096, seed: int = 41):
    """After a rejection whose residual max(0, p - q) is empty, the
    replacement is drawn from p by the inverse CDF: the emitted token is
    searchsorted(cumsum(p), u * sum(p)) with the sampling uniform."""
    V, K = 8, 2
    tl, Qf, P, bump = empty_residual_case(V, K, seed)
    rng = np.random.default_rng(seed + 1)
    x = np.tile(bump, (N, 1))
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = mod.verify(tile_rows(tl, N), None, x, u, 1.0, 0, 1.0, draft_probs=tile_rows(Qf, N))
    rej = n < K
    assert rej.sum() > N // 4, "the case must reject often"
    C = np.cumsum(P, axis=1)
    for r in np.flatnonzero(rej):
        j = n[r]
        ref = int(np.searchsorted(C[j], float(u[r, K]) * P[j].sum(), side="right"))
        ref = min(ref, V - 1)
        assert tok[r, j] == ref, f"empty residual at position {j}: token {tok[r, j]}, p's inverse CDF {ref}"
