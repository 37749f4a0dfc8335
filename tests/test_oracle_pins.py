"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import spec_verify as ov
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked_values():
    with open(os.path.join(GOLDEN, "worked_values.json")) as f:
        return json.load(f)["entries"]


@pytest.mark.parametrize("e", _worked_values(), ids=lambda e: f"{e['source'].split('/')[0]}-a{e['alpha']}-K{e['K']}")
def test_worked_values_closed_form(e):
    """The closed form reproduces every page value marked 'agrees' at the page's
    two-decimal rounding, and each 'erratum' entry is a genuine disagreement
    whose correct value is recorded in the fixture."""
    E = pins.closed_form(e["alpha"], e["K"])
    if e["status"] == "agrees":
        assert abs(E - e["page_value"]) <= 0.005 + 1e-12, (E, e)
    else:
        assert abs(E - e["page_value"]) > 0.01, (E, e)
        assert abs(E - e["closed_form"]) < 5e-5, (E, e)


def test_erratum_095_is_closed_form_at_k3():
    # the value printed for K=5 at alpha 0.8 is the closed form at K=3
    assert abs(pins.closed_form(0.8, 3) - 2.95) <= 0.005


@pytest.mark.parametrize("alpha,K", [(0.75, 5), (0.8, 5), (0.6, 6), (0.9, 6), (0.4, 6), (0.8, 3), (0.6, 5)])
def test_oracle_accept_count_matches_closed_form(alpha, K):
    """Mean emitted tokens of the oracle on fixed-alpha rows equals
    (1 - a^(K+1)) / (1 - a) within 4 standard errors, and the accepted count is
    truncated-geometric.  (0.75, 5) is the pages' 3.29 example."""
    pins.check_accept_count(ov, alpha, K)


@pytest.mark.parametrize("case", ["random", "close", "equal", "disjoint", "masked"])
def test_oracle_lossless_chi2(case):
    pins.check_lossless(ov, case, N=1_000_000)


@pytest.mark.parametrize("seed", [3, 4])
def test_oracle_exact_integration(seed):
    pins.check_exact_integration(ov, seed=seed)


def test_oracle_softmax_matches_scipy():
    pins.check_softmax(ov)


def test_oracle_inverse_cdf_matches_searchsorted():
    pins.check_inverse_cdf(ov)


def test_oracle_greedy_is_argmax_matching():
    pins.check_greedy(ov)


def test_oracle_filters_brute_force():
    pins.check_filters(ov)


def test_oracle_zero_weight_tokens():
    pins.check_zero_weight_never_sampled(ov)


def test_topk1_equals_greedy_on_unique_maxima():
    rng = np.random.default_rng(7)
    N, K, V = 500, 3, 40
    tl = rng.normal(0, 1, (N, K + 1, V)).astype(np.float32)
    dl = (tl[:, :K] + rng.normal(0, 0.5, (N, K, V))).astype(np.float32)
    x = rng.integers(0, V, (N, K))
    x[:, 0] = np.argmax(tl[:, 0], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    a = oracle.verify(tl, dl, x, u, 1.0, 1, 1.0)
    b = oracle.verify(tl, dl, x, u, 0.0, 0, 1.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_filters_off_are_identity():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 2, (8, 100))
    base = oracle.filtered_probs(z, 0.8, 0, 1.0)
    assert np.array_equal(oracle.filtered_probs(z, 0.8, 100, 1.0), base)
    assert np.array_equal(oracle.filtered_probs(z, 0.8, 1000, 1.0), base)


def test_single_token_vocabulary():
    N, K = 10, 4
    tl = np.zeros((N, K + 1, 1), np.float32)
    dl = np.zeros((N, K, 1), np.float32)
    tok, n = oracle.verify(tl, dl, np.zeros((N, K), int), np.random.default_rng(0).random((N, K + 1), dtype=np.float32), 1.0, 0, 1.0)
    assert np.all(n == K) and np.all(tok == 0)


def test_no_drafts_is_plain_sampling():
    rng = np.random.default_rng(2)
    N, V = 300, 50
    tl = rng.normal(0, 1, (N, 1, V)).astype(np.float32)
    u = rng.random((N, 1), dtype=np.float32)
    tok, n = oracle.verify(tl, np.zeros((N, 0, V), np.float32), np.zeros((N, 0), int), u, 1.0, 0, 1.0)
    assert np.all(n == 0)
    P = pins.softmax_rows(tl[:, 0])
    for r in range(N):
        C = np.cumsum(P[r])
        assert tok[r, 0] == np.searchsorted(C, u[r, 0].astype(np.float64) * P[r].sum(), side="right")


def test_sentinels():
    rng = np.random.default_rng(0)
    B, K, V = 4, 2, 16
    tl = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    dl = rng.normal(0, 1, (B, K, V)).astype(np.float32)
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1), dtype=np.float32)
    tl[1, 2] = -np.inf            # a target row with no distribution
    x[2, 1] = V                   # a drafted token out of range
    dl[3, 0] = -np.inf            # a draft row with no distribution
    tok, n = oracle.verify(tl, dl, x, u, 1.0, 0, 1.0)
    assert list(n[1:]) == [-1, -1, -1] and n[0] >= 0
    assert np.all(tok[1:] == -1)
    # at temperature 0 the draft rows are not part of the rule
    tok0, n0 = oracle.verify(tl, dl, x, u, 0.0, 0, 1.0)
    assert n0[3] >= 0 and n0[1] == -1 and n0[2] == -1
    bad = tl.copy()
    bad[0, 0, 0] = np.nan
    with pytest.raises(ValueError):
        oracle.verify(bad, dl, x, u, 1.0, 0, 1.0)


def test_parameter_validation():
    z = np.zeros((1, 4))
    for T, k, p in [(-1.0, 0, 1.0), (float("nan"), 0, 1.0), (1.0, -1, 1.0), (1.0, 0, 0.0), (1.0, 0, 1.5)]:
        with pytest.raises(ValueError):
            oracle.filtered_probs(z, T, k, p)


def test_bf16_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    w = oracle.widen(bits, "bf16")
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    finite = np.isfinite(f)
    assert np.array_equal(w[finite], f[finite].astype(np.float64))


# --- the drafting draw (oracle.sample) ---------------------------------------

def test_sample_worked_case():
    # logits 0, ln 2, ln 3, -inf at T = 1: q = 1/6, 2/6, 3/6, 0; the inverse
    # CDF in vocabulary order splits [0, 1) at 1/6 and 1/2
    z = np.array([[0.0, np.log(2.0), np.log(3.0), -np.inf]] * 5, dtype=np.float32)
    u = np.array([0.0, 0.1, 0.2, 0.6, 0.999])
    tok, prob = oracle.sample(z, 1.0, 0, 1.0, u)
    assert tok.tolist() == [0, 0, 1, 2, 2]
    want = np.array([1, 1, 2, 3, 3]) / 6.0
    assert np.allclose(prob, want, rtol=1e-7, atol=0)


def test_sample_follows_q_chi2():
    from scipy import stats
    rng = np.random.default_rng(11)
    V, N = 12, 60000
    row = rng.normal(0, 1.5, V).astype(np.float32)
    for T, k, p in [(1.0, 0, 1.0), (0.7, 0, 0.9), (1.3, 5, 1.0)]:
        q = oracle.filtered_probs(row[None].astype(np.float64), T, k, p)[0]
        tok, prob = oracle.sample(np.repeat(row[None], N, 0), T, k, p, rng.random(N))
        counts = np.bincount(tok, minlength=V)
        assert np.all(counts[q == 0] == 0), "a token outside the kept set was drawn"
        keep = q > 0
        res = stats.chisquare(counts[keep], q[keep] / q[keep].sum() * N)
        assert res.pvalue > 1e-4, (T, k, p, res.pvalue)
        assert np.allclose(prob, q[tok], rtol=0, atol=0)


def test_sample_agrees_with_verify_without_drafts():
    rng = np.random.default_rng(12)
    N, V = 200, 40
    z = rng.normal(0, 2, (N, V)).astype(np.float32)
    u = rng.random((N, 1), dtype=np.float32)
    for T, k, p in [(1.0, 0, 1.0), (0.8, 7, 0.95), (0.0, 0, 1.0)]:
        tok, prob = oracle.sample(z, T, k, p, u[:, 0])
        vt, n = oracle.verify(z[:, None, :], np.zeros((N, 0, V), np.float32), np.zeros((N, 0), int), u, T, k, p)
        assert np.all(n == 0)
        assert np.array_equal(tok, vt[:, 0])


def test_sample_greedy_and_dead_rows():
    z = np.array([[1.0, 3.0, 3.0, -1.0], [-np.inf] * 4, [0.5, -np.inf, 0.5, 0.5]], dtype=np.float32)
    tok, prob = oracle.sample(z, 0.0, 0, 1.0, np.array([0.99, 0.5, 0.3]))
    assert tok.tolist() == [1, -1, 0]
    assert prob[0] == 1.0 and np.isnan(prob[1]) and prob[2] == 1.0


# --- drafts sampled at their own temperature ----------------------------------

def test_draft_temperature_keeps_the_law():
    p_wrong = pins.check_lossless_draft_temperature(oracle, T=1.0, Td=0.5)
    # the pin has power: ignoring the draft temperature is detected
    assert p_wrong < 1e-6, p_wrong


def test_draft_temperature_equal_or_greedy_changes_nothing():
    rng = np.random.default_rng(31)
    B, K, V = 50, 3, 30
    tl = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    dl = rng.normal(0, 2, (B, K, V)).astype(np.float32)
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1), dtype=np.float32)
    for T, k, p in [(0.8, 0, 1.0), (1.0, 5, 0.9)]:
        a = oracle.verify(tl, dl, x, u, T, k, p)
        b = oracle.verify(tl, dl, x, u, T, k, p, draft_temperature=T)
        assert all(np.array_equal(i, j) for i, j in zip(a, b))
    g = oracle.verify(tl, dl, x, u, 0.0, 0, 1.0)
    h = oracle.verify(tl, dl, x, u, 0.0, 0, 1.0, draft_temperature=0.3)
    assert all(np.array_equal(i, j) for i, j in zip(g, h))
    with pytest.raises(ValueError):
        oracle.verify(tl, dl, x, u, 1.0, 0, 1.0, draft_temperature=0.0)


def test_draft_probs_keep_the_law():
    pins.check_lossless_draft_probs(ov)


def test_draft_probs_count_law():
    """q given as probabilities with sum_x min(p, q) = alpha exactly: the
    accepted count is truncated geometric."""
    rng = np.random.default_rng(9)
    V, K, alpha, N = 8, 4, 0.6, 100_000
    h = V // 2
    tl = np.full((K + 1, V), -np.inf, dtype=np.float32)
    Q = np.zeros((K, V))
    for i in range(K + 1):
        p = rng.dirichlet(np.ones(h))
        tl[i, :h] = np.log(p)
        if i < K:
            Q[i] = np.concatenate([alpha * p, (1 - alpha) * rng.dirichlet(np.ones(V - h))])
    P = pins.softmax_rows(tl)
    Q32 = Q.astype(np.float32)
    a_true = np.minimum(P[:K], Q32.astype(np.float64)).sum(axis=1)
    x = np.stack([rng.choice(V, size=N, p=Q[i]) for i in range(K)], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    _, n = ov.verify(pins.tile_rows(tl, N), None, x, u, 1.0, 0, 1.0, draft_probs=pins.tile_rows(Q32, N))
    probs = np.empty(K + 1)
    run = 1.0
    for j in range(K):
        probs[j] = run * (1 - a_true[j])
        run *= a_true[j]
    probs[K] = run
    assert pins._chi2_pvalue(np.bincount(n, minlength=K + 1), probs) > pins.CHI2_MIN_P


def test_draft_probs_equal_to_the_logit_q_reproduce_verify():
    """Consistency: q supplied as the filtered draft distribution (float64)
    gives exactly the logit path's outcome."""
    rng = np.random.default_rng(12)
    B, K, V = 6, 3, 50
    t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, .6, (B, K, V))).astype(np.float32)
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1), dtype=np.float32)
    for T, k, p in ((1.0, 0, 1.0), (0.8, 7, 0.9), (0.0, 0, 1.0)):
        Q = ov.filtered_probs(d.reshape(-1, V).astype(np.float64), T, k, p).reshape(B, K, V)
        a = ov.verify(t, d, x, u, T, k, p, diag=True)
        b = ov.verify(t, None, x, u, T, k, p, diag=True, draft_probs=Q)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        if T > 0:
            assert np.array_equal(a[2]["qx"], b[2]["qx"]) and np.array_equal(a[2]["Z"], b[2]["Z"])


def test_draft_probs_validation():
    t = np.zeros((1, 2, 4), np.float32)
    u = np.zeros((1, 2), np.float32)
    for bad in (np.array([[[0.5, -0.1, 0.3, 0.3]]], np.float32), np.array([[[np.nan, 0, 0, 1]]], np.float32)):
        with pytest.raises(ValueError):
            ov.verify(t, None, np.zeros((1, 1)), u, 1.0, 0, 1.0, draft_probs=bad)
    with pytest.raises(TypeError):
        ov.verify(t, None, np.zeros((1, 1)), u, 1.0, 0, 1.0, draft_probs=np.zeros((1, 1, 4), np.float16))


def test_empty_residual_draws_from_p():
    """A given q at or above p everywhere: after a rejection the residual is
    empty and the oracle draws from p (pinned to p's inverse CDF by
    searchsorted, not by the oracle's own sampler)."""
    pins.check_empty_residual(ov)


def test_top_p_mass_reaches_every_float32_top_p():
    """The top-p cut's cumulative mass ends within 2^-31 of 1 even on the
    widest rows and on rows of one dominant token among many tiny ones, so
    every float32 top_p < 1 (at most 1 - 2^-24) is reached by some prefix and
    the oracle never needs a fallback cut."""
    rng = np.random.default_rng(7)
    tp = float(np.nextafter(np.float32(1.0), np.float32(0.0)))
    rows = [rng.normal(0, 3, 1 << 21), np.concatenate([[60.0], rng.normal(0, 1, (1 << 21) - 1)]),
            np.concatenate([rng.normal(0, 0.01, 1 << 20), np.full(1 << 20, -30.0)]), np.zeros(1 << 21)]
    for z in rows:
        e = np.exp(z - z.max())
        pi = e / e.sum()
        mass = np.cumsum(-np.sort(-pi))
        assert mass[-1] >= 1.0 - 2.0 ** -31
        assert mass[-1] >= tp
    # the oracle's top-p filter at that top_p keeps a prefix and raises nothing
    z = rng.normal(0, 2, (3, 5000))
    p = ov.filtered_probs(z, 1.0, 0, tp)
    assert np.all((p > 0).sum(axis=1) >= 4990)
