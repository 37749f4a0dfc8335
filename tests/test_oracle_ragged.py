"""Pins of the oracle's ragged verification (a draft length per sequence) and
of its draft-length controller, against facts that do not come from the
oracle: hand-derived outcomes of the rule, the truncated-geometric law of the
accepted count per draft length, the target law of every emitted token, and
hand-traced controller runs of the rule on page www.2kiu.com/news/5895634
§4.4."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import spec_verify as sv
from tests import pins


def _lg(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


def check_ragged_worked_case(mod):
    """Three sequences of 2, 0 and 1 drafts over a 4-token vocabulary.  The
    outcomes follow from the rule by hand:
    * sequence 0: x0 = 0 has p/q = 0.5/0.25 > 1, accepted for any u; x1 = 1 has
      p = 0, rejected; the residual max(0, p1 - q1) is mass 0.75 on token 2 only.
    * sequence 1 (no drafts): the bonus draw from p = (.1, .2, .3, .4) with
      u = 0.35 lands in [0.3, 0.6), token 2.
    * sequence 2: x0 = 1 has p/q = 0.25/0.5, u = 0.4 < 0.5 accepts; the bonus
      row is one-hot at token 0."""
    t = np.stack([
        _lg([.5, .5, 0, 0]), _lg([0, 0, 1, 0]), _lg([.3, .3, .2, .2]),   # sequence 0: K+1 = 3 rows
        _lg([.1, .2, .3, .4]),                                           # sequence 1: 1 row
        _lg([.25, .25, .25, .25]), _lg([1, 0, 0, 0]),                    # sequence 2: 2 rows
    ])
    d = np.stack([_lg([.25] * 4), _lg([.25] * 4), _lg([.5, .5, 0, 0])])
    x = np.array([0, 1, 1], dtype=np.int32)
    u = np.array([0.9, 0.5, 0.99, 0.35, 0.4, 0.7], dtype=np.float32)
    cu = np.array([0, 2, 2, 3])
    tok, n = mod.verify_ragged(t, d, x, u, cu, 1.0, 0, 1.0)
    assert n.tolist() == [1, 0, 1]
    assert tok.tolist() == [[0, 2, -1], [2, -1, -1], [1, 0, -1]]
    tok4, n4 = mod.verify_ragged(t, d, x, u, cu, 1.0, 0, 1.0, max_k=4)
    assert tok4.shape == (3, 5) and np.array_equal(tok4[:, :3], tok) and np.all(tok4[:, 3:] == -1)


def test_ragged_worked_case():
    check_ragged_worked_case(sv)


def _ragged_batch(rng, tl, dl, ks):
    """Packs sequence b as rows 0..K_b of tl and 0..K_b-1 of dl."""
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    t = np.concatenate([tl[:k + 1] for k in ks])
    d = np.concatenate([dl[:k] for k in ks]) if cu[-1] > 0 else np.zeros((0, tl.shape[1]), np.float32)
    return cu, t, d


def test_ragged_count_law_per_length():
    """Positions with sum_x min(p, q) = alpha: the accepted count of a
    sequence with K_b drafts is truncated geometric with that K_b."""
    rng = np.random.default_rng(7)
    V, alpha, Kmax = 8, 0.7, 6
    tl, dl = pins.exact_alpha_rows(V, alpha, Kmax, rng)
    P, Q = pins.softmax_rows(tl), pins.softmax_rows(dl)
    a_true = np.minimum(P[:Kmax], Q).sum(axis=1)
    N = 60_000
    ks = rng.choice([0, 2, 4, 6], size=N)
    cu, t, d = _ragged_batch(rng, tl, dl, ks)
    pos = np.concatenate([np.arange(k) for k in ks]).astype(np.int64)
    x = np.array([rng.choice(V, p=Q[i]) for i in pos], dtype=np.int64) if pos.size else np.zeros(0, np.int64)
    u = rng.random(cu[-1] + N, dtype=np.float32)
    tok, n = oracle.verify_ragged(t, d, x, u, cu, 1.0, 0, 1.0)
    assert tok.shape == (N, Kmax + 1)
    for K in (0, 2, 4, 6):
        sel = ks == K
        probs = np.empty(K + 1)
        run = 1.0
        for j in range(K):
            probs[j] = run * (1 - a_true[j])
            run *= a_true[j]
        probs[K] = run
        counts = np.bincount(n[sel], minlength=K + 1)
        assert counts.shape[0] == K + 1, "a count above the sequence's own K"
        assert pins._chi2_pvalue(counts, probs) > pins.CHI2_MIN_P
        assert np.all(tok[sel, K + 1:] == -1)


def check_ragged_lossless(mod, N: int = 120_000):
    """Every emitted token follows the target row of its position, whatever
    the sequence's draft length (residual draws and bonus draws alike)."""
    rng = np.random.default_rng(13)
    V, Kmax = 8, 3
    tl, dl = pins.lossless_case("close", V, Kmax, seed=13)
    P, Q = pins.softmax_rows(tl), pins.softmax_rows(dl)
    ks = rng.integers(0, Kmax + 1, size=N)
    cu, t, d = _ragged_batch(rng, tl, dl, ks)
    pos = np.concatenate([np.arange(k) for k in ks]).astype(np.int64)
    cq = np.cumsum(Q, axis=1)
    x = np.minimum((rng.random(pos.size)[:, None] >= cq[pos]).sum(axis=1), V - 1)
    u = rng.random(cu[-1] + N, dtype=np.float32)
    tok, n = mod.verify_ragged(t, d, x, u, cu, 1.0, 0, 1.0)
    assert np.all((n >= 0) & (n <= ks))
    for j in range(Kmax + 1):
        sel = n >= j
        counts = np.bincount(tok[sel, j], minlength=V)
        assert pins._chi2_pvalue(counts, P[j]) > pins.CHI2_MIN_P, f"position {j}"


def test_ragged_lossless_chi2():
    check_ragged_lossless(sv)


def test_ragged_bad_offsets_are_sentinels():
    rng = np.random.default_rng(1)
    tl = rng.normal(0, 1, (4, 6)).astype(np.float32)
    dl = rng.normal(0, 1, (3, 6)).astype(np.float32)
    ks = np.array([1, 2])
    cu, t, d = _ragged_batch(rng, tl, dl, ks)
    x = np.zeros(3, np.int32)
    u = rng.random(5, dtype=np.float32)
    ok_tok, ok_n = oracle.verify_ragged(t, d, x, u, cu, 1.0, 0, 1.0)
    assert np.all(ok_n >= 0)
    for bad_cu, mk in (([1, 1, 3], None), ([0, 2, 1], None), ([0, 1, 3], 1)):
        # cu[0] != 0 / cu[B] != rows; a decrease; a K_b above max_k
        tok, n = oracle.verify_ragged(t, d, x, u, np.array(bad_cu), 1.0, 0, 1.0, max_k=mk if mk else 2)
        assert np.all(n == -1) and np.all(tok == -1)
    with pytest.raises(ValueError):
        oracle.verify_ragged(t[:-1], d, x, u, cu, 1.0, 0, 1.0)
    assert oracle.ragged_offsets_ok(cu, 3, 2) and not oracle.ragged_offsets_ok(cu, 3, 1)


def test_ragged_with_one_length_is_the_batch_rule():
    """Consistency: equal draft lengths reproduce the rectangular batch."""
    rng = np.random.default_rng(4)
    B, K, V = 5, 3, 40
    t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, .5, (B, K, V))).astype(np.float32)
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1), dtype=np.float32)
    ref_t, ref_n, ref_d = sv.verify(t, d, x, u, 0.8, 5, 0.9, diag=True)
    cu = np.arange(B + 1) * K
    got_t, got_n, got_d = oracle.verify_ragged(t.reshape(-1, V), d.reshape(-1, V), x.reshape(-1), u.reshape(-1), cu,
                                                0.8, 5, 0.9, diag=True)
    assert np.array_equal(ref_t, got_t) and np.array_equal(ref_n, got_n)
    assert np.array_equal(ref_d["px"].reshape(-1), got_d["px"]) and np.array_equal(ref_d["Z"], got_d["Z"])


# ---------------------------------------------------------------------------
# the draft-length controller
# ---------------------------------------------------------------------------
def check_controller_hand_trace(cls):
    """window 3, thresholds 0.8 / 0.6, K in [2, 4], start 3.  Traced by hand:
    three batches at rate 1 raise K to 4 and restart the window; at K = 4 the
    upper bound holds K (the window keeps sliding); a window of rates
    (1, 1, 0) = 2/3 keeps K; then (1, 0, 0) = 1/3 lowers it to 3.  The
    restarted window fills with 1/3, 1, 1: pooled 7/9 keeps K; one more
    batch at rate 1 slides the 1/3 out and raises K to 4."""
    c = cls(window=3, k_min=2, k_max=4, k_init=3)
    obs = [(3, 3), (3, 3), (3, 3), (4, 4), (4, 4), (4, 4), (4, 4), (0, 4), (0, 4), (1, 3), (3, 3), (3, 3), (3, 3)]
    want = [3, 3, 4, 4, 4, 4, 4, 4, 3, 3, 3, 3, 4]
    assert [c.observe(a, d) for a, d in obs] == want


def test_controller_hand_trace():
    check_controller_hand_trace(oracle.DynamicK)


def test_controller_strict_thresholds_and_skips():
    c = oracle.DynamicK(window=2, k_init=5)
    # pooled rate exactly 0.8 (8/10) and exactly 0.6: no change
    assert [c.observe(4, 5), c.observe(4, 5)] == [5, 5]
    c2 = oracle.DynamicK(window=2, k_init=5)
    assert [c2.observe(3, 5), c2.observe(3, 5)] == [5, 5]
    # a batch that drafted nothing is not observed
    c3 = oracle.DynamicK(window=2, k_init=5)
    assert [c3.observe(5, 5), c3.observe(0, 0), c3.observe(5, 5)] == [5, 5, 6]
    # the pooled rate weighs batches by their drafted tokens: 1/1 and 0/9
    c4 = oracle.DynamicK(window=2, k_init=5)
    assert [c4.observe(1, 1), c4.observe(0, 9)] == [5, 4]
    with pytest.raises(ValueError):
        c4.observe(3, 2)
    # after a raise the window restarts: a second raise needs a full window
    c5 = oracle.DynamicK(window=2, k_init=5)
    assert [c5.observe(2, 2) for _ in range(5)] == [5, 6, 6, 7, 7]


def test_controller_page_defaults_walk_to_bounds():
    """With the page's settings (window 100, 0.8 / 0.6, K in [2, 10]): a
    constant rate of 0.9 raises K by one every 100 batches up to 10; at the
    bound the window keeps sliding.  A rate of 0.5 then lowers K once 76 of
    the 100 batches are at 0.5 (after 75 the pooled rate is exactly 0.6,
    not below), and from there by one every 100 batches down to 2."""
    c = oracle.DynamicK()
    ks = [c.observe(9 * c.k, 10 * c.k) for _ in range(1000)]
    assert ks[98] == 5 and ks[99] == 6 and ks[199] == 7 and ks[499] == 10 and ks[-1] == 10
    ks = [c.observe(5 * c.k, 10 * c.k) for _ in range(900)]
    assert ks[74] == 10 and ks[75] == 9 and ks[174] == 9 and ks[175] == 8
    assert ks[774] == 3 and ks[775] == 2 and ks[-1] == 2


def test_controller_with_the_verification_law():
    """Closed loop against the count law: with alpha = 0.9 at every position
    a batch accepts E[n] / K = a(1 - a^K) / ((1 - a) K) of its drafted tokens:
    0.855 at K = 2, 0.813 at K = 3, 0.774 at K = 4.  Fed those exact expected
    counts, the controller climbs from 2 to 4, where the rate falls below 0.8
    but stays above 0.6, and holds there."""
    a = 0.9

    def rate(K):
        return a * (1 - a ** K) / ((1 - a) * K)

    assert rate(3) > 0.8 > rate(4) > 0.6
    c = oracle.DynamicK(window=10, k_init=2)
    seen = []
    for _ in range(200):
        K = c.k
        seen.append(c.observe(round(1000 * K * rate(K)), 1000 * K))
    assert seen[9] == 3 and seen[19] == 4 and seen[-1] == 4
