"""The near-tie rate harness on the CPU: a stand-in device that returns the
oracle's own answers passes with no mismatch; one with a planted wrong draw
or a wrong accepted count is caught as a failure."""
import numpy as np

import oracle
from synth import Workload, make_inputs
from tests.harness import rate_check, rate_inputs


def _small(T=0.8, k=0, p=0.9):
    return Workload("rate-small", 4, 3, 300, "bf16", "zipf", 1.0, 0.5, T, k, p, 5)


def test_oracle_answers_pass():
    for w in [_small(), _small(1.0, 0, 1.0), _small(0.0, 0, 1.0), _small(1.0, 20, 1.0)]:
        d = make_inputs(w)
        tabs, x, u = rate_inputs(w, d, 400)
        tok, n = oracle.verify_given(np.repeat(tabs.P[None], x.shape[0], 0).reshape(-1, w.K + 1, w.V),
                                     np.repeat(tabs.Q[None], x.shape[0], 0).reshape(-1, w.K, w.V),
                                     x.reshape(-1, w.K), u.reshape(-1, w.K + 1))
        stats, fails, flags = rate_check(w, d, tabs, x, u, tok.reshape(x.shape[0], w.B, -1),
                                         n.reshape(x.shape[0], w.B))
        assert stats["sequences"] >= 400 and stats["mismatched"] == 0 and stats["fail"] == 0


def test_planted_device_errors_fail():
    w = _small()
    d = make_inputs(w)
    tabs, x, u = rate_inputs(w, d, 200)
    tok, n = tabs.decide(x, u)
    tok, n = tok.copy(), n.copy()
    # a drawn token replaced by one outside the kept set, and a count off by one
    r, b = 3, 1
    j = n[r, b]
    P_row = tabs.P[b, j]
    tok[r, b, j] = int(np.flatnonzero(P_row == 0)[0])
    r2, b2 = np.argwhere(n == 0)[0]
    n[r2, b2] = 1
    tok[r2, b2, 0] = x[r2, b2, 0]
    tok[r2, b2, 1] = 0
    stats, fails, flags = rate_check(w, d, tabs, x, u, tok, n)
    assert stats["fail"] == 2, (stats, fails)
