"""The oracle's batched decisions for many draws on fixed rows (oracle/rate.py)
against ``verify_given`` element for element, and ``verify_given`` against
``verify`` on the logit path (CPU)."""
import numpy as np
import pytest

import oracle
from oracle import spec_verify as ov
from oracle.rate import DrawTables
from tests import pins


def _rows(rng, B, K, V, T, k, tp, shape="normal"):
    tl = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    if shape == "ties":
        tl = (np.round(tl * 2) / 2).astype(np.float32)
    dl = (tl[:, :K] + rng.normal(0, 0.7, (B, K, V))).astype(np.float32)
    P = ov.filtered_probs(tl.reshape(-1, V).astype(np.float64), T, k, tp).reshape(B, K + 1, V)
    Q = ov.filtered_probs(dl.reshape(-1, V).astype(np.float64), T, k, tp).reshape(B, K, V)
    return tl, dl, P, Q


@pytest.mark.parametrize("case", [(6, 3, 50, 1.0, 0, 1.0, "normal"), (5, 4, 40, 0.7, 0, 0.8, "ties"),
                                  (4, 2, 64, 1.3, 5, 1.0, "normal"), (3, 0, 30, 1.0, 0, 1.0, "normal"),
                                  (4, 3, 20, 0.9, 6, 0.7, "ties")])
def test_draw_tables_equal_verify_given(case):
    B, K, V, T, k, tp, shape = case
    rng = np.random.default_rng(B * 100 + K)
    tl, dl, P, Q = _rows(rng, B, K, V, T, k, tp, shape)
    R = 300
    tabs = DrawTables(P, Q)
    x = tabs.draw_drafts(rng.random((R, B, K)))
    x[5, 0, :1] = V + 3  # a drafted token out of range makes a sentinel
    u = rng.random((R, B, K + 1), dtype=np.float32)
    u[7] = 0.0
    u[8] = np.nextafter(np.float32(1.0), np.float32(0.0))
    tok, n = tabs.decide(x, u)
    ref_tok, ref_n = ov.verify_given(np.repeat(P[None], R, 0).reshape(R * B, K + 1, V),
                                     np.repeat(Q[None], R, 0).reshape(R * B, K, V),
                                     x.reshape(R * B, K), u.reshape(R * B, K + 1))
    assert np.array_equal(tok.reshape(R * B, K + 1), ref_tok)
    assert np.array_equal(n.reshape(-1), ref_n)
    assert K == 0 or n[5, 0] == -1


def test_draw_tables_empty_residual_and_dead_rows():
    """The empty-residual fallback and a row with no distribution, through
    both paths."""
    V, K = 8, 2
    tl, Qf, P64, bump = pins.empty_residual_case(V, K)
    P = ov.filtered_probs(tl.astype(np.float64), 1.0, 0, 1.0)[None]
    Q = Qf.astype(np.float64)[None]
    P2 = P.copy()
    P2[0, 1] = np.nan  # a target row with no distribution
    for PP in (P, P2):
        tabs = DrawTables(PP, Q)
        R = 500
        rng = np.random.default_rng(3)
        x = np.tile(bump, (R, 1, 1))
        u = rng.random((R, 1, K + 1), dtype=np.float32)
        tok, n = tabs.decide(x, u)
        ref_tok, ref_n = ov.verify_given(np.repeat(PP, R, 0), np.repeat(Q, R, 0), x[:, 0], u[:, 0])
        assert np.array_equal(tok[:, 0], ref_tok) and np.array_equal(n[:, 0], ref_n)
    assert (n == -1).all()


@pytest.mark.parametrize("params", [(1.0, 0, 1.0), (0.7, 0, 0.9), (1.0, 7, 1.0), (0.0, 0, 1.0)])
def test_verify_given_is_verify_on_filtered_rows(params):
    T, k, tp = params
    rng = np.random.default_rng(17)
    B, K, V = 20, 3, 200
    tl, dl, P, Q = _rows(rng, B, K, V, T if T > 0 else 1.0, k, tp)
    if T == 0.0:
        P = ov.filtered_probs(tl.reshape(-1, V).astype(np.float64), 0.0, 0, 1.0).reshape(B, K + 1, V)
        Q = ov.filtered_probs(dl.reshape(-1, V).astype(np.float64), 0.0, 0, 1.0).reshape(B, K, V)
    x = DrawTables(P, Q).draw_drafts(rng.random((1, B, K)))[0]
    u = rng.random((B, K + 1), dtype=np.float32)
    a = ov.verify(tl, dl, x, u, T, k, tp, diag=True)
    b = ov.verify_given(P, Q, x, u, diag=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[2]["px"], b[2]["px"]) and np.array_equal(a[2]["Z"], b[2]["Z"])


def test_at_risk_marks_boundary_uniforms():
    rng = np.random.default_rng(2)
    tl, dl, P, Q = _rows(rng, 2, 1, 10, 1.0, 0, 1.0)
    tabs = DrawTables(P, Q)
    x = np.zeros((2, 2, 1), np.int64)
    u = rng.random((2, 2, 2), dtype=np.float32)
    r = P[0, 0, 0] / Q[0, 0, 0]
    u[0, 0, 0] = np.float32(min(r, 0.999))  # an accept test on its boundary
    risk = tabs.at_risk(x, u)
    assert risk[0, 0] == (r < 0.999)
    ref = ov.verify_one(tl[1], dl[1], x[1, 1], u[1, 1], 1.0, 0, 1.0)
    assert risk[1, 1] == oracle.at_risk(ref, u[1, 1])
