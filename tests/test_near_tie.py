"""The mismatch classifier on hand-built near-ties and gross errors (CPU)."""
import numpy as np

import oracle
from oracle import FAIL, FLAGGED, MATCH, classify


def _case():
    tl = np.array([[0.0, 1.0, -0.5, 0.3], [0.2, -1.0, 0.7, 0.1]], dtype=np.float32)
    dl = np.array([[1.0, 0.0, 0.4, -0.2]], dtype=np.float32)
    return tl, dl


def test_match():
    tl, dl = _case()
    u = np.array([0.3, 0.4], np.float32)
    tok, n = oracle.verify(tl[None], dl[None], np.array([[1]]), u[None], 1.0, 0, 1.0)
    assert classify(tl, dl, [1], u, 1.0, 0, 1.0, "f32", tok[0], n[0])[0] == MATCH


def test_accept_near_tie_is_flagged_and_far_is_fail():
    tl, dl = _case()
    ref = oracle.verify_one(tl, dl, [0], np.array([0.5, 0.5], np.float32), 1.0, 0, 1.0)
    r = ref["px"][0] / ref["qx"][0]
    assert r < 1.0
    # u just above p/q: the oracle rejects; a device that accepted is a near-tie
    u_hi = np.array([np.nextafter(np.float32(r), np.float32(1)), 0.5], np.float32)
    ref2 = oracle.verify_one(tl, dl, [0], u_hi, 1.0, 0, 1.0)
    assert ref2["n"] == 0
    dev_tok = np.array([0, 2])
    assert classify(tl, dl, [0], u_hi, 1.0, 0, 1.0, "f32", dev_tok, 1)[0] == FLAGGED
    # u far above p/q: the same device answer is a failure
    u_far = np.array([min(0.99, r + 0.2), 0.5], np.float32)
    assert classify(tl, dl, [0], u_far, 1.0, 0, 1.0, "f32", dev_tok, 1)[0] == FAIL


def test_sampling_near_tie_is_flagged_and_far_is_fail():
    tl, dl = _case()
    # bonus path: draft equals target so the draft is always accepted
    d = tl[:1].copy()
    P1 = oracle.verify_one(tl, d, [1], np.array([0.1, 0.5], np.float32), 1.0, 0, 1.0)["w"]
    C = np.cumsum(P1)
    # put u*Z a hair above the breakpoint between tokens 1 and 2
    u_s = np.float32(C[1] / C[-1])
    while np.float64(u_s) * C[-1] < C[1]:
        u_s = np.nextafter(u_s, np.float32(1))
    u = np.array([0.1, u_s], np.float32)
    ref = oracle.verify_one(tl, d, [1], u, 1.0, 0, 1.0)
    assert ref["n"] == 1 and ref["token"] == 2
    assert classify(tl, d, [1], u, 1.0, 0, 1.0, "f32", np.array([1, 1]), 1)[0] == FLAGGED
    assert classify(tl, d, [1], u, 1.0, 0, 1.0, "f32", np.array([1, 0]), 1)[0] == FAIL


def test_malformed_and_sentinel():
    tl, dl = _case()
    u = np.array([0.3, 0.4], np.float32)
    tok, n = oracle.verify(tl[None], dl[None], np.array([[1]]), u[None], 1.0, 0, 1.0)
    assert classify(tl, dl, [1], u, 1.0, 0, 1.0, "f32", np.array([-1, -1]), -1)[0] == FAIL
    bad = tok[0].copy()
    if n[0] == 0:
        bad[1] = 3  # garbage after the sampled token
    else:
        bad[0] = 3 if bad[0] != 3 else 2  # accepted prefix differs from the draft
    assert classify(tl, dl, [1], u, 1.0, 0, 1.0, "f32", bad, n[0])[0] == FAIL


def test_top_p_boundary_near_tie():
    # two tokens whose mass straddles top_p within 1e-6: the kept set depends
    # on rounding, which the classifier must admit as a near-tie
    p = np.array([0.6, 0.3 + 2e-7, 0.1 - 2e-7])
    tl = np.log(p).astype(np.float32)[None].repeat(2, 0)
    d = tl[:1].copy()
    tp = 0.9
    ref = oracle.verify_one(tl, d, [0], np.array([0.2, 0.95], np.float32), 1.0, 0, tp)
    kept = (ref["P"][1] > 0).sum()
    # a device that kept the other set (3 tokens instead of 2 or vice versa)
    # samples token 2 with u=0.95 only if 3 tokens are kept
    alt = 2 if kept == 2 else 1
    dev = np.array([0, alt])
    v, why = classify(tl, d, [0], np.array([0.2, 0.95], np.float32), 1.0, 0, tp, "f32", dev, 1)
    assert v == FLAGGED, why


def test_sample_classifier():
    from oracle import classify_sample
    row = np.log(np.array([0.25, 0.25, 0.5]))  # running sums 0.25, 0.5, 1
    # u*Z a hair below the boundary at 0.5: the next token is a near-tie
    assert classify_sample(row, 1.0, 0, 1.0, 0.5 - 1e-9, 2, 1) == FLAGGED
    # far from any boundary a different token is a failure
    assert classify_sample(row, 1.0, 0, 1.0, 0.3, 2, 1) == FAIL
    assert classify_sample(row, 1.0, 0, 1.0, 0.3, 1, 1) == MATCH
    # top_p = 0.5 keeps token 2 alone: a token outside the kept set is never a near-tie
    assert classify_sample(row, 1.0, 0, 0.5, 0.49, 2, 2) == MATCH
    assert classify_sample(row, 1.0, 0, 0.5, 0.49, 0, 2) == FAIL


def test_accept_near_tie_then_wrong_draw_is_fail():
    """A device that flips an accept decision at a near-tie must still draw
    what the oracle draws on the device's path: a wrong bonus token after the
    flip is a failure, the right one is flagged."""
    tl, dl = _case()
    ref = oracle.verify_one(tl, dl, [0], np.array([0.5, 0.5], np.float32), 1.0, 0, 1.0)
    r = ref["px"][0] / ref["qx"][0]
    u_hi = np.array([np.nextafter(np.float32(r), np.float32(1)), 0.5], np.float32)
    # the device accepted draft 0 and drew its bonus from p_1 with u = 0.5
    P1 = ref["P"][1]
    C = np.cumsum(P1)
    good = int(np.searchsorted(C, 0.5 * P1.sum(), side="right"))
    far = [j for j in range(4) if j != good and not (C[j] - P1[j] <= 0.5 * P1.sum() + 1e-5 and
                                                      C[j] > 0.5 * P1.sum() - 1e-5)]
    assert classify(tl, dl, [0], u_hi, 1.0, 0, 1.0, "f32", np.array([0, good]), 1)[0] == FLAGGED
    v, why = classify(tl, dl, [0], u_hi, 1.0, 0, 1.0, "f32", np.array([0, far[0]]), 1)
    assert v == FAIL, why
    # and a device that rejected where the oracle accepted must draw the residual
    u_lo = np.array([np.nextafter(np.float32(r), np.float32(0)), 0.5], np.float32)
    assert oracle.verify_one(tl, dl, [0], u_lo, 1.0, 0, 1.0)["n"] == 1
    w = np.maximum(0.0, ref["P"][0] - ref["Q"][0])
    Cw = np.cumsum(w)
    res_tok = int(np.searchsorted(Cw, 0.5 * w.sum(), side="right"))
    assert classify(tl, dl, [0], u_lo, 1.0, 0, 1.0, "f32", np.array([res_tok, -1]), 0)[0] == FLAGGED
    wrong = [j for j in range(4) if w[j] == 0.0][0]
    assert classify(tl, dl, [0], u_lo, 1.0, 0, 1.0, "f32", np.array([wrong, -1]), 0)[0] == FAIL
