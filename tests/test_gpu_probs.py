"""GPU parity of verification with the draft distributions given as
probabilities (sv_spec_verify_probs) with the fp64 oracle: tokens and counts
identical except flagged near-ties, p(x) within 1e-6, q(x) exactly the given
value."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs
from tests.harness import compare_probs, log, run_device_probs

pytestmark = pytest.mark.gpu

PROB_TOL = 1e-6


def _filtered_q(w, d):
    """q_i: the draft rows' filtered distribution (fp64 oracle), as float32."""
    rows = oracle.widen(d["draft"].reshape(w.B * w.K, w.V), w.dtype)
    return oracle.filtered_probs(rows, w.temperature, w.top_k, w.top_p).reshape(w.B, w.K, w.V).astype(np.float32)


def _dirichlet_q(w, seed, alpha=0.05, zero_frac=0.3):
    """Arbitrary draft distributions: sparse Dirichlet draws with a share of
    exact zeros, float32."""
    rng = np.random.default_rng(seed)
    Q = rng.gamma(alpha, size=(w.B, w.K, w.V))
    Q[rng.random(Q.shape) < zero_frac] = 0.0
    Q /= Q.sum(axis=2, keepdims=True)
    return Q.astype(np.float32)


def _draw_x(w, d, Q):
    """x_i ~ q_i (the given rows, widened), by the oracle's inverse CDF."""
    q64 = Q.reshape(w.B * w.K, w.V).astype(np.float64)
    tok, _ = oracle.inverse_cdf(q64, d["draft_u"].reshape(-1))
    return tok.reshape(w.B, w.K).astype(np.int32)


def _check(w, d, Q, x=None):
    log(f"[probs] {w.name} B={w.B} K={w.K} V={w.V} T={w.temperature} top_k={w.top_k} top_p={w.top_p}")
    if x is None:
        x = _draw_x(w, d, Q)
    tok, n, dbg = run_device_probs(w, d, Q, x)
    stats, fails = compare_probs(w, d, Q, x, tok, n, dbg)
    log(f"   match={stats['match']} flagged={stats['flagged']} fail={stats['fail']} "
        f"max|dp|={stats['max_prob_err']:.2e} mean_n={np.mean(n):.3f}")
    assert stats["fail"] == 0, fails[:5]
    assert stats["flagged"] == 0
    assert stats["max_prob_err"] <= PROB_TOL
    if w.temperature > 0:
        ok = n >= 0
        want = np.take_along_axis(Q.astype(np.float64), x[:, :, None].astype(np.int64), axis=2)[:, :, 0]
        assert np.array_equal(dbg["q"][ok], want[ok]), "q(x) must be the given value"
    return tok, n, dbg


@pytest.mark.parametrize("name", [
    "b64-k6-v128256-bf16-zipf-t0.7-topp0.9",
    "b8-k5-v32000-f32-zipf",
    "b32-k6-v128256-bf16-normal-s1.0",
    "b32-k6-v128256-bf16-normal-greedy",
])
def test_probs_filtered_draft_distribution(name):
    w = WORKLOADS[name]
    d = make_inputs(w)
    _check(w, d, _filtered_q(w, d))


@pytest.mark.parametrize("name,seed", [
    ("b64-k6-v128256-bf16-zipf-t0.7-topp0.9", 1),
    ("b8-k5-v32000-f32-zipf", 2),
])
def test_probs_arbitrary_draft_distribution(name, seed):
    """q unrelated to the draft logits (sparse, with zeros): more rejections
    and residual draws."""
    w = WORKLOADS[name]
    d = make_inputs(w)
    _check(w, d, _dirichlet_q(w, seed))


def test_probs_top_k_and_large_kept_sets():
    # top-k on the peaked rows (kept lists), then a nucleus far above 256
    # tokens (the full-row draw with the given q row)
    w = replace(WORKLOADS["b256-k8-v152064-f32-peaked-topk50"], B=24, seed=61)
    d = make_inputs(w)
    _check(w, d, _filtered_q(w, d))
    w2 = replace(WORKLOADS["b8-k5-v32000-f32-zipf"], name="b8-k5-v32000-f32-normal-topp0.99", shape="normal",
                 target_sigma=1.0, top_p=0.99, seed=62)
    d2 = make_inputs(w2)
    _check(w2, d2, _dirichlet_q(w2, 5, alpha=0.5, zero_frac=0.1))


def test_probs_equal_to_the_logit_q_match_the_logit_call():
    """q given as the draft's own filtered distribution (float32-rounded)
    against the logit entry point: identical tokens wherever no decision
    lies within the float32 rounding of q."""
    from tests.harness import run_device

    w = WORKLOADS["b8-k5-v32000-f32-zipf"]
    d = make_inputs(w)
    Q = _filtered_q(w, d)
    x = _draw_x(w, d, Q)
    a_tok, a_n, a_dbg = run_device(w, d, x, debug=True)
    b_tok, b_n, b_dbg = run_device_probs(w, d, Q, x)
    assert np.max(np.abs(a_dbg["q"] - b_dbg["q"])) < 1e-7
    assert np.array_equal(a_dbg["p"], b_dbg["p"])
    same = (a_n == b_n) & np.all(a_tok == b_tok, axis=1)
    assert same.mean() > 0.95


@pytest.mark.parametrize("V,dtype,T,k,p,K", [
    (4099, "f32", 1.0, 0, 1.0, 1),    # element loads, unfiltered: the full-row residual with the given q
    (5003, "bf16", 0.9, 20, 0.9, 3),  # element loads, top-k then top-p
])
def test_probs_element_path(V, dtype, T, k, p, K):
    w = replace(WORKLOADS["b8-k5-v32000-f32-zipf"], name=f"b10-k{K}-v{V}-{dtype}", B=10, K=K, V=V, dtype=dtype,
                temperature=T, top_k=k, top_p=p, seed=80 + K)
    d = make_inputs(w)
    _check(w, d, _dirichlet_q(w, 9, alpha=0.3, zero_frac=0.2))


def test_probs_bad_token_is_a_sentinel():
    w = WORKLOADS["b8-k5-v32000-f32-zipf"]
    d = make_inputs(w)
    Q = _filtered_q(w, d)
    x = _draw_x(w, d, Q)
    x[2, 1] = -3
    tok, n, _ = run_device_probs(w, d, Q, x)
    assert n[2] == -1 and np.all(tok[2] == -1)
    ref_tok, ref_n = oracle.verify(d["target"], None, x, d["uniforms"], w.temperature, w.top_k, w.top_p,
                                   dtype=w.dtype, draft_probs=Q)
    assert np.array_equal(n, ref_n) and np.array_equal(tok, ref_tok)


@pytest.mark.parametrize("params", [(1.0, 0, 0.9, "zipf", 1.0), (1.0, 0, 1.0, "normal", 2.0),
                                    (1.0, 0, 0.995, "normal", 0.05)],
                         ids=["kept-lists", "unfiltered", "large-kept-set"])
def test_empty_residual_draws_from_p(params):
    """A given q at or above p at every token, with extra mass on the drafted
    token: every rejection leaves max(0, p - q) empty and the replacement is
    drawn from p (the oracle's reading, pinned on the CPU).  Covers the draw
    from kept lists, the unfiltered full-row draw and the draw from a kept set
    too large for a list."""
    from synth import Workload

    T, k, p, shape, sig = params
    w = Workload("empty-res", 16, 3, 3000, "f32", shape, sig, 0.5, T, k, p, 13)
    d = make_inputs(w)
    P = oracle.filtered_probs(oracle.widen(d["target"].reshape(-1, w.V), w.dtype), T, k, p).reshape(w.B, w.K + 1,
                                                                                                      w.V)
    rng = np.random.default_rng(14)
    x = np.stack([rng.choice(np.flatnonzero(P[b, i] > 0)) for b in range(w.B) for i in range(w.K)]).reshape(w.B, w.K)
    Q = P[:, :w.K] * (1.0 + 1e-6)
    Q[np.arange(w.B)[:, None], np.arange(w.K)[None, :], x] += 0.3
    Qf = Q.astype(np.float32)
    Qf = np.where(Qf.astype(np.float64) < Q, np.nextafter(Qf, np.float32(np.inf)), Qf)
    tok, n, dbg = _check(w, d, Qf, x.astype(np.int32))
    assert (n < w.K).sum() >= w.B // 2, "the case must reject often"
