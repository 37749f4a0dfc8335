"""GPU parity of ragged verification (sv_spec_verify_ragged: a draft length
per sequence) with the fp64 oracle, and a closed draft-length control loop
(library controller + GPU verification against oracle controller + oracle
verification).  Same bar as the rectangular parity tests: tokens and counts
identical except flagged near-ties, p(x) and q(x) within 1e-6."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs, pack_ragged, ragged_lengths
from tests.harness import compare_ragged, log, ragged_draft_tokens, run_device, run_device_ragged

pytestmark = pytest.mark.gpu

PROB_TOL = 1e-6


def _ragged_case(w, k_lo, k_hi, seed=0):
    """Lengths in [k_lo, k_hi]; rows cut from a rectangular batch at K = k_hi."""
    wk = replace(w, K=k_hi)
    ks = ragged_lengths(w.B, k_lo, k_hi, w.seed + seed)
    r = pack_ragged(make_inputs(wk), ks)
    return wk, ks, r


def _check(w, ks, r, max_k, Td=None):
    log(f"[ragged] {w.name} B={w.B} K_b in [{ks.min()}, {ks.max()}] N={int(r['cu'][-1])} max_k={max_k} "
        f"T={w.temperature} Td={Td} top_k={w.top_k} top_p={w.top_p}")
    x = ragged_draft_tokens(w, r, Td)
    tok, n, dbg = run_device_ragged(w, r, x, max_k, draft_temperature=Td)
    stats, fails = compare_ragged(w, r, x, max_k, tok, n, dbg, draft_temperature=Td)
    log(f"   match={stats['match']} flagged={stats['flagged']} fail={stats['fail']} "
        f"max|dp|={stats['max_prob_err']:.2e} mean_n={np.mean(n):.3f}")
    assert stats["fail"] == 0, fails[:5]
    assert stats["flagged"] == 0
    assert stats["max_prob_err"] <= PROB_TOL
    assert tok.shape == (w.B, max_k + 1)
    return tok, n, dbg, x


@pytest.mark.parametrize("name,k_lo,k_hi", [
    ("b64-k6-v128256-bf16-zipf-t0.7-topp0.9", 2, 10),
    ("b8-k5-v32000-f32-zipf", 0, 8),
    ("b32-k6-v128256-bf16-normal-s1.0", 0, 6),
    ("b32-k6-v128256-bf16-normal-greedy", 2, 10),
])
def test_ragged_workloads(name, k_lo, k_hi):
    w, ks, r = _ragged_case(WORKLOADS[name], k_lo, k_hi)
    _check(w, ks, r, k_hi)


def test_ragged_top_k_and_draft_temperature():
    base = replace(WORKLOADS["b256-k8-v152064-f32-peaked-topk50"], B=24, seed=51)
    w, ks, r = _ragged_case(base, 1, 8)
    _check(w, ks, r, 8)
    w2, ks2, r2 = _ragged_case(WORKLOADS["b8-k5-v32000-f32-zipf"], 0, 6, seed=3)
    _check(w2, ks2, r2, 9, Td=0.5)


def test_ragged_equal_lengths_equal_the_rectangular_call():
    w = WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"]
    d = make_inputs(w)
    x = np.zeros((w.B, w.K), dtype=np.int32)
    for i in range(w.K):
        x[:, i] = oracle.sample_tokens(oracle.widen(d["draft"][:, i], w.dtype), w.temperature, w.top_k, w.top_p,
                                       d["draft_u"][:, i])
    a_tok, a_n, a_dbg = run_device(w, d, x, debug=True)
    r = pack_ragged(d, np.full(w.B, w.K))
    b_tok, b_n, b_dbg = run_device_ragged(w, r, x.reshape(-1), w.K)
    assert np.array_equal(a_tok, b_tok) and np.array_equal(a_n, b_n)
    assert np.array_equal(a_dbg["p"].reshape(-1), b_dbg["p"]) and np.array_equal(a_dbg["q"].reshape(-1), b_dbg["q"])
    assert np.array_equal(a_dbg["z"], b_dbg["z"])


def test_ragged_no_drafts_at_all():
    """Every K_b = 0: each sequence only draws its bonus token."""
    w = replace(WORKLOADS["b8-k5-v32000-f32-zipf"], name="b16-k0-v32000-f32-zipf", B=16, seed=8)
    wk, ks, r = _ragged_case(w, 0, 0)
    tok, n, _, _ = _check(wk, ks, r, 3)
    assert np.all(n == 0) and np.all(tok[:, 1:] == -1)


def test_ragged_bad_offsets_then_a_good_call():
    """Offsets that describe no packing give sentinels for every sequence, and
    leave nothing behind that would disturb the next call."""
    w, ks, r = _ragged_case(WORKLOADS["b8-k5-v32000-f32-zipf"], 1, 5, seed=2)
    x = ragged_draft_tokens(w, r)
    cu = r["cu"].copy()
    bad = cu.copy()
    bad[3], bad[4] = bad[4], bad[3]  # a decrease
    assert not oracle.ragged_offsets_ok(bad, int(cu[-1]), 5)
    log(f"[ragged] malformed offsets {bad.tolist()}")
    tok, n, _ = run_device_ragged(w, r, x, 5, cu=bad)
    assert np.all(n == -1) and np.all(tok == -1)
    over = cu.copy()
    over[1:] += 1  # cu[0] = 0 but cu[B] != total drafts
    tok, n, _ = run_device_ragged(w, r, x, 5, cu=over)
    assert np.all(n == -1) and np.all(tok == -1)
    _check(w, ks, r, 5)


def test_closed_loop_draft_length_control():
    """Per-sequence draft lengths chosen by the library's controller from the
    GPU's accepted counts, step after step, against the oracle's controller
    fed by the oracle's verification: identical lengths and outputs."""
    import torch  # noqa: F401

    from rejection_sampling_verify_09_amd import DraftLengthController

    base = replace(WORKLOADS["b8-k5-v32000-f32-zipf"], name="b16-v4096-f32-zipf", B=16, V=4096, draft_sigma=0.4)
    B, k_max = base.B, 8
    ctrl = DraftLengthController(B, window=2, k_min=1, k_max=k_max, k_init=3)
    ref = [oracle.DynamicK(window=2, k_min=1, k_max=k_max, k_init=3) for _ in range(B)]
    ks = np.full(B, 3)
    seen = set()
    for step in range(12):
        w = replace(base, K=k_max, seed=1000 + step)
        r = pack_ragged(make_inputs(w), ks)
        x = ragged_draft_tokens(w, r)
        tok, n = run_device_ragged(w, r, x, k_max, debug=False)
        ref_tok, ref_n = oracle.verify_ragged(r["target"], r["draft"], x, r["uniforms"], r["cu"], w.temperature,
                                              w.top_k, w.top_p, dtype=w.dtype, max_k=k_max)
        assert np.array_equal(tok, ref_tok) and np.array_equal(n, ref_n), step
        nxt = ctrl.observe(n.tolist(), ks.tolist())
        want = [c.observe(int(a), int(k)) for c, a, k in zip(ref, ref_n, ks)]
        assert nxt == want, step
        seen.update(nxt)
        ks = np.array(nxt)
        log(f"   step {step}: mean n {n.mean():.2f}  next K {ks.tolist()}")
    assert len(seen) > 1, "the loop never changed a draft length"
    ctrl.close()


@pytest.mark.parametrize("V,dtype,T,k,p", [
    (4099, "f32", 1.0, 7, 1.0),      # element loads (row length not a multiple of 16 bytes), top-k
    (5003, "bf16", 0.8, 0, 0.95),    # element loads, top-p
    (3001, "f32", 1.0, 0, 1.0),      # unfiltered: the full-row draw per sequence
])
def test_ragged_element_path(V, dtype, T, k, p):
    base = replace(WORKLOADS["b8-k5-v32000-f32-zipf"], name=f"b12-v{V}-{dtype}", B=12, V=V, dtype=dtype,
                   temperature=T, top_k=k, top_p=p, seed=70 + V % 7)
    w, ks, r = _ragged_case(base, 0, 7)
    _check(w, ks, r, 7)


def test_ragged_longest_drafts():
    """K_b up to the 64-draft limit (129 rows for one sequence)."""
    base = replace(WORKLOADS["b8-k5-v32000-f32-zipf"], name="b4-v2048-f32-zipf-k64", B=4, V=2048, seed=77,
                   temperature=0.9, top_p=0.9)
    w, ks, r = _ragged_case(base, 60, 64, seed=1)
    _check(w, ks, r, 64)


def test_ragged_bad_token_is_a_sentinel_for_its_sequence_only():
    w, ks, r = _ragged_case(WORKLOADS["b8-k5-v32000-f32-zipf"], 1, 5, seed=4)
    x = ragged_draft_tokens(w, r)
    b = 3
    x[int(r["cu"][b])] = w.V + 5  # out of range
    tok, n, _ = run_device_ragged(w, r, x, 5)
    assert n[b] == -1 and np.all(tok[b] == -1)
    ref_tok, ref_n = oracle.verify_ragged(r["target"], r["draft"], x, r["uniforms"], r["cu"], w.temperature, w.top_k,
                                          w.top_p, dtype=w.dtype, max_k=5)
    assert np.array_equal(n, ref_n) and np.array_equal(tok, ref_tok)
