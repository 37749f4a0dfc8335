"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Token ids and accepted counts must be identical except for flagged near-ties
(the first differing decision within 1e-5 of its boundary); probabilities of
the drafted tokens and full filtered rows within 1e-6 absolute.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, Workload, make_inputs
from tests import pins
from tests.harness import compare, draft_tokens_for, log, run_device, to_device

pytestmark = pytest.mark.gpu

PROB_TOL = 1e-6


def _check(w: Workload, d=None, x=None, max_flagged=0):
    log(f"[parity] {w.name} B={w.B} K={w.K} V={w.V} {w.dtype} T={w.temperature} top_k={w.top_k} top_p={w.top_p}")
    if d is None:
        d = make_inputs(w)
    if x is None:
        x = draft_tokens_for(w, d)
    tok, n, dbg = run_device(w, d, x, debug=True)
    stats, fails = compare(w, d, x, tok, n, dbg)
    log(f"   match={stats['match']} flagged={stats['flagged']} fail={stats['fail']} "
        f"max|dp|={stats['max_prob_err']:.2e} oracle={stats['oracle_s']:.1f}s mean_n={np.mean(n):.3f}")
    for b, why in fails[:10]:
        log(f"   FAIL seq {b}: {why}")
    for b, why in stats["flags"][:5]:
        log(f"   flagged seq {b}: {why}")
    assert stats["fail"] == 0, fails[:5]
    assert stats["flagged"] <= max_flagged
    assert stats["max_prob_err"] <= PROB_TOL
    return tok, n


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    _check(WORKLOADS[name])


SMALL = [
    # (B, K, V, dtype, shape, T, top_k, top_p)
    (64, 3, 8, "f32", "normal", 1.0, 0, 1.0),
    (50, 2, 1, "f32", "normal", 1.0, 0, 1.0),
    (17, 0, 1000, "f32", "normal", 1.0, 0, 1.0),
    (33, 4, 1001, "f32", "normal", 0.8, 0, 1.0),        # unaligned rows: element loads
    (33, 4, 1001, "bf16", "zipf", 0.8, 0, 0.9),
    (9, 5, 8193, "bf16", "normal", 1.3, 0, 1.0),        # one logit into a second chunk
    (9, 5, 16384, "f32", "peaked", 1.0, 20, 1.0),
    (12, 3, 20000, "bf16", "zipf", 0.7, 40, 0.8),       # top-k then top-p
    (12, 3, 20000, "f32", "zipf", 1.0, 0, 0.5),
    (20, 6, 5000, "bf16", "normal", 0.0, 0, 1.0),       # greedy
    (20, 6, 5000, "f32", "peaked", 0.0, 7, 0.3),        # greedy ignores the filters
    (6, 2, 3000, "f32", "normal", 2.0, 1, 1.0),         # top-k = 1
    (6, 2, 40000, "bf16", "zipf", 0.5, 300, 1.0),       # top-k > 256: full-row threshold
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}-K{}-V{}-{}-{}-T{}-k{}-p{}".format(*c))
def test_small_shapes(case):
    B, K, V, dt, shape, T, k, p = case
    w = Workload(f"small-{B}-{K}-{V}", B, K, V, dt, shape, 2.0 if shape != "zipf" else 1.0, 0.7, T, k, p, 11)
    _check(w)


LARGEST = [
    # (B, K, V, dtype, shape, T, top_k, top_p): the boundary's largest vocabulary
    # (256 chunks of 8192, 4096 draw segments per row) and drafts per sequence
    (2, 2, 2097152, "bf16", "zipf", 0.8, 0, 0.9),
    (2, 1, 2097152, "f32", "normal", 1.0, 50, 1.0),
    (2, 2, 2097152, "bf16", "normal", 1.0, 0, 1.0),      # unfiltered: the full-row draw's tail
    (3, 64, 1024, "f32", "zipf", 1.0, 0, 0.9),           # 129 rows a sequence
    (2, 64, 1024, "bf16", "normal", 1.0, 0, 1.0),
]


@pytest.mark.parametrize("case", LARGEST, ids=lambda c: "B{}-K{}-V{}-{}-{}-T{}-k{}-p{}".format(*c))
def test_largest_shapes(case):
    B, K, V, dt, shape, T, k, p = case
    w = Workload(f"largest-{B}-{K}-{V}", B, K, V, dt, shape, 2.0 if shape != "zipf" else 1.0, 0.7, T, k, p, 12)
    _check(w)


def test_flat_rows_take_the_full_row_paths():
    """Nearly uniform rows: the top-p nucleus is thousands of tokens (beyond
    the candidate window and the kept-list capacity)."""
    w = Workload("flat", 4, 3, 30000, "f32", "normal", 0.05, 0.05, 1.0, 0, 0.9, 21)
    _check(w)
    w = Workload("flat-topk", 4, 2, 30000, "bf16", "normal", 0.05, 0.05, 1.0, 2000, 1.0, 22)
    _check(w)
    w = Workload("flat-topk-topp", 3, 2, 30000, "f32", "normal", 0.05, 0.05, 1.0, 500, 0.7, 23)
    _check(w)


def test_nucleus_below_the_window():
    """Broad rows whose top-p nucleus reaches below the candidate window but
    whose cut region is sparse: the two-pass full-row cut decides them (kept
    sets that fit a list, and ones that do not), in both dtypes."""
    for w in [Workload("wide-list", 6, 3, 3000, "f32", "normal", 3.5, 0.5, 1.0, 0, 0.9, 31),
              Workload("wide-big", 4, 3, 30000, "f32", "normal", 3.0, 0.5, 1.0, 0, 0.9, 32),
              Workload("wide-bf16", 4, 4, 32000, "bf16", "normal", 3.0, 0.7, 1.0, 0, 0.85, 33),
              Workload("wide-t07", 4, 3, 20000, "f32", "normal", 2.0, 0.5, 0.7, 0, 0.95, 34)]:
        log(f"[nucleus below window] {w.name}")
        _check(w)


def test_ties_at_the_cut():
    """bf16-coarse logits with many equal values: top-k and top-p keep whole tie groups."""
    rng = np.random.default_rng(5)
    B, K, V = 16, 3, 4096
    base = np.round(rng.normal(0, 2, (B, K + 1, V)) * 2) / 2
    tgt = base.astype(np.float32)
    drf = (base[:, :K] + np.round(rng.normal(0, 1, (B, K, V)) * 2) / 2).astype(np.float32)
    for (T, k, p) in [(1.0, 10, 1.0), (1.0, 0, 0.6), (0.9, 25, 0.9)]:
        w = Workload("ties", B, K, V, "f32", "normal", 1, 1, T, k, p, 0)
        d = dict(target=tgt, draft=drf, uniforms=rng.random((B, K + 1), dtype=np.float32),
                 draft_u=rng.random((B, K)))
        _check(w, d=d)


def test_sentinel_rows():
    rng = np.random.default_rng(3)
    B, K, V = 6, 3, 2000
    for T, k, p in [(1.0, 0, 1.0), (0.8, 0, 0.9), (1.0, 30, 1.0), (0.0, 0, 1.0)]:
        w = Workload("sentinel", B, K, V, "f32", "normal", 2, 0.5, T, k, p, 0)
        d = make_inputs(w)
        x = draft_tokens_for(w, d)
        d["target"][1, 2] = -np.inf  # a target row with no distribution
        x[2, 0] = V + 5              # a drafted token out of range
        x[4, 2] = -1
        d["draft"][3, 1] = -np.inf   # a draft row with no distribution (irrelevant at T = 0)
        d["target"][5, :, ::2] = -np.inf  # masked tokens are fine
        tok, n = _check(w, d=d, x=x)
        assert n[1] == -1 and n[2] == -1 and n[4] == -1
        assert (n[3] == -1) == (T != 0.0)
        assert np.all(tok[n == -1] == -1)


def test_deterministic_across_calls():
    import torch
    from rejection_sampling_verify_09_amd import spec_verify

    for name in ["b64-k6-v128256-bf16-zipf-t0.7-topp0.9", "b8-k5-v32000-f32-zipf"]:
        w = WORKLOADS[name]
        log(f"[determinism] {name}")
        d = make_inputs(w)
        x = draft_tokens_for(w, d)
        tgt, drf = to_device(d["target"], w.dtype), to_device(d["draft"], w.dtype)
        X = torch.from_numpy(x).cuda()
        U = torch.from_numpy(d["uniforms"]).cuda()
        outs = [tuple(o.clone() for o in spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p))
                for _ in range(5)]
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])


@pytest.mark.parametrize("mode", [(1.0, 0, 1.0), (0.7, 0, 0.9), (1.0, 50, 1.0), (0.8, 40, 0.8)])
def test_filtered_probs_within_tolerance(mode):
    import torch
    from rejection_sampling_verify_09_amd import filtered_probs

    T, k, p = mode
    for dt, shape in [("bf16", "zipf"), ("f32", "peaked")]:
        w = Workload("probs", 4, 2, 50000, dt, shape, 2.0, 0.5, T, k, p, 9)
        d = make_inputs(w)
        rows = d["target"].reshape(-1, w.V)
        log(f"[probs] {dt} {shape} T={T} k={k} p={p}")
        got = filtered_probs(to_device(rows, dt), T, k, p).cpu().numpy()
        ref = oracle.filtered_probs(oracle.widen(rows, dt), T, k, p)
        assert np.array_equal(got > 0, ref > 0), "kept sets differ"
        assert np.abs(got.astype(np.float64) - ref).max() <= PROB_TOL


@pytest.mark.parametrize("case", ["random", "close", "equal", "disjoint", "masked"])
def test_gpu_lossless_chi2(case):
    """The emitted token at every position follows p, on GPU outputs."""
    import torch
    from rejection_sampling_verify_09_amd import spec_verify

    V, K, N = 8, 3, 1_000_000
    tl, dl = pins.lossless_case(case, V, K, 11)
    P, Q = pins.softmax_rows(tl), pins.softmax_rows(dl)
    rng = np.random.default_rng(12)
    x = np.stack([rng.choice(V, size=N, p=Q[i]) for i in range(K)], axis=1).astype(np.int32)
    u = rng.random((N, K + 1), dtype=np.float32)
    log(f"[chi2] {case} N={N}")
    tgt = torch.from_numpy(tl).cuda().expand(N, K + 1, V).contiguous()
    drf = torch.from_numpy(dl).cuda().expand(N, K, V).contiguous()
    tok, n = spec_verify(tgt, drf, torch.from_numpy(x).cuda(), torch.from_numpy(u).cuda(), 1.0, 0, 1.0)
    tok, n = tok.cpu().numpy(), n.cpu().numpy()
    assert np.all((n >= 0) & (n <= K))
    for j in range(K + 1):
        sel = n >= j
        if sel.sum() < 1000:
            continue
        pv = pins._chi2_pvalue(np.bincount(tok[sel, j], minlength=V), P[j])
        assert pv > pins.CHI2_MIN_P, (case, j, pv)
    # the device agrees with the oracle on a slice of the same inputs
    m = 20000
    ref_tok, ref_n = oracle.verify(tl[None].repeat(m, 0), dl[None].repeat(m, 0), x[:m], u[:m], 1.0, 0, 1.0)
    assert np.array_equal(ref_n, n[:m]) and np.array_equal(ref_tok, tok[:m])


def test_top_p_just_below_one():
    """top_p = 1 - 2^-24 (the largest float32 below 1): the nucleus is the
    whole row but for its least probable tokens, and the device's mass sums may
    fall just short of top_p.  No failure is allowed; sequences whose kept set
    differs only at that boundary are near-ties (top_p moved by 1e-5)."""
    tp = float(np.nextafter(np.float32(1.0), np.float32(0.0)))
    for dt in ("f32", "bf16"):
        w = Workload(f"topp-near-one-{dt}", 8, 3, 3000, dt, "normal", 2.0, 0.5, 1.0, 0, tp, 31)
        _check(w, max_flagged=w.B)
