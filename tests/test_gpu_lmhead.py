"""GPU parity of verification fed by the output projections
(sv_lm_logits, sv_spec_verify_lmhead) with the fp64 oracle.

Grid inputs (every hidden value a multiple of 2^-3 in [-1, 1], every weight
a multiple of 2^-6 below 4 in magnitude, d <= 8192) make every partial sum
of the float32 accumulation an exactly representable number, so the
device's logits must equal the oracle's float64 logits bit for bit and the
verification is held to the bar of given logits: tokens and counts
identical except flagged near-ties, p(x) and q(x) within 1e-6.  Plain
bfloat16 normals are held to the worst-case float32 summation bound
|fl(sum) - sum| <= gamma_d * sum |h_i w_ji|, gamma_d = d u / (1 - d u),
u = 2^-24 (exact products, d - 1 rounded additions in any order)."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from synth.lmhead import LM_HEADLINE, LM_WORKLOADS, grid_hidden_weight, make_lm_inputs
from tests.harness import (compare_lmhead, lm_draft_tokens, lm_oracle_logits, log, run_device_lmhead,
                           to_device)

pytestmark = pytest.mark.gpu

PROB_TOL = 1e-6
U32 = 2.0 ** -24


def _gamma(d):
    return d * U32 / (1.0 - d * U32)


def _device_logits(Hb, Wb):
    import torch

    from rejection_sampling_verify_09_amd import lm_logits

    out = lm_logits(to_device(Hb, "bf16"), to_device(Wb, "bf16"))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("M,V,d", [
    (1, 1, 64),          # one row, one vocabulary entry: every tile guard
    (9, 3001, 128),      # rows below one 32-row block, a ragged last column tile
    (130, 5000, 192),    # one partial 192-row tile, three k blocks
    (448, 20000, 4096),  # the target's row count and width
    (200, 128256, 256),  # the full vocabulary
    (257, 4099, 8192),   # two 192-row tiles (65 rows in the second), V not a multiple of 4, the widest exact grid
    (130, 3000, 320),    # 192-row tiles, five k blocks: the two-block pipeline's odd tail
    (200, 1500, 448),    # one partial 256-row tile, seven k blocks
    (384, 2049, 2048),   # the draft's row count (two 192-row tiles), one column past a panel
])
def test_lm_logits_exact_on_the_grid(M, V, d):
    g = np.random.default_rng(M * 7 + V + d)
    Hb, Wb = grid_hidden_weight(g, M, V, d)
    log(f"[lm_logits grid] M={M} V={V} d={d}")
    got = _device_logits(Hb, Wb)
    want = oracle.lm_logits(Hb, Wb, "bf16")
    assert got.shape == (M, V)
    bad = np.argwhere(got.astype(np.float64) != want)
    assert bad.size == 0, f"{len(bad)} logits differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,V,d", [(96, 7001, 1024), (33, 1000, 4096), (5, 300, 8192)])
def test_lm_logits_within_the_float32_bound(M, V, d):
    g = np.random.default_rng(M + V + d)
    Hb, Wb = grid_hidden_weight(g, M, V, d, grid=False)
    got = _device_logits(Hb, Wb).astype(np.float64)
    want = oracle.lm_logits(Hb, Wb, "bf16")
    absdot = np.abs(oracle.widen(Hb, "bf16")) @ np.abs(oracle.widen(Wb, "bf16")).T
    err = np.abs(got - want)
    log(f"[lm_logits normal] M={M} V={V} d={d} max err {err.max():.3g} "
        f"max err / bound {np.max(err / (_gamma(d) * absdot + 1e-300)):.3g}")
    assert np.all(err <= _gamma(d) * absdot)


def _check(w, d=None, max_flag=0):
    log(f"[lmhead] {w.name} B={w.B} K={w.K} V={w.V} d={w.d_t}/{w.d_d} T={w.temperature} "
        f"top_k={w.top_k} top_p={w.top_p} grid={w.grid}")
    if d is None:
        d = make_lm_inputs(w)
    log("   inputs drawn; oracle logits")
    lt, ld = lm_oracle_logits(d, w.temperature == 0.0)
    x = lm_draft_tokens(w, ld, d["draft_u"])
    log("   device")
    tok, n, dbg = run_device_lmhead(w, d, x)
    log("   oracle verification")
    stats, fails = compare_lmhead(w, d, lt, ld, x, tok, n, dbg)
    log(f"   match={stats['match']} flagged={stats['flagged']} fail={stats['fail']} "
        f"max|dp|={stats['max_prob_err']:.2e} mean_n={np.mean(n):.3f}")
    assert stats["fail"] == 0, fails[:5]
    assert stats["flagged"] <= max_flag, stats["flags"][:5]
    return tok, n, dbg, stats, lt, ld, x


@pytest.mark.parametrize("name", [
    "lm-b3-k2-v3001-d128-dd64-t0.8-topp0.95",
    "lm-b8-k5-v32000-d1024-dd512-t1.0",
    "lm-b16-k4-v50001-d512-dd256-topk50",
    "lm-b12-k3-v20000-d256-dd128-t0.9-topk40-topp0.8",
])
def test_lmhead_parity_grid(name):
    w = LM_WORKLOADS[name]
    _, _, _, stats, _, _, _ = _check(w)
    assert stats["max_prob_err"] <= PROB_TOL


_FUSED_TOPK = [
    # V % 4 == 0: chunk records from the projections' tile records
    replace(LM_WORKLOADS["lm-b16-k4-v50001-d512-dd256-topk50"], name="lm-b16-k4-v50000-topk50", V=50000, seed=41),
    # 64 < k <= 128: the bound by sorting all tile maxima of a chunk
    replace(LM_WORKLOADS["lm-b12-k3-v20000-d256-dd128-t0.9-topk40-topp0.8"], name="lm-b6-k3-v20000-topk100",
            B=6, top_k=100, top_p=1.0, seed=42),
    # k > 128 tiles per chunk: no bound from the tile maxima, every tile read back
    replace(LM_WORKLOADS["lm-b12-k3-v20000-d256-dd128-t0.9-topk40-topp0.8"], name="lm-b4-k2-v20000-topk200",
            B=4, K=2, top_k=200, top_p=1.0, seed=43),
    # flat rows at T = 1.5: chunks with more candidate units than their list holds
    replace(LM_WORKLOADS["lm-b8-k5-v32000-d1024-dd512-t1.0"], name="lm-b4-k3-v32000-t1.5-topp0.95",
            B=4, K=3, temperature=1.5, top_p=0.95, seed=44),
]


@pytest.mark.parametrize("w", _FUSED_TOPK, ids=lambda w: w.name)
def test_lmhead_parity_fused_filters(w):
    """Filtered rows whose chunk records come from the projections' tile
    records: top-k bounds over tile maxima (both sorting paths and none),
    and top-p chunks whose candidates overflow their list."""
    _, _, _, stats, _, _, _ = _check(w)
    assert stats["max_prob_err"] <= PROB_TOL


_FUSED_EDGES = [
    replace(LM_WORKLOADS["lm-b3-k2-v3001-d128-dd64-t0.8-topp0.95"], name=f"lm-b3-k2-v{V}-{tag}", V=V,
            temperature=T, top_k=k, top_p=p, seed=50 + i)
    for i, (V, tag, T, k, p) in enumerate([
        (68, "topp", 0.8, 0, 0.95),      # two tiles, the second with 4 columns
        (68, "topk3", 1.0, 3, 1.0),
        (8196, "topp", 0.8, 0, 0.95),    # a second chunk of 4 logits in one partial tile
        (8196, "plain", 1.0, 0, 1.0),
        (8196, "greedy", 0.0, 0, 1.0),
        (4, "topp", 1.0, 0, 0.9),        # one tile of 4 columns
    ])
]


@pytest.mark.parametrize("w", _FUSED_EDGES, ids=lambda w: w.name)
def test_lmhead_parity_fused_edges(w):
    """Tile records of partial tiles and of a chunk holding a few logits
    (V % 4 = 0, so the chunk records come from the tile records)."""
    _, _, _, stats, _, _, _ = _check(w)
    assert stats["max_prob_err"] <= PROB_TOL


def test_lmhead_parity_plain_normals():
    """Plain bfloat16 normals: decisions may move only where the float32
    logits' rounding could move them (flagged near-ties), and p(x), q(x)
    stay within the bound the logit error implies:
    |dp| <= p (exp(2 delta / T) - 1), delta the row's worst logit bound."""
    w = LM_WORKLOADS["lm-b8-k5-v32000-d1024-dd512-t1.0-normal"]
    d = make_lm_inputs(w)
    tok, n, dbg, stats, lt, ld, x = _check(w, d, max_flag=1)
    ht = oracle.widen(d["hidden_t"], "bf16")
    hd = oracle.widen(d["hidden_d"], "bf16")
    bt = _gamma(w.d_t) * (np.abs(ht) @ np.abs(oracle.widen(d["weight_t"], "bf16")).T).max(axis=-1)[:, :w.K]
    bd = _gamma(w.d_d) * (np.abs(hd) @ np.abs(oracle.widen(d["weight_d"], "bf16")).T).max(axis=-1)
    ref = stats["ref_dg"]
    tp = ref["px"] * (np.exp(2 * bt / w.temperature) - 1.0)
    tq = ref["qx"] * (np.exp(2 * bd / w.temperature) - 1.0)
    log(f"   max |dp| / bound {np.max(np.abs(dbg['p'] - ref['px']) / tp):.3g}")
    assert np.all(np.abs(dbg["p"] - ref["px"]) <= tp)
    assert np.all(np.abs(dbg["q"] - ref["qx"]) <= tq)


@pytest.mark.timeout(900)
def test_lmhead_headline_parity():
    """B=64, K=6, V=128256, target width 4096, draft width 2048, T=0.7,
    top_p 0.9: the shape the streaming path is measured on, fed by its
    projections."""
    _, _, _, stats, _, _, _ = _check(LM_HEADLINE)
    assert stats["max_prob_err"] <= PROB_TOL


@pytest.mark.timeout(900)
def test_lmhead_greedy_full_vocabulary():
    """Temperature 0: the draft head is not needed (no draft arguments)."""
    _check(LM_WORKLOADS["lm-b32-k6-v128256-d4096-dd2048-greedy"])


def test_lmhead_no_drafts():
    """K = 0: each sequence draws its bonus token from the target head."""
    w = replace(LM_WORKLOADS["lm-b3-k2-v3001-d128-dd64-t0.8-topp0.95"], name="lm-b5-k0-v3001", B=5, K=0, seed=31)
    tok, n, _, _, _, _, _ = _check(w)
    assert np.all(n == 0)


def test_lmhead_equals_logits_then_verify():
    """The fused entry point decides as the projection entry point followed
    by verification of its float32 logits: the same logits, the same tokens
    and counts; its chunk sums come from the projections' tile records
    (V % 4 == 0), so p(x) and q(x) may differ in float rounding, within
    twice the 1e-6 bound each meets against the oracle."""
    import torch

    from rejection_sampling_verify_09_amd import lm_logits, spec_verify

    w = LM_WORKLOADS["lm-b8-k5-v32000-d1024-dd512-t1.0-normal"]
    d = make_lm_inputs(w)
    lt, ld = lm_oracle_logits(d, False)
    x = lm_draft_tokens(w, ld, d["draft_u"])
    tok, n, dbg = run_device_lmhead(w, d, x)
    gt = lm_logits(to_device(d["hidden_t"], "bf16"), to_device(d["weight_t"], "bf16"))
    gd = lm_logits(to_device(d["hidden_d"], "bf16"), to_device(d["weight_d"], "bf16"))
    t2, n2, dbg2 = spec_verify(gt, gd, torch.from_numpy(x).cuda(), torch.from_numpy(d["uniforms"]).cuda(),
                               w.temperature, w.top_k, w.top_p, debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(tok, t2.cpu().numpy()) and np.array_equal(n, n2.cpu().numpy())
    dp = np.abs(dbg["p"] - dbg2["p"].cpu().numpy())
    dq = np.abs(dbg["q"] - dbg2["q"].cpu().numpy())
    log(f"   fused against streamed: max |dp| {np.nanmax(dp):.2e} max |dq| {np.nanmax(dq):.2e}")
    assert np.nanmax(dp) <= 2 * PROB_TOL and np.nanmax(dq) <= 2 * PROB_TOL
    assert np.array_equal(np.isnan(dbg["p"]), np.isnan(dbg2["p"].cpu().numpy()))
