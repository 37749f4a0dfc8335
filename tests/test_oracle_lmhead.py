"""Pins of the oracle's language-model-head verification (logits formed from
hidden states and the output projection, then verified): a hidden state that
selects one coordinate gives that column of the projection as the logits;
doubling the hidden states and the temperature together changes nothing (the
scaled logit x / T is the same number); and the emitted tokens follow p."""
import numpy as np

import oracle
from oracle import spec_verify as sv
from synth import f32_to_bf16_bits
from tests import pins


def test_one_hot_hidden_selects_a_column():
    rng = np.random.default_rng(3)
    B, K, V, d = 4, 3, 40, 12
    Wt = rng.normal(0, 1, (V, d)).astype(np.float32)
    Wd = rng.normal(0, 1, (V, d)).astype(np.float32)
    it = rng.integers(0, d, (B, K + 1))
    idd = rng.integers(0, d, (B, K))
    ht = np.eye(d, dtype=np.float32)[it]
    hd = np.eye(d, dtype=np.float32)[idd]
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1), dtype=np.float32)
    for T, k, p in ((1.0, 0, 1.0), (0.7, 0, 0.9), (1.0, 5, 1.0), (0.0, 0, 1.0)):
        got = oracle.verify_lmhead(ht, Wt, hd, Wd, x, u, T, k, p)
        lt = Wt.T[it]          # [B, K+1, V]: column it of the projection
        ld = Wd.T[idd]
        want = sv.verify(lt, ld, x, u, T, k, p)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    # bf16 inputs: the same selection, from bit patterns
    Wb = f32_to_bf16_bits(Wt)
    hb = f32_to_bf16_bits(ht)
    lb = oracle.lm_logits(hb, Wb, "bf16")
    assert np.array_equal(lb, sv.widen(Wb, "bf16").T[it])


def test_scaling_hidden_and_temperature_together():
    rng = np.random.default_rng(5)
    B, K, V, d = 6, 4, 64, 16
    Wt = rng.normal(0, 0.5, (V, d)).astype(np.float32)
    Wd = rng.normal(0, 0.5, (V, d)).astype(np.float32)
    ht = rng.normal(0, 1, (B, K + 1, d)).astype(np.float32)
    hd = (ht[:, :K] + rng.normal(0, 0.3, (B, K, d))).astype(np.float32)
    x = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1), dtype=np.float32)
    for T, k, p in ((1.0, 0, 1.0), (0.5, 0, 0.9), (1.0, 8, 1.0)):
        a = oracle.verify_lmhead(ht, Wt, hd, Wd, x, u, T, k, p, diag=True)
        b = oracle.verify_lmhead(2 * ht, Wt, 2 * hd, Wd, x, u, 2 * T, k, p, diag=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert np.array_equal(a[2]["px"], b[2]["px"]) and np.array_equal(a[2]["Z"], b[2]["Z"])


def test_lmhead_lossless_chi2():
    """Drafts drawn from the draft head's q; emitted tokens follow the target
    head's p at every position."""
    rng = np.random.default_rng(9)
    V, K, d, N = 8, 3, 6, 200_000
    Wt = rng.normal(0, 1, (V, d)).astype(np.float32)
    Wd = (Wt + rng.normal(0, 0.4, (V, d))).astype(np.float32)
    ht = rng.normal(0, 1, (K + 1, d)).astype(np.float32)
    hd = ht[:K].copy()
    P = pins.softmax_rows(oracle.lm_logits(ht, Wt, "f32").astype(np.float64))
    Q = pins.softmax_rows(oracle.lm_logits(hd, Wd, "f32").astype(np.float64))
    x = np.stack([rng.choice(V, size=N, p=Q[i]) for i in range(K)], axis=1)
    u = rng.random((N, K + 1), dtype=np.float32)
    tok, n = oracle.verify_lmhead(pins.tile_rows(ht, N), Wt, pins.tile_rows(hd, N), Wd, x, u, 1.0, 0, 1.0)
    for j in range(K + 1):
        sel = n >= j
        assert pins._chi2_pvalue(np.bincount(tok[sel, j], minlength=V), P[j]) > pins.CHI2_MIN_P
