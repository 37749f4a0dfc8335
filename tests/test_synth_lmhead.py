"""The projection inputs' grid claim: on the grid, a float32 accumulation in
any order gives the exact sum (so device and oracle logits can agree bit for
bit), including the largest magnitudes the grid allows at d = 8192."""
import numpy as np

from synth.gen import bf16_bits_to_f32
from synth.lmhead import GRID_H, GRID_W, MAX_HQ, MAX_WQ, LM_WORKLOADS, grid_hidden_weight, make_lm_inputs


def _exact_in_any_order(H, W):
    """float32 sums in three orders (BLAS, forward, reversed) against the
    float64 sum."""
    ref = H.astype(np.float64) @ W.astype(np.float64).T
    blas = (H @ W.T).astype(np.float64)
    fwd = np.zeros(ref.shape, dtype=np.float32)
    rev = np.zeros(ref.shape, dtype=np.float32)
    d = H.shape[1]
    for i in range(d):
        fwd += np.outer(H[:, i], W[:, i]).astype(np.float32)
        rev += np.outer(H[:, d - 1 - i], W[:, d - 1 - i]).astype(np.float32)
    return np.array_equal(blas, ref) and np.array_equal(fwd.astype(np.float64), ref) and \
        np.array_equal(rev.astype(np.float64), ref)


def test_grid_values_are_exact_bfloat16():
    g = np.random.default_rng(0)
    Hb, Wb = grid_hidden_weight(g, 8, 64, 128)
    H, W = bf16_bits_to_f32(Hb), bf16_bits_to_f32(Wb)
    assert np.all(H * GRID_H == np.rint(H * GRID_H)) and np.all(np.abs(H * GRID_H) <= MAX_HQ)
    assert np.all(W * GRID_W == np.rint(W * GRID_W)) and np.all(np.abs(W * GRID_W) <= MAX_WQ)


def test_float32_accumulation_is_exact_on_the_grid():
    g = np.random.default_rng(1)
    Hb, Wb = grid_hidden_weight(g, 6, 40, 512)
    assert _exact_in_any_order(bf16_bits_to_f32(Hb), bf16_bits_to_f32(Wb))
    # the extreme: every product at its largest magnitude, d = 8192
    d = 8192
    H = np.full((2, d), MAX_HQ / GRID_H, dtype=np.float32)
    W = np.full((3, d), MAX_WQ / GRID_W, dtype=np.float32)
    W[1] *= -1
    W[2, ::2] *= -1
    assert _exact_in_any_order(H, W)


def test_plain_normals_do_round():
    """Off the grid the float32 sums round (the other test family)."""
    g = np.random.default_rng(2)
    Hb, Wb = grid_hidden_weight(g, 6, 40, 512, grid=False)
    assert not _exact_in_any_order(bf16_bits_to_f32(Hb), bf16_bits_to_f32(Wb))


def test_workload_inputs_on_the_grid():
    w = LM_WORKLOADS["lm-b3-k2-v3001-d128-dd64-t0.8-topp0.95"]
    d = make_lm_inputs(w)
    assert d["hidden_t"].shape == (3, 3, 128) and d["weight_t"].shape == (3001, 128)
    assert d["hidden_d"].shape == (3, 2, 64) and d["weight_d"].shape == (3001, 64)
    for k, sc, lim in (("hidden_t", GRID_H, MAX_HQ), ("hidden_d", GRID_H, MAX_HQ), ("weight_t", GRID_W, MAX_WQ),
                       ("weight_d", GRID_W, MAX_WQ)):
        x = bf16_bits_to_f32(d[k]) * sc
        assert np.all(x == np.rint(x)) and np.all(np.abs(x) <= lim), k
    # deterministic
    d2 = make_lm_inputs(w)
    assert all(np.array_equal(d[k], d2[k]) for k in d)
