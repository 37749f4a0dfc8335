"""Planted mistakes in a copy of the oracle must fail at least one pin.

Each mutant is the oracle's own source with one plausible slip (a sign, an
index, an operand swap, a comparison) applied textually and loaded as a
separate module on the CPU; the real oracle is untouched.  The listed pin must
reject the mutant, which shows the pins can see that class of mistake.
"""
import importlib.util
import os
import types

import pytest

from tests import pins
from tests import test_oracle_ragged as rag

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE, "spec_verify.py")

MUTANTS = {
    # residual with the operands swapped: max(0, q - p)
    "residual_sign": ("np.maximum(0.0, P[idx, nr] - Q[idx, nr])", "np.maximum(0.0, Q[idx, nr] - P[idx, nr])",
                      lambda m: pins.check_lossless(m, "random", N=200_000)),
    # resample from the target instead of the residual
    "resample_from_p": ("res = np.maximum(0.0, P[idx, nr] - Q[idx, nr])", "res = P[idx, nr].copy()",
                        lambda m: pins.check_lossless(m, "random", N=200_000)),
    # accept test with p and q transposed
    "accept_transposed": ("acc = u[:, :K] * qx < px", "acc = u[:, :K] * px < qx",
                          lambda m: pins.check_lossless(m, "random", N=200_000)),
    # non-strict accept comparison
    "accept_le": ("acc = u[:, :K] * qx < px", "acc = u[:, :K] * qx <= px",
                  lambda m: pins.check_zero_weight_never_sampled(m)),
    # the sampling uniform taken from an accept column
    "sample_uniform_index": ("tok, Z = inverse_cdf(w, u[:, K])", "tok, Z = inverse_cdf(w, u[:, 0])",
                             lambda m: pins.check_lossless(m, "close", N=200_000)),
    # bonus drawn from the previous position
    "bonus_row": ("rows_p = P[np.arange(nb), n]", "rows_p = P[np.arange(nb), np.maximum(n - 1, 0)]",
                  lambda m: pins.check_lossless(m, "equal", N=200_000)),
    # first acceptance instead of first rejection
    "first_reject": ("np.argmin(acc, axis=1)", "np.argmax(acc, axis=1)",
                     lambda m: pins.check_accept_count(m, 0.75, 5, N=50_000)),
    # temperature multiplies instead of dividing
    "temperature": ("z = z / T", "z = z * T", lambda m: pins.check_softmax(m)),
    # top-p cut not tie-inclusive
    "topp_ties": ("keep &= pi >= tau[:, None]", "keep &= pi > tau[:, None]", lambda m: pins.check_filters(m)),
    # top-k off by one
    "topk_index": ("kth = np.partition(z, V - k, axis=1)[:, V - k]", "kth = np.partition(z, V - k + 1, axis=1)[:, V - k + 1]",
                   lambda m: pins.check_filters(m)),
    # inverse CDF with a non-strict comparison
    "cdf_le": ("hit = t[:, None] < C", "hit = t[:, None] <= C", lambda m: pins.check_zero_weight_never_sampled(m)),
    # greedy ties to the highest index
    "greedy_ties": ("a = np.argmax(z, axis=1)", "a = z.shape[1] - 1 - np.argmax(z[:, ::-1], axis=1)",
                    lambda m: pins.check_greedy(m)),
    # given draft probabilities used at the wrong position
    "draft_probs_position": ("            Q = draft[s:e]\n", "            Q = np.roll(draft[s:e], 1, axis=1)\n",
                             lambda m: pins.check_lossless_draft_probs(m, N=150_000)),
    # an empty residual drawn from q instead of p
    "empty_residual_from_q": ("res[empty] = P[idx[empty], nr[empty]]", "res[empty] = Q[idx[empty], nr[empty]]",
                              lambda m: pins.check_empty_residual(m)),
    # an empty residual left empty (nothing to draw from)
    "empty_residual_kept_empty": ("res[empty] = P[idx[empty], nr[empty]]", "res[empty] = 0.0",
                                  lambda m: pins.check_empty_residual(m)),
    # ragged: a sequence's uniforms taken from its draft offset, not cu[b] + b
    "ragged_uniform_base": ("U[t_idx]", "U[t_idx - bs[:, None]]",
                            lambda m: rag.check_ragged_worked_case(m)),
    # ragged: target rows taken from the draft offset
    "ragged_target_base": ("target[t_idx]", "target[cu[bs][:, None] + np.arange(K + 1)[None, :]]",
                           lambda m: rag.check_ragged_lossless(m, N=60_000)),
}

# planted mistakes in the language-model-head verification (oracle/lmhead.py)
LMHEAD_MUTANTS = {
    # the draft's logits formed with the target's projection
    "draft_head_weights": ("ld = lm_logits(hidden_d, weight_d, dtype)", "ld = lm_logits(hidden_d, weight_t, dtype)"),
    # the projection's rows taken in reverse vocabulary order
    "vocab_order": ("return np.matmul(h, w.T)", "return np.matmul(h, w[::-1].T)"),
}


@pytest.mark.parametrize("name", sorted(LMHEAD_MUTANTS))
def test_lmhead_mutant_is_caught(name):
    import sys

    from tests import test_oracle_lmhead as lmt

    old, new = LMHEAD_MUTANTS[name]
    path = os.path.join(ORACLE, "lmhead.py")
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1
    # the module imports its siblings relatively: load it as part of the package
    mod = types.ModuleType("oracle.lmhead_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    saved = lmt.oracle
    try:
        shim = types.SimpleNamespace(verify_lmhead=mod.verify_lmhead, lm_logits=mod.lm_logits)
        lmt.oracle = shim
        with pytest.raises(AssertionError):
            lmt.test_one_hot_hidden_selects_a_column()
            lmt.test_lmhead_lossless_chi2()
    finally:
        lmt.oracle = saved


# planted mistakes in the draft-length controller (oracle/dynamic_k.py)
CONTROLLER_MUTANTS = {
    # the window kept across a change of K
    "no_restart": ("            self.k += 1\n            self.hist = []", "            self.k += 1"),
    # non-strict comparison
    "raise_ge": ("rate > self.hi", "rate >= self.hi"),
    # the lower bound ignored
    "lower_bound": ("elif rate < self.lo and self.k > self.k_min:", "elif rate < self.lo:"),
    # a decision before the window is full
    "early": ("if len(self.hist) < self.window:", "if len(self.hist) < 1:"),
}


def _load_mutant(name, old, new, path=SRC):
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new, pin = MUTANTS[name]
    mod = _load_mutant(name, old, new)
    with pytest.raises(AssertionError):
        pin(mod)


def _controller_pins(cls):
    rag.check_controller_hand_trace(cls)
    c = cls(window=2, k_init=5)
    assert [c.observe(4, 5), c.observe(4, 5)] == [5, 5]
    c = cls(window=1, k_min=2, k_init=2)
    assert [c.observe(0, 4), c.observe(0, 4)] == [2, 2]
    # after a raise the window restarts: a second raise needs a full window
    c = cls(window=2, k_init=5)
    assert [c.observe(2, 2) for _ in range(3)] == [5, 6, 6]


@pytest.mark.parametrize("name", sorted(CONTROLLER_MUTANTS))
def test_controller_mutant_is_caught(name):
    old, new = CONTROLLER_MUTANTS[name]
    mod = _load_mutant(name, old, new, os.path.join(ORACLE, "dynamic_k.py"))
    with pytest.raises(AssertionError):
        _controller_pins(mod.DynamicK)


def test_controller_pins_pass_on_the_oracle():
    from oracle.dynamic_k import DynamicK
    _controller_pins(DynamicK)
