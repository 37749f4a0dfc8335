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

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "spec_verify.py")

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
}


def _load_mutant(name, old, new):
    with open(SRC) as f:
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
