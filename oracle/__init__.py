"""fp64 CPU oracle for the speculative-sampling verification step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
from .spec_verify import (F64, filtered_probs, inverse_cdf, ragged_offsets_ok, sample, sample_tokens, verify,  # noqa: F401
                          verify_one, verify_ragged, widen)
from .dynamic_k import DynamicK  # noqa: F401
from .lmhead import lm_logits, verify_lmhead  # noqa: F401
from .near_tie import classify, classify_sample, at_risk, MATCH, FLAGGED, FAIL  # noqa: F401
