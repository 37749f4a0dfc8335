"""fp64 CPU oracle for the speculative-sampling verification step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
from .spec_verify import (F64, decide, filtered_probs, inverse_cdf, ragged_offsets_ok, sample,  # noqa: F401
                          sample_tokens, verify, verify_given, verify_one, verify_ragged, widen)
from .dynamic_k import DynamicK  # noqa: F401
from .lmhead import lm_logits, verify_lmhead  # noqa: F401
from .near_tie import classify, classify_sample, at_risk, MATCH, FLAGGED, FAIL  # noqa: F401
from .rate import DrawTables  # noqa: F401
