"""Verification fed by the language-model head: logits = hidden states times
the output projection, then the verification step of ``spec_verify``.

TEST INFRASTRUCTURE ONLY (see ``oracle/spec_verify.py``).

Each decoding step runs the model forward up to its output projection and
then samples, and its time goes to reading the weights (page
www.2kiu.com/news/5895634 §1; page www.cf-1.com/news/5155685 §2.1).  The
target scores all K+1 positions in one forward (page www.gsyq.cn/news/428210
§3.1); its output projection W [V, d] maps each position's hidden state h
(length d) to V logits, logit_j = sum_i h_i W[j, i].  The
oracle forms those logits in float64 from exactly widened inputs (a product
of two bfloat16 values is exact in float64; the sums round only at float64
precision) and hands them to ``spec_verify.verify`` unchanged.

Reading: the draft's logits come from its own hidden states and its own
projection (a smaller model may have another width d_d); both share the
vocabulary (page www.2kiu.com/news/5895634 §4.1: same-family pairs).
"""
from __future__ import annotations

import numpy as np

from .spec_verify import F64, verify, widen


def lm_logits(hidden, weight, dtype: str) -> np.ndarray:
    """hidden [..., d], weight [V, d] (float32, or uint16 bf16 patterns with
    dtype == "bf16") -> float64 logits [..., V]."""
    h = widen(hidden, dtype)
    w = widen(weight, dtype)
    if h.shape[-1] != w.shape[1]:
        raise ValueError("hidden width and weight width differ")
    return np.matmul(h, w.T)


def verify_lmhead(hidden_t, weight_t, hidden_d, weight_d, draft_tokens, uniforms, temperature, top_k, top_p,
                  dtype: str = "f32", diag: bool = False):
    """hidden_t [B, K+1, d], weight_t [V, d]; hidden_d [B, K, d_d], weight_d
    [V, d_d] (draft unused at temperature 0, may then be None).  Returns
    ``verify``'s results on the float64 logits."""
    lt = lm_logits(hidden_t, weight_t, dtype)
    B, K1, V = lt.shape
    if hidden_d is None or float(np.float32(temperature)) == 0.0:
        ld = np.zeros((B, K1 - 1, V))
    else:
        ld = lm_logits(hidden_d, weight_d, dtype)
    return verify(lt, ld, draft_tokens, uniforms, temperature, top_k, top_p, dtype=F64, diag=diag)
