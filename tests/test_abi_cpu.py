"""The C-ABI library loads and exports what include/specverify.h declares;
argument validation answers before any HIP call (CPU, no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

from rejection_sampling_verify_09_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ["sv_spec_verify", "sv_spec_verify_debug", "sv_spec_verify_dt", "sv_filtered_probs", "sv_sample",
              "sv_release", "sv_scratch_bytes",
              "sv_status_string", "sv_version", "sv_profile_start", "sv_profile_stop"]:
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for s in declared_symbols():
        assert hasattr(lib, s), f"{s} is declared but not exported"


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.sv_version() >= 100
    for code in range(-6, 1):
        assert L.status_string(code).startswith("SV_")
    assert L.status_string(123) == "unknown status"
    assert lib.sv_scratch_bytes(0) == 0
    assert lib.sv_scratch_bytes(-1) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def call_verify(B=2, K=3, V=16, T=1.0, top_k=0, top_p=1.0, dtype=L.SV_F32, tgt=FAKE, drf=FAKE, X=FAKE, U=FAKE,
                out_t=FAKE, out_n=FAKE):
    return L.lib().sv_spec_verify(tgt, drf, X, U, T, top_k, top_p, out_t, out_n, B, K, V, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), L.SV_ERR_SHAPE),
    (dict(K=-1), L.SV_ERR_SHAPE),
    (dict(K=L.SV_MAX_K + 1), L.SV_ERR_SHAPE),
    (dict(V=0), L.SV_ERR_SHAPE),
    (dict(V=2097153), L.SV_ERR_SHAPE),
    (dict(dtype=7), L.SV_ERR_DTYPE),
    (dict(T=-0.5), L.SV_ERR_PARAM),
    (dict(T=float("nan")), L.SV_ERR_PARAM),
    (dict(T=float("inf")), L.SV_ERR_PARAM),
    (dict(T=1e-45), L.SV_ERR_PARAM),
    (dict(top_k=-3), L.SV_ERR_PARAM),
    (dict(top_p=0.0), L.SV_ERR_PARAM),
    (dict(top_p=1.5), L.SV_ERR_PARAM),
    (dict(top_p=float("nan")), L.SV_ERR_PARAM),
    (dict(tgt=None), L.SV_ERR_NULL),
    (dict(drf=None), L.SV_ERR_NULL),
    (dict(X=None), L.SV_ERR_NULL),
    (dict(U=None), L.SV_ERR_NULL),
    (dict(out_t=None), L.SV_ERR_NULL),
    (dict(out_n=None), L.SV_ERR_NULL),
    (dict(B=1 << 30, K=64, V=1 << 20), L.SV_ERR_SHAPE),
    (dict(B=1 << 17, K=64, V=1 << 20), L.SV_ERR_SHAPE),
])
def test_validation_codes(kw, code):
    assert call_verify(**kw) == code


def test_empty_batch_touches_nothing():
    assert call_verify(B=0, tgt=None, drf=None, X=None, U=None, out_t=None, out_n=None) == L.SV_OK


def test_greedy_does_not_need_draft_logits_but_validates_the_rest():
    # at T = 0 a NULL draft pointer is accepted; a NULL uniforms pointer is not
    assert call_verify(T=0.0, drf=None, U=None) == L.SV_ERR_NULL


def test_filtered_probs_validation():
    f = L.lib().sv_filtered_probs
    assert f(FAKE, -1, 10, 0, 1.0, 0, 1.0, FAKE, None) == L.SV_ERR_SHAPE
    assert f(FAKE, 4, 0, 0, 1.0, 0, 1.0, FAKE, None) == L.SV_ERR_SHAPE
    assert f(FAKE, 4, 10, 2, 1.0, 0, 1.0, FAKE, None) == L.SV_ERR_DTYPE
    assert f(FAKE, 4, 10, 0, 0.0, 0, 1.0, FAKE, None) == L.SV_ERR_PARAM
    assert f(None, 4, 10, 0, 1.0, 0, 1.0, FAKE, None) == L.SV_ERR_NULL
    assert f(None, 0, 10, 0, 1.0, 0, 1.0, None, None) == L.SV_OK


def test_sample_validation():
    f = L.lib().sv_sample  # (logits, uniforms, T, top_k, top_p, out_tokens, out_prob, rows, V, dtype, stream)
    assert f(FAKE, FAKE, 1.0, 0, 1.0, FAKE, None, -1, 10, 0, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, 1.0, 0, 1.0, FAKE, None, 4, 0, 0, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, 1.0, 0, 1.0, FAKE, None, 4, 2097153, 0, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, 1.0, 0, 1.0, FAKE, None, 4, 10, 5, None) == L.SV_ERR_DTYPE
    assert f(FAKE, FAKE, -1.0, 0, 1.0, FAKE, None, 4, 10, 0, None) == L.SV_ERR_PARAM
    assert f(FAKE, FAKE, 1.0, 0, 2.0, FAKE, None, 4, 10, 0, None) == L.SV_ERR_PARAM
    assert f(None, FAKE, 1.0, 0, 1.0, FAKE, None, 4, 10, 0, None) == L.SV_ERR_NULL
    assert f(FAKE, None, 1.0, 0, 1.0, FAKE, None, 4, 10, 0, None) == L.SV_ERR_NULL
    assert f(FAKE, FAKE, 1.0, 0, 1.0, None, None, 4, 10, 0, None) == L.SV_ERR_NULL
    # greedy draws need neither draft logits nor drafted tokens, but the rest is validated
    assert f(FAKE, None, 0.0, 0, 1.0, FAKE, None, 4, 10, 0, None) == L.SV_ERR_NULL
    assert f(None, None, 1.0, 0, 1.0, None, None, 0, 10, 0, None) == L.SV_OK


def test_draft_temperature_validation():
    def f(T=1.0, Td=0.5, B=2, out_n=FAKE):
        return L.lib().sv_spec_verify_dt(FAKE, FAKE, FAKE, FAKE, T, Td, 0, 1.0, FAKE, out_n, None, None, None, B, 3,
                                         16, 0, None)
    assert f(Td=0.0) == L.SV_ERR_PARAM            # a sampling draft needs a temperature above 0
    assert f(Td=-1.0) == L.SV_ERR_PARAM
    assert f(Td=float("nan")) == L.SV_ERR_PARAM
    assert f(Td=float("inf")) == L.SV_ERR_PARAM
    assert f(B=-1) == L.SV_ERR_SHAPE
    assert f(out_n=None) == L.SV_ERR_NULL
    assert f(B=0) == L.SV_OK


def test_profile_without_calls_reports_nothing():
    L.profile_start()
    r = L.profile_stop()
    assert r == dict(stream_kernel_ms=0.0, other_kernels_ms=0.0, calls=0)
