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
    for s in ["sv_spec_verify", "sv_spec_verify_debug", "sv_spec_verify_dt", "sv_spec_verify_ragged",
              "sv_spec_verify_probs", "sv_lm_logits", "sv_spec_verify_lmhead",
              "sv_filtered_probs", "sv_sample", "sv_dynk_create", "sv_dynk_observe", "sv_dynk_k", "sv_dynk_destroy",
              "sv_release", "sv_scratch_bytes", "sv_init", "sv_stream_release", "sv_spec_verify_noalloc",
              "sv_status_string", "sv_version", "sv_profile_start", "sv_profile_stop", "sv_read_floor"]:
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


def test_read_floor_validation():
    lib = L.lib()
    assert lib.sv_read_floor(FAKE, -1, 0, FAKE, None) == L.SV_ERR_SHAPE
    assert lib.sv_read_floor(FAKE, 24, 0, FAKE, None) == L.SV_ERR_SHAPE
    assert lib.sv_read_floor(FAKE, (1 << 62), 0, FAKE, None) == L.SV_ERR_SHAPE
    assert lib.sv_read_floor(None, 0, 0, None, None) == L.SV_OK
    assert lib.sv_read_floor(None, 16, 0, FAKE, None) == L.SV_ERR_NULL
    assert lib.sv_read_floor(FAKE, 16, 0, None, None) == L.SV_ERR_NULL


def test_profile_without_calls_reports_nothing():
    L.profile_start()
    r = L.profile_stop()
    assert r == dict(stream_kernel_ms=0.0, other_kernels_ms=0.0, calls=0)


def test_ragged_validation():
    def f(B=3, N=5, max_k=4, V=16, T=1.0, Td=1.0, dtype=0, cu=FAKE, tgt=FAKE, drf=FAKE, X=FAKE, U=FAKE, out_t=FAKE,
          out_n=FAKE):
        return L.lib().sv_spec_verify_ragged(tgt, drf, X, U, cu, T, Td, 0, 1.0, out_t, out_n, None, None, None, B, N,
                                             max_k, V, dtype, None)
    assert f(B=-1) == L.SV_ERR_SHAPE
    assert f(N=-1) == L.SV_ERR_SHAPE
    assert f(max_k=-1) == L.SV_ERR_SHAPE
    assert f(max_k=L.SV_MAX_K + 1) == L.SV_ERR_SHAPE
    assert f(N=13, max_k=4) == L.SV_ERR_SHAPE       # more drafts than B * max_k
    assert f(V=0) == L.SV_ERR_SHAPE
    assert f(dtype=9) == L.SV_ERR_DTYPE
    assert f(Td=0.0) == L.SV_ERR_PARAM
    assert f(cu=None) == L.SV_ERR_NULL
    assert f(X=None) == L.SV_ERR_NULL
    assert f(drf=None) == L.SV_ERR_NULL
    assert f(U=None) == L.SV_ERR_NULL
    assert f(out_t=None) == L.SV_ERR_NULL
    assert f(out_n=None) == L.SV_ERR_NULL
    # no drafts at all: neither drafted tokens nor draft logits are needed
    assert f(N=0, X=None, drf=None, U=None) == L.SV_ERR_NULL
    # greedy: no draft logits needed
    assert f(T=0.0, drf=None, U=None) == L.SV_ERR_NULL
    assert f(B=0, N=0, cu=None, tgt=None, drf=None, X=None, U=None, out_t=None, out_n=None) == L.SV_OK


def test_controller_matches_the_oracle():
    """The library's controller (host code) against the oracle's on random
    acceptance traces, several lanes at once."""
    import numpy as np
    from oracle import DynamicK
    rng = np.random.default_rng(5)
    for window, lo, hi, kmin, kmax, k0 in [(100, 0.6, 0.8, 2, 10, 5), (3, 0.6, 0.8, 2, 4, 3), (1, 0.5, 0.5, 0, 6, 0),
                                           (7, 0.3, 0.9, 1, 12, 12)]:
        lanes = 6
        c = L.DraftLengthController(lanes, window, hi, lo, kmin, kmax, k0)
        ref = [DynamicK(window, hi, lo, kmin, kmax, k0) for _ in range(lanes)]
        bias = rng.random(lanes)
        for step in range(3000):
            ks = [r.k for r in ref]
            dr = [int(k * rng.integers(0, 3)) if rng.random() < 0.95 else 0 for k in ks]
            acc = [int(rng.binomial(d, bias[i])) for i, d in enumerate(dr)]
            got = c.observe(acc, dr)
            want = [r.observe(a, d) for r, a, d in zip(ref, acc, dr)]
            assert got == want, (window, step)
            if step % 500 == 0:
                bias = rng.random(lanes)
        assert [c.k(i) for i in range(lanes)] == [r.k for r in ref]
        c.close()


def test_controller_errors():
    lib = L.lib()
    assert not lib.sv_dynk_create(0, 100, 0.8, 0.6, 2, 10, 5)
    assert not lib.sv_dynk_create(1, 0, 0.8, 0.6, 2, 10, 5)
    assert not lib.sv_dynk_create(1, 100, 0.5, 0.6, 2, 10, 5)   # lower above raise
    assert not lib.sv_dynk_create(1, 100, 0.8, 0.6, 2, 10, 11)  # start outside [k_min, k_max]
    assert not lib.sv_dynk_create(1, 100, 1.5, 0.6, 2, 10, 5)
    c = L.DraftLengthController(2, window=2, k_init=5)
    with pytest.raises(L.SpecVerifyError):
        c.observe([3, 1], [2, 1])          # accepted above drafted: nothing recorded
    with pytest.raises(L.SpecVerifyError):
        c.observe([-1, 0], [2, 1])
    assert c.observe([2, 2], [2, 2]) == [5, 5]
    assert c.observe([2, 0], [2, 2]) == [6, 4]
    assert lib.sv_dynk_observe(None, None, None, None) == L.SV_ERR_NULL
    assert lib.sv_dynk_k(None, 0) == -1 and c.k(2) == -1 and c.k(0) == 6
    lib.sv_dynk_destroy(None)
    c.close()


def test_probs_validation():
    def f(B=2, K=3, V=16, T=1.0, q=FAKE, X=FAKE, U=FAKE, tgt=FAKE, out_t=FAKE, out_n=FAKE, top_p=1.0):
        return L.lib().sv_spec_verify_probs(tgt, q, X, U, T, 0, top_p, out_t, out_n, None, None, None, B, K, V, 0,
                                            None)
    assert f(B=-1) == L.SV_ERR_SHAPE
    assert f(K=L.SV_MAX_K + 1) == L.SV_ERR_SHAPE
    assert f(top_p=0.0) == L.SV_ERR_PARAM
    assert f(q=None) == L.SV_ERR_NULL
    assert f(X=None) == L.SV_ERR_NULL
    assert f(tgt=None) == L.SV_ERR_NULL
    # greedy and K == 0 need no draft probabilities
    assert f(T=0.0, q=None, U=None) == L.SV_ERR_NULL
    assert f(K=0, q=None, X=None, U=None) == L.SV_ERR_NULL
    assert f(B=0, q=None, X=None, U=None, tgt=None, out_t=None, out_n=None) == L.SV_OK


def test_lm_logits_validation():
    f = L.lib().sv_lm_logits  # (hidden, weight, out_logits, M, V, d, stream)
    odd = ctypes.c_void_p(0x1002)
    assert f(FAKE, FAKE, FAKE, -1, 10, 64, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 0, 64, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 2097153, 64, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 10, 100, None) == L.SV_ERR_SHAPE     # d not a multiple of 64
    assert f(FAKE, FAKE, FAKE, 4, 10, 0, None) == L.SV_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 10, 1 << 17, None) == L.SV_ERR_SHAPE
    assert f(odd, FAKE, FAKE, 4, 10, 64, None) == L.SV_ERR_SHAPE       # operands must be 16-byte aligned
    assert f(FAKE, odd, FAKE, 4, 10, 64, None) == L.SV_ERR_SHAPE
    assert f(None, FAKE, FAKE, 4, 10, 64, None) == L.SV_ERR_NULL
    assert f(FAKE, None, FAKE, 4, 10, 64, None) == L.SV_ERR_NULL
    assert f(FAKE, FAKE, None, 4, 10, 64, None) == L.SV_ERR_NULL
    assert f(None, None, None, 0, 10, 64, None) == L.SV_OK


def test_spec_verify_lmhead_validation():
    v = L.lib().sv_spec_verify_lmhead

    def f(B=2, K=3, V=16, dt=64, dd=128, T=1.0, top_p=1.0, ht=FAKE, wt=FAKE, hd=FAKE, wd=FAKE, X=FAKE, U=FAKE,
          out_t=FAKE, out_n=FAKE):
        return v(ht, wt, hd, wd, X, U, T, 0, top_p, out_t, out_n, None, None, None, B, K, V, dt, dd, None)
    assert f(B=-1) == L.SV_ERR_SHAPE
    assert f(K=L.SV_MAX_K + 1) == L.SV_ERR_SHAPE
    assert f(V=0) == L.SV_ERR_SHAPE
    assert f(dt=96) == L.SV_ERR_SHAPE
    assert f(dd=32) == L.SV_ERR_SHAPE
    assert f(ht=ctypes.c_void_p(0x1008)) == L.SV_ERR_SHAPE
    assert f(T=-1.0) == L.SV_ERR_PARAM
    assert f(top_p=0.0) == L.SV_ERR_PARAM
    assert f(ht=None) == L.SV_ERR_NULL
    assert f(wd=None) == L.SV_ERR_NULL
    assert f(X=None) == L.SV_ERR_NULL
    assert f(U=None) == L.SV_ERR_NULL
    assert f(out_n=None) == L.SV_ERR_NULL
    # greedy needs no draft head (its width is not even checked), the rest is validated
    assert f(T=0.0, hd=None, wd=None, dd=0, U=None) == L.SV_ERR_NULL
    assert f(B=0) == L.SV_OK


def test_lm_bindings_check_their_arguments_before_any_call():
    import torch

    from rejection_sampling_verify_09_amd import lm_logits, spec_verify_lmhead

    h = torch.zeros((2, 64), dtype=torch.bfloat16)
    w = torch.zeros((10, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        lm_logits(h.float(), w)
    with pytest.raises(ValueError):
        lm_logits(h, torch.zeros((10, 128), dtype=torch.bfloat16))
    x = torch.zeros((1, 2), dtype=torch.int32)
    u = torch.zeros((1, 3))
    with pytest.raises(ValueError):  # a draft head is needed at T > 0
        spec_verify_lmhead(torch.zeros((1, 3, 64), dtype=torch.bfloat16), w, None, None, x, u, 1.0)
    with pytest.raises(ValueError):  # draft rows of the wrong count
        spec_verify_lmhead(torch.zeros((1, 3, 64), dtype=torch.bfloat16), w,
                           torch.zeros((1, 3, 64), dtype=torch.bfloat16), w, x, u, 1.0)


def call_noalloc(B=2, K=3, V=16, T=1.0, top_k=0, top_p=1.0, dtype=L.SV_F32):
    return L.lib().sv_spec_verify_noalloc(FAKE, FAKE, FAKE, FAKE, T, top_k, top_p, FAKE, FAKE, B, K, V, dtype, None)


def test_noalloc_validation_and_capacity():
    """The no-allocation entry point validates like sv_spec_verify and refuses,
    before any HIP call, a call whose scratch would exceed its fixed array."""
    assert call_noalloc(B=-1) == L.SV_ERR_SHAPE
    assert call_noalloc(T=-1.0) == L.SV_ERR_PARAM
    assert call_noalloc(dtype=9) == L.SV_ERR_DTYPE
    assert call_noalloc(B=0) == L.SV_OK
    # B = 256, K = 8, V = 152064: far beyond the array
    assert call_noalloc(B=256, K=8, V=152064, top_k=50) == L.SV_ERR_WORKSPACE
    # the largest call the header promises fits (any mode): past the size check
    for k, p in [(0, 0.9), (50, 0.9), (50, 1.0), (0, 1.0)]:
        assert call_noalloc(B=64, K=6, V=128256, T=0.7, top_k=k, top_p=p, dtype=L.SV_BF16) != L.SV_ERR_WORKSPACE
        assert call_noalloc(B=64, K=6, V=128256, T=0.7, top_k=k, top_p=p, dtype=L.SV_F32) != L.SV_ERR_WORKSPACE
    assert L.SV_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_init_validation():
    lib = L.lib()
    assert lib.sv_init(-1, None, 64, 6, 128256, 0) == L.SV_ERR_PARAM
    assert lib.sv_init(64, None, 64, 6, 128256, 0) == L.SV_ERR_PARAM
    assert lib.sv_init(0, None, -1, 6, 128256, 0) == L.SV_ERR_SHAPE
    assert lib.sv_init(0, None, 64, L.SV_MAX_K + 1, 128256, 0) == L.SV_ERR_SHAPE
    assert lib.sv_init(0, None, 64, 6, 0, 0) == L.SV_ERR_SHAPE
    assert lib.sv_init(0, None, 64, 6, 128256, 2) == L.SV_ERR_PARAM
