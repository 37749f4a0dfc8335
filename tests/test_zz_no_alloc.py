"""The entry point that allocates nothing (sv_spec_verify_noalloc), through
the C ABI, against sv_spec_verify on the same inputs: identical tokens and
counts on two calls in a row, the second with a smaller batch (the fixed
array keeps the first call's contents, which the second must not depend on).
"""
import numpy as np
import pytest

from synth import WORKLOADS, Workload, make_inputs
from tests.harness import draft_tokens_for, log, to_device

pytestmark = pytest.mark.gpu


def _inputs(w):
    import torch

    d = make_inputs(w)
    x = draft_tokens_for(w, d)
    return (to_device(d["target"], w.dtype), to_device(d["draft"], w.dtype), torch.from_numpy(x).cuda(),
            torch.from_numpy(d["uniforms"]).cuda())


def test_noalloc_matches_spec_verify_on_two_calls():
    import torch

    from rejection_sampling_verify_09_amd._lib import SV_BF16, SV_F32, SV_OK, lib, spec_verify

    L = lib()
    big = WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"]
    small = Workload("b5-k3-v20000-f32-topk", 5, 3, 20000, "f32", "peaked", 2.0, 0.5, 0.9, 30, 0.95, 41)
    for w in (big, small):
        log(f"[noalloc] {w.name}")
        tgt, drf, X, U = _inputs(w)
        ref_tok, ref_n = spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p)
        out_t = torch.full((w.B, w.K + 1), -7, dtype=torch.int32, device="cuda")
        out_n = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
        st = L.sv_spec_verify_noalloc(tgt.data_ptr(), drf.data_ptr(), X.data_ptr(), U.data_ptr(),
                                      float(w.temperature), int(w.top_k), float(w.top_p), out_t.data_ptr(),
                                      out_n.data_ptr(), w.B, w.K, w.V, SV_BF16 if w.dtype == "bf16" else SV_F32,
                                      torch.cuda.current_stream().cuda_stream)
        assert st == SV_OK
        torch.cuda.synchronize()
        assert torch.equal(out_n, ref_n) and torch.equal(out_t, ref_tok)
        log(f"   identical: mean n {out_n.float().mean().item():.3f}")
