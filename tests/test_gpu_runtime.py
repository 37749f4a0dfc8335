"""GPU behaviour of the library around the kernels: calls on a side stream,
scratch growth and release between calls of different sizes, the launch
timing API, and the accepted-count law on device outputs (truncated
geometric at an exact per-position alpha; page www.gsyq.cn/news/428210 §3.2)."""
import numpy as np
import pytest

import oracle
from synth import WORKLOADS, Workload, make_inputs
from tests import pins
from tests.harness import compare, draft_tokens_for, log, run_device, to_device

pytestmark = pytest.mark.gpu


def _dev_inputs(w, d, x):
    import torch

    return (to_device(d["target"], w.dtype), to_device(d["draft"], w.dtype), torch.from_numpy(x).cuda(),
            torch.from_numpy(d["uniforms"]).cuda())


def test_side_stream_gives_the_same_results():
    import torch

    from rejection_sampling_verify_09_amd import spec_verify

    w = WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"]
    d = make_inputs(w)
    x = draft_tokens_for(w, d)
    tgt, drf, X, U = _dev_inputs(w, d, x)
    ref = [t.clone() for t in spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p, stream=side)
    side.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_scratch_grows_and_is_released():
    """A small call, a larger one (the scratch grows), a release, and a small
    call again: every result matches the oracle."""
    import torch

    from rejection_sampling_verify_09_amd import lib, release

    dev = torch.cuda.current_device()
    for name in ["b8-k5-v32000-f32-zipf", "b64-k6-v128256-bf16-zipf-t0.7-topp0.9", "b8-k5-v32000-f32-zipf"]:
        w = WORKLOADS[name]
        log(f"[scratch] {name} held {lib().sv_scratch_bytes(dev)} bytes")
        d = make_inputs(w)
        x = draft_tokens_for(w, d)
        tok, n, dbg = run_device(w, d, x)
        stats, fails = compare(w, d, x, tok, n, dbg)
        assert stats["fail"] == 0 and stats["flagged"] == 0, fails[:3]
        held = lib().sv_scratch_bytes(dev)
        assert held > 0
        if name.startswith("b64"):
            release()
            assert lib().sv_scratch_bytes(dev) == 0


def test_profile_counts_every_call():
    import torch

    from rejection_sampling_verify_09_amd import profile_start, profile_stop, spec_verify

    w = WORKLOADS["b8-k5-v32000-f32-zipf"]
    d = make_inputs(w)
    x = draft_tokens_for(w, d)
    tgt, drf, X, U = _dev_inputs(w, d, x)
    profile_start()
    for _ in range(7):
        spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p)
    torch.cuda.synchronize()
    r = profile_stop()
    assert r["calls"] == 7
    assert r["stream_kernel_ms"] > 0.0 and r["other_kernels_ms"] > 0.0
    # timing stopped: later calls are not counted
    spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p)
    torch.cuda.synchronize()
    profile_start()
    assert profile_stop()["calls"] == 0


@pytest.mark.parametrize("alpha,K", [(0.75, 5), (0.5, 3)])
def test_accept_count_law_on_device(alpha, K):
    """Rows with sum_x min(p, q) = alpha at every position: the device's
    accepted counts are truncated geometric, and their mean matches the
    closed form 1 + a + ... + a^K."""
    import torch

    from rejection_sampling_verify_09_amd import spec_verify

    class Device:
        @staticmethod
        def verify(t, dl, x, u, T, k, p):
            tok, n = spec_verify(torch.from_numpy(np.ascontiguousarray(t)).cuda(),
                                 torch.from_numpy(np.ascontiguousarray(dl)).cuda(),
                                 torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda(),
                                 torch.from_numpy(np.ascontiguousarray(u)).cuda(), T, k, p)
            return tok.cpu().numpy(), n.cpu().numpy()

    log(f"[count law] alpha={alpha} K={K}")
    mean, se, E = pins.check_accept_count(Device, alpha, K, N=400_000, seed=17)
    log(f"   mean emitted {mean:.4f} (se {se:.4f}) closed form {E:.4f}")


def test_small_batch_after_large_batch_rectangular_and_ragged():
    """Alternating entry points and sizes on one scratch buffer."""
    from dataclasses import replace

    from synth import pack_ragged, ragged_lengths
    from tests.harness import compare_ragged, ragged_draft_tokens, run_device_ragged

    big = WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"]
    small = Workload("b3-k2-v3000-f32", 3, 2, 3000, "f32", "normal", 2.0, 0.5, 0.9, 0, 0.95, 33)
    for w in (big, small, replace(small, B=5, seed=34)):
        d = make_inputs(w)
        x = draft_tokens_for(w, d)
        tok, n, dbg = run_device(w, d, x)
        stats, fails = compare(w, d, x, tok, n, dbg)
        assert stats["fail"] == 0 and stats["flagged"] == 0, fails[:3]
        wr = replace(w, name=w.name + "-ragged")
        r = pack_ragged(d, ragged_lengths(w.B, 0, w.K, w.seed))
        xr = ragged_draft_tokens(wr, r)
        tok, n, dbg = run_device_ragged(wr, r, xr, w.K)
        stats, fails = compare_ragged(wr, r, xr, w.K, tok, n, dbg)
        assert stats["fail"] == 0 and stats["flagged"] == 0, fails[:3]


def _expected(w, d, x):
    """The oracle's results for a batch (all sequences must match exactly:
    the batches used here have no near-tie)."""
    return oracle.verify(d["target"], d["draft"], x, d["uniforms"], w.temperature, w.top_k, w.top_p, dtype=w.dtype)


def test_concurrent_streams_match_the_oracle():
    """Two streams of default priority verify different batches at the same
    time, with no ordering between them (each stream has its own scratch):
    every call on both equals the oracle."""
    import torch

    from rejection_sampling_verify_09_amd import spec_verify

    ws = [WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"], WORKLOADS["b32-k6-v128256-bf16-normal-s0.6"]]
    batches = []
    for w in ws:
        d = make_inputs(w)
        x = draft_tokens_for(w, d)
        ref_tok, ref_n = _expected(w, d, x)
        batches.append((w, _dev_inputs(w, d, x), ref_tok, ref_n))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    reps = 12
    outs = [[], []]
    for r in range(reps):
        for i, (w, (tgt, drf, X, U), _, _) in enumerate(batches):
            with torch.cuda.stream(streams[i]):
                outs[i].append(spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p, stream=streams[i]))
    torch.cuda.synchronize()
    for i, (w, _, ref_tok, ref_n) in enumerate(batches):
        log(f"[streams] {w.name}: {reps} calls on stream {i}")
        for tok, n in outs[i]:
            assert np.array_equal(n.cpu().numpy(), ref_n) and np.array_equal(tok.cpu().numpy(), ref_tok)


def test_concurrent_host_threads_on_their_own_streams():
    """Two host threads, each with its own stream and batch, calling at the
    same time: both match the oracle."""
    import threading

    import torch

    from rejection_sampling_verify_09_amd import spec_verify

    ws = [WORKLOADS["b8-k5-v32000-f32-zipf"], WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"]]
    res, errs = {}, []

    def work(i, w, d, x):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            tgt, drf, X, U = _dev_inputs(w, d, x)
            s.wait_stream(torch.cuda.current_stream())
            outs = []
            with torch.cuda.stream(s):
                for _ in range(10):
                    outs.append(spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p, stream=s))
            s.synchronize()
            res[i] = [(t.cpu().numpy(), n.cpu().numpy()) for t, n in outs]
        except Exception as e:  # reported below
            errs.append(repr(e))

    inputs = []
    for w in ws:
        d = make_inputs(w)
        inputs.append((w, d, draft_tokens_for(w, d)))
    th = [threading.Thread(target=work, args=(i, *inp)) for i, inp in enumerate(inputs)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not errs, errs
    for i, (w, d, x) in enumerate(inputs):
        ref_tok, ref_n = _expected(w, d, x)
        log(f"[threads] {w.name}: {len(res[i])} calls")
        for tok, n in res[i]:
            assert np.array_equal(n, ref_n) and np.array_equal(tok, ref_tok)


def test_init_sizes_the_stream_scratch_once():
    """After sv_init on a stream, calls within its bounds (every variant and
    mode) leave the library's scratch unchanged: no allocation."""
    import torch

    from rejection_sampling_verify_09_amd import init, sample, scratch_bytes, spec_verify, stream_release

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    init(64, 8, 152064, stream=s)
    held = scratch_bytes()
    log(f"[init] scratch after sv_init: {held} bytes")
    cases = [WORKLOADS["b64-k6-v128256-bf16-zipf-t0.7-topp0.9"], WORKLOADS["b8-k5-v32000-f32-zipf"],
             WORKLOADS["b32-k6-v128256-bf16-normal-greedy"],
             Workload("b16-k8-v152064-topk", 16, 8, 152064, "f32", "peaked", 2.5, 0.6, 1.0, 50, 1.0, 3)]
    with torch.cuda.stream(s):
        for w in cases:
            d = make_inputs(w)
            x = draft_tokens_for(w, d)
            tgt, drf, X, U = _dev_inputs(w, d, x)
            tok, n = spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p, stream=s)
            s.synchronize()
            ref_tok, ref_n = _expected(w, d, x)
            assert np.array_equal(n.cpu().numpy(), ref_n) and np.array_equal(tok.cpu().numpy(), ref_tok)
            rows = drf.reshape(-1, w.V)
            sample(rows, torch.rand(rows.shape[0], device="cuda"), max(w.temperature, 0.5), w.top_k, w.top_p,
                   stream=s)
            s.synchronize()
            assert scratch_bytes() == held, (w.name, scratch_bytes(), held)
    stream_release(s)
    assert scratch_bytes() < held


def test_read_floor_reads_every_block():
    """sv_read_floor: the xor of each 16 KiB block's words, taken on the
    host, is the key that makes the kernel write that block's word (and no
    other); a tail block shorter than 16 KiB is read up to the end only."""
    import torch

    from rejection_sampling_verify_09_amd import read_floor

    rng = np.random.default_rng(5)
    nbytes = 5 * 16384 + 4096 + 48
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    data = torch.from_numpy(words.view(np.int32)).cuda()
    nblk = -(-nbytes // 16384)
    xors = [int(np.bitwise_xor.reduce(words[i * 4096:(i + 1) * 4096])) for i in range(nblk)]
    for blk in (0, 3, nblk - 1):
        out = torch.full((nblk,), 7, dtype=torch.int32, device="cuda")
        read_floor(data, key=xors[blk], out=out)
        got = out.cpu().numpy().view(np.uint32)
        want = np.full(nblk, 7, dtype=np.uint32)
        want[[i for i in range(nblk) if xors[i] == xors[blk]]] = xors[blk]
        log(f"[read floor] block {blk} of {nblk}")
        assert np.array_equal(got, want)
