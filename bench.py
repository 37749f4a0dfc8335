"""Benchmark of the speculative-sampling verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --sampler [--steps K] [--warmup W] [--workload NAME]
    python bench.py --draft-temperature TD [--steps K] [--warmup W] [--workload NAME]
    python bench.py --ragged K_LO K_HI [--steps K] [--warmup W] [--workload NAME]
    python bench.py --draft-probs [--steps K] [--warmup W] [--workload NAME]
    python bench.py --lmhead [--steps K] [--warmup W] [--workload NAME]

One step = one sv_spec_verify call (the whole hot path: streaming pass,
filter thresholds, accept tests, first-rejection scan, final draw) over one
batch whose logits are already resident in HBM.  The input batch is rotated
over several device copies whose total exceeds the 256 MB last-level cache,
so every step reads its logits from HBM.  Prints one JSON line.

With --ragged K_LO K_HI, one step is one sv_spec_verify_ragged call over a
batch whose sequences draft K_b ~ uniform[K_LO, K_HI] tokens each (drafts
drawn on the GPU before timing).

With --draft-probs, one step is one sv_spec_verify_probs call (the draft
distributions given as float32 probabilities; only the target rows are
streamed).

With --sampler, one step is one sv_sample call (the drafting draw: x ~ q and
q(x)) over the workload's B*K draft rows, with their draft uniforms.  With
--draft-temperature, the drafts are drawn on the GPU (sv_sample) at that
temperature before timing, and one step is one sv_spec_verify_dt call.

With --lmhead, one step is one sv_spec_verify_lmhead call: the target's and
the draft's output projections (bf16 hidden states times bf16 weights on the
matrix cores) and the verification of their float32 logits; its roofline is
the projection kernel against the bf16 matrix peak.

The CPU-baseline leg times the fp64 oracle (test infrastructure) on a bounded
sample of the same workload; it is a reported baseline, not the target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "rejection_sampling_verify_09_amd", "csrc", f)
                  for f in ("sv_common.hpp", "sv_kernels.hip")]
LM_SOURCES = [os.path.join(ROOT, "rejection_sampling_verify_09_amd", "csrc", f) for f in ("sv_lmhead.hip", "sv_common.hpp")]
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_draft_tokens(name: str, B: int, K: int):
    import numpy as np

    path = os.path.join(ROOT, "tests", "golden", "draft_tokens", f"{name}.txt")
    rows = [list(map(int, ln.split())) for ln in open(path) if ln.strip() and not ln.startswith("#")]
    x = np.array(rows, dtype=np.int32).reshape(B, K)
    return x


def measured_traffic(key: str, kernel: str = "stream_kernel", sources=None):
    """HBM bytes per launch of ``kernel`` (the streaming kernel unless named)
    from the committed counter summary for ``key`` (the workload name,
    "sample-" + name for the draft draw, "ragged-LO-HI-" + name for a ragged
    batch, "probs-" + name for q given as probabilities, the projection
    workload's name for "lm_gemm", the two projections), or None when the summary is absent
    or predates the kernel source."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{key}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_bytes.group(1))


CPU_SHARE = 16  # host threads one GPU's job may use on the GPU hosts


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline_single(w, d, x, budget_s: float, draft_temperature=None):
    """Time the fp64 oracle on whole batches of the workload, in this
    process, until about budget_s has been spent (at least one batch)."""
    import numpy as np

    import oracle

    sample_B = w.B
    t0 = time.perf_counter()
    n_done = 0
    toks = 0
    while True:
        tok, n = oracle.verify(d["target"], d["draft"], x, d["uniforms"], w.temperature, w.top_k, w.top_p,
                               dtype=w.dtype, draft_temperature=draft_temperature)
        n_done += sample_B
        toks += int(np.sum(n + 1))
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=n_done / el, unit="sequences/s", cores=1, kind="oracle", cpu=cpu_model(),
                sample=f"{n_done // sample_B} x the full {sample_B}-sequence batch of {w.name}, "
                       f"fp64 NumPy, single thread, {el:.1f} s", tokens_per_s=toks / el)


_CPU_JOB = {}


def _cpu_one_sequence(b: int) -> int:
    """One sequence of the batch in _CPU_JOB through the oracle (a worker of
    the all-cores leg; the batch reaches it by fork)."""
    import oracle

    w, d, x = _CPU_JOB["w"], _CPU_JOB["d"], _CPU_JOB["x"]
    _, n = oracle.verify(d["target"][b:b + 1], d["draft"][b:b + 1], x[b:b + 1], d["uniforms"][b:b + 1],
                         w.temperature, w.top_k, w.top_p, dtype=w.dtype)
    return int(n[0])


def cpu_baseline(w, d, x, budget_s: float):
    """The fp64 oracle on all the host cores this job may use: one forked
    worker per core (at most CPU_SHARE), each verifying whole sequences of
    the batch, over repeated passes of the batch until about budget_s.  Must
    run before this process initialises the GPU."""
    import multiprocessing as mp

    visible = len(os.sched_getaffinity(0))
    workers = max(1, min(visible, CPU_SHARE))
    _CPU_JOB.update(w=w, d=d, x=x)
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_cpu_one_sequence, range(min(w.B, workers)), chunksize=1)  # workers import the oracle
        t0 = time.perf_counter()
        n_done = 0
        while True:
            n_done += len(pool.map(_cpu_one_sequence, range(w.B), chunksize=1))
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    _CPU_JOB.clear()
    return dict(value=n_done / el, unit="sequences/s", cores=workers, kind="oracle", cpu=cpu_model(),
                cores_visible=visible,
                sample=f"{n_done // w.B} x the full {w.B}-sequence batch of {w.name}, one sequence per task, "
                       f"{workers} forked workers (fp64 NumPy, one thread each), {el:.1f} s")


def _percentiles(ms):
    import numpy as np

    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "calls": int(a.size)}


def measure_verify(w, d, x, steps: int, warmup: int, copies: int, Td=None) -> dict:
    """Time sv_spec_verify on one batch of workload w (logits resident in
    HBM, rotated over enough copies to defeat the last-level cache).  Three
    timed regions of `steps` calls each: back to back (the step time),
    with the library's launch timing (the streaming kernel's duration), and
    one event pair around each call (the per-call distribution)."""
    import numpy as np
    import torch

    from rejection_sampling_verify_09_amd import profile_start, profile_stop, spec_verify

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    tgt0 = dev(d["target"])
    drf0 = dev(d["draft"]) if w.K > 0 else None
    bytes_per_step = w.logit_bytes  # every logit the step must read, once
    R = copies or max(3, -(-640_000_000 // bytes_per_step))
    tgts = [tgt0] + [tgt0.clone() for _ in range(R - 1)]
    drfs = [drf0] + [drf0.clone() for _ in range(R - 1)] if drf0 is not None else [None] * R
    X = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    U = torch.from_numpy(d["uniforms"]).cuda()
    out_t = torch.empty((w.B, w.K + 1), dtype=torch.int32, device="cuda")
    out_n = torch.empty((w.B,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        spec_verify(tgts[i % R], drfs[i % R], X, U, w.temperature, w.top_k, w.top_p, out_tokens=out_t,
                    out_num_accepted=out_n, draft_temperature=Td)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # region 1 (the step time): `steps` calls back to back, events on the
    # launch stream around the whole loop
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_per_step = ev0.elapsed_time(ev1) / steps

    # region 2 (the roofline): the library records HIP events around its
    # streaming kernel on the launch stream, so that kernel's own average
    # duration is measured live (the extra event records would inflate the
    # step time, hence a region of their own)
    profile_start()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prof = profile_stop()
    stream_ms = prof["stream_kernel_ms"] / max(1, prof["calls"])
    other_ms = prof["other_kernels_ms"] / max(1, prof["calls"])

    # region 3 (per-call distribution): an event pair around each call
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (e0, e1) in enumerate(pairs):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_call = _percentiles([e0.elapsed_time(e1) for e0, e1 in pairs])

    n_host = out_n.cpu().numpy()
    emitted = int(np.sum(n_host[n_host >= 0] + 1))
    del tgts, drfs
    return {
        "value": w.B / (ms_per_step / 1e3),
        "ms_per_step": ms_per_step,
        "per_call_ms": per_call,
        "wall_s_timed": t_wall,
        "tokens_per_s": emitted / (ms_per_step / 1e3),
        "mean_emitted_per_sequence": emitted / w.B,
        "bytes_per_step": bytes_per_step,
        "input_copies": R,
        "achieved": bytes_per_step / (stream_ms / 1e3) / 1e9,  # the streaming kernel reads every logit once
        "kernel_ms": stream_ms,
        "other_kernels_ms": other_ms,
        "timed_calls": prof["calls"],
        "step_frac": bytes_per_step / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
    }


def read_floor_leg(nbytes: int, steps: int, warmup: int, stream_kernel_ms: float) -> dict:
    """The plain-read floor (sv_read_floor) over as many bytes as one step
    streams, one launch per step over rotating copies, each launch timed by
    an event pair on the launch stream."""
    import torch

    from rejection_sampling_verify_09_amd import read_floor

    R = max(3, -(-640_000_000 // nbytes))
    bufs = [torch.empty((nbytes,), dtype=torch.uint8, device="cuda").fill_(1 + i % 250) for i in range(R)]
    outs = [torch.zeros((-(-nbytes // 16384),), dtype=torch.int32, device="cuda") for _ in range(R)]
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        read_floor(bufs[i % R], out=outs[i % R])
    torch.cuda.synchronize()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (e0, e1) in enumerate(pairs):
        e0.record(stream)
        read_floor(bufs[i % R], out=outs[i % R])
        e1.record(stream)
    torch.cuda.synchronize()
    pc = _percentiles([e0.elapsed_time(e1) for e0, e1 in pairs])
    del bufs, outs
    gbs = nbytes / (pc["mean"] / 1e3) / 1e9
    return {"kernel": "read_kernel (sv_read_floor)", "what": "one plain read of the step's logit bytes with the "
            "streaming kernel's 16-byte buffer loads and nothing else", "bytes": nbytes, "ms": pc["mean"],
            "ms_p50": pc["p50"], "achieved": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "stream_kernel_over_floor": stream_kernel_ms / pc["mean"]}


def cpu_baseline_sample(w, rows, u, budget_s: float):
    """Time the fp64 oracle's draw on the draft rows until about budget_s."""
    import oracle

    t0 = time.perf_counter()
    n_done = 0
    while True:
        oracle.sample(rows, w.temperature, w.top_k, w.top_p, u.astype("float64"), w.dtype)
        n_done += rows.shape[0]
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=n_done / el, unit="rows/s", cores=1, kind="oracle",
                sample=f"{n_done // rows.shape[0]} x the {rows.shape[0]} draft rows of {w.name}, fp64 NumPy, "
                       f"single thread, {el:.1f} s")


def run_sampler(args, w, d):
    """The drafting draw over the workload's B*K draft rows."""
    import numpy as np
    import torch

    from rejection_sampling_verify_09_amd import profile_start, profile_stop, sample

    rows_np = d["draft"].reshape(w.B * w.K, w.V)
    u_np = d["draft_u"].reshape(-1).astype(np.float32)
    n_rows = rows_np.shape[0]
    esz = 2 if w.dtype == "bf16" else 4
    bytes_per_step = n_rows * w.V * esz

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    L0 = dev(rows_np)
    R = args.copies or max(3, -(-640_000_000 // bytes_per_step))
    Ls = [L0] + [L0.clone() for _ in range(R - 1)]
    U = torch.from_numpy(u_np).cuda()
    out_t = torch.empty((n_rows,), dtype=torch.int32, device="cuda")
    out_p = torch.empty((n_rows,), dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        sample(Ls[i % R], U, w.temperature, w.top_k, w.top_p, out_tokens=out_t, out_prob=out_p)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    profile_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = profile_stop()
    stream_ms = prof["stream_kernel_ms"] / max(1, prof["calls"])
    other_ms = prof["other_kernels_ms"] / max(1, prof["calls"])
    achieved = bytes_per_step / (stream_ms / 1e3) / 1e9
    result = {
        "metric": f"draft-draw rows/s + % HBM peak at {n_rows} rows V={w.V} {w.dtype}",
        "value": n_rows / (ms_per_step / 1e3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded draft logits of the workload's shape; no model weights)",
        "config": {"workload": f"draft rows of {w.name}", "rows": n_rows, "V": w.V, "logits": w.dtype,
                   "temperature": w.temperature, "top_k": w.top_k, "top_p": w.top_p, "input_copies": R,
                   "logit_bytes_per_step": bytes_per_step},
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("sample-" + w.name),
            "kernel": "stream_kernel", "kernel_ms": stream_ms, "other_kernels_ms": other_ms,
            "timed_calls": prof["calls"],
            "step_frac": bytes_per_step / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_sample(w, rows_np, u_np, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_ragged(args, w, k_lo: int, k_hi: int):
    """Verification of a batch whose sequences draft between k_lo and k_hi
    tokens each (sv_spec_verify_ragged), rows cut from the workload drawn at
    K = k_hi; the drafts are drawn on the GPU before timing."""
    from dataclasses import replace

    import numpy as np
    import torch

    from rejection_sampling_verify_09_amd import profile_start, profile_stop, sample, spec_verify_ragged
    from synth import make_inputs, pack_ragged, ragged_lengths

    wk = replace(w, K=k_hi)
    ks = ragged_lengths(w.B, k_lo, k_hi, w.seed)
    r = pack_ragged(make_inputs(wk), ks)
    N = int(r["cu"][-1])
    esz = 2 if w.dtype == "bf16" else 4
    rows = (N + w.B) + (0 if w.temperature == 0.0 else N)
    bytes_per_step = rows * w.V * esz

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    tgt0, drf0 = dev(r["target"]), dev(r["draft"])
    ud = torch.from_numpy(r["draft_u"].astype(np.float32)).cuda()
    xt, _ = sample(drf0, ud, w.temperature, w.top_k, w.top_p, with_prob=False)  # x ~ q, not timed
    R = args.copies or max(3, -(-640_000_000 // bytes_per_step))
    tgts = [tgt0] + [tgt0.clone() for _ in range(R - 1)]
    drfs = [drf0] + [drf0.clone() for _ in range(R - 1)]
    U = torch.from_numpy(r["uniforms"]).cuda()
    CU = torch.from_numpy(r["cu"]).cuda()
    out_t = torch.empty((w.B, k_hi + 1), dtype=torch.int32, device="cuda")
    out_n = torch.empty((w.B,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        spec_verify_ragged(tgts[i % R], drfs[i % R], xt, U, CU, k_hi, w.temperature, w.top_k, w.top_p,
                           out_tokens=out_t, out_num_accepted=out_n)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    profile_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = profile_stop()
    stream_ms = prof["stream_kernel_ms"] / max(1, prof["calls"])
    other_ms = prof["other_kernels_ms"] / max(1, prof["calls"])
    n_host = out_n.cpu().numpy()
    emitted = int(np.sum(n_host[n_host >= 0] + 1))
    achieved = bytes_per_step / (stream_ms / 1e3) / 1e9
    result = {
        "metric": f"spec-verify sequences/s + % HBM peak at B={w.B} K_b in [{k_lo},{k_hi}] V={w.V} {w.dtype} "
                  "(ragged)",
        "value": w.B / (ms_per_step / 1e3),
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded logits of the workload's shape; no model weights)",
        "config": {"workload": f"{w.name} with K_b uniform in [{k_lo}, {k_hi}]", "B": w.B, "total_drafts": N,
                   "mean_K": N / w.B, "V": w.V, "logits": w.dtype, "temperature": w.temperature, "top_k": w.top_k,
                   "top_p": w.top_p, "rows": rows, "input_copies": R, "logit_bytes_per_step": bytes_per_step},
        "tokens_per_s": emitted / (ms_per_step / 1e3),
        "mean_emitted_per_sequence": emitted / w.B,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(f"ragged-{k_lo}-{k_hi}-{w.name}"),
            "kernel": "stream_kernel", "kernel_ms": stream_ms, "other_kernels_ms": other_ms,
            "timed_calls": prof["calls"],
            "step_frac": bytes_per_step / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        },
    }
    if not args.no_cpu_baseline:
        import oracle

        x = xt.cpu().numpy()
        t0 = time.perf_counter()
        n_done = 0
        while True:
            oracle.verify_ragged(r["target"], r["draft"], x, r["uniforms"], r["cu"], w.temperature, w.top_k,
                                 w.top_p, dtype=w.dtype, max_k=k_hi)
            n_done += w.B
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        result["cpu_baseline"] = dict(value=n_done / el, unit="sequences/s", cores=1, kind="oracle",
                                      sample=f"{n_done // w.B} x the full ragged {w.B}-sequence batch, fp64 NumPy, "
                                             f"single thread, {el:.1f} s")
    print(json.dumps(result), flush=True)


def run_probs(args, w):
    """Verification with the draft distributions given as probabilities
    (sv_spec_verify_probs).  q is the draft rows' filtered distribution, made
    by the library (sv_filtered_probs) and the drafts are drawn from the
    draft logits (sv_sample), both before timing; only the target rows are
    streamed."""
    import numpy as np
    import torch

    from rejection_sampling_verify_09_amd import (filtered_probs, profile_start, profile_stop, sample,
                                                  spec_verify_probs)
    from synth import make_inputs

    d = make_inputs(w)
    esz = 2 if w.dtype == "bf16" else 4
    bytes_per_step = w.B * (w.K + 1) * w.V * esz  # every target logit once; q is read only where needed

    def dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    drows = dev(d["draft"].reshape(w.B * w.K, w.V))
    Q = filtered_probs(drows, w.temperature, w.top_k, w.top_p).reshape(w.B, w.K, w.V)
    ud = torch.from_numpy(d["draft_u"].reshape(-1).astype(np.float32)).cuda()
    xt, _ = sample(drows, ud, w.temperature, w.top_k, w.top_p, with_prob=False)
    X = xt.reshape(w.B, w.K).contiguous()
    del drows
    tgt0 = dev(d["target"])
    R = args.copies or max(3, -(-640_000_000 // (bytes_per_step + Q.numel() * 4)))
    tgts = [tgt0] + [tgt0.clone() for _ in range(R - 1)]
    Qs = [Q] + [Q.clone() for _ in range(R - 1)]
    U = torch.from_numpy(d["uniforms"]).cuda()
    out_t = torch.empty((w.B, w.K + 1), dtype=torch.int32, device="cuda")
    out_n = torch.empty((w.B,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        spec_verify_probs(tgts[i % R], Qs[i % R], X, U, w.temperature, w.top_k, w.top_p, out_tokens=out_t,
                          out_num_accepted=out_n)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    profile_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = profile_stop()
    stream_ms = prof["stream_kernel_ms"] / max(1, prof["calls"])
    other_ms = prof["other_kernels_ms"] / max(1, prof["calls"])
    n_host = out_n.cpu().numpy()
    emitted = int(np.sum(n_host[n_host >= 0] + 1))
    achieved = bytes_per_step / (stream_ms / 1e3) / 1e9
    result = {
        "metric": f"spec-verify sequences/s + % HBM peak at B={w.B} K={w.K} V={w.V} {w.dtype} (q as probabilities)",
        "value": w.B / (ms_per_step / 1e3),
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded logits of the workload's shape; no model weights)",
        "config": {"workload": f"{w.name} with q given as float32 probabilities", "B": w.B, "K": w.K, "V": w.V,
                   "logits": w.dtype, "temperature": w.temperature, "top_k": w.top_k, "top_p": w.top_p,
                   "rows": w.B * (w.K + 1), "input_copies": R, "logit_bytes_per_step": bytes_per_step},
        "tokens_per_s": emitted / (ms_per_step / 1e3),
        "mean_emitted_per_sequence": emitted / w.B,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(f"probs-{w.name}"),
            "kernel": "stream_kernel", "kernel_ms": stream_ms, "other_kernels_ms": other_ms,
            "timed_calls": prof["calls"],
            "step_frac": bytes_per_step / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        },
    }
    if not args.no_cpu_baseline:
        import oracle

        Qh, xh = Q.cpu().numpy(), X.cpu().numpy()
        t0 = time.perf_counter()
        n_done = 0
        while True:
            oracle.verify(d["target"], None, xh, d["uniforms"], w.temperature, w.top_k, w.top_p, dtype=w.dtype,
                          draft_probs=Qh)
            n_done += w.B
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        result["cpu_baseline"] = dict(value=n_done / el, unit="sequences/s", cores=1, kind="oracle",
                                      sample=f"{n_done // w.B} x the full {w.B}-sequence batch with given q, "
                                             f"fp64 NumPy, single thread, {el:.1f} s")
    print(json.dumps(result), flush=True)


def run_lmhead(args):
    """Verification fed by the output projections (sv_spec_verify_lmhead):
    the target's B(K+1) hidden states times its projection, the draft's BK
    times its own, then verification.  The drafts are drawn on the GPU
    (sv_lm_logits of the draft rows, then sv_sample) before timing.  The two
    projections (lm_gemm_w8<4> for the target's 448 rows, lm_gemm_w8<3> for
    the draft's 384, whose epilogues also write the tile records the chunk
    records are formed from) are the dominant work; the
    weights (more than the 256 MB last-level cache) are read from HBM at
    every step."""
    import numpy as np
    import torch

    from rejection_sampling_verify_09_amd import lm_logits, profile_start, profile_stop, sample, spec_verify_lmhead
    from synth.lmhead import LM_HEADLINE, LM_WORKLOADS, make_lm_inputs

    w = LM_WORKLOADS[args.workload] if args.workload else LM_HEADLINE
    d = make_lm_inputs(w)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    ht, wt, hd, wd = dev(d["hidden_t"]), dev(d["weight_t"]), dev(d["hidden_d"]), dev(d["weight_d"])
    ud = torch.from_numpy(d["draft_u"].reshape(-1).astype(np.float32)).cuda()
    if w.K > 0:
        ql = lm_logits(hd.reshape(w.B * w.K, w.d_d), wd)
        xt, _ = sample(ql, ud, w.temperature, w.top_k, w.top_p, with_prob=False)
        X = xt.reshape(w.B, w.K).contiguous()
        del ql
    else:
        X = torch.empty((w.B, 0), dtype=torch.int32, device="cuda")
    U = torch.from_numpy(d["uniforms"]).cuda()
    greedy = w.temperature == 0.0
    mt, md = w.B * (w.K + 1), (0 if greedy else w.B * w.K)
    flops = 2.0 * (mt * w.V * w.d_t + md * w.V * w.d_d)
    w_bytes = 2 * w.V * (w.d_t + (0 if greedy else w.d_d))
    stream = torch.cuda.current_stream()
    out = [None, None]

    def step(i):
        out[0], out[1] = spec_verify_lmhead(ht, wt, None if greedy else hd, None if greedy else wd, X, U,
                                            w.temperature, w.top_k, w.top_p)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    profile_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = profile_stop()
    gemm_ms = prof["stream_kernel_ms"] / max(1, prof["calls"])
    other_ms = prof["other_kernels_ms"] / max(1, prof["calls"])
    n_host = out[1].cpu().numpy()
    emitted = int(np.sum(n_host[n_host >= 0] + 1))
    achieved = flops / (gemm_ms / 1e3) / 1e12
    result = {
        "metric": f"spec-verify sequences/s at B={w.B} K={w.K} V={w.V}, logits from bf16 projections "
                  f"(d={w.d_t}, draft d={w.d_d})",
        "value": w.B / (ms_per_step / 1e3),
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded hidden states and projection weights of the workload's shape; no model weights)",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "V": w.V, "d_target": w.d_t, "d_draft": w.d_d,
                   "temperature": w.temperature, "top_k": w.top_k, "top_p": w.top_p,
                   "projection_flops_per_step": flops, "weight_bytes_per_step": w_bytes},
        "tokens_per_s": emitted / (ms_per_step / 1e3),
        "mean_emitted_per_sequence": emitted / w.B,
        "roofline": {
            "bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK_TFS,
            "traffic": measured_traffic(w.name, "lm_gemm", LM_SOURCES),
            "kernel": "lm_gemm_w8<4> + lm_gemm_w8<3> (the target's and the draft's projections together, "
                      "with their tile records); other_kernels_ms: tile_chunk_kernel and the sequence kernel",
            "kernel_ms": gemm_ms,
            "other_kernels_ms": other_ms, "timed_calls": prof["calls"],
            "weight_read_GBs": w_bytes / (gemm_ms / 1e3) / 1e9,
        },
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        import oracle

        nb = min(4, w.B)
        t0 = time.perf_counter()
        n_done = 0
        with threadpool_limits(limits=1):
            while True:
                oracle.verify_lmhead(d["hidden_t"][:nb], d["weight_t"], d["hidden_d"][:nb], d["weight_d"],
                                     X[:nb].cpu().numpy(), d["uniforms"][:nb], w.temperature, w.top_k, w.top_p,
                                     dtype="bf16")
                n_done += nb
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        result["cpu_baseline"] = dict(value=n_done / el, unit="sequences/s", cores=1, kind="oracle",
                                      sample=f"{n_done // nb} x {nb} sequences of {w.name} (projections in "
                                             f"float64 and verification), NumPy, one BLAS thread, {el:.1f} s")
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--copies", type=int, default=0, help="device copies of the inputs (0 = enough for 640 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload measurements that follow the headline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--sampler", action="store_true",
                    help="measure the drafting draw (sv_sample) over the workload's draft rows instead")
    ap.add_argument("--draft-temperature", type=float, default=None,
                    help="verify drafts drawn (on the GPU) at this temperature (sv_spec_verify_dt)")
    ap.add_argument("--draft-probs", action="store_true",
                    help="verify with the draft distributions given as probabilities (sv_spec_verify_probs)")
    ap.add_argument("--ragged", type=int, nargs=2, metavar=("K_LO", "K_HI"), default=None,
                    help="verify a batch whose sequences draft K_b ~ uniform[K_LO, K_HI] tokens "
                         "(sv_spec_verify_ragged)")
    ap.add_argument("--lmhead", action="store_true",
                    help="verification fed by the output projections (sv_spec_verify_lmhead)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the verification step shards over sequences with no communication, so one GPU's "
              "throughput is the figure.", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    from synth import HEADLINE, WORKLOADS, make_inputs

    headline_path = not (args.copy_calibration or args.lmhead or args.ragged or args.draft_probs or args.sampler
                         or args.draft_temperature is not None)
    if not headline_path:
        # the headline path first runs the oracle on the host (forking), and
        # only then touches the GPU
        import torch

        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        torch.cuda.set_device(0)

    if args.copy_calibration:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "dispatches": 5}), flush=True)
        return

    if args.lmhead:
        run_lmhead(args)
        return
    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    if args.ragged:
        run_ragged(args, w, *args.ragged)
        return
    if args.draft_probs:
        run_probs(args, w)
        return
    d = make_inputs(w)
    if args.sampler:
        run_sampler(args, w, d)
        return
    Td = args.draft_temperature
    cpu = None
    if Td is None:
        x = load_draft_tokens(name, w.B, w.K)
        if not args.no_cpu_baseline:
            # before this process touches the GPU: the all-cores leg forks
            cpu = cpu_baseline(w, d, x, args.cpu_seconds)
            cpu["single_core"] = cpu_baseline_single(w, d, x, args.cpu_seconds)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from rejection_sampling_verify_09_amd import sample

    if Td is not None:
        # the drafts x ~ q at Td, drawn by the library itself (not timed)
        rows = torch.from_numpy(np.ascontiguousarray(d["draft"].reshape(w.B * w.K, w.V)))
        if w.dtype == "bf16":
            rows = rows.view(torch.int16).view(torch.bfloat16)
        ud = torch.from_numpy(d["draft_u"].reshape(-1).astype(np.float32)).cuda()
        xt, _ = sample(rows.cuda(), ud, Td if w.temperature > 0 else 0.0, w.top_k, w.top_p, with_prob=False)
        x = xt.cpu().numpy().reshape(w.B, w.K).astype(np.int32)
        del rows, ud, xt

    m = measure_verify(w, d, x, args.steps, args.warmup, args.copies, Td=Td)
    bytes_per_step = m["bytes_per_step"]
    result = {
        "metric": "spec-verify sequences/s + % HBM peak at B=64 K=6 V=128256 bf16"
                  + ("" if Td is None else f" (drafts at T_d={Td})"),
        "value": m["value"],
        "unit": "sequences/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded logits of the workload's shape; no model weights)",
        "config": {
            "workload": name, "B": w.B, "K": w.K, "V": w.V, "logits": w.dtype, "temperature": w.temperature,
            "top_k": w.top_k, "top_p": w.top_p, "rows": w.rows, "input_copies": m["input_copies"],
            "logit_bytes_per_step": bytes_per_step,
            **({} if Td is None else {"draft_temperature": Td}),
        },
        "tokens_per_s": m["tokens_per_s"],
        "mean_emitted_per_sequence": m["mean_emitted_per_sequence"],
        "per_call_ms": m["per_call_ms"],
        "wall_s_timed": m["wall_s_timed"],
        "roofline": {
            "bound": "hbm",
            "achieved": m["achieved"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": m["achieved"] / HBM_PEAK_GBS,
            "traffic": measured_traffic(name),
            "kernel": "stream_kernel",
            "kernel_ms": m["kernel_ms"],
            "other_kernels_ms": m["other_kernels_ms"],
            "timed_calls": m["timed_calls"],
            "step_frac": m["step_frac"],
        },
        "achievable": read_floor_leg(bytes_per_step, args.steps, args.warmup, m["kernel_ms"]),
    }
    if not args.no_configs and Td is None:
        per = []
        for cname, cw in WORKLOADS.items():
            if cname == name:
                continue
            cd = make_inputs(cw)
            cm = measure_verify(cw, cd, load_draft_tokens(cname, cw.B, cw.K), min(args.steps, 100),
                                min(args.warmup, 10), 0)
            del cd
            line = {"workload": cname, "value": cm["value"], "unit": "sequences/s", "ms_per_step": cm["ms_per_step"],
                    "per_call_ms": cm["per_call_ms"], "tokens_per_s": cm["tokens_per_s"],
                    "logit_bytes_per_step": cm["bytes_per_step"], "stream_kernel_ms": cm["kernel_ms"],
                    "other_kernels_ms": cm["other_kernels_ms"], "frac": cm["achieved"] / HBM_PEAK_GBS,
                    "step_frac": cm["step_frac"], "steps": min(args.steps, 100)}
            print(json.dumps({"config_line": line}), file=sys.stderr, flush=True)
            per.append(line)
            torch.cuda.empty_cache()
        result["per_config"] = per
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu if cpu is not None else \
            cpu_baseline_single(w, d, x, args.cpu_seconds, draft_temperature=Td)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
