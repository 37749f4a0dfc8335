"""Shared GPU-vs-oracle comparison used by the GPU tests and the smoke check."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from synth import Workload, make_inputs


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def draft_tokens_for(w: Workload, d: dict) -> np.ndarray:
    """x[b, i] ~ filtered q_i, drawn by the oracle's inverse CDF with the
    workload's draft-sampling uniforms (greedy: the draft row's arg-max)."""
    B, K = w.B, w.K
    x = np.zeros((B, K), dtype=np.int32)
    for i in range(K):
        rows = oracle.widen(d["draft"][:, i], w.dtype)
        x[:, i] = oracle.sample_tokens(rows, w.temperature, w.top_k, w.top_p, d["draft_u"][:, i])
    return x


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def run_device(w: Workload, d: dict, x: np.ndarray, debug: bool = True, draft_temperature=None):
    import torch

    from rejection_sampling_verify_09_amd import spec_verify

    tgt = to_device(d["target"], w.dtype)
    drf = to_device(d["draft"], w.dtype) if w.K > 0 else None
    X = torch.from_numpy(x.astype(np.int32)).cuda()
    U = torch.from_numpy(d["uniforms"]).cuda()
    res = spec_verify(tgt, drf, X, U, w.temperature, w.top_k, w.top_p, debug=debug,
                      draft_temperature=draft_temperature)
    torch.cuda.synchronize()
    out = [r.cpu().numpy() if not isinstance(r, dict) else {k: v.cpu().numpy() for k, v in r.items()} for r in res]
    return out


def compare(w: Workload, d: dict, x: np.ndarray, dev_tok, dev_n, dev_dbg=None, prob_tol: float = 1e-6,
            draft_temperature=None):
    """Compare device outputs with the oracle.  Returns a dict of counts and
    the list of failures (sequence, reason)."""
    t0 = time.time()
    ref_tok, ref_n, ref_dg = oracle.verify(d["target"], d["draft"], x, d["uniforms"], w.temperature, w.top_k,
                                           w.top_p, dtype=w.dtype, diag=True, draft_temperature=draft_temperature)
    t_oracle = time.time() - t0
    stats = dict(match=0, flagged=0, fail=0, oracle_s=t_oracle, max_prob_err=0.0)
    fails, flags = [], []
    for b in range(w.B):
        if dev_n[b] == ref_n[b] and np.array_equal(dev_tok[b], ref_tok[b]):
            stats["match"] += 1
            continue
        v, why = oracle.classify(d["target"][b], d["draft"][b], x[b], d["uniforms"][b], w.temperature, w.top_k,
                                 w.top_p, w.dtype, dev_tok[b], dev_n[b], draft_temperature=draft_temperature)
        if v == oracle.MATCH:
            stats["match"] += 1
        elif v == oracle.FLAGGED:
            stats["flagged"] += 1
            flags.append((b, why))
        else:
            stats["fail"] += 1
            fails.append((b, why))
    if dev_dbg is not None and w.K > 0:
        ok = ref_n >= 0
        if ok.any():
            ep = np.abs(dev_dbg["p"][ok] - ref_dg["px"][ok]).max()
            err = ep
            if w.temperature != 0.0:
                eq = np.abs(dev_dbg["q"][ok] - ref_dg["qx"][ok]).max()
                err = max(ep, eq)
            stats["max_prob_err"] = float(err)
    stats["flags"] = flags
    return stats, fails


# ---------------------------------------------------------------------------
# ragged batches (a draft length per sequence)
# ---------------------------------------------------------------------------
def ragged_draft_tokens(w: Workload, r: dict, Td=None) -> np.ndarray:
    """x ~ filtered q for every packed draft row, with its draft-sampling
    uniform (greedy: the row's arg-max)."""
    if r["draft"].shape[0] == 0:
        return np.zeros(0, dtype=np.int32)
    T = w.temperature if Td is None or w.temperature == 0.0 else Td
    rows = oracle.widen(r["draft"], w.dtype)
    return oracle.sample_tokens(rows, T, w.top_k, w.top_p, r["draft_u"]).astype(np.int32)


def run_device_ragged(w: Workload, r: dict, x: np.ndarray, max_k: int, debug: bool = True, draft_temperature=None,
                      cu=None):
    import torch

    from rejection_sampling_verify_09_amd import spec_verify_ragged

    tgt = to_device(r["target"], w.dtype)
    drf = to_device(r["draft"], w.dtype) if r["draft"].shape[0] > 0 else None
    X = torch.from_numpy(x.astype(np.int32)).cuda()
    U = torch.from_numpy(r["uniforms"]).cuda()
    CU = torch.from_numpy((r["cu"] if cu is None else cu).astype(np.int32)).cuda()
    res = spec_verify_ragged(tgt, drf, X, U, CU, max_k, w.temperature, w.top_k, w.top_p,
                             draft_temperature=draft_temperature, debug=debug)
    torch.cuda.synchronize()
    return [v.cpu().numpy() if not isinstance(v, dict) else {k: t.cpu().numpy() for k, t in v.items()} for v in res]


def compare_ragged(w: Workload, r: dict, x: np.ndarray, max_k: int, dev_tok, dev_n, dev_dbg=None,
                   draft_temperature=None):
    """Ragged device outputs against the oracle; near-ties classified per
    sequence exactly as for rectangular batches."""
    cu = r["cu"].astype(np.int64)
    B = cu.shape[0] - 1
    ref_tok, ref_n, ref_dg = oracle.verify_ragged(r["target"], r["draft"], x, r["uniforms"], cu, w.temperature,
                                                  w.top_k, w.top_p, dtype=w.dtype, max_k=max_k, diag=True,
                                                  draft_temperature=draft_temperature)
    stats = dict(match=0, flagged=0, fail=0, max_prob_err=0.0)
    fails, flags = [], []
    for b in range(B):
        if dev_n[b] == ref_n[b] and np.array_equal(dev_tok[b], ref_tok[b]):
            stats["match"] += 1
            continue
        c0, c1 = int(cu[b]), int(cu[b + 1])
        K = c1 - c0
        t0 = c0 + b
        if np.any(dev_tok[b, K + 1:] != -1):
            stats["fail"] += 1
            fails.append((b, "entries past the sequence's own K are not -1"))
            continue
        v, why = oracle.classify(r["target"][t0:t0 + K + 1], r["draft"][c0:c1], x[c0:c1], r["uniforms"][t0:t0 + K + 1],
                                 w.temperature, w.top_k, w.top_p, w.dtype, dev_tok[b, :K + 1], dev_n[b],
                                 draft_temperature=draft_temperature)
        if v == oracle.MATCH:
            stats["match"] += 1
        elif v == oracle.FLAGGED:
            stats["flagged"] += 1
            flags.append((b, why))
        else:
            stats["fail"] += 1
            fails.append((b, why))
    if dev_dbg is not None and cu[-1] > 0:
        ok = np.repeat(ref_n >= 0, np.diff(cu))
        if ok.any():
            err = np.abs(dev_dbg["p"][ok] - ref_dg["px"][ok]).max()
            if w.temperature != 0.0:
                err = max(err, np.abs(dev_dbg["q"][ok] - ref_dg["qx"][ok]).max())
            stats["max_prob_err"] = float(err)
    stats["flags"] = flags
    return stats, fails


# ---------------------------------------------------------------------------
# q given as probabilities
# ---------------------------------------------------------------------------
def run_device_probs(w: Workload, d: dict, Q: np.ndarray, x: np.ndarray, debug: bool = True):
    import torch

    from rejection_sampling_verify_09_amd import spec_verify_probs

    tgt = to_device(d["target"], w.dtype)
    qd = torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float32)).cuda() if w.K > 0 else None
    X = torch.from_numpy(x.astype(np.int32)).cuda()
    U = torch.from_numpy(d["uniforms"]).cuda()
    res = spec_verify_probs(tgt, qd, X, U, w.temperature, w.top_k, w.top_p, debug=debug)
    torch.cuda.synchronize()
    return [v.cpu().numpy() if not isinstance(v, dict) else {k: t.cpu().numpy() for k, t in v.items()} for v in res]


def compare_probs(w: Workload, d: dict, Q: np.ndarray, x: np.ndarray, dev_tok, dev_n, dev_dbg=None):
    ref_tok, ref_n, ref_dg = oracle.verify(d["target"], None, x, d["uniforms"], w.temperature, w.top_k, w.top_p,
                                           dtype=w.dtype, diag=True, draft_probs=Q)
    stats = dict(match=0, flagged=0, fail=0, max_prob_err=0.0)
    fails, flags = [], []
    for b in range(w.B):
        if dev_n[b] == ref_n[b] and np.array_equal(dev_tok[b], ref_tok[b]):
            stats["match"] += 1
            continue
        v, why = oracle.classify(d["target"][b], None, x[b], d["uniforms"][b], w.temperature, w.top_k, w.top_p,
                                 w.dtype, dev_tok[b], dev_n[b], draft_probs_b=Q[b])
        if v == oracle.MATCH:
            stats["match"] += 1
        elif v == oracle.FLAGGED:
            stats["flagged"] += 1
            flags.append((b, why))
        else:
            stats["fail"] += 1
            fails.append((b, why))
    if dev_dbg is not None and w.K > 0:
        ok = ref_n >= 0
        if ok.any():
            err = np.abs(dev_dbg["p"][ok] - ref_dg["px"][ok]).max()
            if w.temperature != 0.0:
                err = max(err, np.abs(dev_dbg["q"][ok] - ref_dg["qx"][ok]).max())
            stats["max_prob_err"] = float(err)
    stats["flags"] = flags
    return stats, fails


# ---------------------------------------------------------------------------
# verification fed by the output projections
# ---------------------------------------------------------------------------
def lm_oracle_logits(d: dict, greedy: bool):
    """The oracle's float64 logits of both heads (the draft's are still
    formed when greedy: the drafts are its arg-max)."""
    lt = oracle.lm_logits(d["hidden_t"], d["weight_t"], "bf16")
    if d["hidden_d"].shape[1] == 0:
        ld = np.zeros(lt.shape[:1] + (lt.shape[1] - 1, lt.shape[2]))
    else:
        ld = oracle.lm_logits(d["hidden_d"], d["weight_d"], "bf16")
    return lt, ld


def lm_draft_tokens(w, ld: np.ndarray, draft_u: np.ndarray) -> np.ndarray:
    """x[b, i] ~ filtered q_i of the oracle's draft logits (greedy: arg-max)."""
    B, K = draft_u.shape
    x = np.zeros((B, K), dtype=np.int32)
    if w.temperature == 0.0:
        return np.argmax(ld, axis=-1).astype(np.int32) if K > 0 else x
    for i in range(K):
        x[:, i] = oracle.sample_tokens(ld[:, i], w.temperature, w.top_k, w.top_p, draft_u[:, i])
    return x


def run_device_lmhead(w, d: dict, x: np.ndarray, debug: bool = True):
    import torch

    from rejection_sampling_verify_09_amd import spec_verify_lmhead

    greedy = w.temperature == 0.0
    ht = to_device(d["hidden_t"], "bf16")
    wt = to_device(d["weight_t"], "bf16")
    hd = None if greedy else to_device(d["hidden_d"], "bf16")
    wd = None if greedy else to_device(d["weight_d"], "bf16")
    X = torch.from_numpy(x.astype(np.int32)).cuda()
    U = torch.from_numpy(d["uniforms"]).cuda()
    res = spec_verify_lmhead(ht, wt, hd, wd, X, U, w.temperature, w.top_k, w.top_p, debug=debug)
    torch.cuda.synchronize()
    return [v.cpu().numpy() if not isinstance(v, dict) else {k: t.cpu().numpy() for k, t in v.items()} for v in res]


def compare_lmhead(w, d: dict, lt: np.ndarray, ld: np.ndarray, x: np.ndarray, dev_tok, dev_n, dev_dbg=None):
    """Device outputs against the oracle's verification of its own float64
    logits; near-ties classified per sequence as for given logits."""
    ref_tok, ref_n, ref_dg = oracle.verify(lt, ld, x, d["uniforms"], w.temperature, w.top_k, w.top_p,
                                           dtype=oracle.F64, diag=True)
    stats = dict(match=0, flagged=0, fail=0, max_prob_err=0.0)
    fails, flags = [], []
    for b in range(w.B):
        if dev_n[b] == ref_n[b] and np.array_equal(dev_tok[b], ref_tok[b]):
            stats["match"] += 1
            continue
        v, why = oracle.classify(lt[b], ld[b], x[b], d["uniforms"][b], w.temperature, w.top_k, w.top_p, oracle.F64,
                                 dev_tok[b], dev_n[b])
        if v == oracle.MATCH:
            stats["match"] += 1
        elif v == oracle.FLAGGED:
            stats["flagged"] += 1
            flags.append((b, why))
        else:
            stats["fail"] += 1
            fails.append((b, why))
    if dev_dbg is not None and w.K > 0:
        ok = ref_n >= 0
        if ok.any():
            err = np.abs(dev_dbg["p"][ok] - ref_dg["px"][ok]).max()
            if w.temperature != 0.0:
                err = max(err, np.abs(dev_dbg["q"][ok] - ref_dg["qx"][ok]).max())
            stats["max_prob_err"] = float(err)
    stats["flags"] = flags
    stats["ref_dg"] = ref_dg
    return stats, fails


# ---------------------------------------------------------------------------
# near-tie rates over many verifications of the same rows
# ---------------------------------------------------------------------------
def filtered_rows(rows: np.ndarray, dtype: str, T, top_k, top_p, block: int = 256) -> np.ndarray:
    """The oracle's filtered distributions of logit rows [N, V], a block of
    rows at a time (bounded temporaries at full vocabulary sizes)."""
    out = np.empty(rows.shape, dtype=np.float64)
    for s in range(0, rows.shape[0], block):
        out[s:s + block] = oracle.filtered_probs(oracle.widen(rows[s:s + block], dtype), T, top_k, top_p)
    return out


def rate_inputs(w: Workload, d: dict, n_min: int, seed_key: int = 7):
    """Draw tables of the batch ``d`` and R = ceil(n_min / B) fresh draws of
    (drafted tokens, uniforms) for it.  Drafts follow the filtered q (greedy:
    the target's arg-max with probability 0.6, else a uniform token).
    Returns (tables, x [R, B, K], u [R, B, K+1] float32)."""
    from oracle.rate import DrawTables

    B, K, V = w.B, w.K, w.V
    P = filtered_rows(d["target"].reshape(-1, V), w.dtype, w.temperature, w.top_k, w.top_p).reshape(B, K + 1, V)
    if w.temperature == 0.0:
        # greedy: q is one-hot at the draft's arg-max and drops out of the rule
        Q = filtered_rows(d["draft"].reshape(-1, V), w.dtype, 0.0, 0, 1.0).reshape(B, K, V) if K > 0 else \
            np.zeros((B, 0, V))
    else:
        Q = filtered_rows(d["draft"].reshape(-1, V), w.dtype, w.temperature, w.top_k, w.top_p).reshape(B, K, V)
    tabs = DrawTables(P, Q)
    R = -(-n_min // B)
    rng = np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=tuple(w.spawn_key) + (seed_key,)))
    if w.temperature == 0.0:
        amax = np.argmax(P[:, :K], axis=2)
        x = np.where(rng.random((R, B, K)) < 0.6, amax[None], rng.integers(0, V, (R, B, K)))
    else:
        x = tabs.draw_drafts(rng.random((R, B, K)))
    u = rng.random((R, B, K + 1), dtype=np.float32)
    return tabs, x, u


def rate_check(w: Workload, d: dict, tabs, x: np.ndarray, u: np.ndarray, dev_tok: np.ndarray, dev_n: np.ndarray):
    """Compare R verifications of the batch with the oracle's: exact matches,
    near-ties (flagged) and failures, with the informational count of
    sequences whose own decisions lie within 1e-5 of a boundary (at risk)."""
    ref_tok, ref_n = tabs.decide(x, u)
    risk = tabs.at_risk(x, u)
    mism = (dev_tok != ref_tok).any(axis=2) | (dev_n != ref_n)
    stats = dict(sequences=int(dev_n.size), mismatched=int(mism.sum()), flagged=0, fail=0,
                 at_risk=int(risk.sum()), accepted_mean=float(np.mean(ref_n[ref_n >= 0])) if (ref_n >= 0).any() else 0.0)
    fails, flags = [], []
    for r, b in np.argwhere(mism):
        v, why = oracle.classify(d["target"][b], d["draft"][b], x[r, b], u[r, b], w.temperature, w.top_k, w.top_p,
                                 w.dtype, dev_tok[r, b], dev_n[r, b])
        if v == oracle.FLAGGED:
            stats["flagged"] += 1
            flags.append((int(r), int(b), why))
        elif v == oracle.FAIL:
            stats["fail"] += 1
            fails.append((int(r), int(b), why))
    stats["flagged_rate"] = stats["flagged"] / max(1, stats["sequences"])
    return stats, fails, flags


def run_device_many(w: Workload, d: dict, x: np.ndarray, u: np.ndarray):
    """R calls of the library's verification on the same device rows, one per
    draw of (drafted tokens, uniforms); outputs gathered on the device and
    copied back once."""
    import torch

    from rejection_sampling_verify_09_amd import spec_verify

    R, B, K = x.shape
    tgt = to_device(d["target"], w.dtype)
    drf = to_device(d["draft"], w.dtype) if K > 0 else None
    X = torch.from_numpy(x.astype(np.int32)).cuda()
    U = torch.from_numpy(np.ascontiguousarray(u)).cuda()
    out_t = torch.empty((R, B, K + 1), dtype=torch.int32, device="cuda")
    out_n = torch.empty((R, B), dtype=torch.int32, device="cuda")
    for r in range(R):
        spec_verify(tgt, drf, X[r], U[r], w.temperature, w.top_k, w.top_p, out_tokens=out_t[r],
                    out_num_accepted=out_n[r])
    torch.cuda.synchronize()
    return out_t.cpu().numpy(), out_n.cpu().numpy()
