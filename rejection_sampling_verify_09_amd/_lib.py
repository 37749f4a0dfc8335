"""ctypes binding of libspecverify.so (argument marshalling only).

Every step of the verification runs in the library's HIP kernels; this module
only checks tensor metadata, passes device pointers and the current HIP
stream, and allocates the output tensors.  It never falls back to another
implementation: if the library is missing it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_PARAM, SV_ERR_HIP, SV_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5, -6
SV_F32, SV_BF16 = 0, 1
SV_MAX_K = 64
SV_INIT_LMHEAD = 1
SV_NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with rejection_sampling_verify_09_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        L.sv_spec_verify.argtypes = [vp, vp, vp, vp, f32, i32, f32, vp, vp, i32, i32, i32, i32, vp]
        L.sv_spec_verify.restype = ctypes.c_int
        L.sv_spec_verify_debug.argtypes = [vp, vp, vp, vp, f32, i32, f32, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.sv_spec_verify_debug.restype = ctypes.c_int
        L.sv_filtered_probs.argtypes = [vp, i32, i32, i32, f32, i32, f32, vp, vp]
        L.sv_filtered_probs.restype = ctypes.c_int
        L.sv_sample.argtypes = [vp, vp, f32, i32, f32, vp, vp, i32, i32, i32, vp]
        L.sv_sample.restype = ctypes.c_int
        L.sv_spec_verify_dt.argtypes = [vp, vp, vp, vp, f32, f32, i32, f32, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.sv_spec_verify_dt.restype = ctypes.c_int
        L.sv_spec_verify_ragged.argtypes = [vp, vp, vp, vp, vp, f32, f32, i32, f32, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, vp]
        L.sv_spec_verify_ragged.restype = ctypes.c_int
        L.sv_spec_verify_probs.argtypes = [vp, vp, vp, vp, f32, i32, f32, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.sv_spec_verify_probs.restype = ctypes.c_int
        L.sv_lm_logits.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.sv_lm_logits.restype = ctypes.c_int
        L.sv_spec_verify_lmhead.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, f32, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, vp]
        L.sv_spec_verify_lmhead.restype = ctypes.c_int
        L.sv_dynk_create.argtypes = [i32, i32, ctypes.c_double, ctypes.c_double, i32, i32, i32]
        L.sv_dynk_create.restype = vp
        L.sv_dynk_observe.argtypes = [vp, vp, vp, vp]
        L.sv_dynk_observe.restype = ctypes.c_int
        L.sv_dynk_k.argtypes = [vp, i32]
        L.sv_dynk_k.restype = i32
        L.sv_dynk_destroy.argtypes = [vp]
        L.sv_dynk_destroy.restype = None
        L.sv_release.argtypes = []
        L.sv_release.restype = ctypes.c_int
        L.sv_spec_verify_noalloc.argtypes = [vp, vp, vp, vp, f32, i32, f32, vp, vp, i32, i32, i32, i32, vp]
        L.sv_spec_verify_noalloc.restype = ctypes.c_int
        L.sv_init.argtypes = [ctypes.c_int, vp, i32, i32, i32, i32]
        L.sv_init.restype = ctypes.c_int
        L.sv_stream_release.argtypes = [vp]
        L.sv_stream_release.restype = ctypes.c_int
        L.sv_scratch_bytes.argtypes = [ctypes.c_int]
        L.sv_scratch_bytes.restype = ctypes.c_int64
        L.sv_status_string.argtypes = [ctypes.c_int]
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_version.argtypes = []
        L.sv_version.restype = ctypes.c_int
        L.sv_read_floor.argtypes = [vp, ctypes.c_int64, ctypes.c_uint32, vp, vp]
        L.sv_read_floor.restype = ctypes.c_int
        L.sv_profile_start.argtypes = []
        L.sv_profile_start.restype = ctypes.c_int
        L.sv_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
        L.sv_profile_stop.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sv_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def spec_verify(target_logits: torch.Tensor, draft_logits: torch.Tensor | None, draft_tokens: torch.Tensor,
                uniforms: torch.Tensor, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                out_tokens: torch.Tensor | None = None, out_num_accepted: torch.Tensor | None = None,
                stream=None, debug: bool = False, draft_temperature: float | None = None):
    """Verify one round of drafted tokens on the GPU.

    target_logits [B, K+1, V] and draft_logits [B, K, V] (float32 or
    bfloat16, same dtype); draft_tokens [B, K] int32; uniforms [B, K+1]
    float32.  draft_temperature: the temperature the drafts were sampled at,
    when it differs from the target's.  Returns (out_tokens [B, K+1] int32,
    out_num_accepted [B] int32), plus a dict of p(x), q(x) and Z when
    ``debug``.
    """
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    dev = target_logits.device
    tp = _dev(target_logits, "target_logits")
    if draft_logits is not None and K > 0:
        if tuple(draft_logits.shape) != (B, K, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [B, K, V] with the target's dtype")
        dp = _dev(draft_logits, "draft_logits")
    elif float(temperature) == 0.0 or K == 0:
        dp = None
    else:
        raise ValueError("draft_logits are required unless temperature == 0")
    if tuple(draft_tokens.shape) != (B, K) or tuple(uniforms.shape) != (B, K + 1):
        raise ValueError("draft_tokens must be [B, K] and uniforms [B, K+1]")
    xp = _dev(draft_tokens, "draft_tokens", torch.int32) if K > 0 else None
    up = _dev(uniforms, "uniforms", torch.float32)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    op = _dev(out_tokens, "out_tokens", torch.int32)
    onp = _dev(out_num_accepted, "out_num_accepted", torch.int32)
    s = _stream(stream)
    if draft_temperature is not None:
        out_p = torch.empty((B, K), dtype=torch.float64, device=dev) if debug else None
        out_q = torch.empty((B, K), dtype=torch.float64, device=dev) if debug else None
        out_z = torch.empty((B,), dtype=torch.float64, device=dev) if debug else None
        st = lib().sv_spec_verify_dt(tp, dp, xp, up, float(temperature), float(draft_temperature), int(top_k),
                                     float(top_p), op, onp,
                                     out_p.data_ptr() if debug and K > 0 else None,
                                     out_q.data_ptr() if debug and K > 0 else None,
                                     out_z.data_ptr() if debug else None, B, K, V, code, s)
        if st != SV_OK:
            raise SpecVerifyError(st, "sv_spec_verify_dt")
        if debug:
            return out_tokens, out_num_accepted, dict(p=out_p, q=out_q, z=out_z)
        return out_tokens, out_num_accepted
    if debug:
        out_p = torch.empty((B, K), dtype=torch.float64, device=dev)
        out_q = torch.empty((B, K), dtype=torch.float64, device=dev)
        out_z = torch.empty((B,), dtype=torch.float64, device=dev)
        st = lib().sv_spec_verify_debug(tp, dp, xp, up, float(temperature), int(top_k), float(top_p), op, onp,
                                        out_p.data_ptr() if K > 0 else None, out_q.data_ptr() if K > 0 else None,
                                        out_z.data_ptr(), B, K, V, code, s)
        if st != SV_OK:
            raise SpecVerifyError(st, "sv_spec_verify_debug")
        return out_tokens, out_num_accepted, dict(p=out_p, q=out_q, z=out_z)
    st = lib().sv_spec_verify(tp, dp, xp, up, float(temperature), int(top_k), float(top_p), op, onp, B, K, V, code, s)
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_spec_verify")
    return out_tokens, out_num_accepted


def spec_verify_noalloc(target_logits: torch.Tensor, draft_logits: torch.Tensor | None, draft_tokens: torch.Tensor,
                        uniforms: torch.Tensor, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                        out_tokens: torch.Tensor | None = None, out_num_accepted: torch.Tensor | None = None,
                        stream=None):
    """spec_verify through sv_spec_verify_noalloc: the library allocates
    nothing (its scratch is a fixed per-device array; calls that overlap on
    one device race on it).  Pass the output tensors to allocate nothing on
    this side either."""
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    dev = target_logits.device
    tp = _dev(target_logits, "target_logits")
    if draft_logits is not None and K > 0:
        if tuple(draft_logits.shape) != (B, K, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [B, K, V] with the target's dtype")
        dp = _dev(draft_logits, "draft_logits")
    elif float(temperature) == 0.0 or K == 0:
        dp = None
    else:
        raise ValueError("draft_logits are required unless temperature == 0")
    if tuple(draft_tokens.shape) != (B, K) or tuple(uniforms.shape) != (B, K + 1):
        raise ValueError("draft_tokens must be [B, K] and uniforms [B, K+1]")
    xp = _dev(draft_tokens, "draft_tokens", torch.int32) if K > 0 else None
    up = _dev(uniforms, "uniforms", torch.float32)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    st = lib().sv_spec_verify_noalloc(tp, dp, xp, up, float(temperature), int(top_k), float(top_p),
                                      _dev(out_tokens, "out_tokens", torch.int32),
                                      _dev(out_num_accepted, "out_num_accepted", torch.int32), B, K, V, code,
                                      _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_spec_verify_noalloc")
    return out_tokens, out_num_accepted


def spec_verify_ragged(target_logits: torch.Tensor, draft_logits: torch.Tensor | None, draft_tokens: torch.Tensor,
                       uniforms: torch.Tensor, cu_num_draft: torch.Tensor, max_k: int, temperature: float = 1.0,
                       top_k: int = 0, top_p: float = 1.0, draft_temperature: float | None = None,
                       out_tokens: torch.Tensor | None = None, out_num_accepted: torch.Tensor | None = None,
                       stream=None, debug: bool = False):
    """Verify a batch of sequences with different draft lengths on the GPU.

    Packed: target_logits [N + B, V] (sequence b's K_b + 1 rows from row
    cu[b] + b), draft_logits [N, V] (its K_b rows from row cu[b]),
    draft_tokens [N] int32, uniforms [N + B] float32, cu_num_draft [B + 1]
    int32 on the device, N = total drafts (from the tensors' shapes, not from
    the device offsets).  Returns (out_tokens [B, max_k + 1] int32,
    out_num_accepted [B] int32), plus p(x), q(x) [N] and Z [B] when ``debug``.
    """
    if target_logits.dim() != 2 or cu_num_draft.dim() != 1:
        raise ValueError("target_logits must be [N + B, V] and cu_num_draft [B + 1]")
    B = cu_num_draft.shape[0] - 1
    NT, V = target_logits.shape
    N = NT - B
    if B < 0 or N < 0:
        raise ValueError("target_logits needs N + B rows")
    code = _dtype_code(target_logits)
    dev = target_logits.device
    tp = _dev(target_logits, "target_logits")
    if draft_logits is not None and N > 0:
        if tuple(draft_logits.shape) != (N, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [N, V] with the target's dtype")
        dp = _dev(draft_logits, "draft_logits")
    elif float(temperature) == 0.0 or N == 0:
        dp = None
    else:
        raise ValueError("draft_logits are required unless temperature == 0")
    if tuple(draft_tokens.shape) != (N,) or tuple(uniforms.shape) != (N + B,):
        raise ValueError("draft_tokens must be [N] and uniforms [N + B]")
    xp = _dev(draft_tokens, "draft_tokens", torch.int32) if N > 0 else None
    up = _dev(uniforms, "uniforms", torch.float32)
    cp = _dev(cu_num_draft, "cu_num_draft", torch.int32)
    if out_tokens is None:
        out_tokens = torch.empty((B, int(max_k) + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if tuple(out_tokens.shape) != (B, int(max_k) + 1):
        raise ValueError("out_tokens must be [B, max_k + 1]")
    out_p = torch.empty((N,), dtype=torch.float64, device=dev) if debug else None
    out_q = torch.empty((N,), dtype=torch.float64, device=dev) if debug else None
    out_z = torch.empty((B,), dtype=torch.float64, device=dev) if debug else None
    Td = float(temperature) if draft_temperature is None else float(draft_temperature)
    st = lib().sv_spec_verify_ragged(tp, dp, xp, up, cp, float(temperature), Td, int(top_k), float(top_p),
                                     _dev(out_tokens, "out_tokens", torch.int32),
                                     _dev(out_num_accepted, "out_num_accepted", torch.int32),
                                     out_p.data_ptr() if debug and N > 0 else None,
                                     out_q.data_ptr() if debug and N > 0 else None,
                                     out_z.data_ptr() if debug else None, B, N, int(max_k), V, code, _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_spec_verify_ragged")
    if debug:
        return out_tokens, out_num_accepted, dict(p=out_p, q=out_q, z=out_z)
    return out_tokens, out_num_accepted


def spec_verify_probs(target_logits: torch.Tensor, draft_probs: torch.Tensor | None, draft_tokens: torch.Tensor,
                      uniforms: torch.Tensor, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                      out_tokens: torch.Tensor | None = None, out_num_accepted: torch.Tensor | None = None,
                      stream=None, debug: bool = False):
    """Verify one round of drafted tokens whose draft distributions are given
    as probabilities: target_logits [B, K+1, V] (float32 or bfloat16),
    draft_probs [B, K, V] float32 (the q each draft was drawn from),
    draft_tokens [B, K] int32, uniforms [B, K+1] float32.  Returns
    (out_tokens [B, K+1], out_num_accepted [B]), plus p(x), q(x), Z when
    ``debug``."""
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    code = _dtype_code(target_logits)
    dev = target_logits.device
    if draft_probs is not None and K > 0:
        if tuple(draft_probs.shape) != (B, K, V):
            raise ValueError("draft_probs must be [B, K, V]")
        qp = _dev(draft_probs, "draft_probs", torch.float32)
    elif float(temperature) == 0.0 or K == 0:
        qp = None
    else:
        raise ValueError("draft_probs are required unless temperature == 0")
    if tuple(draft_tokens.shape) != (B, K) or tuple(uniforms.shape) != (B, K + 1):
        raise ValueError("draft_tokens must be [B, K] and uniforms [B, K+1]")
    xp = _dev(draft_tokens, "draft_tokens", torch.int32) if K > 0 else None
    up = _dev(uniforms, "uniforms", torch.float32)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    out_p = torch.empty((B, K), dtype=torch.float64, device=dev) if debug else None
    out_q = torch.empty((B, K), dtype=torch.float64, device=dev) if debug else None
    out_z = torch.empty((B,), dtype=torch.float64, device=dev) if debug else None
    st = lib().sv_spec_verify_probs(_dev(target_logits, "target_logits"), qp, xp, up, float(temperature), int(top_k),
                                    float(top_p), _dev(out_tokens, "out_tokens", torch.int32),
                                    _dev(out_num_accepted, "out_num_accepted", torch.int32),
                                    out_p.data_ptr() if debug and K > 0 else None,
                                    out_q.data_ptr() if debug and K > 0 else None,
                                    out_z.data_ptr() if debug else None, B, K, V, code, _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_spec_verify_probs")
    if debug:
        return out_tokens, out_num_accepted, dict(p=out_p, q=out_q, z=out_z)
    return out_tokens, out_num_accepted


def lm_logits(hidden: torch.Tensor, weight: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """Output projection: hidden [..., d] bfloat16 times weight [V, d]
    bfloat16, transposed -> float32 logits [..., V]."""
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if weight.dim() != 2 or hidden.shape[-1] != weight.shape[1]:
        raise ValueError("hidden [..., d] and weight [V, d] must share d")
    V, d = weight.shape
    M = hidden.numel() // d if d > 0 else 0
    shape = tuple(hidden.shape[:-1]) + (V,)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=hidden.device)
    elif tuple(out.shape) != shape:
        raise ValueError(f"out must be {shape}")
    st = lib().sv_lm_logits(_dev(hidden, "hidden"), _dev(weight, "weight"), _dev(out, "out", torch.float32), M, V, d,
                            _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_lm_logits")
    return out


def spec_verify_lmhead(hidden_target: torch.Tensor, weight_target: torch.Tensor, hidden_draft: torch.Tensor | None,
                       weight_draft: torch.Tensor | None, draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                       temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, stream=None,
                       debug: bool = False):
    """Verification fed by the output projections: hidden_target [B, K+1, d]
    and weight_target [V, d] (bfloat16), hidden_draft [B, K, d_d] and
    weight_draft [V, d_d] (bfloat16; may be None at temperature 0),
    draft_tokens [B, K] int32, uniforms [B, K+1] float32.  Returns
    (out_tokens, out_num_accepted), plus p(x), q(x), Z when ``debug``."""
    if hidden_target.dim() != 3 or weight_target.dim() != 2:
        raise ValueError("hidden_target must be [B, K+1, d] and weight_target [V, d]")
    B, K1, d = hidden_target.shape
    K = K1 - 1
    V = weight_target.shape[0]
    if weight_target.shape[1] != d:
        raise ValueError("hidden_target and weight_target must share d")
    for t, n in ((hidden_target, "hidden_target"), (weight_target, "weight_target")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
    dev = hidden_target.device
    use_d = float(temperature) != 0.0 and K > 0
    hd = wd = None
    dd = 64
    if use_d:
        if hidden_draft is None or weight_draft is None:
            raise ValueError("hidden_draft and weight_draft are required unless temperature == 0")
        if hidden_draft.dtype != torch.bfloat16 or weight_draft.dtype != torch.bfloat16:
            raise TypeError("hidden_draft and weight_draft must be bfloat16")
        dd = weight_draft.shape[1]
        if tuple(hidden_draft.shape) != (B, K, dd) or tuple(weight_draft.shape) != (V, dd):
            raise ValueError("hidden_draft must be [B, K, d_d] and weight_draft [V, d_d]")
        hd, wd = _dev(hidden_draft, "hidden_draft"), _dev(weight_draft, "weight_draft")
    if tuple(draft_tokens.shape) != (B, K) or tuple(uniforms.shape) != (B, K + 1):
        raise ValueError("draft_tokens must be [B, K] and uniforms [B, K+1]")
    xp = _dev(draft_tokens, "draft_tokens", torch.int32) if K > 0 else None
    up = _dev(uniforms, "uniforms", torch.float32)
    out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    out_p = torch.empty((B, K), dtype=torch.float64, device=dev) if debug else None
    out_q = torch.empty((B, K), dtype=torch.float64, device=dev) if debug else None
    out_z = torch.empty((B,), dtype=torch.float64, device=dev) if debug else None
    st = lib().sv_spec_verify_lmhead(_dev(hidden_target, "hidden_target"), _dev(weight_target, "weight_target"), hd, wd,
                                     xp, up, float(temperature), int(top_k), float(top_p), out_tokens.data_ptr(),
                                     out_n.data_ptr(), out_p.data_ptr() if debug and K > 0 else None,
                                     out_q.data_ptr() if debug and K > 0 else None,
                                     out_z.data_ptr() if debug else None, B, K, V, d, dd, _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_spec_verify_lmhead")
    if debug:
        return out_tokens, out_n, dict(p=out_p, q=out_q, z=out_z)
    return out_tokens, out_n


class DraftLengthController:
    """Host handle of the library's draft-length controller (``lanes``
    independent controllers: 1 for a batch-wide K, B for one per sequence)."""

    def __init__(self, lanes: int = 1, window: int = 100, raise_above: float = 0.8, lower_below: float = 0.6,
                 k_min: int = 2, k_max: int = 10, k_init: int = 5):
        self._lib = lib()
        self.lanes = int(lanes)
        h = self._lib.sv_dynk_create(self.lanes, int(window), float(raise_above), float(lower_below), int(k_min),
                                     int(k_max), int(k_init))
        if not h:
            raise ValueError("invalid controller settings")
        self._h = ctypes.c_void_p(h)

    def observe(self, accepted, drafted):
        """One batch: per-lane accepted drafts and drafted tokens (host
        sequences of ints).  Returns the next draft length of every lane."""
        if len(accepted) != self.lanes or len(drafted) != self.lanes:
            raise ValueError("one value per lane")
        if not self._h:
            raise ValueError("the controller is closed")
        acc = (ctypes.c_int64 * self.lanes)(*[int(v) for v in accepted])
        dr = (ctypes.c_int64 * self.lanes)(*[int(v) for v in drafted])
        out = (ctypes.c_int32 * self.lanes)()
        st = self._lib.sv_dynk_observe(self._h, acc, dr, out)
        if st != SV_OK:
            raise SpecVerifyError(st, "sv_dynk_observe")
        return list(out)

    def k(self, lane: int = 0) -> int:
        return int(self._lib.sv_dynk_k(self._h, int(lane)))

    def close(self) -> None:
        if self._h:
            self._lib.sv_dynk_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def filtered_probs(logits: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Filtered probabilities of every row of ``logits`` [rows, V] (float32 out)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, V]")
    rows, V = logits.shape
    code = _dtype_code(logits)
    if out is None:
        out = torch.empty((rows, V), dtype=torch.float32, device=logits.device)
    st = lib().sv_filtered_probs(_dev(logits, "logits"), rows, V, code, float(temperature), int(top_k),
                                 float(top_p), _dev(out, "out", torch.float32), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_filtered_probs")
    return out


def sample(logits: torch.Tensor, uniforms: torch.Tensor, temperature: float = 1.0, top_k: int = 0,
           top_p: float = 1.0, out_tokens: torch.Tensor | None = None, out_prob: torch.Tensor | None = None,
           with_prob: bool = True, stream=None):
    """Draw one token per row of ``logits`` [rows, V] from its filtered
    distribution with ``uniforms`` [rows] float32.  Returns (tokens [rows]
    int32, the drawn tokens' probabilities [rows] float64 or None)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, V]")
    rows, V = logits.shape
    code = _dtype_code(logits)
    if tuple(uniforms.shape) != (rows,):
        raise ValueError("uniforms must be [rows]")
    dev = logits.device
    if out_tokens is None:
        out_tokens = torch.empty((rows,), dtype=torch.int32, device=dev)
    if with_prob and out_prob is None:
        out_prob = torch.empty((rows,), dtype=torch.float64, device=dev)
    pp = _dev(out_prob, "out_prob", torch.float64) if with_prob else None
    st = lib().sv_sample(_dev(logits, "logits"), _dev(uniforms, "uniforms", torch.float32), float(temperature),
                         int(top_k), float(top_p), _dev(out_tokens, "out_tokens", torch.int32), pp, rows, V, code,
                         _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_sample")
    return out_tokens, (out_prob if with_prob else None)


READ_BLOCK = 16384  # bytes per workgroup of sv_read_floor


def read_floor(data: torch.Tensor, key: int = 0, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Plain read of a contiguous device tensor's bytes (sv_read_floor), the
    floor the streaming pass is measured against.  Returns out: one int32
    word per 16 KiB block, written only where the block's words xor to key."""
    if not data.is_cuda or not data.is_contiguous() or data.data_ptr() % 16 != 0:
        raise ValueError("data must be a contiguous, 16-byte aligned device tensor")
    nbytes = data.numel() * data.element_size()
    nblk = max(1, -(-nbytes // READ_BLOCK))
    if out is None:
        out = torch.zeros((nblk,), dtype=torch.int32, device=data.device)
    if out.dtype != torch.int32 or not out.is_cuda or out.numel() < nblk:
        raise ValueError("out must be an int32 device tensor of one word per 16 KiB block")
    st = lib().sv_read_floor(ctypes.c_void_p(data.data_ptr()), nbytes, int(key) & 0xFFFFFFFF,
                             ctypes.c_void_p(out.data_ptr()), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_read_floor")
    return out


def profile_start() -> None:
    """Start timing every verification call's kernels with HIP events."""
    st = lib().sv_profile_start()
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_profile_start")


def profile_stop() -> dict:
    """Stop timing; returns the summed streaming-kernel and follow-up kernel
    durations (ms) and the number of calls timed."""
    a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    st = lib().sv_profile_stop(ctypes.byref(a), ctypes.byref(b), ctypes.byref(n))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_profile_stop")
    return dict(stream_kernel_ms=a.value, other_kernels_ms=b.value, calls=n.value)


def release() -> None:
    st = lib().sv_release()
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_release")


def init(max_B: int, max_K: int, max_V: int, stream=None, device: int | None = None, lmhead: bool = False) -> None:
    """Size the scratch of calls on ``stream`` (the current stream by
    default) up front (sv_init): calls within the bounds then never allocate
    or synchronise."""
    dev = torch.cuda.current_device() if device is None else int(device)
    st = lib().sv_init(dev, _stream(stream), int(max_B), int(max_K), int(max_V), SV_INIT_LMHEAD if lmhead else 0)
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_init")


def stream_release(stream=None) -> None:
    """Free the scratch bound to ``stream`` on the current device."""
    st = lib().sv_stream_release(_stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_stream_release")


def scratch_bytes(device: int | None = None) -> int:
    """Bytes of scratch the library holds on ``device`` (all streams)."""
    return int(lib().sv_scratch_bytes(torch.cuda.current_device() if device is None else int(device)))
