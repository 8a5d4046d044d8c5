"""ctypes binding of libkla.so: argument marshalling only.

Every function here checks the torch tensors it is given (device, dtype, shape,
contiguity), passes their device pointers and the current HIP stream to the C ABI
declared in include/kla.h, and raises KLAError on a non-zero status. All arithmetic
happens in the HIP kernels; there is no fallback of any kind. If the shared library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import pathlib
import re

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libkla.so")
HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "kla.h"

KLA_OK, KLA_ERR_INVALID_VALUE, KLA_ERR_NOT_SUPPORTED, KLA_ERR_LAUNCH = 0, 1, 2, 3
KLA_F32, KLA_BF16 = 0, 1
CHUNK = 64

_lib = None

_c_void_p, _i64, _f32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
_SIGNATURES = {
    "kla_prepare_beta": (_int, [_c_void_p] * 5 + [_i64] * 5 + [_f32, _int, _c_void_p]),
    "kla_chunk_fwd_workspace_size": (ctypes.c_size_t, [_i64] * 6 + [_int]),
    "kla_chunk_fwd": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_f32, _int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_chunk_fwd_noalloc": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_f32, _int, _c_void_p]),
    "kla_chunk_fwd_seg_workspace_size": (ctypes.c_size_t, [_i64] * 7 + [_int]),
    "kla_chunk_fwd_seg": (_int, [_c_void_p] * 8 + [_i64] * 7 + [_f32, _int, _c_void_p, ctypes.c_size_t,
                                                                _c_void_p]),
    "kla_decode_step": (_int, [_c_void_p] * 7 + [_i64] * 4 + [_f32, _int, _c_void_p]),
    "kla_gdn_chunk_fwd": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_gdn_decode_step": (_int, [_c_void_p] * 7 + [_i64] * 4 + [_int, _c_void_p]),
    "kla_chunk_bwd_workspace_size": (ctypes.c_size_t, [_i64] * 6 + [_int]),
    "kla_chunk_bwd": (_int, [_c_void_p] * 14 + [_i64] * 6 + [_f32, _int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_gdn_chunk_bwd": (_int, [_c_void_p] * 14 + [_i64] * 6 + [_int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_chunk_fwd_train": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_f32, _int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_gdn_chunk_fwd_train": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_chunk_bwd_saved": (_int, [_c_void_p] * 14 + [_i64] * 6 + [_f32, _int, _c_void_p, ctypes.c_size_t,
                                                                    _c_void_p]),
    "kla_gdn_chunk_bwd_saved": (_int, [_c_void_p] * 14 + [_i64] * 6 + [_int, _c_void_p, ctypes.c_size_t, _c_void_p]),
    "kla_kda_chunk_fwd_workspace_size": (ctypes.c_size_t, [_i64] * 6 + [_int]),
    "kla_kda_chunk_fwd": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_f32, _int, _int, _c_void_p, ctypes.c_size_t,
                                                               _c_void_p]),
    "kla_kda_decode_step": (_int, [_c_void_p] * 7 + [_i64] * 4 + [_f32, _int, _int, _c_void_p]),
    "kla_kda_chunk_fwd_train": (_int, [_c_void_p] * 8 + [_i64] * 6 + [_f32, _int, _int, _c_void_p, ctypes.c_size_t,
                                                                     _c_void_p]),
    "kla_kda_chunk_bwd_saved": (_int, [_c_void_p] * 14 + [_i64] * 6 + [_f32, _int, _int, _c_void_p,
                                                                         ctypes.c_size_t, _c_void_p]),
    "kla_kda_chunk_bwd_workspace_size": (ctypes.c_size_t, [_i64] * 6 + [_int]),
    "kla_kda_chunk_bwd": (_int, [_c_void_p] * 14 + [_i64] * 6 + [_f32, _int, _int, _c_void_p, ctypes.c_size_t,
                                                                   _c_void_p]),
    "kla_status_string": (ctypes.c_char_p, [_int]),
    "kla_last_error": (ctypes.c_char_p, []),
}


class KLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"status {status}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded C library (loaded on first use). Raises if it has not been built.

    PyTorch is imported first when it is installed: it ships its own HIP runtime, and the
    library's dependency on libamdhip64.so.7 must resolve to that same, already loaded runtime
    (one runtime per process, so torch's device pointers and streams are the library's). Loaded
    the other way round, the system runtime comes in first and torch then finds no GPU."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_18_amd.build`")
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover
            pass
        handle = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def declared_functions() -> list:
    """Names of the functions include/kla.h declares."""
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(kla_[a-z_]+)\s*\(", text)))


def check(status: int) -> None:
    if status != KLA_OK:
        L = lib()
        raise KLAError(status, f"{L.kla_status_string(status).decode()} — {L.kla_last_error().decode()}")


# ------------------------------------------------------------------------- torch-facing wrappers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KLA_BF16
    if t.dtype == torch.float32:
        return KLA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device, stream):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def kla_prepare_beta(k, eta, log_alpha, eps=1e-6, chunk=CHUNK, with_gcum=True, beta_out=None, gcum_out=None,
                     stream=None):
    """beta = eta / (||k||^2 + eps) and the chunk-local log-decay prefix, [B, T, H] fp32 each.
    k [B, T, H, d_k] bf16/fp32 on a GPU; eta, log_alpha [B, T, H] fp32."""
    torch = _torch()
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, d_k]")
    B, T, H, dk = k.shape
    dev = k.device
    _need(k, "k", (B, T, H, dk), k.dtype, dev)
    _need(eta, "eta", (B, T, H), torch.float32, dev)
    _need(log_alpha, "log_alpha", (B, T, H), torch.float32, dev)
    if beta_out is None:
        beta_out = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _need(beta_out, "beta_out", (B, T, H), torch.float32, dev)
    if with_gcum and gcum_out is None:
        gcum_out = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    if gcum_out is not None:
        _need(gcum_out, "gcum_out", (B, T, H), torch.float32, dev)
    check(lib().kla_prepare_beta(_ptr(k), _ptr(eta), _ptr(log_alpha), _ptr(beta_out), _ptr(gcum_out),
                                 B, T, H, dk, chunk, float(eps), _dtype_code(k), _stream(dev, stream)))
    return beta_out, gcum_out


def kla_chunk_fwd_workspace_size(B, T, H, d_k, d_v, chunk=CHUNK, dtype_code=KLA_BF16, segments=None) -> int:
    """Workspace bytes of kla_chunk_fwd (segments None) or of kla_chunk_fwd_seg with that plan."""
    if segments is None:
        return int(lib().kla_chunk_fwd_workspace_size(B, T, H, d_k, d_v, chunk, dtype_code))
    return int(lib().kla_chunk_fwd_seg_workspace_size(B, T, H, d_k, d_v, chunk, segments, dtype_code))


def kla_chunk_fwd(q, k, v, eta, log_alpha, eps=1e-6, state_in=None, return_state=True, o=None, state_out=None,
                  chunk=CHUNK, workspace=None, stream=None, segments=None):
    """Chunkwise KLA forward. q, k [B, T, H, d_k], v [B, T, H, d_v] (bf16 or fp32, one dtype);
    eta, log_alpha [B, T, H] fp32; state_in [B, H, d_k, d_v] fp32 or None (zeros).
    segments None calls kla_chunk_fwd (the library's plan); an int calls kla_chunk_fwd_seg with
    that many sequence segments (0: the library's plan, 1: the one-pass scan).
    Returns (o [B, T, H, d_v] in the input dtype, final state [B, H, d_k, d_v] fp32 or None)."""
    torch = _torch()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, T, H, dk), dt, dev)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(eta, "eta", (B, T, H), torch.float32, dev)
    _need(log_alpha, "log_alpha", (B, T, H), torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(o, "o", (B, T, H, dv), dt, dev)
    if return_state and state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", (B, H, dk, dv), torch.float32, dev)
    code = _dtype_code(q)
    need = kla_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, code, segments)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(log_alpha), _ptr(state_in), _ptr(state_out), _ptr(o),
            B, T, H, dk, dv, chunk)
    tail = (float(eps), code, _ptr(workspace), ws_bytes, _stream(dev, stream))
    if segments is None:
        check(lib().kla_chunk_fwd(*head, *tail))
    else:
        check(lib().kla_chunk_fwd_seg(*head, int(segments), *tail))
    return o, state_out


def kla_chunk_fwd_noalloc(q, k, v, eta, log_alpha, o, eps=1e-6, state_in=None, state_out=None, chunk=CHUNK,
                          stream=None):
    """kla_chunk_fwd through the entry point that allocates nothing (its workspace is the library's
    static scratch): the caller passes every output (o, and state_out or None). Returns (o, state_out)."""
    torch = _torch()
    B, T, H, dk, dv, dev, o, state_out = _fwd_tensors(q, k, v, "eta", eta, log_alpha, False, state_in, False, o,
                                                      state_out)
    check(lib().kla_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(log_alpha), _ptr(state_in),
                                      _ptr(state_out), _ptr(o), B, T, H, dk, dv, chunk, float(eps), _dtype_code(q),
                                      _stream(dev, stream)))
    return o, state_out


def kla_decode_step(q, k, v, eta, log_alpha, state, eps=1e-6, o=None, stream=None):
    """One decode step, in place on ``state``. q, k [B, H, d_k], v [B, H, d_v] (bf16 or fp32);
    eta, log_alpha [B, H] fp32; state [B, H, d_k, d_v] fp32. Returns o [B, H, d_v]."""
    torch = _torch()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, H, dk), dt, dev)
    _need(k, "k", (B, H, dk), dt, dev)
    _need(v, "v", (B, H, dv), dt, dev)
    _need(eta, "eta", (B, H), torch.float32, dev)
    _need(log_alpha, "log_alpha", (B, H), torch.float32, dev)
    _need(state, "state", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _need(o, "o", (B, H, dv), dt, dev)
    check(lib().kla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(log_alpha), _ptr(state), _ptr(o),
                                B, H, dk, dv, float(eps), _dtype_code(q), _stream(dev, stream)))
    return o


def _fwd_tensors(q, k, v, gate_name, gate, log_alpha, log_alpha_optional, state_in, return_state, o, state_out):
    torch = _torch()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, T, H, dk), dt, dev)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(gate, gate_name, (B, T, H), torch.float32, dev)
    if log_alpha is not None or not log_alpha_optional:
        _need(log_alpha, "log_alpha", (B, T, H), torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _need(o, "o", (B, T, H, dv), dt, dev)
    if return_state and state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", (B, H, dk, dv), torch.float32, dev)
    return B, T, H, dk, dv, dev, o, state_out


def kla_gdn_chunk_fwd(q, k, v, beta, log_alpha=None, state_in=None, return_state=True, o=None, state_out=None,
                      chunk=CHUNK, workspace=None, stream=None):
    """Chunkwise gated DeltaNet forward with beta given: as kla_chunk_fwd with beta [B, T, H] fp32
    in place of eta (no key normalisation, no eps); log_alpha None means alpha = 1 (DeltaNet)."""
    torch = _torch()
    B, T, H, dk, dv, dev, o, state_out = _fwd_tensors(q, k, v, "beta", beta, log_alpha, True, state_in,
                                                      return_state, o, state_out)
    code = _dtype_code(q)
    need = kla_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().kla_gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(state_in),
                                  _ptr(state_out), _ptr(o), B, T, H, dk, dv, chunk, code, _ptr(workspace), ws_bytes,
                                  _stream(dev, stream)))
    return o, state_out


def kla_gdn_decode_step(q, k, v, beta, log_alpha, state, o=None, stream=None):
    """One gated DeltaNet decode step with beta [B, H] fp32 given, in place on ``state``;
    log_alpha [B, H] fp32 or None (alpha = 1). Returns o [B, H, d_v]."""
    torch = _torch()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, H, dk), dt, dev)
    _need(k, "k", (B, H, dk), dt, dev)
    _need(v, "v", (B, H, dv), dt, dev)
    _need(beta, "beta", (B, H), torch.float32, dev)
    if log_alpha is not None:
        _need(log_alpha, "log_alpha", (B, H), torch.float32, dev)
    _need(state, "state", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _need(o, "o", (B, H, dv), dt, dev)
    check(lib().kla_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(state), _ptr(o),
                                    B, H, dk, dv, _dtype_code(q), _stream(dev, stream)))
    return o


def kla_chunk_bwd_workspace_size(B, T, H, d_k, d_v, chunk=CHUNK, dtype_code=KLA_BF16) -> int:
    return int(lib().kla_chunk_bwd_workspace_size(B, T, H, d_k, d_v, chunk, dtype_code))


def _bwd(fn_name, gate_name, q, k, v, gate, log_alpha, log_alpha_optional, do, state_in, dstate_out, eps,
         want_dstate_in, chunk, workspace, stream, out):
    torch = _torch()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, T, H, dk), dt, dev)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(do, "do", (B, T, H, dv), dt, dev)
    _need(gate, gate_name, (B, T, H), torch.float32, dev)
    if log_alpha is not None or not log_alpha_optional:
        _need(log_alpha, "log_alpha", (B, T, H), torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", (B, H, dk, dv), torch.float32, dev)
    if dstate_out is not None:
        _need(dstate_out, "dstate_out", (B, H, dk, dv), torch.float32, dev)
    out = dict(out or {})
    shapes = {"dq": ((B, T, H, dk), dt), "dk": ((B, T, H, dk), dt), "dv": ((B, T, H, dv), dt),
              "d" + gate_name: ((B, T, H), torch.float32), "dlog_alpha": ((B, T, H), torch.float32),
              "dstate_in": ((B, H, dk, dv), torch.float32)}
    for name, (shape, dtype) in shapes.items():
        if name == "dlog_alpha" and log_alpha is None:
            out[name] = None
            continue
        if name == "dstate_in" and not want_dstate_in:
            out[name] = None
            continue
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=dtype, device=dev)
        _need(out[name], name, shape, dtype, dev)
    code = _dtype_code(q)
    need = kla_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(log_alpha), _ptr(state_in), _ptr(do), _ptr(dstate_out),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["d" + gate_name]), _ptr(out["dlog_alpha"]),
            _ptr(out["dstate_in"]), B, T, H, dk, dv, chunk]
    args += [float(eps)] if eps is not None else []
    args += [code, _ptr(workspace), ws_bytes, _stream(dev, stream)]
    check(getattr(lib(), fn_name)(*args))
    return out


def kla_chunk_bwd(q, k, v, eta, log_alpha, do, eps=1e-6, state_in=None, dstate_out=None, want_dstate_in=True,
                  chunk=CHUNK, workspace=None, stream=None, out=None):
    """Gradients of L = sum(do * o) + sum(dstate_out * S_T) through kla_chunk_fwd on the same inputs.
    q, k [B, T, H, d_k], v, do [B, T, H, d_v] (bf16 or fp32, one dtype); eta, log_alpha [B, T, H] fp32;
    state_in, dstate_out [B, H, d_k, d_v] fp32 or None (zeros). Returns a dict with dq, dk, dv (input
    dtype), deta, dlog_alpha (fp32) and dstate_in (fp32, or None when not wanted); tensors given in
    ``out`` under those names are written in place."""
    return _bwd("kla_chunk_bwd", "eta", q, k, v, eta, log_alpha, False, do, state_in, dstate_out, eps,
                want_dstate_in, chunk, workspace, stream, out)


def kla_gdn_chunk_bwd(q, k, v, beta, log_alpha, do, state_in=None, dstate_out=None, want_dstate_in=True,
                      chunk=CHUNK, workspace=None, stream=None, out=None):
    """kla_chunk_bwd for the gated DeltaNet form (beta given, log_alpha None for alpha = 1).
    Returns dq, dk, dv, dbeta, dlog_alpha (None when log_alpha is) and dstate_in."""
    return _bwd("kla_gdn_chunk_bwd", "beta", q, k, v, beta, log_alpha, True, do, state_in, dstate_out, None,
                want_dstate_in, chunk, workspace, stream, out)


def _fwd_train(fn_name, gate_name, q, k, v, gate, log_alpha, log_alpha_optional, eps, state_in, return_state, o,
               state_out, chunk, workspace, stream):
    torch = _torch()
    B, T, H, dk, dv, dev, o, state_out = _fwd_tensors(q, k, v, gate_name, gate, log_alpha, log_alpha_optional,
                                                      state_in, return_state, o, state_out)
    code = _dtype_code(q)
    need = kla_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(log_alpha), _ptr(state_in), _ptr(state_out), _ptr(o),
            B, T, H, dk, dv, chunk]
    args += [float(eps)] if eps is not None else []
    args += [code, _ptr(workspace), ws_bytes, _stream(dev, stream)]
    check(getattr(lib(), fn_name)(*args))
    return o, state_out, workspace


def kla_chunk_fwd_train(q, k, v, eta, log_alpha, eps=1e-6, state_in=None, return_state=True, o=None, state_out=None,
                        chunk=CHUNK, workspace=None, stream=None):
    """kla_chunk_fwd for training: also fills the backward's workspace (kla_chunk_bwd_workspace_size
    bytes; allocated when None) for kla_chunk_bwd_saved. Returns (o, final state or None, workspace)."""
    return _fwd_train("kla_chunk_fwd_train", "eta", q, k, v, eta, log_alpha, False, eps, state_in, return_state, o,
                      state_out, chunk, workspace, stream)


def kla_gdn_chunk_fwd_train(q, k, v, beta, log_alpha=None, state_in=None, return_state=True, o=None,
                            state_out=None, chunk=CHUNK, workspace=None, stream=None):
    """kla_gdn_chunk_fwd for training (as kla_chunk_fwd_train). Returns (o, final state or None, workspace)."""
    return _fwd_train("kla_gdn_chunk_fwd_train", "beta", q, k, v, beta, log_alpha, True, None, state_in,
                      return_state, o, state_out, chunk, workspace, stream)


def kla_chunk_bwd_saved(q, k, v, eta, log_alpha, do, workspace, eps=1e-6, state_in=None, dstate_out=None,
                        want_dstate_in=True, chunk=CHUNK, stream=None, out=None):
    """kla_chunk_bwd from the workspace kla_chunk_fwd_train filled for the same inputs (no recompute)."""
    if workspace is None and q.shape[1] > 0:
        raise ValueError("kla_chunk_bwd_saved needs the workspace kla_chunk_fwd_train filled")
    return _bwd("kla_chunk_bwd_saved", "eta", q, k, v, eta, log_alpha, False, do, state_in, dstate_out, eps,
                want_dstate_in, chunk, workspace, stream, out)


def kla_gdn_chunk_bwd_saved(q, k, v, beta, log_alpha, do, workspace, state_in=None, dstate_out=None,
                            want_dstate_in=True, chunk=CHUNK, stream=None, out=None):
    """kla_gdn_chunk_bwd from the workspace kla_gdn_chunk_fwd_train filled for the same inputs."""
    if workspace is None and q.shape[1] > 0:
        raise ValueError("kla_gdn_chunk_bwd_saved needs the workspace kla_gdn_chunk_fwd_train filled")
    return _bwd("kla_gdn_chunk_bwd_saved", "beta", q, k, v, beta, log_alpha, True, do, state_in, dstate_out, None,
                want_dstate_in, chunk, workspace, stream, out)


def kla_kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, chunk=CHUNK, dtype_code=KLA_BF16) -> int:
    return int(lib().kla_kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, chunk, dtype_code))


def kla_kda_chunk_fwd(q, k, v, eta, log_a, eps=1e-6, beta_given=False, state_in=None, return_state=True, o=None,
                      state_out=None, chunk=CHUNK, workspace=None, stream=None):
    """Chunkwise forward with a per-channel decay (KDA's gate): log_a [B, T, H, d_k] fp32; eta
    [B, T, H] fp32 is eta of the Kaczmarz step, or beta itself when beta_given. Otherwise as
    kla_chunk_fwd. Returns (o, final state or None)."""
    o, state_out, _ = _kda_fwd("kla_kda_chunk_fwd", kla_kda_chunk_fwd_workspace_size, q, k, v, eta, log_a, eps,
                               beta_given, state_in, return_state, o, state_out, chunk, workspace, stream)
    return o, state_out


def kla_kda_chunk_fwd_train(q, k, v, eta, log_a, eps=1e-6, beta_given=False, state_in=None, return_state=True,
                            o=None, state_out=None, chunk=CHUNK, workspace=None, stream=None):
    """kla_kda_chunk_fwd for training: also fills the backward's workspace (kla_kda_chunk_bwd_workspace_size
    bytes; allocated when None) for kla_kda_chunk_bwd_saved. Returns (o, final state or None, workspace)."""
    return _kda_fwd("kla_kda_chunk_fwd_train", kla_kda_chunk_bwd_workspace_size, q, k, v, eta, log_a, eps,
                    beta_given, state_in, return_state, o, state_out, chunk, workspace, stream)


def _kda_fwd(fn_name, size_fn, q, k, v, eta, log_a, eps, beta_given, state_in, return_state, o, state_out, chunk,
             workspace, stream):
    torch = _torch()
    B, T, H, dk, dv, dev, o, state_out = _fwd_tensors(q, k, v, "eta", eta, None, True, state_in, return_state, o,
                                                      state_out)
    _need(log_a, "log_a", (B, T, H, dk), torch.float32, dev)
    code = _dtype_code(q)
    need = size_fn(B, T, H, dk, dv, chunk, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(getattr(lib(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(log_a), _ptr(state_in),
                                  _ptr(state_out), _ptr(o), B, T, H, dk, dv, chunk, float(eps), int(bool(beta_given)),
                                  code, _ptr(workspace), ws_bytes, _stream(dev, stream)))
    return o, state_out, workspace


def kla_kda_decode_step(q, k, v, eta, log_a, state, eps=1e-6, beta_given=False, o=None, stream=None):
    """One decode step with a per-channel decay, in place on ``state``: log_a [B, H, d_k] fp32;
    eta [B, H] (eta of the Kaczmarz step, or beta when beta_given). Returns o [B, H, d_v]."""
    torch = _torch()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [B, H, d]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, H, dk), dt, dev)
    _need(k, "k", (B, H, dk), dt, dev)
    _need(v, "v", (B, H, dv), dt, dev)
    _need(eta, "eta", (B, H), torch.float32, dev)
    _need(log_a, "log_a", (B, H, dk), torch.float32, dev)
    _need(state, "state", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _need(o, "o", (B, H, dv), dt, dev)
    check(lib().kla_kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(log_a), _ptr(state), _ptr(o),
                                    B, H, dk, dv, float(eps), int(bool(beta_given)), _dtype_code(q),
                                    _stream(dev, stream)))
    return o



def kla_kda_chunk_bwd_workspace_size(B, T, H, d_k, d_v, chunk=CHUNK, dtype_code=KLA_BF16) -> int:
    return int(lib().kla_kda_chunk_bwd_workspace_size(B, T, H, d_k, d_v, chunk, dtype_code))


def kla_kda_chunk_bwd(q, k, v, eta, log_a, do, eps=1e-6, beta_given=False, state_in=None, dstate_out=None,
                      want_dstate_in=True, chunk=CHUNK, workspace=None, stream=None, out=None):
    """Gradients of L = sum(do * o) + sum(dstate_out * S_T) through kla_kda_chunk_fwd on the same
    inputs: log_a [B, T, H, d_k] fp32, eta [B, T, H] fp32 (beta itself when beta_given), the rest as
    kla_chunk_bwd. Returns a dict with dq, dk, dv (input dtype), deta (d beta when beta_given),
    dlog_a [B, T, H, d_k] (fp32) and dstate_in (fp32, or None when not wanted); tensors given in
    ``out`` under those names are written in place."""
    return _kda_bwd("kla_kda_chunk_bwd", q, k, v, eta, log_a, do, eps, beta_given, state_in, dstate_out,
                    want_dstate_in, chunk, workspace, stream, out)


def kla_kda_chunk_bwd_saved(q, k, v, eta, log_a, do, workspace, eps=1e-6, beta_given=False, state_in=None,
                            dstate_out=None, want_dstate_in=True, chunk=CHUNK, stream=None, out=None):
    """kla_kda_chunk_bwd from the workspace kla_kda_chunk_fwd_train filled for the same inputs."""
    if workspace is None and q.shape[1] > 0:
        raise ValueError("kla_kda_chunk_bwd_saved needs the workspace kla_kda_chunk_fwd_train filled")
    return _kda_bwd("kla_kda_chunk_bwd_saved", q, k, v, eta, log_a, do, eps, beta_given, state_in, dstate_out,
                    want_dstate_in, chunk, workspace, stream, out)


def _kda_bwd(fn_name, q, k, v, eta, log_a, do, eps, beta_given, state_in, dstate_out, want_dstate_in, chunk,
             workspace, stream, out):
    torch = _torch()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need(q, "q", (B, T, H, dk), dt, dev)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(do, "do", (B, T, H, dv), dt, dev)
    _need(eta, "eta", (B, T, H), torch.float32, dev)
    _need(log_a, "log_a", (B, T, H, dk), torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", (B, H, dk, dv), torch.float32, dev)
    if dstate_out is not None:
        _need(dstate_out, "dstate_out", (B, H, dk, dv), torch.float32, dev)
    out = dict(out or {})
    shapes = {"dq": ((B, T, H, dk), dt), "dk": ((B, T, H, dk), dt), "dv": ((B, T, H, dv), dt),
              "deta": ((B, T, H), torch.float32), "dlog_a": ((B, T, H, dk), torch.float32),
              "dstate_in": ((B, H, dk, dv), torch.float32)}
    for name, (shape, dtype) in shapes.items():
        if name == "dstate_in" and not want_dstate_in:
            out[name] = None
            continue
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=dtype, device=dev)
        _need(out[name], name, shape, dtype, dev)
    code = _dtype_code(q)
    need = kla_kda_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(getattr(lib(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(log_a), _ptr(state_in), _ptr(do),
                                  _ptr(dstate_out), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                  _ptr(out["deta"]), _ptr(out["dlog_a"]), _ptr(out["dstate_in"]), B, T, H, dk, dv,
                                  chunk, float(eps), int(bool(beta_given)), code, _ptr(workspace), ws_bytes,
                                  _stream(dev, stream)))
    return out
