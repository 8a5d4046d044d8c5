"""Seeded synthetic inputs for the Kaczmarz Linear Attention hot path.

Both sides of every comparison take their inputs from here: the HIP library
(through the Python binding) and the CPU oracle. This module holds random draws
and dtype rounding only, none of the method's arithmetic.

Distributions (per element i.i.d.; scalars are per (b, t, h)):
  q     = N(0, 1) / sqrt(d_k)
  k     = N(0, 1) / sqrt(d_k) * s_t,  s_t = exp(U(ln 0.25, ln 4))   (unnormalised keys)
  v     = N(0, 1)
  eta   = sigmoid(N(0, eta_std))                                   (already activated)
  log_alpha = -U(a_lo, a_hi)                                       (alpha = exp(log_alpha))
  S0    = N(0, s0_std) fp32, or zeros
  do    = N(0, 1) (the cotangent of o for gradient checks; bf16-rounded for bf16 workloads)
  dS_T  = N(0, dst_std) fp32 (the cotangent of the final state), or absent
  log a = -U(a_lo, a_hi) per channel (per-channel decay, [.., d_k]), the scalar gate's range
bf16 workloads round q, k, v from fp32 to bf16 (round to nearest even); the
arrays returned here hold those rounded values as fp32, so that an fp64 upcast
is exact and both sides see the very same numbers.

Every head (b, h) of every tensor has its own generator stream keyed by
(SEED, workload id, tensor id, b, h), so a subset of heads can be regenerated
without drawing the rest. Decode workloads draw all steps of one head from one
stream: step s is row s.
"""
from __future__ import annotations

import concurrent.futures
import math
import multiprocessing
import os
from dataclasses import dataclass, field, replace

import numpy as np

SEED = 20260509

# Stream ids per tensor (prefill tensors, then decode-step tensors).
_TID = {
    "q": 1, "k": 2, "v": 3, "eta": 4, "log_alpha": 5, "scale": 6, "S0": 7,
    "dec_q": 11, "dec_k": 12, "dec_v": 13, "dec_eta": 14, "dec_log_alpha": 15, "dec_scale": 16,
    "do": 21, "dST": 22, "S0_prefill": 23, "log_a": 24, "dec_log_a": 25,
}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype and input distributions."""
    name: str
    wid: int                 # stream key; distinct per workload
    B: int
    H: int
    dk: int
    dv: int
    T: int = 0               # prefill length (0: no prefill)
    steps: int = 0           # decode steps (0: no decode)
    dtype: str = "bf16"      # "bf16" or "f32" for q, k, v, o
    eps: float = 1e-6
    chunk: int = 64
    eta_std: float = 1.0
    log_alpha_range: tuple = (0.001, 0.1)
    key_scale_range: tuple = (0.25, 4.0)
    s0_std: float = 0.0      # decode-only workloads start from N(0, s0_std)
    return_state: bool = True
    note: str = field(default="", compare=False)

    @property
    def heads(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the benchmark description. Parity tests use all of them;
# the benchmark's default step is the mixed prefill + decode one.
WORKLOADS = {
    "fwd_tiny_f32": Workload("fwd_tiny_f32", 0, B=1, H=1, dk=64, dv=64, T=256, dtype="f32",
                             note="KLA fwd B1 H1 T256 d64 fp32, chunk 64"),
    "fwd_b8h8_t4096": Workload("fwd_b8h8_t4096", 1, B=8, H=8, dk=128, dv=128, T=4096,
                               note="KLA chunked fwd B8 H8 T4096 d128 bf16"),
    "fwd_long_t65536": Workload("fwd_long_t65536", 2, B=1, H=16, dk=128, dv=128, T=65536,
                                note="KLA chunked fwd B1 H16 T65536 d128 bf16, returns S_T"),
    "decode_b64h16": Workload("decode_b64h16", 3, B=64, H=16, dk=128, dv=128, steps=1024,
                              s0_std=0.02,
                              note="KLA decode B64 H16 d128, 1024 steps, S0~N(0,0.02)"),
    "mixed_b4h16": Workload("mixed_b4h16", 4, B=4, H=16, dk=128, dv=128, T=32768, steps=512,
                            eta_std=2.0, log_alpha_range=(0.0, 0.2),
                            note="KLA prefill B4 H16 T32768 then 512 decode steps, d128 bf16"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(w: Workload, tensor: str, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng([SEED, w.wid, _TID[tensor], b, h])


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _draw_tokens(w: Workload, prefix: str, b: int, h: int, n: int) -> dict:
    """q, k, v [n, d], eta, log_alpha [n] for head (b, h)."""
    p = prefix
    q = _rng(w, p + "q", b, h).standard_normal((n, w.dk), dtype=np.float32) / np.float32(math.sqrt(w.dk))
    lo, hi = w.key_scale_range
    s = np.exp(_rng(w, p + "scale", b, h).uniform(math.log(lo), math.log(hi), n)).astype(np.float32)
    k = _rng(w, p + "k", b, h).standard_normal((n, w.dk), dtype=np.float32) / np.float32(math.sqrt(w.dk))
    k *= s[:, None]
    v = _rng(w, p + "v", b, h).standard_normal((n, w.dv), dtype=np.float32)
    eta = _sigmoid(_rng(w, p + "eta", b, h).normal(0.0, w.eta_std, n)).astype(np.float32)
    a_lo, a_hi = w.log_alpha_range
    log_alpha = (-_rng(w, p + "log_alpha", b, h).uniform(a_lo, a_hi, n)).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return {"q": q, "k": k, "v": v, "eta": eta, "log_alpha": log_alpha}


def head_prefill(w: Workload, b: int, h: int) -> dict:
    """Prefill inputs of one head: q, k [T, dk], v [T, dv], eta, log_alpha [T]."""
    return _draw_tokens(w, "", b, h, w.T)


def head_decode(w: Workload, b: int, h: int) -> dict:
    """Decode inputs of one head for all steps: q, k [steps, dk], v [steps, dv], eta, log_alpha [steps],
    plus S0 [dk, dv] (zeros unless the workload starts from a random state)."""
    d = _draw_tokens(w, "dec_", b, h, w.steps)
    if w.s0_std > 0:
        d["S0"] = _rng(w, "S0", b, h).normal(0.0, w.s0_std, (w.dk, w.dv)).astype(np.float32)
    else:
        d["S0"] = np.zeros((w.dk, w.dv), np.float32)
    return d


def _heads_block(fn, w: Workload, heads) -> list:
    return [fn(w, b, h) for b, h in heads]


def _per_head(fn, w: Workload, elements: int, workers=None) -> list:
    """fn(w, b, h) for every head in (b, h) order. Large workloads (more than 2^26 drawn elements)
    are drawn in worker processes (`workers`, default the CPUs available up to 16; 1 draws in this
    process), one block of heads each; every head has its own stream, so the values do not depend
    on how the heads are split."""
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    nw = min(len(os.sched_getaffinity(0)) if workers is None else workers, 16, len(heads))
    if elements < (1 << 26) or nw < 2:
        return _heads_block(fn, w, heads)
    blocks = [heads[i * len(heads) // nw:(i + 1) * len(heads) // nw] for i in range(nw)]
    with concurrent.futures.ProcessPoolExecutor(nw, mp_context=multiprocessing.get_context("spawn")) as ex:
        parts = ex.map(_heads_block, [fn] * nw, [w] * nw, blocks)
        return [d for part in parts for d in part]


def prefill_inputs(w: Workload, workers=None) -> dict:
    """All heads in the library layout: q, k [B, T, H, dk], v [B, T, H, dv], eta, log_alpha [B, T, H]."""
    out = {
        "q": np.empty((w.B, w.T, w.H, w.dk), np.float32),
        "k": np.empty((w.B, w.T, w.H, w.dk), np.float32),
        "v": np.empty((w.B, w.T, w.H, w.dv), np.float32),
        "eta": np.empty((w.B, w.T, w.H), np.float32),
        "log_alpha": np.empty((w.B, w.T, w.H), np.float32),
    }
    for i, d in enumerate(_per_head(head_prefill, w, w.heads * w.T * (2 * w.dk + w.dv), workers)):
        b, h = divmod(i, w.H)
        for name, arr in d.items():
            out[name][b, :, h] = arr
    return out


def decode_inputs(w: Workload, workers=None) -> dict:
    """All heads, all steps: q, k [steps, B, H, dk], v [steps, B, H, dv], eta, log_alpha [steps, B, H],
    S0 [B, H, dk, dv]. Step s is the slice [s]."""
    out = {
        "q": np.empty((w.steps, w.B, w.H, w.dk), np.float32),
        "k": np.empty((w.steps, w.B, w.H, w.dk), np.float32),
        "v": np.empty((w.steps, w.B, w.H, w.dv), np.float32),
        "eta": np.empty((w.steps, w.B, w.H), np.float32),
        "log_alpha": np.empty((w.steps, w.B, w.H), np.float32),
        "S0": np.empty((w.B, w.H, w.dk, w.dv), np.float32),
    }
    for i, d in enumerate(_per_head(head_decode, w, w.heads * (w.steps * (2 * w.dk + w.dv) + w.dk * w.dv),
                                    workers)):
        b, h = divmod(i, w.H)
        for name, arr in d.items():
            if name == "S0":
                out[name][b, h] = arr
            else:
                out[name][:, b, h] = arr
    return out


def custom(name: str, wid: int, **kw) -> Workload:
    """A test workload with its own stream key (wid >= 100 keeps it apart from the named ones)."""
    return Workload(name=name, wid=wid, **kw)


def head_grad(w: Workload, b: int, h: int, s0_std: float = 0.0, dst_std: float = 0.0) -> dict:
    """Cotangents of one head: do [T, dv] (bf16-rounded for bf16 workloads), and, when the std is
    positive, an initial state S0 and a final-state cotangent dST [dk, dv] fp32 (else None)."""
    x = _rng(w, "do", b, h).standard_normal((w.T, w.dv), dtype=np.float32)
    return {
        "do": round_to_bf16(x) if w.dtype == "bf16" else x,
        "S0": _rng(w, "S0_prefill", b, h).normal(0.0, s0_std, (w.dk, w.dv)).astype(np.float32) if s0_std > 0 else None,
        "dST": _rng(w, "dST", b, h).normal(0.0, dst_std, (w.dk, w.dv)).astype(np.float32) if dst_std > 0 else None,
    }


def grad_inputs(w: Workload, s0_std: float = 0.0, dst_std: float = 0.0) -> dict:
    """Cotangents for gradient checks, all heads: do [B, T, H, dv] and, when the std is positive,
    S0 and dST [B, H, dk, dv] (else None), as head_grad."""
    do = np.empty((w.B, w.T, w.H, w.dv), np.float32)
    S0 = np.empty((w.B, w.H, w.dk, w.dv), np.float32) if s0_std > 0 else None
    dST = np.empty((w.B, w.H, w.dk, w.dv), np.float32) if dst_std > 0 else None
    for b in range(w.B):
        for h in range(w.H):
            d = head_grad(w, b, h, s0_std, dst_std)
            do[b, :, h] = d["do"]
            if S0 is not None:
                S0[b, h] = d["S0"]
            if dST is not None:
                dST[b, h] = d["dST"]
    return {"do": do, "S0": S0, "dST": dST}


def head_channel_log_decay(w: Workload, b: int, h: int, decode: bool = False) -> np.ndarray:
    """Per-channel log decays of one head: [T, dk] (prefill) or [steps, dk] (decode), each element
    -U(a_lo, a_hi) with the workload's scalar-gate range."""
    a_lo, a_hi = w.log_alpha_range
    n = w.steps if decode else w.T
    return (-_rng(w, "dec_log_a" if decode else "log_a", b, h).uniform(a_lo, a_hi, (n, w.dk))).astype(np.float32)


def channel_log_decay(w: Workload, decode: bool = False) -> np.ndarray:
    """Per-channel log decays for all heads: [B, T, H, dk] (prefill) or [steps, B, H, dk]
    (decode), as head_channel_log_decay."""
    n = w.steps if decode else w.T
    out = np.empty((n, w.B, w.H, w.dk) if decode else (w.B, n, w.H, w.dk), np.float32)
    for b in range(w.B):
        for h in range(w.H):
            x = head_channel_log_decay(w, b, h, decode)
            if decode:
                out[:, b, h] = x
            else:
                out[b, :, h] = x
    return out

