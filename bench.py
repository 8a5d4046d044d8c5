#!/usr/bin/env python3
"""Benchmark of the Kaczmarz Linear Attention hot path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input. The
default workload, mixed_b4h16, is a chunkwise prefill over B=4, H=16, T=32768,
d_k=d_v=128 (bf16 q/k/v/o, fp32 state and gates) followed by 512 recurrent decode
steps that continue from the prefill's final states, so every stage runs: the
beta/decay prologue, the chunk products, the triangular solve, the state scan, the
output and the decode step. Other workloads (--workload) time one part alone.
--pass bwd times the chunkwise backward (kla_chunk_bwd: the gradients of a loss on the
prefill outputs with respect to every input) on a prefill workload instead, as its own
JSON line; --pass train times a training step, the training forward (kla_chunk_fwd_train)
and the backward from its workspace (kla_chunk_bwd_saved).

Inputs are generated (seeded) and copied to HBM before the timed region. Kernels
are launched through the C ABI with pre-marshalled pointers on torch's current
stream; the decode steps of a bench step are replayed from a HIP graph captured
once before timing (--decode-launch eager issues them one call at a time). HIP
events on that stream time each part. Prints one JSON line.

After the timed steps, the default run also times, each alone and outside `value`, the
other named workloads (B8 H8 T4096 and B1 H16 T65536 prefill behind a 512 MiB cache-evicting
write, the B64 H16 1024-step decode), a decode whose 512 MiB state exceeds the last-level
cache, and a B8 H8 T4096 training step with the scalar gate and with the per-channel decay,
under parts["extra:<name>"] (--no-extras skips them). The CPU baseline
times the fp64 oracle on the host's cores (worker processes, at most 16) on a bounded
sample of the prefill and of the decode steps.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "chunked-fwd tokens/s + decode tokens/s at 1 GPU; % MFMA / HBM roofline"
METRIC_BWD = "chunked-bwd tokens/s at 1 GPU; % MFMA / HBM roofline"
METRIC_TRAIN = "chunked training step (fwd + bwd) tokens/s at 1 GPU; % MFMA / HBM roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA


def chunk_flops_per_head_token(dk, dv, C=64):
    """Dense chunk-product count: K K^T, Q K^T, T (beta K), T (beta V), P Delta (C-wide),
    W S, Q S, K^T Delta (d_k x d_v-wide)."""
    return 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv


def chunk_bytes(w, es):
    """Algorithmic HBM bytes of one prefill launch: q, k, v, o, eta, log_alpha once, plus the
    final state written (and the initial one read when given)."""
    per_tok = (2 * w.dk + 2 * w.dv) * es + 8
    return w.heads * w.T * per_tok + w.heads * w.dk * w.dv * 4


def bwd_flops_per_head_token(dk, dv, C=64):
    """Dense chunk-product count of the backward: the per-chunk factors again (K K^T, Q K^T),
    the recompute scan (K S, T R, K^T Delta), the reverse scan (K dS', P^T dO, T^T R',
    Q^T dO, K^T Zb) and the gradient kernel (K K^T, Q K^T, Zb Delta^T, dO Delta^T, four
    C x C x d_k products, three C x d_k x d_v products)."""
    return C * (16 * dk + 10 * dv) + 16 * dk * dv


def train_flops_per_head_token(dk, dv, C=64):
    """A training step: the forward's products and the backward's, less the backward's recompute
    of the forward (K K^T and Q K^T of the per-chunk factors, K S, T R and K^T Delta of the
    scan), which the training forward's saved workspace makes unnecessary."""
    return chunk_flops_per_head_token(dk, dv, C) + bwd_flops_per_head_token(dk, dv, C) - (4 * C * dk + 2 * C * dv +
                                                                                          4 * dk * dv)


def bwd_bytes(w, es, kda=False):
    """Algorithmic HBM bytes of one backward launch: q, k, v, do, eta, log_alpha read once;
    dq, dk, dv, deta, dlog_alpha written once (no initial state, no state cotangent). With the
    per-channel decay, log a and dlog a are d_k fp32 per head-token."""
    gate = 8 + (8 * w.dk if kda else 8)
    return w.heads * w.T * ((3 * w.dk + 3 * w.dv) * es + gate)


def decode_bytes(w, es):
    """Algorithmic HBM bytes of one decode launch: the fp32 state read and written once,
    q, k, v, o, eta, log_alpha."""
    return w.heads * (2 * w.dk * w.dv * 4 + (2 * w.dk + 2 * w.dv) * es + 8)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source files of each timed part; the recorded HBM traffic of a part is only reported while
# the code in these files (comments and whitespace aside) is the code the counters were taken on.
CSRC = os.path.join(ROOT, "gated_delta_rule_18_amd", "csrc")
PART_SOURCES = {
    "chunk_fwd": ["chunk_common.h", "chunk_prep.hip", "chunk_scan.hip", "chunk_seg.hip", "tile_ops.h",
                  "kla_device.h", "kla_launch.h"],
    "decode": ["decode.hip", "kla_device.h", "kla_launch.h"],
    "chunk_bwd": ["chunk_common.h", "chunk_prep.hip", "chunk_scan.hip", "chunk_bwd_scan.hip", "chunk_bwd_grad.hip",
                  "tile_ops.h", "kla_device.h", "kla_launch.h"],
}
# The per-channel decay runs other kernels (or other instantiations) of the same files.
PART_SOURCES["chunk_fwd_kda"] = PART_SOURCES["chunk_fwd"]
PART_SOURCES["decode_kda"] = PART_SOURCES["decode"]
PART_SOURCES["chunk_bwd_kda"] = PART_SOURCES["chunk_bwd"] + ["chunk_bwd_grad_kda.hip"]
# A training step (the saving forward, then the backward from its workspace) runs the same files.
PART_SOURCES["chunk_train"] = PART_SOURCES["chunk_bwd"]
PART_SOURCES["chunk_train_kda"] = PART_SOURCES["chunk_bwd_kda"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def sources_sha(part):
    """Hash of the part's kernel sources with comments and whitespace removed, so that an edit of
    comments alone keeps the recorded traffic of unchanged code."""
    h = hashlib.sha256()
    for f in PART_SOURCES[part]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_key(part, mode):
    """Name under which the traffic of `part` in decay mode `mode` is recorded."""
    return part if mode == "kla" else part + "_kda"


def recorded_traffic(workload, part):
    """HBM bytes per launch of `part` on `workload` (bytes read plus bytes written), from the
    rocprofv3 request-size counter runs recorded in profiles/hbm_traffic.txt, or None if there is
    no record for the current sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = sources_sha(part)
    for line in open(TRAFFIC_FILE):
        if not line.startswith("traffic "):
            continue
        kv = dict(f.split("=", 1) for f in line.split()[1:])
        if kv.get("workload") == workload and kv.get("part") == part and kv.get("sources_sha") == want:
            return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def unit_keys(k):
    """Keys scaled to unit norm: input preparation for the beta-given modes, which are used with
    normalised keys (the plain delta rule diverges when beta ||k||^2 exceeds 2)."""
    n = np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
    return (k / np.maximum(n, 1e-3)).astype(np.float32)


def _oracle_leg(w, heads, n, leg, mode):
    """One worker of the CPU baseline: regenerates the inputs of `heads` (the first n prefill tokens,
    or n decode steps) and times the fp64 oracle on them alone. Returns (seconds, head-tokens)."""
    import oracle
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    if leg == "decode":
        d = [wl.head_decode(w.with_(steps=n), b, h) for b, h in heads]
        st = lambda key: np.stack([x[key] for x in d])
        args = (st("q"), st("k"), st("v"), st("eta"), st("log_alpha"), w.eps, st("S0"))
        run = lambda: oracle.kla_recurrent(*args)
    else:
        ws = w.with_(T=n)
        d = [wl.head_prefill(ws, b, h) for b, h in heads]
        st = lambda key: np.stack([x[key] for x in d])
        if mode == "kda":
            la = np.stack([wl.head_channel_log_decay(ws, b, h) for b, h in heads])
            k = st("k")
            args = (st("q"), k, st("v"), oracle.kaczmarz_step_size(k, st("eta"), w.eps), la)
            run = lambda: oracle.kda_recurrent(*args)
        elif mode in ("gdn", "deltanet"):
            la = st("log_alpha") if mode == "gdn" else np.zeros((len(heads), n))
            args = (st("q"), unit_keys(st("k")), st("v"), st("eta"), la)
            run = lambda: oracle.gated_delta_recurrent(*args)
        else:
            args = (st("q"), st("k"), st("v"), st("eta"), st("log_alpha"), w.eps)
            run = lambda: oracle.kla_recurrent(*args)
    t0 = time.perf_counter()
    run()
    return time.perf_counter() - t0, len(heads) * n


def _oracle_pool_time(w, n, leg, mode, cores):
    """Times the oracle over every head of w (n tokens or steps each), split over `cores` worker
    processes that run at once. The leg's time is that of the slowest worker (input generation
    excluded); also returns the mean rate of one worker, in head-tokens per second per core."""
    import concurrent.futures
    import multiprocessing
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    groups = [heads[i::cores] for i in range(cores) if heads[i::cores]]
    with concurrent.futures.ProcessPoolExecutor(len(groups), mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_leg, [w] * len(groups), groups, [n] * len(groups), [leg] * len(groups),
                          [mode] * len(groups)))
    secs = max(t for t, _ in res)
    per_core = sum(ht / t for t, ht in res) / len(res)
    return secs, len(heads) * n, per_core, len(groups)


def cpu_baseline(w, head_tokens, mode="kla"):
    """The fp64 oracle, as it stands, timed on the host's cores (at most 16 worker processes, one
    thread each) on a bounded sample of the same workload: every head over the first
    head_tokens / (B H) prefill tokens, and every head over the workload's decode steps (at most
    head_tokens / (B H)). The recurrence costs the same per token at any position, so each leg's
    rate scales to the whole workload; value is one bench step's tokens (prefill B T plus decode
    B steps) over the oracle time those rates give."""
    avail = len(os.sched_getaffinity(0))
    cores = max(1, min(avail, 16, w.heads))
    legs, what = {}, []
    if w.T:
        n = max(1, min(head_tokens // w.heads, w.T))
        secs, ht, per_core, used = _oracle_pool_time(w, n, "prefill", mode, cores)
        legs["prefill"] = {"tokens_per_s": w.B * n / secs, "head_tokens": ht, "seconds": secs,
                           "head_tokens_per_s_per_core": per_core}
        what.append(f"prefill: all {w.heads} heads x the first {n} tokens ({ht} head-tokens) in {secs:.2f} s")
    if w.steps:
        n = max(1, min(head_tokens // w.heads, w.steps))
        secs, ht, per_core, used = _oracle_pool_time(w, n, "decode", "kla", cores)
        legs["decode"] = {"tokens_per_s": w.B * n / secs, "head_tokens": ht, "seconds": secs,
                          "head_tokens_per_s_per_core": per_core}
        what.append(f"decode: all {w.heads} heads x {n} steps ({ht} head-steps) in {secs:.2f} s")
    t_step = (w.B * w.T / legs["prefill"]["tokens_per_s"] if w.T else 0.0) + (
        w.B * w.steps / legs["decode"]["tokens_per_s"] if w.steps else 0.0)
    single = 1.0 / ((w.heads * w.T / legs["prefill"]["head_tokens_per_s_per_core"] if w.T else 0.0) +
                    (w.heads * w.steps / legs["decode"]["head_tokens_per_s_per_core"] if w.steps else 0.0))
    return {"value": (w.B * w.T + w.B * w.steps) / t_step, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cores_available": avail, "legs": legs,
            "single_core_value": (w.B * w.T + w.B * w.steps) * single,
            "sample": (f"fp64 oracle ({'kda_recurrent' if mode == 'kda' else 'gated_delta_recurrent' if mode != 'kla' else 'kla_recurrent'}"
                       f", numpy) in {cores} worker processes of one thread each, heads split between them; "
                       + "; ".join(what) + "; a leg's time is its slowest worker's, input generation excluded")}


def cpu_baseline_bwd(w, head_tokens, kda=False):
    """The fp64 gradient oracle (the adjoint of the token loop), as it stands, on a bounded sample:
    every head over the first head_tokens / (B H) prefill tokens, in worker processes."""
    import concurrent.futures
    import multiprocessing
    avail = len(os.sched_getaffinity(0))
    cores = max(1, min(avail, 16, w.heads))
    n = max(1, min(head_tokens // w.heads, w.T))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    groups = [heads[i::cores] for i in range(cores) if heads[i::cores]]
    with concurrent.futures.ProcessPoolExecutor(len(groups), mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_bwd_leg, [w] * len(groups), groups, [n] * len(groups), [kda] * len(groups)))
    secs = max(t for t, _ in res)
    return {"value": w.B * n / secs, "unit": "tokens/s", "cores": len(groups), "kind": "oracle",
            "cores_available": avail,
            "sample": f"oracle {'kda' if kda else 'kla'}_adjoint (fp64 numpy, one thread per worker) on all {w.heads} heads x the first "
                      f"{n} prefill tokens in {len(groups)} worker processes: {len(heads) * n} head-tokens in "
                      f"{secs:.2f} s (slowest worker; input generation excluded)"}


def _oracle_bwd_leg(w, heads, n, kda=False):
    import oracle
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    ws = w.with_(T=n)
    d = [wl.head_prefill(ws, b, h) for b, h in heads]
    g = [wl.head_grad(ws, b, h) for b, h in heads]
    st = lambda key, src=d: np.stack([x[key] for x in src])
    if kda:
        la = np.stack([wl.head_channel_log_decay(ws, b, h) for b, h in heads])
        t0 = time.perf_counter()
        oracle.kda_adjoint(st("q"), st("k"), st("v"), st("eta"), la, w.eps, None, st("do", g))
    else:
        t0 = time.perf_counter()
        oracle.kla_adjoint(st("q"), st("k"), st("v"), st("eta"), st("log_alpha"), w.eps, None, st("do", g))
    return time.perf_counter() - t0, len(heads) * n


def measure_bwd(w, mode, train, steps, warmup):
    """Times kla_chunk_bwd (kla_gdn_chunk_bwd, kla_kda_chunk_bwd; mode kla, gdn, deltanet or kda)
    over the workload's prefill, or with train the pair kla_chunk_fwd_train + kla_chunk_bwd_saved
    (their gdn / KDA forms), for `steps` steps after `warmup`. Returns (part, elapsed seconds)."""
    import torch
    from gated_delta_rule_18_amd import _lib as K
    device = torch.device("cuda:0")
    es = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = K.KLA_BF16 if w.dtype == "bf16" else K.KLA_F32
    L = K.lib()
    gdn = mode in ("gdn", "deltanet")
    kda = mode == "kda"
    log(f"[bench] generating {w.name} ({w.note}) and its output cotangent ...")
    on = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(device)
    x = wl.prefill_inputs(w, GEN_WORKERS)
    if gdn:
        x["k"] = unit_keys(x["k"])
    x["do"] = wl.grad_inputs(w)["do"]
    if kda:
        x["log_alpha"] = wl.channel_log_decay(w)
    t = {n: on(x[n], tdt if n in ("q", "k", "v", "do") else torch.float32) for n in x}
    del x
    out = {"dq": torch.empty_like(t["q"]), "dk": torch.empty_like(t["k"]), "dv": torch.empty_like(t["v"]),
           "deta": torch.empty_like(t["eta"]), "dla": torch.empty_like(t["log_alpha"])}
    ws_fn = L.kla_kda_chunk_bwd_workspace_size if kda else L.kla_chunk_bwd_workspace_size
    ws_bytes = int(ws_fn(w.B, w.T, w.H, w.dk, w.dv, 64, code))
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())
    la = None if mode == "deltanet" else P(t["log_alpha"])
    dla = None if mode == "deltanet" else P(out["dla"])
    head = (P(t["q"]), P(t["k"]), P(t["v"]), P(t["eta"]), la, None, P(t["do"]), None, P(out["dq"]), P(out["dk"]),
            P(out["dv"]), P(out["deta"]), dla, None, w.B, w.T, w.H, w.dk, w.dv, 64)
    if train:
        o = torch.empty_like(t["v"])
        fhead = (P(t["q"]), P(t["k"]), P(t["v"]), P(t["eta"]), la, None, None, P(o), w.B, w.T, w.H, w.dk, w.dv, 64)
        if kda:
            eps = ctypes.c_float(w.eps)
            call = lambda: (L.kla_kda_chunk_fwd_train(*fhead, eps, 0, code, P(workspace), ws_bytes, sp) or
                            L.kla_kda_chunk_bwd_saved(*head, eps, 0, code, P(workspace), ws_bytes, sp))
        elif gdn:
            call = lambda: (L.kla_gdn_chunk_fwd_train(*fhead, code, P(workspace), ws_bytes, sp) or
                            L.kla_gdn_chunk_bwd_saved(*head, code, P(workspace), ws_bytes, sp))
        else:
            eps = ctypes.c_float(w.eps)
            call = lambda: (L.kla_chunk_fwd_train(*fhead, eps, code, P(workspace), ws_bytes, sp) or
                            L.kla_chunk_bwd_saved(*head, eps, code, P(workspace), ws_bytes, sp))
    elif gdn:
        call = lambda: L.kla_gdn_chunk_bwd(*head, code, P(workspace), ws_bytes, sp)
    elif kda:
        call = lambda: L.kla_kda_chunk_bwd(*head, ctypes.c_float(w.eps), 0, code, P(workspace), ws_bytes, sp)
    else:
        call = lambda: L.kla_chunk_bwd(*head, ctypes.c_float(w.eps), code, P(workspace), ws_bytes, sp)
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    log(f"[bench] warmup {warmup} step(s)")
    for _ in range(warmup):
        K.check(call())
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} step(s)")
    evs = [ev() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        st = call()
        e[1].record(stream)
        if st:
            K.check(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed region {elapsed * 1e3:.2f} ms")
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    tkey = "chunk_train" if train else "chunk_bwd"  # name of its recorded traffic
    tokens = w.B * w.T
    flops = (train_flops_per_head_token if train else bwd_flops_per_head_token)(w.dk, w.dv) * w.heads * w.T
    # (a training step: both passes' bytes; the KDA forward reads log a per channel, d_k fp32)
    nbytes = bwd_bytes(w, es, kda) + ((chunk_bytes(w, es) + (w.heads * w.T * 4 * (w.dk - 1) if kda else 0))
                                      if train else 0)
    peak_mfma = PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS
    part = {"kernel": ("chunk_prep_kda_kernel + chunk_scan_kernel (KDA, saving) + chunk_rscan_kernel + "
                       "chunk_grad_kda_kernel" if train and kda else
                       "chunk_prep_kernel + chunk_scan_kernel (saving) + chunk_rscan_kernel + chunk_grad_kernel"
                       if train else
                       "chunk_prep_kda_kernel + chunk_scan_kernel (recompute) + chunk_rscan_kernel + "
                       "chunk_grad_kda_kernel" if kda else
                       "chunk_prep_kernel + chunk_scan_kernel (recompute) + chunk_rscan_kernel + chunk_grad_kernel"),
            "launches_per_step": 1, "ms_per_step": ms, "kernel_avg_us": ms * 1e3, "tokens": tokens,
            "tokens_per_s": tokens / (ms * 1e-3), "algorithmic_flop": flops, "algorithmic_bytes": nbytes,
            "mfma_tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / peak_mfma,
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "workspace_bytes": ws_bytes, "sources_sha": sources_sha(traffic_key(tkey, mode))}
    part["hbm_traffic_bytes_per_launch"] = (recorded_traffic(w.name, traffic_key(tkey, mode))
                                            if mode in ("kla", "kda") else None)
    del t, out, workspace
    if train:
        del o
    torch.cuda.empty_cache()
    return part, elapsed


def run_bwd(args, w):
    """--pass bwd: time kla_chunk_bwd (kla_gdn_chunk_bwd, kla_kda_chunk_bwd) over the workload's prefill.
    --pass train: time kla_chunk_fwd_train and kla_chunk_bwd_saved (their gdn forms) per step."""
    train = args.pass_ == "train"
    gdn = args.mode in ("gdn", "deltanet")
    kda = args.mode == "kda"
    part, elapsed = measure_bwd(w, args.mode, train, args.steps, args.warmup)
    es = 2 if w.dtype == "bf16" else 4
    peak_mfma = PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS
    tokens = w.B * w.T
    roof = {"bound": "mfma", "kernel": part["kernel"], "achieved": part["mfma_tflops"], "peak": peak_mfma,
            "unit": "TFLOP/s", "frac": part["mfma_frac"], "traffic": part["hbm_traffic_bytes_per_launch"],
            "hbm_view": {"achieved": part["hbm_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": part["hbm_frac"]}}
    result = {
        "metric": METRIC_TRAIN if train else METRIC_BWD, "value": tokens * args.steps / elapsed, "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; distributions of the workload description; do ~ N(0, 1))",
        "config": {"workload": w.name, "pass": args.pass_, "mode": args.mode, "B": w.B, "H": w.H, "T": w.T,
                   "d_k": w.dk, "d_v": w.dv, "chunk": 64, "parallelism": "single GPU"},
        "parts": {"chunk_train" if train else "chunk_bwd": part}, "roofline": roof}
    if not args.no_cpu_baseline and not gdn and not train:
        log("[bench] cpu baseline: gradient oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline_bwd(w, args.cpu_bwd_head_tokens, kda)
    print(json.dumps(result), flush=True)


# Extra workloads timed after the default step (in its JSON line, under parts["extra:<name>"]): the
# other named workloads, each in its own launch configuration, and one decode whose state exceeds
# the 256 MB last-level cache. Prefill launches follow a 512 MiB write that evicts the caches.
EXTRAS = ("fwd_b8h8_t4096", "fwd_long_t65536", "decode_b64h16", "decode_b512h16")
TRAIN_EXTRAS = (("fwd_b8h8_t4096", "kla"), ("fwd_b8h8_t4096", "kda"))
BIG_DECODE = wl.Workload("decode_b512h16", 5, B=512, H=16, dk=128, dv=128, steps=16, s0_std=0.02,
                         note="KLA decode B512 H16 d128: 512 MiB fp32 state, twice the last-level cache")
FLUSH_BYTES = 512 << 20


def workload(name):
    """A named workload, or the large-state decode (an extra, also selectable with --workload)."""
    return BIG_DECODE if name == BIG_DECODE.name else wl.WORKLOADS[name]
GEN_WORKERS = None  # --gen-workers


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def launch_floor_us(torch, device, n=512):
    """Per-launch time of n graph-replayed kernels that do almost nothing (a 64-element add): the
    floor under any one-kernel decode step on this stack."""
    z = torch.zeros(64, device=device)
    z.add_(1.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            z.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    ev = _events(torch, 3)
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return min(a.elapsed_time(b) for a, b in ev) * 1e3 / n


def prefill_part(w, ms_list, es, extra=False):
    ms = float(np.median(ms_list))
    tokens = w.B * w.T
    flops = chunk_flops_per_head_token(w.dk, w.dv) * w.heads * w.T
    nbytes = chunk_bytes(w, es)
    peak = PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS
    part = {"kernel": "chunk_prep_kernel + chunk_scan_kernel (+ seg_combine_kernel + seg_fix_kernel when the plan "
                      "segments)", "launches_per_step": 1, "ms_per_step": ms, "kernel_avg_us": ms * 1e3,
            "tokens": tokens, "tokens_per_s": tokens / (ms * 1e-3), "algorithmic_flop": flops,
            "algorithmic_bytes": nbytes, "mfma_tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / peak, "hbm_gbs": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if extra:
        part.update({"extra": True, "launches_timed": len(ms_list), "ms_min": float(min(ms_list)),
                     "timing": "median of launches each preceded by a 512 MiB write (caches cold), HIP events"})
    return part


def decode_part(w, per_ms, es, launch, extra=False, launches=None):
    nbytes = decode_bytes(w, es)
    part = {"kernel": "decode_step_kernel", "launches_per_step": w.steps, "launch": launch,
            "ms_per_step": per_ms * w.steps, "kernel_avg_us": per_ms * 1e3, "tokens": w.B * w.steps,
            "tokens_per_s": w.B / (per_ms * 1e-3), "algorithmic_bytes_per_launch": nbytes,
            "hbm_gbs": nbytes / (per_ms * 1e-3) / 1e9, "hbm_frac": nbytes / (per_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "state_bytes": w.heads * w.dk * w.dv * 4}
    if extra:
        part.update({"extra": True, "launches_timed": launches,
                     "timing": "graph-replayed consecutive steps, best of 3 replays, HIP events"})
    return part


def time_extra(name, torch, K, L, device, stream, flush):
    """Times one extra workload alone (kla mode) and returns its part."""
    w = workload(name)
    es = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = K.KLA_BF16 if w.dtype == "bf16" else K.KLA_F32
    on = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    log(f"[bench] extra {name}: generating ...")
    if w.T:
        x = wl.prefill_inputs(w, GEN_WORKERS)
        t = {n: on(x[n], tdt if n in ("q", "k", "v") else torch.float32) for n in x}
        del x
        o = torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=device)
        state = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=device)
        ws_bytes = int(L.kla_chunk_fwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv, 64, code))
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
        args = (P(t["q"]), P(t["k"]), P(t["v"]), P(t["eta"]), P(t["log_alpha"]), None, P(state), P(o),
                w.B, w.T, w.H, w.dk, w.dv, 64, ctypes.c_float(w.eps), code, P(ws), ws_bytes, sp)
        for _ in range(2):
            K.check(L.kla_chunk_fwd(*args))
        iters = 10 if w.heads * w.T <= (1 << 19) else 6
        ev = _events(torch, iters)
        for a, b in ev:
            flush.fill_(1)
            a.record(stream)
            st = L.kla_chunk_fwd(*args)
            b.record(stream)
            K.check(st)
        torch.cuda.synchronize()
        part = prefill_part(w, [a.elapsed_time(b) for a, b in ev], es, extra=True)
        part["hbm_traffic_bytes_per_launch"] = recorded_traffic(w.name, "chunk_fwd")
        part["workspace_bytes"] = ws_bytes
        del t, o, state, ws
    else:
        x = wl.decode_inputs(w, GEN_WORKERS)
        t = {n: on(x[n], tdt if n in ("q", "k", "v") else torch.float32) for n in x}
        del x
        state = t["S0"].clone()
        out = torch.empty((w.steps, w.B, w.H, w.dv), dtype=tdt, device=device)
        # 1024 steps for the named decode workload; the large-state one cycles its 16 input sets
        # through 64 steps (the state still changes every step).
        nlaunch = w.steps if w.steps >= 64 else 64
        calls = []
        for i in range(nlaunch):
            s_ = i % w.steps
            calls.append((P(t["q"][s_]), P(t["k"][s_]), P(t["v"][s_]), P(t["eta"][s_]), P(t["log_alpha"][s_]),
                          P(state), P(out[s_]), w.B, w.H, w.dk, w.dv, ctypes.c_float(w.eps), code))
        for c in calls[:2]:
            K.check(L.kla_decode_step(*c, sp))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gs = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
            for c in calls:
                K.check(L.kla_decode_step(*c, gs))
        torch.cuda.synchronize()
        g.replay()
        ev = _events(torch, 3)
        for a, b in ev:
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        per = min(a.elapsed_time(b) for a, b in ev) / nlaunch
        part = decode_part(w, per, es, "graph", extra=True, launches=nlaunch)
        part["hbm_traffic_bytes_per_launch"] = recorded_traffic(w.name, "decode")
        if w is BIG_DECODE:
            # What a plain device copy of the state (read and write once, beyond the last-level
            # cache) reaches on this device: the practical ceiling for a state read and rewritten.
            dst = torch.empty_like(state)
            dst.copy_(state)
            ev = _events(torch, 5)
            for a, b in ev:
                a.record(stream)
                dst.copy_(state)
                b.record(stream)
            torch.cuda.synchronize()
            cms = min(a.elapsed_time(b) for a, b in ev)
            cgbs = 2 * state.numel() * 4 / (cms * 1e-3) / 1e9
            part["copy_reference"] = {"bytes": 2 * state.numel() * 4, "us": cms * 1e3, "gbs": cgbs,
                                      "hbm_frac": cgbs / PEAK_HBM_GBS, "decode_frac_of_copy": part["hbm_gbs"] / cgbs}
            del dst
        del t, state, out, g
    part["sources_sha"] = sources_sha("chunk_fwd" if w.T else "decode")
    part["workload"] = w.note
    torch.cuda.empty_cache()
    return part


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed_b4h16", choices=sorted(wl.WORKLOADS) + [BIG_DECODE.name])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the chosen workload (the default run also times " + ", ".join(EXTRAS) + ")")
    ap.add_argument("--mode", default="kla", choices=("kla", "gdn", "deltanet", "kda"),
                    help="kla: Kaczmarz step from eta (the headline); gdn: beta given (kla_gdn_* entry points, "
                         "beta drawn like eta, unit-norm keys); deltanet: gdn without the gate; kda: the Kaczmarz "
                         "step with a per-channel decay (kla_kda_* entry points, log a per channel drawn like "
                         "log alpha)")
    ap.add_argument("--decode-launch", default="graph", choices=("graph", "eager"),
                    help="decode steps replayed from a HIP graph (default) or launched one call at a time")
    ap.add_argument("--cpu-head-tokens", type=int, default=1048576,
                    help="size of the oracle's bounded sample, in head-tokens")
    ap.add_argument("--pass", dest="pass_", default="fwd", choices=("fwd", "bwd", "train"),
                    help="fwd: the hot path (default); bwd: the chunkwise backward over a prefill workload; "
                         "train: a training step (training forward and the backward from its workspace)")
    ap.add_argument("--cpu-bwd-head-tokens", type=int, default=65536,
                    help="size of the gradient oracle's bounded sample, in head-tokens")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--gen-workers", type=int, default=None,
                    help="processes that draw the inputs (default: the CPUs available, up to 16); 1 draws them "
                         "in this process, as profiled runs need (a profiler's preload would open the GPU in "
                         "every worker)")
    args = ap.parse_args()
    global GEN_WORKERS
    GEN_WORKERS = args.gen_workers

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads would shard across GPUs with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_18_amd as kla  # noqa: F401  (loads the library or raises)
    from gated_delta_rule_18_amd import _lib as K

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))
        return

    if args.pass_ in ("bwd", "train"):
        w = workload("fwd_b8h8_t4096" if args.workload == "mixed_b4h16" else args.workload)
        if not w.T:
            print(f"--pass {args.pass_} needs a prefill workload", file=sys.stderr)
            sys.exit(2)
        return run_bwd(args, w.with_(steps=0))

    w = workload(args.workload)
    es = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = K.KLA_BF16 if w.dtype == "bf16" else K.KLA_F32
    L = K.lib()

    log(f"[bench] generating {w.name} ({w.note}) ...")
    t_gen = time.perf_counter()
    on = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(device)
    pre = dec = None
    gdn = args.mode in ("gdn", "deltanet")
    kda = args.mode == "kda"
    if w.T:
        x = wl.prefill_inputs(w, GEN_WORKERS)
        if gdn:
            x["k"] = unit_keys(x["k"])
        if kda:
            x["log_a"] = wl.channel_log_decay(w)
        pre = {n: on(x[n], tdt if n in ("q", "k", "v") else torch.float32) for n in x}
        del x
        pre["o"] = torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=device)
    state = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=device)
    if w.steps:
        x = wl.decode_inputs(w, GEN_WORKERS)
        if gdn:
            x["k"] = unit_keys(x["k"])
        if kda:
            x["log_a"] = wl.channel_log_decay(w, decode=True)
        dec = {n: on(x[n], tdt if n in ("q", "k", "v") else torch.float32) for n in x}
        del x
        dec["o"] = torch.empty((w.steps, w.B, w.H, w.dv), dtype=tdt, device=device)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t_gen:.1f} s)")

    stream = torch.cuda.current_stream(device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    fwd_args = None
    if pre is not None:
        ws_fn = L.kla_kda_chunk_fwd_workspace_size if kda else L.kla_chunk_fwd_workspace_size
        ws_bytes = int(ws_fn(w.B, w.T, w.H, w.dk, w.dv, 64, code))
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
        la = None if args.mode == "deltanet" else P(pre["log_a" if kda else "log_alpha"])
        if kda:
            fwd_args = (P(pre["q"]), P(pre["k"]), P(pre["v"]), P(pre["eta"]), la, None, P(state), P(pre["o"]),
                        w.B, w.T, w.H, w.dk, w.dv, 64, ctypes.c_float(w.eps), 0, code, P(workspace), ws_bytes, sp)
        elif gdn:  # beta drawn like eta
            fwd_args = (P(pre["q"]), P(pre["k"]), P(pre["v"]), P(pre["eta"]), la, None, P(state), P(pre["o"]),
                        w.B, w.T, w.H, w.dk, w.dv, 64, code, P(workspace), ws_bytes, sp)
        else:
            fwd_args = (P(pre["q"]), P(pre["k"]), P(pre["v"]), P(pre["eta"]), la, None, P(state), P(pre["o"]),
                        w.B, w.T, w.H, w.dk, w.dv, 64, ctypes.c_float(w.eps), code, P(workspace), ws_bytes, sp)
    dec_args = []
    if dec is not None:
        for s in range(w.steps):
            la = None if args.mode == "deltanet" else P(dec["log_a" if kda else "log_alpha"][s])
            tail = (code, sp) if gdn else (ctypes.c_float(w.eps), 0, code, sp) if kda else (ctypes.c_float(w.eps), code, sp)
            dec_args.append((P(dec["q"][s]), P(dec["k"][s]), P(dec["v"][s]), P(dec["eta"][s]), la, P(state),
                             P(dec["o"][s]), w.B, w.H, w.dk, w.dv) + tail)
    fwd_fn, dec_fn = ((L.kla_gdn_chunk_fwd, L.kla_gdn_decode_step) if gdn else
                      (L.kla_kda_chunk_fwd, L.kla_kda_decode_step) if kda else
                      (L.kla_chunk_fwd, L.kla_decode_step))

    if pre is None:  # decode-only workloads start from their S0 and keep decoding step after step
        state.copy_(dec["S0"])

    def run_decode(launch_stream):
        for a in dec_args:
            st = dec_fn(*a[:-1], launch_stream)
            if st:
                K.check(st)

    # The decode steps of one bench step are replayed from a HIP graph (as a serving loop
    # would issue them): one kernel per token either way, but the host's per-call cost
    # (several microseconds through ctypes) no longer paces a kernel that runs in about as long.
    dec_graph = None
    if dec_args and args.decode_launch == "graph":
        saved = state.clone()
        run_decode(sp)  # first launches outside capture (module load)
        torch.cuda.synchronize()
        dec_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dec_graph):
            run_decode(ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))
        torch.cuda.synchronize()
        state.copy_(saved)
        del saved

    def one_step(ev):
        if fwd_args is not None:
            ev["fwd"][0].record(stream)
            st = fwd_fn(*fwd_args)
            ev["fwd"][1].record(stream)
            if st:
                K.check(st)
        if dec_args:
            ev["dec"][0].record(stream)
            if dec_graph is not None:
                dec_graph.replay()
            else:
                run_decode(sp)
            ev["dec"][1].record(stream)

    def new_events():
        return {p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for p in ("fwd", "dec")}

    log(f"[bench] warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        one_step(new_events())
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} step(s)")
    evs = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed region {elapsed * 1e3:.2f} ms")

    parts = {}
    fwd_tokens = w.B * w.T
    dec_tokens = w.B * w.steps
    if fwd_args is not None:
        ms = sum(e["fwd"][0].elapsed_time(e["fwd"][1]) for e in evs) / args.steps
        part = prefill_part(w, [ms], es)
        if kda:
            part["kernel"] = "chunk_prep_kda_kernel + chunk_scan_kernel (KDA mode)"
        parts["chunk_fwd"] = part
    if dec_args:
        ms = sum(e["dec"][0].elapsed_time(e["dec"][1]) for e in evs) / args.steps
        parts["decode"] = decode_part(w, ms / w.steps, es, args.decode_launch)

    for name, part in parts.items():
        part["sources_sha"] = sources_sha(traffic_key(name, args.mode))
        part["hbm_traffic_bytes_per_launch"] = (recorded_traffic(w.name, traffic_key(name, args.mode))
                                                if args.mode in ("kla", "kda") else None)
    dom_name = max(parts, key=lambda p: parts[p]["ms_per_step"])
    dom = parts[dom_name]
    roof = {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["hbm_gbs"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": dom["hbm_frac"], "traffic": dom["hbm_traffic_bytes_per_launch"]}
    if dom_name == "chunk_fwd":
        roof["mfma_view"] = {"achieved": dom["mfma_tflops"],
                             "peak": PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS,
                             "unit": "TFLOP/s", "frac": dom["mfma_frac"]}
    else:
        # A graph-replayed kernel cannot take less than the launch floor measured here; state it
        # beside the roofline so that the fraction is read against it.
        floor = launch_floor_us(torch, device)
        roof["launch_floor_us"] = floor
        roof["kernel_avg_us"] = dom["kernel_avg_us"]
        roof["note"] = (f"{dom['kernel_avg_us']:.2f} us per launch against a {floor:.2f} us per-launch floor (512 "
                        f"graph-replayed 64-element adds); the HBM time of its algorithmic bytes is "
                        f"{dom['algorithmic_bytes_per_launch'] / PEAK_HBM_GBS / 1e3:.2f} us")

    tokens_per_step = fwd_tokens + dec_tokens
    ms_step = elapsed * 1e3 / args.steps
    result = {
        "metric": METRIC,
        "value": tokens_per_step * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; distributions of the workload description)",
        "config": {"workload": w.name, "mode": args.mode, "B": w.B, "H": w.H, "T": w.T, "decode_steps": w.steps,
                   "d_k": w.dk, "d_v": w.dv, "chunk": 64, "parallelism": "single GPU"},
        "parts": parts,
        "roofline": roof,
    }

    # The other workloads, each alone (the default run only; they are not part of `value`).
    if not args.no_extras and args.mode == "kla" and args.workload == "mixed_b4h16":
        del pre, dec, workspace, dec_graph
        torch.cuda.empty_cache()
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=device)
        for name in EXTRAS:
            parts["extra:" + name] = time_extra(name, torch, K, L, device, stream, flush)
        del flush
        torch.cuda.empty_cache()
        # Training steps (the forward into the backward's workspace, then the backward from it),
        # scalar gate and per-channel decay, on the B8 H8 T4096 shape.
        for wname, mode in TRAIN_EXTRAS:
            tw = wl.WORKLOADS[wname]
            log(f"[bench] extra training step {wname} ({mode})")
            part, _ = measure_bwd(tw, mode, True, 10, 2)
            part.update({"extra": True, "launches_timed": 10, "timing": "mean of 10 steps after 2, HIP events",
                         "workload": tw.note + (" with per-channel decay (KDA)" if mode == "kda" else "") +
                         ": training step, kla_" + ("kda_" if mode == "kda" else "") + "chunk_fwd_train + kla_" +
                         ("kda_" if mode == "kda" else "") + "chunk_bwd_saved"})
            parts["extra:train_" + wname + ("_kda" if mode == "kda" else "")] = part

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on a bounded sample ({args.cpu_head_tokens} head-tokens)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_head_tokens, args.mode)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
