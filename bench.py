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
JSON line.

Inputs are generated (seeded) and copied to HBM before the timed region. Kernels
are launched through the C ABI with pre-marshalled pointers on torch's current
stream; the decode steps of a bench step are replayed from a HIP graph captured
once before timing (--decode-launch eager issues them one call at a time). HIP
events on that stream time each part. Prints one JSON line.
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


def bwd_bytes(w, es):
    """Algorithmic HBM bytes of one backward launch: q, k, v, do, eta, log_alpha read once;
    dq, dk, dv, deta, dlog_alpha written once (no initial state, no state cotangent)."""
    return w.heads * w.T * ((3 * w.dk + 3 * w.dv) * es + 16)


def decode_bytes(w, es):
    """Algorithmic HBM bytes of one decode launch: the fp32 state read and written once,
    q, k, v, o, eta, log_alpha."""
    return w.heads * (2 * w.dk * w.dv * 4 + (2 * w.dk + 2 * w.dv) * es + 8)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source files of each timed part; the recorded HBM traffic of a part is only reported while
# these files are byte-identical to the ones the counters were taken on.
CSRC = os.path.join(ROOT, "gated_delta_rule_18_amd", "csrc")
PART_SOURCES = {
    "chunk_fwd": ["chunk_common.h", "chunk_prep.hip", "chunk_scan.hip", "chunk_seg.hip", "tile_ops.h",
                  "kla_device.h", "kla_launch.h"],
    "decode": ["decode.hip", "kla_device.h", "kla_launch.h"],
    "chunk_bwd": ["chunk_common.h", "chunk_prep.hip", "chunk_scan.hip", "chunk_bwd_scan.hip", "chunk_bwd_grad.hip",
                  "tile_ops.h", "kla_device.h", "kla_launch.h"],
}
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


def recorded_traffic(workload, part):
    """HBM bytes per launch of `part` on `workload`, from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs recorded in profiles/hbm_traffic.txt (each already scaled by the copy calibration),
    or None if there is no record for the current sources."""
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


def cpu_baseline(w, head_tokens, mode="kla"):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload: every head
    of the batch over the first head_tokens / (B H) prefill tokens (or decode steps). Single
    threaded; the recurrence costs the same per token at any position."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    n = max(1, min(head_tokens // w.heads, w.T if w.T else w.steps))
    if w.T and mode == "kda":
        x = wl.prefill_inputs(w.with_(T=n))
        la = wl.channel_log_decay(w.with_(T=n))
        args = (x["q"], x["k"], x["v"], x["eta"], la, w.eps)
        run = lambda: oracle.kda_forward(*args)
        what = f"oracle kda_forward on all {w.heads} heads (B={w.B}, H={w.H}) of the first {n} prefill tokens"
    elif w.T and mode != "kla":
        x = wl.prefill_inputs(w.with_(T=n))
        heads = lambda a: np.moveaxis(a, 2, 1).reshape(w.heads, n, *a.shape[3:])  # [B, T, H, ...] -> [BH, T, ...]
        la = x["log_alpha"] if mode == "gdn" else np.zeros_like(x["log_alpha"])
        args = (heads(x["q"]), heads(unit_keys(x["k"])), heads(x["v"]), heads(x["eta"]), heads(la))
        run = lambda: oracle.gated_delta_recurrent(*args)
        what = (f"oracle gated_delta_recurrent ({mode}) on all {w.heads} heads (B={w.B}, H={w.H}) of the first "
                f"{n} prefill tokens")
    elif w.T:
        x = wl.prefill_inputs(w.with_(T=n))
        args = (x["q"], x["k"], x["v"], x["eta"], x["log_alpha"], w.eps)
        run = lambda: oracle.kla_forward(*args)
        what = f"oracle kla_forward on all {w.heads} heads (B={w.B}, H={w.H}) of the first {n} prefill tokens"
    else:
        x = wl.decode_inputs(w.with_(steps=n))
        args = (x["q"], x["k"], x["v"], x["eta"], x["log_alpha"], w.eps, x["S0"])
        run = lambda: oracle.kla_decode_steps(*args)
        what = f"oracle decode on all {w.heads} heads (B={w.B}, H={w.H}) for the first {n} steps"
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    if ctx:
        with ctx:
            run()
    else:
        run()
    dt = time.perf_counter() - t0
    tokens = w.B * n
    return {"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}: {tokens} tokens in {dt:.2f} s (fp64 numpy, one thread)"}


def cpu_baseline_bwd(w, head_tokens):
    """The fp64 gradient oracle (autodiff of the token loop), as it stands, on a bounded sample:
    the first 8 heads (or all, if fewer) over the first head_tokens / 8 prefill tokens."""
    import oracle
    import torch
    torch.set_num_threads(1)
    nh = min(8, w.heads)
    n = max(1, min(head_tokens // nh, w.T))
    sub = w.with_(T=n)
    x = wl.prefill_inputs(sub)
    g = wl.grad_inputs(sub)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:nh]
    sel = lambda a: np.stack([a[b, :, h] for b, h in heads])
    args = (sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["eta"]), sel(x["log_alpha"]), w.eps, None, sel(g["do"]))
    t0 = time.perf_counter()
    oracle.kla_vjp(*args)
    dt = time.perf_counter() - t0
    return {"value": nh * n / dt / w.H, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle kla_vjp (fp64 autodiff of the token loop, one thread) on {nh} heads x the first {n} "
                      f"prefill tokens: {nh * n} head-tokens in {dt:.2f} s, reported per token of all {w.H} heads"}


def run_bwd(args, w):
    """--pass bwd: time kla_chunk_bwd (or kla_gdn_chunk_bwd) over the workload's prefill."""
    import torch
    from gated_delta_rule_18_amd import _lib as K
    device = torch.device("cuda:0")
    es = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = K.KLA_BF16 if w.dtype == "bf16" else K.KLA_F32
    L = K.lib()
    gdn = args.mode != "kla"
    log(f"[bench] generating {w.name} ({w.note}) and its output cotangent ...")
    on = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(device)
    x = wl.prefill_inputs(w)
    if gdn:
        x["k"] = unit_keys(x["k"])
    x["do"] = wl.grad_inputs(w)["do"]
    t = {n: on(x[n], tdt if n in ("q", "k", "v", "do") else torch.float32) for n in x}
    del x
    out = {"dq": torch.empty_like(t["q"]), "dk": torch.empty_like(t["k"]), "dv": torch.empty_like(t["v"]),
           "deta": torch.empty_like(t["eta"]), "dla": torch.empty_like(t["log_alpha"])}
    ws_bytes = int(L.kla_chunk_bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv, 64, code))
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())
    la = None if args.mode == "deltanet" else P(t["log_alpha"])
    dla = None if args.mode == "deltanet" else P(out["dla"])
    head = (P(t["q"]), P(t["k"]), P(t["v"]), P(t["eta"]), la, None, P(t["do"]), None, P(out["dq"]), P(out["dk"]),
            P(out["dv"]), P(out["deta"]), dla, None, w.B, w.T, w.H, w.dk, w.dv, 64)
    if gdn:
        call = lambda: L.kla_gdn_chunk_bwd(*head, code, P(workspace), ws_bytes, sp)
    else:
        call = lambda: L.kla_chunk_bwd(*head, ctypes.c_float(w.eps), code, P(workspace), ws_bytes, sp)
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    log(f"[bench] warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        K.check(call())
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} step(s)")
    evs = [ev() for _ in range(args.steps)]
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
    ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    tokens = w.B * w.T
    flops = bwd_flops_per_head_token(w.dk, w.dv) * w.heads * w.T
    nbytes = bwd_bytes(w, es)
    peak_mfma = PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS
    part = {"kernel": "chunk_prep_kernel + chunk_scan_kernel (recompute) + chunk_rscan_kernel + chunk_grad_kernel",
            "launches_per_step": 1, "ms_per_step": ms, "kernel_avg_us": ms * 1e3, "tokens": tokens,
            "tokens_per_s": tokens / (ms * 1e-3), "algorithmic_flop": flops, "algorithmic_bytes": nbytes,
            "mfma_tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / peak_mfma,
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "workspace_bytes": ws_bytes, "sources_sha": sources_sha("chunk_bwd")}
    part["hbm_traffic_bytes_per_launch"] = recorded_traffic(w.name, "chunk_bwd") if args.mode == "kla" else None
    roof = {"bound": "mfma", "kernel": part["kernel"], "achieved": part["mfma_tflops"], "peak": peak_mfma,
            "unit": "TFLOP/s", "frac": part["mfma_frac"], "traffic": part["hbm_traffic_bytes_per_launch"],
            "hbm_view": {"achieved": part["hbm_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": part["hbm_frac"]}}
    result = {
        "metric": METRIC_BWD, "value": tokens * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; distributions of the workload description; do ~ N(0, 1))",
        "config": {"workload": w.name, "pass": "bwd", "mode": args.mode, "B": w.B, "H": w.H, "T": w.T,
                   "d_k": w.dk, "d_v": w.dv, "chunk": 64, "parallelism": "single GPU"},
        "parts": {"chunk_bwd": part}, "roofline": roof}
    if not args.no_cpu_baseline and not gdn:
        log("[bench] cpu baseline: gradient oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline_bwd(w, args.cpu_bwd_head_tokens)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed_b4h16", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="kla", choices=("kla", "gdn", "deltanet", "kda"),
                    help="kla: Kaczmarz step from eta (the headline); gdn: beta given (kla_gdn_* entry points, "
                         "beta drawn like eta, unit-norm keys); deltanet: gdn without the gate; kda: the Kaczmarz "
                         "step with a per-channel decay (kla_kda_* entry points, log a per channel drawn like "
                         "log alpha)")
    ap.add_argument("--decode-launch", default="graph", choices=("graph", "eager"),
                    help="decode steps replayed from a HIP graph (default) or launched one call at a time")
    ap.add_argument("--cpu-head-tokens", type=int, default=1048576,
                    help="size of the oracle's bounded sample, in head-tokens")
    ap.add_argument("--pass", dest="pass_", default="fwd", choices=("fwd", "bwd"),
                    help="fwd: the hot path (default); bwd: the chunkwise backward over a prefill workload")
    ap.add_argument("--cpu-bwd-head-tokens", type=int, default=8192,
                    help="size of the gradient oracle's bounded sample, in head-tokens")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads would shard across GPUs with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_18_amd as kla
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

    if args.pass_ == "bwd":
        w = wl.WORKLOADS["fwd_b8h8_t4096" if args.workload == "mixed_b4h16" else args.workload]
        if not w.T:
            print("--pass bwd needs a prefill workload", file=sys.stderr)
            sys.exit(2)
        return run_bwd(args, w.with_(steps=0))

    w = wl.WORKLOADS[args.workload]
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
        x = wl.prefill_inputs(w)
        if gdn:
            x["k"] = unit_keys(x["k"])
        if kda:
            x["log_a"] = wl.channel_log_decay(w)
        pre = {n: on(x[n], tdt if n in ("q", "k", "v") else torch.float32) for n in x}
        del x
        pre["o"] = torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=device)
    state = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=device)
    if w.steps:
        x = wl.decode_inputs(w)
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
        flops = chunk_flops_per_head_token(w.dk, w.dv) * w.heads * w.T
        nbytes = chunk_bytes(w, es)
        segs = 1 if w.heads * (w.dv // (32 if es == 2 else 64)) >= 256 or w.T < 32 * 64 else None
        parts["chunk_fwd"] = {
            "kernel": "chunk_prep_kda_kernel + chunk_scan_kernel (KDA mode)" if args.mode == "kda" else
                      "chunk_prep_kernel + chunk_scan_kernel" + (
                          "" if segs == 1 else " (+ seg_combine_kernel + seg_fix_kernel when the plan segments)"),
            "launches_per_step": 1, "ms_per_step": ms,
            "kernel_avg_us": ms * 1e3, "tokens": fwd_tokens, "tokens_per_s": fwd_tokens / (ms * 1e-3),
            "algorithmic_flop": flops, "algorithmic_bytes": nbytes,
            "mfma_tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / (PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS),
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if dec_args:
        ms = sum(e["dec"][0].elapsed_time(e["dec"][1]) for e in evs) / args.steps
        per = ms / w.steps
        nbytes = decode_bytes(w, es)
        parts["decode"] = {
            "kernel": "decode_step_kernel", "launches_per_step": w.steps, "launch": args.decode_launch,
            "ms_per_step": ms,
            "kernel_avg_us": per * 1e3, "tokens": dec_tokens, "tokens_per_s": dec_tokens / (ms * 1e-3),
            "algorithmic_bytes_per_launch": nbytes,
            "hbm_gbs": nbytes / (per * 1e-3) / 1e9, "hbm_frac": nbytes / (per * 1e-3) / 1e9 / PEAK_HBM_GBS}

    for name, part in parts.items():
        part["sources_sha"] = sources_sha(name)
        part["hbm_traffic_bytes_per_launch"] = recorded_traffic(w.name, name) if args.mode == "kla" else None
    dom_name = max(parts, key=lambda p: parts[p]["ms_per_step"])
    dom = parts[dom_name]
    roof = {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["hbm_gbs"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": dom["hbm_frac"], "traffic": dom["hbm_traffic_bytes_per_launch"]}
    if dom_name == "chunk_fwd":
        roof["mfma_view"] = {"achieved": dom["mfma_tflops"],
                             "peak": PEAK_BF16_TFLOPS if es == 2 else PEAK_FP32_MFMA_TFLOPS,
                             "unit": "TFLOP/s", "frac": dom["mfma_frac"]}

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
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on a bounded sample ({args.cpu_head_tokens} head-tokens)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_head_tokens, args.mode)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
