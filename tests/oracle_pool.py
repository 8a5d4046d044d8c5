"""Full-size parity: the fp64 oracle over every head of a workload, in worker processes.

Test infrastructure. The parent hands each worker a group of heads together with the library's
results for those heads (fp32 arrays). The worker regenerates the heads' inputs from their own
seeded streams (workloads.py), runs the oracle, and returns, for every output, the squared error
and the squared reference per head and per 64-token chunk (per 64 steps for decode). The parent
forms three relative L2 errors from those sums and checks each against the bar:
  * over the whole tensor,
  * per head (the worst head),
  * per head and chunk (the worst 64-token chunk of any head),
so that a wrong head, or a few wrong tokens, cannot hide in the whole-tensor figure.
"""
from __future__ import annotations

import concurrent.futures
import multiprocessing
import os

import numpy as np

import oracle
import workloads as wl

CHUNK = 64


def n_workers() -> int:
    """Worker processes: the CPUs this process may run on, at most 16."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _chunk_sums(x, ref):
    """x, ref [n, L, ...] -> (sum of squared error, sum of squared ref) per head and 64-row block
    along L, each [n, ceil(L / 64)]."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n, L = ref.shape[:2]
    e = ((x - ref) ** 2).reshape(n, L, -1).sum(-1)
    r = (ref ** 2).reshape(n, L, -1).sum(-1)
    nc = (L + CHUNK - 1) // CHUNK
    pad = nc * CHUNK - L
    e = np.pad(e, ((0, 0), (0, pad))).reshape(n, nc, CHUNK).sum(-1)
    r = np.pad(r, ((0, 0), (0, pad))).reshape(n, nc, CHUNK).sum(-1)
    return e, r, bool(np.isfinite(x).all())


def _state_sums(x, ref):
    """x, ref [n, dk, dv] -> per-head sums [n, 1]."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return (((x - ref) ** 2).sum((1, 2))[:, None], (ref ** 2).sum((1, 2))[:, None], bool(np.isfinite(x).all()))


def _stack(dicts, key):
    return np.stack([d[key] for d in dicts])


def _job_forward(w, heads, got, kind="kla"):
    """Prefill from a zero state (and, for a workload with decode steps, the steps continuing from
    its final state) of `heads`, oracle against `got`: o [n, T, dv], optionally od [n, steps, dv],
    S [n, dk, dv]. kind "kla" (scalar gate) or "kda" (per-channel decay, Kaczmarz step)."""
    pre = [wl.head_prefill(w, b, h) for b, h in heads]
    q, k, v, eta = (_stack(pre, n) for n in ("q", "k", "v", "eta"))
    if kind == "kda":
        la = np.stack([wl.head_channel_log_decay(w, b, h) for b, h in heads])
    else:
        la = _stack(pre, "log_alpha")
    if w.steps:  # one uninterrupted recurrence over the prefill and the decode steps
        dec = [wl.head_decode(w, b, h) for b, h in heads]
        q, k, v, eta, la = (np.concatenate([a, _stack(dec, n)], 1)
                            for a, n in ((q, "q"), (k, "k"), (v, "v"), (eta, "eta"), (la, "log_alpha")))
    if kind == "kda":
        o, S = oracle.kda_recurrent(q, k, v, oracle.kaczmarz_step_size(k, eta, w.eps), la)
    else:
        o, S = oracle.kla_recurrent(q, k, v, eta, la, w.eps)
    out = {"o": _chunk_sums(got["o"], o[:, :w.T])}
    if w.steps:
        out["decode_o"] = _chunk_sums(got["od"], o[:, w.T:])
    if "S" in got:
        out["S_T"] = _state_sums(got["S"], S)
    return out


def _job_decode(w, heads, got):
    """Decode steps from the workload's S0 for `heads`: od [n, steps, dv], S [n, dk, dv]."""
    dec = [wl.head_decode(w, b, h) for b, h in heads]
    o, S = oracle.kla_recurrent(*(_stack(dec, n) for n in ("q", "k", "v", "eta", "log_alpha")), w.eps,
                                _stack(dec, "S0"))
    return {"decode_o": _chunk_sums(got["od"], o), "S": _state_sums(got["S"], S)}


def _job_backward(w, heads, got, s0_std, dst_std):
    """Gradients of `heads` (KLA step): dq, dk, dv [n, T, d], deta, dlog_alpha [n, T], dS0."""
    pre = [wl.head_prefill(w, b, h) for b, h in heads]
    gr = [wl.head_grad(w, b, h, s0_std, dst_std) for b, h in heads]
    S0 = _stack(gr, "S0") if s0_std > 0 else None
    dST = _stack(gr, "dST") if dst_std > 0 else None
    g = oracle.kla_adjoint(*(_stack(pre, n) for n in ("q", "k", "v", "eta", "log_alpha")), w.eps, S0,
                           _stack(gr, "do"), dST)
    out = {n: _chunk_sums(got[n], g[n]) for n in ("dq", "dk", "dv", "deta", "dlog_alpha")}
    out["dS0"] = _state_sums(got["dS0"], g["dS0"])
    return out


def _job_kda_backward(w, heads, got, s0_std, dst_std):
    """Gradients of `heads` with the per-channel decay (Kaczmarz step): dq, dk, dv, deta [n, T, ...],
    dlog_a [n, T, d_k], dS0."""
    pre = [wl.head_prefill(w, b, h) for b, h in heads]
    gr = [wl.head_grad(w, b, h, s0_std, dst_std) for b, h in heads]
    la = np.stack([wl.head_channel_log_decay(w, b, h) for b, h in heads])
    S0 = _stack(gr, "S0") if s0_std > 0 else None
    dST = _stack(gr, "dST") if dst_std > 0 else None
    g = oracle.kda_adjoint(*(_stack(pre, n) for n in ("q", "k", "v", "eta")), la, w.eps, S0, _stack(gr, "do"), dST)
    out = {n: _chunk_sums(got[n], g[n]) for n in ("dq", "dk", "dv", "deta", "dlog_a")}
    out["dS0"] = _state_sums(got["dS0"], g["dS0"])
    return out


_JOBS = {"forward": _job_forward, "decode": _job_decode, "backward": _job_backward,
         "kda_backward": _job_kda_backward}


def run(job, w, got_for, extra=(), heads=None):
    """Runs `job` over every head of `w` (or `heads`) in worker processes. got_for(list of heads)
    returns the library's results of those heads (dict of arrays, head first). Returns the merged
    sums: {output: (err [n_heads, n_blocks], ref [n_heads, n_blocks], finite)} in head order."""
    heads = [(b, h) for b in range(w.B) for h in range(w.H)] if heads is None else list(heads)
    nw = n_workers()
    groups = [heads[i::nw] for i in range(nw) if heads[i::nw]]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(len(groups), mp_context=ctx, initializer=_init_worker) as ex:
        futs = [ex.submit(_JOBS[job], w, g, got_for(g), *extra) for g in groups]
        parts = [f.result() for f in futs]
    order = [hd for g in groups for hd in g]
    perm = np.argsort([heads.index(hd) for hd in order])
    merged = {}
    for name in parts[0]:
        e = np.concatenate([p[name][0] for p in parts])[perm]
        r = np.concatenate([p[name][1] for p in parts])[perm]
        merged[name] = (e, r, all(p[name][2] for p in parts))
    return merged, heads


def errors(merged):
    """{output: (whole-tensor, worst head, worst block, (head index, block index) of the worst block)}."""
    out = {}
    for name, (e, r, _) in merged.items():
        whole = float(np.sqrt(e.sum() / max(r.sum(), 1e-300)))
        per_head = np.sqrt(e.sum(1) / np.maximum(r.sum(1), 1e-300))
        per_block = np.sqrt(e / np.maximum(r, 1e-300))
        worst = np.unravel_index(int(np.argmax(per_block)), per_block.shape)
        out[name] = (whole, float(per_head.max()), float(per_block.max()), tuple(int(i) for i in worst))
    return out


def check(label, merged, heads, tol, block_tol=None):
    """Asserts every output finite and its whole-tensor, per-head and per-block relative L2 errors
    within `tol` (`block_tol` for the per-block figure if given); prints all three."""
    errs = errors(merged)
    for name, (whole, head, block, (hi, ci)) in errs.items():
        print(f"[parity] {label} {name}: whole={whole:.3e} worst_head={head:.3e} worst_chunk={block:.3e} "
              f"(head {heads[hi]}, chunk {ci}) over {len(heads)} heads", flush=True)
    bad = {}
    for name, (whole, head, block, _) in errs.items():
        if not merged[name][2]:
            bad[name] = "non-finite"
        elif not (whole <= tol and head <= tol and block <= (tol if block_tol is None else block_tol)):
            bad[name] = errs[name][:3]
    assert not bad, bad
    return errs
