"""The full-size parity checker itself (CPU only): exact results pass, and a wrong head or a few
wrong tokens are caught by the per-head and per-chunk bars even where the whole-tensor error
stays under the bar."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pool as op


def _exact(w):
    x = wl.prefill_inputs(w)
    o, S = oracle.kla_forward(x["q"], x["k"], x["v"], x["eta"], x["log_alpha"], w.eps)
    return o.astype(np.float32), S.astype(np.float32)


def _got(o, S):
    return lambda g: {"o": np.stack([o[b, :, h] for b, h in g]), "S": np.stack([S[b, h] for b, h in g])}


def test_exact_results_pass():
    w = wl.custom("pool", 600, B=2, H=3, dk=16, dv=16, T=150, dtype="f32")
    o, S = _exact(w)
    merged, heads = op.run("forward", w, _got(o, S))
    errs = op.check("exact", merged, heads, 1e-6)
    assert set(errs) == {"o", "S_T"}
    assert merged["o"][0].shape == (6, 3)  # 6 heads x 3 chunks (the last one ragged)


def test_wrong_tokens_are_caught_per_chunk():
    w = wl.custom("pool_bad", 601, B=2, H=4, dk=16, dv=16, T=640, dtype="f32")
    o, S = _exact(w)
    bad = o.copy()
    bad[1, 300:302, 2] *= 1.5  # two tokens of one head
    merged, heads = op.run("forward", w, _got(bad, S))
    whole, head, block, where = op.errors(merged)["o"]
    assert whole < 2e-2 and block > 2e-2
    assert heads[where[0]] == (1, 2) and where[1] == 300 // 64
    with pytest.raises(AssertionError):
        op.check("planted", merged, heads, 2e-2)


def test_decode_and_backward_jobs_run_on_exact_results():
    w = wl.custom("pool_dec", 602, B=2, H=2, dk=16, dv=16, steps=70, dtype="f32", s0_std=0.05)
    d = wl.decode_inputs(w)
    o, S = oracle.kla_decode_steps(d["q"], d["k"], d["v"], d["eta"], d["log_alpha"], w.eps, d["S0"])
    got = lambda g: {"od": np.stack([o[:, b, h] for b, h in g]), "S": np.stack([S[b, h] for b, h in g])}
    merged, heads = op.run("decode", w, got)
    op.check("decode exact", merged, heads, 1e-9)
    wb = wl.custom("pool_bwd", 603, B=1, H=3, dk=8, dv=8, T=100, dtype="f32")
    x, gr = wl.prefill_inputs(wb), wl.grad_inputs(wb, 0.1, 0.5)
    ref = oracle.kla_backward(x["q"], x["k"], x["v"], x["eta"], x["log_alpha"], wb.eps, gr["S0"], gr["do"], gr["dST"])
    got = lambda g: {**{n: np.stack([ref[n][b, :, h] for b, h in g]) for n in ("dq", "dk", "dv", "deta", "dlog_alpha")},
                     "dS0": np.stack([ref["dS0"][b, h] for b, h in g])}
    merged, heads = op.run("backward", wb, got, (0.1, 0.5))
    op.check("backward exact", merged, heads, 1e-9)
