"""kla_chunk_fwd_noalloc: the chunkwise forward whose workspace is the library's static scratch
(for callers that cannot allocate). Its results must be kla_chunk_fwd's, bit for bit, on calls in
a row that reuse the scratch (the second one smaller), and both must meet the oracle's bar."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as wl
from gated_delta_rule_18_amd import _lib as K
from tests.kla_testutil import TOL, dev, host, rel_l2, report

SCRATCH = 128 << 20


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """A size whose workspace exceeds the static scratch is refused before anything is enqueued
    (host-only: no device is touched), with both sizes in the message."""
    A = 1 << 20
    p = lambda x: ctypes.c_void_p(x)
    B, T, H = 8, 8192, 8  # 8192 chunks of ~17 KiB: ~139 MiB
    assert K.lib().kla_chunk_fwd_workspace_size(B, T, H, 128, 128, 64, K.KLA_BF16) > SCRATCH
    st = K.lib().kla_chunk_fwd_noalloc(p(A), p(A * 2), p(A * 3), p(A * 4), p(A * 5), None, None, p(A * 6),
                                       B, T, H, 128, 128, 64, 1e-6, K.KLA_BF16, None)
    assert st == K.KLA_ERR_NOT_SUPPORTED
    assert b"static scratch" in K.lib().kla_last_error()


@pytest.mark.gpu
def test_noalloc_matches_kla_chunk_fwd_on_consecutive_calls():
    import torch
    import gated_delta_rule_18_amd as kla
    # Two calls in a row on the shared scratch, the second smaller; the first fills most of the
    # scratch (B8 H8 T4096: 4096 chunks, ~68 MiB), the second reads only what it wrote itself.
    cases = [wl.WORKLOADS["fwd_b8h8_t4096"].with_(name="noalloc_big", wid=700),
             wl.custom("noalloc_small", 701, B=2, H=3, dk=128, dv=128, T=250)]
    for w in cases:
        need = kla.kla_chunk_fwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv)
        assert 0 < need <= SCRATCH
        inp = wl.prefill_inputs(w)
        args = (dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype), dev(inp["eta"]),
                dev(inp["log_alpha"]))
        o_ref, S_ref = kla.kla_chunk_fwd(*args, eps=w.eps)
        o = torch.full_like(o_ref, float("nan"))
        S = torch.full_like(S_ref, float("nan"))
        kla.kla_chunk_fwd_noalloc(*args, o=o, eps=w.eps, state_out=S)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), w.name
        heads = [(0, 0), (w.B - 1, w.H - 1)]
        sel = lambda x: np.stack([x[b, :, h] for b, h in heads])
        ro, rS = oracle.kla_recurrent(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["eta"]),
                                      sel(inp["log_alpha"]), w.eps)
        eo = rel_l2(sel(host(o)), ro)
        eS = rel_l2(np.stack([host(S)[b, h] for b, h in heads]), rS)
        report(f"noalloc {w.name}", o=eo, S_T=eS)
        assert eo <= TOL[w.dtype] and eS <= TOL[w.dtype]
