"""GPU parity of the segment scan of the chunkwise forward (segments scanned at once, a
sequential combine of their end states, and an output correction) against the fp64 oracle.
The segment count is forced through kla_chunk_fwd_seg; kla_chunk_fwd segments only when few
heads would leave compute units idle (the B1 H16 T65536 workload is such a case and is covered
by the workload test in test_gpu_parity.py)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.kla_testutil import TOL, dev, host, rel_l2, report

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gated_delta_rule_18_amd as kla  # noqa: E402


def run_and_compare(name, w, S0, nseg, tol=None):
    tol = TOL[w.dtype] if tol is None else tol
    inp = wl.prefill_inputs(w)
    o, S = kla.kla_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                             dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps,
                             state_in=None if S0 is None else dev(S0), segments=nseg)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    sel = lambda x: np.stack([x[b, :, h] for b, h in heads])
    s0 = None if S0 is None else np.stack([S0[b, h] for b, h in heads])
    ro, rS = oracle.kla_recurrent(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["eta"]),
                                  sel(inp["log_alpha"]), w.eps, s0)
    eo = rel_l2(sel(host(o)), ro)
    eS = rel_l2(np.stack([host(S)[b, h] for b, h in heads]), rS)
    report(name, o=eo, S_T=eS)
    assert np.isfinite(host(o)).all()
    assert eo <= tol and eS <= tol, (eo, eS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nseg,T", [(2, 640), (3, 650), (5, 1000), (4, 300)])
def test_segment_scan(dtype, nseg, T):
    w = wl.custom("seg", 400 + nseg, B=1, H=3, dk=128, dv=128, T=T, dtype=dtype)
    S0 = np.random.default_rng(nseg).normal(0, 0.05, (1, 3, 128, 128)).astype(np.float32)
    run_and_compare(f"segments={nseg} {dtype} T={T}", w, S0, nseg)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_segment_scan_head_sizes(dtype, dk, dv):
    w = wl.custom("seg_hs", 410, B=2, H=1, dk=dk, dv=dv, T=777, dtype=dtype)
    run_and_compare(f"segments=3 {dtype} dk={dk} dv={dv}", w, None, 3)


def test_segment_scan_mixed_gates():
    """The mixed workload's gates (near-0/1 eta, log alpha in [-0.2, 0]) across segment borders."""
    w = wl.WORKLOADS["mixed_b4h16"].with_(B=1, H=2, T=2048, steps=0, wid=411)
    run_and_compare("segments=4 mixed gates", w, None, 4)


def test_segment_count_does_not_change_the_result_beyond_rounding():
    """One segment against several on the same inputs (the plan is a pure reassociation)."""
    w = wl.custom("seg_vs_one", 412, B=1, H=2, dk=128, dv=128, T=1500)
    inp = wl.prefill_inputs(w)
    args = (dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["eta"]),
            dev(inp["log_alpha"]))
    o1, S1 = kla.kla_chunk_fwd(*args, eps=w.eps, segments=1)
    o6, S6 = kla.kla_chunk_fwd(*args, eps=w.eps, segments=6)
    torch.cuda.synchronize()
    eo, eS = rel_l2(host(o6), host(o1)), rel_l2(host(S6), host(S1))
    report("segments 6 vs 1", o=eo, S_T=eS)
    assert eo <= 1e-2 and eS <= 1e-2
