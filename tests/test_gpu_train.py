"""GPU parity of the training pair: kla_chunk_fwd_train (the forward that leaves the backward's
workspace filled) and kla_chunk_bwd_saved (the backward from it, without recomputing the
forward), their beta-given forms and the per-channel decay's pair (kla_kda_chunk_fwd_train,
kla_kda_chunk_bwd_saved). Outputs against kla_chunk_fwd (bit for bit where both run
the same arithmetic) and the fp64 oracle; gradients against the fp64 gradient oracle with the
backward's bars (relative L2 <= 1e-4 fp32, <= 2e-2 bf16) and against kla_chunk_bwd."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pool as op
from tests.kla_testutil import TOL, dev, heads_of, host, rel_l2, report, states_of
from tests import test_gpu_kda_bwd as kb
from tests.test_gpu_bwd import NAMES, _sel, _unit_keys, all_heads, compare, gpu_bwd, oracle_bwd

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gated_delta_rule_18_amd as kla  # noqa: E402


def train_pair(w, inp, g, beta=None, la_given=True, dos=None):
    """kla_chunk_fwd_train, then kla_chunk_bwd_saved once per cotangent in `dos` (default: g's).
    Returns (o, S_T, [gradients per cotangent]) on the host as fp64."""
    q, k, v = dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype)
    s0 = None if g["S0"] is None else dev(g["S0"])
    dst = None if g["dST"] is None else dev(g["dST"])
    la = dev(inp["log_alpha"]) if la_given else None
    if beta is None:
        o, S, ws = kla.kla_chunk_fwd_train(q, k, v, dev(inp["eta"]), la, eps=w.eps, state_in=s0)
    else:
        o, S, ws = kla.kla_gdn_chunk_fwd_train(q, k, v, dev(beta), la, state_in=s0)
    grads = []
    for do_np in (dos if dos is not None else [g["do"]]):
        do = dev(do_np, w.dtype)
        if beta is None:
            out = kla.kla_chunk_bwd_saved(q, k, v, dev(inp["eta"]), la, do, ws, eps=w.eps, state_in=s0,
                                          dstate_out=dst)
            gate = out["deta"]
        else:
            out = kla.kla_gdn_chunk_bwd_saved(q, k, v, dev(beta), la, do, ws, state_in=s0, dstate_out=dst)
            gate = out["dbeta"]
        torch.cuda.synchronize()
        r = {"dq": host(out["dq"]), "dk": host(out["dk"]), "dv": host(out["dv"]), "deta": host(gate),
             "dS0": host(out["dstate_in"])}
        r["dlog_alpha"] = None if out["dlog_alpha"] is None else host(out["dlog_alpha"])
        grads.append(r)
    return host(o), host(S), grads


@pytest.mark.parametrize("dtype,dk,dv,T", [
    ("bf16", 128, 128, 250), ("bf16", 64, 64, 131), ("bf16", 128, 64, 64), ("bf16", 64, 128, 1),
    ("f32", 64, 64, 77), ("f32", 128, 128, 100),
])
def test_train_pair_shapes(dtype, dk, dv, T):
    """The training forward's outputs are kla_chunk_fwd's bit for bit (the same arithmetic, with
    stores added); the gradients from its workspace meet the oracle's bars, and in fp32, where the
    saved states are formed exactly as the backward's recompute forms them, equal kla_chunk_bwd's."""
    w = wl.custom("train", 400 + T, B=2, H=2, dk=dk, dv=dv, T=T, dtype=dtype)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    o, S, (got,) = train_pair(w, inp, g)
    of, Sf = kla.kla_chunk_fwd(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype), dev(inp["eta"]),
                               dev(inp["log_alpha"]), eps=w.eps, state_in=dev(g["S0"]))
    torch.cuda.synchronize()
    assert np.array_equal(o, host(of)) and np.array_equal(S, host(Sf))
    heads = all_heads(w)
    compare(f"train pair {dtype} dk={dk} dv={dv} T={T}", w, got, oracle_bwd(w, inp, g, heads), heads)
    ref = gpu_bwd(w, inp, g)
    errs = {n: rel_l2(got[n], ref[n]) for n in NAMES}
    report(f"train pair vs kla_chunk_bwd {dtype} dk={dk} dv={dv} T={T}", **errs)
    if dtype == "f32":
        for n in NAMES:
            assert np.array_equal(got[n], ref[n]), n
    else:  # both within the bf16 bar of the oracle; between them, the saved states' rounding
        assert all(e <= TOL[dtype] for e in errs.values()), errs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gated", [True, False], ids=["gdn", "deltanet"])
def test_gdn_train_pair(dtype, gated):
    """beta given (of either sign, and zero on a stretch), with and without the decay gate: the
    training forward's outputs and the saved-workspace gradients against the oracle."""
    w = wl.custom("gdn_train", 420, B=1, H=3, dk=128, dv=128, T=190, dtype=dtype)
    inp = wl.prefill_inputs(w)
    inp["k"] = wl.round_to_bf16(_unit_keys(inp["k"])) if dtype == "bf16" else _unit_keys(inp["k"])
    beta = (inp["eta"] * np.where(np.arange(w.T) % 4 == 0, -0.5, 1.0)[None, :, None]).astype(np.float32)
    beta[:, 20:60] = 0.0
    if not gated:
        inp["log_alpha"] = np.zeros_like(inp["log_alpha"])
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    o, S, (got,) = train_pair(w, inp, g, beta=beta, la_given=gated)
    heads = all_heads(w)
    ro, rS = oracle.gated_delta_recurrent(_sel(inp["q"], heads), _sel(inp["k"], heads), _sel(inp["v"], heads),
                                          _sel(beta, heads), _sel(inp["log_alpha"], heads),
                                          np.stack([g["S0"][b, h] for b, h in heads]))
    eo, eS = rel_l2(_sel(o, heads), ro), rel_l2(states_of(S, heads), rS)
    report(f"gdn train forward {dtype} {'gated' if gated else 'deltanet'}", o=eo, S_T=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)
    compare(f"gdn train pair {dtype} {'gated' if gated else 'deltanet'}", w, got,
            oracle_bwd(w, inp, g, heads, beta=beta, la_given=gated), heads, la_given=gated)


def test_bwd_saved_reuses_the_workspace():
    """Two backward calls from one training forward (two cotangents of the outputs, e.g. two
    losses): both meet the oracle, and repeating the first reproduces it bit for bit (the saved
    part of the workspace is read, not consumed)."""
    w = wl.custom("train_reuse", 430, B=1, H=2, dk=128, dv=128, T=200)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    do2 = np.random.default_rng(5).normal(0, 1, g["do"].shape).astype(np.float32)
    _, _, (g1, g2, g1b) = train_pair(w, inp, g, dos=[g["do"], do2, g["do"]])
    heads = all_heads(w)
    compare("bwd saved, first cotangent", w, g1, oracle_bwd(w, inp, g, heads), heads)
    compare("bwd saved, second cotangent", w, g2, oracle_bwd(w, inp, {**g, "do": do2}, heads), heads)
    for n in NAMES:
        assert np.array_equal(g1[n], g1b[n]), n


def test_train_pair_b8h8_t4096_all_heads():
    """The B8 H8 T4096 d128 bf16 workload at full size, in the benchmark's launch: the training
    forward's outputs equal kla_chunk_fwd's, and every gradient of every head from its workspace
    against the oracle (whole tensor, worst head, worst 64-token chunk)."""
    w = wl.WORKLOADS["fwd_b8h8_t4096"]
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w)
    o, S, (got,) = train_pair(w, inp, g)
    of, Sf = kla.kla_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                               dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps)
    torch.cuda.synchronize()
    assert np.array_equal(o, host(of)) and np.array_equal(S, host(Sf))
    del inp, g, o, S, of, Sf
    got_for = lambda hd: {**{n: heads_of(got[n], hd) for n in ("dq", "dk", "dv", "deta", "dlog_alpha")},
                          "dS0": states_of(got["dS0"], hd)}
    merged, heads = op.run("backward", w, got_for, (0.0, 0.0))
    op.check("train pair b8h8_t4096", merged, heads, TOL[w.dtype])


# ----------------------------------------------------------------------------- per-channel decay (KDA)

def kda_train_pair(w, inp, la, g, beta_given=False):
    """kla_kda_chunk_fwd_train, then kla_kda_chunk_bwd_saved: (o, S_T, gradients) on the host."""
    q, k, v = dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype)
    s0 = None if g["S0"] is None else dev(g["S0"])
    dst = None if g["dST"] is None else dev(g["dST"])
    eta, lad = dev(inp["eta"]), dev(la)
    o, S, ws = kla.kla_kda_chunk_fwd_train(q, k, v, eta, lad, eps=w.eps, beta_given=beta_given, state_in=s0)
    out = kla.kla_kda_chunk_bwd_saved(q, k, v, eta, lad, dev(g["do"], w.dtype), ws, eps=w.eps, beta_given=beta_given,
                                      state_in=s0, dstate_out=dst)
    torch.cuda.synchronize()
    got = {"dq": host(out["dq"]), "dk": host(out["dk"]), "dv": host(out["dv"]), "deta": host(out["deta"]),
           "dlog_a": host(out["dlog_a"]), "dS0": host(out["dstate_in"])}
    return host(o), host(S), got


@pytest.mark.parametrize("dtype,dk,dv,T,beta_given", [
    ("bf16", 128, 128, 250, False), ("bf16", 64, 64, 131, False), ("bf16", 128, 64, 100, False),
    ("bf16", 128, 128, 190, True), ("f32", 64, 64, 77, False), ("f32", 64, 64, 130, True),
])
def test_kda_train_pair_shapes(dtype, dk, dv, T, beta_given):
    """As test_train_pair_shapes, with per-channel decays: outputs against kla_kda_chunk_fwd's (bit
    for bit with the Kaczmarz step, whose factors are the forward's; against the oracle with beta
    given, whose factors the backward makes unbalanced), gradients against the oracle and against
    kla_kda_chunk_bwd (fp32: bit for bit)."""
    w = wl.custom("kda_train", 640 + T, B=2, H=2, dk=dk, dv=dv, T=T, dtype=dtype, log_alpha_range=(0.0, 0.3))
    inp = wl.prefill_inputs(w)
    if beta_given:
        inp["k"] = wl.round_to_bf16(_unit_keys(inp["k"])) if dtype == "bf16" else _unit_keys(inp["k"])
    la = wl.channel_log_decay(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    o, S, got = kda_train_pair(w, inp, la, g, beta_given)
    heads = kb.all_heads(w)
    of, Sf = kla.kla_kda_chunk_fwd(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype), dev(inp["eta"]),
                                   dev(la), eps=w.eps, beta_given=beta_given, state_in=dev(g["S0"]))
    torch.cuda.synchronize()
    if beta_given:
        eo, eS = rel_l2(o, host(of)), rel_l2(S, host(Sf))
        report(f"kda train forward vs kla_kda_chunk_fwd {dtype} beta given", o=eo, S_T=eS)
        assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)
    else:
        assert np.array_equal(o, host(of)) and np.array_equal(S, host(Sf))
    kb.compare(f"kda train pair {dtype} dk={dk} dv={dv} T={T} beta_given={beta_given}", w, got,
               kb.oracle_bwd(w, inp, la, g, heads, beta_given), heads)
    ref = kb.gpu_bwd(w, inp, la, g, beta_given)
    errs = {n: rel_l2(got[n], ref[n]) for n in kb.NAMES}
    report(f"kda train pair vs kla_kda_chunk_bwd {dtype} dk={dk} dv={dv} T={T}", **errs)
    if dtype == "f32":
        for n in kb.NAMES:
            assert np.array_equal(got[n], ref[n]), n
    else:
        assert all(e <= TOL[dtype] for e in errs.values()), errs


def test_kda_train_pair_b8h8_t4096_all_heads():
    """The B8 H8 T4096 d128 bf16 shape at full size with per-channel decays, in the benchmark's
    launch: outputs equal kla_kda_chunk_fwd's, every gradient of every head from the training
    forward's workspace against the oracle."""
    w = wl.WORKLOADS["fwd_b8h8_t4096"]
    inp = wl.prefill_inputs(w)
    la = wl.channel_log_decay(w)
    g = wl.grad_inputs(w)
    o, S, got = kda_train_pair(w, inp, la, g)
    of, Sf = kla.kla_kda_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                                   dev(inp["eta"]), dev(la), eps=w.eps)
    torch.cuda.synchronize()
    assert np.array_equal(o, host(of)) and np.array_equal(S, host(Sf))
    del inp, g, la, o, S, of, Sf
    got_for = lambda hd: {**{n: heads_of(got[n], hd) for n in ("dq", "dk", "dv", "deta", "dlog_a")},
                          "dS0": states_of(got["dS0"], hd)}
    merged, heads = op.run("kda_backward", w, got_for, (0.0, 0.0))
    op.check("kda train pair b8h8_t4096", merged, heads, TOL[w.dtype])
