"""GPU parity: the HIP path (through the C ABI binding) against the fp64 oracle on the
same seeded inputs. Bars: relative L2 <= 1e-4 for fp32 inputs and <= 2e-2 for bf16
inputs with fp32 accumulation, on o and on the final state."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pool as op
from tests.kla_testutil import TOL, dev, heads_of, host, host32, rel_l2, report, states_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gated_delta_rule_18_amd as kla  # noqa: E402


def _sel(x, heads):
    return np.stack([x[b, :, h] for b, h in heads])


def gpu_fwd(w, inp, S0=None, return_state=True):
    o, S = kla.kla_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                             dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps,
                             state_in=None if S0 is None else dev(S0), return_state=return_state)
    torch.cuda.synchronize()
    return host(o), (None if S is None else host(S))


def oracle_fwd(w, inp, heads, S0=None):
    s0 = None if S0 is None else np.stack([S0[b, h] for b, h in heads])
    return oracle.kla_recurrent(_sel(inp["q"], heads), _sel(inp["k"], heads), _sel(inp["v"], heads),
                                _sel(inp["eta"], heads), _sel(inp["log_alpha"], heads), w.eps, s0)


def check_fwd(name, w, inp, heads, S0=None, tol=None):
    tol = TOL[w.dtype] if tol is None else tol
    o, S = gpu_fwd(w, inp, S0)
    ro, rS = oracle_fwd(w, inp, heads, S0)
    eo = rel_l2(_sel(o, heads), ro)
    eS = rel_l2(np.stack([S[b, h] for b, h in heads]), rS)
    report(name, o=eo, S_T=eS)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= tol and eS <= tol, (eo, eS)
    return o, S


def all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


# ----------------------------------------------------------------------------- prologue

@pytest.mark.parametrize("dtype,dk,T", [("bf16", 128, 250), ("f32", 64, 130), ("bf16", 64, 64), ("f32", 128, 1)])
def test_prepare_beta(dtype, dk, T):
    w = wl.custom("prep", 200, B=2, H=3, dk=dk, dv=dk, T=T, dtype=dtype)
    inp = wl.prefill_inputs(w)
    beta, G = kla.kla_prepare_beta(dev(inp["k"], dtype), dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps)
    torch.cuda.synchronize()
    rb, rG = oracle.kla_prepare_beta(inp["k"], inp["eta"], inp["log_alpha"], w.eps, 64)
    report(f"prepare_beta {dtype} dk={dk} T={T}", beta=rel_l2(host(beta), rb), G=rel_l2(host(G), rG))
    np.testing.assert_allclose(host(beta), rb, rtol=2e-6, atol=0)
    np.testing.assert_allclose(host(G), rG, rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv,B,H", [(128, 128, 2, 3), (64, 64, 2, 3), (128, 64, 1, 5), (64, 128, 3, 1),
                                       (128, 128, 3, 5), (128, 128, 64, 17), (64, 64, 64, 17), (64, 128, 64, 17),
                                       (128, 64, 64, 17), (128, 128, 37, 14)])
def test_decode_steps_small(dtype, dk, dv, B, H):
    w = wl.custom("dec", 201, B=B, H=H, dk=dk, dv=dv, steps=12, dtype=dtype, s0_std=0.05)
    inp = wl.decode_inputs(w)
    S = dev(inp["S0"])
    outs = []
    for s in range(w.steps):
        o = kla.kla_decode_step(dev(inp["q"][s], dtype), dev(inp["k"][s], dtype), dev(inp["v"][s], dtype),
                                dev(inp["eta"][s]), dev(inp["log_alpha"][s]), S, eps=w.eps)
        outs.append(host(o))
    torch.cuda.synchronize()
    ro, rS = oracle.kla_decode_steps(inp["q"], inp["k"], inp["v"], inp["eta"], inp["log_alpha"], w.eps, inp["S0"])
    eo, eS = rel_l2(np.stack(outs), ro), rel_l2(host(S), rS)
    report(f"decode {dtype} dk={dk} dv={dv} B={B} H={H}", o=eo, S=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype]


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
def test_decode_state_beyond_the_cache(dtype, dk):
    """A state of 512 MiB or more (twice the last-level cache) is rewritten with streaming stores:
    8 192 heads at d = 128 bf16 (512 MiB) and 32 768 heads at d = 64 fp32 (512 MiB), four steps,
    every head against the oracle."""
    B, H = (512, 16) if dk == 128 else (2048, 16)
    w = wl.custom("dec_big", 204, B=B, H=H, dk=dk, dv=dk, steps=4, dtype=dtype, s0_std=0.02)
    inp = wl.decode_inputs(w)
    S = dev(inp["S0"])
    outs = []
    for s in range(w.steps):
        o = kla.kla_decode_step(dev(inp["q"][s], dtype), dev(inp["k"][s], dtype), dev(inp["v"][s], dtype),
                                dev(inp["eta"][s]), dev(inp["log_alpha"][s]), S, eps=w.eps)
        outs.append(host(o))
    torch.cuda.synchronize()
    ro, rS = oracle.kla_decode_steps(inp["q"], inp["k"], inp["v"], inp["eta"], inp["log_alpha"], w.eps, inp["S0"])
    eo, eS = rel_l2(np.stack(outs), ro), rel_l2(host(S), rS)
    report(f"decode {dtype} d={dk} B={B} H={H} (streaming state stores)", o=eo, S=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype]


def test_decode_workload_b64h16_1024_steps():
    """Decode B64 H16 d128, 1024 consecutive steps from S0 ~ N(0, 0.02): every one of the 1024 heads
    against the oracle (whole tensor, worst head, worst 64-step window)."""
    w = wl.WORKLOADS["decode_b64h16"]
    inp = wl.decode_inputs(w)
    S = dev(inp["S0"])
    q, k, v = dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype)
    eta, la = dev(inp["eta"]), dev(inp["log_alpha"])
    del inp
    o_all = torch.empty((w.steps, w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda:0")
    for s in range(w.steps):
        kla.kla_decode_step(q[s], k[s], v[s], eta[s], la[s], S, eps=w.eps, o=o_all[s])
    torch.cuda.synchronize()
    o_h, S_h = host32(o_all), host32(S)
    merged, heads = op.run("decode", w, lambda g: {"od": heads_of(o_h, g, 0), "S": states_of(S_h, g)})
    op.check("decode_b64h16", merged, heads, TOL["bf16"])


# ----------------------------------------------------------------------------- chunked forward

# T spans 1 to 8 chunks: every count of chunks modulo the scan's ring of operand buffers (three
# for the bf16 one-pass forward), with full and ragged last chunks.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 15, 63, 64, 65, 192, 250, 300, 449])
def test_chunk_fwd_small_shapes(dtype, T):
    w = wl.custom("fwd", 202 + T, B=2, H=3, dk=128, dv=128, T=T, dtype=dtype)
    check_fwd(f"chunk_fwd {dtype} T={T}", w, wl.prefill_inputs(w), all_heads(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_chunk_fwd_head_sizes(dtype, dk, dv):
    w = wl.custom("fwd_d", 210 + dk + dv, B=1, H=9, dk=dk, dv=dv, T=200, dtype=dtype)
    check_fwd(f"chunk_fwd {dtype} dk={dk} dv={dv}", w, wl.prefill_inputs(w), all_heads(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_fwd_initial_state_and_aliasing(dtype):
    w = wl.custom("fwd_s0", 220, B=2, H=2, dk=128, dv=128, T=190, dtype=dtype)
    inp = wl.prefill_inputs(w)
    S0 = np.random.default_rng(5).normal(0, 0.05, (2, 2, 128, 128)).astype(np.float32)
    check_fwd(f"chunk_fwd {dtype} with S0", w, inp, all_heads(w), S0=S0)
    # in place: state_out is state_in
    S = dev(S0)
    o, S_out = kla.kla_chunk_fwd(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype),
                                 dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps, state_in=S, state_out=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    _, rS = oracle_fwd(w, inp, all_heads(w), S0)
    assert rel_l2(host(S).reshape(-1, 128, 128), rS) <= TOL[dtype]


def test_chunk_fwd_zero_length_copies_state():
    S0 = dev(np.random.default_rng(6).normal(0, 1, (2, 3, 64, 64)).astype(np.float32))
    z = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((2, 0, 3), dtype=torch.float32, device="cuda:0")
    o, S = kla.kla_chunk_fwd(z, z, z, g, g, state_in=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64)
    assert torch.equal(S, S0)


def test_chunk_fwd_fwd_tiny_f32_workload():
    """fp32 B1 H1 T256 d64: the whole output and state against the oracle (bar 1e-4)."""
    w = wl.WORKLOADS["fwd_tiny_f32"]
    check_fwd("fwd_tiny_f32", w, wl.prefill_inputs(w), all_heads(w))


def full_size_fwd(name, w):
    """A prefill workload at full size, in the launch the benchmark times (kla_chunk_fwd with the
    library's plan): every head against the oracle (whole tensor, worst head, worst 64-token chunk),
    on o and S_T."""
    inp = wl.prefill_inputs(w)
    o, S = kla.kla_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                             dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps)
    del inp
    torch.cuda.synchronize()
    o_h, S_h = host32(o), host32(S)
    merged, heads = op.run("forward", w, lambda g: {"o": heads_of(o_h, g), "S": states_of(S_h, g)})
    op.check(name, merged, heads, TOL[w.dtype])


def test_chunk_fwd_b8h8_t4096_workload():
    full_size_fwd("fwd_b8h8_t4096", wl.WORKLOADS["fwd_b8h8_t4096"])


def test_chunk_fwd_long_t65536_workload():
    """B1 H16 T65536: the plan segments this one (few heads, long sequence)."""
    full_size_fwd("fwd_long_t65536", wl.WORKLOADS["fwd_long_t65536"])


def test_mixed_prefill_then_decode_workload():
    """Prefill B4 H16 T32768, then 512 decode steps from its final states: every head against one
    uninterrupted oracle recurrence over T + 512 tokens (prefill o, decode o, final state)."""
    w = wl.WORKLOADS["mixed_b4h16"]
    inp = wl.prefill_inputs(w)
    o, S = kla.kla_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                             dev(inp["eta"]), dev(inp["log_alpha"]), eps=w.eps)
    del inp
    dec = wl.decode_inputs(w)
    q, k, v = dev(dec["q"], w.dtype), dev(dec["k"], w.dtype), dev(dec["v"], w.dtype)
    eta, la = dev(dec["eta"]), dev(dec["log_alpha"])
    del dec
    od = torch.empty((w.steps, w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda:0")
    for s in range(w.steps):
        kla.kla_decode_step(q[s], k[s], v[s], eta[s], la[s], S, eps=w.eps, o=od[s])
    torch.cuda.synchronize()
    o_h, od_h, S_h = host32(o), host32(od), host32(S)
    merged, heads = op.run("forward", w, lambda g: {"o": heads_of(o_h, g), "od": heads_of(od_h, g, 0),
                                                   "S": states_of(S_h, g)})
    op.check("mixed_b4h16", merged, heads, TOL["bf16"])


# ----------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_eta_zero_is_pure_decay(dtype):
    w = wl.custom("eta0", 230, B=1, H=2, dk=128, dv=128, T=150, dtype=dtype)
    inp = wl.prefill_inputs(w)
    inp["eta"][:] = 0.0
    S0 = np.random.default_rng(7).normal(0, 0.1, (1, 2, 128, 128)).astype(np.float32)
    check_fwd(f"eta=0 {dtype}", w, inp, all_heads(w), S0=S0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_no_decay_full_step_and_zero_keys(dtype):
    """alpha = 1 and eta = 1 everywhere, with some all-zero keys (finite, only decay)."""
    w = wl.custom("edge", 231, B=1, H=3, dk=64, dv=64, T=140, dtype=dtype)
    inp = wl.prefill_inputs(w)
    inp["log_alpha"][:] = 0.0
    inp["eta"][:] = 1.0
    inp["k"][0, [0, 5, 63, 64, 100], :, :] = 0.0
    check_fwd(f"alpha=1 eta=1 zero keys {dtype}", w, inp, all_heads(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_extreme_gates(dtype):
    """Strong forgetting (log alpha down to -8 per token) and eta near 0 and 1."""
    w = wl.custom("extreme", 232, B=1, H=4, dk=128, dv=128, T=256, dtype=dtype, eta_std=4.0,
                  log_alpha_range=(0.0, 8.0))
    check_fwd(f"extreme gates {dtype}", w, wl.prefill_inputs(w), all_heads(w))


# ----------------------------------------------------------------------------- properties

def test_deterministic_bitwise():
    w = wl.custom("det", 240, B=2, H=4, dk=128, dv=128, T=300)
    inp = wl.prefill_inputs(w)
    args = (dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["eta"]),
            dev(inp["log_alpha"]))
    o1, S1 = kla.kla_chunk_fwd(*args)
    o2, S2 = kla.kla_chunk_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_passing_split(dtype):
    """fwd(T1) then fwd(T2 | S_T1) agrees with fwd(T1 + T2): only the state crosses."""
    w = wl.custom("split", 241, B=1, H=4, dk=128, dv=128, T=320, dtype=dtype)
    inp = wl.prefill_inputs(w)
    t1 = 131
    first = {n: a[:, :t1].copy() for n, a in inp.items()}
    second = {n: a[:, t1:].copy() for n, a in inp.items()}
    o1, S1 = gpu_fwd(w.with_(T=t1), first)
    o2, S2 = gpu_fwd(w.with_(T=w.T - t1), second, S0=S1.astype(np.float32))
    o, S = gpu_fwd(w, inp)
    e_o = rel_l2(np.concatenate([o1, o2], 1), o)
    e_S = rel_l2(S2, S)
    report(f"state passing {dtype}", o=e_o, S=e_S)
    assert e_o <= TOL[dtype] and e_S <= TOL[dtype]


def test_decode_continues_chunk_fwd():
    """T decode steps from zero agree with one chunked pass over the same T tokens."""
    w = wl.custom("dvc", 242, B=2, H=2, dk=128, dv=128, T=70, dtype="f32")
    inp = wl.prefill_inputs(w)
    o, S = gpu_fwd(w, inp)
    St = torch.zeros((2, 2, 128, 128), dtype=torch.float32, device="cuda:0")
    od = []
    for t in range(w.T):
        od.append(host(kla.kla_decode_step(dev(inp["q"][:, t], "f32"), dev(inp["k"][:, t], "f32"),
                                           dev(inp["v"][:, t], "f32"), dev(inp["eta"][:, t]),
                                           dev(inp["log_alpha"][:, t]), St, eps=w.eps)))
    torch.cuda.synchronize()
    e_o = rel_l2(np.stack(od, 1), o)
    e_S = rel_l2(host(St), S)
    report("decode vs chunk_fwd f32", o=e_o, S=e_S)
    assert e_o <= 1e-4 and e_S <= 1e-4
    assert math.isfinite(e_o)


def test_decode_steps_replayed_from_a_hip_graph():
    """Decode steps captured in a HIP graph (as the benchmark and a serving loop issue them)
    replay to the eager result, bit for bit, on every replay, with eager work in between."""
    w = wl.custom("graph", 243, B=4, H=16, dk=128, dv=128, steps=16, dtype="bf16", s0_std=0.02)
    inp = wl.decode_inputs(w)
    q, k, v = dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16")
    eta, la, S0 = dev(inp["eta"]), dev(inp["log_alpha"]), dev(inp["S0"])
    S = S0.clone()
    o = torch.empty((w.steps, w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda:0")

    def run():
        for s in range(w.steps):
            kla.kla_decode_step(q[s], k[s], v[s], eta[s], la[s], S, eps=w.eps, o=o[s])

    run()
    torch.cuda.synchronize()
    o_ref, S_ref = o.clone(), S.clone()
    g = torch.cuda.CUDAGraph()
    S.copy_(S0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    x = dev(wl.prefill_inputs(wl.custom("graph_eager", 244, B=1, H=2, dk=128, dv=128, T=100))["q"], "bf16")
    for rep in range(3):
        S.copy_(S0)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: outputs differ"
        assert torch.equal(S, S_ref), f"replay {rep}: state differs"
        kla.kla_chunk_fwd(x, x, x, torch.full(x.shape[:3], 0.5, device="cuda:0"),
                          torch.zeros(x.shape[:3], device="cuda:0"))  # eager work between replays
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------- gated DeltaNet / DeltaNet (beta given)

def _unit_keys(k):
    """Keys scaled to unit norm (input preparation for the beta-given modes, which are used with
    normalised keys: with ||k|| up to 4 and beta up to 1 the delta rule itself diverges)."""
    n = np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
    return (k / np.maximum(n, 1e-3)).astype(np.float32)


def _gdn_case(w, with_gate=True, beta_sign=1.0):
    inp = wl.prefill_inputs(w)
    inp["k"] = wl.round_to_bf16(_unit_keys(inp["k"])) if w.dtype == "bf16" else _unit_keys(inp["k"])
    beta = (inp["eta"] * beta_sign).astype(np.float32)  # drawn like eta: sigmoid(N(0, 1))
    la = inp["log_alpha"] if with_gate else np.zeros_like(inp["log_alpha"])
    return inp, beta, la


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gated", [True, False], ids=["gdn", "deltanet"])
@pytest.mark.parametrize("dk,dv,T", [(128, 128, 250), (64, 64, 131), (128, 64, 64)])
def test_gdn_chunk_fwd(dtype, gated, dk, dv, T):
    w = wl.custom("gdn", 250, B=2, H=3, dk=dk, dv=dv, T=T, dtype=dtype)
    inp, beta, la = _gdn_case(w, gated)
    o, S = kla.kla_gdn_chunk_fwd(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype), dev(beta),
                                 dev(la) if gated else None)
    torch.cuda.synchronize()
    heads = all_heads(w)
    ro, rS = oracle.gated_delta_recurrent(_sel(inp["q"], heads), _sel(inp["k"], heads), _sel(inp["v"], heads),
                                          _sel(beta, heads), _sel(la, heads))
    eo = rel_l2(_sel(host(o), heads), ro)
    eS = rel_l2(np.stack([host(S)[b, h] for b, h in heads]), rS)
    report(f"gdn chunk {dtype} {'gated' if gated else 'deltanet'} dk={dk} dv={dv} T={T}", o=eo, S_T=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gdn_chunk_fwd_signed_and_zero_beta(dtype):
    """beta of either sign (the balanced factors use |beta| and its sign), zero beta on a
    stretch of tokens, and an initial state."""
    w = wl.custom("gdn_sign", 251, B=1, H=4, dk=128, dv=128, T=200, dtype=dtype, s0_std=0.05)
    inp, beta, la = _gdn_case(w)
    beta = beta * np.where(np.arange(w.T) % 3 == 0, -0.5, 1.0)[None, :, None].astype(np.float32)
    beta[:, 40:90] = 0.0
    S0 = np.random.default_rng(7).normal(0, 0.05, (1, 4, 128, 128)).astype(np.float32)
    o, S = kla.kla_gdn_chunk_fwd(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype), dev(beta),
                                 dev(la), state_in=dev(S0))
    torch.cuda.synchronize()
    heads = all_heads(w)
    ro, rS = oracle.gated_delta_recurrent(_sel(inp["q"], heads), _sel(inp["k"], heads), _sel(inp["v"], heads),
                                          _sel(beta, heads), _sel(la, heads), np.stack([S0[b, h] for b, h in heads]))
    eo = rel_l2(_sel(host(o), heads), ro)
    eS = rel_l2(np.stack([host(S)[b, h] for b, h in heads]), rS)
    report(f"gdn chunk signed/zero beta {dtype}", o=eo, S_T=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


def test_gdn_with_the_kaczmarz_step_equals_kla():
    """Feeding kla_gdn_chunk_fwd the library's own Kaczmarz step (kla_prepare_beta) reproduces
    kla_chunk_fwd: the two balanced factorisations of the same recurrence agree."""
    w = wl.custom("gdn_vs_kla", 252, B=2, H=2, dk=128, dv=128, T=300)
    inp = wl.prefill_inputs(w)
    q, k, v = dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16")
    eta, la = dev(inp["eta"]), dev(inp["log_alpha"])
    beta, _ = kla.kla_prepare_beta(k, eta, la, eps=w.eps, with_gcum=False)
    o1, S1 = kla.kla_chunk_fwd(q, k, v, eta, la, eps=w.eps)
    o2, S2 = kla.kla_gdn_chunk_fwd(q, k, v, beta, la)
    torch.cuda.synchronize()
    eo, eS = rel_l2(host(o2), host(o1)), rel_l2(host(S2), host(S1))
    report("gdn(kaczmarz beta) vs kla", o=eo, S_T=eS)
    assert eo <= 1e-2 and eS <= 1e-2, (eo, eS)


# Head counts: 15 (16-column slices), 518 (32-column slices) and 1088 (64-column slices).
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gated", [True, False], ids=["gdn", "deltanet"])
@pytest.mark.parametrize("B,H", [(3, 5), (37, 14), (64, 17)])
def test_gdn_decode_steps(dtype, gated, B, H):
    w = wl.custom("gdn_dec", 253, B=B, H=H, dk=128, dv=128, steps=20 if B * H < 256 else 6, dtype=dtype,
                  s0_std=0.05)
    inp = wl.decode_inputs(w)
    kk = _unit_keys(inp["k"])
    kk = wl.round_to_bf16(kk) if dtype == "bf16" else kk
    beta = inp["eta"]
    la = inp["log_alpha"] if gated else np.zeros_like(inp["log_alpha"])
    S = dev(inp["S0"])
    outs = []
    for s in range(w.steps):
        o = kla.kla_gdn_decode_step(dev(inp["q"][s], dtype), dev(kk[s], dtype), dev(inp["v"][s], dtype),
                                    dev(beta[s]), dev(la[s]) if gated else None, S)
        outs.append(host(o))
    torch.cuda.synchronize()
    # oracle: the recurrence over the steps, heads flattened
    N = w.B * w.H
    flat = lambda x: np.moveaxis(x, 0, 2).reshape(N, w.steps, *x.shape[3:])  # [steps, B, H, ...] -> [N, steps, ...]
    ro, rS = oracle.gated_delta_recurrent(flat(inp["q"]), flat(kk), flat(inp["v"]), flat(beta), flat(la),
                                          inp["S0"].reshape(N, w.dk, w.dv))
    eo = rel_l2(flat(np.stack(outs)), ro)
    eS = rel_l2(host(S).reshape(N, w.dk, w.dv), rS)
    report(f"gdn decode {dtype} {'gated' if gated else 'deltanet'} B={B} H={H}", o=eo, S=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)
