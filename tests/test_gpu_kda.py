"""GPU parity of the per-channel decay (KDA's gate) against the fp64 oracle on the same seeded
inputs: chunkwise forward (kla_kda_chunk_fwd) and decode (kla_kda_decode_step), with the
Kaczmarz step and with beta given. Bars: relative L2 <= 1e-4 (fp32), <= 2e-2 (bf16)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pool as op
from tests.kla_testutil import TOL, dev, heads_of, host, host32, rel_l2, report, states_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gated_delta_rule_18_amd as kla  # noqa: E402


def all_heads_of(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def compare_fwd(name, w, inp, log_a, beta_given=False, S0=None, heads=None, tol=None):
    tol = TOL[w.dtype] if tol is None else tol
    o, S = kla.kla_kda_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                                 dev(inp["eta"]), dev(log_a), eps=w.eps, beta_given=beta_given,
                                 state_in=None if S0 is None else dev(S0))
    torch.cuda.synchronize()
    heads = all_heads_of(w) if heads is None else heads
    sub = lambda x: np.stack([x[b, :, h] for b, h in heads])[:, :, None]  # [n, T, 1, ...] (library layout, B=n H=1)
    s0 = None if S0 is None else np.stack([S0[b, h] for b, h in heads])[:, None]
    ro, rS = oracle.kda_forward(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), sub(inp["eta"]), sub(log_a), w.eps, s0,
                                beta_given=beta_given)
    go, gS = host(o), host(S)
    eo = rel_l2(np.stack([go[b, :, h] for b, h in heads]), ro[:, :, 0])
    eS = rel_l2(np.stack([gS[b, h] for b, h in heads]), rS[:, 0])
    report(name, o=eo, S_T=eS)
    assert np.isfinite(go).all() and np.isfinite(gS).all()
    assert eo <= tol and eS <= tol, (eo, eS)
    return o, S


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv,T", [(128, 128, 250), (64, 64, 131), (128, 64, 64), (64, 128, 1)])
def test_kda_chunk_fwd(dtype, dk, dv, T):
    w = wl.custom("kda", 500 + T, B=2, H=2, dk=dk, dv=dv, T=T, dtype=dtype, log_alpha_range=(0.0, 0.3))
    inp = wl.prefill_inputs(w)
    S0 = np.random.default_rng(T).normal(0, 0.05, (2, 2, dk, dv)).astype(np.float32)
    compare_fwd(f"kda chunk {dtype} dk={dk} dv={dv} T={T}", w, inp, wl.channel_log_decay(w), S0=S0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kda_chunk_fwd_beta_given(dtype):
    """KDA proper: beta supplied (drawn like eta), unit-norm keys, signed and zero beta."""
    w = wl.custom("kda_beta", 510, B=1, H=3, dk=128, dv=128, T=200, dtype=dtype)
    inp = wl.prefill_inputs(w)
    n = np.linalg.norm(inp["k"].astype(np.float64), axis=-1, keepdims=True)
    k = (inp["k"] / np.maximum(n, 1e-3)).astype(np.float32)
    inp["k"] = wl.round_to_bf16(k) if dtype == "bf16" else k
    inp["eta"] = (inp["eta"] * np.where(np.arange(w.T) % 5 == 0, -0.5, 1.0)[None, :, None]).astype(np.float32)
    inp["eta"][:, 60:90] = 0.0
    compare_fwd(f"kda chunk beta given {dtype}", w, inp, wl.channel_log_decay(w), beta_given=True)


def test_kda_equal_channels_equal_the_scalar_gate():
    """Every channel with the token's scalar log alpha: the KDA path reproduces kla_chunk_fwd."""
    w = wl.custom("kda_eq", 511, B=2, H=2, dk=128, dv=128, T=300)
    inp = wl.prefill_inputs(w)
    la = np.repeat(inp["log_alpha"][..., None], w.dk, axis=-1)
    args = (dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["eta"]))
    o1, S1 = kla.kla_chunk_fwd(*args, dev(inp["log_alpha"]), eps=w.eps)
    o2, S2 = kla.kla_kda_chunk_fwd(*args, dev(la), eps=w.eps)
    torch.cuda.synchronize()
    eo, eS = rel_l2(host(o2), host(o1)), rel_l2(host(S2), host(S1))
    report("kda(equal channels) vs scalar gate", o=eo, S_T=eS)
    assert eo <= 1e-2 and eS <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kda_strong_and_mixed_decay(dtype):
    """Channels that forget almost at once (log a down to -8 per token) next to channels that
    barely decay: every ratio is formed as exp of a non-positive difference, nothing overflows."""
    w = wl.custom("kda_strong", 512, B=1, H=2, dk=64, dv=64, T=257, dtype=dtype)
    inp = wl.prefill_inputs(w)
    la = wl.channel_log_decay(w.with_(log_alpha_range=(0.0, 8.0)))
    la[..., ::2] = wl.channel_log_decay(w.with_(log_alpha_range=(0.0, 0.01)))[..., ::2]
    compare_fwd(f"kda strong/mixed decay {dtype}", w, inp, la)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kda_diagonal_block_paths(dtype):
    """The prep's two ways with a diagonal 16-token block: matrix products when the block's decay
    span is bounded (here log a = -2 per token: factors up to e^30 inside a block), the exact walk
    when one channel forgets faster (channel 5 at -6 per token over tokens 70..99)."""
    w = wl.custom("kda_paths", 515, B=1, H=2, dk=128 if dtype == "bf16" else 64, dv=64, T=192, dtype=dtype)
    inp = wl.prefill_inputs(w)
    la = np.full((1, w.T, 2, w.dk), -2.0, np.float32)
    la[:, :, 1] = wl.channel_log_decay(w)[:, :, 1]
    la[:, 70:100, :, 5] = -6.0
    compare_fwd(f"kda diagonal-block paths {dtype}", w, inp, la)


def test_kda_b8h8_t4096_all_heads():
    """The B8 H8 T4096 d128 bf16 shape at full size with per-channel decays: every head against the
    oracle (whole tensor, worst head, worst 64-token chunk), on o and S_T."""
    w = wl.WORKLOADS["fwd_b8h8_t4096"]
    inp = wl.prefill_inputs(w)
    o, S = kla.kla_kda_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                                 dev(inp["eta"]), dev(wl.channel_log_decay(w)), eps=w.eps)
    del inp
    torch.cuda.synchronize()
    o_h, S_h = host32(o), host32(S)
    merged, heads = op.run("forward", w, lambda g: {"o": heads_of(o_h, g), "S": states_of(S_h, g)}, ("kda",))
    op.check("kda b8h8_t4096", merged, heads, TOL[w.dtype])


# Head counts: 15 (16-column slices), 518 (32-column slices: a lane holds 16 rows, so k, q and
# log a rows arrive by shuffle) and 1088 (64-column slices, 32 rows per lane).
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("beta_given", [False, True], ids=["kaczmarz", "beta"])
@pytest.mark.parametrize("B,H", [(3, 5), (37, 14), (64, 17)])
def test_kda_decode_steps(dtype, beta_given, B, H):
    w = wl.custom("kda_dec", 513, B=B, H=H, dk=128, dv=128, steps=20 if B * H < 256 else 6, dtype=dtype,
                  s0_std=0.05)
    inp = wl.decode_inputs(w)
    la = wl.channel_log_decay(w, decode=True)
    kk = inp["k"]
    if beta_given:
        n = np.linalg.norm(kk.astype(np.float64), axis=-1, keepdims=True)
        kk = (kk / np.maximum(n, 1e-3)).astype(np.float32)
        kk = wl.round_to_bf16(kk) if dtype == "bf16" else kk
    S = dev(inp["S0"])
    outs = []
    for s in range(w.steps):
        o = kla.kla_kda_decode_step(dev(inp["q"][s], dtype), dev(kk[s], dtype), dev(inp["v"][s], dtype),
                                    dev(inp["eta"][s]), dev(la[s]), S, eps=w.eps, beta_given=beta_given)
        outs.append(host(o))
    torch.cuda.synchronize()
    N = w.B * w.H
    flat = lambda x: np.moveaxis(x, 0, 2).reshape(N, w.steps, *x.shape[3:])
    beta = flat(inp["eta"]) if beta_given else oracle.kaczmarz_step_size(flat(kk), flat(inp["eta"]), w.eps)
    ro, rS = oracle.kda_recurrent(flat(inp["q"]), flat(kk), flat(inp["v"]), beta, flat(la),
                                  inp["S0"].reshape(N, w.dk, w.dv))
    eo = rel_l2(flat(np.stack(outs)), ro)
    eS = rel_l2(host(S).reshape(N, w.dk, w.dv), rS)
    report(f"kda decode {dtype} {'beta' if beta_given else 'kaczmarz'} B={B} H={H}", o=eo, S=eS)
    assert eo <= TOL[dtype] and eS <= TOL[dtype], (eo, eS)


def test_kda_decode_continues_the_chunked_forward():
    """Prefill T tokens with the chunked KDA forward, then decode the next tokens one by one;
    the same as one chunked forward over all of them (state passing across the two paths)."""
    w = wl.custom("kda_cont", 514, B=2, H=2, dk=128, dv=128, T=200)
    inp = wl.prefill_inputs(w)
    la = wl.channel_log_decay(w)
    T0 = 150
    o_all, S_all = kla.kla_kda_chunk_fwd(dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"),
                                         dev(inp["eta"]), dev(la), eps=w.eps)
    _, S = kla.kla_kda_chunk_fwd(dev(inp["q"][:, :T0], "bf16"), dev(inp["k"][:, :T0], "bf16"),
                                 dev(inp["v"][:, :T0], "bf16"), dev(inp["eta"][:, :T0]), dev(la[:, :T0]), eps=w.eps)
    outs = []
    for t in range(T0, w.T):
        o = kla.kla_kda_decode_step(dev(inp["q"][:, t], "bf16"), dev(inp["k"][:, t], "bf16"),
                                    dev(inp["v"][:, t], "bf16"), dev(inp["eta"][:, t]), dev(la[:, t]), S, eps=w.eps)
        outs.append(host(o))
    torch.cuda.synchronize()
    eo = rel_l2(np.stack(outs, 1), host(o_all)[:, T0:])
    eS = rel_l2(host(S), host(S_all))
    report("kda decode after chunked", o=eo, S=eS)
    assert eo <= 1e-2 and eS <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kda_segmented_plan(dtype):
    """Two heads over 32 chunks: the plan cuts each head into segments (pass 1 in the scan's KDA
    segment mode, then the combine and the output correction), with an initial state."""
    w = wl.custom("kda_seg", 515, B=1, H=2, dk=128, dv=128, T=2048, dtype=dtype, log_alpha_range=(0.0, 0.2))
    inp = wl.prefill_inputs(w)
    S0 = np.random.default_rng(515).normal(0, 0.05, (1, 2, 128, 128)).astype(np.float32)
    compare_fwd(f"kda segmented {dtype}", w, inp, wl.channel_log_decay(w), S0=S0)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64)])
def test_kda_segmented_head_sizes(dk, dv):
    w = wl.custom("kda_seg_hs", 516, B=1, H=3, dk=dk, dv=dv, T=2100, dtype="bf16")
    compare_fwd(f"kda segmented dk={dk} dv={dv}", w, wl.prefill_inputs(w), wl.channel_log_decay(w))


def test_kda_long_few_heads_all_heads():
    """B1 H4 T16384 d128 bf16 with per-channel decays (the plan takes 16 segments of 16 chunks):
    every head against the oracle (whole tensor, worst head, worst 64-token chunk)."""
    w = wl.custom("kda_long", 517, B=1, H=4, dk=128, dv=128, T=16384, dtype="bf16")
    inp = wl.prefill_inputs(w)
    o, S = kla.kla_kda_chunk_fwd(dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype),
                                 dev(inp["eta"]), dev(wl.channel_log_decay(w)), eps=w.eps)
    del inp
    torch.cuda.synchronize()
    o_h, S_h = host32(o), host32(S)
    merged, heads = op.run("forward", w, lambda g: {"o": heads_of(o_h, g), "S": states_of(S_h, g)}, ("kda",))
    op.check("kda long b1h4_t16384", merged, heads, TOL[w.dtype])
