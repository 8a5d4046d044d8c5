"""GPU parity of the chunkwise backward (kla_chunk_bwd, kla_gdn_chunk_bwd) against the fp64
gradient oracle on the same seeded inputs. Bars: relative L2 <= 1e-4 (fp32 inputs) and
<= 2e-2 (bf16 inputs) on every gradient: dq, dk, dv, deta (dbeta), dlog_alpha, dS_0."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pool as op
from tests.kla_testutil import TOL, dev, heads_of, host, rel_l2, report, states_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gated_delta_rule_18_amd as kla  # noqa: E402

NAMES = ("dq", "dk", "dv", "deta", "dlog_alpha", "dS0")


def _sel(x, heads):
    """[B, T, H, ...] -> [len(heads), T, ...] for the listed (b, h)."""
    return np.stack([x[b, :, h] for b, h in heads])


def _sel_state(x, heads):
    return None if x is None else np.stack([x[b, h] for b, h in heads])


def gpu_bwd(w, inp, g, beta=None, la_given=True):
    """The library's gradients, on the host as fp64 arrays [B, T, H, ...] / [B, H, dk, dv]."""
    q, k, v = dev(inp["q"], w.dtype), dev(inp["k"], w.dtype), dev(inp["v"], w.dtype)
    do = dev(g["do"], w.dtype)
    s0 = None if g["S0"] is None else dev(g["S0"])
    dst = None if g["dST"] is None else dev(g["dST"])
    if beta is None:
        out = kla.kla_chunk_bwd(q, k, v, dev(inp["eta"]), dev(inp["log_alpha"]), do, eps=w.eps, state_in=s0,
                                dstate_out=dst)
        gate = out["deta"]
    else:
        out = kla.kla_gdn_chunk_bwd(q, k, v, dev(beta), dev(inp["log_alpha"]) if la_given else None, do,
                                    state_in=s0, dstate_out=dst)
        gate = out["dbeta"]
    torch.cuda.synchronize()
    res = {"dq": host(out["dq"]), "dk": host(out["dk"]), "dv": host(out["dv"]), "deta": host(gate),
           "dS0": host(out["dstate_in"])}
    res["dlog_alpha"] = None if out["dlog_alpha"] is None else host(out["dlog_alpha"])
    return res


def oracle_bwd(w, inp, g, heads, beta=None, la_given=True):
    """Oracle gradients of the listed heads, head-major [n, T, ...] / [n, dk, dv]."""
    la = _sel(inp["log_alpha"], heads) if la_given else np.zeros((len(heads), w.T))
    args = (_sel(inp["q"], heads), _sel(inp["k"], heads), _sel(inp["v"], heads))
    s0, dst, do = _sel_state(g["S0"], heads), _sel_state(g["dST"], heads), _sel(g["do"], heads)
    if beta is None:
        r = oracle.kla_vjp(*args, _sel(inp["eta"], heads), la, w.eps, s0, do, dst)
    else:
        r = oracle.gated_delta_vjp(*args, _sel(beta, heads), la, s0, do, dst)
        r["deta"] = r.pop("dbeta")
    return r


def compare(name, w, got, ref, heads, tol=None, la_given=True):
    tol = TOL[w.dtype] if tol is None else tol
    errs = {}
    for n in NAMES:
        if n == "dlog_alpha" and not la_given:
            assert got[n] is None
            continue
        x = _sel_state(got[n], heads) if n == "dS0" else _sel(got[n], heads)
        assert np.isfinite(x).all(), n
        errs[n] = rel_l2(x, ref[n])
    report(name, **errs)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad


def all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


@pytest.mark.parametrize("dtype,dk,dv,T", [
    ("bf16", 128, 128, 250), ("bf16", 128, 128, 64), ("bf16", 64, 64, 131), ("bf16", 128, 64, 100),
    ("bf16", 64, 128, 1), ("f32", 64, 64, 256), ("f32", 64, 64, 77),
    ("f32", 128, 128, 250), ("f32", 128, 128, 64), ("f32", 128, 64, 100), ("f32", 64, 128, 131),
])
def test_chunk_bwd_shapes(dtype, dk, dv, T):
    w = wl.custom("bwd", 300 + T, B=2, H=2, dk=dk, dv=dv, T=T, dtype=dtype)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    compare(f"chunk_bwd {dtype} dk={dk} dv={dv} T={T}", w, gpu_bwd(w, inp, g), oracle_bwd(w, inp, g, all_heads(w)),
            all_heads(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_bwd_without_state_or_state_cotangent(dtype):
    """S_0 = 0 and dS_T = 0 (both pointers null)."""
    w = wl.custom("bwd_nostate", 310, B=1, H=3, dk=64, dv=64, T=200, dtype=dtype)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w)
    compare(f"chunk_bwd {dtype} no state", w, gpu_bwd(w, inp, g), oracle_bwd(w, inp, g, all_heads(w)), all_heads(w))


def test_chunk_bwd_tiny_f32_workload():
    """The fp32 workload's shape (B1 H1 T256 d64) with an initial state and a state cotangent."""
    w = wl.WORKLOADS["fwd_tiny_f32"]
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    compare("chunk_bwd fwd_tiny_f32", w, gpu_bwd(w, inp, g), oracle_bwd(w, inp, g, all_heads(w)), all_heads(w))


def test_chunk_bwd_b8h8_t4096_all_heads():
    """The B8 H8 T4096 d128 bf16 workload at full size, in the benchmark's launch: every gradient of
    every head against the oracle (the adjoint of the token loop; whole tensor, worst head, worst
    64-token chunk)."""
    w = wl.WORKLOADS["fwd_b8h8_t4096"]
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w)
    got = gpu_bwd(w, inp, g)
    del inp, g
    got_for = lambda hd: {**{n: heads_of(got[n], hd) for n in ("dq", "dk", "dv", "deta", "dlog_alpha")},
                          "dS0": states_of(got["dS0"], hd)}
    merged, heads = op.run("backward", w, got_for, (0.0, 0.0))
    op.check("chunk_bwd b8h8_t4096", merged, heads, TOL[w.dtype])


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
def test_chunk_bwd_partial_last_round(dtype, dk):
    """More chunks (5 heads x 62) than the gradient kernel keeps resident, and not a multiple of
    them: with one workgroup per CU (these head sizes) each workgroup walks several chunks and
    the last round is partial. The oracle on the first head and on the last one, whose chunks
    fall in that round."""
    w = wl.custom("bwd_rounds", 313, B=1, H=5, dk=dk, dv=dk, T=64 * 61 + 17, dtype=dtype)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    got = gpu_bwd(w, inp, g)
    for hd in ([(0, 0)], [(0, 4)]):
        compare(f"chunk_bwd {dtype} d{dk} rounds head {hd[0]}", w, got, oracle_bwd(w, inp, g, hd), hd)


def test_chunk_bwd_mixed_gates_extremes():
    """The mixed workload's gates (eta = sigmoid(N(0, 2)), log alpha in [-0.2, 0]) over a
    few chunks."""
    w = wl.WORKLOADS["mixed_b4h16"].with_(B=1, H=2, T=320, steps=0, wid=311)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, dst_std=1.0)
    compare("chunk_bwd mixed gates", w, gpu_bwd(w, inp, g), oracle_bwd(w, inp, g, all_heads(w)), all_heads(w))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_bwd_edge_tokens(dtype):
    """eta = 0 on a stretch (pure decay), zero keys (beta = eta / eps, no update), alpha = 1."""
    w = wl.custom("bwd_edge", 312, B=1, H=2, dk=64, dv=64, T=150, dtype=dtype)
    inp = wl.prefill_inputs(w)
    inp["eta"][:, 20:60] = 0.0
    inp["k"][:, 70:75] = 0.0
    inp["log_alpha"][:, 100:] = 0.0
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    compare(f"chunk_bwd edges {dtype}", w, gpu_bwd(w, inp, g), oracle_bwd(w, inp, g, all_heads(w)), all_heads(w))


def test_chunk_bwd_zero_length():
    """T = 0: dS_0 = dS_T and nothing else is written."""
    w = wl.custom("bwd_t0", 313, B=2, H=3, dk=128, dv=128, T=0)
    g = wl.grad_inputs(w, dst_std=1.0)
    z = lambda *s: torch.zeros(*s, device="cuda:0")
    out = kla.kla_chunk_bwd(z(2, 0, 3, 128).bfloat16(), z(2, 0, 3, 128).bfloat16(), z(2, 0, 3, 128).bfloat16(),
                            z(2, 0, 3), z(2, 0, 3), z(2, 0, 3, 128).bfloat16(), dstate_out=dev(g["dST"]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["dstate_in"]), g["dST"])


def test_chunk_bwd_deterministic_bitwise():
    w = wl.custom("bwd_det", 314, B=2, H=2, dk=128, dv=128, T=300)
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    a, b = gpu_bwd(w, inp, g), gpu_bwd(w, inp, g)
    for n in NAMES:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


def _unit_keys(k):
    n = np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
    return (k / np.maximum(n, 1e-3)).astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gated", [True, False], ids=["gdn", "deltanet"])
def test_gdn_chunk_bwd(dtype, gated):
    """beta given: signed, with a stretch of zeros (d(beta) there is still defined); unit keys."""
    w = wl.custom("gdn_bwd", 315, B=2, H=2, dk=64, dv=64, T=190, dtype=dtype)
    inp = wl.prefill_inputs(w)
    inp["k"] = wl.round_to_bf16(_unit_keys(inp["k"])) if dtype == "bf16" else _unit_keys(inp["k"])
    beta = (inp["eta"] * np.where(np.arange(w.T) % 4 == 0, -0.5, 1.0)[None, :, None]).astype(np.float32)
    beta[:, 30:70] = 0.0
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    got = gpu_bwd(w, inp, g, beta=beta, la_given=gated)
    ref = oracle_bwd(w, inp, g, all_heads(w), beta=beta, la_given=gated)
    compare(f"gdn_chunk_bwd {dtype} {'gated' if gated else 'deltanet'}", w, got, ref, all_heads(w), la_given=gated)


@pytest.mark.parametrize("gated", [True, False], ids=["gdn", "deltanet"])
def test_gdn_chunk_bwd_f32_d128(gated):
    """fp32 with 128-wide heads (the gradient kernel that forms the products over d_v in two
    parts), beta given, signed and zero; also bitwise reproducible."""
    w = wl.custom("gdn_bwd128", 317, B=1, H=2, dk=128, dv=128, T=150, dtype="f32")
    inp = wl.prefill_inputs(w)
    inp["k"] = _unit_keys(inp["k"])
    beta = (inp["eta"] * np.where(np.arange(w.T) % 4 == 0, -0.5, 1.0)[None, :, None]).astype(np.float32)
    beta[:, 30:70] = 0.0
    g = wl.grad_inputs(w, s0_std=0.05, dst_std=1.0)
    got = gpu_bwd(w, inp, g, beta=beta, la_given=gated)
    again = gpu_bwd(w, inp, g, beta=beta, la_given=gated)
    for n in NAMES:
        if got[n] is not None:
            np.testing.assert_array_equal(got[n], again[n], err_msg=n)
    ref = oracle_bwd(w, inp, g, all_heads(w), beta=beta, la_given=gated)
    compare(f"gdn_chunk_bwd f32 d128 {'gated' if gated else 'deltanet'}", w, got, ref, all_heads(w), la_given=gated)


def test_bwd_agrees_with_forward_by_directional_derivative():
    """<grad, direction> equals the change of the library's own forward loss along a direction
    (central difference of the fp32 forward), a check that uses no oracle. Each direction has
    the scale of its input, so the step is a relative one."""
    w = wl.custom("bwd_dir", 316, B=1, H=2, dk=64, dv=64, T=128, dtype="f32")
    inp = wl.prefill_inputs(w)
    g = wl.grad_inputs(w, dst_std=1.0)
    got = gpu_bwd(w, inp, g)
    rng = np.random.default_rng(5)
    scale = {"q": 1 / 8, "k": 1 / 8, "v": 1.0, "log_alpha": 0.05}
    dirs = {n: (scale[n] * rng.standard_normal(inp[n].shape)).astype(np.float32) for n in scale}

    def loss(h):
        x = {n: (inp[n] + h * dirs[n]).astype(np.float32) if n in dirs else inp[n] for n in inp}
        o, S = kla.kla_chunk_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["eta"]), dev(x["log_alpha"]),
                                 eps=w.eps)
        torch.cuda.synchronize()
        return float(np.sum(host(o) * g["do"]) + np.sum(host(S) * g["dST"]))

    h = 2e-3
    fd = (loss(h) - loss(-h)) / (2 * h)
    an = sum(float(np.sum(got["d" + n] * dirs[n])) for n in dirs)
    report("bwd directional", rel=abs(fd - an) / abs(an))
    assert abs(fd - an) <= 5e-3 * abs(an), (fd, an)
