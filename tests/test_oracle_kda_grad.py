"""Pins for the fp64 gradients of the per-channel decay (KDA) loop (CPU only).

Two implementations of the same derivative of ``oracle.kda_recurrent`` ("Deep Dive into KDA",
section 2.3): reverse-mode autodiff (kla_grad.kda_vjp, PyTorch) and the adjoint recurrence
(adjoint.kda_adjoint, NumPy). Each is tied to things other than itself: central finite
differences of the NumPy forward oracle (pinned in test_oracle_kda.py), the reduction to the
scalar gate when every channel decays alike (whose gradients are pinned in test_oracle_grad.py),
the closed form of a pure per-channel decay, exact homogeneity identities, and a planted mistake.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import adjoint

pytestmark = pytest.mark.filterwarnings("error::RuntimeWarning")

IMPLS = {
    "autodiff": oracle.kda_vjp,
    "adjoint": lambda *a, **kw: oracle.kda_adjoint(*a, block=4, **kw),
}
impls = pytest.mark.parametrize("impl", sorted(IMPLS))


def rand_case(rng, N, T, dk, dv):
    q = rng.standard_normal((N, T, dk)) / math.sqrt(dk)
    k = rng.standard_normal((N, T, dk)) / math.sqrt(dk) * np.exp(
        rng.uniform(math.log(0.5), math.log(2.0), (N, T, 1)))
    v = rng.standard_normal((N, T, dv))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, T))))
    la = -rng.uniform(0.001, 0.6, (N, T, dk))
    S0 = 0.5 * rng.standard_normal((N, dk, dv))
    do = rng.standard_normal((N, T, dv))
    dST = rng.standard_normal((N, dk, dv))
    return q, k, v, eta, la, S0, do, dST


def _loss(q, k, v, eta, la, eps, S0, do, dST, beta_given):
    beta = eta if beta_given else oracle.kaczmarz_step_size(k, eta, eps)
    o, S = oracle.kda_recurrent(q, k, v, beta, la, S0)
    return float(np.sum(o * do) + np.sum(S * dST))


def _fd(fun, args, i, h=1e-6):
    """Central differences of fun(*args) with respect to every entry of args[i]."""
    base = [np.array(a, dtype=np.float64, copy=True) if isinstance(a, np.ndarray) else a for a in args]
    x = base[i]
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        x0 = x[idx]
        x[idx] = x0 + h
        fp = fun(*base)
        x[idx] = x0 - h
        fm = fun(*base)
        x[idx] = x0
        g[idx] = (fp - fm) / (2 * h)
    return g


@impls
@pytest.mark.parametrize("beta_given", [False, True])
def test_gradients_match_finite_differences(impl, beta_given):
    rng = np.random.default_rng(300 + beta_given)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 2, 7, 3, 4)
    if beta_given:
        eta = rng.uniform(-0.5, 1.5, eta.shape)
    eps = 0.3
    g = IMPLS[impl](q, k, v, eta, la, eps, S0, do, dST, beta_given=beta_given)
    args = (q, k, v, eta, la, eps, S0, do, dST, beta_given)
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2), ("deta", 3), ("dlog_a", 4), ("dS0", 6)):
        fd = _fd(_loss, args, i)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


@impls
@pytest.mark.parametrize("beta_given", [False, True])
def test_equal_channels_reduce_to_the_scalar_gate(impl, beta_given):
    """log a_t[i] = log alpha_t for every channel is the scalar gate: every gradient equals the
    scalar-gate oracle's, and d log alpha_t is the sum over channels of d log a_t."""
    rng = np.random.default_rng(302)
    q, k, v, eta, _, S0, do, dST = rand_case(rng, 2, 13, 4, 3)
    la = -rng.uniform(0.0, 0.4, (2, 13))
    g = IMPLS[impl](q, k, v, eta, np.repeat(la[..., None], 4, -1), 1e-6, S0, do, dST, beta_given=beta_given)
    if beta_given:
        ref = oracle.gated_delta_vjp(q, k, v, eta, la, S0, do, dST)
        ref["deta"] = ref["dbeta"]
    else:
        ref = oracle.kla_vjp(q, k, v, eta, la, 1e-6, S0, do, dST)
    for n in ("dq", "dk", "dv", "deta", "dS0"):
        np.testing.assert_allclose(g[n], ref[n], rtol=1e-11, atol=1e-13, err_msg=n)
    np.testing.assert_allclose(g["dlog_a"].sum(-1), ref["dlog_alpha"], rtol=1e-11, atol=1e-13)


@impls
def test_pure_per_channel_decay_closed_forms(impl):
    """eta = 0: S_t = Diag(e^{c_t}) S0 with c_t[i] = sum_{j<=t} log a_j[i], o_t = S0^T (e^{c_t} o q_t).
    For L = sum_t do_t.o_t + <S_T, dS_T>: dq_t = e^{c_t} o (S0 do_t);
    dlog a_j[i] = sum_{t>=j} e^{c_t[i]} q_t[i] (S0 do_t)[i] + e^{c_T[i]} sum_m S0[i, m] dS_T[i, m];
    dS0 = sum_t (e^{c_t} o q_t) do_t^T + Diag(e^{c_T}) dS_T; dk = dv = 0."""
    rng = np.random.default_rng(303)
    q, k, v, _, la, S0, do, dST = rand_case(rng, 2, 9, 4, 3)
    eta = np.zeros((2, 9))
    g = IMPLS[impl](q, k, v, eta, la, 1e-6, S0, do, dST)
    c = np.cumsum(la, axis=1)
    ec = np.exp(c)
    Sdo = np.einsum("nij,ntj->nti", S0, do)
    per = ec * q * Sdo
    final = np.exp(c[:, -1]) * np.sum(S0 * dST, axis=2)
    dla = np.cumsum(per[:, ::-1], axis=1)[:, ::-1] + final[:, None, :]
    np.testing.assert_allclose(g["dlog_a"], dla, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g["dq"], ec * Sdo, rtol=1e-12, atol=1e-15)
    dS0 = np.einsum("nti,ntj->nij", ec * q, do) + np.exp(c[:, -1])[:, :, None] * dST
    np.testing.assert_allclose(g["dS0"], dS0, rtol=1e-12, atol=1e-15)
    assert np.abs(g["dv"]).max() == 0 and np.abs(g["dk"]).max() == 0


@impls
def test_homogeneity_identities(impl):
    """As for the scalar gate: o is linear in q, (o, S_T) jointly linear in (v, S0), and with
    eps = 0 and S0 = 0 scaling every key by c scales (o, S_T) by 1/c, so <q, dq> = <o, do>,
    <v, dv> + <S0, dS0> = L and <k, dk> = -L."""
    rng = np.random.default_rng(304)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 3, 20, 5, 4)
    beta = oracle.kaczmarz_step_size(k, eta, 1e-6)
    o, S = oracle.kda_recurrent(q, k, v, beta, la, S0)
    g = IMPLS[impl](q, k, v, eta, la, 1e-6, S0, do, dST)
    L = np.sum(o * do) + np.sum(S * dST)
    assert np.sum(q * g["dq"]) == pytest.approx(np.sum(o * do), rel=1e-11)
    assert np.sum(v * g["dv"]) + np.sum(S0 * g["dS0"]) == pytest.approx(L, rel=1e-11)
    o, S = oracle.kda_recurrent(q, k, v, oracle.kaczmarz_step_size(k, eta, 0.0), la)
    g = IMPLS[impl](q, k, v, eta, la, 0.0, None, do, dST)
    L = np.sum(o * do) + np.sum(S * dST)
    assert np.sum(k * g["dk"]) == pytest.approx(-L, rel=1e-11)


def test_implementations_agree_on_a_longer_sequence():
    """Autodiff and the hand-written adjoint on 150 tokens (the adjoint across several checkpoint
    blocks, one of them partial), with strong per-channel decays."""
    rng = np.random.default_rng(305)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 2, 150, 6, 5)
    la[:, :, 0] = -rng.uniform(2.0, 8.0, (2, 150))
    a = oracle.kda_vjp(q, k, v, eta, la, 1e-6, S0, do, dST)
    b = oracle.kda_adjoint(q, k, v, eta, la, 1e-6, S0, do, dST, block=64)
    for n in a:
        np.testing.assert_allclose(b[n], a[n], rtol=1e-10, atol=1e-12, err_msg=n)


def test_library_layout_wrapper():
    """[B, T, H, d] gradients equal the head-major ones head by head."""
    rng = np.random.default_rng(306)
    B, T, H, dk, dv = 2, 9, 3, 4, 5
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v, do = rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, T, H, dv))
    eta, la = rng.uniform(0, 1, (B, T, H)), -rng.uniform(0, 0.4, (B, T, H, dk))
    S0, dST = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, H, dk, dv))
    for beta_given in (False, True):
        g = oracle.kda_backward(q, k, v, eta, la, 1e-6, S0, do, dST, beta_given=beta_given)
        for b in range(B):
            for h in range(H):
                sl = lambda x: x[b, :, h][None]
                gh = oracle.kda_vjp(sl(q), sl(k), sl(v), sl(eta), sl(la), 1e-6, S0[b, h][None], sl(do),
                                    dST[b, h][None], beta_given=beta_given)
                for n in ("dq", "dk", "dv", "deta", "dlog_a"):
                    np.testing.assert_allclose(g[n][b, :, h], gh[n][0], rtol=1e-13, atol=1e-15, err_msg=n)
                np.testing.assert_allclose(g["dS0"][b, h], gh["dS0"][0], rtol=1e-13, atol=1e-15)


def test_planted_mistake_fails_a_pin(monkeypatch):
    """A decay applied to the state's columns instead of its rows (the orientation slip this
    layout invites when d_k = d_v) leaves the gradients wrong, and the finite-difference pin sees
    it; the real adjoint passes the same check."""
    rng = np.random.default_rng(307)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 1, 6, 3, 3)
    args = (q, k, v, eta, la, 0.3, S0, do, dST, False)
    fd = _fd(_loss, args, 4)
    right = oracle.kda_adjoint(q, k, v, eta, la, 0.3, S0, do, dST, block=4)["dlog_a"]
    np.testing.assert_allclose(right, fd, rtol=1e-6, atol=1e-7)
    step = adjoint._kda_step

    def columns(S, k_t, v_t, b_t, a_t):
        P = a_t[:, None, :] * S
        return step(P, k_t, v_t, b_t, np.ones_like(a_t))

    monkeypatch.setattr(adjoint, "_kda_step", columns)
    wrong = oracle.kda_adjoint(q, k, v, eta, la, 0.3, S0, do, dST, block=4)["dlog_a"]
    assert not np.allclose(wrong, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("block", [1, 5, 64])
def test_adjoint_block_size_only_changes_rounding(block):
    rng = np.random.default_rng(308)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 2, 23, 4, 3)
    ref = oracle.kda_adjoint(q, k, v, eta, la, 1e-6, S0, do, dST, block=23)
    g = oracle.kda_adjoint(q, k, v, eta, la, 1e-6, S0, do, dST, block=block)
    for n in ref:
        np.testing.assert_allclose(g[n], ref[n], rtol=1e-12, atol=1e-14, err_msg=n)
