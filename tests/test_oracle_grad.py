"""Pins for the fp64 gradient oracles (CPU only).

The gradients come from two implementations of the same derivative of the token loop:
reverse-mode autodiff (kla_grad, PyTorch) and the adjoint recurrence written out by hand
(adjoint, NumPy). Each is tied to things other than itself: central finite differences
of the NumPy forward oracle (itself pinned in test_oracle.py), hand-derived closed forms for a
single token and for a pure-decay sequence, and exact homogeneity identities of the recurrence.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import adjoint, kla_grad

pytestmark = pytest.mark.filterwarnings("error::RuntimeWarning")

# (KLA vjp, beta-given vjp) of each implementation; the adjoint checkpoints every 4 tokens here,
# so that the short cases below still cross several recompute blocks.
IMPLS = {
    "autodiff": (oracle.kla_vjp, oracle.gated_delta_vjp),
    "adjoint": (lambda *a: oracle.kla_adjoint(*a, block=4), lambda *a: oracle.gated_delta_adjoint(*a, block=4)),
}
impls = pytest.mark.parametrize("impl", sorted(IMPLS))


def rand_case(rng, N, T, dk, dv, la=(0.001, 0.3)):
    q = rng.standard_normal((N, T, dk)) / math.sqrt(dk)
    k = rng.standard_normal((N, T, dk)) / math.sqrt(dk) * np.exp(
        rng.uniform(math.log(0.5), math.log(2.0), (N, T, 1)))
    v = rng.standard_normal((N, T, dv))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, T))))
    la_ = -rng.uniform(la[0], la[1], (N, T))
    S0 = 0.5 * rng.standard_normal((N, dk, dv))
    do = rng.standard_normal((N, T, dv))
    dST = rng.standard_normal((N, dk, dv))
    return q, k, v, eta, la_, S0, do, dST


def _loss_kla(q, k, v, eta, la, eps, S0, do, dST):
    o, S = oracle.kla_recurrent(q, k, v, eta, la, eps, S0)
    return float(np.sum(o * do) + np.sum(S * dST))


def _loss_gdn(q, k, v, beta, la, S0, do, dST):
    o, S = oracle.gated_delta_recurrent(q, k, v, beta, la, S0)
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
@pytest.mark.parametrize("eps", [0.3, 1e-6])
def test_kla_gradients_match_finite_differences(impl, eps):
    rng = np.random.default_rng(100)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 2, 7, 3, 4)
    g = IMPLS[impl][0](q, k, v, eta, la, eps, S0, do, dST)
    args = (q, k, v, eta, la, eps, S0, do, dST)
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2), ("deta", 3), ("dlog_alpha", 4), ("dS0", 6)):
        fd = _fd(_loss_kla, args, i)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


@impls
def test_gdn_gradients_match_finite_differences(impl):
    rng = np.random.default_rng(101)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 2, 6, 4, 3)
    beta = rng.uniform(-0.5, 1.5, eta.shape)
    g = IMPLS[impl][1](q, k, v, beta, la, S0, do, dST)
    args = (q, k, v, beta, la, S0, do, dST)
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2), ("dbeta", 3), ("dlog_alpha", 4), ("dS0", 5)):
        fd = _fd(_loss_gdn, args, i)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_autodiff_loop_is_the_forward_oracle():
    """The loop that is differentiated produces the NumPy oracle's outputs."""
    import torch
    rng = np.random.default_rng(102)
    q, k, v, eta, la, S0, _, _ = rand_case(rng, 3, 40, 6, 5)
    beta = oracle.kaczmarz_step_size(k, eta, 1e-6)
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    o, S = kla_grad._loop(t(q), t(k), t(v), t(beta), t(la), t(S0))
    o_ref, S_ref = oracle.gated_delta_recurrent(q, k, v, beta, la, S0)
    np.testing.assert_allclose(o.numpy(), o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S.numpy(), S_ref, rtol=0, atol=1e-13)


@impls
def test_single_token_closed_forms(impl):
    """T = 1: o = alpha S0^T q + beta (k.q) (v - alpha S0^T k). By hand, for L = do.o:
    dq = S_1 do; dv = beta (k.q) do; dbeta = (k.q) (v - alpha S0^T k).do;
    dlog_alpha = alpha (S0^T q - beta (k.q) S0^T k).do; dS0 = alpha (q - beta (k.q) k) do^T;
    with beta fixed, dk = beta (v.do) q - alpha beta ((k.S0 do) q + (k.q) S0 do);
    KLA adds dbeta * d(beta)/dk = -2 eta k / (||k||^2 + eps)^2 and deta = dbeta / (||k||^2 + eps)."""
    rng = np.random.default_rng(103)
    dk, dv, eps = 5, 4, 0.2
    for _ in range(5):
        q, k, S0 = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal((dk, dv))
        v, do = rng.standard_normal(dv), rng.standard_normal(dv)
        eta, alpha = rng.uniform(0.1, 1), rng.uniform(0.3, 1)
        n = k @ k
        beta = eta / (n + eps)
        kq = k @ q
        S1 = alpha * S0 + beta * np.outer(k, v - alpha * S0.T @ k)
        dbeta = kq * (v - alpha * S0.T @ k) @ do
        exp = {
            "dq": S1 @ do,
            "dv": beta * kq * do,
            "deta": dbeta / (n + eps),
            "dlog_alpha": alpha * (S0.T @ q - beta * kq * S0.T @ k) @ do,
            "dS0": alpha * np.outer(q - beta * kq * k, do),
            "dk": beta * (v @ do) * q - alpha * beta * ((k @ S0 @ do) * q + kq * S0 @ do)
                  - 2 * dbeta * eta / (n + eps) ** 2 * k,
        }
        g = IMPLS[impl][0](q[None, None], k[None, None], v[None, None], np.array([[eta]]),
                           np.array([[math.log(alpha)]]), eps, S0[None], do[None, None])
        for name, val in exp.items():
            np.testing.assert_allclose(np.squeeze(g[name]), val, rtol=1e-12, atol=1e-14, err_msg=name)


@impls
def test_pure_decay_closed_forms(impl):
    """eta = 0: o_t = e^{c_t} S0^T q_t with c_t = sum_{j<=t} log alpha_j and S_T = e^{c_T} S0, so
    dlog_alpha_j = sum_{t>=j} e^{c_t} do_t.(S0^T q_t) + e^{c_T} <S0, dS_T>, dq_t = e^{c_t} S0 do_t,
    dS0 = sum_t e^{c_t} q_t do_t^T + e^{c_T} dS_T, and dv = dk = 0."""
    rng = np.random.default_rng(104)
    q, k, v, _, la, S0, do, dST = rand_case(rng, 2, 9, 4, 3)
    eta = np.zeros((2, 9))
    g = IMPLS[impl][0](q, k, v, eta, la, 1e-6, S0, do, dST)
    c = np.cumsum(la, axis=1)
    a = np.einsum("ntj,nij,nti->nt", do, S0, q)
    ec = np.exp(c)
    final = np.exp(c[:, -1]) * np.sum(S0 * dST, axis=(1, 2))
    dla = np.cumsum((ec * a)[:, ::-1], axis=1)[:, ::-1] + final[:, None]
    np.testing.assert_allclose(g["dlog_alpha"], dla, rtol=1e-12)
    np.testing.assert_allclose(g["dq"], ec[:, :, None] * np.einsum("nij,ntj->nti", S0, do), rtol=1e-12, atol=1e-15)
    dS0 = np.einsum("nt,nti,ntj->nij", ec, q, do) + np.exp(c[:, -1])[:, None, None] * dST
    np.testing.assert_allclose(g["dS0"], dS0, rtol=1e-12)
    assert np.abs(g["dv"]).max() == 0 and np.abs(g["dk"]).max() == 0


@impls
def test_homogeneity_identities(impl):
    """o is linear in q; (o, S_T) are jointly linear in (v, S0); with eps = 0 and S0 = 0,
    scaling every key by c scales (o, S_T) by 1/c. Euler's identity for each gives
    <q, dq> = <o, do>, <v, dv> + <S0, dS0> = L and <k, dk> = -L, where L = <o, do> + <S_T, dS_T>."""
    rng = np.random.default_rng(105)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 3, 30, 6, 5)
    o, S = oracle.kla_recurrent(q, k, v, eta, la, 1e-6, S0)
    g = IMPLS[impl][0](q, k, v, eta, la, 1e-6, S0, do, dST)
    L = np.sum(o * do) + np.sum(S * dST)
    assert np.sum(q * g["dq"]) == pytest.approx(np.sum(o * do), rel=1e-11)
    assert np.sum(v * g["dv"]) + np.sum(S0 * g["dS0"]) == pytest.approx(L, rel=1e-11)
    o, S = oracle.kla_recurrent(q, k, v, eta, la, 0.0)
    g = IMPLS[impl][0](q, k, v, eta, la, 0.0, None, do, dST)
    L = np.sum(o * do) + np.sum(S * dST)
    assert np.sum(k * g["dk"]) == pytest.approx(-L, rel=1e-11)


def test_library_layout_wrapper():
    """[B, T, H, d] gradients equal the head-major ones head by head; beta_given selects GDN."""
    rng = np.random.default_rng(106)
    B, T, H, dk, dv = 2, 11, 3, 4, 5
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v, do = rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, T, H, dv))
    eta, la = rng.uniform(0, 1, (B, T, H)), -rng.uniform(0, 0.2, (B, T, H))
    S0, dST = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, H, dk, dv))
    for beta_given in (False, True):
        g = oracle.kla_backward(q, k, v, eta, la, 1e-6, S0, do, dST, beta_given=beta_given)
        for b in range(B):
            for h in range(H):
                sl = lambda x: x[b, :, h][None]
                if beta_given:
                    gh = oracle.gated_delta_vjp(sl(q), sl(k), sl(v), sl(eta), sl(la), S0[b, h][None],
                                                sl(do), dST[b, h][None])
                    gh["deta"] = gh["dbeta"]
                else:
                    gh = oracle.kla_vjp(sl(q), sl(k), sl(v), sl(eta), sl(la), 1e-6, S0[b, h][None],
                                        sl(do), dST[b, h][None])
                for n in ("dq", "dk", "dv", "deta", "dlog_alpha"):
                    np.testing.assert_allclose(g[n][b, :, h], gh[n][0], rtol=1e-13, atol=1e-15, err_msg=n)
                np.testing.assert_allclose(g["dS0"][b, h], gh["dS0"][0], rtol=1e-13, atol=1e-15)


def test_planted_mistake_fails_a_pin():
    """Dropping the step size's dependence on k (beta taken as a constant) leaves dk wrong,
    and the finite-difference pin sees it; the real oracle passes the same check."""
    rng = np.random.default_rng(107)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 1, 5, 3, 3)
    eps = 0.3
    fd = _fd(_loss_kla, (q, k, v, eta, la, eps, S0, do, dST), 1)
    beta = oracle.kaczmarz_step_size(k, eta, eps)
    wrong = oracle.gated_delta_vjp(q, k, v, beta, la, S0, do, dST)["dk"]
    assert not np.allclose(wrong, fd, rtol=1e-6, atol=1e-7)
    right = oracle.kla_vjp(q, k, v, eta, la, eps, S0, do, dST)["dk"]
    np.testing.assert_allclose(right, fd, rtol=1e-6, atol=1e-7)


def test_adjoint_planted_mistake_fails_a_pin(monkeypatch):
    """States recomputed without the decay (a slip in the adjoint's forward and block recompute)
    leave the key gradients, which read those states, wrong, and the finite-difference pin sees it."""
    rng = np.random.default_rng(108)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 1, 9, 3, 3)
    fd = _fd(_loss_kla, (q, k, v, eta, la, 0.3, S0, do, dST), 1)
    right = oracle.kla_adjoint(q, k, v, eta, la, 0.3, S0, do, dST, block=4)["dk"]
    np.testing.assert_allclose(right, fd, rtol=1e-6, atol=1e-7)
    step = adjoint._step
    monkeypatch.setattr(adjoint, "_step", lambda S, q_, k_, v_, b_, a_: step(S, q_, k_, v_, b_, np.ones_like(a_)))
    wrong = oracle.kla_adjoint(q, k, v, eta, la, 0.3, S0, do, dST, block=4)["dk"]
    assert not np.allclose(wrong, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("block", [1, 5, 64])
def test_adjoint_block_size_only_changes_rounding(block):
    """The checkpoint spacing is a memory/time trade only: the gradients agree to rounding for
    block sizes that do and do not divide T."""
    rng = np.random.default_rng(109)
    q, k, v, eta, la, S0, do, dST = rand_case(rng, 2, 23, 4, 3)
    ref = oracle.kla_adjoint(q, k, v, eta, la, 1e-6, S0, do, dST, block=23)
    g = oracle.kla_adjoint(q, k, v, eta, la, 1e-6, S0, do, dST, block=block)
    for n in ref:
        np.testing.assert_allclose(g[n], ref[n], rtol=1e-12, atol=1e-14, err_msg=n)
