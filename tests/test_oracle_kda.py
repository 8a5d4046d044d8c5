"""Pins for the per-channel (KDA) decay in the fp64 oracle (CPU only): reduction to the pinned
scalar-gate oracle, a brute-force product of explicit transition matrices, closed forms for
pure decay and for the residual along the key, and the chunkwise form against the loop."""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("error::RuntimeWarning")


def rand(rng, N, T, dk, dv, lo=0.001, hi=0.3):
    q = rng.standard_normal((N, T, dk)) / math.sqrt(dk)
    k = rng.standard_normal((N, T, dk)) / math.sqrt(dk) * np.exp(rng.uniform(-1.4, 1.4, (N, T, 1)))
    v = rng.standard_normal((N, T, dv))
    beta = rng.uniform(0.05, 1.0, (N, T)) / np.sum(k * k, -1)
    log_a = -rng.uniform(lo, hi, (N, T, dk))
    return q, k, v, beta, log_a


def test_equal_channels_reduce_to_the_scalar_gate():
    """Diag(a_t) with every channel equal to alpha_t is the scalar-gated delta rule."""
    rng = np.random.default_rng(300)
    q, k, v, beta, log_a = rand(rng, 2, 40, 6, 5)
    la = log_a[:, :, 0]
    S0 = rng.standard_normal((2, 6, 5))
    o, S = oracle.kda_recurrent(q, k, v, beta, np.repeat(la[:, :, None], 6, axis=2), S0)
    o2, S2 = oracle.gated_delta_recurrent(q, k, v, beta, la, S0)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, S2, rtol=0, atol=1e-13)


def test_brute_force_transition_products():
    """S_t = P_t .. P_1 S0 + sum_s P_t .. P_{s+1} beta_s k_s v_s^T with explicit
    P_r = (I - beta_r k_r k_r^T) Diag(a_r); o_t = S_t^T q_t (T <= 12)."""
    rng = np.random.default_rng(301)
    T, dk, dv = 12, 5, 4
    q, k, v, beta, log_a = rand(rng, 1, T, dk, dv, 0.0, 0.8)
    S0 = rng.standard_normal((dk, dv))
    P = [(np.eye(dk) - beta[0, r] * np.outer(k[0, r], k[0, r])) @ np.diag(np.exp(log_a[0, r])) for r in range(T)]
    o_ref = []
    for t in range(T):
        S_t = S0.copy()
        for r in range(t + 1):
            S_t = P[r] @ S_t + beta[0, r] * np.outer(k[0, r], v[0, r])
        o_ref.append(S_t.T @ q[0, t])
    o, S = oracle.kda_recurrent(q, k, v, beta, log_a, S0[None])
    np.testing.assert_allclose(o[0], np.array(o_ref), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0], S_t, rtol=0, atol=1e-12)


def test_pure_per_channel_decay():
    """beta = 0: S_T = Diag(exp(sum_t log a_t)) S0, o_t = (exp(c_t) o S0-rows)^T q_t."""
    rng = np.random.default_rng(302)
    q, k, v, _, log_a = rand(rng, 2, 30, 7, 3)
    S0 = rng.standard_normal((2, 7, 3))
    o, S = oracle.kda_recurrent(q, k, v, np.zeros((2, 30)), log_a, S0)
    c = np.cumsum(log_a, axis=1)
    np.testing.assert_allclose(S, np.exp(c[:, -1])[:, :, None] * S0, rtol=1e-12)
    np.testing.assert_allclose(o, np.einsum("nti,nij,nti->ntj", np.exp(c), S0, q), rtol=1e-11, atol=1e-14)


def test_residual_along_the_key():
    """v - S_t^T k = (1 - beta ||k||^2) (v - (Diag(a) S_{t-1})^T k); with the Kaczmarz step and
    eta = 1, eps = 0 the new state maps k to v exactly."""
    rng = np.random.default_rng(303)
    dk, dv = 6, 4
    for _ in range(10):
        S = rng.standard_normal((dk, dv))
        k, q, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
        la = -rng.uniform(0, 1, dk)
        beta = rng.uniform(0, 1) / (k @ k)
        _, S1 = oracle.kda_recurrent(q[None, None], k[None, None], v[None, None], np.array([[beta]]),
                                     la[None, None], S[None])
        prior = v - (np.exp(la)[:, None] * S).T @ k
        np.testing.assert_allclose(v - S1[0].T @ k, (1 - beta * (k @ k)) * prior, atol=1e-12)
        _, S2 = oracle.kda_recurrent(q[None, None], k[None, None], v[None, None], np.array([[1 / (k @ k)]]),
                                     la[None, None], S[None])
        np.testing.assert_allclose(S2[0].T @ k, v, atol=1e-12)


@pytest.mark.parametrize("T,chunk", [(64, 64), (150, 64), (37, 16), (200, 32)])
def test_chunked_kda_matches_the_loop(T, chunk):
    rng = np.random.default_rng(304 + T)
    q, k, v, beta, log_a = rand(rng, 2, T, 9, 7, 0.0, 0.5)
    S0 = 0.1 * rng.standard_normal((2, 9, 7))
    o, S = oracle.kda_recurrent(q, k, v, beta, log_a, S0)
    oc, Sc = oracle.kda_chunked(q, k, v, beta, log_a, S0, chunk)
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(Sc, S, rtol=0, atol=1e-11)


def test_strong_decay_chunked_stays_finite():
    """log a down to -8 per token and channel (exp(-8 * 64) underflows): the ratio form never
    divides by a decayed prefix, so the chunked model stays finite and equal to the loop."""
    rng = np.random.default_rng(305)
    q, k, v, beta, log_a = rand(rng, 1, 128, 8, 4, 0.0, 8.0)
    o, S = oracle.kda_recurrent(q, k, v, beta, log_a)
    oc, Sc = oracle.kda_chunked(q, k, v, beta, log_a)
    assert np.isfinite(oc).all()
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-11)


def test_library_layout_and_kaczmarz_step():
    rng = np.random.default_rng(306)
    B, T, H, dk, dv = 2, 9, 3, 5, 4
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    eta, log_a = rng.uniform(0, 1, (B, T, H)), -rng.uniform(0, 0.3, (B, T, H, dk))
    o, S = oracle.kda_forward(q, k, v, eta, log_a, 1e-6)
    for b in range(B):
        for h in range(H):
            sl = lambda x: x[b, :, h][None]
            beta = oracle.kaczmarz_step_size(sl(k), sl(eta), 1e-6)
            oh, Sh = oracle.kda_recurrent(sl(q), sl(k), sl(v), beta, sl(log_a))
            np.testing.assert_allclose(o[b, :, h], oh[0], rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(S[b, h], Sh[0], rtol=1e-14, atol=1e-14)
    o2, _ = oracle.kda_forward(q, k, v, eta, log_a, 0.0, beta_given=True)
    ref, _ = oracle.kda_recurrent(np.moveaxis(q, 2, 1).reshape(B * H, T, dk), np.moveaxis(k, 2, 1).reshape(B * H, T, dk),
                                  np.moveaxis(v, 2, 1).reshape(B * H, T, dv), np.moveaxis(eta, 2, 1).reshape(B * H, T),
                                  np.moveaxis(log_a, 2, 1).reshape(B * H, T, dk))
    np.testing.assert_allclose(np.moveaxis(o2, 1, 2).reshape(B * H, T, dv), ref, rtol=1e-14, atol=1e-14)
