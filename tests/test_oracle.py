"""Pins for the fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: hand-derived values,
exact single-step identities, a brute-force unrolled product, the classical
Kaczmarz limit (pseudo-inverse), special cases with closed forms, and an
algebraic identity between KLA and Gated DeltaNet. The planted-mistake test at
the end shows that plausible slips in the recurrence each fail at least one pin.
"""
import json
import math
import pathlib

import numpy as np
import pytest

import oracle
from oracle import kla_oracle as ko

pytestmark = pytest.mark.filterwarnings("error::RuntimeWarning")

GOLDEN = pathlib.Path(__file__).parent / "golden"


def rand_heads(rng, N, T, dk, dv, la=(0.001, 0.1)):
    q = rng.standard_normal((N, T, dk)) / math.sqrt(dk)
    k = rng.standard_normal((N, T, dk)) / math.sqrt(dk) * np.exp(
        rng.uniform(math.log(0.25), math.log(4.0), (N, T, 1)))
    v = rng.standard_normal((N, T, dv))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, T))))
    log_alpha = -rng.uniform(la[0], la[1], (N, T))
    return q, k, v, eta, log_alpha


# ---------------------------------------------------------------- golden values

def test_golden_hand_examples():
    """Hand-derived d=2 recurrences (tests/golden/kla_hand_d2.json)."""
    data = json.loads((GOLDEN / "kla_hand_d2.json").read_text())
    for case in data["cases"]:
        toks = case["tokens"]
        q = np.array([[t["q"] for t in toks]], float)
        k = np.array([[t["k"] for t in toks]], float)
        v = np.array([[t["v"] for t in toks]], float)
        eta = np.array([[t["eta"] for t in toks]], float)
        la = np.log(np.array([[t["alpha"] for t in toks]], float))
        S0 = np.array([case["S0"]], float)
        o, S = oracle.kla_recurrent(q, k, v, eta, la, case["eps"], S0)
        np.testing.assert_allclose(o[0], case["expected_o"], rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(S[0], case["expected_S"], rtol=0, atol=1e-14, err_msg=case["name"])


def test_step_size_closed_forms():
    """beta = eta / (||k||^2 + eps) on keys with known norms; a zero key gives eta / eps."""
    k = np.array([[3.0, 4.0], [0.0, 0.0], [1.0, 0.0]])
    eta = np.array([0.5, 0.5, 1.0])
    np.testing.assert_allclose(oracle.kaczmarz_step_size(k[[0, 2]], eta[[0, 2]], 0.0), [0.02, 1.0], rtol=1e-15)
    np.testing.assert_allclose(oracle.kaczmarz_step_size(k, eta, 1e-6), [0.5 / (25 + 1e-6), 0.5e6, 1.0 / (1 + 1e-6)],
                               rtol=1e-15)


def test_chunk_local_decay_hand():
    """Chunk-local inclusive prefix sums restart at every chunk boundary."""
    la = np.array([-1.0, -2.0, -3.0, -4.0, -5.0])
    np.testing.assert_array_equal(oracle.chunk_local_log_decay(la, 2), [-1, -3, -3, -7, -5])
    np.testing.assert_array_equal(oracle.chunk_local_log_decay(la, 64), np.cumsum(la))


def test_prepare_beta_layout():
    rng = np.random.default_rng(1)
    B, T, H, d = 2, 70, 3, 8
    k = rng.standard_normal((B, T, H, d))
    eta = rng.uniform(0, 1, (B, T, H))
    la = -rng.uniform(0, 0.2, (B, T, H))
    beta, G = oracle.kla_prepare_beta(k, eta, la, 1e-6, 64)
    for b in range(B):
        for h in range(H):
            for t in (0, 5, 63, 64, 69):
                assert beta[b, t, h] == pytest.approx(eta[b, t, h] / (k[b, t, h] @ k[b, t, h] + 1e-6), rel=1e-14)
                c0 = (t // 64) * 64
                assert G[b, t, h] == pytest.approx(la[b, c0:t + 1, h].sum(), rel=1e-14, abs=1e-15)


# ---------------------------------------------------------------- single-step identities (P1)

def _one_step(S, k, v, q, eta, alpha, eps):
    o, S1 = oracle.kla_decode_step(q[None, None], k[None, None], v[None, None], np.array([[eta]]),
                                   np.array([[math.log(alpha)]]), eps, S[None, None])
    return o[0, 0], S1[0, 0]


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.3])
def test_residual_shrinks_along_key(eps):
    """v - S_t^T k = (1 - eta ||k||^2/(||k||^2+eps)) (v - alpha S_{t-1}^T k)."""
    rng = np.random.default_rng(2)
    for _ in range(20):
        dk, dv = 7, 5
        S = rng.standard_normal((dk, dv))
        k, q, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
        eta, alpha = rng.uniform(0, 1), rng.uniform(0.3, 1)
        _, S1 = _one_step(S, k, v, q, eta, alpha, eps)
        n = k @ k
        np.testing.assert_allclose(v - S1.T @ k, (1 - eta * n / (n + eps)) * (v - alpha * S.T @ k), atol=1e-12)


def test_only_key_direction_is_edited():
    """For x orthogonal to k_t, S_t^T x = alpha_t S_{t-1}^T x."""
    rng = np.random.default_rng(3)
    dk, dv = 9, 4
    for _ in range(20):
        S = rng.standard_normal((dk, dv))
        k, q, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
        x = rng.standard_normal(dk)
        x -= (x @ k) / (k @ k) * k
        eta, alpha = rng.uniform(0, 1), rng.uniform(0.3, 1)
        _, S1 = _one_step(S, k, v, q, eta, alpha, 1e-6)
        np.testing.assert_allclose(S1.T @ x, alpha * S.T @ x, atol=1e-12)


def test_exact_write_alpha1_eta1():
    """alpha = eta = 1, eps = 0: the new state maps k_t to v_t exactly; with eps > 0 the
    residual is eps/(||k||^2+eps) times the prior one."""
    rng = np.random.default_rng(4)
    dk, dv = 6, 6
    S = rng.standard_normal((dk, dv))
    for _ in range(20):
        k, q, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
        prior = v - S.T @ k
        _, S = _one_step(S, k, v, q, 1.0, 1.0, 0.0)
        np.testing.assert_allclose(S.T @ k, v, atol=1e-12)
        _, S2 = _one_step(S, k, 2 * v, q, 1.0, 1.0, 1e-6)
        n = k @ k
        np.testing.assert_allclose(2 * v - S2.T @ k, 1e-6 / (n + 1e-6) * (2 * v - S.T @ k), atol=1e-12)
        assert np.linalg.norm(prior) > 0


# ---------------------------------------------------------------- brute force (P2)

def brute_force_unrolled(q, k, v, eta, log_alpha, eps, S0):
    """S_t = P_{t..1} S0 + sum_s P_{t..s+1} beta_s k_s v_s^T with explicit transition matrices
    P_r = alpha_r (I - beta_r k_r k_r^T); o_t = S_t^T q_t. One head, T <= 16."""
    T, dk = k.shape
    beta = [eta[t] / (k[t] @ k[t] + eps) for t in range(T)]
    P = [math.exp(log_alpha[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    o, S_t = [], None
    for t in range(T):
        prod = np.eye(dk)
        for r in range(t, -1, -1):
            prod = prod @ P[r]
        S_t = prod @ S0
        for s in range(t + 1):
            prod = np.eye(dk)
            for r in range(t, s, -1):
                prod = prod @ P[r]
            S_t = S_t + prod @ (beta[s] * np.outer(k[s], v[s]))
        o.append(S_t.T @ q[t])
    return np.array(o), S_t


@pytest.mark.parametrize("T,dk,dv", [(1, 4, 3), (5, 6, 2), (16, 8, 8), (16, 3, 7)])
def test_brute_force_products(T, dk, dv):
    rng = np.random.default_rng(5 + T)
    q, k, v, eta, la = rand_heads(rng, 1, T, dk, dv, la=(0.0, 0.5))
    S0 = rng.standard_normal((1, dk, dv))
    o, S = oracle.kla_recurrent(q, k, v, eta, la, 1e-6, S0)
    ob, Sb = brute_force_unrolled(q[0], k[0], v[0], eta[0], la[0], 1e-6, S0[0])
    np.testing.assert_allclose(o[0], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0], Sb, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- classical Kaczmarz (P4)

def test_cyclic_kaczmarz_converges_to_min_norm_solution():
    """alpha = eta = 1, eps = 0, S0 = 0 and n <= d_k independent keys fed cyclically:
    the state converges to the minimum-norm solution of S^T k_i = v_i, i.e. pinv(K) V."""
    rng = np.random.default_rng(6)
    n, dk, dv, sweeps = 5, 8, 3, 600
    K = rng.standard_normal((n, dk))
    V = rng.standard_normal((n, dv))
    idx = np.tile(np.arange(n), sweeps)
    T = idx.size
    q = np.zeros((1, T, dk))
    _, S = oracle.kla_recurrent(q, K[idx][None], V[idx][None], np.ones((1, T)), np.zeros((1, T)), 0.0)
    np.testing.assert_allclose(S[0], np.linalg.pinv(K) @ V, atol=1e-10)


# ---------------------------------------------------------------- special cases (P5, P6, zero key)

def test_eta_zero_is_pure_decay():
    rng = np.random.default_rng(7)
    q, k, v, _, la = rand_heads(rng, 2, 40, 6, 5)
    S0 = rng.standard_normal((2, 6, 5))
    o, S = oracle.kla_recurrent(q, k, v, np.zeros((2, 40)), la, 1e-6, S0)
    decay = np.exp(np.cumsum(la, axis=1))
    np.testing.assert_allclose(S, decay[:, -1, None, None] * S0, rtol=1e-12)
    np.testing.assert_allclose(o, decay[:, :, None] * np.einsum("nij,nti->ntj", S0, q), rtol=1e-12, atol=1e-14)


def test_orthogonal_keys_perfect_recall():
    """alpha = eta = 1, eps = 0, S0 = 0, orthogonal keys of any norms: S_T^T k_s = v_s for all s,
    and a query equal to an earlier key reads back its value."""
    rng = np.random.default_rng(8)
    dk, dv, T = 10, 4, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = (Qm.T * rng.uniform(0.5, 3.0, (dk, 1)))[:T]
    vals = rng.standard_normal((T, dv))
    queries = np.stack([keys[t // 2] for t in range(T)])
    o, S = oracle.kla_recurrent(queries[None], keys[None], vals[None], np.ones((1, T)), np.zeros((1, T)), 0.0)
    np.testing.assert_allclose(keys @ S[0], vals, atol=1e-12)
    np.testing.assert_allclose(o[0], np.stack([vals[t // 2] for t in range(T)]), atol=1e-12)


def test_zero_key_token_is_finite_and_only_decays():
    rng = np.random.default_rng(9)
    q, k, v, eta, la = rand_heads(rng, 1, 6, 5, 3)
    k[0, 3] = 0.0
    S0 = rng.standard_normal((1, 5, 3))
    _, S_before = oracle.kla_recurrent(q[:, :3], k[:, :3], v[:, :3], eta[:, :3], la[:, :3], 1e-6, S0)
    o4, S_after = oracle.kla_recurrent(q[:, 3:4], k[:, 3:4], v[:, 3:4], eta[:, 3:4], la[:, 3:4], 1e-6, S_before)
    assert np.all(np.isfinite(S_after))
    np.testing.assert_allclose(S_after, math.exp(la[0, 3]) * S_before, rtol=1e-15)
    np.testing.assert_allclose(o4[0, 0], S_after[0].T @ q[0, 3], rtol=1e-14)


# ---------------------------------------------------------------- KLA == GDN identity (P7)

def test_kla_equals_gdn_on_balanced_inputs():
    """KLA on (k, v, eta, eps) is Gated DeltaNet with beta = eta on k/sqrt(||k||^2+eps),
    v/sqrt(||k||^2+eps); with unit keys and eps = 0, KLA is GDN with beta = eta
    ("Kaczmarz Linear Attention", Abstract: a one-scalar modification of GDN)."""
    rng = np.random.default_rng(10)
    q, k, v, eta, la = rand_heads(rng, 3, 50, 8, 6)
    eps = 0.05
    o, S = oracle.kla_recurrent(q, k, v, eta, la, eps)
    r = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    o2, S2 = oracle.gated_delta_recurrent(q, k / r, v / r, eta, la)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(S, S2, atol=1e-12)
    ku = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o3, _ = oracle.kla_recurrent(q, ku, v, eta, la, 0.0)
    o4, _ = oracle.gated_delta_recurrent(q, ku, v, eta, la)
    np.testing.assert_allclose(o3, o4, atol=1e-12)


# ---------------------------------------------------------------- chunkwise form (P3, P8)

@pytest.mark.parametrize("T,chunk", [(64, 64), (37, 64), (150, 64), (130, 16), (128, 32)])
def test_chunked_matches_token_loop(T, chunk):
    rng = np.random.default_rng(11 + T)
    q, k, v, eta, la = rand_heads(rng, 2, T, 12, 9, la=(0.0, 0.3))
    S0 = 0.1 * rng.standard_normal((2, 12, 9))
    o, S = oracle.kla_recurrent(q, k, v, eta, la, 1e-6, S0)
    oc, Sc = oracle.kla_chunked(q, k, v, eta, la, 1e-6, S0, chunk)
    np.testing.assert_allclose(oc, o, atol=1e-11, rtol=0)
    np.testing.assert_allclose(Sc, S, atol=1e-11, rtol=0)


def test_state_passing_splits():
    """fwd(T1) then fwd(T2 | S_T1) equals fwd(T1 + T2): only the state crosses the split."""
    rng = np.random.default_rng(12)
    q, k, v, eta, la = rand_heads(rng, 2, 200, 8, 8)
    o, S = oracle.kla_recurrent(q, k, v, eta, la, 1e-6)
    o1, S1 = oracle.kla_chunked(q[:, :77], k[:, :77], v[:, :77], eta[:, :77], la[:, :77], 1e-6, None, 32)
    o2, S2 = oracle.kla_chunked(q[:, 77:], k[:, 77:], v[:, 77:], eta[:, 77:], la[:, 77:], 1e-6, S1, 64)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, atol=1e-11)
    np.testing.assert_allclose(S2, S, atol=1e-11)


def test_layouts_and_decode_steps_agree():
    """Library-layout wrappers ([B,T,H,d], [steps,B,H,d]) reproduce the head-major loop."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 2, 9, 3, 5, 4
    q, k, v, eta, la = (rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk)),
                        rng.standard_normal((B, T, H, dv)), rng.uniform(0, 1, (B, T, H)),
                        -rng.uniform(0, 0.2, (B, T, H)))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = oracle.kla_forward(q, k, v, eta, la, 1e-6, S0)
    for b in range(B):
        for h in range(H):
            oh, Sh = oracle.kla_recurrent(q[b, :, h][None], k[b, :, h][None], v[b, :, h][None],
                                          eta[b, :, h][None], la[b, :, h][None], 1e-6, S0[b, h][None])
            np.testing.assert_allclose(o[b, :, h], oh[0], rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(S[b, h], Sh[0], rtol=1e-14, atol=1e-14)
    sw = lambda x: np.moveaxis(x, 1, 0)  # [B,T,H,...] -> [T,B,H,...]
    od, Sd = oracle.kla_decode_steps(sw(q), sw(k), sw(v), sw(eta), sw(la), 1e-6, S0)
    np.testing.assert_allclose(sw(od), o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(Sd, S, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- planted mistakes

def _mutant(kind):
    """Copies of the token loop with one plausible slip planted (CPU only)."""
    def run(q, k, v, eta, log_alpha, eps, S0=None):
        N, T, dk = k.shape
        dv = v.shape[-1]
        S = np.zeros((N, dk, dv)) if S0 is None else np.array(S0, float)
        o = np.empty((N, T, dv))
        for t in range(T):
            kt, qt = k[:, t], q[:, t]
            nrm = np.sum(kt * kt, -1)
            beta = eta[:, t] / (np.sqrt(nrm) + eps if kind == "norm_not_squared" else nrm + eps)
            a = np.exp(log_alpha[:, t])
            if kind != "no_decay":
                S = S * a[:, None, None]
            if kind == "output_before_write":
                o[:, t] = np.einsum("nij,ni->nj", S, qt)
            u = np.einsum("nji,ni->nj", S, kt) if kind == "transposed_recall" else np.einsum("nij,ni->nj", S, kt)
            sign = 1.0 if kind == "wrong_sign" else -1.0
            S = S + beta[:, None, None] * kt[:, :, None] * (v[:, t] + sign * u)[:, None, :]
            if kind == "decay_after_write":
                S = S * a[:, None, None]
            if kind != "output_before_write":
                o[:, t] = np.einsum("nij,ni->nj", S, qt)
        return o, S
    return run


@pytest.mark.parametrize("kind", ["no_decay", "output_before_write", "transposed_recall", "wrong_sign",
                                  "decay_after_write", "norm_not_squared"])
def test_planted_mistakes_fail_a_pin(kind):
    mutant = _mutant(kind)
    rng = np.random.default_rng(14)
    q, k, v, eta, la = rand_heads(rng, 1, 8, 5, 5, la=(0.05, 0.5))
    S0 = rng.standard_normal((1, 5, 5))
    o, S = mutant(q, k, v, eta, la, 1e-6, S0)
    ob, Sb = brute_force_unrolled(q[0], k[0], v[0], eta[0], la[0], 1e-6, S0[0])
    assert not (np.allclose(o[0], ob, atol=1e-9) and np.allclose(S[0], Sb, atol=1e-9))
    # the real oracle passes the very same check
    o, S = oracle.kla_recurrent(q, k, v, eta, la, 1e-6, S0)
    assert np.allclose(o[0], ob, atol=1e-12) and np.allclose(S[0], Sb, atol=1e-12)
