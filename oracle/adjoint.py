"""fp64 reverse pass of the KLA token loop, written out by hand in NumPy — test infrastructure only.

Imported only by the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg. Nothing here is shared with the HIP library.

It computes the same gradients as ``kla_grad`` (reverse-mode autodiff of the token loop, in
PyTorch), for the same loss L = sum(dO * O) + sum(dS_T * S_T), but as the adjoint recurrence of
that loop: linear memory in T and no autodiff graph, so every head of a long sequence can be
checked (the autodiff graph of one 4096-token head holds gigabytes). The pages give no backward
formulas ("Kaczmarz Linear Attention", Abstract: the chunkwise form serves training); the
gradient is the plain derivative of the token loop of "Deep Dive into KDA", section 2.2, in the
[d_k, d_v] state orientation of ``kla_oracle``.

Forward step t (state P, S of shape [d_k, d_v]):
    P = alpha_t S_{t-1};   u = P^T k_t;   e = v_t - u;   S_t = P + beta_t k_t e^T;   o_t = S_t^T q_t
Reverse step t, with G = dL/dS_t on entry (dS_T at t = T):
    G   += q_t do_t^T                        (the read o_t = S_t^T q_t)
    dq_t = S_t do_t
    dbeta_t = k_t^T G e;  dk_t = beta_t G e;  de = beta_t G^T k_t      (the write)
    dv_t = de;  du = -de
    dP = G + k_t du^T;  dk_t += P du                                   (the recall u = P^T k_t)
    dlog_alpha_t = <P, dP>;  dL/dS_{t-1} = alpha_t dP                  (the decay)
With the Kaczmarz step beta_t = eta_t / (||k_t||^2 + eps) ("Kaczmarz Linear Attention",
Abstract): deta_t = dbeta_t / (||k_t||^2 + eps) and dk_t += -2 eta_t dbeta_t k_t / (||k_t||^2 + eps)^2.

The states entering the tokens are recomputed block by block from checkpoints taken every
``block`` tokens during a first forward pass (the same loop as ``gated_delta_recurrent``).

The per-channel decay of KDA ("Deep Dive into KDA", section 2.3: P = Diag(a_t) S_{t-1}, the
rows that the keys index) changes only the decay's two lines of the reverse step:
    dlog_a_t[i] = sum_j P[i, j] dP[i, j];   dL/dS_{t-1} = Diag(a_t) dP     (kda_adjoint)

Pinned in tests/test_oracle_grad.py (KDA: tests/test_oracle_kda_grad.py) by the same pins as
the autodiff oracle: central finite differences of the NumPy forward oracle, single-token and
pure-decay closed forms and the homogeneity identities, plus a planted mistake.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _step(S, q_t, k_t, v_t, beta_t, alpha_t):
    """One token of the loop from S_{t-1}: returns (P, e, S_t)."""
    P = alpha_t[:, None, None] * S
    u = np.einsum("nij,ni->nj", P, k_t)
    e = v_t - u
    S_t = P + beta_t[:, None, None] * (k_t[:, :, None] * e[:, None, :])
    return P, e, S_t


def gated_delta_adjoint(q, k, v, beta, log_alpha, S0, do, dST=None, block=64):
    """Gradients of L = sum(do * o) + sum(dST * S_T) through ``gated_delta_recurrent`` (beta given),
    head-major: q, k [N, T, d_k]; v, do [N, T, d_v]; beta, log_alpha [N, T]; S0, dST [N, d_k, d_v]
    or None (zeros). Returns dq, dk, dv, dbeta, dlog_alpha, dS0 (fp64)."""
    q, k, v, beta, log_alpha, do = map(_f64, (q, k, v, beta, log_alpha, do))
    N, T, dk = k.shape
    dv = v.shape[-1]
    alpha = np.exp(log_alpha)
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    ckpt = []
    for t in range(T):
        if t % block == 0:
            ckpt.append(S.copy())
        S = _step(S, q[:, t], k[:, t], v[:, t], beta[:, t], alpha[:, t])[2]
    G = np.zeros((N, dk, dv)) if dST is None else _f64(dST).copy()
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbeta, dla = np.zeros((N, T)), np.zeros((N, T))
    for b0 in reversed(range(0, T, block)):
        b1 = min(b0 + block, T)
        entering = [ckpt[b0 // block]]
        for t in range(b0, b1 - 1):
            entering.append(_step(entering[-1], q[:, t], k[:, t], v[:, t], beta[:, t], alpha[:, t])[2])
        for t in reversed(range(b0, b1)):
            kt, bt = k[:, t], beta[:, t]
            P, e, S_t = _step(entering[t - b0], q[:, t], kt, v[:, t], bt, alpha[:, t])
            G = G + q[:, t][:, :, None] * do[:, t][:, None, :]
            dq[:, t] = np.einsum("nij,nj->ni", S_t, do[:, t])
            Ge = np.einsum("nij,nj->ni", G, e)
            dbeta[:, t] = np.einsum("ni,ni->n", kt, Ge)
            de = bt[:, None] * np.einsum("nij,ni->nj", G, kt)
            dv_[:, t] = de
            du = -de
            dP = G + kt[:, :, None] * du[:, None, :]
            dk_[:, t] = bt[:, None] * Ge + np.einsum("nij,nj->ni", P, du)
            dla[:, t] = np.einsum("nij,nij->n", P, dP)
            G = alpha[:, t][:, None, None] * dP
    return {"dq": dq, "dk": dk_, "dv": dv_, "dbeta": dbeta, "dlog_alpha": dla, "dS0": G}


def kla_adjoint(q, k, v, eta, log_alpha, eps, S0, do, dST=None, block=64):
    """KLA gradients, head-major: the gated delta rule's adjoint with beta = eta / (||k||^2 + eps),
    plus the step size's dependence on eta and k. Returns dq, dk, dv, deta, dlog_alpha, dS0."""
    k = _f64(k)
    den = np.sum(k * k, axis=-1) + float(eps)
    eta = _f64(eta)
    g = gated_delta_adjoint(q, k, v, eta / den, log_alpha, S0, do, dST, block)
    dbeta = g.pop("dbeta")
    g["deta"] = dbeta / den
    g["dk"] = g["dk"] - (2.0 * eta * dbeta / den ** 2)[..., None] * k
    return g


def _kda_step(S, k_t, v_t, beta_t, a_t):
    """One token of the per-channel-decay loop from S_{t-1}: returns (P, e, S_t)."""
    P = a_t[:, :, None] * S
    u = np.einsum("nij,ni->nj", P, k_t)
    e = v_t - u
    S_t = P + beta_t[:, None, None] * (k_t[:, :, None] * e[:, None, :])
    return P, e, S_t


def kda_adjoint(q, k, v, eta, log_a, eps, S0, do, dST=None, block=64, beta_given=False):
    """Gradients of L = sum(do * o) + sum(dST * S_T) through ``kda_recurrent``, head-major:
    q, k [N, T, d_k]; v, do [N, T, d_v]; eta [N, T]; log_a [N, T, d_k]; S0, dST [N, d_k, d_v] or
    None. The step is beta = eta / (||k||^2 + eps) unless ``beta_given`` (eta is beta). Returns
    dq, dk, dv, deta (d beta when beta_given), dlog_a [N, T, d_k] and dS0 (fp64)."""
    q, k, v, eta, log_a, do = map(_f64, (q, k, v, eta, log_a, do))
    N, T, dk = k.shape
    dv = v.shape[-1]
    den = np.sum(k * k, axis=-1) + float(eps)
    beta = eta if beta_given else eta / den
    a = np.exp(log_a)
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    ckpt = []
    for t in range(T):
        if t % block == 0:
            ckpt.append(S.copy())
        S = _kda_step(S, k[:, t], v[:, t], beta[:, t], a[:, t])[2]
    G = np.zeros((N, dk, dv)) if dST is None else _f64(dST).copy()
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbeta, dla = np.zeros((N, T)), np.zeros((N, T, dk))
    for b0 in reversed(range(0, T, block)):
        b1 = min(b0 + block, T)
        entering = [ckpt[b0 // block]]
        for t in range(b0, b1 - 1):
            entering.append(_kda_step(entering[-1], k[:, t], v[:, t], beta[:, t], a[:, t])[2])
        for t in reversed(range(b0, b1)):
            kt, bt = k[:, t], beta[:, t]
            P, e, S_t = _kda_step(entering[t - b0], kt, v[:, t], bt, a[:, t])
            G = G + q[:, t][:, :, None] * do[:, t][:, None, :]
            dq[:, t] = np.einsum("nij,nj->ni", S_t, do[:, t])
            Ge = np.einsum("nij,nj->ni", G, e)
            dbeta[:, t] = np.einsum("ni,ni->n", kt, Ge)
            de = bt[:, None] * np.einsum("nij,ni->nj", G, kt)
            dv_[:, t] = de
            dP = G - kt[:, :, None] * de[:, None, :]
            dk_[:, t] = bt[:, None] * Ge - np.einsum("nij,nj->ni", P, de)
            dla[:, t] = np.einsum("nij,nij->ni", P, dP)
            G = a[:, t][:, :, None] * dP
    out = {"dq": dq, "dk": dk_, "dv": dv_, "dlog_a": dla, "dS0": G}
    if beta_given:
        out["deta"] = dbeta
    else:
        out["deta"] = dbeta / den
        out["dk"] = dk_ - (2.0 * eta * dbeta / den ** 2)[..., None] * k
    return out
