"""fp64 gradients of the KLA recurrence — test infrastructure only.

Imported only by the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg. Nothing here is shared with the HIP library.

The chunkwise form is "used for prefill and training" ("Kaczmarz Linear Attention",
Abstract, and the KDA pages' section 3), and training needs the reverse pass. The
pages give no backward formulas, so the definition is plain: the gradient of a
scalar loss through the very token loop of ``kla_oracle.gated_delta_recurrent``,

    L = sum(dO * O) + sum(dS_T * S_T),

taken by reverse-mode automatic differentiation of that loop, written out again here
with CPU PyTorch operations in float64 (PyTorch's autograd is the library primitive;
the loop itself is the same three lines per token: decay, recall, write, then read).

The tests pin these gradients without calling back into this module alone: central
finite differences of the NumPy forward oracle, closed forms for one token and for a
pure-decay sequence, and homogeneity identities of the recurrence (o is linear in q;
(o, S_T) are jointly linear in (v, S_0); with eps = 0 and S_0 = 0 they scale as 1/c
when every key is scaled by c).

The per-channel decay of KDA ("Deep Dive into KDA", section 2.3) is differentiated the same
way, through the loop of ``kla_oracle.kda_recurrent`` (``kda_vjp``, ``kda_backward``).

Layouts follow ``kla_oracle``: head-major [N, T, d] inside, library layout
[B, T, H, d] (state [B, H, d_k, d_v]) in the wrappers.
"""
from __future__ import annotations

import numpy as np


def _torch():
    # Imported on first use, so that importing the oracle package does not load PyTorch.
    import torch
    return torch


def _t(x):
    torch = _torch()
    return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=True)


def _loop(q, k, v, beta, log_alpha, S0):
    """The token recurrence ("Deep Dive into KDA", section 2.2, state stored [d_k, d_v]):
    S <- alpha_t S;  u = S^T k_t;  S <- S + beta_t k_t (v_t - u)^T;  o_t = S^T q_t."""
    torch = _torch()
    T = k.shape[1]
    alpha = torch.exp(log_alpha)
    S = S0
    outs = []
    for t in range(T):
        kt = k[:, t]
        S = alpha[:, t, None, None] * S
        u = torch.einsum("nij,ni->nj", S, kt)
        S = S + beta[:, t, None, None] * (kt[:, :, None] * (v[:, t] - u)[:, None, :])
        outs.append(torch.einsum("nij,ni->nj", S, q[:, t]))
    o = torch.stack(outs, 1) if outs else torch.zeros(v.shape, dtype=torch.float64)
    return o, S


def gated_delta_vjp(q, k, v, beta, log_alpha, S0, do, dST=None):
    """Gradients of L = sum(do * o) + sum(dST * S_T) for the gated delta rule with a given
    per-token beta, head-major: q, k [N, T, d_k]; v, do [N, T, d_v]; beta, log_alpha [N, T];
    S0, dST [N, d_k, d_v] or None (zeros). Returns a dict of fp64 arrays:
    dq, dk, dv, dbeta, dlog_alpha, dS0."""
    torch = _torch()
    N, T, dk = np.shape(k)
    dv = np.shape(v)[-1]
    q_, k_, v_, b_, la_ = map(_t, (q, k, v, beta, log_alpha))
    S0_ = _t(np.zeros((N, dk, dv)) if S0 is None else S0)
    o, S = _loop(q_, k_, v_, b_, la_, S0_)
    loss = (o * torch.as_tensor(np.asarray(do, np.float64))).sum()
    if dST is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dST, np.float64))).sum()
    grads = torch.autograd.grad(loss, (q_, k_, v_, b_, la_, S0_), allow_unused=True)
    names = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dS0")
    shapes = ((N, T, dk), (N, T, dk), (N, T, dv), (N, T), (N, T), (N, dk, dv))
    return {n: (np.zeros(s) if g is None else g.numpy()) for n, g, s in zip(names, grads, shapes)}


def kla_vjp(q, k, v, eta, log_alpha, eps, S0, do, dST=None):
    """KLA gradients, head-major. beta_t = eta_t / (||k_t||^2 + eps) ("Kaczmarz Linear
    Attention", Abstract) is formed inside the differentiated graph, so dk includes the
    path through the step size. Returns dq, dk, dv, deta, dlog_alpha, dS0."""
    torch = _torch()
    N, T, dk = np.shape(k)
    dv = np.shape(v)[-1]
    q_, k_, v_, e_, la_ = map(_t, (q, k, v, eta, log_alpha))
    S0_ = _t(np.zeros((N, dk, dv)) if S0 is None else S0)
    beta = e_ / ((k_ * k_).sum(-1) + float(eps))
    o, S = _loop(q_, k_, v_, beta, la_, S0_)
    loss = (o * torch.as_tensor(np.asarray(do, np.float64))).sum()
    if dST is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dST, np.float64))).sum()
    grads = torch.autograd.grad(loss, (q_, k_, v_, e_, la_, S0_), allow_unused=True)
    names = ("dq", "dk", "dv", "deta", "dlog_alpha", "dS0")
    shapes = ((N, T, dk), (N, T, dk), (N, T, dv), (N, T), (N, T), (N, dk, dv))
    return {n: (np.zeros(s) if g is None else g.numpy()) for n, g, s in zip(names, grads, shapes)}


def _to_heads(x):
    x = np.asarray(x)
    B, T, H = x.shape[:3]
    return np.moveaxis(x, 2, 1).reshape((B * H, T) + x.shape[3:])


def _from_heads(x, B, H):
    T = x.shape[1]
    return np.moveaxis(x.reshape((B, H, T) + x.shape[2:]), 1, 2)


def kla_backward(q, k, v, eta, log_alpha, eps, S0, do, dST=None, beta_given=False):
    """Library-layout gradients: q, k [B, T, H, d_k]; v, do [B, T, H, d_v]; eta (or beta when
    ``beta_given``), log_alpha [B, T, H]; S0, dST [B, H, d_k, d_v] or None.
    Returns dq, dk [B, T, H, d_k], dv [B, T, H, d_v], deta (dbeta when ``beta_given``),
    dlog_alpha [B, T, H] and dS0 [B, H, d_k, d_v], all fp64."""
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    s0 = None if S0 is None else np.asarray(S0, np.float64).reshape(B * H, dk, dv)
    dst = None if dST is None else np.asarray(dST, np.float64).reshape(B * H, dk, dv)
    args = (_to_heads(q), _to_heads(k), _to_heads(v), _to_heads(eta), _to_heads(log_alpha))
    if beta_given:
        g = gated_delta_vjp(*args, s0, _to_heads(do), dst)
        g["deta"] = g.pop("dbeta")
    else:
        g = kla_vjp(*args, eps, s0, _to_heads(do), dst)
    out = {n: _from_heads(g[n], B, H) for n in ("dq", "dk", "dv", "deta", "dlog_alpha")}
    out["dS0"] = g["dS0"].reshape(B, H, dk, dv)
    return out


def _kda_loop(q, k, v, beta, log_a, S0):
    """The token recurrence with the per-channel decay ("Deep Dive into KDA", section 2.3, state
    stored [d_k, d_v], so Diag(a_t) scales the rows the keys index):
    S <- Diag(a_t) S;  u = S^T k_t;  S <- S + beta_t k_t (v_t - u)^T;  o_t = S^T q_t."""
    torch = _torch()
    T = k.shape[1]
    a = torch.exp(log_a)
    S = S0
    outs = []
    for t in range(T):
        kt = k[:, t]
        S = a[:, t, :, None] * S
        u = torch.einsum("nij,ni->nj", S, kt)
        S = S + beta[:, t, None, None] * (kt[:, :, None] * (v[:, t] - u)[:, None, :])
        outs.append(torch.einsum("nij,ni->nj", S, q[:, t]))
    o = torch.stack(outs, 1) if outs else torch.zeros(v.shape, dtype=torch.float64)
    return o, S


def kda_vjp(q, k, v, eta, log_a, eps, S0, do, dST=None, beta_given=False):
    """Gradients of L = sum(do * o) + sum(dST * S_T) through the per-channel-decay loop,
    head-major: q, k [N, T, d_k]; v, do [N, T, d_v]; eta [N, T]; log_a [N, T, d_k];
    S0, dST [N, d_k, d_v] or None (zeros). The step is beta = eta / (||k||^2 + eps), formed inside
    the differentiated graph, unless ``beta_given`` (eta is then beta itself and eps unused).
    Returns dq, dk, dv, deta (d beta when beta_given), dlog_a [N, T, d_k] and dS0, fp64."""
    torch = _torch()
    N, T, dk = np.shape(k)
    dv = np.shape(v)[-1]
    q_, k_, v_, e_, la_ = map(_t, (q, k, v, eta, log_a))
    S0_ = _t(np.zeros((N, dk, dv)) if S0 is None else S0)
    beta = e_ if beta_given else e_ / ((k_ * k_).sum(-1) + float(eps))
    o, S = _kda_loop(q_, k_, v_, beta, la_, S0_)
    loss = (o * torch.as_tensor(np.asarray(do, np.float64))).sum()
    if dST is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dST, np.float64))).sum()
    grads = torch.autograd.grad(loss, (q_, k_, v_, e_, la_, S0_), allow_unused=True)
    names = ("dq", "dk", "dv", "deta", "dlog_a", "dS0")
    shapes = ((N, T, dk), (N, T, dk), (N, T, dv), (N, T), (N, T, dk), (N, dk, dv))
    return {n: (np.zeros(s) if g is None else g.numpy()) for n, g, s in zip(names, grads, shapes)}


def kda_backward(q, k, v, eta, log_a, eps, S0, do, dST=None, beta_given=False):
    """Library-layout KDA gradients: q, k, log_a [B, T, H, d_k]; v, do [B, T, H, d_v]; eta (or beta
    when ``beta_given``) [B, T, H]; S0, dST [B, H, d_k, d_v] or None. Returns dq, dk, dlog_a
    [B, T, H, d_k], dv [B, T, H, d_v], deta [B, T, H] and dS0 [B, H, d_k, d_v], all fp64."""
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    s0 = None if S0 is None else np.asarray(S0, np.float64).reshape(B * H, dk, dv)
    dst = None if dST is None else np.asarray(dST, np.float64).reshape(B * H, dk, dv)
    g = kda_vjp(_to_heads(q), _to_heads(k), _to_heads(v), _to_heads(eta), _to_heads(log_a), eps, s0,
                _to_heads(do), dst, beta_given)
    out = {n: _from_heads(g[n], B, H) for n in ("dq", "dk", "dv", "deta", "dlog_a")}
    out["dS0"] = g["dS0"].reshape(B, H, dk, dv)
    return out
