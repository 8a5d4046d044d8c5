"""fp64 reference for Kaczmarz Linear Attention (KLA) — test infrastructure only.

Imported only by the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg. Nothing here is shared with the HIP library.

State orientation (a reading; the printed formula is not self-consistent).
"Deep Dive into KDA", section 2.2, prints the gated delta rule as
``S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t v_t k_t^T`` with ``o_t = S_t q_t``.
Taken literally with a d x d state, the erase acts on the rows while the write
``v k^T`` is a column write, so with alpha = eta = 1 the new state would not map
k_t to v_t — the projection property that section 2.1 describes (erase the old
value along k_t, then write the new one). The self-consistent reading used
throughout: the state is a d_v x d_k map M with
``M_t = alpha_t M_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T`` and ``o_t = M_t q_t``.
It is stored transposed, ``S = M^T`` with shape [d_k, d_v] (d_v contiguous), so

    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,    o_t = S_t^T q_t.

Other readings (each also listed in the design notes):
  * alpha_t decays only the old state; the write is not decayed (section 2.2's form).
  * the output is read after the write (o_t uses S_t).
  * eps is added to the squared L2 norm of the head's key ("Kaczmarz Linear
    Attention", Abstract); eta arrives already activated; q arrives pre-scaled.
  * alpha enters as log(alpha) and every decay product is formed in the log domain
    ("Deep Dive into KDA", section 3 and section 5, on underflow of prefix products).

Array layouts. The library layout is q, k [B, T, H, d_k], v [B, T, H, d_v],
eta, log_alpha [B, T, H], state [B, H, d_k, d_v]. The core loops use a
head-major layout [N, T, d] with N = B * H.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kaczmarz_step_size(k, eta, eps):
    """beta_t = eta_t / (||k_t||_2^2 + eps): the key-norm-normalised step size
    ("Kaczmarz Linear Attention", Abstract). ``k`` [..., d_k], ``eta`` [...]."""
    k = _f64(k)
    return _f64(eta) / (np.sum(k * k, axis=-1) + float(eps))


def chunk_local_log_decay(log_alpha, chunk):
    """Chunk-local inclusive prefix sums of log(alpha) along the last (time) axis.

    G_t = sum of log(alpha_s) over the tokens s <= t of t's chunk; it restarts at
    every chunk boundary. These are the intra-chunk accumulated decays of
    "Deep Dive into KDA", section 3, computed once by prefix sums, in the log domain.
    """
    g = _f64(log_alpha)
    G = np.empty_like(g)
    T = g.shape[-1]
    for c0 in range(0, T, chunk):
        G[..., c0:c0 + chunk] = np.cumsum(g[..., c0:c0 + chunk], axis=-1)
    return G


def gated_delta_recurrent(q, k, v, beta, log_alpha, S0=None):
    """Token-by-token gated delta rule ("Deep Dive into KDA", section 2.2) with a
    given per-token beta, in the [d_k, d_v] state orientation of this module.

    q, k [N, T, d_k]; v [N, T, d_v]; beta, log_alpha [N, T]; S0 [N, d_k, d_v] or None (zeros).
    Returns o [N, T, d_v] and the final state [N, d_k, d_v], fp64.

    Per token: decay S' = alpha_t S_{t-1}; recall u = S'^T k_t; write
    S_t = S' + beta_t k_t (v_t - u)^T, which equals alpha_t (I - beta_t k_t k_t^T) S_{t-1}
    + beta_t k_t v_t^T; read o_t = S_t^T q_t.
    """
    q, k, v, beta, log_alpha = map(_f64, (q, k, v, beta, log_alpha))
    N, T, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((N, T, dv))
    alpha = np.exp(log_alpha)
    for t in range(T):
        kt = k[:, t]
        S *= alpha[:, t, None, None]
        u = np.einsum("nij,ni->nj", S, kt)
        S += beta[:, t, None, None] * (kt[:, :, None] * (v[:, t] - u)[:, None, :])
        o[:, t] = np.einsum("nij,ni->nj", S, q[:, t])
    return o, S


def kla_recurrent(q, k, v, eta, log_alpha, eps, S0=None):
    """KLA in the head-major layout: the gated delta rule with the Kaczmarz step size
    ("Kaczmarz Linear Attention", Abstract: a one-scalar change of Gated DeltaNet)."""
    return gated_delta_recurrent(q, k, v, kaczmarz_step_size(k, eta, eps), log_alpha, S0)


def _to_heads(x):
    """[B, T, H, ...] -> [B*H, T, ...]."""
    x = np.asarray(x)
    B, T, H = x.shape[:3]
    return np.moveaxis(x, 2, 1).reshape((B * H, T) + x.shape[3:])


def _from_heads(x, B, H):
    """[B*H, T, ...] -> [B, T, H, ...]."""
    T = x.shape[1]
    return np.moveaxis(x.reshape((B, H, T) + x.shape[2:]), 1, 2)


def kla_forward(q, k, v, eta, log_alpha, eps, S0=None):
    """KLA forward over a sequence in the library layout.

    q, k [B, T, H, d_k]; v [B, T, H, d_v]; eta, log_alpha [B, T, H]; S0 [B, H, d_k, d_v] or None.
    Returns o [B, T, H, d_v] and S_T [B, H, d_k, d_v] (fp64).
    """
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    s0 = None if S0 is None else _f64(S0).reshape(B * H, dk, dv)
    o, S = kla_recurrent(_to_heads(q), _to_heads(k), _to_heads(v), _to_heads(eta),
                         _to_heads(log_alpha), eps, s0)
    return _from_heads(o, B, H), S.reshape(B, H, dk, dv)


def kla_decode_step(q, k, v, eta, log_alpha, eps, S):
    """One recurrent decode step in the library layout: q, k [B, H, d_k], v [B, H, d_v],
    eta, log_alpha [B, H], S [B, H, d_k, d_v]. Returns o [B, H, d_v] and the new state.
    It is the same token update as the sequence recurrence, for one token."""
    B, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    o, S1 = kla_recurrent(_f64(q).reshape(B * H, 1, dk), _f64(k).reshape(B * H, 1, dk),
                          _f64(v).reshape(B * H, 1, dv), _f64(eta).reshape(B * H, 1),
                          _f64(log_alpha).reshape(B * H, 1), eps, _f64(S).reshape(B * H, dk, dv))
    return o.reshape(B, H, dv), S1.reshape(B, H, dk, dv)


def kla_decode_steps(q, k, v, eta, log_alpha, eps, S0):
    """``steps`` consecutive decode steps: q, k [steps, B, H, d_k], v [steps, B, H, d_v],
    eta, log_alpha [steps, B, H], S0 [B, H, d_k, d_v]. Returns o [steps, B, H, d_v], S_final."""
    n, B, H, dk = np.shape(k)
    dv = np.shape(v)[-1]

    def heads(x):
        x = np.asarray(x)
        return np.moveaxis(x, 0, 2).reshape((B * H, n) + x.shape[3:])

    o, S = kla_recurrent(heads(q), heads(k), heads(v), heads(eta), heads(log_alpha), eps,
                         _f64(S0).reshape(B * H, dk, dv))
    return np.moveaxis(o.reshape(B, H, n, dv), 2, 0), S.reshape(B, H, dk, dv)


def kla_prepare_beta(k, eta, log_alpha, eps, chunk):
    """The prologue in the library layout: beta [B, T, H] (Kaczmarz step size) and
    G [B, T, H], the chunk-local inclusive prefix sum of log(alpha) along T."""
    beta = kaczmarz_step_size(k, eta, eps)
    G = np.moveaxis(chunk_local_log_decay(np.moveaxis(_f64(log_alpha), 1, -1), chunk), -1, 1)
    return beta, G


def kla_chunked(q, k, v, eta, log_alpha, eps, S0=None, chunk=64):
    """Chunkwise form of the same recurrence, head-major layout, fp64.

    Follows "Deep Dive into KDA", section 3 (inter-chunk state update and intra-chunk
    output), specialised to a scalar gate. Per chunk, with S the state entering it,
    G_r the chunk-local inclusive log-decay prefix and beta_r the Kaczmarz step:
      A[r, s] = beta_r exp(G_r - G_s) k_r.k_s for s < r (else 0); T = (I + A)^-1
      W = T diag(beta e^G) K,  U = T diag(beta) V          (the page's W[t], U[t])
      Delta = U - W S
      O = diag(e^G) Q S + (L o Q K^T) Delta,  L[r, s] = exp(G_r - G_s) for s <= r, else 0
      S <- e^{G_C} S + (diag(e^{G_C - G}) K)^T Delta
    The page's Gamma plays two roles (e^{G_C - G_r} in the state update, e^{G_r} in the
    output); its K / Gamma is replaced by the ratio exp(G_r - G_s), which never exceeds 1.
    W and U are not spelled out on the page; the reading here is the one that makes the
    chunk reproduce the token recurrence exactly. The last chunk may be shorter.
    Returns o [N, T, d_v] and the final state.
    """
    q, k, v, eta, log_alpha = map(_f64, (q, k, v, eta, log_alpha))
    N, T, dk = k.shape
    dv = v.shape[-1]
    beta = kaczmarz_step_size(k, eta, eps)
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((N, T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        K, Q, V, b = k[:, sl], q[:, sl], v[:, sl], beta[:, sl]
        C = K.shape[1]
        G = np.cumsum(log_alpha[:, sl], axis=1)
        incl = np.tril(np.ones((C, C), dtype=bool))
        L = np.exp(np.where(incl, G[:, :, None] - G[:, None, :], -np.inf))
        strict = np.tril(np.ones((C, C)), -1)
        A = b[:, :, None] * (K @ K.transpose(0, 2, 1)) * L * strict
        Tinv = np.linalg.solve(np.eye(C) + A, np.broadcast_to(np.eye(C), A.shape))
        W = Tinv @ ((b * np.exp(G))[:, :, None] * K)
        U = Tinv @ (b[:, :, None] * V)
        Delta = U - W @ S
        o[:, sl] = np.exp(G)[:, :, None] * (Q @ S) + (L * (Q @ K.transpose(0, 2, 1))) @ Delta
        Kt = np.exp(G[:, -1:] - G)[:, :, None] * K
        S = np.exp(G[:, -1])[:, None, None] * S + Kt.transpose(0, 2, 1) @ Delta
    return o, S


def kda_recurrent(q, k, v, beta, log_a, S0=None):
    """The delta rule with a per-channel (diagonal) decay ("Deep Dive into KDA", section 2.3),
    in the [d_k, d_v] state orientation of this module: Diag(a_t) scales the state's d_k rows,
    the dimension the keys index ("each memory dimension" forgets at its own rate):

        S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1} + beta_t k_t v_t^T,    o_t = S_t^T q_t.

    Head-major: q, k [N, T, d_k]; v [N, T, d_v]; beta [N, T]; log_a [N, T, d_k]; S0 [N, d_k, d_v]
    or None. Per token: decay S' = Diag(a_t) S; recall u = S'^T k_t; write S_t = S' + beta_t k_t
    (v_t - u)^T; read o_t = S_t^T q_t. Returns o [N, T, d_v] and S_T, fp64."""
    q, k, v, beta, log_a = map(_f64, (q, k, v, beta, log_a))
    N, T, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((N, T, dv))
    a = np.exp(log_a)
    for t in range(T):
        kt = k[:, t]
        S *= a[:, t, :, None]
        u = np.einsum("nij,ni->nj", S, kt)
        S += beta[:, t, None, None] * (kt[:, :, None] * (v[:, t] - u)[:, None, :])
        o[:, t] = np.einsum("nij,ni->nj", S, q[:, t])
    return o, S


def kda_forward(q, k, v, eta, log_a, eps, S0=None, beta_given=False):
    """Library layout: q, k [B, T, H, d_k]; v [B, T, H, d_v]; eta (or beta when beta_given)
    [B, T, H]; log_a [B, T, H, d_k]; S0 [B, H, d_k, d_v] or None. The step is the Kaczmarz
    beta = eta / (||k||^2 + eps) unless beta is given. Returns o [B, T, H, d_v], S_T."""
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    kh = _to_heads(k)
    b = _to_heads(eta) if beta_given else kaczmarz_step_size(kh, _to_heads(eta), eps)
    s0 = None if S0 is None else _f64(S0).reshape(B * H, dk, dv)
    o, S = kda_recurrent(_to_heads(q), kh, _to_heads(v), b, _to_heads(log_a), s0)
    return _from_heads(o, B, H), S.reshape(B, H, dk, dv)


def kda_chunked(q, k, v, beta, log_a, S0=None, chunk=64):
    """Chunkwise form of kda_recurrent ("Deep Dive into KDA", section 3, with the diagonal
    decay: Gamma holds per-channel cumulative decays). Per chunk, with G [C, d_k] the chunk-local
    inclusive prefix of log a and S the entering state:
      A[r, s] = beta_r sum_i k_r[i] k_s[i] exp(G_r[i] - G_s[i])   (s < r)
      P[r, s] = sum_i q_r[i] k_s[i] exp(G_r[i] - G_s[i])          (s <= r)
      Delta   = (I + A)^-1 diag(beta) (V - (K o e^G) S)
      O       = (Q o e^G) S + P Delta
      S      <- Diag(e^{G_C}) S + (K o e^{G_C - G})^T Delta
    The page's K / Gamma is replaced by the ratios exp(G_r - G_s) with s <= r, never above 1.
    Head-major as kda_recurrent; the last chunk may be shorter."""
    q, k, v, beta, log_a = map(_f64, (q, k, v, beta, log_a))
    N, T, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((N, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((N, T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        K, Q, V, b = k[:, sl], q[:, sl], v[:, sl], beta[:, sl]
        C = K.shape[1]
        G = np.cumsum(log_a[:, sl], axis=1)                        # [N, C, dk]
        incl = np.tril(np.ones((C, C), dtype=bool))
        D = np.where(incl[None, :, :, None], G[:, :, None, :] - G[:, None, :, :], -np.inf)
        R = np.exp(D)                                               # [N, C, C, dk], ratios <= 1
        KK = np.einsum("nri,nsi,nrsi->nrs", K, K, R)
        QK = np.einsum("nri,nsi,nrsi->nrs", Q, K, R)
        A = b[:, :, None] * KK * np.tril(np.ones((C, C)), -1)
        Tinv = np.linalg.solve(np.eye(C) + A, np.broadcast_to(np.eye(C), A.shape))
        Delta = Tinv @ (b[:, :, None] * (V - (K * np.exp(G)) @ S))
        o[:, sl] = (Q * np.exp(G)) @ S + QK @ Delta
        S = np.exp(G[:, -1])[:, :, None] * S + (K * np.exp(G[:, -1:] - G)).transpose(0, 2, 1) @ Delta
    return o, S
