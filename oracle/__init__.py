"""CPU fp64 oracle for Kaczmarz Linear Attention — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of the
benchmark may import this package. The HIP library and its Python binding never
import it and share no code with it; a product call that reached this code
would be a CPU fallback, which the library does not have.

Sources (titles as the pages give them):
  * "Kaczmarz Linear Attention", Abstract: the Kaczmarz step size
    beta_t = eta_t / (||k_t||^2 + eps) and the statement that KLA keeps Gated
    DeltaNet's state, gates, recurrence and chunkwise algorithm.
  * "Deep Dive into KDA", section 2.2: the gated delta rule
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t v_t k_t^T, output o_t = S_t q_t;
    section 3: the chunkwise inter-chunk state update and intra-chunk output,
    with log-domain decay prefixes.
  * "Deep Dive into KDA", section 2.3: the per-channel (diagonal) decay of KDA,
    kda_recurrent / kda_forward / kda_chunked.
  * kla_grad: gradients of the same token loop (reverse-mode autodiff in fp64 on
    the CPU), for the chunkwise backward; the pages give no backward formulas.
  * adjoint: the same gradients as the loop's adjoint recurrence written out by
    hand in NumPy (linear memory in T, for full-size comparisons).
  * kda_vjp / kda_backward / kda_adjoint: the gradients of the per-channel decay's
    loop (kda_recurrent), by both routes.

Every function here is pinned by tests that do not call back into it alone:
hand-derived golden values, exact invariants, brute-force products, the
classical Kaczmarz limit (pseudo-inverse) and special cases. No function is
"parity unpinned".
"""
from .kla_oracle import (  # noqa: F401
    kaczmarz_step_size,
    chunk_local_log_decay,
    gated_delta_recurrent,
    kla_recurrent,
    kla_forward,
    kla_decode_step,
    kla_decode_steps,
    kla_chunked,
    kla_prepare_beta,
    kda_recurrent,
    kda_forward,
    kda_chunked,
)
from .adjoint import gated_delta_adjoint, kla_adjoint, kda_adjoint  # noqa: F401,E402
from .kla_grad import gated_delta_vjp, kla_vjp, kla_backward, kda_vjp, kda_backward  # noqa: F401,E402
