"""Kaczmarz Linear Attention hot path for AMD Instinct MI355X (gfx950).

The compute lives in libkla.so (hand-written HIP kernels behind the C ABI of
include/kla.h); this package only marshals torch tensors and streams into it.
"""
from ._lib import (  # noqa: F401
    CHUNK,
    KLA_BF16,
    KLA_F32,
    KLAError,
    kla_chunk_bwd,
    kla_chunk_bwd_workspace_size,
    kla_chunk_fwd,
    kla_chunk_fwd_workspace_size,
    kla_decode_step,
    kla_gdn_chunk_bwd,
    kla_gdn_chunk_fwd,
    kla_gdn_decode_step,
    kla_kda_chunk_fwd,
    kla_kda_chunk_fwd_workspace_size,
    kla_kda_decode_step,
    kla_prepare_beta,
    lib,
)
