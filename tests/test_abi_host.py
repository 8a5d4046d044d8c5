"""C ABI checks that need no GPU: the library loads, exports everything include/kla.h
declares, and rejects bad arguments before it enqueues anything (no compute calls)."""
import ctypes

import pytest

from gated_delta_rule_18_amd import _lib as K

A16 = 1 << 20  # a 16-byte-aligned fake address; never dereferenced: every call below fails validation


def L():
    return K.lib()


def test_exports_every_declared_symbol():
    names = K.declared_functions()
    assert set(names) == {"kla_prepare_beta", "kla_chunk_fwd_workspace_size", "kla_chunk_fwd",
                          "kla_decode_step", "kla_gdn_chunk_fwd", "kla_gdn_decode_step", "kla_status_string",
                          "kla_last_error", "kla_chunk_bwd_workspace_size", "kla_chunk_bwd", "kla_gdn_chunk_bwd",
                          "kla_kda_chunk_fwd_workspace_size", "kla_kda_chunk_fwd", "kla_kda_decode_step",
                          "kla_chunk_fwd_seg_workspace_size", "kla_chunk_fwd_seg", "kla_chunk_fwd_noalloc",
                          "kla_kda_chunk_bwd_workspace_size", "kla_kda_chunk_bwd", "kla_chunk_fwd_train",
                          "kla_gdn_chunk_fwd_train", "kla_chunk_bwd_saved", "kla_gdn_chunk_bwd_saved",
                          "kla_kda_chunk_fwd_train", "kla_kda_chunk_bwd_saved"}
    for n in names:
        assert hasattr(L(), n), n


def test_status_strings():
    for code in range(4):
        assert L().kla_status_string(code).startswith(b"KLA_")
    assert b"unknown" in L().kla_status_string(99)


def p(x=A16):
    return ctypes.c_void_p(x)


def chunk(dk=128, dv=128, chunk_len=64, eps=1e-6, dt=K.KLA_BF16, B=1, T=64, H=1,
          q=A16, k=A16 * 2, v=A16 * 3, eta=A16 * 4, la=A16 * 5, s_in=0, s_out=0, o=A16 * 6, ws=0, ws_bytes=0):
    return L().kla_chunk_fwd(p(q), p(k), p(v), p(eta), p(la), p(s_in) if s_in else None,
                             p(s_out) if s_out else None, p(o), B, T, H, dk, dv, chunk_len, eps, dt,
                             p(ws) if ws else None, ws_bytes, None)


def decode(dk=128, dv=128, eps=1e-6, dt=K.KLA_BF16, B=1, H=1, q=A16, k=A16 * 2, v=A16 * 3, eta=A16 * 4,
           la=A16 * 5, state=A16 * 8, o=A16 * 16):
    return L().kla_decode_step(p(q), p(k), p(v), p(eta), p(la), p(state) if state else None, p(o) if o else None,
                               B, H, dk, dv, eps, dt, None)


def prep(dk=128, chunk_len=64, eps=1e-6, dt=K.KLA_BF16, B=1, T=64, H=1, k=A16, eta=A16 * 2, la=A16 * 3,
         beta=A16 * 4, gcum=A16 * 5):
    return L().kla_prepare_beta(p(k), p(eta), p(la), p(beta), p(gcum) if gcum else None, B, T, H, dk,
                                chunk_len, eps, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), K.KLA_ERR_NOT_SUPPORTED),
    (dict(dv=256), K.KLA_ERR_NOT_SUPPORTED),
    (dict(chunk_len=32), K.KLA_ERR_NOT_SUPPORTED),
    (dict(eps=-1.0), K.KLA_ERR_INVALID_VALUE),
    (dict(eps=float("nan")), K.KLA_ERR_INVALID_VALUE),
    (dict(dt=7), K.KLA_ERR_INVALID_VALUE),
    (dict(T=-1), K.KLA_ERR_INVALID_VALUE),
    (dict(q=0), K.KLA_ERR_INVALID_VALUE),
    (dict(o=0), K.KLA_ERR_INVALID_VALUE),
    (dict(q=A16 + 2), K.KLA_ERR_INVALID_VALUE),          # misaligned
    (dict(eta=A16 * 4 + 2), K.KLA_ERR_INVALID_VALUE),    # misaligned gate
    (dict(o=A16 + 64), K.KLA_ERR_INVALID_VALUE),         # o overlaps q
    (dict(s_in=A16 * 32, s_out=A16 * 32 + 256), K.KLA_ERR_INVALID_VALUE),  # partial state overlap
    (dict(B=1 << 40, T=1 << 30), K.KLA_ERR_INVALID_VALUE),  # size overflow
    (dict(T=1 << 20, H=16), K.KLA_ERR_NOT_SUPPORTED),        # one batch entry past 2 GiB
])
def test_chunk_fwd_rejects(kw, status):
    assert chunk(**kw) == status
    assert L().kla_last_error() != b""


def test_chunk_fwd_empty_batch_is_a_no_op():
    assert chunk(B=0) == K.KLA_OK
    assert chunk(H=0, q=0, k=0) == K.KLA_OK
    assert chunk(T=0) == K.KLA_OK  # no state requested: nothing to write, nothing launched


@pytest.mark.parametrize("segments", [None, 0, 1, 3, 100000])
def test_chunk_fwd_plan_is_host_only_and_total(segments):
    """The workspace size (which depends on the segment plan) is defined for every length and
    every segment count the caller may ask for."""
    for T in (1, 2, 63, 64, 65, 129, 4096, 65536):
        for H in (1, 16, 64):
            if segments is None:
                assert K.lib().kla_chunk_fwd_workspace_size(1, T, H, 128, 128, 64, K.KLA_BF16) > 0
            else:
                assert K.lib().kla_chunk_fwd_seg_workspace_size(1, T, H, 128, 128, 64, segments, K.KLA_BF16) > 0
    assert chunk(T=0) == K.KLA_OK


def test_segment_plan_argument():
    """segments = 0 is the library's plan (kla_chunk_fwd's workspace); 1 is the one-pass scan;
    a negative count is rejected before anything else, and its size query gives 0."""
    ws = lambda B, T, H: K.lib().kla_chunk_fwd_workspace_size(B, T, H, 128, 128, 64, K.KLA_BF16)
    seg = lambda B, T, H, n: K.lib().kla_chunk_fwd_seg_workspace_size(B, T, H, 128, 128, 64, n, K.KLA_BF16)
    for B, T, H in ((1, 65536, 16), (8, 4096, 8), (1, 1000, 3)):
        assert seg(B, T, H, 0) == ws(B, T, H)
    assert seg(1, 1000, 3, 4) > seg(1, 1000, 3, 1)
    assert seg(1, 1000, 3, -1) == 0
    st = L().kla_chunk_fwd_seg(p(A16), p(A16 * 2), p(A16 * 3), p(A16 * 4), p(A16 * 5), None, None, p(A16 * 6),
                               1, 64, 1, 128, 128, 64, -1, 1e-6, K.KLA_BF16, None, 0, None)
    assert st == K.KLA_ERR_INVALID_VALUE and b"segment" in L().kla_last_error()


def test_long_few_head_forward_plans_segments():
    """B1 H16 T65536: the one-pass scan would occupy 64 of the full chip's 256 compute units, so the
    plan segments the sequence and the workspace grows by the segment buffers; B8 H8 T4096 does not.
    (With no device present the plan is made for the full MI355X.)"""
    ws = lambda B, T, H: K.lib().kla_chunk_fwd_workspace_size(B, T, H, 128, 128, 64, K.KLA_BF16)
    one = lambda B, T, H: K.lib().kla_chunk_fwd_seg_workspace_size(B, T, H, 128, 128, 64, 1, K.KLA_BF16)
    assert ws(1, 65536, 16) > one(1, 65536, 16)
    assert ws(8, 4096, 8) == one(8, 4096, 8)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=32), K.KLA_ERR_NOT_SUPPORTED),
    (dict(state=0), K.KLA_ERR_INVALID_VALUE),
    (dict(o=A16 * 8 + 16), K.KLA_ERR_INVALID_VALUE),    # o inside the state
    (dict(k=A16 * 2 + 8), K.KLA_ERR_INVALID_VALUE),     # misaligned
    (dict(eps=float("inf")), K.KLA_ERR_INVALID_VALUE),
    (dict(B=-2), K.KLA_ERR_INVALID_VALUE),
])
def test_decode_step_rejects(kw, status):
    assert decode(**kw) == status


def test_decode_empty_is_a_no_op():
    assert decode(B=0) == K.KLA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(dk=100), K.KLA_ERR_NOT_SUPPORTED),
    (dict(chunk_len=128), K.KLA_ERR_NOT_SUPPORTED),
    (dict(beta=0), K.KLA_ERR_INVALID_VALUE),
    (dict(beta=A16 + 4), K.KLA_ERR_INVALID_VALUE),      # beta overlaps k
    (dict(gcum=A16 * 4), K.KLA_ERR_INVALID_VALUE),      # gcum == beta
])
def test_prepare_beta_rejects(kw, status):
    assert prep(**kw) == status


def test_chunk_fwd_requires_its_workspace():
    need = K.lib().kla_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    assert need > 0
    assert chunk() == K.KLA_ERR_INVALID_VALUE
    assert b"workspace" in L().kla_last_error()
    assert chunk(ws=A16 * 64, ws_bytes=need - 1) == K.KLA_ERR_INVALID_VALUE
    assert chunk(ws=A16 + 256, ws_bytes=need) == K.KLA_ERR_INVALID_VALUE  # overlaps q


def test_workspace_size_is_host_only():
    assert K.lib().kla_chunk_fwd_workspace_size(8, 4096, 8, 128, 128, 64, K.KLA_BF16) >= 0
    assert K.lib().kla_chunk_fwd_workspace_size(8, 4096, 8, 96, 128, 64, K.KLA_BF16) == 0


def test_python_wrapper_rejects_without_gpu_work():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        K.kla_chunk_fwd(q, q, q[..., :32].contiguous(), torch.zeros(1, 4, 2), torch.zeros(1, 4, 1))


def gdn_chunk(dk=128, dv=128, chunk_len=64, dt=K.KLA_BF16, B=1, T=64, H=1, q=A16, k=A16 * 2, v=A16 * 3,
              beta=A16 * 4, la=A16 * 5, o=A16 * 6):
    return L().kla_gdn_chunk_fwd(p(q), p(k), p(v), p(beta) if beta else None, p(la) if la else None, None, None,
                                 p(o), B, T, H, dk, dv, chunk_len, dt, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), K.KLA_ERR_NOT_SUPPORTED),
    (dict(chunk_len=16), K.KLA_ERR_NOT_SUPPORTED),
    (dict(beta=0), K.KLA_ERR_INVALID_VALUE),                      # beta is required
    (dict(beta=A16 * 4 + 2), K.KLA_ERR_INVALID_VALUE),            # misaligned
    (dict(o=A16 * 2 + 64), K.KLA_ERR_INVALID_VALUE),              # o overlaps k
    (dict(la=0, o=A16 * 2 + 64), K.KLA_ERR_INVALID_VALUE),        # log_alpha may be null; o still overlaps k
    (dict(la=0), K.KLA_ERR_INVALID_VALUE),                        # ... and the workspace is still required
])
def test_gdn_chunk_fwd_rejects(kw, status):
    assert gdn_chunk(**kw) == status
    assert L().kla_last_error().startswith(b"kla_gdn_chunk_fwd")


def gdn_decode(dk=128, dv=128, dt=K.KLA_BF16, B=1, H=1, beta=A16 * 4, la=A16 * 5, state=A16 * 8, o=A16 * 16):
    return L().kla_gdn_decode_step(p(A16), p(A16 * 2), p(A16 * 3), p(beta) if beta else None,
                                   p(la) if la else None, p(state) if state else None, p(o), B, H, dk, dv, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=32), K.KLA_ERR_NOT_SUPPORTED),
    (dict(beta=0), K.KLA_ERR_INVALID_VALUE),
    (dict(state=0), K.KLA_ERR_INVALID_VALUE),
    (dict(la=0, o=A16 * 8 + 16), K.KLA_ERR_INVALID_VALUE),        # null log_alpha accepted; o inside the state
    (dict(dt=5), K.KLA_ERR_INVALID_VALUE),
])
def test_gdn_decode_step_rejects(kw, status):
    assert gdn_decode(**kw) == status


def test_gdn_empty_is_a_no_op():
    assert gdn_decode(B=0) == K.KLA_OK
    assert gdn_chunk(B=0) == K.KLA_OK


WS = A16 * 256  # fake workspace address, far from the tensors below


def bwd(dk=128, dv=128, chunk_len=64, eps=1e-6, dt=K.KLA_BF16, B=1, T=64, H=1, q=A16, k=A16 * 2, v=A16 * 3,
        eta=A16 * 4, la=A16 * 5, s_in=0, do=A16 * 6, ds_out=0, dq=A16 * 7, dk_=A16 * 8, dv_=A16 * 9,
        deta=A16 * 10, dla=A16 * 11, ds_in=0, ws=WS, ws_bytes=None, gdn=False, saved=False):
    if ws_bytes is None:
        ws_bytes = max(K.lib().kla_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk_len, dt), 0)
    opt = lambda x: p(x) if x else None
    head = [p(q), p(k), p(v), opt(eta), opt(la), opt(s_in), opt(do), opt(ds_out), opt(dq), opt(dk_), opt(dv_),
            opt(deta), opt(dla), opt(ds_in), B, T, H, dk, dv, chunk_len]
    tail = [dt, opt(ws), ws_bytes, None]
    if gdn:
        return getattr(L(), "kla_gdn_chunk_bwd_saved" if saved else "kla_gdn_chunk_bwd")(*head, *tail)
    return getattr(L(), "kla_chunk_bwd_saved" if saved else "kla_chunk_bwd")(*head, eps, *tail)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), K.KLA_ERR_NOT_SUPPORTED),
    (dict(chunk_len=32), K.KLA_ERR_NOT_SUPPORTED),
    (dict(eps=-1.0), K.KLA_ERR_INVALID_VALUE),
    (dict(T=-3), K.KLA_ERR_INVALID_VALUE),
    (dict(do=0), K.KLA_ERR_INVALID_VALUE),
    (dict(dla=0), K.KLA_ERR_INVALID_VALUE),                    # log_alpha given: dlog_alpha required
    (dict(la=0), K.KLA_ERR_INVALID_VALUE),                     # KLA needs log_alpha
    (dict(deta=A16 * 10 + 2), K.KLA_ERR_INVALID_VALUE),        # misaligned
    (dict(dq=A16 * 2 + 64), K.KLA_ERR_INVALID_VALUE),          # dq overlaps k
    (dict(dv_=A16 * 7), K.KLA_ERR_INVALID_VALUE),              # dv overlaps dq
    (dict(ws=0), K.KLA_ERR_INVALID_VALUE),                     # workspace required
    (dict(ws_bytes=1024), K.KLA_ERR_INVALID_VALUE),            # ... and big enough
    (dict(ws=A16 * 6 + 512), K.KLA_ERR_INVALID_VALUE),         # workspace overlaps do
    (dict(T=1 << 20, H=16), K.KLA_ERR_NOT_SUPPORTED),          # one batch entry past 2 GiB
])
def test_chunk_bwd_rejects(kw, status):
    assert bwd(**kw) == status
    assert L().kla_last_error().startswith(b"kla_chunk_bwd")
    # the backward from a training forward's workspace checks its arguments alike
    assert bwd(saved=True, **kw) == status
    assert L().kla_last_error().startswith(b"kla_chunk_bwd_saved")


@pytest.mark.parametrize("kw,status", [
    (dict(la=0, dla=0, dk=100), K.KLA_ERR_NOT_SUPPORTED),
    (dict(eta=0), K.KLA_ERR_INVALID_VALUE),                    # beta required
    (dict(la=0, deta=0), K.KLA_ERR_INVALID_VALUE),             # dbeta required
    (dict(la=0, dla=0, dk_=A16 * 6), K.KLA_ERR_INVALID_VALUE),  # dk overlaps do
])
def test_gdn_chunk_bwd_rejects(kw, status):
    assert bwd(gdn=True, **kw) == status
    assert L().kla_last_error().startswith(b"kla_gdn_chunk_bwd")
    assert bwd(gdn=True, saved=True, **kw) == status
    assert L().kla_last_error().startswith(b"kla_gdn_chunk_bwd_saved")


def fwd_train(dk=128, dv=128, chunk_len=64, eps=1e-6, dt=K.KLA_BF16, B=1, T=64, H=1, q=A16, k=A16 * 2,
              v=A16 * 3, eta=A16 * 4, la=A16 * 5, o=A16 * 6, ws=WS, ws_bytes=None, gdn=False):
    """kla_chunk_fwd_train / kla_gdn_chunk_fwd_train with fake device addresses; the workspace
    defaults to the backward's size."""
    if ws_bytes is None:
        ws_bytes = max(K.lib().kla_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk_len, dt), 0)
    opt = lambda x: p(x) if x else None
    head = [p(q), p(k), p(v), opt(eta), opt(la), None, None, opt(o), B, T, H, dk, dv, chunk_len]
    tail = [dt, opt(ws), ws_bytes, None]
    if gdn:
        return L().kla_gdn_chunk_fwd_train(*head, *tail)
    return L().kla_chunk_fwd_train(*head, eps, *tail)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), K.KLA_ERR_NOT_SUPPORTED),
    (dict(eps=-1.0), K.KLA_ERR_INVALID_VALUE),
    (dict(la=0), K.KLA_ERR_INVALID_VALUE),                     # KLA needs log_alpha
    (dict(ws=0), K.KLA_ERR_INVALID_VALUE),                     # workspace required
    (dict(o=A16 * 2 + 64), K.KLA_ERR_INVALID_VALUE),           # o overlaps k
])
def test_chunk_fwd_train_rejects(kw, status):
    assert fwd_train(**kw) == status
    assert L().kla_last_error().startswith(b"kla_chunk_fwd_train")


def test_chunk_fwd_train_needs_the_backward_workspace():
    """The forward's own workspace size is not enough: the training forward fills the backward's."""
    fwd_need = K.lib().kla_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    bwd_need = K.lib().kla_chunk_bwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    assert fwd_need < bwd_need
    assert fwd_train(ws_bytes=fwd_need) == K.KLA_ERR_INVALID_VALUE
    assert b"workspace" in L().kla_last_error()
    assert fwd_train(gdn=True, la=0, ws_bytes=bwd_need - 16) == K.KLA_ERR_INVALID_VALUE
    assert L().kla_last_error().startswith(b"kla_gdn_chunk_fwd_train")
    assert fwd_train(gdn=True, eta=0) == K.KLA_ERR_INVALID_VALUE  # beta required
    assert fwd_train(B=0) == K.KLA_OK
    assert fwd_train(T=0, ws=0) == K.KLA_OK  # nothing to write without state_out


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_chunk_bwd_accepts_every_fp32_head_size(dk, dv):
    """fp32 gradients of every head-size pair pass the checks (T = 0: nothing is launched)."""
    assert bwd(dt=K.KLA_F32, dk=dk, dv=dv, T=0, ws=0) == K.KLA_OK


def test_chunk_bwd_empty_is_a_no_op():
    assert bwd(B=0) == K.KLA_OK
    assert bwd(H=0, q=0) == K.KLA_OK
    assert bwd(T=0, ws=0) == K.KLA_OK  # nothing to write without dstate_in


def test_bwd_workspace_size():
    need = K.lib().kla_chunk_bwd_workspace_size(8, 4096, 8, 128, 128, 64, K.KLA_BF16)
    fwd = K.lib().kla_chunk_fwd_workspace_size(8, 4096, 8, 128, 128, 64, K.KLA_BF16)
    # the forward's per-chunk factors, then per chunk two bf16 states and two 64 x 128 blocks
    assert need == fwd + 8 * 8 * 64 * (2 * 128 * 128 + 2 * 64 * 128) * 2
    assert K.lib().kla_chunk_bwd_workspace_size(8, 0, 8, 128, 128, 64, K.KLA_BF16) == 0


def kda_bwd(dk=128, dv=128, chunk_len=64, eps=1e-6, beta_given=0, dt=K.KLA_BF16, B=1, T=64, H=1, la=A16 * 5,
            dla=A16 * 16, dq=A16 * 7, ws=WS, ws_bytes=None):
    """kla_kda_chunk_bwd with fake device addresses (rejected before anything is enqueued).
    log a and dlog a are [B, T, H, d_k] fp32: 32 KiB apart at T = 64, d_k = 128."""
    if ws_bytes is None:
        ws_bytes = max(K.lib().kla_kda_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk_len, dt), 0)
    opt = lambda x: p(x) if x else None
    return L().kla_kda_chunk_bwd(p(A16), p(A16 * 2), p(A16 * 3), p(A16 * 4), opt(la), None, p(A16 * 6), None,
                                 opt(dq), p(A16 * 8), p(A16 * 9), p(A16 * 10), opt(dla), None, B, T, H, dk, dv,
                                 chunk_len, eps, beta_given, dt, opt(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), K.KLA_ERR_NOT_SUPPORTED),
    (dict(dt=K.KLA_F32), K.KLA_ERR_NOT_SUPPORTED),             # fp32 gradients need d = 64
    (dict(la=0), K.KLA_ERR_INVALID_VALUE),                     # the per-channel decay is required
    (dict(la=0, beta_given=1), K.KLA_ERR_INVALID_VALUE),       # ... also with beta given
    (dict(dla=0), K.KLA_ERR_INVALID_VALUE),                    # and its gradient
    (dict(la=A16 * 5 + 4), K.KLA_ERR_INVALID_VALUE),           # log a rows are read 16 bytes at a time
    (dict(dq=A16 * 5 + 4096), K.KLA_ERR_INVALID_VALUE),        # dq inside log a
    (dict(dla=A16 * 5 + 8192), K.KLA_ERR_INVALID_VALUE),       # dlog a overlapping log a
    (dict(ws=0), K.KLA_ERR_INVALID_VALUE),
    (dict(ws_bytes=4096), K.KLA_ERR_INVALID_VALUE),
    (dict(T=300000, H=16), K.KLA_ERR_NOT_SUPPORTED),           # fp32 log a of one batch entry past 2 GiB
])
def test_kda_chunk_bwd_rejects(kw, status):
    assert kda_bwd(**kw) == status
    assert L().kla_last_error().startswith(b"kla_kda_chunk_bwd")


def test_kda_training_pair_checks():
    """kla_kda_chunk_fwd_train fills the KDA backward's workspace and supports what that backward
    does; kla_kda_chunk_bwd_saved checks its arguments as kla_kda_chunk_bwd."""
    need = K.lib().kla_kda_chunk_bwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    kfwd = K.lib().kla_kda_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    lib = L()
    args = lambda dt, dk, ws_bytes: (p(A16), p(A16 * 2), p(A16 * 3), p(A16 * 4), p(A16 * 5), None, None, p(A16 * 6),
                                     1, 64, 1, dk, dk, 64, ctypes.c_float(1e-6), 0, dt, p(WS), ws_bytes, None)
    assert lib.kla_kda_chunk_fwd_train(*args(K.KLA_BF16, 128, kfwd)) == K.KLA_ERR_INVALID_VALUE
    assert lib.kla_last_error().startswith(b"kla_kda_chunk_fwd_train")
    assert lib.kla_kda_chunk_fwd_train(*args(K.KLA_F32, 128, need)) == K.KLA_ERR_NOT_SUPPORTED
    assert lib.kla_kda_chunk_fwd_train(*args(K.KLA_BF16, 96, need)) == K.KLA_ERR_NOT_SUPPORTED
    a = [p(A16), p(A16 * 2), p(A16 * 3), p(A16 * 4), p(A16 * 5), None, p(A16 * 6), None, p(A16 * 7), p(A16 * 8),
         p(A16 * 9), p(A16 * 10), p(A16 * 16), None, 1, 64, 1, 128, 128, 64, ctypes.c_float(1e-6), 0, K.KLA_BF16,
         None, need, None]
    assert lib.kla_kda_chunk_bwd_saved(*a) == K.KLA_ERR_INVALID_VALUE  # workspace required
    assert lib.kla_last_error().startswith(b"kla_kda_chunk_bwd_saved")


def test_kda_bwd_workspace_and_empty():
    need = K.lib().kla_kda_chunk_bwd_workspace_size(8, 4096, 8, 128, 128, 64, K.KLA_BF16)
    kfwd = K.lib().kla_kda_chunk_fwd_workspace_size(8, 4096, 8, 128, 128, 64, K.KLA_BF16)
    # the KDA forward's per-chunk factors and decayed operands, then per chunk two bf16 states and
    # two 64 x 128 blocks (as for the scalar gate's backward)
    assert need == kfwd + 8 * 8 * 64 * (2 * 128 * 128 + 2 * 64 * 128) * 2
    assert K.lib().kla_kda_chunk_bwd_workspace_size(8, 0, 8, 128, 128, 64, K.KLA_BF16) == 0
    assert kda_bwd(B=0) == K.KLA_OK
    assert kda_bwd(T=0, ws=0) == K.KLA_OK


def kda_chunk(dk=128, dv=128, chunk_len=64, eps=1e-6, beta_given=0, dt=K.KLA_BF16, B=1, T=64, H=1, q=A16,
              k=A16 * 2, v=A16 * 3, eta=A16 * 4, la=A16 * 5, o=A16 * 6, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = max(K.lib().kla_kda_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk_len, dt), 0)
    opt = lambda x: p(x) if x else None
    return L().kla_kda_chunk_fwd(opt(q), opt(k), opt(v), opt(eta), opt(la), None, None, opt(o), B, T, H, dk, dv,
                                 chunk_len, eps, beta_given, dt, opt(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), K.KLA_ERR_NOT_SUPPORTED),
    (dict(chunk_len=32), K.KLA_ERR_NOT_SUPPORTED),
    (dict(la=0), K.KLA_ERR_INVALID_VALUE),                     # the per-channel decay is required
    (dict(la=0, beta_given=1), K.KLA_ERR_INVALID_VALUE),       # ... also with beta given
    (dict(la=A16 * 5 + 4), K.KLA_ERR_INVALID_VALUE),           # log a rows are read 16 bytes at a time
    (dict(o=A16 * 5 + 4096), K.KLA_ERR_INVALID_VALUE),         # o inside log a ([B,T,H,d_k] fp32 = 32 KiB)
    (dict(ws=0), K.KLA_ERR_INVALID_VALUE),
    (dict(ws_bytes=4096), K.KLA_ERR_INVALID_VALUE),
    (dict(eps=-1.0), K.KLA_ERR_INVALID_VALUE),
    (dict(T=300000, H=16), K.KLA_ERR_NOT_SUPPORTED),           # fp32 log a of one batch entry past 2 GiB
])
def test_kda_chunk_fwd_rejects(kw, status):
    assert kda_chunk(**kw) == status
    assert L().kla_last_error().startswith(b"kla_kda_chunk_fwd")


def test_kda_workspace_and_empty():
    need = K.lib().kla_kda_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    base = K.lib().kla_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, K.KLA_BF16)
    assert need == base + 128 * (3 * 64 * 2 + 4)  # K o e^G, Q o e^G, K o e^{G_C - G} (bf16), gamma (fp32)
    assert kda_chunk(B=0) == K.KLA_OK
    assert kda_chunk(T=0, ws=0) == K.KLA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(la=0), K.KLA_ERR_INVALID_VALUE),
    (dict(dk=32), K.KLA_ERR_NOT_SUPPORTED),
    (dict(o=A16 * 5 + 64), K.KLA_ERR_INVALID_VALUE),           # o inside log a ([B,H,d_k])
])
def test_kda_decode_step_rejects(kw, status):
    d = dict(dk=128, dv=128, la=A16 * 5, o=A16 * 16)
    d.update(kw)
    st = L().kla_kda_decode_step(p(A16), p(A16 * 2), p(A16 * 3), p(A16 * 4), p(d["la"]) if d["la"] else None,
                                 p(A16 * 8), p(d["o"]), 1, 1, d["dk"], d["dv"], 1e-6, 0, K.KLA_BF16, None)
    assert st == status



def test_kda_forward_plans_segments_like_the_scalar_gate():
    """The per-channel decay's forward takes the same segment plan: a few-head long sequence gets
    the segment buffers on top of the KDA prep's workspace; B8 H8 T4096 stays one pass."""
    kda = lambda B, T, H: K.lib().kla_kda_chunk_fwd_workspace_size(B, T, H, 128, 128, 64, K.KLA_BF16)
    one = lambda B, T, H: K.lib().kla_chunk_fwd_seg_workspace_size(B, T, H, 128, 128, 64, 1, K.KLA_BF16)
    seg = lambda B, T, H: K.lib().kla_chunk_fwd_workspace_size(B, T, H, 128, 128, 64, K.KLA_BF16)
    # KDA adds K o e^G, Q o e^G, K o e^{G_C - G} (bf16) and gamma (fp32) per chunk to the scalar
    # gate's per-chunk factors; the segment buffers of a plan are the same for both gates.
    kda_ops = lambda B, T, H: B * H * (T // 64) * 128 * (3 * 64 * 2 + 4)
    for B, T, H in ((1, 65536, 16), (8, 4096, 8)):
        assert kda(B, T, H) - kda_ops(B, T, H) - one(B, T, H) == seg(B, T, H) - one(B, T, H)
    assert seg(1, 65536, 16) > one(1, 65536, 16) and seg(8, 4096, 8) == one(8, 4096, 8)
