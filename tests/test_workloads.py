"""Seeded generators: determinism, bf16 rounding, per-head streams (CPU only)."""
import numpy as np

import workloads as wl


def test_round_to_bf16_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e-3, 0.0], np.float32)
    r = wl.round_to_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 2.0 ** -6)
    assert r[3] == -2.5 and r[5] == 0.0
    assert (r.view(np.uint32) & 0xFFFF == 0).all()
    assert abs(r[4] - x[4]) <= 2.0 ** -8 * abs(x[4])  # unit roundoff of an 8-bit significand


def test_generators_deterministic_and_per_head():
    w = wl.custom("t", 101, B=2, H=3, dk=64, dv=64, T=100, steps=5)
    a = wl.prefill_inputs(w)
    b = wl.prefill_inputs(w)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])
    h = wl.head_prefill(w, 1, 2)
    np.testing.assert_array_equal(a["k"][1, :, 2], h["k"])
    np.testing.assert_array_equal(a["log_alpha"][1, :, 2], h["log_alpha"])
    d = wl.decode_inputs(w)
    hd = wl.head_decode(w, 0, 1)
    np.testing.assert_array_equal(d["v"][:, 0, 1], hd["v"])
    assert (a["eta"] > 0).all() and (a["eta"] < 1).all()
    assert (a["log_alpha"] <= -0.001).all() and (a["log_alpha"] >= -0.1).all()
    # bf16 values are exactly representable
    assert (a["q"].view(np.uint32) & 0xFFFF == 0).all()


def test_named_workloads_shapes():
    w = wl.WORKLOADS
    assert (w["fwd_tiny_f32"].T, w["fwd_tiny_f32"].dk, w["fwd_tiny_f32"].dtype) == (256, 64, "f32")
    assert w["fwd_b8h8_t4096"].heads == 64 and w["fwd_long_t65536"].T == 65536
    assert w["decode_b64h16"].steps == 1024 and w["decode_b64h16"].s0_std == 0.02
    assert w["mixed_b4h16"].log_alpha_range == (0.0, 0.2) and w["mixed_b4h16"].eta_std == 2.0
