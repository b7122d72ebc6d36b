"""Pins of the mixer references (oracle/mixer_ref.py) against values worked by hand and
against library routines, not against the references themselves.  CPU only.

- gated RMS norm: hand-worked examples whose values are exact multiples of ln 3, with
  eps = 0 (tests/golden/gated_norm_d4.json) and with an eps of the order of each row's
  mean square (tests/golden/gated_norm_eps_d4.json), scale invariance, a zero row;
- causal convolution: impulse response (the filter reversed, nothing before the
  impulse), numpy.convolve per channel, split invariance through the carried state,
  restart at every packed sequence;
- gates: softplus and sigmoid closed forms, the split order of q, k, v.
"""
import json
import math
import os

import numpy as np

from oracle import mixer_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_gated_norm_hand_worked():
    with open(os.path.join(GOLDEN, "gated_norm_d4.json")) as f:
        fx = json.load(f)
    ln3 = math.log(3.0)
    z = np.array([c * ln3 for c in fx["z_in_ln3"]])
    y = mixer_ref.gated_rmsnorm(np.array(fx["y"], float), z, np.array(fx["weight"], float), eps=0.0)
    want = np.array([c * ln3 for c in fx["out_in_ln3"]])
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-14)


def test_gated_norm_hand_worked_with_eps():
    # eps sits inside the square root, added to the mean square: rows whose mean square
    # is comparable to eps pin both its place and its value
    with open(os.path.join(GOLDEN, "gated_norm_eps_d4.json")) as f:
        fx = json.load(f)
    ln3 = math.log(3.0)
    z = np.array(fx["z_in_ln3"], float) * ln3
    y = mixer_ref.gated_rmsnorm(np.array(fx["y"], float), z, np.array(fx["weight"], float), eps=fx["eps"])
    want = np.array(fx["out_in_ln3"], float) * ln3
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-15)


def test_gated_norm_scale_invariance_and_zero_row():
    rng = np.random.default_rng(0)
    y = rng.standard_normal((5, 3, 128))
    z = rng.standard_normal((5, 3, 128))
    w = rng.standard_normal(128)
    a = mixer_ref.gated_rmsnorm(y, z, w, eps=0.0)
    b = mixer_ref.gated_rmsnorm(7.5 * y, z, w, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    # each row of y / rms(y) has unit mean square: with a unit gain and silu(z) -> z for
    # large z, out / z has mean square 1
    big = np.full((5, 3, 128), 40.0)
    u = mixer_ref.gated_rmsnorm(y, big, np.ones(128), eps=0.0) / 40.0
    np.testing.assert_allclose(np.mean(u * u, axis=-1), 1.0, rtol=1e-12)
    zero = mixer_ref.gated_rmsnorm(np.zeros((2, 128)), z[0, :2], w, eps=1e-6)
    assert np.all(zero == 0.0)


def test_conv_impulse_response():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((3, 4))
    x = np.zeros((9, 3))
    x[2, 1] = 1.0
    out, _ = mixer_ref.causal_conv(x, w)
    want = np.zeros((9, 3))
    for t in range(2, 6):
        want[t, 1] = w[1, 3 - (t - 2)]      # the filter read backwards from the impulse
    np.testing.assert_array_equal(out, want)


def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 5))
    w = rng.standard_normal((5, 4))
    out, _ = mixer_ref.causal_conv(x, w)
    for c in range(5):
        ref = np.convolve(x[:, c], w[c, ::-1])[:40]
        np.testing.assert_allclose(out[:, c], ref, rtol=1e-12, atol=1e-12)


def test_conv_state_carries_split_and_packing_restarts():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((30, 4))
    w = rng.standard_normal((4, 4))
    s0 = rng.standard_normal((1, 4, 3))
    full, s_full = mixer_ref.causal_conv(x, w, s0)
    a, s_a = mixer_ref.causal_conv(x[:11], w, s0)
    b, s_b = mixer_ref.causal_conv(x[11:], w, s_a)
    np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(s_b, s_full)
    np.testing.assert_array_equal(s_full[0], x[-3:].T)        # the last three inputs
    # packed: each sequence starts from zeros, as if run alone
    cu = np.array([0, 7, 7, 30])
    packed, st = mixer_ref.causal_conv(x, w, None, cu)
    np.testing.assert_allclose(packed[:7], mixer_ref.causal_conv(x[:7], w)[0], rtol=1e-12)
    np.testing.assert_allclose(packed[7:], mixer_ref.causal_conv(x[7:], w)[0], rtol=1e-12)
    assert np.all(st[1] == 0.0)                                 # the empty sequence saw nothing
    # a short sequence keeps part of its incoming state
    _, s_short = mixer_ref.causal_conv(x[:1], w, s0)
    np.testing.assert_array_equal(s_short[0], np.concatenate([s0[0][:, 1:], x[:1].T], axis=1))


def test_gates_closed_forms_and_split_order():
    A_log = np.log(np.array([2.0, 0.5]))
    dt_bias = np.array([0.0, 1.0])
    a = np.array([[0.0, -1.0], [50.0, 49.0]])
    b = np.array([[0.0, math.log(3.0)], [-math.log(3.0), 0.0]])
    H_qk, d_k, H_v, d_v = 1, 2, 2, 2
    C = 2 * H_qk * d_k + H_v * d_v
    x = np.arange(2 * C, dtype=float).reshape(2, C) / 10.0
    w = np.zeros((C, 4))
    w[:, 3] = 1.0                               # identity filter: conv(x)[t] = x[t]
    r = mixer_ref.prologue(x, w, a, b, A_log, dt_bias, H_qk, d_k, H_v, d_v)
    ln2 = math.log(2.0)
    np.testing.assert_allclose(r["g"][0], [-2.0 * ln2, -0.5 * ln2], rtol=1e-14)
    np.testing.assert_allclose(r["g"][1], [-2.0 * 50.0, -0.5 * 50.0], rtol=1e-14)   # softplus(50) = 50
    np.testing.assert_allclose(r["beta"], [[0.5, 0.75], [0.25, 0.5]], rtol=1e-14)
    sx = mixer_ref.silu(x)
    np.testing.assert_array_equal(r["q"].reshape(2, -1), sx[:, :2])
    np.testing.assert_array_equal(r["k"].reshape(2, -1), sx[:, 2:4])
    np.testing.assert_array_equal(r["v"].reshape(2, -1), sx[:, 4:])
    # silu closed forms: silu(0) = 0, silu(ln 3) = 0.75 ln 3
    np.testing.assert_allclose(mixer_ref.silu([0.0, math.log(3.0)]), [0.0, 0.75 * math.log(3.0)], rtol=1e-15)
