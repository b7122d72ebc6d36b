"""Pins of the oracle against the pure-torch route the pages name (CPU only).

The Qwen3.5 text encyclopedia page (03 · The Notes, "Loading") says its DeltaNet values
come from transformers' pure-torch delta rule when the fused kernels are absent, and its
note "The DeltaNet mixer" names the kernel's arguments (l2-normed q scaled by 1/sqrt(d_k),
l2-normed k, v, g, beta; query/key heads shared by repeat_interleave) and the output norm
norm(y, gate=silu(z)) with gain weight.  transformers is an independent implementation of
those same steps, so agreement here pins the oracle's recurrence, its chunked form and its
gated RMS norm to something other than themselves:

- ``gdn_ref.recurrent`` and ``chunked_ref.chunked`` against
  ``torch_recurrent_gated_delta_rule`` and ``torch_chunk_gated_delta_rule``, with the
  in-kernel l2 norm, GQA (repeat_interleave on this side), a non-zero initial state and
  (token-by-token route only: the chunked one forms e^{G_r}/e^{G_i} and gives NaN there)
  a reset (g = -inf); compared in fp32, the precision transformers computes in;
- ``mixer_ref.gated_rmsnorm`` against ``Qwen3_5RMSNormGated``, including rows whose mean
  square is below eps.

The oracle never imports transformers; these tests skip where it is not importable.
"""
import numpy as np
import pytest

from oracle import chunked_ref, gdn_ref, mixer_ref

torch = pytest.importorskip("torch")
try:
    from transformers.models.qwen3_5 import modeling_qwen3_5 as tfm
except Exception:  # pragma: no cover - depends on the installed transformers
    tfm = None

pytestmark = pytest.mark.skipif(tfm is None, reason="transformers' Qwen3.5 modelling code is not importable")


def _inputs(seed, T, H_qk, H_v, d, reset_at=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, T, H_qk, d)) * rng.uniform(0.1, 4.0, (1, T, H_qk, 1))
    k = rng.standard_normal((1, T, H_qk, d)) * rng.uniform(0.1, 4.0, (1, T, H_qk, 1))
    v = rng.standard_normal((1, T, H_v, d))
    g = -np.logaddexp(0.0, rng.standard_normal((1, T, H_v)) - 1.0)
    if reset_at is not None:
        g[0, reset_at, :] = -np.inf
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H_v))))
    s0 = rng.standard_normal((1, H_v, d, d)) * 0.3
    # the values both sides see: rounded to fp32 once
    return [np.asarray(x, np.float32) for x in (q, k, v, g, beta, s0)]


def _torch_rule(fn, q, k, v, g, beta, s0, **kw):
    R = v.shape[2] // q.shape[2]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    o, fin = fn(t(q).repeat_interleave(R, dim=2), t(k).repeat_interleave(R, dim=2), t(v), t(g), t(beta),
                initial_state=t(s0), output_final_state=True, use_qk_l2norm_in_kernel=True, **kw)
    return o.double().numpy(), fin.double().numpy()


@pytest.mark.parametrize("H_qk,H_v", [(2, 4), (1, 3), (3, 3)])
@pytest.mark.parametrize("reset", [None, 70])
def test_recurrence_matches_transformers(H_qk, H_v, reset):
    q, k, v, g, beta, s0 = _inputs(3, 150, H_qk, H_v, 32, reset_at=reset)
    ref = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, l2norm=True)
    routes = [(tfm.torch_recurrent_gated_delta_rule, {})]
    if reset is None:
        routes.append((tfm.torch_chunk_gated_delta_rule, {"chunk_size": 16}))
    for fn, kw in routes:
        o, fin = _torch_rule(fn, q, k, v, g, beta, s0, **kw)
        rms = np.sqrt(np.mean(ref["o"] ** 2))
        assert np.max(np.abs(o - ref["o"])) <= 2e-5 * rms, fn.__name__
        rel = np.linalg.norm(fin - ref["final"]) / np.linalg.norm(ref["final"])
        assert rel <= 1e-5, fn.__name__


def test_chunked_form_matches_transformers():
    q, k, v, g, beta, s0 = _inputs(4, 90, 2, 4, 16)
    mine = chunked_ref.chunked(q, k, v, g, beta, 16, s0=s0, l2norm=True)
    o, fin = _torch_rule(tfm.torch_chunk_gated_delta_rule, q, k, v, g, beta, s0, chunk_size=16)
    rms = np.sqrt(np.mean(mine["o"] ** 2))
    assert np.max(np.abs(o - mine["o"])) <= 2e-5 * rms
    assert np.linalg.norm(fin - mine["final"]) / np.linalg.norm(mine["final"]) <= 1e-5


def test_oracle_scale_and_norm_are_the_pages():
    # transformers scales q by d_k^-1/2 after the l2 norm and normalises with an eps of
    # 1e-6 inside the square root; leaving out the scale or the norm moves the result far
    # outside the agreement above (the page reports 42% on real data without them)
    q, k, v, g, beta, s0 = _inputs(5, 64, 2, 4, 32)
    o, fin = _torch_rule(tfm.torch_recurrent_gated_delta_rule, q, k, v, g, beta, s0)
    bad = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, l2norm=True, scale=1.0)
    assert np.max(np.abs(o - bad["o"])) > 0.1 * np.sqrt(np.mean(o ** 2))
    bad = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, l2norm=False)
    assert np.linalg.norm(fin - bad["final"]) > 0.05 * np.linalg.norm(fin)


@pytest.mark.parametrize("eps", [1e-6, 1e-5])
def test_gated_norm_matches_transformers(eps):
    rng = np.random.default_rng(6)
    d = 128
    y = rng.standard_normal((6, 4, d))
    y[1, 2] *= 1e-3      # mean square ~1e-6: eps moves it by ~30%
    y[2, 0] *= 2e-4      # mean square ~4e-8: eps dominates
    y[3, 1] = 0.0        # zero row
    z = rng.standard_normal((6, 4, d)) * 2.0
    w = rng.standard_normal(d)
    y, z, w = (np.asarray(x, np.float32) for x in (y, z, w))
    mod = tfm.Qwen3_5RMSNormGated(d, eps=eps)
    with torch.no_grad():
        mod.weight.copy_(torch.from_numpy(w))
        out = mod(torch.from_numpy(y), gate=torch.from_numpy(z)).double().numpy()
    ref = mixer_ref.gated_rmsnorm(y, z, w, eps=eps)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True) + 1e-30
    assert np.max(np.abs(out - ref) / scale) <= 2e-6
    # the small rows differ clearly from an eps-free norm: eps is what makes them agree
    free = mixer_ref.gated_rmsnorm(y, z, w, eps=0.0)
    assert np.max(np.abs(free[1, 2] - out[1, 2])) > 1e-2 * np.max(np.abs(out[1, 2]))
