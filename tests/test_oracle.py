"""Pins of the fp64 oracle (oracle/gdn_ref.c) against facts fixed by the pages and by
mathematics, not by the oracle itself.

Every test here runs on the CPU.  Each pin is chosen so that a plausible mistake in the
oracle (a dropped decay, a read before the write, a wrong sign in the delta, the wrong
query/key head, a transposed state) fails at least one of them:

- hand-worked five-token example (tests/golden/hand_worked_d2.json), exact rationals;
- one-token closed form o = beta (k . q) v;
- delta-rule invariant: g = 0, beta = 1, unit k  =>  S'^T k = v for any S;
- reset: g = -inf restarts the recurrence from a zero state;
- pure decay (beta = 0): closed form;
- orthonormal keys, beta = 1, g = 0: causal linear attention;
- brute-force product of per-token affine maps on random inputs;
- the chunked UT/WY form (oracle/chunked_ref.py) with chunk sizes 1, 2, 4, 16;
- its triangular inverse against numpy.linalg.inv;
- split invariance (carrying the final state), packed == separate sequences;
- the repeat_interleave head mapping and the l2-norm flag.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import chunked_ref, gdn_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H_qk, H_v, dk, dv, unit=True, gshift=0.0):
    q = rng.standard_normal((B, T, H_qk, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H_qk, dk)).astype(np.float32)
    if unit:
        q = (q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
        k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H_v, dv)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H_v))))).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H_v)) + gshift))).astype(np.float32)
    return q, k, v, g, beta


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_d2.json")) as f:
        fx = json.load(f)
    gmap = {"-inf": -np.inf, "ln0.5": math.log(0.5)}
    g = np.array([gmap.get(x, x) if isinstance(x, str) else x for x in fx["g"]], dtype=np.float32)
    sh = lambda a: np.asarray(a, dtype=np.float32).reshape(1, 5, 1, 2)
    r = gdn_ref.recurrent(sh(fx["q"]), sh(fx["k"]), sh(fx["v"]), g.reshape(1, 5, 1),
                          np.asarray(fx["beta"], dtype=np.float32).reshape(1, 5, 1),
                          scale=1.0, want_states=True)
    np.testing.assert_allclose(r["o"].reshape(5, 2), np.asarray(fx["o"]), rtol=1e-8, atol=1e-8)
    np.testing.assert_allclose(r["final"].reshape(2, 2), np.asarray(fx["final"]), rtol=1e-8, atol=1e-8)
    np.testing.assert_allclose(r["states"].reshape(5, 2, 2), np.asarray(fx["states"]),
                               rtol=1e-8, atol=1e-8)
    # tokens 0..3 involve only exactly representable values: bit-exact there
    assert np.array_equal(r["o"].reshape(5, 2)[:4], np.asarray(fx["o"])[:4])


@pytest.mark.parametrize("l2norm", [False, True])
def test_one_token_closed_form(l2norm):
    rng = np.random.default_rng(1)
    q, k, v, g, beta = rand_inputs(rng, 1, 1, 2, 4, 16, 8, unit=False)
    scale = 0.3
    r = gdn_ref.recurrent(q, k, v, g, beta, scale=scale, l2norm=l2norm)
    kd, qd = k.astype(np.float64), q.astype(np.float64)
    if l2norm:
        kd = kd / np.sqrt(np.sum(kd * kd, -1, keepdims=True) + 1e-6)
        qd = qd / np.sqrt(np.sum(qd * qd, -1, keepdims=True) + 1e-6)
    for h in range(4):
        j = h // 2
        kh, qh = kd[0, 0, j], scale * qd[0, 0, j]
        b = float(beta[0, 0, h])
        S1 = b * np.outer(kh, v[0, 0, h])
        np.testing.assert_allclose(r["final"][0, h], S1, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["o"][0, 0, h], b * (kh @ qh) * v[0, 0, h], rtol=1e-12, atol=1e-15)


def exact_unit_vectors(rng, n, d, nnz):
    """Vectors with nnz entries of +-1/sqrt(nnz) (nnz a power of 4): exactly unit in fp32."""
    val = 1.0 / math.sqrt(nnz)
    assert val == np.float32(val)
    out = np.zeros((n, d), dtype=np.float32)
    for i in range(n):
        idx = rng.choice(d, size=nnz, replace=False)
        out[i, idx] = val * rng.choice([-1.0, 1.0], size=nnz)
    return out


@pytest.mark.parametrize("d", [16, 128])
def test_delta_rule_invariant(d):
    """g = 0, beta = 1, unit k: after the write the memory returns v for k exactly."""
    rng = np.random.default_rng(2)
    T = 6
    k = exact_unit_vectors(rng, T, d, 16 if d == 16 else 64).reshape(1, T, 1, d)
    q = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    g = np.zeros((1, T, 1), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    s0 = rng.standard_normal((1, 1, d, d)) * 0.5
    r = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, want_states=True)
    for t in range(T):
        St = r["states"][0, t, 0]
        np.testing.assert_allclose(St.T @ k[0, t, 0].astype(np.float64), v[0, t, 0], atol=1e-13)


def test_reset_on_minus_inf():
    rng = np.random.default_rng(3)
    q, k, v, g, beta = rand_inputs(rng, 1, 24, 2, 4, 16, 16)
    s0 = rng.standard_normal((1, 4, 16, 16))
    t0 = 9
    g[0, t0, :] = -np.inf
    full = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, want_states=True)
    fresh = gdn_ref.recurrent(q[:, t0:], k[:, t0:], v[:, t0:], g[:, t0:], beta[:, t0:], s0=None,
                              want_states=True)
    np.testing.assert_allclose(full["o"][:, t0:], fresh["o"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(full["final"], fresh["final"], rtol=1e-13, atol=1e-14)
    assert np.all(np.isfinite(full["o"]))
    # the state right after the reset token is beta k v^T, whatever came before
    for h in range(4):
        kk = k[0, t0, h // 2].astype(np.float64)
        np.testing.assert_allclose(full["states"][0, t0, h],
                                   beta[0, t0, h] * np.outer(kk, v[0, t0, h]), rtol=1e-13, atol=1e-15)


def test_pure_decay_closed_form():
    rng = np.random.default_rng(4)
    T = 12
    q, k, v, g, _ = rand_inputs(rng, 1, T, 1, 2, 8, 8)
    beta = np.zeros((1, T, 2), np.float32)
    s0 = rng.standard_normal((1, 2, 8, 8))
    scale = 0.7
    r = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, scale=scale)
    for h in range(2):
        G = np.cumsum(g[0, :, h].astype(np.float64))
        for t in range(T):
            np.testing.assert_allclose(r["o"][0, t, h], math.exp(G[t]) * s0[0, h].T @ (scale * q[0, t, 0].astype(np.float64)),
                                       rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r["final"][0, h], math.exp(G[-1]) * s0[0, h], rtol=1e-12)


def hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_orthonormal_keys_linear_attention():
    """beta = 1, g = 0, S0 = 0 and orthonormal keys: the delta rule is causal linear attention."""
    d = 16
    K = (hadamard(d) / 4.0).astype(np.float32)          # rows exactly orthonormal in fp32
    rng = np.random.default_rng(5)
    K = K[rng.permutation(d)]
    T = 10
    k = K[:T].reshape(1, T, 1, d)
    q = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    r = gdn_ref.recurrent(q, k, v, np.zeros((1, T, 1), np.float32), np.ones((1, T, 1), np.float32),
                          scale=1.0)
    kd, qd, vd = k[0, :, 0].astype(np.float64), q[0, :, 0].astype(np.float64), v[0, :, 0].astype(np.float64)
    att = np.tril(qd @ kd.T)
    np.testing.assert_allclose(r["o"][0, :, 0], att @ vd, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["final"][0, 0], kd.T @ vd, rtol=1e-12, atol=1e-13)


def test_brute_force_product_form():
    """S_T = prod_t[a_t (I - b_t k_t k_t^T)] S0 + sum_i prod_{t>i}[...] b_i k_i v_i^T on raw inputs."""
    rng = np.random.default_rng(6)
    T, d = 7, 5
    q, k, v, g, beta = rand_inputs(rng, 1, T, 1, 1, d, 3, unit=False)
    s0 = rng.standard_normal((1, 1, d, 3))
    r = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, scale=1.0, want_states=True)
    kd = k[0, :, 0].astype(np.float64)
    vd = v[0, :, 0].astype(np.float64)
    a = np.exp(g[0, :, 0].astype(np.float64))
    b = beta[0, :, 0].astype(np.float64)
    F = [a[t] * (np.eye(d) - b[t] * np.outer(kd[t], kd[t])) for t in range(T)]
    for t_end in range(T):
        S = s0[0, 0].copy()
        for t in range(t_end + 1):
            S = F[t] @ S
        for i in range(t_end + 1):
            P = np.eye(d)
            for t in range(i + 1, t_end + 1):
                P = F[t] @ P
            S = S + P @ (b[i] * np.outer(kd[i], vd[i]))
        np.testing.assert_allclose(r["states"][0, t_end, 0], S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["o"][0, t_end, 0], S.T @ q[0, t_end, 0].astype(np.float64),
                                   rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("chunk", [1, 2, 4, 16])
def test_chunked_equals_recurrent(chunk):
    rng = np.random.default_rng(7)
    T = 37                                      # ragged against every chunk size
    q, k, v, g, beta = rand_inputs(rng, 2, T, 2, 4, 16, 8, unit=False)
    g[0, 5, 1] = -np.inf                        # a reset inside a chunk
    g[1, 16, 3] = -np.inf                       # a reset on a chunk boundary
    s0 = rng.standard_normal((2, 4, 16, 8)) * 0.3
    ref = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, l2norm=True)
    chk = chunked_ref.chunked(q, k, v, g, beta, chunk, s0=s0, l2norm=True)
    np.testing.assert_allclose(chk["o"], ref["o"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(chk["final"], ref["final"], rtol=1e-10, atol=1e-12)


def test_chunk_inverse_matches_library():
    rng = np.random.default_rng(8)
    A = np.tril(rng.standard_normal((64, 64)) * 0.1, -1)
    T = chunked_ref.unit_lower_inverse(A)
    np.testing.assert_allclose(T, np.linalg.inv(np.eye(64) + A), rtol=1e-12, atol=1e-13)


def test_split_invariance_and_packing():
    rng = np.random.default_rng(9)
    T, T1 = 50, 23
    q, k, v, g, beta = rand_inputs(rng, 1, T, 2, 4, 16, 16)
    s0 = rng.standard_normal((1, 4, 16, 16)) * 0.1
    whole = gdn_ref.recurrent(q, k, v, g, beta, s0=s0)
    a = gdn_ref.recurrent(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], s0=s0)
    b = gdn_ref.recurrent(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], s0=a["final"])
    np.testing.assert_allclose(np.concatenate([a["o"], b["o"]], 1), whole["o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b["final"], whole["final"], rtol=1e-13, atol=1e-15)
    # packing two independent sequences with cu_seqlens == running them separately
    q2, k2, v2, g2, b2 = rand_inputs(rng, 1, 11, 2, 4, 16, 16)
    s1 = rng.standard_normal((1, 4, 16, 16)) * 0.1
    cat = lambda x, y: np.concatenate([x[0], y[0]], 0)
    cu = np.array([0, T, T + 11])
    packed = gdn_ref.recurrent(cat(q, q2), cat(k, k2), cat(v, v2), cat(g, g2), cat(beta, b2),
                               s0=np.concatenate([s0, s1]), cu_seqlens=cu)
    sep2 = gdn_ref.recurrent(q2, k2, v2, g2, b2, s0=s1)
    np.testing.assert_allclose(packed["o"][:T], whole["o"][0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(packed["o"][T:], sep2["o"][0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(packed["final"][1], sep2["final"][0], rtol=1e-13, atol=1e-15)


def test_empty_sequence_keeps_state():
    rng = np.random.default_rng(10)
    q, k, v, g, beta = rand_inputs(rng, 1, 5, 1, 2, 4, 4)
    s0 = rng.standard_normal((3, 2, 4, 4))
    r = gdn_ref.recurrent(q[0], k[0], v[0], g[0], beta[0], s0=s0, cu_seqlens=np.array([0, 0, 5, 5]))
    assert np.array_equal(r["final"][0], s0[0])
    assert np.array_equal(r["final"][2], s0[2])


def test_head_mapping_is_repeat_interleave():
    """H_qk = 2, H_v = 6: value head h reads query/key head h // 3 (not h % 2)."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta = rand_inputs(rng, 1, 9, 2, 6, 8, 8)
    r = gdn_ref.recurrent(q, k, v, g, beta)
    rep = lambda x: np.repeat(x, 3, axis=2)     # numpy's repeat == torch.repeat_interleave
    rr = gdn_ref.recurrent(rep(q), rep(k), v, g, beta)
    np.testing.assert_allclose(r["o"], rr["o"], rtol=1e-14, atol=1e-15)
    mod = gdn_ref.recurrent(q[:, :, [0, 1, 0, 1, 0, 1]], k[:, :, [0, 1, 0, 1, 0, 1]], v, g, beta)
    assert np.max(np.abs(mod["o"] - r["o"])) > 1e-2


def test_l2norm_flag_and_negative_control():
    """The flag normalises q and k; leaving the norm and scale out changes the result a lot
    (the Qwen3.5 page reports a 42% state error on real activations)."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta = rand_inputs(rng, 1, 40, 2, 4, 16, 16, unit=False)
    q *= 3.0
    k *= 0.5
    flag = gdn_ref.recurrent(q, k, v, g, beta, l2norm=True)
    nq = q.astype(np.float64) / np.sqrt(np.sum(q.astype(np.float64) ** 2, -1, keepdims=True) + 1e-6)
    nk = k.astype(np.float64) / np.sqrt(np.sum(k.astype(np.float64) ** 2, -1, keepdims=True) + 1e-6)
    host = chunked_ref.chunked(nq, nk, v, g, beta, 4)
    np.testing.assert_allclose(flag["o"], host["o"], rtol=1e-10, atol=1e-12)
    raw = gdn_ref.recurrent(q, k, v, g, beta, l2norm=False, scale=1.0)
    rel = np.linalg.norm(raw["final"] - flag["final"]) / np.linalg.norm(flag["final"])
    assert rel > 0.2


def test_head_subset_and_states_consistency():
    rng = np.random.default_rng(13)
    q, k, v, g, beta = rand_inputs(rng, 2, 20, 2, 4, 8, 8)
    s0 = rng.standard_normal((2, 4, 8, 8))
    full = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, want_states=True)
    sub = gdn_ref.recurrent(q, k, v, g, beta, s0=s0, heads=[3, 1], want_states=True)
    np.testing.assert_array_equal(sub["o"][:, :, [3, 1]], full["o"][:, :, [3, 1]])
    np.testing.assert_array_equal(sub["states"], full["states"][:, :, [3, 1]])
    np.testing.assert_array_equal(full["states"][:, -1], full["final"])
    scale = 8 ** -0.5
    o_from_states = np.einsum("bthkv,bthk->bthv", full["states"],
                              scale * np.repeat(q.astype(np.float64), 2, axis=2))
    np.testing.assert_allclose(o_from_states, full["o"], rtol=1e-12, atol=1e-14)


def test_threads_do_not_change_result():
    rng = np.random.default_rng(14)
    q, k, v, g, beta = rand_inputs(rng, 3, 30, 2, 4, 16, 16)
    a = gdn_ref.recurrent(q, k, v, g, beta, nthreads=1)
    b = gdn_ref.recurrent(q, k, v, g, beta, nthreads=4)
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["final"], b["final"])
