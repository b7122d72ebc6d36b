"""fp64 references for the steps around the delta rule in the DeltaNet mixer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  The HIP product path
never imports it and shares no code with it.

The Qwen3.5 text encyclopedia page (note "The DeltaNet mixer") and the
Qwen3-Next encyclopedia page (same note) describe the mixer around the kernel;
restated here for channel c, token t and value head h, sigma the logistic
function:

  * a causal convolution of width 4 with one filter per channel,
    xc[t,c] = sum_{i<4} w[c,i] x[t-3+i,c], then SiLU, xc sigma(xc), and a split of
    the channels into q, k and v;
  * the write strength beta = sigma(b) and the log decay
    g = -e^{A_log[h]} softplus(a[t,h] + dt_bias[h]);
  * the gated delta rule on the l2-normed q times d_k^{-1/2}, the l2-normed k, v,
    g and beta;
  * on each value head's output y[t,h,:], an RMS norm with gain weight, multiplied
    by the SiLU of the gate input z[t,h,:], before the output projection.

and the module listing on the first page shows the convolution as a depthwise
Conv1d of kernel size 4 with padding 3 and no bias, and the norm as an RMS norm
whose gain is its weight (the page's note "The readout is the plain
projection": the DeltaNet's own output norm multiplies by its weight, every
other RMS norm of the family by 1 + weight).

Readings taken where the pages leave a step open:
  * the norm is over one value head's d_v outputs, y / sqrt(mean(y^2) + eps),
    then times weight, then times silu(z): the gate multiplies the normalised
    output (the pages' norm(y, gate=...) with gain weight); eps = 1e-6, the
    epsilon every RMS norm of the family prints in the module listing;
  * the causal convolution of width 4 over a sequence sees, before its first
    token, the three previous inputs of that channel when a convolution state is
    given and zeros otherwise (a padding of 3 on the left, output truncated to
    the sequence's length);
  * x_qkv's channels are q (H_qk d_k), then k (H_qk d_k), then v (H_v d_v), the
    plain split of the first page's in_proj_qkv output.
"""
from __future__ import annotations

import numpy as np


def silu(x):
    """x * sigmoid(x), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), in fp64, without overflow for large x."""
    x = np.asarray(x, dtype=np.float64)
    return np.logaddexp(0.0, x)


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gated_rmsnorm(y, z, weight, eps=1e-6):
    """norm(y, gate=silu(z)) with gain weight, over the last axis (one head's d_v values).

    y, z: [..., d_v]; weight: [d_v].  Returns fp64 [..., d_v]:
        weight * y / sqrt(mean(y^2) + eps) * silu(z).
    """
    y = np.asarray(y, dtype=np.float64)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return np.asarray(weight, dtype=np.float64) * (y / np.sqrt(ms + eps)) * silu(z)


def causal_conv(x, w, state=None, cu_seqlens=None):
    """Depthwise causal convolution of width K (no bias), per sequence.

    x: [T, Ch] (one packed axis of tokens); w: [Ch, K]; state: [N, Ch, K-1] or None,
    the K-1 inputs that precede each sequence (oldest first).  Output
    out[t, c] = sum_{i<K} w[c, i] * x[t - (K-1) + i, c], with x before a sequence's first
    token taken from its state (zeros without one).  Returns (out [T, Ch], new_state
    [N, Ch, K-1]: the last K-1 inputs each sequence has seen, counting its state).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, Ch = x.shape
    K = w.shape[1]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    out = np.zeros((T, Ch))
    new_state = np.zeros((N, Ch, K - 1))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        prev = np.zeros((K - 1, Ch)) if state is None else np.asarray(state[n], np.float64).T
        xs = np.concatenate([prev, x[a:b]], axis=0)          # [K-1 + L, Ch]
        for t in range(b - a):
            out[a + t] = np.sum(w.T * xs[t:t + K], axis=0)
        new_state[n] = xs[xs.shape[0] - (K - 1):].T
    return out, new_state


def prologue(x_qkv, conv_w, a, b, A_log, dt_bias, H_qk, d_k, H_v, d_v, conv_state=None,
             cu_seqlens=None):
    """The mixer's steps before the delta rule: q, k, v = split(silu(conv(x_qkv))),
    beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias).

    x_qkv: [T, 2 H_qk d_k + H_v d_v]; conv_w: [channels, 4]; a, b: [T, H_v];
    A_log, dt_bias: [H_v].  Returns dict q, k [T, H_qk, d_k], v [T, H_v, d_v], g, beta
    [T, H_v] and conv_state [N, channels, 3], all fp64.
    """
    c, st = causal_conv(x_qkv, conv_w, conv_state, cu_seqlens)
    c = silu(c)
    T = c.shape[0]
    nq = H_qk * d_k
    q = c[:, :nq].reshape(T, H_qk, d_k)
    k = c[:, nq:2 * nq].reshape(T, H_qk, d_k)
    v = c[:, 2 * nq:].reshape(T, H_v, d_v)
    beta = sigmoid(b)
    g = -np.exp(np.asarray(A_log, np.float64)) * softplus(np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64))
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "conv_state": st}
