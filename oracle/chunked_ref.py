"""Chunked fp64 form of the gated delta rule, used only to check the oracle's recurrence.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` alone).  It is a second, independent
derivation of the same result as ``gdn_ref.recurrent``: a plain numpy reading of the
chunk algebra, with no blocking, fusion or reordering beyond the algebra itself.

Derivation (per value head; the recurrence is the one the Qwen3.5 text encyclopedia
page states in its note "The DeltaNet mixer"):  write one token's update as
S_r = a_r S_{r-1} + k_r u_r^T with a_r = exp(g_r) and u_r = b_r (v_r - a_r S_{r-1}^T k_r).
Inside a chunk whose first token is 0, unrolling gives

    S_r = e^{G_r} S_0 + sum_{i<=r} e^{G_r - G_i} k_i u_i^T,     G_r = sum_{m<=r} g_m,

so the write vectors satisfy the unit-lower-triangular system

    (I + A) U = diag(b) V - diag(b e^{G}) K S_0,   A[r,i] = b_r e^{G_r-G_i} (k_r . k_i), i < r,

i.e. U = T diag(b) V - T diag(b e^G) K S_0 with T = (I + A)^{-1} (the UT / WY form),
and then

    O       = diag(e^G) Q S_0 + (M o Q K^T) U,      M[r,i] = e^{G_r-G_i} for i <= r, else 0
    S_chunk = e^{G_last} S_0 + K^T diag(e^{G_last - G}) U.

Every decay factor e^{G_r - G_i} is formed from the segment sum sum_{i<m<=r} g_m, never as
a quotient of two exponentials, so a token with g = -inf zeroes exactly the factors that
span it and produces no NaN.  T is built row by row by forward substitution, so that a test
can pin it against a library inverse.
"""
from __future__ import annotations

import numpy as np


def unit_lower_inverse(A):
    """(I + A)^{-1} for strictly lower-triangular A, by forward substitution over rows."""
    n = A.shape[0]
    T = np.zeros((n, n), dtype=np.float64)
    for r in range(n):
        T[r, r] = 1.0
        for i in range(r):
            # row r of (I + A) T = I:  T[r,:] = e_r - sum_{m<r} A[r,m] T[m,:]
            T[r, :] -= A[r, i] * T[i, :]
    return T


def _segment_decay(gc):
    """D[r, i] = sum_{i<m<=r} g_m for i <= r (0 on the diagonal), -inf above it."""
    n = gc.shape[0]
    D = np.full((n, n), -np.inf)
    for r in range(n):
        acc = 0.0
        D[r, r] = 0.0
        for i in range(r - 1, -1, -1):
            acc += gc[i + 1]
            D[r, i] = acc
    return D


def chunk_step(S0, q, k, v, g, beta):
    """One chunk for one head.  q, k [C, d_k] (already normalised and scaled as wanted),
    v [C, d_v], g, beta [C].  Returns (O [C, d_v], S_end [d_k, d_v], U [C, d_v])."""
    C = q.shape[0]
    D = _segment_decay(g)                      # e^{G_r - G_i} = exp(D[r, i])
    head = np.array([np.sum(g[: r + 1]) for r in range(C)])        # G_r
    tail = np.array([np.sum(g[r + 1:]) for r in range(C)])          # G_last - G_r
    M = np.exp(D)                               # lower triangular incl. diagonal
    A = np.tril(beta[:, None] * M * (k @ k.T), -1)
    T = unit_lower_inverse(A)
    U = T @ (beta[:, None] * v) - T @ ((beta * np.exp(head))[:, None] * k) @ S0
    O = np.exp(head)[:, None] * (q @ S0) + (M * (q @ k.T)) @ U
    S_end = np.exp(head[-1]) * S0 + k.T @ (np.exp(tail)[:, None] * U)
    return O, S_end, U


def chunked(q, k, v, g, beta, chunk, s0=None, cu_seqlens=None, scale=None, l2norm=False):
    """Same contract as ``gdn_ref.recurrent`` (o and final state), computed chunk by chunk.
    Chunks restart at every sequence start; the last chunk of a sequence may be short."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if cu_seqlens is None:
        B, Tn = q.shape[:2]
        cu = np.arange(B + 1) * Tn
        lead = q.shape[:2]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        lead = q.shape[:-2]
    H_qk, d_k = q.shape[-2:]
    H_v, d_v = v.shape[-2:]
    qf = q.reshape(-1, H_qk, d_k)
    kf = k.reshape(-1, H_qk, d_k)
    vf = v.reshape(-1, H_v, d_v)
    gf = g.reshape(-1, H_v)
    bf = beta.reshape(-1, H_v)
    if scale is None:
        scale = d_k ** -0.5
    n_seq = len(cu) - 1
    group = H_v // H_qk
    o = np.zeros(vf.shape)
    fin = np.zeros((n_seq, H_v, d_k, d_v))
    for n in range(n_seq):
        for h in range(H_v):
            j = h // group
            S = np.zeros((d_k, d_v)) if s0 is None else np.array(s0[n, h], dtype=np.float64)
            for c0 in range(cu[n], cu[n + 1], chunk):
                c1 = min(c0 + chunk, cu[n + 1])
                kc = kf[c0:c1, j]
                qc = qf[c0:c1, j]
                if l2norm:
                    kc = kc / np.sqrt(np.sum(kc * kc, axis=1, keepdims=True) + 1e-6)
                    qc = qc / np.sqrt(np.sum(qc * qc, axis=1, keepdims=True) + 1e-6)
                O, S, _ = chunk_step(S, scale * qc, kc, vf[c0:c1, h], gf[c0:c1, h], bf[c0:c1, h])
                o[c0:c1, h] = O
            fin[n, h] = S
    return {"o": o.reshape(tuple(lead) + (H_v, d_v)), "final": fin}
