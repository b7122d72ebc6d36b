"""Seeded synthetic inputs for the gated delta rule workloads.

This module holds input recipes only: random draws, the host-side L2 normalisation the
recipes ask for, and rounding to the storage dtype.  It contains none of the method's
arithmetic, imports neither the HIP binding nor the oracle, and serves both sides.

The statistics follow the pages: queries and keys are L2-normalised per head before the
kernel (Qwen3.5 text encyclopedia page, note "The DeltaNet mixer"), betas are a sigmoid
write strength, decays are per-token log decays <= 0 whose kept fraction exp(g) ranges
over 0.05 ... 0.999 across heads (same note), and the state is float32 (Qwen3-Next page,
same note).  Head counts are the Qwen3.5-9B / Qwen3-Next ones: 16 query/key heads served
to 32 value heads, key/value width 128.

Every workload draws from one ``numpy.random.default_rng(seed)`` stream in the order
q, k, v, beta-normal, g-normal, initial state.  The packed workload's sequence lengths
come from a separate ``default_rng(seed)`` stream, drawn before anything else.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

try:  # torch is only needed for bf16 rounding (round-to-nearest-even)
    import torch
except Exception:  # pragma: no cover
    torch = None


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                      # rows (dense) or 1 (packed)
    T: int                      # tokens per row (dense) or total tokens (packed)
    H_qk: int
    H_v: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str                  # "fp32" or "bf16": storage type of q, k, v
    g_shift: float              # g = -softplus(N(0,1) + g_shift)
    s0_std: Optional[float]     # None: zero initial state; else N(0, s0_std^2)
    lengths: Optional[Tuple[int, ...]] = None   # packed sequence lengths (cu_seqlens)
    steps: int = 0              # decode: steps timed
    pool: int = 0               # decode: number of pre-drawn input sets, used cyclically

    @property
    def num_seqs(self) -> int:
        return len(self.lengths) if self.lengths is not None else self.B

    @property
    def tokens(self) -> int:
        return self.B * self.T


def packed_lengths(seed: int = 0, n: int = 8, lo: int = 1024, hi: int = 16384) -> Tuple[int, ...]:
    """Integer lengths drawn uniformly from [lo, hi], both ends included."""
    return tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, size=n))


_LENS = packed_lengths(0)

WORKLOADS = {
    # tiny fp32 case the oracle finishes instantly: every tensor compared in full
    "tiny_fp32": Workload("tiny_fp32", 1, 64, 2, 2, 16, 16, 16, "fp32", 0.0, None),
    # one DeltaNet layer's prefill of a 4096-token prompt, Qwen3.5-9B head shapes
    "prefill_t4096": Workload("prefill_t4096", 1, 4096, 16, 32, 128, 128, 64, "bf16", 2.0, None),
    # one decode step for 256 sequences, state updated in place, 1000 steps
    "decode_b256": Workload("decode_b256", 256, 1, 16, 32, 128, 128, 64, "bf16", 2.0, 0.02,
                            steps=1000, pool=16),
    # 8 packed prompts of seeded lengths, non-zero initial states
    "packed_8seq": Workload("packed_8seq", 1, int(sum(_LENS)), 16, 32, 128, 128, 64, "bf16", 2.0,
                            0.02, lengths=_LENS),
    # per-token state readout of a 2048-token prompt (4 GiB of fp32 states)
    "states_t2048": Workload("states_t2048", 1, 2048, 16, 32, 128, 128, 64, "bf16", 2.0, None),
}


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; returns float32 holding the exact values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype != "bf16":
        raise ValueError(dtype)
    if torch is None:
        raise RuntimeError("bf16 rounding needs torch")
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _unit(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _softplus(x):
    x = x.astype(np.float64)
    return np.where(x > 30, x, np.log1p(np.exp(np.minimum(x, 30))))


def make_inputs(w: Workload, seed: int = 0, T: Optional[int] = None, B: Optional[int] = None,
                lengths: Optional[Tuple[int, ...]] = None, g_shift: Optional[float] = None,
                normalise: bool = True, raw_norm_range: Optional[Tuple[float, float]] = None,
                s0_std: Optional[float] = "default"):
    """Draw one input set for workload ``w`` (optionally resized).

    Returns a dict of numpy arrays: ``q``, ``k`` [B, T, H_qk, d_k]; ``v`` [B, T, H_v, d_v];
    ``g``, ``beta`` [B, T, H_v] (float32); ``s0`` [N, H_v, d_k, d_v] float32 or None;
    ``cu_seqlens`` int32 [N+1] or None.  q, k, v hold values exactly representable in
    ``w.dtype`` (as float32).  With ``normalise=False`` q and k are left un-normalised and,
    if ``raw_norm_range`` is given, rescaled to per-token norms log-uniform in that range.
    """
    if lengths is None and w.lengths is not None and T is None:
        lengths = w.lengths
    if lengths is not None:
        B_, T_ = 1, int(sum(lengths))
    else:
        B_ = w.B if B is None else B
        T_ = w.T if T is None else T
    gs = w.g_shift if g_shift is None else g_shift
    std = w.s0_std if s0_std == "default" else s0_std
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B_, T_, w.H_qk, w.d_k))
    k = _normal(rng, (B_, T_, w.H_qk, w.d_k))
    v = _normal(rng, (B_, T_, w.H_v, w.d_v))
    bn = _normal(rng, (B_, T_, w.H_v))
    gn = _normal(rng, (B_, T_, w.H_v))
    N = len(lengths) if lengths is not None else B_
    s0 = None
    if std is not None:
        s0 = (_normal(rng, (N, w.H_v, w.d_k, w.d_v)) * np.float32(std)).astype(np.float32)
    if normalise:
        q, k = _unit(q), _unit(k)
    elif raw_norm_range is not None:
        lo, hi = np.log(raw_norm_range[0]), np.log(raw_norm_range[1])
        nq = np.exp(rng.uniform(lo, hi, size=q.shape[:-1] + (1,))).astype(np.float32)
        nk = np.exp(rng.uniform(lo, hi, size=k.shape[:-1] + (1,))).astype(np.float32)
        q, k = _unit(q) * nq, _unit(k) * nk
    out = {
        "q": round_to(q, w.dtype),
        "k": round_to(k, w.dtype),
        "v": round_to(v, w.dtype),
        "beta": (1.0 / (1.0 + np.exp(-bn.astype(np.float64)))).astype(np.float32),
        "g": (-_softplus(gn + gs)).astype(np.float32),
        "s0": s0,
        "cu_seqlens": None,
        "dtype": w.dtype,
    }
    if lengths is not None:
        out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return out


def make_decode_pool(w: Workload, seed: int = 0, pool: Optional[int] = None, B: Optional[int] = None):
    """Decode inputs: ``pool`` token sets (step s uses set s % pool) and one initial state.

    Returns q, k [pool, B, 1, H_qk, d_k]; v [pool, B, 1, H_v, d_v]; g, beta [pool, B, 1, H_v];
    s0 [B, H_v, d_k, d_v] float32 ~ N(0, s0_std^2).
    """
    P = w.pool if pool is None else pool
    B_ = w.B if B is None else B
    rng = np.random.default_rng(seed)
    q = _unit(_normal(rng, (P, B_, 1, w.H_qk, w.d_k)))
    k = _unit(_normal(rng, (P, B_, 1, w.H_qk, w.d_k)))
    v = _normal(rng, (P, B_, 1, w.H_v, w.d_v))
    bn = _normal(rng, (P, B_, 1, w.H_v))
    gn = _normal(rng, (P, B_, 1, w.H_v))
    s0 = (_normal(rng, (B_, w.H_v, w.d_k, w.d_v)) * np.float32(w.s0_std or 0.0)).astype(np.float32)
    return {
        "q": round_to(q, w.dtype), "k": round_to(k, w.dtype), "v": round_to(v, w.dtype),
        "beta": (1.0 / (1.0 + np.exp(-bn.astype(np.float64)))).astype(np.float32),
        "g": (-_softplus(gn + w.g_shift)).astype(np.float32),
        "s0": s0, "dtype": w.dtype,
    }


def make_mixer_inputs(w: Workload, seed: int = 0, T: Optional[int] = None, B: Optional[int] = None,
                      lengths: Optional[Tuple[int, ...]] = None, with_conv_state: bool = False):
    """Inputs of the mixer steps around the delta rule, for workload ``w``'s head layout.

    Returns a dict of numpy arrays:
      ``x``        [B, T, C] in ``w.dtype`` (as float32), C = 2 H_qk d_k + H_v d_v: the
                   convolution's input, channels q | k | v, ~ N(0, 1);
      ``conv_w``   [C, 4] float32 ~ N(0, 0.5^2);
      ``a``, ``b`` [B, T, H_v] float32 ~ N(0, 1);
      ``A_log``    [H_v] float32, log of U(1, 16);
      ``dt_bias``  [H_v] float32, log(expm1(dt)) with dt log-uniform in [1e-3, 1e-1];
      ``z``        [B, T, H_v, d_v] in ``w.dtype`` ~ N(0, 1): the output gate's input;
      ``norm_w``   [d_v] float32 ~ 1 + N(0, 0.1^2): the output norm's gain;
      ``conv_state`` [N, C, 3] float32 (dtype-exact values) ~ N(0, 1), or None;
      ``cu_seqlens`` int32 [N+1] or None.
    """
    if lengths is None and w.lengths is not None and T is None:
        lengths = w.lengths
    if lengths is not None:
        B_, T_ = 1, int(sum(lengths))
    else:
        B_ = w.B if B is None else B
        T_ = w.T if T is None else T
    C = 2 * w.H_qk * w.d_k + w.H_v * w.d_v
    N = len(lengths) if lengths is not None else B_
    rng = np.random.default_rng(seed)
    x = _normal(rng, (B_, T_, C))
    conv_w = (_normal(rng, (C, 4)) * np.float32(0.5)).astype(np.float32)
    a = _normal(rng, (B_, T_, w.H_v))
    b = _normal(rng, (B_, T_, w.H_v))
    A_log = np.log(rng.uniform(1.0, 16.0, size=w.H_v)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=w.H_v))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    z = _normal(rng, (B_, T_, w.H_v, w.d_v))
    norm_w = (1.0 + 0.1 * _normal(rng, (w.d_v,))).astype(np.float32)
    cs = round_to(_normal(rng, (N, C, 3)), w.dtype) if with_conv_state else None
    out = {"x": round_to(x, w.dtype), "conv_w": conv_w, "a": a, "b": b, "A_log": A_log, "dt_bias": dt_bias,
           "z": round_to(z, w.dtype), "norm_w": norm_w, "conv_state": cs, "cu_seqlens": None,
           "dtype": w.dtype}
    if lengths is not None:
        out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return out
