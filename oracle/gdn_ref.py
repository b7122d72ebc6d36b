"""gdn_ref: Python face of the fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  The HIP product path
never imports it and shares no code with it.

``recurrent`` marshals numpy arrays into ``libgdn_ref.so`` (oracle/gdn_ref.c),
the plain token-by-token recurrence in double precision:

    S <- exp(g_t) S;  S <- S + k_t (beta_t (v_t - S^T k_t))^T;  o_t = S^T q_t

(Qwen3.5 text encyclopedia page, note "The DeltaNet mixer": the delta-rule call
on l2-normed q/sqrt(128) and k, per-token log decay g, write strength beta; the
same page's value table for the zero initial state, state_output and states).

``build`` compiles the C file with gcc; it is what ``__graft_entry__.build``
calls, since building the checker is not using it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_ref.c")
_LIB = os.path.join(_HERE, "libgdn_ref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle/gdn_ref.c into oracle/libgdn_ref.so (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.gdn_ref_forward.restype = ctypes.c_int
        lib.gdn_ref_forward.argtypes = [I64, P, I64, I64, I64, I64, P, P, P, P, P, P,
                                        ctypes.c_double, ctypes.c_int, P, I64, P, P, P,
                                        ctypes.c_int]
        lib.gdn_ref_max_threads.restype = ctypes.c_int
        lib.gdn_ref_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdn_ref_max_threads())


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def recurrent(q, k, v, g, beta, s0=None, cu_seqlens=None, scale=None, l2norm=False,
              heads=None, want_o=True, want_final=True, want_states=False, nthreads=0):
    """Run the fp64 recurrence.

    Shapes follow the pages' tensors: q, k [B, T, H_qk, d_k] (or packed [T, H_qk, d_k]
    with ``cu_seqlens``), v [B, T, H_v, d_v], g and beta [B, T, H_v], float32 values.
    ``s0`` [N, H_v, d_k, d_v] (any float dtype, taken as float64) or None for zeros.
    ``scale`` defaults to d_k ** -0.5 and multiplies the (optionally normalised) query.
    ``heads`` restricts the work to a list of value heads (others are left zero).

    Returns a dict with float64 arrays: ``o`` [..., T, H_v, d_v], ``final``
    [N, H_v, d_k, d_v] and, if asked, ``states`` [..., T, len(heads), d_k, d_v].
    """
    lib = _load()
    q = _f32(q); k = _f32(k); v = _f32(v); g = _f32(g); beta = _f32(beta)
    if cu_seqlens is None:
        if q.ndim != 4:
            raise ValueError("dense inputs are [B, T, H, d]")
        B, T = q.shape[0], q.shape[1]
        cu = np.arange(B + 1, dtype=np.int64) * T
        lead = (B, T)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        if q.ndim == 4:
            if q.shape[0] != 1:
                raise ValueError("packed inputs have B == 1")
            lead = (1, q.shape[1])
        else:
            lead = (q.shape[0],)
    H_qk, d_k = q.shape[-2], q.shape[-1]
    H_v, d_v = v.shape[-2], v.shape[-1]
    n_seq = cu.shape[0] - 1
    T_tot = int(np.prod(lead))
    if int(cu[-1]) != T_tot or int(cu[0]) != 0:
        raise ValueError("cu_seqlens must start at 0 and end at the token count")
    if scale is None:
        scale = d_k ** -0.5
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64).reshape(n_seq, H_v, d_k, d_v)
    if heads is not None:
        heads = np.ascontiguousarray(heads, dtype=np.int64)
        n_heads = heads.shape[0]
    else:
        n_heads = H_v
    o = np.zeros(lead + (H_v, d_v), dtype=np.float64) if want_o else None
    fin = np.zeros((n_seq, H_v, d_k, d_v), dtype=np.float64) if want_final else None
    st = np.zeros(lead + (n_heads, d_k, d_v), dtype=np.float64) if want_states else None
    rc = lib.gdn_ref_forward(n_seq, _ptr(cu), H_qk, H_v, d_k, d_v, _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(beta), _ptr(s0), float(scale), int(bool(l2norm)),
                             _ptr(heads), n_heads, _ptr(o), _ptr(fin), _ptr(st), int(nthreads))
    if rc != 0:
        raise ValueError(f"gdn_ref_forward failed with code {rc}")
    out = {}
    if want_o:
        out["o"] = o
    if want_final:
        out["final"] = fin
    if want_states:
        out["states"] = st
    return out
