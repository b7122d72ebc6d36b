"""ctypes binding of libgdn (include/gdn.h).

Argument marshalling only: each function checks the tensors' device, dtype, shape and
contiguity, allocates outputs and the workspace through PyTorch when the caller passes
none, and calls the C entry point of the same name on the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no CPU fallback, and
a missing library raises ``GdnError``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same ABI (the host-sanitized copy of
# `python -m gated_deltanet_linear_amd.build --sanitize`, for CPU runs of the ABI tests).
library_path = os.environ.get("GDN_LIBRARY") or os.path.join(_PKG, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_QK_L2NORM = 1

_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class GdnShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H_qk", ctypes.c_int32),
                ("H_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


EXPORTS = ("gdn_chunk_fwd", "gdn_chunk_fwd_workspace", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_gated",
           "gdn_recurrent_step", "gdn_states_fwd",
           "gdn_states_fwd_strided", "gdn_states_fwd_workspace", "gdn_gated_norm", "gdn_recurrent_step_gated",
           "gdn_mixer_prologue", "gdn_set_timing_events", "gdn_status_string",
           "gdn_last_error", "gdn_version")

_lib = None


def load_library(path: Optional[str] = None):
    """Load libgdn.so (built in-tree by gated_deltanet_linear_amd.build) and declare its ABI."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path
    if not os.path.exists(p):
        raise GdnError(-1, f"libgdn is not built: {p} is missing "
                           "(run `python -m gated_deltanet_linear_amd.build`)")
    lib = ctypes.CDLL(p)
    P, S, Z, I = ctypes.c_void_p, ctypes.POINTER(GdnShape), ctypes.c_size_t, ctypes.c_int32
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [S, P, P, P, P, P, P, P, I, P, P, P, Z, P]
    lib.gdn_chunk_fwd_workspace.restype = Z
    lib.gdn_chunk_fwd_workspace.argtypes = [S, I]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [S, P, P, P, P, P, P, P, I, P, P, P]
    lib.gdn_states_fwd.restype = ctypes.c_int
    lib.gdn_states_fwd.argtypes = [S, P, P, P, P, P, P, P, I, P, P, P, P, Z, P]
    lib.gdn_states_fwd_strided.restype = ctypes.c_int
    lib.gdn_states_fwd_strided.argtypes = [S, P, P, P, P, P, P, P, I, P, P, I, I, I, P, P, Z, P]
    lib.gdn_states_fwd_workspace.restype = Z
    lib.gdn_states_fwd_workspace.argtypes = [S, I]
    lib.gdn_recurrent_step.restype = ctypes.c_int
    lib.gdn_recurrent_step.argtypes = [S, P, P, P, P, P, P, P, P]
    F = ctypes.c_float
    lib.gdn_recurrent_step_gated.restype = ctypes.c_int
    lib.gdn_recurrent_step_gated.argtypes = [S, P, P, P, P, P, P, P, P, F, P, P]
    lib.gdn_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdn_chunk_fwd_gated.argtypes = [S, P, P, P, P, P, P, P, I, P, P, F, P, P, P, Z, P]
    lib.gdn_gated_norm.restype = ctypes.c_int
    lib.gdn_gated_norm.argtypes = [S, P, P, P, F, P, P]
    lib.gdn_mixer_prologue.restype = ctypes.c_int
    lib.gdn_mixer_prologue.argtypes = [S, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_version.restype = ctypes.c_int
    lib.gdn_set_timing_events.restype = ctypes.c_int
    lib.gdn_set_timing_events.argtypes = [P, ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def _check(lib, st: int, what: str):
    if st != 0:
        msg = lib.gdn_last_error().decode()
        raise GdnError(st, f"{what}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(q, v, chunk, scale, l2norm, o_dtype, B, T):
    H_qk, d_k = q.shape[-2], q.shape[-1]
    H_v, d_v = v.shape[-2], v.shape[-1]
    if q.dtype not in _DT:
        raise ValueError(f"q dtype {q.dtype} is not float32 or bfloat16")
    if o_dtype not in _DT:
        raise ValueError(f"o_dtype {o_dtype} is not float32 or bfloat16")
    if chunk is None:
        chunk = 16 if q.shape[-1] == 16 else 64
    if scale is None:
        scale = d_k ** -0.5
    s = GdnShape(B, T, H_qk, H_v, d_k, d_v, chunk, float(scale), _DT[q.dtype], _DT[o_dtype],
                 GDN_QK_L2NORM if l2norm else 0)
    return s


def _common(q, k, v, g, beta, initial_state, cu_seqlens):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("libgdn runs on the GPU: tensors must be on a cuda (HIP) device")
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H_qk, d_k]")
    B, T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[-2], v.shape[-1]
    _need(q, "q", (B, T, H_qk, d_k), q.dtype, dev)
    _need(k, "k", (B, T, H_qk, d_k), q.dtype, dev)
    _need(v, "v", (B, T, H_v, d_v), q.dtype, dev)
    _need(g, "g", (B, T, H_v), torch.float32, dev)
    _need(beta, "beta", (B, T, H_v), torch.float32, dev)
    N = B
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need B == 1")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of N+1 offsets")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H_v, d_k, d_v), torch.float32, dev)
    return dev, B, T, H_qk, H_v, d_k, d_v, N


def gdn_chunk_fwd_workspace(shape: GdnShape, num_seqs: int) -> int:
    return int(load_library().gdn_chunk_fwd_workspace(ctypes.byref(shape), int(num_seqs)))


def gdn_states_fwd_workspace(shape: GdnShape, num_seqs: int) -> int:
    return int(load_library().gdn_states_fwd_workspace(ctypes.byref(shape), int(num_seqs)))


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None, chunk=None,
                  l2norm=False, o_dtype=torch.float32, output_final_state=True, o=None,
                  final_state=None, workspace=None):
    """The chunked prompt path.  Returns (o [B,T,H_v,d_v], final_state [N,H_v,d_k,d_v] or None)."""
    lib = load_library()
    dev, B, T, H_qk, H_v, d_k, d_v, N = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    s = _shape(q, v, chunk, scale, l2norm, o_dtype, B, T)
    if o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=o_dtype, device=dev)
    _need(o, "o", (B, T, H_v, d_v), o_dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H_v, d_k, d_v), torch.float32, dev)
    nseq = N if cu_seqlens is not None else 0
    need = int(lib.gdn_chunk_fwd_workspace(ctypes.byref(s), nseq))
    if need == 0:
        _check(lib, lib.gdn_chunk_fwd(ctypes.byref(s), *([None] * 7), nseq, None, None, None, 0, None),
               "gdn_chunk_fwd")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib.gdn_chunk_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(initial_state), _ptr(cu_seqlens), nseq, _ptr(o), _ptr(final_state),
                           _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(lib, st, "gdn_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None, chunk=None,
                          l2norm=False, o_dtype=torch.float32, output_final_state=True, o=None,
                          final_state=None):
    """gdn_chunk_fwd through the entry point that allocates nothing (its workspace is the
    library's static device scratch).  Pass o and final_state to allocate nothing here
    either.  Returns (o, final_state or None)."""
    lib = load_library()
    dev, B, T, H_qk, H_v, d_k, d_v, N = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    s = _shape(q, v, chunk, scale, l2norm, o_dtype, B, T)
    if o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=o_dtype, device=dev)
    _need(o, "o", (B, T, H_v, d_v), o_dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H_v, d_k, d_v), torch.float32, dev)
    nseq = N if cu_seqlens is not None else 0
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(initial_state), _ptr(cu_seqlens), nseq, _ptr(o), _ptr(final_state),
                                   _stream(dev))
    _check(lib, st, "gdn_chunk_fwd_noalloc")
    return o, final_state


def gdn_chunk_fwd_gated(q, k, v, g, beta, z, weight, eps=1e-6, initial_state=None, cu_seqlens=None,
                        scale=None, chunk=None, l2norm=False, o_dtype=torch.float32,
                        output_final_state=True, out=None, final_state=None, workspace=None):
    """The chunked prompt path followed by the mixer's output norm: returns
    (weight * o / sqrt(mean(o^2) + eps) * silu(z) per value head [B,T,H_v,d_v], final_state
    or None); z is [B,T,H_v,d_v] in q's dtype, weight [d_v] fp32."""
    lib = load_library()
    dev, B, T, H_qk, H_v, d_k, d_v, N = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    _need(z, "z", (B, T, H_v, d_v), q.dtype, dev)
    _need(weight, "weight", (d_v,), torch.float32, dev)
    s = _shape(q, v, chunk, scale, l2norm, o_dtype, B, T)
    if out is None:
        out = torch.empty((B, T, H_v, d_v), dtype=o_dtype, device=dev)
    _need(out, "out", (B, T, H_v, d_v), o_dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H_v, d_k, d_v), torch.float32, dev)
    nseq = N if cu_seqlens is not None else 0
    need = int(lib.gdn_chunk_fwd_workspace(ctypes.byref(s), nseq))
    if need == 0:
        _check(lib, lib.gdn_chunk_fwd_gated(ctypes.byref(s), *([None] * 7), nseq, None, None, float(eps),
                                            None, None, None, 0, None), "gdn_chunk_fwd_gated")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib.gdn_chunk_fwd_gated(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(initial_state), _ptr(cu_seqlens), nseq, _ptr(z), _ptr(weight),
                                 float(eps), _ptr(out), _ptr(final_state), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(lib, st, "gdn_chunk_fwd_gated")
    return out, final_state


def gdn_states_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None, chunk=None,
                   l2norm=False, o_dtype=torch.float32, want_o=True, output_final_state=True,
                   states=None, o=None, final_state=None, workspace=None, t_begin=0, t_end=None, t_step=1):
    """gdn_chunk_fwd plus the per-token states.  Returns (o or None, states, final or None).

    With the default selection every token's state is kept (states [B, T, H_v, d_k, d_v]); otherwise
    the tokens t_begin, t_begin + t_step, ... < t_end of every row (gdn_states_fwd_strided; states
    [B, n, H_v, d_k, d_v], n = ceil((t_end - t_begin) / t_step))."""
    lib = load_library()
    dev, B, T, H_qk, H_v, d_k, d_v, N = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    s = _shape(q, v, chunk, scale, l2norm, o_dtype, B, T)
    t_end = T if t_end is None else int(t_end)
    t_begin, t_step = int(t_begin), int(t_step)
    strided = (t_begin, t_end, t_step) != (0, T, 1)
    if not (0 <= t_begin <= t_end <= T and t_step >= 1):
        raise GdnError(2, f"token selection [{t_begin}, {t_end}) step {t_step} is not within [0, {T})")
    n_sel = (t_end - t_begin + t_step - 1) // t_step
    if want_o and o is None:
        o = torch.empty((B, T, H_v, d_v), dtype=o_dtype, device=dev)
    if o is not None:
        _need(o, "o", (B, T, H_v, d_v), o_dtype, dev)
    if states is None:
        states = torch.empty((B, n_sel, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    _need(states, "states", (B, n_sel, H_v, d_k, d_v), torch.float32, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (N, H_v, d_k, d_v), torch.float32, dev)
    nseq = N if cu_seqlens is not None else 0
    need = int(lib.gdn_states_fwd_workspace(ctypes.byref(s), nseq))
    if need == 0:
        _check(lib, lib.gdn_states_fwd(ctypes.byref(s), *([None] * 7), nseq, None, None, None, None, 0,
                                       None), "gdn_states_fwd")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if strided:
        st = lib.gdn_states_fwd_strided(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(initial_state), _ptr(cu_seqlens), nseq, _ptr(o), _ptr(states),
                                        t_begin, t_end, t_step, _ptr(final_state), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev))
        _check(lib, st, "gdn_states_fwd_strided")
        return o, states, final_state
    st = lib.gdn_states_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(initial_state), _ptr(cu_seqlens), nseq, _ptr(o), _ptr(states),
                            _ptr(final_state), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev))
    _check(lib, st, "gdn_states_fwd")
    return o, states, final_state


def gdn_recurrent_step(q, k, v, g, beta, state, scale=None, l2norm=False, o_dtype=torch.float32, o=None):
    """One decode token per sequence; ``state`` [B,H_v,d_k,d_v] fp32 is updated in place.
    q, k [B,1,H_qk,d_k]; v [B,1,H_v,d_v]; g, beta [B,1,H_v].  Returns o [B,1,H_v,d_v]."""
    lib = load_library()
    dev, B, T, H_qk, H_v, d_k, d_v, N = _common(q, k, v, g, beta, None, None)
    if T != 1:
        raise ValueError("the decode step takes one token per sequence (T == 1)")
    _need(state, "state", (B, H_v, d_k, d_v), torch.float32, dev)
    s = _shape(q, v, 1, scale, l2norm, o_dtype, B, T)
    if o is None:
        o = torch.empty((B, 1, H_v, d_v), dtype=o_dtype, device=dev)
    _need(o, "o", (B, 1, H_v, d_v), o_dtype, dev)
    st = lib.gdn_recurrent_step(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(state), _ptr(o), _stream(dev))
    _check(lib, st, "gdn_recurrent_step")
    return o


def gdn_recurrent_step_gated(q, k, v, g, beta, state, z, weight, eps=1e-6, scale=None, l2norm=False,
                             o_dtype=torch.float32, out=None):
    """gdn_recurrent_step with the output norm fused: returns
    weight * o / sqrt(mean(o^2) + eps) * silu(z) per value head, [B,1,H_v,d_v]; z is
    [B,1,H_v,d_v] in q's dtype, weight [d_v] fp32.  ``state`` is updated in place."""
    lib = load_library()
    dev, B, T, H_qk, H_v, d_k, d_v, N = _common(q, k, v, g, beta, None, None)
    if T != 1:
        raise ValueError("the decode step takes one token per sequence (T == 1)")
    _need(state, "state", (B, H_v, d_k, d_v), torch.float32, dev)
    _need(z, "z", (B, 1, H_v, d_v), q.dtype, dev)
    _need(weight, "weight", (d_v,), torch.float32, dev)
    s = _shape(q, v, 1, scale, l2norm, o_dtype, B, T)
    if out is None:
        out = torch.empty((B, 1, H_v, d_v), dtype=o_dtype, device=dev)
    _need(out, "out", (B, 1, H_v, d_v), o_dtype, dev)
    st = lib.gdn_recurrent_step_gated(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(state), _ptr(z), _ptr(weight), float(eps), _ptr(out), _stream(dev))
    _check(lib, st, "gdn_recurrent_step_gated")
    return out


def gdn_gated_norm(y, z, weight, eps=1e-6, out=None):
    """The mixer's output norm, per (token, value head): weight * y / sqrt(mean(y^2) + eps)
    * silu(z).  y [B,T,H_v,d_v] fp32 or bf16 (the delta rule's o); z [B,T,H_v,d_v] fp32 or
    bf16; weight [d_v] fp32.  ``out`` (y's dtype) may be y itself."""
    lib = load_library()
    dev = y.device
    if dev.type != "cuda":
        raise ValueError("libgdn runs on the GPU: tensors must be on a cuda (HIP) device")
    if y.dim() != 4:
        raise ValueError("y must be [B, T, H_v, d_v]")
    B, T, H_v, d_v = y.shape
    if y.dtype not in _DT or z.dtype not in _DT:
        raise ValueError("y and z must be float32 or bfloat16")
    _need(y, "y", (B, T, H_v, d_v), y.dtype, dev)
    _need(z, "z", (B, T, H_v, d_v), z.dtype, dev)
    _need(weight, "weight", (d_v,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(y)
    _need(out, "out", (B, T, H_v, d_v), y.dtype, dev)
    s = GdnShape(B, T, 1, H_v, 1, d_v, 1, 1.0, _DT[z.dtype], _DT[y.dtype], 0)
    st = lib.gdn_gated_norm(ctypes.byref(s), _ptr(y), _ptr(z), _ptr(weight), float(eps), _ptr(out),
                            _stream(dev))
    _check(lib, st, "gdn_gated_norm")
    return out


def gdn_mixer_prologue(x, conv_w, a, b, A_log, dt_bias, H_qk, d_k, H_v, d_v, conv_state=None,
                       cu_seqlens=None, update_conv_state=False, conv_state_out=None):
    """The mixer's steps before the delta rule: q, k, v = split(silu(conv1d(x))) with a
    causal width-4 depthwise filter, beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias).

    x [B,T,C] fp32 or bf16 with C = 2 H_qk d_k + H_v d_v (channels q | k | v); conv_w [C,4]
    fp32 (tap 3 multiplies the current token); a, b [B,T,H_v] fp32; A_log, dt_bias [H_v]
    fp32; conv_state [N,C,3] fp32 or None (zeros).  With update_conv_state the new
    convolution state is written back into conv_state (in place); with conv_state_out it
    goes there.  Returns (q, k, v, g, beta, conv_state_out or None).
    """
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("libgdn runs on the GPU: tensors must be on a cuda (HIP) device")
    if x.dim() != 3 or x.dtype not in _DT:
        raise ValueError("x must be [B, T, C] float32 or bfloat16")
    B, T, C = x.shape
    if C != 2 * H_qk * d_k + H_v * d_v:
        raise ValueError(f"x has {C} channels, expected 2*H_qk*d_k + H_v*d_v = {2 * H_qk * d_k + H_v * d_v}")
    _need(x, "x", (B, T, C), x.dtype, dev)
    _need(conv_w, "conv_w", (C, 4), torch.float32, dev)
    _need(a, "a", (B, T, H_v), torch.float32, dev)
    _need(b, "b", (B, T, H_v), torch.float32, dev)
    _need(A_log, "A_log", (H_v,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H_v,), torch.float32, dev)
    N = B
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need B == 1")
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
        N = cu_seqlens.numel() - 1
    if conv_state is not None:
        _need(conv_state, "conv_state", (N, C, 3), torch.float32, dev)
    if update_conv_state:
        if conv_state is None:
            raise ValueError("update_conv_state needs conv_state")
        conv_state_out = conv_state
    if conv_state_out is not None:
        _need(conv_state_out, "conv_state_out", (N, C, 3), torch.float32, dev)
    q = torch.empty((B, T, H_qk, d_k), dtype=x.dtype, device=dev)
    k = torch.empty((B, T, H_qk, d_k), dtype=x.dtype, device=dev)
    v = torch.empty((B, T, H_v, d_v), dtype=x.dtype, device=dev)
    g = torch.empty((B, T, H_v), dtype=torch.float32, device=dev)
    beta = torch.empty((B, T, H_v), dtype=torch.float32, device=dev)
    s = GdnShape(B, T, H_qk, H_v, d_k, d_v, 1, 1.0, _DT[x.dtype], GDN_F32, 0)
    nseq = N if cu_seqlens is not None else 0
    st = lib.gdn_mixer_prologue(ctypes.byref(s), _ptr(x), _ptr(conv_w), _ptr(conv_state), _ptr(conv_state_out),
                                _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), nseq,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _stream(dev))
    _check(lib, st, "gdn_mixer_prologue")
    return q, k, v, g, beta, conv_state_out


def plan_status(workspace: torch.Tensor) -> int:
    """The device status word a chunked call leaves at the start of its workspace: 0, or bit 0
    when the call's cu_seqlens were malformed (every kernel then did nothing), bit 1 when a
    stored o or final-state value of the bf16 chunk-64 path is not finite."""
    return int(workspace[:4].view(torch.int32).item())


def gdn_set_timing_events(events, n: int):
    """Install (or with events=None remove) the per-kernel timing hook of the chunked calls.
    ``events`` is a ctypes array of hipEvent_t handles (torch.cuda.Event.cuda_event)."""
    lib = load_library()
    _check(lib, lib.gdn_set_timing_events(events, int(n)), "gdn_set_timing_events")
