"""The C ABI on the CPU: the library loads, exports every symbol include/gdn.h declares,
and refuses invalid calls on the host before any launch (no compute calls here: every
pointer below is a fake address that validation rejects before it could be used)."""
import ctypes
import os
import re

import pytest

from gated_deltanet_linear_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(binding.library_path):
        pytest.skip("libgdn.so is not built")
    return binding.load_library()


def test_every_declared_symbol_is_exported():
    lib = _lib()
    with open(os.path.join(ROOT, "include", "gdn.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text))
    assert declared == set(binding.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.gdn_version() >= 100
    assert lib.gdn_status_string(0) == b"GDN_OK"


def _shape(**kw):
    base = dict(B=1, T=128, H_qk=16, H_v=32, d_k=128, d_v=128, chunk=64, scale=128 ** -0.5,
                dtype=binding.GDN_BF16, o_dtype=binding.GDN_F32, flags=0)
    base.update(kw)
    return binding.GdnShape(**base)


FAKE = 1 << 40   # 16-byte aligned fake device address, never dereferenced


def _ptrs(n, step=1 << 32):
    return [ctypes.c_void_p(FAKE + i * step) for i in range(n)]


def _call_chunk(lib, s, ws_bytes=None, **over):
    q, k, v, g, b, s0, o, fin, ws = _ptrs(9)
    args = dict(q=q, k=k, v=v, g=g, b=b, s0=None, cu=None, n=0, o=o, fin=fin, ws=ws)
    args.update(over)
    need = lib.gdn_chunk_fwd_workspace(ctypes.byref(s), args["n"])
    return lib.gdn_chunk_fwd(ctypes.byref(s), args["q"], args["k"], args["v"], args["g"], args["b"],
                             args["s0"], args["cu"], args["n"], args["o"], args["fin"], args["ws"],
                             need if ws_bytes is None else ws_bytes, None)


def test_validation_errors_return_codes():
    lib = _lib()
    s = _shape()
    assert lib.gdn_chunk_fwd_workspace(ctypes.byref(s), 0) > 0
    assert _call_chunk(lib, _shape(H_v=24)) == 2                       # H_v % H_qk
    assert _call_chunk(lib, _shape(dtype=7)) == 3                      # dtype
    assert _call_chunk(lib, _shape(d_k=64)) == 4                       # no kernel built
    assert _call_chunk(lib, s, q=None) == 1                            # NULL input
    assert _call_chunk(lib, s, ws_bytes=16) == 7                       # workspace too small
    assert _call_chunk(lib, s, q=ctypes.c_void_p(FAKE + 8)) == 6       # misaligned
    # o overlapping v
    q, k, v, g, b, s0, o, fin, ws = _ptrs(9)
    assert _call_chunk(lib, s, o=ctypes.c_void_p(v.value + 256)) == 5
    # final_state == initial_state exactly is allowed past validation; a shifted overlap is not
    assert _call_chunk(lib, s, s0=s0, fin=ctypes.c_void_p(s0.value + 4096)) == 5
    assert b"GDN_ERR_ALIAS" in lib.gdn_last_error()
    # decode step: T must be 1
    st = lib.gdn_recurrent_step(ctypes.byref(_shape(T=2)), *_ptrs(7), None)
    assert st == 2
    assert lib.gdn_chunk_fwd_workspace(ctypes.byref(_shape(H_v=24)), 0) == 0


def test_workspace_query_matches_layout():
    lib = _lib()
    s = _shape(T=4096)
    w = lib.gdn_chunk_fwd_workspace(ctypes.byref(s), 0)
    ws = lib.gdn_states_fwd_workspace(ctypes.byref(s), 0)
    chunks = 4096 // 64
    per = 2 * 6 * 64 * 16 + 8 * 64 * 4  # T diag(beta) fragments (fp16 hi and lo) and per-token factors
    assert w >= chunks * 32 * per
    assert ws >= w + 4096 * 32 * 128 * 4 + chunks * 32 * 128 * 128 * 4


def test_strided_states_selection_is_validated():
    """gdn_states_fwd_strided refuses a token selection outside [0, T) or a step below 1, and
    sizes states by the selection (an overlap with the selection's extent is refused)."""
    lib = _lib()
    s = _shape()   # T = 128
    need = lib.gdn_states_fwd_workspace(ctypes.byref(s), 0)
    q, k, v, g, b, o, st, fin, ws = _ptrs(9)

    def call(t0, t1, step, states=st):
        return lib.gdn_states_fwd_strided(ctypes.byref(s), q, k, v, g, b, None, None, 0, o, states,
                                          t0, t1, step, fin, ws, need, None)
    assert call(-1, 128, 1) == 2
    assert call(0, 129, 1) == 2
    assert call(5, 4, 1) == 2
    assert call(0, 128, 0) == 2
    assert b"token selection" in lib.gdn_last_error()
    assert call(0, 128, 1, states=None) == 1
    # 3 selected tokens of 32 heads x 128 x 128 fp32 = 6 MiB of states: placed to end inside v
    states = ctypes.c_void_p(v.value - 2 * 1024 * 1024)
    assert call(0, 128, 50, states=states) == 5


def test_gated_chunk_call_is_validated():
    """gdn_chunk_fwd_gated: the norm's widths, eps >= 0, z and weight present, aligned and
    disjoint from every output."""
    lib = _lib()
    q, k, v, g, b, o, fin, ws, z, w = _ptrs(10)

    def call(s, z=z, w=w, eps=1e-6, out=o):
        need = lib.gdn_chunk_fwd_workspace(ctypes.byref(s), 0)
        return lib.gdn_chunk_fwd_gated(ctypes.byref(s), q, k, v, g, b, None, None, 0, z, w, eps, out, fin,
                                       ws, need, None)
    s = _shape()
    assert call(_shape(d_v=48)) == 4                                   # no norm of width 48
    assert call(s, eps=-1.0) == 2
    assert call(s, eps=float("nan")) == 2
    assert call(s, z=None) == 1
    assert call(s, w=None) == 1
    assert call(s, z=ctypes.c_void_p(z.value + 2)) == 6                # z: 4 elements
    assert call(s, w=ctypes.c_void_p(w.value + 4)) == 6                # weight: 16 bytes
    assert call(s, out=ctypes.c_void_p(z.value + 256)) == 5            # out overlaps z
    assert b"overlaps z" in lib.gdn_last_error()
    assert call(s, w=ctypes.c_void_p(fin.value + 64)) == 5             # final_state overlaps weight
    assert b"overlaps weight" in lib.gdn_last_error()
