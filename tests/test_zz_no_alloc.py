"""gdn_chunk_fwd_noalloc, the chunked entry point that allocates nothing, against
gdn_chunk_fwd on the same inputs, through the C ABI (GPU).

Two calls in a row on the static scratch, the second on a smaller input than the first
(the array keeps the first call's contents); each must equal the workspace entry point's
result (they share their kernels, so bit for bit) and meet the bf16 parity bar against
the oracle.  A shape whose workspace exceeds the static scratch is refused before any
launch.  Collected last, so that it runs alone or after every other GPU test.
"""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import binding, synth
from oracle import gdn_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu

GDN_ERR_WORKSPACE = 7


def _noalloc_abi(lib, d, nseq, o, fin):
    """gdn_chunk_fwd_noalloc called directly through ctypes."""
    q = d["q"]
    B, T, H_qk, d_k = q.shape
    H_v, d_v = d["v"].shape[-2:]
    s = binding.GdnShape(B, T, H_qk, H_v, d_k, d_v, 64, float(d_k) ** -0.5, binding.GDN_BF16, binding.GDN_F32, 0)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gdn_chunk_fwd_noalloc(ctypes.byref(s), P(q), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]),
                                     P(d["s0"]), P(d["cu"]), nseq, P(o), P(fin), stream)


@pytest.mark.parametrize("case", ["two_calls"])
def test_noalloc_matches_workspace_entry_point(case):
    lib = binding.load_library()
    w = synth.WORKLOADS["prefill_t4096"]
    inputs = [synth.make_inputs(w, seed=21, T=700, s0_std=0.02),                       # larger first
              synth.make_inputs(w, seed=22, lengths=(130, 1, 64, 77), s0_std=0.02)]    # then smaller, packed
    for i, inp in enumerate(inputs):
        print(f"noalloc call {i}: T={inp['q'].shape[1]} packed={inp['cu_seqlens'] is not None}", flush=True)
        d = to_dev(inp)
        nseq = 0 if inp["cu_seqlens"] is None else len(inp["cu_seqlens"]) - 1
        o_ws, fin_ws = binding.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                             cu_seqlens=d["cu"])
        N = fin_ws.shape[0]
        o = torch.full_like(o_ws, float("nan"))
        fin = torch.full_like(fin_ws, float("nan"))
        st = _noalloc_abi(lib, d, nseq, o, fin)
        assert st == 0, lib.gdn_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws) and torch.equal(fin, fin_ws)
        ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"],
                                cu_seqlens=inp["cu_seqlens"])
        eo, ef = rel_max(host(o), ref["o"]), rel_fro(host(fin), ref["final"])
        print(f"  o {eo:.2e}  final {ef:.2e}  (N={N})", flush=True)
        assert eo <= TOL_BF16_O and ef <= TOL_BF16_STATE


def test_noalloc_refuses_shapes_beyond_its_scratch():
    lib = binding.load_library()
    s = binding.GdnShape(1, 1 << 20, 16, 32, 128, 128, 64, 128 ** -0.5, binding.GDN_BF16, binding.GDN_F32, 0)
    assert lib.gdn_chunk_fwd_workspace(ctypes.byref(s), 0) > (64 << 20)
    fake = ctypes.c_void_p(1 << 40)   # never dereferenced: the call is refused on the host
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(s), fake, fake, fake, fake, fake, None, None, 0, fake, None, None)
    assert st == GDN_ERR_WORKSPACE
    assert b"static scratch" in lib.gdn_last_error()
