"""GPU parity of the chunked paths beyond the benchmark's bf16 / chunk-64 configuration.

fp32 q, k, v at key/value width 128 (the width of every head of the family, Qwen3.5 text
encyclopedia page, note "The DeltaNet mixer"; the float32 route is the one the page's
note "Loading" measures), at chunk 16, 32 and 64, and bf16 at chunk 32.  fp32 inputs are
held to max|d| <= 1e-4 x RMS(oracle) on o, the final state and the per-token states; bf16
inputs to 2e-2 x RMS on o and 1e-3 relative on the states.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import synth
from oracle import gdn_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, TOL_F32, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu


def _gdn():
    import gated_deltanet_linear_amd as gdn
    return gdn


def _w(dtype, H_qk=2, H_v=4):
    return dataclasses.replace(synth.WORKLOADS["prefill_t4096"], dtype=dtype, H_qk=H_qk, H_v=H_v)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_d128_all_heads_packed(chunk):
    """Every head, every output, packed ragged sequences with initial states."""
    gdn = _gdn()
    inp = synth.make_inputs(_w("fp32"), seed=11, lengths=(1, 63, 130, 70, 0, 33), g_shift=-1.0, s0_std=0.3)
    print(f"fp32 d128 chunk {chunk}: T={inp['q'].shape[1]}", flush=True)
    d = to_dev(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"],
                            cu_seqlens=inp["cu_seqlens"], want_states=True)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                               cu_seqlens=d["cu"], chunk=chunk)
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                      cu_seqlens=d["cu"], chunk=chunk)
    torch.cuda.synchronize()
    errs = [rel_max(host(o), ref["o"]), rel_max(host(fin), ref["final"]), rel_max(host(o2), ref["o"]),
            rel_max(host(fin2), ref["final"]), rel_max(host(st), ref["states"])]
    print("  errors", ["%.2e" % e for e in errs], flush=True)
    assert max(errs) <= TOL_F32


@pytest.mark.parametrize("chunk", [32, 64])
def test_fp32_d128_dense_rows_l2norm(chunk):
    """Dense rows, raw q/k normalised in the kernel, a reset inside a chunk."""
    gdn = _gdn()
    inp = synth.make_inputs(_w("fp32", 2, 6), seed=12, B=2, T=150, normalise=False,
                            raw_norm_range=(0.09, 4.1), s0_std=0.1)
    inp["g"][1, 77, 3] = -np.inf
    d = to_dev(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"], l2norm=True)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"], chunk=chunk,
                               l2norm=True)
    torch.cuda.synchronize()
    eo, ef = rel_max(host(o), ref["o"]), rel_max(host(fin), ref["final"])
    print(f"fp32 d128 l2norm chunk {chunk}: o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL_F32 and ef <= TOL_F32


def test_fp32_d128_prefill_t4096_sampled_heads():
    """The 4096-token prefill shape (16 qk / 32 v heads) in fp32, chunk 64: o, the final state
    and the per-token states of sampled heads against the oracle."""
    gdn = _gdn()
    w = dataclasses.replace(synth.WORKLOADS["prefill_t4096"], dtype="fp32")
    inp = synth.make_inputs(w, seed=0, g_shift=-3.0)
    heads = [0, 13, 31]
    print("fp32 d128 T4096: states call", flush=True)
    d = to_dev(inp)
    o, st, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64)
    torch.cuda.synchronize()
    o_c, fin_c = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64)
    torch.cuda.synchronize()
    st_h = host(st[:, :, heads])
    del st
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], heads=heads, want_states=True)
    errs = [rel_max(host(o_c[..., heads, :]), ref["o"][..., heads, :]),
            rel_max(host(fin_c[:, heads]), ref["final"][:, heads]),
            rel_max(host(o[..., heads, :]), ref["o"][..., heads, :]),
            rel_max(host(fin[:, heads]), ref["final"][:, heads]),
            rel_max(st_h, ref["states"])]
    print("  errors", ["%.2e" % e for e in errs], flush=True)
    assert max(errs) <= TOL_F32


def test_bf16_chunk32_all_heads():
    gdn = _gdn()
    inp = synth.make_inputs(_w("bf16"), seed=13, lengths=(200, 31, 96), s0_std=0.02)
    d = to_dev(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"],
                            cu_seqlens=inp["cu_seqlens"], want_states=True)
    o, st, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                    cu_seqlens=d["cu"], chunk=32)
    torch.cuda.synchronize()
    eo, ef, es = rel_max(host(o), ref["o"]), rel_fro(host(fin), ref["final"]), rel_fro(host(st), ref["states"])
    print(f"bf16 chunk 32: o {eo:.2e} final {ef:.2e} states {es:.2e}", flush=True)
    assert eo <= TOL_BF16_O and ef <= TOL_BF16_STATE and es <= TOL_BF16_STATE


def test_bf16_chunk64_dv48_all_heads():
    """Value width 48 (three 16-column tiles) on the bf16 chunk-64 path, packed, with states."""
    gdn = _gdn()
    w = dataclasses.replace(synth.WORKLOADS["prefill_t4096"], dtype="bf16", H_qk=2, H_v=4, d_v=48)
    inp = synth.make_inputs(w, seed=14, lengths=(130, 1, 64, 77), s0_std=0.02)
    d = to_dev(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"],
                            cu_seqlens=inp["cu_seqlens"], want_states=True)
    o, st, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                    cu_seqlens=d["cu"], chunk=64)
    torch.cuda.synchronize()
    eo, ef, es = rel_max(host(o), ref["o"]), rel_fro(host(fin), ref["final"]), rel_fro(host(st), ref["states"])
    print(f"bf16 chunk 64, d_v 48: o {eo:.2e} final {ef:.2e} states {es:.2e}", flush=True)
    assert eo <= TOL_BF16_O and ef <= TOL_BF16_STATE and es <= TOL_BF16_STATE
    assert eo <= 2e-3
