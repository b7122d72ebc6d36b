"""GPU parity of the head-wide chain (taken for bf16 chunk-64 calls at d_v 128 once sequences
x value heads reach the compute-unit count; one workgroup per sequence and value head on dense
rows, two per head, each with half its columns, on packed sequences) in the cases the other
tests leave out:

- raw (un-normalised) keys and queries with the in-kernel l2 norm and no initial state, on the
  plain, gated and per-token-states calls, every head (packed: the split heads);
- more sequences than the plan kernel orders by length (4096), which then keeps their own order;
- dense rows (whole heads per workgroup): the plain and per-token-states calls, every head.

Tolerances as for the bf16 prompt path: o (or the normed output) 2e-2 x RMS and inside 1e-2,
final state and states 1e-3 relative.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import synth
from oracle import gdn_ref, mixer_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["packed_8seq"]
EPS = 1e-6


def _gdn():
    import gated_deltanet_linear_amd as gdn
    return gdn


def test_wide_l2norm_raw_keys_no_initial_state():
    gdn = _gdn()
    lens = (65, 1, 130, 0, 77, 64, 200, 33, 5)
    print(f"packed lengths {lens}, raw q/k norms in [0.3, 5], l2norm in the kernel", flush=True)
    inp = synth.make_inputs(W, seed=41, lengths=lens, normalise=False, raw_norm_range=(0.3, 5.0), s0_std=None)
    assert inp["s0"] is None
    d = to_dev(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu_seqlens=inp["cu_seqlens"],
                            l2norm=True, want_states=True, heads=[0, 17, 31])
    full = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu_seqlens=inp["cu_seqlens"],
                             l2norm=True)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], l2norm=True)
    torch.cuda.synchronize()
    eo, ef = rel_max(host(o), full["o"]), rel_fro(host(fin), full["final"])
    print(f"  chunk: o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL_BF16_O and eo <= 1e-2 and ef <= TOL_BF16_STATE
    # the gated call on the same inputs (the norm inside the chain)
    mi = synth.make_mixer_inputs(W, seed=42, lengths=lens)
    z = torch.from_numpy(mi["z"]).to("cuda", torch.bfloat16)
    nw = torch.from_numpy(mi["norm_w"]).cuda()
    out, fin2 = gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["g"], d["beta"], z, nw, eps=EPS,
                                        cu_seqlens=d["cu"], l2norm=True)
    torch.cuda.synchronize()
    want = mixer_ref.gated_rmsnorm(full["o"], mi["z"], mi["norm_w"], eps=EPS)
    eg = rel_max(host(out), want)
    print(f"  gated: out {eg:.2e}", flush=True)
    assert eg <= TOL_BF16_O and eg <= 1e-2
    assert torch.equal(fin2, fin)
    # the states (head-wide chain, then the stream kernel), sampled heads
    o3, st, fin3 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                                      l2norm=True)
    torch.cuda.synchronize()
    es = rel_fro(host(st[:, :, [0, 17, 31]]), ref["states"])
    print(f"  states: {es:.2e}", flush=True)
    assert es <= TOL_BF16_STATE
    assert torch.equal(o3, o) and torch.equal(fin3, fin)


def test_more_sequences_than_the_length_order_covers():
    gdn = _gdn()
    rng = np.random.default_rng(43)
    lens = tuple(int(x) for x in rng.integers(0, 4, size=4100))
    print(f"{len(lens)} packed sequences of 0-3 tokens ({sum(lens)} tokens), 32 value heads", flush=True)
    inp = synth.make_inputs(W, seed=44, lengths=lens, s0_std=0.02)
    d = to_dev(inp)
    heads = [3, 28]
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"],
                            cu_seqlens=inp["cu_seqlens"], heads=heads)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                               cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    eo = rel_max(host(o[..., heads, :]), ref["o"][..., heads, :])
    ef = rel_fro(host(fin[:, heads]), ref["final"][:, heads])
    print(f"  o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL_BF16_O and eo <= 1e-2 and ef <= TOL_BF16_STATE
    # empty sequences hand their initial state straight through
    empty = [n for n, L in enumerate(lens) if L == 0][:5]
    assert torch.equal(fin[empty], d["s0"][empty])


def test_wide_dense_rows_whole_heads():
    gdn = _gdn()
    print("dense B=8 T=150, 32 value heads (whole heads per workgroup), chunk and states", flush=True)
    inp = synth.make_inputs(W, seed=45, B=8, T=150, s0_std=0.02)
    d = to_dev(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"],
                            want_states=True, heads=[1, 30])
    full = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"])
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    eo, ef = rel_max(host(o), full["o"]), rel_fro(host(fin), full["final"])
    print(f"  chunk: o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL_BF16_O and eo <= 1e-2 and ef <= TOL_BF16_STATE
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    es = rel_fro(host(st[:, :, [1, 30]]), ref["states"])
    print(f"  states: {es:.2e}", flush=True)
    assert es <= TOL_BF16_STATE
    assert torch.equal(o2, o) and torch.equal(fin2, fin)
