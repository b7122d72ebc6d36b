"""GPU parity of gdn_chunk_fwd_gated -- the chunked prompt path followed by the mixer's output
norm, out = weight * o / sqrt(mean(o^2) + eps) * silu(z) per (token, value head) -- against
the oracle composed the same way: mixer_ref.gated_rmsnorm(gdn_ref.recurrent(...)["o"], ...).

Where the chain runs one workgroup per (sequence, value head) -- bf16 at chunk 64, d_v 128,
dense rows with sequences x value heads at least the compute-unit count (256 on an
MI355X) -- the norm is applied in the chain's output stage and o never reaches memory:
8 rows x 32 value heads (all heads, both output dtypes) and 8 rows of 4096 tokens (sampled
heads, with the plain chunk call on them).  Elsewhere the chain writes o and
the norm runs in place over it: packed sequences (whose heads the chain splits over two
workgroups) at the 8-sequence workload's full size (sampled heads) and a 9-sequence case
(all heads, both output dtypes), the 4096-token prefill (sampled heads), and small dense
and fp32 cases (all heads).

Tolerances: the fp32 output at the bf16 prompt path's 2e-2 x RMS, as for o (the norm rescales
each row by its own RMS, so an error relative to the row's scale carries over), and checked
inside 1e-2; the final state as for gdn_chunk_fwd; a bf16 output is the fp32 output of the
same call rounded once where the norm is fused, and within three roundings where it follows
the chain (o itself is then stored in bf16 before the norm reads it).  In the all-heads
cases the fp32 output also matches gdn_chunk_fwd followed by gdn_gated_norm on the GPU to
1e-5 (the same o; only the order of the sum of squares may differ), and every call's
status word is 0.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import binding, synth
from oracle import gdn_ref, mixer_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, TOL_F32, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _gdn():
    import gated_deltanet_linear_amd as gdn
    return gdn


def _gate(w, seed, inp):
    """z and the norm's gain for the value-head layout of ``w`` and the token axis of ``inp``."""
    B, T = inp["v"].shape[:2]
    lens = None if inp.get("cu_seqlens") is None else tuple(np.diff(inp["cu_seqlens"]).tolist())
    mi = synth.make_mixer_inputs(w, seed=seed, lengths=lens) if lens else \
        synth.make_mixer_inputs(w, seed=seed, T=T, B=B)
    assert mi["z"].shape == inp["v"].shape
    return mi["z"], mi["norm_w"]


def _run(inp, z, nw, o_dtype=torch.float32):
    gdn = _gdn()
    d = to_dev(inp)
    zd = torch.from_numpy(np.ascontiguousarray(z)).to("cuda", dtype=d["q"].dtype)
    wd = torch.from_numpy(nw).to("cuda")
    B, T = inp["v"].shape[:2]
    nseq = 0 if d["cu"] is None else d["cu"].numel() - 1
    need = binding.gdn_chunk_fwd_workspace(binding._shape(d["q"], d["v"], None, None, False, o_dtype, B, T), nseq)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out, fin = gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["g"], d["beta"], zd, wd, eps=EPS,
                                       initial_state=d["s0"], cu_seqlens=d["cu"], o_dtype=o_dtype,
                                       workspace=ws)
    torch.cuda.synchronize()
    status = binding.plan_status(ws)
    return d, zd, wd, out, fin, status


def _check(inp, z, nw, heads=None, bf16_out=False, fused=True):
    """fp32 output against the oracle; with ``bf16_out`` also the bf16 output of the same call:
    where the norm is fused, the fp32 one rounded once (|bf16 - fp32| <= 2^-8 |fp32| + 1e-6);
    where it follows the chain, o is rounded to bf16 first, so two roundings and the mean of
    squares of the rounded o (<= 3 * 2^-8 |fp32| + 1e-6)."""
    d, zd, wd, out, fin, status = _run(inp, z, nw)
    assert status == 0, f"status word {status}"
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp.get("s0"),
                            cu_seqlens=inp.get("cu_seqlens"), heads=heads)
    sel = slice(None) if heads is None else heads
    want = mixer_ref.gated_rmsnorm(ref["o"][..., sel, :], z[..., sel, :], nw, eps=EPS)
    got = host(out[..., sel, :])
    eo = rel_max(got, want)
    ef = rel_fro(host(fin[:, sel]), ref["final"][:, sel])
    print(f"  gated out {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL_BF16_O and ef <= TOL_BF16_STATE
    assert eo <= 1e-2
    if bf16_out:
        _, _, _, outb, finb, status = _run(inp, z, nw, torch.bfloat16)
        assert status == 0, f"status word {status}"
        a, b = host(outb), host(out).astype(np.float64)
        bound = 2.0 ** -8 if fused else 3 * 2.0 ** -8
        print(f"  bf16 out: max |bf16 - fp32| / |fp32| = {np.max(np.abs(a - b) / (np.abs(b) + 1e-6)):.2e}",
              flush=True)
        assert np.all(np.abs(a - b) <= bound * np.abs(b) + 1e-6)
        assert torch.equal(finb, fin)
    return d, zd, wd, out


def _composition(d, zd, wd, out):
    """The same o through gdn_chunk_fwd, then gdn_gated_norm on the GPU: within 1e-5 of the
    gated call's fp32 output (only the order of the sum of squares may differ)."""
    gdn = _gdn()
    o, _ = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                             cu_seqlens=d["cu"])
    comp = gdn.gdn_gated_norm(o, zd, wd, eps=EPS)
    torch.cuda.synchronize()
    assert rel_max(host(out), host(comp)) <= 1e-5


def test_gated_dense_wide_fused_all_heads():
    """8 dense rows x 32 value heads: the head-wide chain with the norm inside."""
    w = synth.WORKLOADS["packed_8seq"]
    print("dense B=8 T=150, 32 value heads, fused norm, fp32 and bf16 out", flush=True)
    inp = synth.make_inputs(w, seed=37, B=8, T=150, s0_std=0.02)
    z, nw = _gate(w, 38, inp)
    d, zd, wd, out = _check(inp, z, nw, bf16_out=True)
    _composition(d, zd, wd, out)


def test_gated_dense_8x4096_fused_sampled_heads():
    """8 dense rows of the prefill's shape (64 chunks per row, whole heads per workgroup, P
    formed in the chain): the fused norm and the plain chunk call on sampled heads."""
    w = synth.WORKLOADS["prefill_t4096"]
    print("dense B=8 T=4096, fused norm, heads [6, 25]", flush=True)
    inp = synth.make_inputs(w, seed=39, B=8)
    z, nw = _gate(w, 40, inp)
    d, _, _, _ = _check(inp, z, nw, heads=[6, 25])
    gdn = _gdn()
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], heads=[6, 25])
    eo = rel_max(host(o[..., [6, 25], :]), ref["o"][..., [6, 25], :])
    ef = rel_fro(host(fin[:, [6, 25]]), ref["final"][:, [6, 25]])
    print(f"  chunk: o {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL_BF16_O and eo <= 1e-2 and ef <= TOL_BF16_STATE


def test_gated_packed_9seq_all_heads():
    """Nine packed sequences x 32 value heads: the split head-wide chain, then the norm."""
    lens = (65, 1, 130, 0, 77, 64, 200, 33, 5)
    w = synth.WORKLOADS["packed_8seq"]
    print(f"packed lengths {lens}, norm after the chain, fp32 and bf16 out", flush=True)
    inp = synth.make_inputs(w, seed=31, lengths=lens, s0_std=0.02)
    z, nw = _gate(w, 32, inp)
    d, zd, wd, out = _check(inp, z, nw, bf16_out=True, fused=False)
    _composition(d, zd, wd, out)


def test_gated_packed_8seq_full_size_sampled_heads():
    w = synth.WORKLOADS["packed_8seq"]
    print(f"packed_8seq lengths {w.lengths}, norm after the chain, heads [5, 26]", flush=True)
    inp = synth.make_inputs(w, seed=0)
    z, nw = _gate(w, 1, inp)
    _check(inp, z, nw, heads=[5, 26])


def test_gated_prefill_t4096_sampled_heads():
    w = synth.WORKLOADS["prefill_t4096"]
    print("prefill T=4096, norm after the chain, heads [0, 13, 31]", flush=True)
    inp = synth.make_inputs(w, seed=0)
    z, nw = _gate(w, 2, inp)
    _check(inp, z, nw, heads=[0, 13, 31])


def test_gated_dense_rows_all_heads():
    w = synth.WORKLOADS["packed_8seq"]
    print("dense B=2 T=150 bf16, norm after the chain, bf16 out", flush=True)
    inp = synth.make_inputs(w, seed=33, B=2, T=150, s0_std=0.02)
    z, nw = _gate(w, 34, inp)
    _check(inp, z, nw, bf16_out=True, fused=False)


def test_gated_fp32_all_heads():
    w = dataclasses.replace(synth.WORKLOADS["tiny_fp32"], T=100)
    print("fp32 B=1 T=100 2/2 heads d 16, norm after the chain", flush=True)
    inp = synth.make_inputs(w, seed=35)
    z, nw = _gate(w, 36, inp)
    d, zd, wd, out, fin, status = _run(inp, z, nw)
    assert status == 0
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    want = mixer_ref.gated_rmsnorm(ref["o"], z, nw, eps=EPS)
    assert rel_max(host(out), want) <= TOL_F32
    assert rel_fro(host(fin), ref["final"]) <= TOL_F32
