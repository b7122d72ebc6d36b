"""The fp16 operand range of the bf16 chunk-64 path (stated in include/gdn.h): inputs whose
state or per-chunk values stay inside it give parity with the oracle and a zero status word;
inputs that push them past it either still give parity or set bit 1 (value 2) of the status
word at the start of the workspace -- never a silent wrong answer.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import binding, synth
from oracle import gdn_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu


def _scaled_case(v_scale, seed):
    import dataclasses
    w = dataclasses.replace(synth.WORKLOADS["prefill_t4096"], H_qk=2, H_v=4)
    inp = synth.make_inputs(w, seed=seed, T=300, g_shift=-5.0)
    # v scaled, then rounded to bf16 so that the oracle sees the values the kernel reads
    v = torch.from_numpy(inp["v"] * np.float32(v_scale)).to(torch.bfloat16).float().numpy()
    inp["v"] = v
    return inp


def _run(inp):
    d = to_dev(inp)
    ws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    o, fin = binding.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64, workspace=ws)
    torch.cuda.synchronize()
    return o, fin, binding.plan_status(ws)


def test_inside_range_parity_and_zero_status():
    inp = _scaled_case(1e2, seed=31)
    print("v x 1e2, slow decay, T=300", flush=True)
    o, fin, status = _run(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    eo, ef = rel_max(host(o), ref["o"]), rel_fro(host(fin), ref["final"])
    print(f"  status {status} o {eo:.2e} final {ef:.2e} max|S| {np.abs(ref['final']).max():.3g}", flush=True)
    assert status == 0
    assert eo <= TOL_BF16_O and ef <= TOL_BF16_STATE


def test_past_range_parity_or_status():
    inp = _scaled_case(1e4, seed=32)
    print("v x 1e4, slow decay, T=300", flush=True)
    o, fin, status = _run(inp)
    ref = gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    oh, fh = host(o), host(fin)
    finite = bool(np.isfinite(oh).all() and np.isfinite(fh).all())
    eo, ef = rel_max(oh, ref["o"]), rel_fro(fh, ref["final"])
    print(f"  status {status} finite {finite} o {eo:.2e} final {ef:.2e} max|S| {np.abs(ref['final']).max():.3g}",
          flush=True)
    assert status in (0, 2)
    if status == 0:
        assert finite and eo <= TOL_BF16_O and ef <= TOL_BF16_STATE
    else:
        assert not finite  # the flag reports a non-finite value in o or the final state


def test_overflow_sets_status():
    """v x 1e6: V itself is past fp16's range, so the status word must report it."""
    inp = _scaled_case(1e6, seed=33)
    print("v x 1e6, slow decay, T=300", flush=True)
    o, fin, status = _run(inp)
    finite = bool(np.isfinite(host(o)).all() and np.isfinite(host(fin)).all())
    print(f"  status {status} finite {finite}", flush=True)
    assert status == 2 and not finite
