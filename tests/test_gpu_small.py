"""GPU parity of libgdn against the fp64 oracle on sizes the oracle finishes in seconds.

Every call goes through the C ABI (the ctypes binding).  Sizes span several 64-token
chunks and end in a ragged tail; the edge cases are the method's own: a -inf decay
(reset), empty sequences, carried state, in-place continuation, other head ratios.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import synth
from oracle import gdn_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, TOL_F32, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    import gated_deltanet_linear_amd as gdn
    return gdn


def _ref(inp, **kw):
    return gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp.get("s0"),
                             cu_seqlens=inp.get("cu_seqlens"), **kw)


def test_tiny_fp32_all_outputs():
    """The tiny fp32 workload: o, final state and every per-token state within 1e-4 RMS."""
    gdn = _lib()
    inp = synth.make_inputs(synth.WORKLOADS["tiny_fp32"], seed=0)
    d = to_dev(inp)
    ref = _ref(inp, want_states=True)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=16)
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=16)
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_F32
    assert rel_max(host(fin), ref["final"]) <= TOL_F32
    assert rel_max(host(o2), ref["o"]) <= TOL_F32
    assert rel_max(host(fin2), ref["final"]) <= TOL_F32
    assert rel_max(host(st), ref["states"]) <= TOL_F32


def test_tiny_fp32_decode_steps_match_oracle():
    gdn = _lib()
    inp = synth.make_inputs(synth.WORKLOADS["tiny_fp32"], seed=0)
    d = to_dev(inp)
    ref = _ref(inp)
    state = torch.zeros((1, 2, 16, 16), device="cuda")
    outs = []
    for t in range(64):
        sl = slice(t, t + 1)
        outs.append(gdn.gdn_recurrent_step(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                                           d["v"][:, sl].contiguous(), d["g"][:, sl].contiguous(),
                                           d["beta"][:, sl].contiguous(), state))
    o = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_F32
    assert rel_max(host(state), ref["final"]) <= TOL_F32


def _bf16_case(T=200, seed=3, **kw):
    w = synth.WORKLOADS["prefill_t4096"]
    return synth.make_inputs(w, seed=seed, T=T, **kw)


@pytest.mark.parametrize("T", [1, 63, 64, 200])
def test_bf16_ragged_prefill(T):
    gdn = _lib()
    inp = _bf16_case(T)
    d = to_dev(inp)
    ref = _ref(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE
    # far inside the bound: the products carry fp32-level precision
    assert rel_max(host(o), ref["o"]) <= 2e-3


def test_bf16_slow_decay_and_initial_state():
    """Kept fraction ~0.99 per token: the carry between chunks dominates."""
    gdn = _lib()
    inp = _bf16_case(T=300, seed=4, g_shift=-5.0, s0_std=0.02)
    d = to_dev(inp)
    ref = _ref(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE


def test_packed_sequences_with_empty_ones():
    gdn = _lib()
    w = synth.WORKLOADS["packed_8seq"]
    lens = (70, 0, 1, 130, 64, 0)
    inp = synth.make_inputs(w, seed=5, lengths=lens)
    d = to_dev(inp)
    ref = _ref(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                               cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE
    # an empty sequence passes its initial state through untouched
    np.testing.assert_array_equal(host(fin)[1], inp["s0"][1])
    np.testing.assert_array_equal(host(fin)[5], inp["s0"][5])


@pytest.mark.parametrize("case", ["beta0", "no_decay_full_write", "zero_q", "zero_k_l2norm"])
def test_degenerate_regimes(case):
    """The method's degenerate regimes against the oracle (150 tokens: two chunks and a ragged tail,
    32 heads, initial state, kept fraction ~0.99 a token): beta = 0 (nothing written; the state only decays, to its closed form
    e^{sum g} S0), g = 0 with beta = 1 (no decay, full delta writes), zero queries (o exactly 0) and
    zero keys with the in-kernel l2 norm (normalised to 0: nothing written)."""
    gdn = _lib()
    inp = _bf16_case(T=150, seed=21, s0_std=0.02, g_shift=-5.0)  # slow decay: the state stays well above 0
    l2 = False
    if case == "beta0":
        inp["beta"][:] = 0.0
    elif case == "no_decay_full_write":
        inp["g"][:] = 0.0
        inp["beta"][:] = 1.0
    elif case == "zero_q":
        inp["q"][:] = 0.0
    else:
        inp["k"][:] = 0.0
        l2 = True
    d = to_dev(inp)
    ref = _ref(inp, l2norm=l2)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"], l2norm=l2)
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                      l2norm=l2)
    torch.cuda.synchronize()
    if case == "zero_q":
        assert float(o.abs().max()) == 0.0 and float(o2.abs().max()) == 0.0
    else:
        assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
        assert rel_max(host(o2), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE
    assert rel_fro(host(st[:, -1]), ref["final"]) <= TOL_BF16_STATE
    if case in ("beta0", "zero_k_l2norm"):
        decay = np.exp(inp["g"].astype(np.float64).sum(axis=1))[0]          # [H_v]
        closed = inp["s0"][0].astype(np.float64) * decay[:, None, None]
        assert rel_fro(host(fin)[0], closed) <= 1e-5


@pytest.mark.parametrize("case", ["beta0", "no_decay_full_write", "zero_q", "zero_k_l2norm"])
def test_decode_degenerate_regimes(case):
    """The same regimes through the decode step: 4 rows of 32 heads, 5 consecutive in-place steps
    against the oracle run over the same 5 tokens."""
    gdn = _lib()
    inp = _bf16_case(T=5, seed=22, s0_std=0.02, g_shift=-5.0, B=4)
    l2 = False
    if case == "beta0":
        inp["beta"][:] = 0.0
    elif case == "no_decay_full_write":
        inp["g"][:] = 0.0
        inp["beta"][:] = 1.0
    elif case == "zero_q":
        inp["q"][:] = 0.0
    else:
        inp["k"][:] = 0.0
        l2 = True
    d = to_dev(inp)
    ref = _ref(inp, l2norm=l2)
    state = d["s0"].clone()
    outs = []
    for t in range(5):
        sl = slice(t, t + 1)
        outs.append(gdn.gdn_recurrent_step(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                                           d["v"][:, sl].contiguous(), d["g"][:, sl].contiguous(),
                                           d["beta"][:, sl].contiguous(), state, l2norm=l2))
    o = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    if case == "zero_q":
        assert float(o.abs().max()) == 0.0
    else:
        assert rel_max(host(o), ref["o"]) <= TOL_F32
    assert rel_max(host(state), ref["final"]) <= TOL_F32


def test_minus_inf_resets_without_nan():
    gdn = _lib()
    inp = _bf16_case(T=150, seed=6, s0_std=0.02)
    inp["g"][0, 10, :5] = -np.inf       # inside the first chunk
    inp["g"][0, 64, 5:9] = -np.inf      # first token of the second chunk
    inp["g"][0, 149, 9:] = -np.inf      # the very last token
    d = to_dev(inp)
    ref = _ref(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(fin).all() and torch.isfinite(st).all()
    assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE
    assert rel_fro(host(fin2), ref["final"]) <= TOL_BF16_STATE


def test_l2norm_flag_on_raw_inputs():
    """The in-kernel l2 norm on un-normalised q, k with norms 0.09 .. 4.1."""
    gdn = _lib()
    inp = _bf16_case(T=130, seed=7, normalise=False, raw_norm_range=(0.09, 4.1))
    d = to_dev(inp)
    ref = _ref(inp, l2norm=True)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], l2norm=True)
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], l2norm=True)
    state = torch.zeros((1, 32, 128, 128), device="cuda")
    for t in range(130):
        sl = slice(t, t + 1)
        gdn.gdn_recurrent_step(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                               d["v"][:, sl].contiguous(), d["g"][:, sl].contiguous(),
                               d["beta"][:, sl].contiguous(), state, l2norm=True)
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE
    assert rel_fro(host(fin2), ref["final"]) <= TOL_BF16_STATE
    assert rel_fro(host(state), ref["final"]) <= TOL_BF16_STATE
    # negative control: without the norm the result is far off
    raw = _ref(inp, l2norm=False)
    assert rel_fro(raw["final"], ref["final"]) > 0.1


def test_split_invariance_and_inplace_continuation():
    gdn = _lib()
    inp = _bf16_case(T=230, seed=8, s0_std=0.02)
    d = to_dev(inp)
    o_all, fin_all = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    T1 = 101                                 # not a multiple of the chunk
    cache = d["s0"].clone()
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o1, _ = gdn.gdn_chunk_fwd(sl(d["q"], 0, T1), sl(d["k"], 0, T1), sl(d["v"], 0, T1), sl(d["g"], 0, T1),
                              sl(d["beta"], 0, T1), initial_state=cache, final_state=cache)
    o2, _ = gdn.gdn_chunk_fwd(sl(d["q"], T1, 230), sl(d["k"], T1, 230), sl(d["v"], T1, 230),
                              sl(d["g"], T1, 230), sl(d["beta"], T1, 230), initial_state=cache,
                              final_state=cache)
    torch.cuda.synchronize()
    ref = _ref(inp)
    assert rel_max(host(torch.cat([o1, o2], 1)), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(cache), ref["final"]) <= TOL_BF16_STATE
    assert rel_fro(host(cache), host(fin_all)) <= 1e-5


@pytest.mark.parametrize("H_qk,H_v", [(4, 4), (2, 6), (8, 8), (8, 24)])
def test_other_head_ratios(H_qk, H_v):
    """Head ratios 1 and 3 beside the 2 of the workloads; (8, 8) and (8, 24) also take the
    prep kernel's XCD-aligned head order (query/key and value heads multiples of 8)."""
    gdn = _lib()
    w = synth.Workload("ratio", 2, 100, H_qk, H_v, 128, 128, 64, "bf16", 2.0, 0.02)
    inp = synth.make_inputs(w, seed=9)
    d = to_dev(inp)
    ref = _ref(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    assert rel_max(host(o), ref["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE


def test_chunk_equals_repeated_decode_steps():
    """Cross-kernel: T decode steps from the same state give the chunked result."""
    gdn = _lib()
    inp = _bf16_case(T=70, seed=10, s0_std=0.02)
    d = to_dev(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    state = d["s0"].clone()
    outs = []
    for t in range(70):
        sl = slice(t, t + 1)
        outs.append(gdn.gdn_recurrent_step(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                                           d["v"][:, sl].contiguous(), d["g"][:, sl].contiguous(),
                                           d["beta"][:, sl].contiguous(), state))
    torch.cuda.synchronize()
    ref = _ref(inp)
    od = torch.cat(outs, 1)
    assert rel_max(host(od), ref["o"]) <= 1e-4          # the step is fp32 throughout
    assert rel_fro(host(state), ref["final"]) <= 1e-5
    assert rel_max(host(o), host(od)) <= TOL_BF16_O
    assert rel_fro(host(fin), host(state)) <= TOL_BF16_STATE


def test_states_match_oracle_and_final():
    gdn = _lib()
    inp = _bf16_case(T=150, seed=11, s0_std=0.02)
    d = to_dev(inp)
    heads = [0, 17, 31]
    ref = _ref(inp, heads=heads, want_states=True)
    o, st, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    sth = host(st[:, :, heads])
    assert rel_fro(sth, ref["states"]) <= TOL_BF16_STATE
    assert rel_max(host(o)[:, :, heads], ref["o"][:, :, heads]) <= TOL_BF16_O
    assert rel_fro(host(st[:, -1]), host(fin)) <= 1e-5


def test_strided_states_fp32_and_bf16():
    """gdn_states_fwd_strided keeps the tokens t_begin, t_begin + t_step, ... < t_end of every row:
    the oracle's per-token states at those tokens (selection is plain indexing of the recurrence's
    states), with o and the final state complete.  fp32 path (d = 16, chunk 16) to 1e-4 RMS; bf16
    path over four rows and a ragged tail, the selection starting mid-chunk and crossing chunks."""
    gdn = _lib()
    inp = synth.make_inputs(synth.WORKLOADS["tiny_fp32"], seed=0)
    d = to_dev(inp)
    ref = _ref(inp, want_states=True)
    for t0, t1, step in ((3, 50, 7), (0, 64, 16), (63, 64, 1), (10, 10, 3)):
        o, st, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=16,
                                        t_begin=t0, t_end=t1, t_step=step)
        torch.cuda.synchronize()
        assert st.shape[1] == len(range(t0, t1, step))
        if st.shape[1]:
            assert rel_max(host(st), ref["states"][:, t0:t1:step]) <= TOL_F32
        assert rel_max(host(o), ref["o"]) <= TOL_F32
        assert rel_max(host(fin), ref["final"]) <= TOL_F32

    inp = _bf16_case(T=150, seed=21, s0_std=0.02, B=4)
    d = to_dev(inp)
    heads = [0, 13, 31]
    ref = _ref(inp, heads=heads, want_states=True)
    o, st_all, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    # the first three keep under half of each row's tokens (expanded from the chunk-start
    # states), the last three at least half (streamed by the chain: a window that starts
    # and ends inside chunks, and every second token)
    for t0, t1, step in ((5, 150, 64), (37, 101, 1), (149, 150, 5), (20, 150, 1), (0, 140, 1), (0, 150, 2)):
        o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                          t_begin=t0, t_end=t1, t_step=step)
        torch.cuda.synchronize()
        assert rel_fro(host(st[:, :, heads]), ref["states"][:, t0:t1:step]) <= TOL_BF16_STATE
        # A selection keeping under half of the tokens is expanded from the chunk-start
        # states; the full readout is streamed by the chain from the initial state: two
        # fp32 orders of the same recurrence, equal up to rounding.  o and the final state
        # come from the same chain arithmetic: bit for bit.
        assert rel_fro(host(st), host(st_all[:, t0:t1:step])) <= 1e-5
        assert torch.equal(o2, o) and torch.equal(fin2, fin)


def test_strided_states_packed_rows():
    """With cu_seqlens the selection runs along the one packed row, across sequence boundaries."""
    gdn = _lib()
    lengths = (70, 0, 131, 5)
    inp = synth.make_inputs(synth.WORKLOADS["packed_8seq"], seed=22, lengths=lengths)
    d = to_dev(inp)
    heads = [2, 30]
    ref = _ref(inp, heads=heads, want_states=True)
    # a sparse selection (expanded from the chunk-start states) and a dense one (streamed
    # by the chain), both across sequence boundaries
    for t0, t1, step in ((3, sum(lengths), 9), (3, sum(lengths) - 2, 1)):
        o, st, fin = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"],
                                        cu_seqlens=d["cu"], t_begin=t0, t_end=t1, t_step=step)
        torch.cuda.synchronize()
        assert st.shape[:2] == (1, len(range(t0, t1, step)))
        assert rel_fro(host(st[:, :, heads]), ref["states"][:, t0:t1:step]) <= TOL_BF16_STATE


@pytest.mark.parametrize("d_v", [32, 64, 96])
@pytest.mark.parametrize("B", [1, 8])
def test_other_value_widths(d_v, B):
    """The bf16 path at value widths 32, 64, 96 (d_k = 128): one row (16-column chains) and eight
    rows (32- or 64-column chains, 64 only where d_v is a multiple of 64), with the states path."""
    import dataclasses
    gdn = _lib()
    w = dataclasses.replace(synth.WORKLOADS["prefill_t4096"], d_v=d_v)
    inp = synth.make_inputs(w, seed=30 + d_v + B, T=150, B=B, s0_std=0.02)
    d = to_dev(inp)
    heads = [0, 31]
    ref = _ref(inp, heads=heads, want_states=True)
    full = _ref(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    assert rel_max(host(o), full["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), full["final"]) <= TOL_BF16_STATE
    assert rel_max(host(o2), full["o"]) <= TOL_BF16_O
    assert rel_fro(host(st[:, :, heads]), ref["states"]) <= TOL_BF16_STATE


@pytest.mark.parametrize("B", [2, 4])
def test_many_rows_both_paths(B):
    """Two or four rows of 32 heads: enough (row, head) pairs that the carry runs on 32-column
    (B = 2) or 64-column (B = 4) blocks of the state, the layouts for launches that fill every
    compute unit."""
    gdn = _lib()
    inp = _bf16_case(T=150, seed=16, s0_std=0.02, B=B)
    d = to_dev(inp)
    heads = [0, 13, 31]
    ref = _ref(inp, heads=heads, want_states=True)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    full = _ref(inp)
    assert rel_max(host(o), full["o"]) <= TOL_BF16_O
    assert rel_fro(host(fin), full["final"]) <= TOL_BF16_STATE
    assert rel_max(host(o2), full["o"]) <= TOL_BF16_O
    assert rel_fro(host(st[:, :, heads]), ref["states"]) <= TOL_BF16_STATE
    assert rel_fro(host(fin2), full["final"]) <= TOL_BF16_STATE


def test_empty_prompt_passes_state_through():
    gdn = _lib()
    inp = _bf16_case(T=0, seed=12, s0_std=0.02)
    d = to_dev(inp)
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    assert o.numel() == 0
    np.testing.assert_array_equal(host(fin), inp["s0"])


def test_bitwise_deterministic():
    gdn = _lib()
    inp = _bf16_case(T=257, seed=13)
    d = to_dev(inp)
    a = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    b = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_bf16_output_dtype():
    gdn = _lib()
    inp = _bf16_case(T=90, seed=14)
    d = to_dev(inp)
    o, _ = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = _ref(inp)["o"]
    # One rounding to bf16 (relative error <= 2^-9) on top of the fp32-level error; where
    # a value sits on a rounding boundary the two sides may round apart by one ulp.
    rms = np.sqrt(np.mean(ref * ref))
    err = np.abs(host(o).astype(np.float64) - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-3 * rms)


def test_bad_cu_seqlens_makes_the_call_a_noop():
    gdn = _lib()
    from gated_deltanet_linear_amd import binding
    inp = synth.make_inputs(synth.WORKLOADS["packed_8seq"], seed=15, lengths=(20, 30))
    d = to_dev(inp)
    bad = torch.tensor([0, 40, 30], dtype=torch.int32, device="cuda")   # decreasing
    s = binding._shape(d["q"], d["v"], None, None, False, torch.float32, 1, 50)
    ws = torch.zeros(binding.gdn_chunk_fwd_workspace(s, 2), dtype=torch.uint8, device="cuda")
    o = torch.full((1, 50, 32, 128), 7.0, device="cuda")
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=bad, o=o, workspace=ws,
                      output_final_state=False)
    torch.cuda.synchronize()
    assert binding.plan_status(ws) != 0
    assert torch.all(o == 7.0)


def test_nan_decay_propagates():
    """A NaN decay at token t of one head reaches that head's o and state from t on (as in the
    oracle's recurrence) and no other head.  The chunk form may also carry it to the earlier
    tokens of t's chunk (a zero of T~ or P times a NaN row in one MFMA), so those tokens are
    left unchecked; the chunks before it match the oracle, and the call sets bit 1 of the
    status word."""
    from gated_deltanet_linear_amd import binding
    gdn = _lib()
    inp = _bf16_case(T=150, seed=13, s0_std=0.02)
    hn, tn = 7, 100                      # head 7, token 36 of the second chunk
    inp["g"][0, tn, hn] = np.nan
    d = to_dev(inp)
    ref = _ref(inp)
    assert np.isnan(ref["o"][0, tn:, hn]).all() and np.isfinite(ref["o"][0, :tn, hn]).all()
    need = binding.gdn_chunk_fwd_workspace(binding._shape(d["q"], d["v"], None, None, False, torch.float32, 1, 150), 0)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o, fin = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"], workspace=ws)
    o2, st, fin2 = gdn.gdn_states_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["s0"])
    torch.cuda.synchronize()
    assert binding.plan_status(ws) & 2
    others = [h for h in range(32) if h != hn]
    oh, sth = host(o), host(st)
    assert np.isfinite(oh[:, :, others]).all() and np.isfinite(host(fin)[:, others]).all()
    assert rel_max(oh[:, :, others], ref["o"][:, :, others]) <= TOL_BF16_O
    assert rel_fro(host(fin)[:, others], ref["final"][:, others]) <= TOL_BF16_STATE
    # the NaN head: exact before t's chunk, non-finite from t on, in o, the states and the final state
    assert rel_max(oh[:, :64, hn], ref["o"][:, :64, hn]) <= TOL_BF16_O
    assert not np.isfinite(oh[0, tn:, hn]).any()
    assert not np.isfinite(host(fin)[0, hn]).any()
    assert np.isfinite(sth[0, :64, hn]).all() and not np.isfinite(sth[0, tn:, hn]).any()
    assert torch.equal(o2, o) or np.array_equal(host(o2), oh, equal_nan=True)
    assert np.array_equal(host(fin2), host(fin), equal_nan=True)
