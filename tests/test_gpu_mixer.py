"""GPU parity of the mixer steps around the delta rule (gdn_mixer_prologue, gdn_gated_norm,
gdn_recurrent_step_gated) against the fp64 references in oracle/mixer_ref.py.

Every call goes through the C ABI.  Tolerances:
- fp32 outputs (the norm's out, g, beta): max|gpu - ref| <= 1e-4 * RMS(ref), as for the
  fp32 delta-rule paths, and checked far inside that (1e-5);
- bf16 outputs (q, k, v of the prologue, a bf16 norm output): one rounding to bf16 on top
  of fp32 arithmetic, |gpu - ref| <= 2^-8 |ref| + 1e-5 elementwise (where the exact value
  sits next to a rounding boundary the two sides may round apart by one ulp);
- convolution states: bit-exact (they are copies of inputs).
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_amd import synth
from oracle import gdn_ref, mixer_ref
from parity_util import TOL_BF16_O, TOL_BF16_STATE, TOL_F32, host, rel_fro, rel_max, to_dev

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["prefill_t4096"]


def _gdn():
    import gated_deltanet_linear_amd as gdn
    return gdn


def _dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dtype)


def _bf16_close(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(gpu - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5))


@pytest.mark.parametrize("d_v,rows_T", [(128, 4096), (16, 37), (64, 5), (256, 3)])
def test_gated_norm_fp32(d_v, rows_T):
    gdn = _gdn()
    rng = np.random.default_rng(d_v)
    y = rng.standard_normal((1, rows_T, 32, d_v)).astype(np.float32)
    y[0, 0, 0] = 0.0                                    # a zero row: eps alone
    z = synth.round_to(rng.standard_normal((1, rows_T, 32, d_v)).astype(np.float32), "bf16")
    w = (1.0 + 0.1 * rng.standard_normal(d_v)).astype(np.float32)
    out = gdn.gdn_gated_norm(_dev(y), _dev(z, torch.bfloat16), _dev(w), eps=1e-6)
    torch.cuda.synchronize()
    ref = mixer_ref.gated_rmsnorm(y, z, w, eps=1e-6)
    assert rel_max(host(out), ref) <= TOL_F32
    assert rel_max(host(out), ref) <= 1e-5
    assert np.all(host(out)[0, 0, 0] == 0.0)


def test_gated_norm_bf16_in_place():
    gdn = _gdn()
    rng = np.random.default_rng(7)
    y = synth.round_to(rng.standard_normal((2, 33, 32, 128)).astype(np.float32), "bf16")
    z = synth.round_to(rng.standard_normal((2, 33, 32, 128)).astype(np.float32), "bf16")
    w = (1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    yd = _dev(y, torch.bfloat16)
    out = gdn.gdn_gated_norm(yd, _dev(z, torch.bfloat16), _dev(w), eps=1e-6, out=yd)
    torch.cuda.synchronize()
    assert out.data_ptr() == yd.data_ptr()
    assert _bf16_close(host(out), mixer_ref.gated_rmsnorm(y, z, w, eps=1e-6))


def test_decode_step_gated_matches_oracle_and_composition():
    gdn = _gdn()
    B = 8
    pool = synth.make_decode_pool(synth.WORKLOADS["decode_b256"], seed=3, pool=4, B=B)
    mi = synth.make_mixer_inputs(W, seed=4, T=4, B=B)
    w = _dev(mi["norm_w"])
    s_a = _dev(pool["s0"])
    s_b = s_a.clone()
    S = pool["s0"].astype(np.float64)
    for step in range(4):
        q, k, v = (_dev(pool[n][step], torch.bfloat16) for n in ("q", "k", "v"))
        g, beta = _dev(pool["g"][step]), _dev(pool["beta"][step])
        z = _dev(mi["z"][:, step:step + 1], torch.bfloat16)
        out = gdn.gdn_recurrent_step_gated(q, k, v, g, beta, s_a, z, w, eps=1e-6)
        o = gdn.gdn_recurrent_step(q, k, v, g, beta, s_b)
        comp = gdn.gdn_gated_norm(o, z, w, eps=1e-6)
        torch.cuda.synchronize()
        ref = gdn_ref.recurrent(pool["q"][step], pool["k"][step], pool["v"][step], pool["g"][step],
                                pool["beta"][step], s0=S.astype(np.float32))
        S = ref["final"]
        want = mixer_ref.gated_rmsnorm(ref["o"], mi["z"][:, step:step + 1], mi["norm_w"], eps=1e-6)
        assert rel_max(host(out), want) <= TOL_F32
        assert rel_max(host(out), host(comp)) <= 1e-5
        assert torch.equal(s_a, s_b)                 # the fused norm leaves the state alone


def _prologue_ref(mi, H_qk, d_k, H_v, d_v, cu=None, state=None):
    T = mi["x"].shape[1]
    r = mixer_ref.prologue(mi["x"].reshape(-1, mi["x"].shape[-1]), mi["conv_w"],
                           mi["a"].reshape(-1, H_v), mi["b"].reshape(-1, H_v), mi["A_log"], mi["dt_bias"],
                           H_qk, d_k, H_v, d_v, conv_state=state, cu_seqlens=cu)
    return r, T


def _run_prologue(mi, conv_state=None, update=False, cu=None):
    gdn = _gdn()
    dt = torch.bfloat16 if mi["dtype"] == "bf16" else torch.float32
    cs = _dev(conv_state)
    res = gdn.gdn_mixer_prologue(_dev(mi["x"], dt), _dev(mi["conv_w"]), _dev(mi["a"]), _dev(mi["b"]),
                                 _dev(mi["A_log"]), _dev(mi["dt_bias"]), W.H_qk, W.d_k, W.H_v, W.d_v,
                                 conv_state=cs, cu_seqlens=None if cu is None else _dev(cu, torch.int32),
                                 update_conv_state=update)
    torch.cuda.synchronize()
    return res, cs


def _check_prologue(res, r, B):
    q, k, v, g, beta, _ = res
    assert _bf16_close(host(q).reshape(-1, W.H_qk, W.d_k), r["q"])
    assert _bf16_close(host(k).reshape(-1, W.H_qk, W.d_k), r["k"])
    assert _bf16_close(host(v).reshape(-1, W.H_v, W.d_v), r["v"])
    assert rel_max(host(g).reshape(-1, W.H_v), r["g"]) <= 1e-5
    assert rel_max(host(beta).reshape(-1, W.H_v), r["beta"]) <= 1e-5


def test_prologue_full_prefill_size():
    """x [1, 4096, 8192] bf16: the 4096-token prefill's convolution input."""
    mi = synth.make_mixer_inputs(W, seed=5)
    res, _ = _run_prologue(mi)
    r, _ = _prologue_ref(mi, W.H_qk, W.d_k, W.H_v, W.d_v)
    _check_prologue(res, r, 1)


def test_prologue_packed_with_state_in_place():
    lens = (70, 0, 1, 2, 130, 5)
    mi = synth.make_mixer_inputs(W, seed=6, lengths=lens, with_conv_state=True)
    state0 = mi["conv_state"].copy()
    res, cs = _run_prologue(mi, conv_state=state0, update=True, cu=mi["cu_seqlens"])
    r, _ = _prologue_ref(mi, W.H_qk, W.d_k, W.H_v, W.d_v, cu=mi["cu_seqlens"], state=state0)
    _check_prologue(res, r, 1)
    assert res[5].data_ptr() == cs.data_ptr()
    np.testing.assert_array_equal(host(cs), r["conv_state"])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prologue_narrow_channel_layouts(dtype):
    """Layouts off the 16-byte path: query/key width 4 (the q | k boundary is not a multiple of
    8 channels) in bf16, and fp32 input, both 4 channels a thread; packed with an empty
    sequence and a convolution state updated in place."""
    import dataclasses
    w = dataclasses.replace(W, H_qk=1, d_k=4, H_v=3, d_v=4, dtype=dtype)
    lens = (5, 0, 17, 2)
    mi = synth.make_mixer_inputs(w, seed=12, lengths=lens, with_conv_state=True)
    state0 = mi["conv_state"].copy()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gdn = _gdn()
    cs = _dev(state0)
    q, k, v, g, beta, _ = gdn.gdn_mixer_prologue(
        _dev(mi["x"], dt), _dev(mi["conv_w"]), _dev(mi["a"]), _dev(mi["b"]), _dev(mi["A_log"]),
        _dev(mi["dt_bias"]), w.H_qk, w.d_k, w.H_v, w.d_v, conv_state=cs,
        cu_seqlens=_dev(mi["cu_seqlens"], torch.int32), update_conv_state=True)
    torch.cuda.synchronize()
    r = mixer_ref.prologue(mi["x"][0], mi["conv_w"], mi["a"][0], mi["b"][0], mi["A_log"], mi["dt_bias"],
                           w.H_qk, w.d_k, w.H_v, w.d_v, conv_state=state0, cu_seqlens=mi["cu_seqlens"])
    for got, ref in ((q, r["q"]), (k, r["k"]), (v, r["v"])):
        got = host(got)[0]
        if dtype == "bf16":
            assert _bf16_close(got, ref)
        else:
            assert rel_max(got, ref) <= 1e-5
    assert rel_max(host(g)[0], r["g"]) <= 1e-5
    assert rel_max(host(beta)[0], r["beta"]) <= 1e-5
    np.testing.assert_array_equal(host(cs), r["conv_state"])


@pytest.mark.parametrize("dtype,narrow,lens,with_state", [
    ("bf16", False, (70, 0, 1, 2, 130, 5), True),
    ("bf16", False, (0, 33, 2, 0, 1), False),
    ("fp32", True, (5, 0, 17, 2), True),
    ("bf16", True, None, True),
])
def test_prologue_state_to_separate_buffer(dtype, narrow, lens, with_state):
    """The outgoing convolution state written to its own buffer (the convolution kernel
    writes it at each sequence's last token, and copies it for empty sequences), with and
    without an incoming state, packed with empty and 1-2 token sequences, or dense rows;
    the incoming state is left as it was."""
    import dataclasses
    w = dataclasses.replace(W, H_qk=1, d_k=4, H_v=3, d_v=4, dtype=dtype) if narrow else W
    if lens is None:
        mi = synth.make_mixer_inputs(w, seed=14, T=9, B=3, with_conv_state=with_state)
    else:
        mi = synth.make_mixer_inputs(w, seed=13, lengths=lens, with_conv_state=with_state)
    state0 = mi["conv_state"].copy() if with_state else None
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    N = len(lens) if lens is not None else mi["x"].shape[0]
    C = 2 * w.H_qk * w.d_k + w.H_v * w.d_v
    gdn = _gdn()
    cs_in = _dev(state0) if with_state else None
    cs_out = torch.full((N, C, 3), float("nan"), dtype=torch.float32, device="cuda")
    cu = None if lens is None else _dev(mi["cu_seqlens"], torch.int32)
    q, k, v, g, beta, so = gdn.gdn_mixer_prologue(
        _dev(mi["x"], dt), _dev(mi["conv_w"]), _dev(mi["a"]), _dev(mi["b"]), _dev(mi["A_log"]),
        _dev(mi["dt_bias"]), w.H_qk, w.d_k, w.H_v, w.d_v, conv_state=cs_in, cu_seqlens=cu,
        conv_state_out=cs_out)
    torch.cuda.synchronize()
    assert so.data_ptr() == cs_out.data_ptr()
    refs = []
    if lens is None:
        for b in range(N):
            refs.append(mixer_ref.prologue(mi["x"][b], mi["conv_w"], mi["a"][b], mi["b"][b], mi["A_log"],
                                           mi["dt_bias"], w.H_qk, w.d_k, w.H_v, w.d_v,
                                           conv_state=None if state0 is None else state0[b:b + 1]))
        ref_state = np.concatenate([r["conv_state"] for r in refs])
        got_rows = [(host(t), [r[key] for r in refs]) for t, key in ((q, "q"), (k, "k"), (v, "v"))]
        for got, ref in got_rows:
            for b in range(N):
                assert (_bf16_close(got[b], ref[b]) if dtype == "bf16" else rel_max(got[b], ref[b]) <= 1e-5)
        for b in range(N):
            assert rel_max(host(g)[b], refs[b]["g"]) <= 1e-5
            assert rel_max(host(beta)[b], refs[b]["beta"]) <= 1e-5
    else:
        r = mixer_ref.prologue(mi["x"][0], mi["conv_w"], mi["a"][0], mi["b"][0], mi["A_log"], mi["dt_bias"],
                               w.H_qk, w.d_k, w.H_v, w.d_v, conv_state=state0, cu_seqlens=mi["cu_seqlens"])
        ref_state = r["conv_state"]
        for got, ref in ((q, r["q"]), (k, r["k"]), (v, r["v"])):
            got = host(got)[0]
            assert (_bf16_close(got, ref) if dtype == "bf16" else rel_max(got, ref) <= 1e-5)
        assert rel_max(host(g)[0], r["g"]) <= 1e-5
        assert rel_max(host(beta)[0], r["beta"]) <= 1e-5
    np.testing.assert_array_equal(host(cs_out), ref_state)
    if with_state:
        np.testing.assert_array_equal(host(cs_in), state0)


def test_prologue_decode_steps_carry_the_state():
    """B rows of one token, the convolution state updated in place step after step, equal
    the whole sequences convolved at once."""
    B, steps = 4, 6
    mi = synth.make_mixer_inputs(W, seed=8, T=steps, B=B, with_conv_state=True)
    full = [mixer_ref.prologue(mi["x"][b], mi["conv_w"], mi["a"][b], mi["b"][b], mi["A_log"], mi["dt_bias"],
                               W.H_qk, W.d_k, W.H_v, W.d_v, conv_state=mi["conv_state"][b:b + 1])
            for b in range(B)]
    gdn = _gdn()
    cs = _dev(mi["conv_state"])
    for t in range(steps):
        q, k, v, g, beta, _ = gdn.gdn_mixer_prologue(
            _dev(np.ascontiguousarray(mi["x"][:, t:t + 1]), torch.bfloat16), _dev(mi["conv_w"]),
            _dev(np.ascontiguousarray(mi["a"][:, t:t + 1])), _dev(np.ascontiguousarray(mi["b"][:, t:t + 1])),
            _dev(mi["A_log"]), _dev(mi["dt_bias"]), W.H_qk, W.d_k, W.H_v, W.d_v, conv_state=cs,
            update_conv_state=True)
        torch.cuda.synchronize()
        for b in range(B):
            assert _bf16_close(host(q)[b, 0], full[b]["q"][t])
            assert _bf16_close(host(v)[b, 0], full[b]["v"][t])
            assert rel_max(host(g)[b, 0], full[b]["g"][t]) <= 1e-5
    for b in range(B):
        np.testing.assert_array_equal(host(cs)[b], full[b]["conv_state"][0])


def test_mixer_end_to_end():
    """prologue -> chunked delta rule (in-kernel l2 norm, 1/sqrt(d_k) scale) -> output norm,
    against the references composed the same way."""
    gdn = _gdn()
    T = 150
    mi = synth.make_mixer_inputs(W, seed=9, T=T)
    q, k, v, g, beta, _ = _run_prologue(mi)[0]
    o, fin = gdn.gdn_chunk_fwd(q, k, v, g, beta, l2norm=True)
    out = gdn.gdn_gated_norm(o, _dev(mi["z"], torch.bfloat16), _dev(mi["norm_w"]), eps=1e-6)
    torch.cuda.synchronize()
    r, _ = _prologue_ref(mi, W.H_qk, W.d_k, W.H_v, W.d_v)
    # the delta rule's reference takes the prologue's outputs as the GPU stored them (bf16)
    ref = gdn_ref.recurrent(host(q), host(k), host(v), host(g), host(beta), l2norm=True)
    want = mixer_ref.gated_rmsnorm(ref["o"], mi["z"], mi["norm_w"], eps=1e-6)
    assert rel_max(host(out), want) <= TOL_BF16_O
    assert rel_fro(host(fin), ref["final"]) <= TOL_BF16_STATE
    # and the stored q, k, v are the prologue reference's, rounded once
    assert _bf16_close(host(q).reshape(-1, W.H_qk, W.d_k), r["q"])
