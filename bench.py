#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X: the gated delta rule's prompt, decode and states paths.

A step is one gdn_chunk_fwd call over the 4096-token single-layer prefill (B=1, 16
query/key heads over 32 value heads, width 128, bf16 q/k/v, fp32 g/beta/state/o, chunk
64): the whole chunked hot path, input in HBM, output o and final state written.  The
headline `value` is its token throughput.  The same JSON line also carries, each with its
own roofline, the decode step (256 sequences, 1000 consecutive in-place steps), the packed
8-sequence prefill (49,802 tokens) and the per-token states readout (2048 tokens, 4 GiB of
fp32 states), and the fp64 CPU oracle timed on the host beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu] [--calib]

Each roofline's `traffic` (measured HBM bytes per launch) comes from
profiles/traffic.json, which holds rocprofv3 FETCH_SIZE + WRITE_SIZE readings per
kernel scaled by a plain-copy calibration, with a hash of the kernel's source file:
when the source has changed since the counters were taken, `traffic` is null.
`--calib` only runs a 256 MiB device-to-device copy (the calibration kernel).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
N_SETS = 3                      # independent input/output sets rotated per step (cold reads)
# Calls timed per row of the longer workloads (packed, states): the fixed cost of a timed
# region (the first launch after a synchronisation, the wake-up at its end) is ~0.1-0.2 ms,
# so a few calls of ~1 ms would carry it into every call's figure
NSTEPS_LONG = 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib", action="store_true")
    return ap.parse_args()


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rocm_version():
    """The ROCm release of /opt/rocm and torch's HIP version."""
    ver = None
    try:
        with open("/opt/rocm/.info/version") as f:
            ver = f.read().strip()
    except OSError:
        pass
    try:
        import torch
        hip = torch.version.hip
    except Exception:
        hip = None
    return {"rocm": ver, "torch_hip": hip}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic.json, or None when absent
    or when the kernel's source file no longer matches the hash recorded with it."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[kernel]
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["sha256"]:
                return None
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


class Prepared:
    """One chunked call with every pointer and the workspace bound once, so the timed
    loop issues the C call directly (no per-call tensor checks)."""

    def __init__(self, lib, fn, shape, args):
        self.lib, self.fn, self.shape, self.args = lib, fn, shape, args

    def __call__(self):
        st = self.fn(ctypes.byref(self.shape), *self.args)
        if st != 0:
            raise RuntimeError(self.lib.gdn_last_error().decode())

    def check_status(self):
        """The int32 status word at the start of the workspace after the last call: 0, or
        the call's results are invalid (bad cu_seqlens, an fp16 overflow, a late hand-over)."""
        import torch
        word = int(self.ws[:4].view(torch.int32).item())
        if word != 0:
            raise RuntimeError(f"status word {word} after the timed calls")


def prepare_chunk(lib, b, d, states=False, select=None, gated=None):
    """Bind a gdn_chunk_fwd (or gdn_states_fwd) call on device inputs d; with states and
    select = (t_begin, t_end, t_step), a gdn_states_fwd_strided call; with gated = (z,
    weight), a gdn_chunk_fwd_gated call (eps 1e-6)."""
    import torch
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    B, T, H_qk, d_k = d["q"].shape
    H_v, d_v = d["v"].shape[-2:]
    N = B if d["cu"] is None else d["cu"].numel() - 1
    s = b.GdnShape(B, T, H_qk, H_v, d_k, d_v, 64, d_k ** -0.5, b.GDN_BF16, b.GDN_F32, 0)
    nseq = 0 if d["cu"] is None else N
    dev = d["q"].device
    o = torch.empty((B, T, H_v, d_v), dtype=torch.float32, device=dev)
    fin = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if states:
        need = lib.gdn_states_fwd_workspace(ctypes.byref(s), nseq)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        if select is None:
            st = torch.empty((B, T, H_v, d_k, d_v), dtype=torch.float32, device=dev)
            args = [P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["s0"]), P(d["cu"]), nseq,
                    P(o), P(st), P(fin), P(ws), need, stream]
            fn = lib.gdn_states_fwd
        else:
            t0, t1, step = select
            st = torch.empty((B, len(range(t0, t1, step)), H_v, d_k, d_v), dtype=torch.float32, device=dev)
            args = [P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["s0"]), P(d["cu"]), nseq,
                    P(o), P(st), t0, t1, step, P(fin), P(ws), need, stream]
            fn = lib.gdn_states_fwd_strided
        keep = (o, fin, ws, st)
    else:
        need = lib.gdn_chunk_fwd_workspace(ctypes.byref(s), nseq)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        if gated is None:
            args = [P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["s0"]), P(d["cu"]), nseq,
                    P(o), P(fin), P(ws), need, stream]
            fn = lib.gdn_chunk_fwd
        else:
            args = [P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["s0"]), P(d["cu"]), nseq,
                    P(gated[0]), P(gated[1]), ctypes.c_float(1e-6), P(o), P(fin), P(ws), need, stream]
            fn = lib.gdn_chunk_fwd_gated
        keep = (o, fin, ws) + (gated or ())
    call = Prepared(lib, fn, s, args)
    call.ws = ws
    call.keep = keep + (d,)   # the C call holds raw pointers: keep every tensor alive
    return call


def timed_chunk_calls(lib, calls, steps, warmup, n_kernels):
    """Warm up, then time `steps` calls (rotating over `calls`) with the host clock between
    synchronisations and no instrumentation; then time each kernel over another `steps`
    calls with HIP events that the library's timing hook records on the launch stream
    between its kernels.  Returns (ms per call, [ms per kernel])."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_kernels + 1)] for _ in range(steps)]
    for row in evs:          # torch creates an event's handle at its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    arrays = [(ctypes.c_void_p * (n_kernels + 1))(*[ctypes.c_void_p(e.cuda_event) for e in row])
              for row in evs]
    assert all(e.cuda_event for row in evs for e in row)
    for i in range(steps):
        lib.gdn_set_timing_events(arrays[i], n_kernels + 1)
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    lib.gdn_set_timing_events(None, 0)
    for c in calls:
        c.check_status()
    per_kernel = [sum(row[j].elapsed_time(row[j + 1]) for row in evs) / steps for j in range(n_kernels)]
    return (t1 - t0) * 1e3 / steps, per_kernel


def roofline(bound, achieved, peak, unit, traffic=None, **extra):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    r.update(extra)
    return r


def chunk_work(tokens, H_v, d_k=128, d_v=128, C=64):
    """Algorithmic work of the chunked path per token and value head (method's own count):
    6 d_k d_v (state terms) + C (3 d_k + 2 d_v) (intra-chunk products) + C^2/3 (solve) FLOP;
    bytes: q, k at query/key-head width (128 + 128), v 256, o fp32 512, g and beta 4 + 4."""
    flop = 6 * d_k * d_v + C * (3 * d_k + 2 * d_v) + C * C / 3
    carry_flop = 6 * d_k * d_v   # the chain kernel's share: the three products with the state
    nbytes = 128 + 128 + 256 + 512 + 4 + 4
    carry_bytes = 128 + 128 + 256 + 512
    th = tokens * H_v
    return flop * th, nbytes * th, carry_flop * th, carry_bytes * th


def bench_prefill(lib, b, synth, to_dev, steps, warmup):
    w = synth.WORKLOADS["prefill_t4096"]
    calls = []
    for s in range(N_SETS):
        calls.append(prepare_chunk(lib, b, to_dev(synth.make_inputs(w, seed=s))))
    ms, kern = timed_chunk_calls(lib, calls, steps, warmup, 3)
    tokens = w.B * w.T
    flop, nbytes, cflop, cbytes = chunk_work(tokens, w.H_v)
    names = ["plan", "solve", "chain"]
    dom = max(range(3), key=lambda i: kern[i])
    return w, ms, dict(zip(names, kern)), names[dom], flop, nbytes, cflop, cbytes


def timed_launches(fn, iters, warmup, torch):
    """Mean GPU time (ms) of `fn`, a bound C call that enqueues on the current stream,
    over `iters` back-to-back calls between two events on that stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def bench_next_rows(lib, b, synth, to_dev, dev, torch, np):
    """The widened rows: the 4096-token prefill at head ratios 1 (16/16) and 3 (16/48), the
    mixer's output norm and input prologue at that prefill's shape, and the decode step with
    the output norm fused, each with its roofline."""
    import dataclasses
    P = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = {}
    base = synth.WORKLOADS["prefill_t4096"]
    for H_v in (16, 48):
        w = dataclasses.replace(base, H_v=H_v)
        calls = [prepare_chunk(lib, b, to_dev(synth.make_inputs(w, seed=s))) for s in range(N_SETS)]
        ms, kern = timed_chunk_calls(lib, calls, 40, 3, 3)
        flop, nbytes, cflop, cbytes = chunk_work(w.T, H_v)
        out[f"prefill_t4096_h16_{H_v}"] = {
            "H_qk": 16, "H_v": H_v, "us_per_call": round(ms * 1e3, 2),
            "tokens_per_s": round(w.T / (ms / 1e3), 1),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain"], kern)},
            "roofline": roofline("mfma", cflop / (kern[2] / 1e3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
                                 kernel="chain_kernel")}
        log(f"prefill 16/{H_v} heads: {ms * 1e3:.1f} us/call")
        del calls
    # the output norm fused into the head-wide chain: 8 dense rows of the prefill's shape
    # (8 x 32 sequence-heads, one workgroup each), gdn_chunk_fwd_gated against
    # gdn_chunk_fwd followed by gdn_gated_norm in place over o
    w8 = dataclasses.replace(base, B=8)
    d8 = to_dev(synth.make_inputs(w8, seed=0))
    mi = synth.make_mixer_inputs(w8, seed=1, T=w8.T, B=w8.B)
    z8 = torch.from_numpy(mi["z"]).to(dev, torch.bfloat16)
    nw8 = torch.from_numpy(mi["norm_w"]).to(dev)
    del mi
    call8 = prepare_chunk(lib, b, d8)
    callg8 = prepare_chunk(lib, b, d8, gated=(z8, nw8))
    _, kg8 = timed_chunk_calls(lib, [callg8], 20, 2, 3)
    _, k8 = timed_chunk_calls(lib, [call8], 20, 2, 3)
    # both compositions timed the same way: back-to-back calls between two events
    msg8 = timed_launches(callg8, 20, 2, torch)
    callg8.check_status()
    o8 = call8.keep[0]
    sn8 = b.GdnShape(w8.B, w8.T, 1, w8.H_v, 1, w8.d_v, 1, 1.0, b.GDN_BF16, b.GDN_F32, 0)
    nargs8 = [P(o8), P(z8), P(nw8), ctypes.c_float(1e-6), P(o8), stream]

    def chunk_then_norm8():
        call8()
        if lib.gdn_gated_norm(ctypes.byref(sn8), *nargs8) != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    msn8 = timed_launches(chunk_then_norm8, 20, 2, torch)
    call8.check_status()
    el8 = w8.B * w8.T * w8.H_v * w8.d_v
    out["gated_dense_b8_t4096"] = {
        "B": w8.B, "T": w8.T, "us_per_call_fused": round(msg8 * 1e3, 2),
        "kernel_us_fused": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain"], kg8)},
        "us_per_call_chunk_then_norm": round(msn8 * 1e3, 2),
        "kernel_us_chunk": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain"], k8)},
        "o_bytes_not_moved": el8 * (4 + 4),
        "chain_traffic_fused": measured_traffic("wide_kernel_gated"),
        "chain_traffic_unfused": measured_traffic("wide_kernel_dense"),
        "note": "fused: the chain applies the norm and writes only the normed output (fp32); "
                "unfused: the chain writes o (fp32), the norm reads it back with z and rewrites it"}
    log(f"dense 8 x 4096 with the output norm: fused {msg8 * 1e3:.1f} us/call, "
        f"chunk then norm {msn8 * 1e3:.1f}")
    del d8, z8, nw8, call8, callg8, o8
    # mixer steps at the prefill's shape (T = 4096, 16 qk / 32 v heads, d = 128), each timed
    # over N_SETS input and output sets in turn (more than the last-level cache holds)
    w = base
    bf = torch.bfloat16
    T = w.T
    psets, nsets = [], []
    for si in range(N_SETS):
        mi = synth.make_mixer_inputs(w, seed=si)
        x = torch.from_numpy(mi["x"]).to(dev, bf)
        C = x.shape[2]
        ps = dict(x=x, conv_w=torch.from_numpy(mi["conv_w"]).to(dev), a=torch.from_numpy(mi["a"]).to(dev),
                  b=torch.from_numpy(mi["b"]).to(dev), A_log=torch.from_numpy(mi["A_log"]).to(dev),
                  dt_bias=torch.from_numpy(mi["dt_bias"]).to(dev),
                  q=torch.empty((1, T, w.H_qk, w.d_k), dtype=bf, device=dev),
                  k=torch.empty((1, T, w.H_qk, w.d_k), dtype=bf, device=dev),
                  v=torch.empty((1, T, w.H_v, w.d_v), dtype=bf, device=dev),
                  g=torch.empty((1, T, w.H_v), dtype=torch.float32, device=dev),
                  beta=torch.empty((1, T, w.H_v), dtype=torch.float32, device=dev))
        ps["args"] = [P(ps["x"]), P(ps["conv_w"]), P(None), P(None), P(ps["a"]), P(ps["b"]), P(ps["A_log"]),
                      P(ps["dt_bias"]), P(None), 0, P(ps["q"]), P(ps["k"]), P(ps["v"]), P(ps["g"]),
                      P(ps["beta"]), stream]
        psets.append(ps)
        y = torch.from_numpy(np.random.default_rng(1 + si).standard_normal((1, T, w.H_v, w.d_v),
                                                                             dtype=np.float32)).to(dev)
        ns = dict(y=y, z=torch.from_numpy(mi["z"]).to(dev, bf), norm_w=torch.from_numpy(mi["norm_w"]).to(dev),
                  yo=torch.empty_like(y))
        ns["args"] = [P(ns["y"]), P(ns["z"]), P(ns["norm_w"]), ctypes.c_float(1e-6), P(ns["yo"]), stream]
        nsets.append(ns)
    sp = b.GdnShape(1, T, w.H_qk, w.H_v, w.d_k, w.d_v, 1, 1.0, b.GDN_BF16, b.GDN_F32, 0)
    turn = [0]

    def prologue():
        ps = psets[turn[0] % N_SETS]
        turn[0] += 1
        if lib.gdn_mixer_prologue(ctypes.byref(sp), *ps["args"]) != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    ms = timed_launches(prologue, 51, 6, torch)
    pbytes = T * C * 2 + C * 4 * 4 + 2 * T * w.H_v * 4 + T * C * 2 + 2 * T * w.H_v * 4
    # the same bytes moved by the runtime's device copy (half read, half written), over
    # as many rotated buffers: what a plain stream of this size reaches on this GPU
    csets = [(torch.empty(pbytes // 2, dtype=torch.uint8, device=dev),
              torch.empty(pbytes // 2, dtype=torch.uint8, device=dev)) for _ in range(N_SETS)]

    def copy_same():
        src, dst = csets[turn[0] % N_SETS]
        turn[0] += 1
        dst.copy_(src)
    ms_copy = timed_launches(copy_same, 51, 6, torch)
    del csets
    out["prologue_t4096"] = {"us_per_call": round(ms * 1e3, 2), "input_sets_rotated": N_SETS,
                             "device_copy_same_bytes_us": round(ms_copy * 1e3, 2),
                             "device_copy_same_bytes_hbm_frac": round(pbytes / (ms_copy / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                             "roofline": roofline("hbm", pbytes / (ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                                  traffic=measured_traffic("conv_silu_kernel"),
                                                  kernel="conv_silu_kernel (gates in the same launch)",
                                                  algorithmic_bytes=pbytes)}
    log(f"prologue: {ms * 1e3:.1f} us/call")
    sn = b.GdnShape(1, T, 1, w.H_v, 1, w.d_v, 1, 1.0, b.GDN_BF16, b.GDN_F32, 0)

    def norm():
        ns = nsets[turn[0] % N_SETS]
        turn[0] += 1
        if lib.gdn_gated_norm(ctypes.byref(sn), *ns["args"]) != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    ms = timed_launches(norm, 51, 6, torch)
    nbytes = T * w.H_v * w.d_v * (4 + 2 + 4) + w.d_v * 4
    out["gated_norm_t4096"] = {"us_per_call": round(ms * 1e3, 2), "input_sets_rotated": N_SETS,
                               "roofline": roofline("hbm", nbytes / (ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                                    traffic=measured_traffic("gated_norm_kernel"),
                                                    kernel="gated_norm_kernel", algorithmic_bytes=nbytes)}
    log(f"gated norm: {ms * 1e3:.1f} us/call")
    norm_w = nsets[0]["norm_w"]
    del psets, nsets
    # the decode step with the output norm fused (256 sequences, as the decode row)
    wd = synth.WORKLOADS["decode_b256"]
    pool = synth.make_decode_pool(wd, seed=0)
    qd = torch.from_numpy(pool["q"][0]).to(dev, bf)
    kd = torch.from_numpy(pool["k"][0]).to(dev, bf)
    vd = torch.from_numpy(pool["v"][0]).to(dev, bf)
    gd = torch.from_numpy(pool["g"][0]).to(dev)
    bd = torch.from_numpy(pool["beta"][0]).to(dev)
    state = torch.from_numpy(pool["s0"]).to(dev)
    zd = torch.from_numpy(synth.make_mixer_inputs(base, seed=2, T=1, B=wd.B)["z"]).to(dev, bf)
    od = torch.empty((wd.B, 1, wd.H_v, wd.d_v), dtype=torch.float32, device=dev)
    sd = b.GdnShape(wd.B, 1, wd.H_qk, wd.H_v, 128, 128, 64, 128 ** -0.5, b.GDN_BF16, b.GDN_F32, 0)
    dargs = [P(qd), P(kd), P(vd), P(gd), P(bd), P(state), P(zd), P(norm_w), ctypes.c_float(1e-6), P(od), stream]

    def gated_step():
        if lib.gdn_recurrent_step_gated(ctypes.byref(sd), *dargs) != 0:
            raise RuntimeError(lib.gdn_last_error().decode())
    ms = timed_launches(gated_step, 200, 10, torch)
    dbytes = 2 * wd.B * wd.H_v * 128 * 128 * 4 + wd.B * (2 * wd.H_qk * 128 * 2 + wd.H_v * 128 * 2 +
                                                        2 * wd.H_v * 4 + wd.H_v * 128 * (4 + 2))
    out["decode_gated_b256"] = {"us_per_step": round(ms * 1e3, 2),
                                "roofline": roofline("hbm", dbytes / (ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                                     traffic=measured_traffic("step_kernel_gated"),
                                                     kernel="step_kernel (norm fused)", algorithmic_bytes=dbytes)}
    log(f"decode step with the norm fused: {ms * 1e3:.1f} us/step")
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from gated_deltanet_linear_amd import binding as b
    from gated_deltanet_linear_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib:
        # the calibration kernel for the HBM byte counters: 256 MiB read + 256 MiB written
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib": "copy", "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4}))
        return
    lib = b.load_library()

    def to_dev(inp):
        out = {key: torch.from_numpy(np.ascontiguousarray(inp[key])).to(dev, torch.bfloat16)
               for key in ("q", "k", "v")}
        for key in ("g", "beta"):
            out[key] = torch.from_numpy(inp[key]).to(dev)
        out["s0"] = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).to(dev)
        out["cu"] = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(dev)
        return out

    # ---- headline: prefill, T = 4096 -------------------------------------------------
    log("prefill_t4096: generating inputs and timing")
    w, ms, kern, dom, flop, nbytes, cflop, cbytes = bench_prefill(lib, b, synth, to_dev, args.steps,
                                                                  args.warmup)
    tokens = w.B * w.T
    value = tokens / (ms / 1e3)
    kd = kern["chain"]
    log(f"prefill: {ms * 1e3:.1f} us/step, kernels(us) " +
        ", ".join(f"{k}={v * 1e3:.1f}" for k, v in kern.items()))
    # the chain kernel (state carry and output) dominates; its algorithmic work is its
    # share of the method's FLOPs (the three state products K S, K^T U'', Q S), priced
    # against dense bf16 MFMA
    rl = roofline("mfma", cflop / (kd / 1e3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
                  traffic=measured_traffic("chain_kernel"), kernel="chain_kernel",
                  kernel_us=round(kd * 1e3, 2), algorithmic_flop=cflop,
                  hbm_achieved=round(cbytes / (kd / 1e3) / 1e9, 1), hbm_peak=HBM_PEAK_GBS,
                  hbm_frac=round(cbytes / (kd / 1e3) / 1e9 / HBM_PEAK_GBS, 4))
    path = {"us_per_call": round(ms * 1e3, 2),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
            "hbm_GBs": round(nbytes / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_TFLOPs": round(flop / (ms / 1e3) / 1e12, 2),
            "mfma_frac": round(flop / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_flop": flop, "algorithmic_bytes": nbytes}
    ts, tc = measured_traffic("solve_kernel"), measured_traffic("chain_kernel")
    path["traffic"] = None if ts is None or tc is None else ts + tc
    path["traffic_over_algorithmic"] = None if path["traffic"] is None else round(path["traffic"] / nbytes, 3)
    result = {
        "metric": "GDN prefill tokens/s + decode steps/s on 1 MI355X; % MFMA/HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_t4096", "B": 1, "T": 4096, "H_qk": 16, "H_v": 32, "d_k": 128,
                   "d_v": 128, "chunk": 64, "inputs": "bf16 q/k/v, fp32 g/beta", "o": "fp32",
                   "input_sets_rotated": N_SETS},
        "roofline": rl,
        "path": path,
        "software": rocm_version(),
    }

    if not args.headline_only:
        # ---- decode: 256 sequences, 1000 consecutive steps ---------------------------
        log("decode_b256: timing 1000 steps")
        wd = synth.WORKLOADS["decode_b256"]
        pool = synth.make_decode_pool(wd, seed=0)
        qp = torch.from_numpy(pool["q"]).to(dev, torch.bfloat16)
        kp = torch.from_numpy(pool["k"]).to(dev, torch.bfloat16)
        vp = torch.from_numpy(pool["v"]).to(dev, torch.bfloat16)
        gp = torch.from_numpy(pool["g"]).to(dev)
        bp = torch.from_numpy(pool["beta"]).to(dev)
        state = torch.from_numpy(pool["s0"]).to(dev)
        o = torch.empty((wd.B, 1, wd.H_v, wd.d_v), dtype=torch.float32, device=dev)
        s = b.GdnShape(wd.B, 1, wd.H_qk, wd.H_v, 128, 128, 64, 128 ** -0.5, b.GDN_BF16, b.GDN_F32, 0)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        dargs = [[P(qp[i]), P(kp[i]), P(vp[i]), P(gp[i]), P(bp[i]), P(state), P(o), stream]
                 for i in range(wd.pool)]
        for i in range(16):
            lib.gdn_recurrent_step(ctypes.byref(s), *dargs[i % wd.pool])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nsteps = args.decode_steps
        t0 = time.perf_counter()
        e0.record()
        for i in range(nsteps):
            st = lib.gdn_recurrent_step(ctypes.byref(s), *dargs[i % wd.pool])
            if st != 0:
                raise RuntimeError(lib.gdn_last_error().decode())
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / nsteps
        step_ms = e0.elapsed_time(e1) / nsteps
        dbytes = 2 * wd.B * wd.H_v * 128 * 128 * 4 + wd.B * (2 * wd.H_qk * 128 * 2 + wd.H_v * 128 * 2 +
                                                            2 * wd.H_v * 4 + wd.H_v * 128 * 4)
        del qp, kp, vp, gp, bp, state, o
        # the same bytes moved by the runtime's device copy (half read, half written; each
        # half is twice the last-level cache): what a plain stream of this size reaches
        csrc = torch.empty(dbytes // 2, dtype=torch.uint8, device=dev)
        cdst = torch.empty(dbytes // 2, dtype=torch.uint8, device=dev)
        ms_copy = timed_launches(lambda: cdst.copy_(csrc), 50, 5, torch)
        del csrc, cdst
        result["decode"] = {
            "workload": "decode_b256", "steps": nsteps, "us_per_step": round(step_ms * 1e3, 2),
            "wall_us_per_step": round(wall * 1e6, 2),
            "steps_per_s": round(1e3 / step_ms, 1), "tokens_per_s": round(wd.B * 1e3 / step_ms, 1),
            "device_copy_same_bytes_us": round(ms_copy * 1e3, 2),
            "device_copy_same_bytes_hbm_frac": round(dbytes / (ms_copy / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": roofline("hbm", dbytes / (step_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                 traffic=measured_traffic("step_kernel"), kernel="step_kernel",
                                 algorithmic_bytes=dbytes)}
        log(f"decode: {step_ms * 1e3:.1f} us/step (device copy of the same bytes {ms_copy * 1e3:.1f} us)")

        # ---- packed prefill: 8 sequences, 49,802 tokens ------------------------------
        log("packed_8seq: generating inputs and timing")
        wp = synth.WORKLOADS["packed_8seq"]
        dp = to_dev(synth.make_inputs(wp, seed=0))
        callp = prepare_chunk(lib, b, dp)
        msp, kp_ = timed_chunk_calls(lib, [callp], NSTEPS_LONG, 2, 3)
        flop_p, bytes_p, cflop_p, cbytes_p = chunk_work(wp.T, wp.H_v)
        result["packed"] = {
            "workload": "packed_8seq", "tokens": wp.T, "us_per_call": round(msp * 1e3, 2),
            "tokens_per_s": round(wp.T / (msp / 1e3), 1),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain"], kp_)},
            "roofline": roofline("mfma", cflop_p / (kp_[2] / 1e3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s",
                                 traffic=measured_traffic("wide_kernel_packed"),
                                 kernel="wide_kernel (two workgroups per sequence and value head, half "
                                        "of its columns each)",
                                 mfma_frac=round(cflop_p / (kp_[2] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)),
            "path_mfma_frac": round(flop_p / (msp / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "path_hbm_frac": round(bytes_p / (msp / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"packed: {msp * 1e3:.1f} us/call")
        # the same call with the mixer's output norm (gdn_chunk_fwd_gated): packed sequences
        # split each head over two workgroups, so the norm follows the chain in place over o;
        # against gdn_chunk_fwd followed by gdn_gated_norm
        mi = synth.make_mixer_inputs(wp, seed=1)
        zp = torch.from_numpy(mi["z"]).to(dev, torch.bfloat16)
        nwp = torch.from_numpy(mi["norm_w"]).to(dev)
        del mi
        callg = prepare_chunk(lib, b, dp, gated=(zp, nwp))
        _, kg_ = timed_chunk_calls(lib, [callg], NSTEPS_LONG, 2, 3)
        # both compositions timed the same way: back-to-back calls between two events
        msg = timed_launches(callg, NSTEPS_LONG, 2, torch)
        callg.check_status()
        op = callp.keep[0]
        sn = b.GdnShape(1, wp.T, 1, wp.H_v, 1, wp.d_v, 1, 1.0, b.GDN_BF16, b.GDN_F32, 0)
        nargs = [ctypes.c_void_p(op.data_ptr()), ctypes.c_void_p(zp.data_ptr()), ctypes.c_void_p(nwp.data_ptr()),
                 ctypes.c_float(1e-6), ctypes.c_void_p(op.data_ptr()),
                 ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)]

        def chunk_then_norm():
            callp()
            if lib.gdn_gated_norm(ctypes.byref(sn), *nargs) != 0:
                raise RuntimeError(lib.gdn_last_error().decode())
        msn = timed_launches(chunk_then_norm, NSTEPS_LONG, 2, torch)
        callp.check_status()
        result["packed"]["gated"] = {
            "us_per_call": round(msg * 1e3, 2),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain"], kg_)},
            "us_per_call_chunk_then_norm": round(msn * 1e3, 2),
            "route": "chain with each head split over two workgroups, then the norm in place over o"}
        log(f"packed with the output norm: {msg * 1e3:.1f} us/call, chunk then norm {msn * 1e3:.1f}")
        del dp, callp, callg, zp, nwp

        # ---- states readout: T = 2048, 4 GiB of fp32 states --------------------------
        log("states_t2048: generating inputs and timing")
        ws_ = synth.WORKLOADS["states_t2048"]
        dsx = to_dev(synth.make_inputs(ws_, seed=0))
        calls = prepare_chunk(lib, b, dsx, states=True)
        mss, ks_ = timed_chunk_calls(lib, [calls], NSTEPS_LONG, 2, 4)
        # every state is kept: the chain kernel streams them itself (no stream kernel runs);
        # its bytes are the states plus the path's q, k, v, g, beta and o
        sbytes = ws_.T * ws_.H_v * 128 * 128 * 4
        cbytes_s = sbytes + ws_.T * ws_.H_v * 1032
        kchain = ks_[2] + ks_[3]
        result["states"] = {
            "workload": "states_t2048", "tokens": ws_.T, "us_per_call": round(mss * 1e3, 2),
            "tokens_per_s": round(ws_.T / (mss / 1e3), 1),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain", "stream"], ks_)},
            "roofline": roofline("hbm", cbytes_s / (kchain / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                 traffic=measured_traffic("chain_kernel_states"),
                                 kernel="chain_kernel (32-column blocks streaming the states)",
                                 algorithmic_bytes=cbytes_s),
            "path_hbm_frac": round(cbytes_s / (mss / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"states: {mss * 1e3:.1f} us/call")
        del calls
        # the same call keeping one state per 64-token chunk (the chunk-boundary states)
        callx = prepare_chunk(lib, b, dsx, states=True, select=(63, ws_.T, 64))
        msx, kx_ = timed_chunk_calls(lib, [callx], NSTEPS_LONG, 3, 4)
        result["states"]["strided_t_step_64"] = {
            "us_per_call": round(msx * 1e3, 2), "tokens_per_s": round(ws_.T / (msx / 1e3), 1),
            "states_kept": len(range(63, ws_.T, 64)),
            "route": "the chain writes chunk-start states and write vectors; the stream kernel expands the kept ones",
            "kernel_us": {k: round(v * 1e3, 2) for k, v in zip(["plan", "solve", "chain", "stream"], kx_)}}
        log(f"states, one per chunk: {msx * 1e3:.1f} us/call")
        del dsx, callx

        result["next_rows"] = bench_next_rows(lib, b, synth, to_dev, dev, torch, np)

    # ---- the fp64 CPU oracle on the host, on the same workload -------------------------
    if not args.no_cpu:
        from oracle import gdn_ref
        inp = synth.make_inputs(w, seed=0)
        nthr = int(os.environ.get("OMP_NUM_THREADS", "0")) or gdn_ref.max_threads()
        heads = list(range(w.H_v))
        t0 = time.perf_counter()
        reps = 0
        while True:  # a bounded sample: at least 10 s of oracle work
            gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], heads=heads,
                              want_final=False, nthreads=nthr)
            reps += 1
            if time.perf_counter() - t0 >= 10.0 or reps >= 400:
                break
        dt = (time.perf_counter() - t0) / reps
        # the same oracle on one core: 8 of the 32 heads, at least 5 s, scaled to all heads
        heads1 = list(range(8))
        t0 = time.perf_counter()
        reps1 = 0
        while True:
            gdn_ref.recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], heads=heads1,
                              want_final=False, nthreads=1)
            reps1 += 1
            if time.perf_counter() - t0 >= 5.0 or reps1 >= 100:
                break
        dt1 = (time.perf_counter() - t0) / reps1 * (w.H_v / len(heads1))
        result["cpu_baseline"] = {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": nthr,
                                  "kind": "oracle", "cpu_model": cpu_model(),
                                  "value_1core": round(tokens / dt1, 1),
                                  "sample": f"prefill_t4096, all 32 value heads x 4096 tokens, "
                                            f"fp64 recurrence, {reps} repetition(s) of {dt:.2f} s on "
                                            f"{nthr} threads; one core: heads 0-7, {reps1} repetition(s), "
                                            f"scaled to 32 heads ({dt1:.2f} s per prefill)"}
        log(f"cpu oracle: {dt:.2f} s per prefill on {nthr} threads, {dt1:.2f} s on one core")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
