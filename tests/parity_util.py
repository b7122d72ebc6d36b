"""Shared helpers of the parity tests: moving seeded inputs to the GPU and comparing
against the fp64 oracle with the stated tolerances.

Tolerances (max-abs error relative to the RMS of the oracle's output):
- fp32 inputs:  max|o - o_ref| <= 1e-4 * RMS(o_ref); the same bound for states and the
  final state;
- bf16 inputs:  max|o - o_ref| <= 2e-2 * RMS(o_ref); final state (and states) within
  1e-3 relative Frobenius norm over the compared tensor.
"""
import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16_O = 2e-2
TOL_BF16_STATE = 1e-3


def to_dev(inp, device="cuda"):
    """Seeded numpy inputs -> device tensors in the storage dtype (bf16 values are exact)."""
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(device=device, dtype=dt)
    for key in ("g", "beta"):
        out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(device)
    out["s0"] = None if inp.get("s0") is None else torch.from_numpy(inp["s0"]).to(device)
    cu = inp.get("cu_seqlens")
    out["cu"] = None if cu is None else torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).to(device)
    return out


def rel_max(gpu, ref):
    """max |gpu - ref| / RMS(ref)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(gpu - ref))) / max(rms, 1e-30)


def rel_fro(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((gpu - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


def host(t):
    return t.detach().float().cpu().numpy()
