"""Host-side checks of bench.py (CPU): the one-GPU contract and the algorithmic work it prices
the kernels against."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_chunk_work_per_token_and_head():
    # 6 d_k d_v (the state terms) + C (3 d_k + 2 d_v) (the in-chunk products) + C^2 / 3 (the
    # solve) FLOP, and q, k (128 + 128 at the query/key-head width), v 256, o fp32 512, g, beta 4 + 4 bytes
    flop, nbytes, cflop, cbytes = bench.chunk_work(1, 1)
    assert flop == pytest.approx(6 * 128 * 128 + 64 * (3 * 128 + 2 * 128) + 64 * 64 / 3)
    assert flop == pytest.approx(140629.33, abs=0.01)
    assert nbytes == 1032 and cflop == 98304 and cbytes == 1024
    # the 4096-token prefill at 32 value heads: 18.4 GFLOP, 135.3 MB, 12.9 GFLOP in the chain
    flop, nbytes, cflop, _ = bench.chunk_work(4096, 32)
    assert flop == pytest.approx(18.43e9, rel=1e-3)
    assert nbytes == 4096 * 32 * 1032 and cflop == 12884901888


def test_roofline_fraction():
    r = bench.roofline("hbm", 6400.0, 8000.0, "GB/s", traffic=123, kernel="k")
    assert r["frac"] == 0.8 and r["bound"] == "hbm" and r["traffic"] == 123 and r["kernel"] == "k"


def test_status_word_check():
    # a timed row fails when a call left a nonzero status word at the start of its workspace
    import torch
    call = bench.Prepared(None, None, None, [])
    call.ws = torch.zeros(64, dtype=torch.uint8)
    call.check_status()
    call.ws[:4].view(torch.int32)[0] = 2
    with pytest.raises(RuntimeError, match="status word 2"):
        call.check_status()
