"""Build libgdn.so in-tree: hipcc for gfx950, one object per source, then a shared link.

Usage: python -m gated_deltanet_linear_amd.build   (or call build()).

`python -m gated_deltanet_linear_amd.build --sanitize` builds a second copy,
_build_san/libgdn_san.so, whose host code (validation, dispatch, the workspace layout)
carries AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built as
usual.  It is for CPU runs of the ABI tests only: load it through GDN_LIBRARY with the
ASan runtime preloaded (the command is printed at the end of the build).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libgdn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SAN_DIR = os.path.join(ROOT, "_build_san")
SAN_OUT = os.path.join(SAN_DIR, "libgdn_san.so")
# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]

SOURCES = ["gdn_api.cpp", "gdn_step.hip", "gdn_chunk.hip", "gdn_mixer.hip", "gdn_noalloc.hip",
           "gdn_fused.hip"]

# Packed-fp32 VALU forms are kept out of the generated code (the compiler would
# otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in ordinary VGPRs: the kernels post-process every
          # accumulator with vector ALU code, which would otherwise copy it out of AGPRs
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_DIR if sanitize else BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + (SAN_FLAGS if sanitize else []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def asan_runtime() -> str:
    """The shared ASan runtime of hipcc's clang (to LD_PRELOAD into a Python process)."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(p):
        raise RuntimeError("ASan runtime not found")
    return p


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link gated_deltanet_linear_amd/libgdn.so
    (with sanitize: the host-sanitized copy _build_san/libgdn_san.so)."""
    out = SAN_OUT if sanitize else OUT
    os.makedirs(SAN_DIR if sanitize else BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if sanitize:
        cmd += ["-shared-libsan"] + SAN_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
        if sanitize:
            print(f"run: GDN_LIBRARY={out} LD_PRELOAD={asan_runtime()} ASAN_OPTIONS=detect_leaks=0 "
                  "python -m pytest tests/test_abi.py")
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
