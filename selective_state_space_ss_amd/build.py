"""Build the gfx950 HIP library libssscan.so in-tree with hipcc.

    python -m selective_state_space_ss_amd.build

Each translation unit under csrc/ is compiled to an object in _build/ (in
parallel), then linked into selective_state_space_ss_amd/libssscan.so.
Packed-FP32 instructions are switched off for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssscan.so")
ARCH = "gfx950"

SOURCES = ["ss_abi.hip", "scan_fwd.hip", "scan_states.hip", "scan_rows.hip", "state_update.hip", "gated_scan.hip", "effective_attention.hip", "producers.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source additions. The chunked prompt scan and its states variants are
# scheduled with LLVM's iterative-ILP machine scheduler. On MI355X it measured
# 342 against 346.5 us at batch 8 x 5120 channels x 2048 tokens, 85.7 against
# 89.0 us at 4 x 1536 x 2048 (no change with resets), and 360 against 374 us
# (one selected state) and 1445 against 1456 us (every state) at the first
# shape, with identical results. The other files keep the default: with it
# the producers, the attention and the decode step measured no change, and
# this toolchain's compiler aborts on gated_scan.hip (max-ilp made that
# kernel 14 % slower).
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"scan_fwd.hip": _ILP, "scan_states.hip": _ILP}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssscan.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass reports the device-only feature flag as unknown; that line is noise
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
