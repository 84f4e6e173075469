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
# measurement support for bench.py (issue-rate probe), kept out of the scan's library
PROBE_LIB = os.path.join(PKG, "libssprobe.so")
PROBE_SOURCES = ["probe_issue.hip", "probe_lds.hip"]
ARCH = "gfx950"

# the race check of the chunked scan's B/C stage (tests only): the sources
# that instantiate the chunked kernel, rebuilt with SS_LDS_POISON=1 and linked
# with the other objects of the library
POISON_LIB = os.path.join(PKG, "libssscan_lds_poison.so")
POISON_SOURCES = ["scan_fwd.hip", "scan_fwd_reset.hip", "scan_fwd_conv.hip", "scan_states.hip"]
SOURCES = ["ss_abi.hip", "scan_fwd.hip", "scan_fwd_reset.hip", "scan_fwd_conv.hip", "scan_states.hip", "scan_rows.hip", "state_update.hip", "gated_scan.hip", "effective_attention.hip", "producers.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source additions. The chunked prompt scan's instances with a reset mask
# (scan_fwd_reset.hip) and the states variants are scheduled with LLVM's
# iterative-ILP machine scheduler; the plain scan without resets
# (scan_fwd.hip) keeps the default one. Measured on MI355X (same-box A/B, the
# current kernels): packed sequences with resets 312.6 us with iterative-ILP
# against 318.1 us with the default scheduler (4 x 2048 x 8192); without
# resets 333.7 against 330.2 us (8 x 5120 x 2048) and 84.7 against 83.7 us
# (4 x 1536 x 2048). The states variants measured 360 against 374 us (one
# selected state) and 1445 against 1456 us (every state) with it. The other
# files keep the default: with it the producers, the attention and the decode
# step measured no change, and this toolchain's compiler aborts on
# gated_scan.hip (max-ilp made that kernel 14 % slower).
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"scan_fwd_reset.hip": _ILP, "scan_states.hip": _ILP}


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

    def compile_one(job):
        src, poison = job
        obj = os.path.join(BUILD, src.replace(".hip", "_lds_poison.o" if poison else ".o"))
        defs = ["-DSS_LDS_POISON=1"] if poison else []
        out = _run([cc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *defs, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out)
        return obj

    jobs = [(s, False) for s in SOURCES + PROBE_SOURCES] + [(s, True) for s in POISON_SOURCES]
    with ThreadPoolExecutor(len(jobs)) as ex:
        objs = dict(zip(jobs, ex.map(compile_one, jobs)))
    poison_objs = [objs[(n, n in POISON_SOURCES)] for n in SOURCES]
    for lib, names in ((LIB, [objs[(n, False)] for n in SOURCES]), (PROBE_LIB, [objs[(n, False)] for n in PROBE_SOURCES]),
                       (POISON_LIB, poison_objs)):
        tmp = lib + ".tmp%d" % os.getpid()
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *names])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
