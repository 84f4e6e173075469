#!/usr/bin/env python3
"""Benchmark of the MI355X selective scan: one JSON line on stdout.

A step is one pass of the whole hot path at the Mamba-2.8B layer shape
(d_inner 5120, state_dim 16, bf16 I/O, fp32 state):
  * the prompt scan ss_scan_fwd over batch 8 x 2048 tokens, silu(z) gate and
    a random initial state (workload "mamba2p8b"), then
  * the single-token decode update ss_state_update of a batch-256 cached
    state, in place (workload "decode").
Inputs are seeded synthetic tensors of those shapes (no trained weights, no
dataset), resident in HBM before the timed region. W untimed warm-up steps
(continued until --warmup-seconds of wall time have passed, so the clocks
have ramped), then K timed steps between two device synchronisations.

value = whole-step algorithmic bytes / step time (GB/s). The per-kernel
durations come from HIP events recorded around each launch on the stream the
kernels run on.

roofline: the prompt scan dominates the step. Its roofline is the larger of
two times, as a fraction of the kernel time: the algorithmic bytes at the
8 TB/s HBM peak, and the transcendentals the method needs (one exp2 per token
and state coordinate for the decay, exp and log for the softplus, exp and rcp
for the gate) at the transcendental rate measured on MI355X by the issue-rate
probe (profiles/issue_rates_gfx950.json, written by --probe-issue). A second
figure, issue_frac, prices the method's whole minimum VALU work (the
transcendentals plus the FMA-class operations) at the probe's measured rates:
on gfx950 an exp2 occupies the same VALU issue slots as ordinary fp32 work
(about two FMA slots each; the probe finds no overlap), so that is the bound
the kernel actually runs against.

cpu_baseline: the fp64 CPU oracle (oracle/), unchanged, timed on this host's
cores over a bounded sample of the prompt workload's rows.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 matrix / packed vector, published (the unpacked VALU issues half)
ISSUE_FILE = os.path.join(ROOT, "profiles", "issue_rates_gfx950.json")
# Nominal gfx950 rates, used only if the measured file is missing: per CU and
# clock 64 fp32 FMA lanes (a wave64 VALU instruction every 4 clocks on each of
# 4 SIMDs) and 32 exp2 lanes, 256 CUs at 2.4 GHz.
NOMINAL_FMA_RATE = 64 * 256 * 2.4e9
NOMINAL_EXP_RATE = 32 * 256 * 2.4e9


def issue_rates():
    """(fp32 FMA lane-ops/s, exp2 lane-ops/s, source) from the committed
    probe measurement; the nominal rates if it is missing."""
    try:
        with open(ISSUE_FILE) as f:
            r = json.load(f)
        return r["fma_lane_ops_per_s"], r["exp2_lane_ops_per_s"], os.path.relpath(ISSUE_FILE, ROOT)
    except (OSError, ValueError, KeyError):
        return NOMINAL_FMA_RATE, NOMINAL_EXP_RATE, "nominal (64 FMA and 32 exp2 lanes per CU and clock, 2.4 GHz)"


def scan_work(w):
    """Algorithmic work of one prompt-scan launch of workload w.

    bytes: every input read once and every output written once.
    trans: transcendentals the method needs: per channel-token one exp2 per
    state coordinate (the decay), exp and log (softplus), and exp and rcp
    (the gate, when on).
    fma: the other fp32 operations, in FMA-class instructions: per token and
    state coordinate dt*A, (dt x)*B, h = a h + b, y += C h (4); per
    channel-token dt + bias, the softplus' max, add and log scaling (3), dt*x,
    y += D x (2) and, with the gate, 1 + e, z * r, y * silu (3)."""
    from selective_state_space_ss_amd.workloads import algorithmic_bytes
    ct = w.batch * w.channels * max(w.seqlen, 1)
    trans = ct * (w.state_dim + 2 + (2 if w.gate else 0))
    fma = ct * (4 * w.state_dim + 6 + (3 if w.gate else 0))
    return {"channel_tokens": ct, "bytes": algorithmic_bytes(w), "trans": trans, "fma": fma}


def scan_roofline(w, us: float, rates) -> dict:
    """Per-launch figures of a prompt scan that took `us` microseconds:
    GB/s, channel-tokens/s, the HBM and transcendental fractions, frac =
    max(HBM time, transcendental time) / kernel time, and issue_frac = the
    method's minimum VALU time (transcendentals at the exp2 rate plus the
    FMA-class work at the FMA rate, which share the issue slots) / kernel
    time."""
    fma_rate, exp_rate, _ = rates
    wk = scan_work(w)
    t = us * 1e-6
    hbm_s = wk["bytes"] / (PEAK_HBM_GBS * 1e9)
    exp_s = wk["trans"] / exp_rate
    issue_s = exp_s + wk["fma"] / fma_rate
    return {"us": round(us, 2), "GB_s": round(wk["bytes"] / t / 1e9, 1),
            "channel_tokens_per_s": round(wk["channel_tokens"] / t, 1), "algorithmic_bytes": wk["bytes"],
            "transcendentals": wk["trans"], "hbm_frac": round(hbm_s / t, 4), "exp_frac": round(exp_s / t, 4),
            "frac": round(max(hbm_s, exp_s) / t, 4), "issue_frac": round(issue_s / t, 4)}


def decode_roofline(w, us: float) -> dict:
    """The decode update is bound by HBM: frac = algorithmic bytes at 8 TB/s /
    kernel time."""
    from selective_state_space_ss_amd.workloads import algorithmic_bytes
    nbytes = algorithmic_bytes(w)
    t = us * 1e-6
    return {"us": round(us, 2), "GB_s": round(nbytes / t / 1e9, 1),
            "channel_updates_per_s": round(w.batch * w.channels / t, 1), "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ss_scan_fwd_mamba2p8b.json")
COPY_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=1.5,
                    help="keep warming up (untimed) until this much wall time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-token-states, gated-scan, effective-attention and producer measurements")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-configuration timings (tiny, Mamba-130M, packed reset, cold runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-time budget of the oracle sample")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run a 256 MiB device copy, then 3 steps, for a rocprofv3 --pmc pass (no JSON)")
    ap.add_argument("--counter-workload", metavar="NAME",
                    help="with --counter-pass: run 3 launches of that configuration's scan (tiny_fp32, mamba130m, "
                         "packed_reset, mamba2p8b), of ss_dt_proj at the producers' shape (dt_proj) or of "
                         "ss_gated_scan at its bench shape (gated), instead of the steps")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the FETCH_SIZE and WRITE_SIZE passes into " + TRAFFIC_FILE)
    ap.add_argument("--summarize-trace", metavar="KT_DIR",
                    help="print a markdown table of a rocprofv3 --kernel-trace directory, one row per kernel and "
                         "launch shape (grid x block), and exit")
    ap.add_argument("--probe-issue", metavar="OUT_JSON",
                    help="run the fp32 FMA / transcendental issue-rate probe, write its JSON to OUT_JSON, exit")
    ap.add_argument("--probe-lds", action="store_true",
                    help="launch the LDS bank probe once per offset pattern (for a rocprofv3 --pmc "
                         "SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS pass), print the pattern names as JSON, exit")
    ap.add_argument("--summarize-lds", metavar="PMC_DIR",
                    help="print a markdown table of conflict cycles per instruction from a --probe-lds pass, exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="print a markdown table of the counters of --pmc passes (one directory per pass) over the "
                         "dispatches of the kernel named by --counter-kernel: each counter summed over the chip's "
                         "counter instances per dispatch, then the median over the dispatches; exit")
    ap.add_argument("--counter-kernel", metavar="SUBSTRING", default="scan_fwd_kernel",
                    help="with --summarize-counters: the kernel name to select (a substring)")
    return ap.parse_args()


# (exp2 chains, FMA chains) per loop iteration of the issue-rate probe
# (libssprobe.so); the pure kernels give the two peaks, the mixed ones show
# whether the two kinds of work overlap.
PROBE_MIXES = [(0, 8), (0, 16), (8, 0), (16, 0), (1, 8), (2, 8), (4, 8), (8, 8), (1, 4), (1, 5), (4, 4)]
PROBE_BLOCKS, PROBE_ITERS, PROBE_THREADS = 2048, 32768, 256


def measure_issue_rates():
    """Lane operations per second of fp32 FMA and of the exp2 transcendental
    on this GPU, each alone and mixed (2048 blocks of 256 threads, 8 waves per
    SIMD, independent chains, no memory traffic). Returns a dict with the two
    peaks (lane-ops/s and per CU per measured clock) and, for every mix, the
    measured time against the no-overlap sum and the full-overlap max of the
    pure rates."""
    import ctypes
    from selective_state_space_ss_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.ssprobe_issue.restype = ctypes.c_int
    lib.ssprobe_issue.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)] * 2
    lanes = PROBE_BLOCKS * PROBE_THREADS * PROBE_ITERS
    runs = {}
    for ne, nf in PROBE_MIXES:
        ms, mhz = ctypes.c_double(), ctypes.c_double()
        rc = lib.ssprobe_issue(ne, nf, PROBE_ITERS, PROBE_BLOCKS, ctypes.byref(ms), ctypes.byref(mhz))
        if rc != 0:
            raise RuntimeError(f"ssprobe_issue({ne}, {nf}) returned {rc}")
        runs[(ne, nf)] = (ms.value * 1e-3, mhz.value)
        print(f"probe exp2 x{ne} fma x{nf}: {ms.value:.3f} ms, clock {mhz.value:.0f} MHz", file=sys.stderr, flush=True)
    fma_rate = max(lanes * nf / t for (ne, nf), (t, _) in runs.items() if ne == 0)
    exp_rate = max(lanes * ne / t for (ne, nf), (t, _) in runs.items() if nf == 0)
    clocks = sorted(m for _, m in runs.values() if m > 0)
    mhz = clocks[len(clocks) // 2] if clocks else 0.0
    cus = 256
    per_clk = (lambda r: r / (cus * mhz * 1e6)) if mhz else (lambda r: None)
    mixes = []
    for (ne, nf), (t, m) in runs.items():
        if ne and nf:
            te, tf = lanes * ne / exp_rate, lanes * nf / fma_rate
            mixes.append({"exp2_per_iter": ne, "fma_per_iter": nf, "s": t, "no_overlap_s": te + tf,
                          "full_overlap_s": max(te, tf), "measured_over_no_overlap": round(t / (te + tf), 4)})
    # dependent chains at 1 and 2 waves per SIMD (256 and 512 blocks of 4
    # waves): how many independent chains a wave needs to keep its SIMD busy
    chains = []
    for blocks in (256, 512):
        for ne, nf in ((0, 1), (0, 2), (0, 4), (0, 8), (1, 0), (2, 0), (4, 0), (8, 0)):
            cms, cmhz = ctypes.c_double(), ctypes.c_double()
            iters = PROBE_ITERS // 4
            if lib.ssprobe_issue(ne, nf, iters, blocks, ctypes.byref(cms), ctypes.byref(cmhz)) != 0:
                raise RuntimeError(f"ssprobe_issue({ne}, {nf}) at {blocks} blocks failed")
            waves_per_simd = blocks * PROBE_THREADS // 64 // (4 * 256)
            kclk = cms.value * 1e-3 * cmhz.value * 1e6
            per_instr = kclk / (iters * (ne + nf) * waves_per_simd)   # SIMD clocks per wave instruction
            chains.append({"waves_per_simd": waves_per_simd, "exp2_chains": ne, "fma_chains": nf,
                           "simd_clocks_per_instruction": round(per_instr, 2)})
            print(f"chains exp2 x{ne} fma x{nf} at {waves_per_simd} waves/SIMD: {per_instr:.2f} clocks/instr",
                  file=sys.stderr, flush=True)
    return {
        "probe": "libssprobe.so ssprobe_issue: %d blocks x %d threads x %d iterations per kernel"
                 % (PROBE_BLOCKS, PROBE_THREADS, PROBE_ITERS),
        "dependent_chains": chains,
        "fma_lane_ops_per_s": fma_rate,
        "exp2_lane_ops_per_s": exp_rate,
        "clock_mhz_measured": mhz,
        "fma_lane_ops_per_cu_clk": per_clk(fma_rate),
        "exp2_lane_ops_per_cu_clk": per_clk(exp_rate),
        "exp2_cost_in_fma_slots": fma_rate / exp_rate,
        "mixes": mixes,
    }


SCAN_SOURCES = ("scan_fwd.hip", "scan_chunked.h", "ss_device.h", "ss_launch.h")


def kernel_source_digest() -> str:
    """Digest of the sources and compiler flags the prompt-scan kernel is
    built from: a traffic figure is reported only while it matches (the
    kernel has not changed since the counters were taken)."""
    import hashlib
    from selective_state_space_ss_amd.build import HIPCC_FLAGS, SOURCE_FLAGS
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_ss_amd", "csrc")
    for name in SCAN_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    flags = [f for f in HIPCC_FLAGS if not f.startswith("/")] + SOURCE_FLAGS.get("scan_fwd.hip", [])
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def _read_counter(dirname, counter):
    """Per-dispatch values of one counter from a rocprofv3 CSV directory:
    {kernel name: [values in dispatch order]}."""
    import csv
    import glob
    vals = {}
    for f in sorted(glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)):
        rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def summarize_traffic(fetch_dir, write_dir):
    """HBM bytes per scan launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    of the scan, each scaled by what the same counter reads for the 256 MiB
    copy (which moves exactly COPY_BYTES each way)."""
    out = {"kernel_source_digest": kernel_source_digest(), "copy_bytes": COPY_BYTES}
    for label, d, ctr in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        v = _read_counter(d, ctr)
        copy = [x for k, xs in v.items() if "scan_fwd" not in k and "state_update" not in k for x in xs]
        scan = [x for k, xs in v.items() if "scan_fwd" in k for x in xs]
        assert copy and scan, f"{ctr}: copy or scan dispatch missing in {d}"
        factor = COPY_BYTES / (max(copy) * 1024.0)   # the copy is the largest non-scan dispatch
        out[f"{label}_kib_per_scan"] = sum(scan) / len(scan)
        out[f"{label}_kib_copy"] = max(copy)
        out[f"{label}_scale"] = factor
        out[f"{label}_bytes_per_scan"] = sum(scan) / len(scan) * 1024.0 * factor
    out["traffic_bytes_per_scan"] = out["fetch_bytes_per_scan"] + out["write_bytes_per_scan"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_trace(kt_dir):
    """One row per (kernel, grid, block) of a rocprofv3 kernel-trace CSV: calls,
    average / median / min / max duration. Launches of one kernel instance at
    different shapes (say two workloads sharing a template instance) get rows
    of their own."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True)
    assert files, f"no *kernel_trace.csv under {kt_dir}"
    groups = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                   int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in groups.values())
    print("| kernel | grid (work-items) | block | calls | average ns | median ns | min ns | max ns | share |")
    print("|---|---|---|---|---|---|---|---|---|")
    for (name, grid, block), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short = name.split("(")[0].replace("void ", "") if "(anonymous namespace)" not in name else \
            name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
        print(f"| `{short}` | {grid} | {block} | {len(d)} | {sum(d) / len(d):.0f} | {statistics.median(d):.0f} | "
              f"{min(d)} | {max(d)} | {100.0 * sum(d) / total:.2f} % |")
    step = step_launches(files)
    if step:
        d = sorted(step)
        print()
        print(f"In the bench step: {len(d)} decode launches that start after a Mamba-2.8B prompt scan ends (the "
              f"step's order; the two-stream extra's overlapping ones excluded): mean {sum(d) / len(d):.0f} ns, "
              f"median {statistics.median(d):.0f} ns, p10 {d[len(d) // 10]} ns, p90 {d[9 * len(d) // 10]} ns.")


STEP_SCAN = "scan_fwd_kernel<ss::bf16_t, 16, 8, 16, true, false, 0, 0, 16>"
STEP_DECODE = "state_update_kernel<ss::bf16_t, 1, true, true>"


def step_launches(files) -> list:
    """Durations (ns) of the decode launches that directly follow a launch of
    the Mamba-2.8B prompt scan in start order and begin after it has ended:
    the decode of the bench step, cold after the scan, as the kernel itself
    ran (no HIP events around it)."""
    import csv
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    out = []
    for (s0, e0, n0), (s1, e1, n1) in zip(rows, rows[1:]):
        if STEP_SCAN in n0 and STEP_DECODE in n1 and s1 >= e0:
            out.append(e1 - s1)
    return out


def recorded_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t["traffic_bytes_per_scan"]


EXTRA_WARM_S = 0.3   # each extra kernel runs this long before it is timed


# timed steps whose two kernels record their own dispatch events (the rest
# run untimed, so that the instrumentation adds little to the step's wall time)
KERNEL_SAMPLE = 4


def time_launches(f, stream, reps: int) -> float:
    """Average microseconds per call of f (HIP events on `stream`), after
    EXTRA_WARM_S seconds of untimed calls (clocks and caches settle)."""
    import torch
    t0 = time.time()
    while True:
        f()
        torch.cuda.synchronize()
        if time.time() - t0 >= EXTRA_WARM_S:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        f()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def measure_states(ss, P, w, scan_bytes: int, stream, reps: int = 20):
    """ss_scan_fwd_states at the prompt workload's shape, outside the timed
    step: every token's state ([batch, channels, N, seq] fp32, 4 N bytes per
    channel-token more to write: bound by HBM) and one selected step (the
    plain scan's cost). Per-launch HIP-event averages after a warm-up."""
    import torch
    ct = w.batch * w.channels * w.seqlen
    res = {}
    for label, ts, extra in (("every_token", None, ct * w.state_dim * 4),
                             ("one_step", w.seqlen // 2, w.batch * w.channels * w.state_dim * 4)):
        shape = ((w.batch, w.channels, w.state_dim, w.seqlen) if ts is None
                 else (w.batch, w.channels, w.state_dim))
        states = torch.empty(shape, dtype=torch.float32, device=P["x"].device)
        y = torch.empty_like(P["x"])
        h = torch.empty(w.batch, w.channels, w.state_dim, dtype=torch.float32, device=P["x"].device)
        f = lambda: ss.ss_scan_fwd_states(P["x"], P["dt"], P["A"], P["B"], P["C"], D=P["D"], z=P["z"],
                                          dt_bias=P["dt_bias"], h0=P["h0"], time_step=ts, y=y, h_last=h,
                                          states=states)
        us = time_launches(f, stream, reps)
        nbytes = scan_bytes + extra
        res[label] = {"us": round(us, 2), "algorithmic_bytes": nbytes, "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del states
    return res


GATED_SHAPE = (640, 2048, 128, 64)   # batch x heads, seq, dk, dv


def gated_work(batch, L, dk, dv, es):
    """Algorithmic bytes (q, k, v, y in the I/O dtype, gamma and the fp32
    final state) and matrix-core flops of one scalar-gated scan launch. The
    flops are those of the chunked form over 16-token chunks, per token:
    q.k over the chunk (2 * 16 dk), the weighted sum of v (2 * 16 dv), q^T S
    (2 dk dv) and the state update (2 dk dv)."""
    tok = batch * L
    nbytes = tok * (2 * dk + 2 * dv) * es + tok * 4 + batch * dk * dv * 4
    flops = tok * (32.0 * dk + 32.0 * dv + 4.0 * dk * dv)
    return nbytes, flops


def measure_gated(ss, stream, reps: int = 20):
    """ss_gated_scan at batch x heads 640, seq 2048, dk 128, dv 64, bf16 I/O,
    fp32 final state (a Mamba-2 2.7B-shaped layer at batch 8: 80 heads of
    width 64, state 128). Per-launch HIP-event average after a warm-up.
    Reported against HBM and against what the bf16 matrix cores execute
    (split terms included); the model's flops (the chunked form as fp32
    work) are given as a rate only: the fp32-accurate products run on the
    bf16 matrix cores, so no fp32 peak applies to them."""
    import torch
    from selective_state_space_ss_amd.workloads import make_gated_case
    batch, L, dk, dv = GATED_SHAPE
    c = make_gated_case(1010, batch, L, dk, dv, "bf16", device="cuda")
    y = torch.empty(batch, L, dv, dtype=torch.bfloat16, device="cuda")
    fs = torch.empty(batch, dk, dv, dtype=torch.float32, device="cuda")
    f = lambda: ss.ss_gated_scan(c["q"], c["k"], c["v"], c["gamma"], y=y, final_state=fs)
    us = time_launches(f, stream, reps)
    nbytes, flops = gated_work(batch, L, dk, dv, 2)
    tf = flops / (us * 1e-6) / 1e12
    # executed on the bf16 matrix cores (bf16 I/O): per 16-token chunk and
    # 16 value columns, q k^T 16 x 16 x dk, the three split terms of M v
    # (16 x 16 x 16 each), of q S (16 x 16 x dk each) and of the state update
    # (dk x 16 x 16 each)
    chunks = (L + 15) // 16
    per = 2 * 16 * 16 * dk + 3 * 2 * 16 * 16 * 16 + 3 * 2 * 16 * 16 * dk + 3 * 2 * dk * 16 * 16
    executed = float(batch * ((dv + 15) // 16) * chunks * per)
    te = executed / (us * 1e-6) / 1e12
    return {"shape": {"batch_x_heads": batch, "seq": L, "dk": dk, "dv": dv, "io": "bf16", "state": "f32"},
            "us": round(us, 2), "algorithmic_bytes": nbytes, "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "model_flops": flops, "model_TFLOP_s": round(tf, 2),
            "bf16_mfma_flops_executed": executed, "bf16_mfma_TFLOP_s": round(te, 2),
            "bf16_mfma_frac": round(te / PEAK_BF16_TFLOPS, 4),
            # the roofline: the larger of the HBM time and the matrix cores'
            # time for the work they execute, over the kernel time
            "frac": round(max(nbytes / (PEAK_HBM_GBS * 1e9), executed / (PEAK_BF16_TFLOPS * 1e12)) / (us * 1e-6), 4),
            "bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) >= executed / (PEAK_BF16_TFLOPS * 1e12) else "mfma"}


ATTN_SHAPE = (1, 1536, 16, 256)   # batch, channels, state_dim, seq


def measure_attention(ss, stream, reps: int = 20):
    """ss_effective_attention at batch 1, channels 1536, state_dim 16, seq 256,
    bf16 inputs (a Mamba-130M-shaped layer on a short sequence), summed over
    the state coordinate, fp32 output. Algorithmic bytes: the output (4 L^2
    per channel) plus dt, B and C once; the row loop's work is 2 N VALU
    operations per lower-triangle element."""
    import torch
    from selective_state_space_ss_amd.workloads import make_case
    batch, channels, N, L = ATTN_SHAPE
    inp = {k: (None if v is None else v.cuda())
           for k, v in make_case(1020, batch, channels, N, L, "bf16", gate=False, h0=False).items()}
    out = torch.empty(batch, channels, L, L, dtype=torch.float32, device="cuda")
    f = lambda: ss.ss_effective_attention(inp["dt"], inp["A"], inp["B"], inp["C"], inp["dt_bias"], out=out)
    us = time_launches(f, stream, reps)
    nbytes = batch * channels * L * L * 4 + batch * channels * L * 2 + 2 * batch * N * L * 2 + channels * (N + 1) * 4
    return {"shape": {"batch": batch, "channels": channels, "state_dim": N, "seq": L, "io": "bf16", "out": "f32"},
            "us": round(us, 2), "algorithmic_bytes": nbytes, "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


PRODUCER_SHAPE = (8, 5120, 2048, 4, 160)   # batch, channels, seq, conv width, dt rank


def measure_fused_conv(ss, P, w, stream, rates, reps: int = 20):
    """ss_scan_fwd_conv (the conv1d + SiLU of width 4 fused into the scan, x
    never written) at the Mamba-2.8B prompt shape, next to the two-kernel
    chain it replaces: ss_conv1d_silu, then ss_scan_fwd on the written x.
    Algorithmic bytes of the fused call: the scan's with x_pre in place of x,
    plus the conv weights; of the chain: the conv's (read x_pre, write x) plus
    the scan's."""
    import torch
    from selective_state_space_ss_amd.workloads import algorithmic_bytes, make_producer_case
    width = 4
    c = make_producer_case(1030, w.batch, w.channels, w.seqlen, width, 1, "bf16", device="cuda")
    y = torch.empty_like(P["x"])
    h = torch.empty(w.batch, w.channels, w.state_dim, dtype=torch.float32, device="cuda")
    x = torch.empty_like(P["x"])
    fused = lambda: ss.ss_scan_fwd_conv(c["x_pre"], P["dt"], P["A"], P["B"], P["C"], c["conv_w"], c["conv_b"],
                                        D=P["D"], z=P["z"], dt_bias=P["dt_bias"], h0=P["h0"], y=y, h_last=h)

    def chain():
        ss.ss_conv1d_silu(c["x_pre"], c["conv_w"], c["conv_b"], out=x)
        ss.ss_scan_fwd(x, P["dt"], P["A"], P["B"], P["C"], D=P["D"], z=P["z"], dt_bias=P["dt_bias"], h0=P["h0"],
                       y=y, h_last=h)
    us_f = time_launches(fused, stream, reps)
    us_c = time_launches(chain, stream, reps)
    scan_bytes = algorithmic_bytes(w)
    conv_extra = w.channels * (width + 1) * 4
    r = scan_roofline(w, us_f, rates)
    r["algorithmic_bytes"] = scan_bytes + conv_extra
    r["GB_s"] = round((scan_bytes + conv_extra) / (us_f * 1e-6) / 1e9, 1)
    return {"shape": {"batch": w.batch, "channels": w.channels, "state_dim": w.state_dim, "seq": w.seqlen,
                      "width": width, "io": "bf16"},
            "fused": r,
            "conv1d_silu_then_scan_us": round(us_c, 2),
            "chain_algorithmic_bytes": scan_bytes + conv_extra + 2 * w.batch * w.channels * w.seqlen * 2,
            "speedup": round(us_c / us_f, 3)}


def measure_producers(ss, stream, reps: int = 20):
    """The scan's input side at the Mamba-2.8B layer shape (batch 8, channels
    5120, seq 2048, bf16): ss_conv1d_silu (width 4; bytes: read x_pre, write
    x) and ss_dt_proj (rank 160, with bias and softplus, and without them;
    bytes: read w_dt and delta, write dt; flops 2 R per output). Per-launch
    HIP-event averages."""
    import torch
    from selective_state_space_ss_amd.workloads import make_producer_case
    batch, channels, L, W, R = PRODUCER_SHAPE
    c = make_producer_case(1030, batch, channels, L, W, R, "bf16", device="cuda")
    x = torch.empty_like(c["x_pre"])
    dt = torch.empty(batch, channels, L, dtype=torch.bfloat16, device="cuda")
    calls = {
        "ss_conv1d_silu": (lambda: ss.ss_conv1d_silu(c["x_pre"], c["conv_w"], c["conv_b"], out=x),
                           2 * batch * channels * L * 2 + channels * (W + 1) * 4, 0.0),
        "ss_dt_proj": (lambda: ss.ss_dt_proj(c["w_dt"], c["delta"], c["dt_bias"], apply_softplus=True, out=dt),
                       batch * channels * L * 2 + batch * L * R * 2 + channels * R * 2 + channels * 4,
                       2.0 * batch * channels * L * R),
        # the plain product, as a Mamba layer feeds its scan (which then
        # applies softplus(dt + dt_bias) itself)
        "ss_dt_proj_raw": (lambda: ss.ss_dt_proj(c["w_dt"], c["delta"], None, apply_softplus=False, out=dt),
                           batch * channels * L * 2 + batch * L * R * 2 + channels * R * 2,
                           2.0 * batch * channels * L * R),
    }
    res = {"shape": {"batch": batch, "channels": channels, "seq": L, "width": W, "rank": R, "io": "bf16"}}
    for name, (f, nbytes, flops) in calls.items():
        us = time_launches(f, stream, reps)
        r = {"us": round(us, 2), "algorithmic_bytes": nbytes, "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
             "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        if flops:
            r["TFLOP_s"] = round(flops / (us * 1e-6) / 1e12, 2)
        res[name] = r
    return res


FLUSH_BYTES = 1 << 30
PCT_REPS = 50   # launches behind each configuration's p10 / median / p90


def _event_pairs(n: int, stream):
    """n pairs of timing events, each recorded once (torch creates an event at
    its first record) so that its raw handle exists."""
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in pairs:
        e0.record(stream)
        e1.record(stream)
    return pairs


def _timed_launches(f, stream, reps: int, before=None, kernel_timed: bool = False):
    """Per-launch microseconds of `reps` launches of f, each with an event
    pair around the call; with kernel_timed, f(kev) also passes a second pair
    (raw handles) that the kernel's own dispatch records, and those durations
    are returned first. Returns (kernel or call times, call times)."""
    import torch
    call = _event_pairs(reps, stream)
    kern = _event_pairs(reps, stream) if kernel_timed else None
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(call):
        if before is not None:
            before()
        e0.record(stream)
        if kernel_timed:
            f((kern[i][0].cuda_event, kern[i][1].cuda_event))
        else:
            f()
        e1.record(stream)
    torch.cuda.synchronize()
    call_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in call]
    if kernel_timed:
        return [k0.elapsed_time(k1) * 1e3 for k0, k1 in kern], call_us
    return call_us, call_us


def time_cold(f, stream, reps: int, flush, kernel_timed: bool = False) -> float:
    """Average microseconds of f when the caches hold none of its data: before
    each timed launch a read of the 1 GiB `flush` tensor (a sum) streams
    through the L2s and the 256 MB last-level cache, leaving them full of
    clean lines (outside the timed region; HIP events on `stream` bracket f
    alone, and with kernel_timed the kernel's own dispatch records a second
    pair: f(kev)). A read rather than a fill: written lines would still be
    draining to HBM while f runs."""
    import torch
    t0 = time.time()
    while time.time() - t0 < EXTRA_WARM_S:
        f(None) if kernel_timed else f()
        torch.cuda.synchronize()
    each, call = _timed_launches(f, stream, reps, before=lambda: flush.sum(), kernel_timed=kernel_timed)
    LAST_EACH[:] = each
    LAST_CALL[:] = call
    return sum(each) / reps


# per-launch microseconds of the last time_cold / time_each call (the
# kernel's own duration where it was timed so, else the call's), and of the
# calls themselves
LAST_EACH: list = []
LAST_CALL: list = []


def time_each(f, stream, reps: int, kernel_timed: bool = False) -> list:
    """Microseconds of each of `reps` back-to-back launches of f (an event pair
    around every launch, and with kernel_timed the pair the kernel's dispatch
    records; the caches keep what the previous launch left)."""
    each, call = _timed_launches(f, stream, reps, kernel_timed=kernel_timed)
    LAST_CALL[:] = call
    return each


def percentiles(each: list) -> dict:
    """p10 / median / p90 of per-launch times (nearest rank)."""
    v = sorted(each)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"p10_us": round(pick(0.1), 2), "median_us": round(pick(0.5), 2), "p90_us": round(pick(0.9), 2)}


def measure_workloads(ss, stream, rates, P, wp, Dd, wd, reps: int = 20):
    """Every configuration the scan is specified on, each as its own launch
    (the library's default kernel choice; no tuning override): the tiny fp32
    case, the Mamba-130M layer, the packed-sequence scan with resets, the
    Mamba-2.8B layer (the step's scan) and the decode step. Each is timed
    back to back after a warm-up (warm: the inputs of a small case stay in
    the 256 MB last-level cache between launches) and with the caches flushed
    before every launch (cold). Each also carries p10 / median / p90 of 50
    launches timed one by one: the kernel's duration, from the event pair its
    own dispatch records, and as `median_call_us` the median of an event pair
    around each call (the dispatch gap included). Cold `us` is the mean
    kernel duration of those 50 launches; warm `us` is the average over 20
    back-to-back launches between two events."""
    import torch
    from selective_state_space_ss_amd.workloads import WORKLOADS, make_inputs
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    res = {}
    for name in ("tiny_fp32", "mamba130m", "packed_reset", "mamba2p8b"):
        w = WORKLOADS[name]
        if name == "mamba2p8b":
            d = P
        else:
            d = {k: (None if v is None else v.cuda()) for k, v in make_inputs(w).items()}
        y = torch.empty_like(d["x"])
        h = torch.empty(w.batch, w.channels, w.state_dim, dtype=torch.float32, device="cuda")
        f = lambda kev=None, d=d, y=y, h=h: ss.ss_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"],
                                                           z=d["z"], dt_bias=d["dt_bias"], h0=d["h0"],
                                                           reset=d["reset"], y=y, h_last=h, timing_events=kev)
        warm = scan_roofline(w, time_launches(f, stream, reps), rates)
        warm.update(percentiles(time_each(f, stream, PCT_REPS, kernel_timed=True)))
        warm["median_call_us"] = percentiles(LAST_CALL)["median_us"]
        cold = scan_roofline(w, time_cold(f, stream, PCT_REPS, flush, kernel_timed=True), rates)
        cold.update(percentiles(LAST_EACH))
        cold["median_call_us"] = percentiles(LAST_CALL)["median_us"]
        res[name] = {"shape": {"batch": w.batch, "channels": w.channels, "state_dim": w.state_dim,
                               "seq": w.seqlen, "io": w.io_dtype, "gate": w.gate, "h0": w.h0 is not None,
                               "reset": w.reset_mean_doc is not None},
                     "warm": warm, "cold": cold}
        del d, y, h
    state = Dd["state"].clone()
    yd = torch.empty_like(Dd["x"])
    fd = lambda kev=None: ss.ss_state_update(state, Dd["x"], Dd["dt"], Dd["A"], Dd["B"], Dd["C"], D=Dd["D"],
                                             z=Dd["z"], dt_bias=Dd["dt_bias"], y=yd, timing_events=kev)
    res["decode"] = {"shape": {"batch": wd.batch, "channels": wd.channels, "state_dim": wd.state_dim,
                               "io": wd.io_dtype, "gate": wd.gate},
                     "warm": decode_roofline(wd, time_launches(fd, stream, reps)),
                     "cold": decode_roofline(wd, time_cold(fd, stream, PCT_REPS, flush, kernel_timed=True))}
    res["decode"]["cold"].update(percentiles(LAST_EACH))
    res["decode"]["cold"]["median_call_us"] = percentiles(LAST_CALL)["median_us"]
    res["decode"]["warm"].update(percentiles(time_each(fd, stream, PCT_REPS, kernel_timed=True)))
    res["decode"]["warm"]["median_call_us"] = percentiles(LAST_CALL)["median_us"]
    # The achievable rate of the decode's access pattern on this machine: an
    # in-place read-modify-write of a tensor of the state's size (torch's own
    # elementwise kernel), timed the same two ways.
    buf = torch.randn_like(state)
    fc = lambda: buf.mul_(1.0000001)
    moved = 2 * buf.numel() * buf.element_size()
    ceil = {"bytes_moved": moved}
    for kind, us in (("warm", time_launches(fc, stream, reps)), ("cold", time_cold(fc, stream, reps, flush))):
        gbs = moved / (us * 1e-6) / 1e9
        ceil[kind] = {"us": round(us, 2), "GB_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        dec = res["decode"][kind]
        dec["frac_of_inplace_rw"] = round(dec["GB_s"] / gbs, 4)
    res["decode"]["inplace_rw_same_size"] = ceil
    del flush, state, buf
    return res


def probe_live():
    """The two pure issue-rate kernels, run in this process: a cross-check of
    the committed rates on the box the bench runs on."""
    import ctypes
    from selective_state_space_ss_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.ssprobe_issue.restype = ctypes.c_int
    lib.ssprobe_issue.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)] * 2
    lanes = PROBE_BLOCKS * PROBE_THREADS * PROBE_ITERS
    out = {}
    for key, ne, nf in (("fma_lane_ops_per_s", 0, 16), ("exp2_lane_ops_per_s", 16, 0)):
        ms, mhz = ctypes.c_double(), ctypes.c_double()
        if lib.ssprobe_issue(ne, nf, PROBE_ITERS, PROBE_BLOCKS, ctypes.byref(ms), ctypes.byref(mhz)) != 0:
            return None
        out[key] = lanes * (ne + nf) / (ms.value * 1e-3)
        out["clock_mhz"] = round(mhz.value, 1)
    return out


COPY_CEILING_BYTES = 1 << 30   # each way


def measure_two_streams(ss, P, Dd, y, h_last, yd, state, stream, steps: int = 50):
    """The bench step with its two independent halves on two streams: the
    prompt scan (VALU-bound) on the bench stream and the decode update
    (HBM-bound, its own batch) on a second stream of default priority, so the
    decode's memory traffic can run under the scan's arithmetic. Steps stay
    ordered per stream (the decode's state is updated in place). Reports the
    time per step next to the sequential step's figure."""
    import torch
    side = torch.cuda.Stream()

    def scan():
        ss.ss_scan_fwd(P["x"], P["dt"], P["A"], P["B"], P["C"], D=P["D"], z=P["z"], dt_bias=P["dt_bias"],
                       h0=P["h0"], y=y, h_last=h_last, stream=stream)

    def decode():
        ss.ss_state_update(state, Dd["x"], Dd["dt"], Dd["A"], Dd["B"], Dd["C"], D=Dd["D"], z=Dd["z"],
                           dt_bias=Dd["dt_bias"], y=yd, stream=side)

    def run(n):
        side.wait_stream(stream)
        for _ in range(n):
            scan()
            decode()
        stream.wait_stream(side)

    t0 = time.time()
    while time.time() - t0 < EXTRA_WARM_S:
        run(5)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    run(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    return {"steps": steps, "us_per_step": round(e0.elapsed_time(e1) / steps * 1e3, 2)}


def measure_copy(stream, reps: int = 20):
    """A plain device-to-device copy of 1 GiB (read 1 GiB, write 1 GiB), the
    achievable streaming rate on this machine next to the 8 TB/s peak."""
    import torch
    src = torch.empty(COPY_CEILING_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    us = time_launches(lambda: dst.copy_(src), stream, reps)
    moved = 2 * COPY_CEILING_BYTES
    del src, dst
    return {"bytes_moved": moved, "us": round(us, 2), "GB_s": round(moved / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(moved / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def cpu_baseline(inp, w, budget_s: float):
    """The oracle over whole (b, c) rows of the prompt workload, row blocks of
    every batch row in turn, until the time budget is spent."""
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))  # a one-GPU share of the host
    rows_per_call = max(threads * 4, 32)
    done_rows = 0
    t_total = 0.0
    b = 0
    c0 = 0
    while t_total < budget_s and done_rows < w.batch * w.channels:
        cs = slice(c0, min(c0 + rows_per_call, w.channels))
        f64 = lambda t, bb=b: t[bb:bb + 1, cs].double().numpy()
        args = (f64(inp["x"]), f64(inp["dt"]), inp["A"][cs].double().numpy(), inp["B"][b:b + 1].double().numpy(),
                inp["C"][b:b + 1].double().numpy())
        kw = dict(D=inp["D"][cs].double().numpy(), z=f64(inp["z"]) if inp["z"] is not None else None,
                  dt_bias=inp["dt_bias"][cs].double().numpy(),
                  h0=f64(inp["h0"]) if inp["h0"] is not None else None, threads=threads)
        t0 = time.perf_counter()
        oracle.scan(*args, **kw)
        t_total += time.perf_counter() - t0
        done_rows += cs.stop - cs.start
        c0 = cs.stop
        if c0 >= w.channels:
            c0 = 0
            b += 1
    ct = done_rows * w.seqlen
    from selective_state_space_ss_amd.workloads import algorithmic_bytes
    bytes_per_ct = algorithmic_bytes(w) / (w.batch * w.channels * w.seqlen)
    return {
        "value": round(ct * bytes_per_ct / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done_rows} of {w.batch * w.channels} (batch, channel) rows of the {w.name} prompt scan "
                  f"({ct} channel-tokens, fp64 sequential token loop, {t_total:.1f} s wall)",
        "channel_tokens_per_s": round(ct / t_total, 1),
        "wall_s": round(t_total, 3),
        "host": host_cpu(),
    }


def host_cpu():
    """The host's CPU model and counts (the oracle's threads are capped at a
    one-GPU share of them)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_single_thread(names=("tiny_fp32", "mamba130m"), budget_s: float = 1.5):
    """The oracle on one thread over whole (b, c) rows of small prompt
    workloads (the tiny case whole; others until the budget is spent)."""
    import oracle
    from selective_state_space_ss_amd.workloads import WORKLOADS, algorithmic_bytes, make_inputs
    out = {}
    for name in names:
        w = WORKLOADS[name]
        rows = max(1, min(w.channels, 8))  # channels per call
        inp = make_inputs(w, batch=1)
        t_total, done = 0.0, 0
        c0 = 0
        while done < w.channels and (t_total < budget_s or done == 0):
            cs = slice(c0, min(c0 + rows, w.channels))
            f64 = lambda t: t[:, cs].double().numpy()
            kw = dict(D=inp["D"][cs].double().numpy(), z=f64(inp["z"]) if inp["z"] is not None else None,
                      dt_bias=inp["dt_bias"][cs].double().numpy(),
                      h0=f64(inp["h0"]) if inp["h0"] is not None else None, threads=1)
            t0 = time.perf_counter()
            oracle.scan(f64(inp["x"]), f64(inp["dt"]), inp["A"][cs].double().numpy(), inp["B"].double().numpy(),
                        inp["C"].double().numpy(), **kw)
            t_total += time.perf_counter() - t0
            done += cs.stop - cs.start
            c0 = cs.stop
        ct = done * w.seqlen
        bytes_per_ct = algorithmic_bytes(w) / (w.batch * w.channels * w.seqlen)
        out[name] = {"rows": done, "channel_tokens": ct, "wall_s": round(t_total, 4),
                     "channel_tokens_per_s": round(ct / t_total, 1),
                     "GB_s": round(ct * bytes_per_ct / t_total / 1e9, 5)}
    return out


# LDS bank probe (libssprobe.so ssprobe_lds): (name, access bytes, write?,
# byte offset of each of the 64 lanes). The first launch warms up and is not
# a pattern.
LDS_PROBE_ITERS = 1000


def lds_patterns():
    L = range(64)
    pats = [
        ("read b128, lanes contiguous", 16, 0, [16 * l for l in L]),
        ("read b128, every lane one address", 16, 0, [0] * 64),
        ("read b128, lane stride 32 B", 16, 0, [32 * l for l in L]),
        ("read b128, lane stride 64 B", 16, 0, [64 * l for l in L]),
        ("read b128, lane stride 256 B", 16, 0, [256 * l for l in L]),
        ("read b128, 16 lanes contiguous, 4 rows alike", 16, 0, [16 * (l % 16) for l in L]),
        ("read b128, 16 lanes contiguous, rows 256 B apart", 16, 0, [16 * (l % 16) + 256 * (l // 16) for l in L]),
        ("read b128, scan B/C: lane stride 80 B, 4 rows alike", 16, 0, [80 * (l % 16) for l in L]),
        ("read b128, lane stride 64 B, 4 rows alike", 16, 0, [64 * (l % 16) for l in L]),
        ("read b128, dt_proj delta: lane stride 336 B, rows +16 B", 16, 0,
         [336 * (l % 16) + 16 * (l // 16) for l in L]),
        ("read b128, lane stride 336 B, 4 rows alike", 16, 0, [336 * (l % 16) for l in L]),
        ("read b128, lane stride 80 B, rows +16 B", 16, 0, [80 * (l % 16) + 16 * (l // 16) for l in L]),
        ("read b64, lanes contiguous", 8, 0, [8 * l for l in L]),
        ("read b64, lane stride 16 B", 8, 0, [16 * l for l in L]),
        ("read b32, lanes contiguous", 4, 0, [4 * l for l in L]),
        ("read b32, lane stride 8 B", 4, 0, [8 * l for l in L]),
        ("write b128, lanes contiguous", 16, 1, [16 * l for l in L]),
        ("write b128, lane stride 32 B", 16, 1, [32 * l for l in L]),
        ("write b128, scan B/C staging (bf16, 16 tokens per lane)", 16, 1,
         [4 * (((l % 32) // 2) * 20 + 8 * (l % 2)) + 4 * 320 * (l // 32) for l in L]),
        ("write b64, lanes contiguous", 8, 1, [8 * l for l in L]),
        ("write b64, lane stride 16 B", 8, 1, [16 * l for l in L]),
        ("write b32, lanes contiguous", 4, 1, [4 * l for l in L]),
    ]
    for name, width, _, offs in pats:
        assert len(offs) == 64 and all(0 <= o <= 65536 - 16 and o % width == 0 for o in offs), name
    return pats


def probe_lds():
    import ctypes
    import torch
    from selective_state_space_ss_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.ssprobe_lds.restype = ctypes.c_int
    lib.ssprobe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
    pats = lds_patterns()
    out = torch.empty(64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    offs = [torch.tensor(o, dtype=torch.int32, device="cuda") for _, _, _, o in pats]
    for k, (name, width, write, _) in enumerate([pats[0]] + pats):
        t = offs[max(k - 1, 0)]
        if lib.ssprobe_lds(t.data_ptr(), width, LDS_PROBE_ITERS, write, out.data_ptr(), stream) != 0:
            raise RuntimeError(f"ssprobe_lds failed on {name}")
    torch.cuda.synchronize()
    print(json.dumps([p[0] for p in pats]), flush=True)


def summarize_lds(pmc_dir: str):
    import csv
    import glob
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if "lds_probe_kernel" not in r["Kernel_Name"]:
                continue
            d = per.setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[1:]  # the first launch is the warm-up
    pats = lds_patterns()
    if len(ids) != len(pats):
        raise SystemExit(f"expected {len(pats)} probe launches after the warm-up, found {len(ids)}")
    print("| pattern | bytes per lane | conflict cycles per instruction |")
    print("|---|---|---|")
    for (name, width, _, _), i in zip(pats, ids):
        c = per[i]
        print(f"| {name} | {width} | {c.get('SQ_LDS_BANK_CONFLICT', 0.0) / LDS_PROBE_ITERS:.2f} |")


def summarize_counters(pmc_dirs, kernel: str):
    """Counter table of one kernel over rocprofv3 --pmc passes: per dispatch
    and counter, the sum over the counter's instances (XCDs, SEs, ...); then,
    per counter, the median over the selected dispatches."""
    import csv
    import glob
    import statistics
    per = {}  # counter -> {(pass, dispatch): value}
    names = set()
    for d in pmc_dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                if kernel not in r["Kernel_Name"]:
                    continue
                names.add(r["Kernel_Name"])
                key = (f, int(r["Dispatch_Id"]))
                c = per.setdefault(r["Counter_Name"], {})
                c[key] = c.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r} in {pmc_dirs}")
    print("Kernel(s): " + "; ".join(f"`{n}`" for n in sorted(names)))
    print()
    print("| counter | value | dispatches |")
    print("|---|---|---|")
    for name in sorted(per):
        v = list(per[name].values())
        print(f"| {name} | {statistics.median(v):,.0f} | {len(v)} |")


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.counter_kernel)
        return
    if args.summarize_lds:
        summarize_lds(args.summarize_lds)
        return
    if args.probe_lds:
        probe_lds()
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.probe_issue:
        r = measure_issue_rates()
        with open(args.probe_issue, "w") as f:
            json.dump(r, f, indent=1)
        print(json.dumps(r), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the scan would shard over "
              "batch rows and channels, which exchange nothing, so one GPU's share is the measured case)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import selective_state_space_ss_amd as ss
    from selective_state_space_ss_amd.workloads import WORKLOADS, algorithmic_bytes, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    ss.load_library()
    wp, wd = WORKLOADS["mamba2p8b"], WORKLOADS["decode"]
    cpu_p = make_inputs(wp)
    cpu_d = make_inputs(wd)
    P = {k: (None if v is None else v.to(dev)) for k, v in cpu_p.items()}
    Dd = {k: (None if v is None else v.to(dev)) for k, v in cpu_d.items()}
    y = torch.empty_like(P["x"])
    h_last = torch.empty(wp.batch, wp.channels, wp.state_dim, dtype=torch.float32, device=dev)
    yd = torch.empty_like(Dd["x"])
    state = Dd["state"]
    stream = torch.cuda.current_stream(dev)

    def step(ev=None, kev=None):
        # ev: three events recorded on the stream around the two calls (a
        # call's time then includes the dispatch gap before its kernel); kev:
        # raw handles of two event pairs that the kernels' own dispatches
        # record (ss_scan_fwd_timed / ss_state_update_timed: the kernel's
        # duration, what a kernel trace reports)
        if ev is not None:
            ev[0].record(stream)
        ss.ss_scan_fwd(P["x"], P["dt"], P["A"], P["B"], P["C"], D=P["D"], z=P["z"], dt_bias=P["dt_bias"],
                       h0=P["h0"], y=y, h_last=h_last, timing_events=None if kev is None else kev[0:2])
        if ev is not None:
            ev[1].record(stream)
        ss.ss_state_update(state, Dd["x"], Dd["dt"], Dd["A"], Dd["B"], Dd["C"], D=Dd["D"], z=Dd["z"],
                           dt_bias=Dd["dt_bias"], y=yd, timing_events=None if kev is None else kev[2:4])
        if ev is not None:
            ev[2].record(stream)

    if args.counter_pass:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        if args.counter_workload == "dt_proj":
            from selective_state_space_ss_amd.workloads import make_producer_case
            batch, channels, L, W, R = PRODUCER_SHAPE
            pc = make_producer_case(1030, batch, channels, L, W, R, "bf16", device="cuda")
            dt = torch.empty(batch, channels, L, dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                ss.ss_dt_proj(pc["w_dt"], pc["delta"], pc["dt_bias"], apply_softplus=True, out=dt)
        elif args.counter_workload == "gated":
            from selective_state_space_ss_amd.workloads import make_gated_case
            batch, L, dk, dv = GATED_SHAPE
            gc = make_gated_case(1010, batch, L, dk, dv, "bf16", device="cuda")
            gy = torch.empty(batch, L, dv, dtype=torch.bfloat16, device=dev)
            gs = torch.empty(batch, dk, dv, dtype=torch.float32, device=dev)
            for _ in range(3):
                ss.ss_gated_scan(gc["q"], gc["k"], gc["v"], gc["gamma"], y=gy, final_state=gs)
        elif args.counter_workload:
            c = {k: (None if v is None else v.to(dev)) for k, v in make_inputs(args.counter_workload).items()}
            for _ in range(3):
                ss.ss_scan_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"], dt_bias=c["dt_bias"],
                               h0=c["h0"], reset=c["reset"])
        else:
            for _ in range(3):
                step()
        torch.cuda.synchronize()
        print("counter pass done", flush=True)
        return
    # W untimed steps, then more untimed steps until the clocks have ramped
    # (a cold GPU runs the first few hundred microseconds of work slower)
    t_w = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    while time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w
    # The timed steps: each kernel's duration from the event pair its own
    # dispatch records, on every KERNEL_SAMPLE-th step (a launch that records
    # events adds about 5 us of wall time, 3 % of the step if every launch
    # did; measured on MI355X, 100 steps: 377.8 us plain, 388.4 us with every
    # launch timed so). torch creates an event at its first record, so each is
    # recorded once on the stream before its raw handle is taken.
    sampled = list(range(0, args.steps, KERNEL_SAMPLE))
    kevents = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in sampled]
    for ks in kevents:
        for e in ks:
            e.record(stream)
    handles = {i: [e.cuda_event for e in ks] for i, ks in zip(sampled, kevents)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(kev=handles.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scan_ms = sum(k[0].elapsed_time(k[1]) for k in kevents) / len(kevents)
    upd_ms = sum(k[2].elapsed_time(k[3]) for k in kevents) / len(kevents)
    ms_step = wall * 1e3 / args.steps
    # The same steps timed per call, with events recorded on the stream around
    # each call (the dispatch gap included), for comparison
    n_call = min(args.steps, 50)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_call)]
    for i in range(n_call):
        step(events[i])
    torch.cuda.synchronize()
    scan_call_ms = sum(e[0].elapsed_time(e[1]) for e in events) / n_call
    upd_call_ms = sum(e[1].elapsed_time(e[2]) for e in events) / n_call

    bytes_p, bytes_d = algorithmic_bytes(wp), algorithmic_bytes(wd)
    ct_p, ct_d = wp.channel_tokens, wd.channel_tokens
    rates = issue_rates()
    scan_r = scan_roofline(wp, scan_ms * 1e3, rates)
    dec_r = decode_roofline(wd, upd_ms * 1e3)
    for r, call_ms in ((scan_r, scan_call_ms), (dec_r, upd_call_ms)):
        r["us_call"] = round(call_ms * 1e3, 2)
        r["timing"] = ("us: the kernel's mean duration, from events its own dispatch records, on every %d-th "
                       "timed step (%d launches); us_call: events recorded on the stream around the call in 50 "
                       "more steps (adds the dispatch gap before the kernel)" % (KERNEL_SAMPLE, len(kevents)))
    wk = scan_work(wp)
    out = {
        "metric": "selective-scan GB/s + channel-tokens/s at Mamba-2.8B layer shape; % roofline",
        "value": round((bytes_p + bytes_d) / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_seconds": round(warm_s, 2),
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 I/O, f32 compute and state",
        "data": "synthetic (seeded; Mamba-2.8B layer shapes, random-init A = -(n+1))",
        "config": {
            "workload": "mamba2p8b prompt scan (batch 8, channels 5120, state_dim 16, seq 2048, gate, h0) + "
                        "decode update (batch 256, channels 5120, state_dim 16)",
            "global_batch": wp.batch,
            "seq_len": wp.seqlen,
            "parallelism": "single GPU",
        },
        "channel_tokens_per_s": round((ct_p + ct_d) / (ms_step * 1e-3), 1),
        "kernels": {"ss_scan_fwd": scan_r, "ss_state_update": dec_r},
        "roofline": {
            "bound": "alu",
            "kernel": "ss_scan_fwd",
            "achieved": round(wk["trans"] / (scan_ms * 1e-3) / 1e12, 4),
            "peak": round(rates[1] / 1e12, 4),
            "unit": "T transcendental lane-ops/s",
            "frac": scan_r["frac"],
            "traffic": recorded_traffic(),
            "hbm_frac": scan_r["hbm_frac"],
            "exp_frac": scan_r["exp_frac"],
            "issue_frac": scan_r["issue_frac"],
            "model": f"frac = max(HBM time, transcendental time) / kernel time. HBM: {bytes_p} algorithmic "
                     f"bytes at {PEAK_HBM_GBS / 1e3:g} TB/s. Transcendental: {wk['trans']:.4g} per launch "
                     f"(16 decay exp2 + softplus exp, log + gate exp, rcp per channel-token) at "
                     f"{rates[1]:.4g} lane-ops/s, measured ({rates[2]}). issue_frac adds the "
                     f"{wk['fma']:.4g} FMA-class operations the method needs at {rates[0]:.4g} lane-ops/s "
                     f"(the same VALU issue slots).",
        },
    }
    if not args.no_workloads:
        out["workloads"] = measure_workloads(ss, stream, rates, P, wp, Dd, wd)
    out["issue_probe_live"] = probe_live()
    if not args.no_extras:
        out["extras"] = {"ss_scan_fwd_states": measure_states(ss, P, wp, bytes_p, stream),
                         "ss_gated_scan": measure_gated(ss, stream),
                         "ss_effective_attention": measure_attention(ss, stream),
                         "producers": measure_producers(ss, stream),
                         "ss_scan_fwd_conv": measure_fused_conv(ss, P, wp, stream, rates),
                         "stream_copy_1GiB": measure_copy(stream)}
        two = measure_two_streams(ss, P, Dd, y, h_last, yd, state, stream)
        two["GB_s"] = round((bytes_p + bytes_d) / (two["us_per_step"] * 1e-6) / 1e9, 1)
        two["sequential_us_per_step"] = round(ms_step * 1e3, 2)
        out["extras"]["step_two_streams"] = two
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cpu_p, wp, args.cpu_seconds)
        # the GPU's speed-up over the oracle on the same workload and unit (the scan's kernel time)
        cb["gpu_speedup"] = round(out["kernels"]["ss_scan_fwd"]["GB_s"] / cb["value"], 1)
        cb["single_thread"] = cpu_single_thread()
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
