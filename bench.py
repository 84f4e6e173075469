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

roofline: the prompt scan dominates and is bound by VALU issue (one
transcendental and five FMA-class operations per token and state
coordinate), so it is reported against the fp32 vector peak in
FMA-equivalent work; see the FLOP model in roofline_flops().

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

PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
TRANS_FLOP_EQ = 8.0        # one transcendental issues at 1/4 the FMA rate: 4 FMA slots = 8 flops


def roofline_flops(w) -> float:
    """FMA-equivalent arithmetic the scan needs per launch (FMA = 2, mul/add = 1,
    transcendental = 8). Per token and state coordinate: dt*A (1), exp (8),
    (dt x)*B (1), h = a h + b (2), y += C h (2) = 14. Per token: dt + bias (1),
    softplus = exp + log (16) plus max/add (2), dt*x (1), y += D x (2); with
    the gate silu = exp + rcp (16) plus add and two muls (3)."""
    ct = w.batch * w.channels * max(w.seqlen, 1)
    per_ct = 1 + 18 + 1 + 2 + (19 if w.gate else 0)
    return float(ct) * (14.0 * w.state_dim + per_ct)


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
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-time budget of the oracle sample")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run a 256 MiB device copy, then 3 steps, for a rocprofv3 --pmc pass (no JSON)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the FETCH_SIZE and WRITE_SIZE passes into " + TRAFFIC_FILE)
    return ap.parse_args()


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
    Reported against the model's flops (the chunked form, as fp32 work) and
    against what the bf16 matrix cores execute (split terms included)."""
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
            "model_frac_of_fp32_peak": round(tf / PEAK_FP32_TFLOPS, 4),
            "bf16_mfma_flops_executed": executed, "bf16_mfma_TFLOP_s": round(te, 2),
            "bf16_mfma_frac": round(te / PEAK_BF16_TFLOPS, 4)}


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


def measure_producers(ss, stream, reps: int = 20):
    """The scan's input side at the Mamba-2.8B layer shape (batch 8, channels
    5120, seq 2048, bf16): ss_conv1d_silu (width 4; bytes: read x_pre, write
    x) and ss_dt_proj (rank 160, with bias and softplus; bytes: read w_dt and
    delta, write dt; flops 2 R per output). Per-launch HIP-event averages."""
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


COPY_CEILING_BYTES = 1 << 30   # each way


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
    }


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
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

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ss.ss_scan_fwd(P["x"], P["dt"], P["A"], P["B"], P["C"], D=P["D"], z=P["z"], dt_bias=P["dt_bias"],
                       h0=P["h0"], y=y, h_last=h_last)
        if ev is not None:
            ev[1].record(stream)
        ss.ss_state_update(state, Dd["x"], Dd["dt"], Dd["A"], Dd["B"], Dd["C"], D=Dd["D"], z=Dd["z"],
                           dt_bias=Dd["dt_bias"], y=yd)
        if ev is not None:
            ev[2].record(stream)

    if args.counter_pass:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
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
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scan_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    upd_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    ms_step = wall * 1e3 / args.steps

    bytes_p, bytes_d = algorithmic_bytes(wp), algorithmic_bytes(wd)
    ct_p, ct_d = wp.channel_tokens, wd.channel_tokens
    flops = roofline_flops(wp)
    achieved = flops / (scan_ms * 1e-3) / 1e12
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
        "kernels": {
            "ss_scan_fwd": {"us": round(scan_ms * 1e3, 2), "GB_s": round(bytes_p / (scan_ms * 1e-3) / 1e9, 1),
                            "channel_tokens_per_s": round(ct_p / (scan_ms * 1e-3), 1),
                            "algorithmic_bytes": bytes_p},
            "ss_state_update": {"us": round(upd_ms * 1e3, 2), "GB_s": round(bytes_d / (upd_ms * 1e-3) / 1e9, 1),
                                "hbm_frac": round(bytes_d / (upd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "algorithmic_bytes": bytes_d},
        },
        "roofline": {
            "bound": "alu",
            "kernel": "ss_scan_fwd",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
            "traffic": recorded_traffic(),
            "flop_model": "FMA-equivalent per launch (FMA 2, mul 1, transcendental 8): "
                          f"{flops:.4g}; HBM side: {bytes_p} algorithmic bytes = "
                          f"{bytes_p / (scan_ms * 1e-3) / 1e9 / PEAK_HBM_GBS:.3f} of 8 TB/s",
        },
    }
    if not args.no_extras:
        out["extras"] = {"ss_scan_fwd_states": measure_states(ss, P, wp, bytes_p, stream),
                         "ss_gated_scan": measure_gated(ss, stream),
                         "ss_effective_attention": measure_attention(ss, stream),
                         "producers": measure_producers(ss, stream),
                         "stream_copy_1GiB": measure_copy(stream)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cpu_p, wp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
