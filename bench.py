#!/usr/bin/env python3
"""Selective-scan forward benchmark on one MI355X.

One step = one ss_scan_fwd call over the whole Mamba-130M-like layer (batch 8, 1536 channels,
L 2048, N 16; bf16 u/delta/z/B/C, f32 A/D/delta_bias, softplus and silu gate on, y in f32),
inputs resident in HBM.  Prints one JSON line:

  value         elements (batch*channels*L) per second over the K timed steps
  roofline      the scan kernel against the VALU (ALU) ceiling, and its HBM rate
  cpu_baseline  the CPU oracle (float64, all host cores) on the same workload

Usage: python bench.py [--steps K] [--warmup W] [--workload 0-4] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "selective-scan fwd elems/s (B·D·L/s) + achieved HBM GB/s vs peak, 1 GPU"

# MI355X published peaks
HBM_PEAK_GBPS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3  # 256 CU x 128 FP32 FMA lanes/clk x 2 FLOP x 2.4 GHz
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
FP32_MATRIX_PEAK_TFLOPS = 157.3  # dense fp32 matrix-core peak

# ALU work model, per element (one (b, d, t)), in FP32 FLOP-equivalents: an FMA is 2, a
# multiply or add 1, and a transcendental (v_exp/v_log/v_rcp, which issues at a quarter of the
# FMA rate on gfx950) 8, i.e. the four FMA issue slots it occupies.  The counts are the
# method's own operations (the minimum any implementation performs), not the kernel's
# instruction count: per (t, n) one exp, dt*A, (dt*u)*B, the state FMA and the readout FMA.
TRANS = 8.0


def flop_equiv_per_element(N, softplus, gate, scalar_decay, P=64):
    if scalar_decay:
        # per (t, p, n): dt*u*B multiply 1, state FMA 2, readout FMA 2; the decay exp is per head
        per = 5.0 * N + (TRANS + 1.0) / P
    else:
        # per (t, n): exp 8, dt*A 1, (dt*u)*B 1, state FMA 2, readout FMA 2
        per = 14.0 * N
    per += 1.0 + 2.0  # dt*u, D*u FMA
    if softplus:
        per += 2 * TRANS + 4.0  # exp, log1p, bias add, max, adds
    if gate:
        per += 2 * TRANS + 3.0  # exp, reciprocal, add, two multiplies
    return per


# source file of each scan kernel
KERNEL_SOURCE = {"diag_fwd_kernel": "ss_diag.hip", "scalar_head_kernel": "ss_scalar.hip",
                 "ssd_scan_kernel": "ss_ssd.hip", "conv1d_kernel": "ss_conv.hip",
                 "bwd_kernel": "ss_bwd.hip", "ssdb_main_kernel": "ss_ssd_bwd.hip"}


def scan_kernel(p):
    """Name of the kernel that dominates one call on this workload (the library's own choice:
    scalar decay with bf16 inputs and heads of a multiple of 64 channels takes the matrix form)."""
    if not p.scalar_decay:
        return "diag_fwd_kernel"
    P = p.channels // p.heads
    cpg = p.channels // p.groups
    if p.in_dtype == "bf16" and P % 64 == 0 and cpg % 64 == 0:
        return "ssd_scan_kernel"
    return "scalar_head_kernel"


def kernel_source_digest(kernel):
    """sha256 of the HIP source of the kernel (to match stored counters)."""
    import hashlib

    name = KERNEL_SOURCE[kernel]
    path = os.path.join(ROOT, "selective_state_space_88_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_traffic(kernel, workload, digest, mode=None):
    """HBM bytes per launch from the committed counter summary, if it was taken on this source.

    The summary (profiles/traffic_<kernel>[_<mode>]_w<workload>.txt) holds `key: value` lines written
    from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by the same counter's
    reading for a plain copy of known size in the same process.
    """
    tag = "" if mode is None else "_" + mode
    path = os.path.join(ROOT, "profiles", "traffic_%s%s_w%d.txt" % (kernel, tag, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def describe(p):
    """One line naming the workload: its name, input types and flags."""
    ins = "u/delta" + ("/z" if p.gate else "") + "/B/C"
    flags = ["softplus" if p.softplus else "raw delta"] + (["silu gate"] if p.gate else ["no gate"])
    return "%s: %s %s, f32 A/D/delta_bias, %s, y f32" % (p.name, p.in_dtype, ins, " + ".join(flags))


def algorithmic_bytes(p, y_bytes):
    ib = 2 if p.in_dtype == "bf16" else 4
    E = p.batch * p.channels * p.length
    n = E * ib + E * y_bytes                      # u, y
    n += p.batch * p.heads * p.length * ib        # delta
    if p.gate:
        n += E * ib                               # z
    n += 2 * p.batch * p.groups * p.nstate * p.length * ib  # B, C
    n += p.A.size * 4 + (p.D.size * 4 if p.D is not None else 0)
    n += p.delta_bias.size * 4 if p.delta_bias is not None else 0
    return n


def copy_calibration(args, dev):
    """A plain streaming kernel of known size: the elementwise multiply reads and writes
    copy_calibration * 10^6 bytes per launch (its own kernel name in the profile)."""
    import torch

    if not args.copy_calibration:
        return
    n = args.copy_calibration * 1000000 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def decode_bench(args, p, to_dev, dev):
    """One decoding step per call (ss_scan_step) on the workload's shapes: step 0 of its inputs
    and a seeded state.  The step reads and writes the f32 state (8 N bytes per row) and reads
    one token of inputs, so its roofline is HBM; at these sizes a call is also close to the
    launch latency."""
    import torch

    from selective_state_space_88_amd import inputs
    from selective_state_space_88_amd.scan import scan_step

    s = inputs.step_slice(p, 0)
    t = {k: to_dev(getattr(s, k)) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    h = to_dev(inputs.random_state(7, p.batch, p.channels, p.nstate, scale=0.1))
    y = torch.empty((p.batch, p.channels), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        scan_step(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], h,
                  softplus=p.softplus, y=y, stream=stream.cuda_stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # steps captured in a HIP graph and replayed, as a serving loop runs them (a Python call per
    # step would time the host, not the GPU); replays are checked against eager steps in the tests
    G = 50
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(G):
                scan_step(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], h,
                          softplus=p.softplus, y=y)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    R = max(1, args.steps // G)
    K = R * G
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(R):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = e0.elapsed_time(e1) * 1e-3 / K
    rows = p.batch * p.channels
    ib = 2 if p.in_dtype == "bf16" else 4
    nbytes = rows * (8 * p.nstate + ib * (2 if p.gate else 1) + 4)       # state r/w, u (z), y
    nbytes += p.batch * p.heads * ib + 2 * p.batch * p.groups * p.nstate * ib
    gbps = nbytes / per_call / 1e9
    out = {
        "metric": "selective-scan decode step rows/s (batch*channels per second), 1 GPU",
        "value": rows * K / wall, "unit": "rows/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode step, " + describe(p), "batch": p.batch, "channels": p.channels,
                   "nstate": p.nstate, "heads": p.heads, "kernel": "step_kernel"},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "call_us": per_call * 1e6,
                     "hbm_algorithmic_bytes_per_call": nbytes},
        "cpu_baseline": None,
    }
    print(json.dumps(out))


# Backward ALU work per (t, n), FLOP-equivalents as in the forward: the recomputed decay exp (8)
# and dt*A (1), dt*u*B (1), the recomputed state FMA (2), the adjoint FMA (2) and its decay
# product (1), dC (1), dB (1), du (2), ddt (4: two FMAs), dA (2: multiply, FMA) = 25; per
# element the forward's per-step terms (softplus, gate, D) and their derivatives (~2x).
def bwd_flop_equiv_per_element(N, softplus, gate, scalar_decay=False):
    # scalar decay: the exp and dt*A are per step, not per (t, n)
    per = (16.0 * N + TRANS + 1.0 if scalar_decay else 25.0 * N) + 2 * 3.0
    if softplus:
        per += 2 * (2 * TRANS + 4.0)
    if gate:
        per += 2 * (2 * TRANS + 3.0)
    return per


def backward_bench(args, p, to_dev, dev):
    """ss_scan_bwd on the workload with a seeded upstream gradient dy (f32): the checkpoint pass,
    the zeroing of the summed gradients and the backward kernel, all inside the timed call."""
    import torch

    from selective_state_space_88_amd import inputs
    from selective_state_space_88_amd.scan import scan_bwd

    t = {k: to_dev(getattr(p, k)) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    dy = to_dev(inputs.seeded_normal(12, (p.batch, p.channels, p.length)))
    stream = torch.cuda.current_stream(dev)

    def call():
        return scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], dy,
                        softplus=p.softplus, stream=stream.cuda_stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    copy_calibration(args, dev)
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)])) * 1e-3
    E = p.batch * p.channels * p.length
    flops = E * bwd_flop_equiv_per_element(p.nstate, p.softplus, p.gate, p.scalar_decay)
    ib = 2 if p.in_dtype == "bf16" else 4
    # reads u, z, dy (f32), delta, B, C; writes du, dz, ddelta (f32) and dB, dC (f32)
    nbytes = E * (ib * (2 if p.gate else 1) + 4 + 4 * (2 if p.gate else 1))
    nbytes += p.batch * p.heads * p.length * (ib + 4)
    nbytes += p.batch * p.groups * p.nstate * p.length * 2 * (ib + 4)
    tf = flops / per / 1e12
    P = p.channels // p.heads
    matrix = p.scalar_decay and not p.gate and P % 64 == 0 and (p.channels // p.groups) % 64 == 0
    dominant = "ssdb_main_kernel" if matrix else "bwd_kernel"
    traffic = stored_traffic(dominant, args.workload, kernel_source_digest(dominant), mode="backward")
    out = {
        "metric": "selective-scan bwd elems/s (B*D*L/s), 1 GPU", "value": E * K / wall, "unit": "elems/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": wall / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "backward, " + describe(p), "batch": p.batch, "channels": p.channels,
                   "seq_len": p.length, "nstate": p.nstate,
                   "kernel": dominant},
        "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / FP32_VECTOR_PEAK_TFLOPS, "traffic": traffic, "call_ms": per * 1e3,
                     "flop_equiv_per_call": flops, "hbm_algorithmic_bytes_per_call": nbytes,
                     "hbm_achieved_GBps": nbytes / per / 1e9},
        "cpu_baseline": None,
    }
    if matrix:
        # The scalar-decay backward is a chain of dense contractions on v_mfma_f32_16x16x4_f32
        # (2048 flops each), so its roofline is the fp32 matrix peak.  Per (batch, head, 64-channel
        # slab, 32-step chunk) each of 4 waves issues 32 + 40 NT in the reverse pass and 8 NT in the
        # forward pass (NT = 16-state tiles: 2, 4 or 8), and per (batch, group, chunk) C B^T takes
        # 4 NT per wave; the time is the whole call.
        NT = 2 if p.nstate <= 32 else 4 if p.nstate <= 64 else 8
        nch = (p.length + 31) // 32
        blocks = p.batch * p.heads * (P // 64)
        mf = (blocks * nch * 4 * (32 + 48 * NT) + p.batch * p.groups * nch * 4 * 4 * NT) * 2048.0
        rl = out["roofline"]
        out["roofline"] = {
            "bound": "mfma", "achieved": mf / per / 1e12, "peak": FP32_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": mf / per / 1e12 / FP32_MATRIX_PEAK_TFLOPS, "traffic": traffic, "call_ms": rl["call_ms"],
            "mfma_flops_per_call": mf, "alu_flop_equiv_per_call": flops, "alu_equiv_TFLOPs": tf,
            "hbm_algorithmic_bytes_per_call": nbytes, "hbm_achieved_GBps": nbytes / per / 1e9,
        }
    print(json.dumps(out))


def conv_bench(args, p, to_dev, dev):
    """ss_conv1d (causal depthwise convolution, silu on, W taps) on the workload's scan input
    shape: x = the workload's u (bf16 or f32), f32 taps and bias drawn as in the tests, out in
    the input dtype (the scan's next input).  It reads x and writes out once, so its roofline is
    HBM."""
    import torch

    from selective_state_space_88_amd import inputs
    from selective_state_space_88_amd.scan import conv1d

    W = args.conv_width
    c = inputs.random_conv(31, 1, p.channels, 0, W, with_state=False)
    x = to_dev(p.u)
    w, b = to_dev(c["w"]), to_dev(c["bias"])
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def call():
        conv1d(x, w, b, silu=True, out=out, stream=stream.cuda_stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    copy_calibration(args, dev)
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = e0.elapsed_time(e1) * 1e-3 / K
    E = p.batch * p.channels * p.length
    ib = 2 if p.in_dtype == "bf16" else 4
    nbytes = 2 * E * ib + p.channels * (W + 1) * 4
    gbps = nbytes / per / 1e9
    traffic = stored_traffic("conv1d_kernel", args.workload, kernel_source_digest("conv1d_kernel"),
                             mode="conv")
    out_line = {
        "metric": "causal conv1d elems/s (B*D*L/s), 1 GPU", "value": E * K / wall, "unit": "elems/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": wall / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "causal depthwise conv (W=%d, bias, silu) on the scan input of %s, out %s"
                               % (W, p.name, p.in_dtype),
                   "batch": p.batch, "channels": p.channels, "seq_len": p.length, "width": W,
                   "kernel": "conv1d_kernel"},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic, "launch_ms": per * 1e3,
                     "hbm_algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": None,
    }
    print(json.dumps(out_line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clock ramps up over the first tens of milliseconds of sustained work (workload 1:
    # 0.142 ms per launch over 100 back-to-back launches, 0.129 over 1000), so the defaults warm
    # up for ~25 ms and time ~0.13 s of steady state.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--decode", action="store_true",
                    help="time the decoding step (ss_scan_step: one token for every (batch, channel) "
                         "row of the workload's shapes, state updated in place) instead of the scan")
    ap.add_argument("--zoh", action="store_true",
                    help="zero-order-hold input coefficient (SS_ZOH) instead of exponential-Euler")
    ap.add_argument("--trapezoid", action="store_true",
                    help="exponential-trapezoidal rule (SS_TRAPEZOID) instead of exponential-Euler")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (ss_scan_bwd: gradients of every input for an upstream "
                         "gradient dy) on the workload instead of the forward")
    ap.add_argument("--conv", action="store_true",
                    help="time the causal depthwise convolution in front of the scan (ss_conv1d, silu) "
                         "on the workload's scan input instead of the scan")
    ap.add_argument("--conv-width", type=int, default=4, help="taps of --conv (1..8)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run a plain device copy of MB megabytes (10^6 B) per step, so that "
                         "HBM byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan's rows are independent, so more GPUs would "
              "each run the same kernel on their own share; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_88_amd import inputs
    from selective_state_space_88_amd.scan import fwd_launcher

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    p = inputs.make(args.workload)

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    if args.decode:
        decode_bench(args, p, to_dev, dev)
        return
    if args.backward:
        backward_bench(args, p, to_dev, dev)
        return
    if args.conv:
        conv_bench(args, p, to_dev, dev)
        return

    t = {k: to_dev(getattr(p, k)) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    y = torch.empty(p.u.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # one ss_scan_fwd call per step, its descriptors built once (the per-call marshalling of
    # scan_fwd takes host time comparable to the kernel, which would leave the GPU idle between
    # launches)
    step = fwd_launcher(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], y,
                        softplus=p.softplus, stream=stream.cuda_stream, zoh=args.zoh, trapezoid=args.trapezoid)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    copy_calibration(args, dev)

    # timed region: K back-to-back steps, bracketed by device synchronisation; HIP events on the
    # launch stream around the K launches give the kernel's average duration (the step is that
    # one kernel)
    K = args.steps
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(K):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = e_start.elapsed_time(e_end) * 1e-3 / K

    E = p.batch * p.channels * p.length
    value = E * K / wall
    nbytes = algorithmic_bytes(p, 4)
    flops = E * flop_equiv_per_element(p.nstate, p.softplus, p.gate, p.scalar_decay,
                                       P=p.channels // p.heads)
    alu_tflops = flops / avg_launch_s / 1e12
    hbm_gbps = nbytes / avg_launch_s / 1e9
    # the kernel that dominates the step (the diagonal path is that one kernel alone)
    kernel = scan_kernel(p)
    traffic = stored_traffic(kernel, args.workload, kernel_source_digest(kernel))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": describe(p) + (", zero-order hold" if args.zoh else "") +
                        (", exponential-trapezoidal" if args.trapezoid else ""),
            "batch": p.batch, "channels": p.channels, "seq_len": p.length, "nstate": p.nstate,
            "heads": p.heads, "inputs": p.in_dtype, "y": "f32",
            "kernel": kernel,
        },
        "roofline": {
            "bound": "alu",
            "achieved": alu_tflops,
            "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": alu_tflops / FP32_VECTOR_PEAK_TFLOPS,
            "traffic": traffic,
            "launch_ms": avg_launch_s * 1e3,
            "flop_equiv_per_launch": flops,
            "hbm_algorithmic_bytes_per_launch": nbytes,
            "hbm_achieved_GBps": hbm_gbps,
            "hbm_frac": hbm_gbps / HBM_PEAK_GBPS,
        },
        "cpu_baseline": None,
    }

    if kernel == "ssd_scan_kernel":
        # The matrix form is a dense contraction on v_mfma_f32_16x16x32_bf16 (16*16*32*2 flops
        # each), so its roofline is the bf16 matrix peak.  Per (batch, head, 64-channel slab,
        # 32-step chunk) each of 4 waves issues 4 for the masked product, Np/8 for the readout
        # from the carried state and Np/8 for the state update (Np = N padded to a multiple of
        # 32), counting the bf16 hi/lo split passes; the state pass that hands state between
        # sequence segments is not counted.  The time is the whole call (pre-pass, state pass
        # and output pass), so the rate is a lower bound for the output pass.  The ALU figures
        # are kept beside it: the matrix form does less than the recurrence's own arithmetic.
        Np = (p.nstate + 31) // 32 * 32
        nch = (p.length + 31) // 32
        mf = p.batch * p.heads * (p.channels // p.heads // 64) * nch * 4 * (4 + Np // 4) * 16384.0
        mf_tflops = mf / avg_launch_s / 1e12
        rl = out["roofline"]
        out["roofline"] = {
            "bound": "mfma", "achieved": mf_tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": mf_tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": traffic,
            "launch_ms": rl["launch_ms"], "mfma_flops_per_launch": mf,
            "alu_flop_equiv_per_launch": flops, "alu_equiv_TFLOPs": alu_tflops,
            "alu_equiv_frac": alu_tflops / FP32_VECTOR_PEAK_TFLOPS,
            "hbm_algorithmic_bytes_per_launch": nbytes, "hbm_achieved_GBps": hbm_gbps,
            "hbm_frac": hbm_gbps / HBM_PEAK_GBPS,
        }

    if not args.no_cpu_baseline:
        import oracle

        cores = oracle.default_threads()
        # bounded sample: the whole workload when it is small, else a prefix of its rows
        total_rows = p.batch * p.channels
        budget = 2.0e9  # state-steps (t, n) per repeat: a few seconds on a few dozen cores
        nrows = int(min(total_rows, max(1, budget // (p.length * p.nstate))))
        rows = np.arange(nrows, dtype=np.int64) if nrows < total_rows else None
        best = None
        for _ in range(max(1, args.cpu_repeats)):
            c0 = time.perf_counter()
            oracle.scan_problem(p, rows=rows, threads=cores)
            dt = time.perf_counter() - c0
            best = dt if best is None else min(best, dt)
        out["cpu_baseline"] = {
            "value": nrows * p.length / best,
            "unit": "elems/s",
            "cores": cores,
            "kind": "oracle",
            "sample": "%s rows of %d (each L=%d, N=%d) of the same workload, best of %d runs, "
                      "float64 sequential recurrence, %d threads"
                      % ("all" if rows is None else str(nrows), total_rows, p.length, p.nstate,
                         max(1, args.cpu_repeats), cores),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
