#!/usr/bin/env python3
"""Selective-scan forward benchmark on one MI355X.

One step = one ss_scan_fwd call over a whole synthetic layer, inputs resident in HBM.  The
default layer is the largest single-GPU configuration of the benchmark set, the long-sequence
layer (batch 1, 1024 channels, L = 1,048,576, N 16; bf16 u/delta/z/B/C, f32 A/D/delta_bias,
softplus and silu gate on, y in f32).  Prints one JSON line:

  value         elements (batch*channels*L) per second over the K timed steps
  roofline      the dominant kernel against the HBM roofline (8 TB/s): algorithmic bytes per
                launch / the launch's average duration (HIP events on the launch stream); the
                plain-ALU ceiling of the method's arithmetic is reported beside it
  cpu_baseline  the CPU oracle (float64, all host cores) on a bounded sample of the same layer

Usage: python bench.py [--steps K] [--warmup W] [--workload 0-4] [--no-cpu-baseline]
                       [--report FILE]   (also measure workloads 1-4 and write one JSON line each)
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
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
FP32_MATRIX_PEAK_TFLOPS = 157.3  # dense fp32 matrix-core peak
FP32_VECTOR_UNPACKED_TFLOPS = 78.6  # FP32 FMA without packed FP32 (which this build compiles out)
MALL_BYTES = 256 * 2 ** 20       # Infinity Cache (last-level cache in front of HBM)

# Plain-ALU ceiling of the method's arithmetic (the competing bound of the diagonal path).
# Unpacked VALU issue: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 3.93e13 lane-operations/s; a
# transcendental (v_exp/v_log/v_rcp) takes TRANS_SLOTS issue slots of an FMA (quarter rate).
VALU_LANE_OPS = 256 * 64 * 2.4e9
TRANS_SLOTS = 4.0


def alu_slots_per_element(p):
    """Issue slots per element (one (b, d, t)) of the method's own operations, the minimum any
    implementation performs: per (t, n) an exp and four FP32 operations (dt*A, (dt*u)*B, the
    state FMA, the readout FMA); per element ~14 FP32 operations (bias, dt*u, D*u, the softplus
    and gate arithmetic) and the softplus's two and the gate's two transcendentals.  Scalar
    decay (one exp per head and step, shared by its P channels): per (t, p, n) the input
    multiply, the state FMA and the readout FMA."""
    if p.scalar_decay:
        P = p.channels // p.heads
        per = 3.0 * p.nstate + 8.0 + TRANS_SLOTS * (1.0 + (2.0 if p.softplus else 0.0)) / P
    else:
        per = p.nstate * (TRANS_SLOTS + 4.0) + 14.0 + TRANS_SLOTS * (2.0 if p.softplus else 0.0)
    if p.gate:
        per += 2 * TRANS_SLOTS
    return per



# source file of each scan kernel
KERNEL_SOURCE = {"diag_fwd_kernel": "ss_diag.hip", "diag_slots_kernel": "ss_diag.hip",
                 "scalar_head_kernel": "ss_scalar.hip",
                 "ssd_scan_kernel": "ss_ssd.hip", "conv1d_kernel": "ss_conv.hip",
                 "bwd_kernel": "ss_bwd.hip", "ssdb_main_kernel": "ss_ssd_bwd.hip"}


def scan_kernel(p, cus=256):
    """Name of the kernel that dominates one call on this workload (the library's own choice:
    scalar decay with bf16 inputs and heads of a multiple of 64 channels takes the matrix form; a
    diagonal decay with bf16 inputs, N >= 5, at least three 1024-step windows and at most one row
    per SIMD (4 x `cus` rows) takes the window-slot kernel; the bench's rows are aligned)."""
    if not p.scalar_decay:
        if (p.in_dtype == "bf16" and p.nstate >= 5 and p.length % 8 == 0 and (p.length + 1023) // 1024 >= 3
                and p.batch * p.channels <= 4 * cus):
            return "diag_slots_kernel"
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
def bwd_alu_slots_per_element(N, softplus, gate, scalar_decay=False):
    """VALU issue slots per element of the backward's own operations (a transcendental = 4): per
    (t, n) the recomputed state (exp, dt A, dt u B, the FMA: 7), the adjoint (its FMA and the
    decay: 2) and the gradient terms (dC, dB, du, g h a, ddt, dA: 7), plus the readout of the
    output before the gate when there is one; scalar decay takes the exp and dt A once per step.
    Per element: du/ddt/dD/dbias (5), softplus and its derivative, silu and its derivative."""
    per_tn = (11.0 if scalar_decay else 16.0) + (1.0 if gate else 0.0)
    per = per_tn * N + (TRANS_SLOTS + 1.0 if scalar_decay else 0.0) + 5.0
    if softplus:
        per += (2 * TRANS_SLOTS + 4.0) + (2 * TRANS_SLOTS + 2.0)
    if gate:
        per += (2 * TRANS_SLOTS + 3.0) + (2 * TRANS_SLOTS + 5.0)
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
    # FMA-equivalent flops: every VALU slot counted as one FMA (2 flops), against the unpacked
    # FP32 FMA rate (packed FP32 is compiled out)
    slots = bwd_alu_slots_per_element(p.nstate, p.softplus, p.gate, p.scalar_decay)
    flops = 2.0 * E * slots
    ib = 2 if p.in_dtype == "bf16" else 4
    # reads u, z, dy (f32), delta, B, C; writes du, dz, ddelta (f32) and dB, dC (f32)
    nbytes = E * (ib * (2 if p.gate else 1) + 4 + 4 * (2 if p.gate else 1))
    nbytes += p.batch * p.heads * p.length * (ib + 4)
    nbytes += p.batch * p.groups * p.nstate * p.length * 2 * (ib + 4)
    tf = flops / per / 1e12
    P = p.channels // p.heads
    matrix = p.scalar_decay and P % 64 == 0 and (p.channels // p.groups) % 64 == 0
    dominant = "ssdb_main_kernel" if matrix else "bwd_kernel"
    traffic = stored_traffic(dominant, args.workload, kernel_source_digest(dominant), mode="backward")
    out = {
        "metric": "selective-scan bwd elems/s (B*D*L/s), 1 GPU", "value": E * K / wall, "unit": "elems/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": wall / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "backward, " + describe(p), "batch": p.batch, "channels": p.channels,
                   "seq_len": p.length, "nstate": p.nstate,
                   "kernel": dominant},
        "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_VECTOR_UNPACKED_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / FP32_VECTOR_UNPACKED_TFLOPS, "traffic": traffic, "call_ms": per * 1e3,
                     "valu_slots_per_element": slots, "flop_equiv_per_call": flops,
                     "hbm_algorithmic_bytes_per_call": nbytes,
                     "hbm_achieved_GBps": nbytes / per / 1e9},
        "cpu_baseline": None,
    }
    if matrix:
        # The scalar-decay backward is a chain of dense contractions on the matrix cores, so its
        # roofline is the matrix peak of the dtype it runs in; the work is the MFMA instructions
        # executed (split passes counted), the time the whole call.  NT = 16-state tiles (2, 4
        # or 8), NB = max(NT / 4, 1), NR = NT / 2; per (batch, head, 64-channel slab, 32-step chunk)
        # the reverse pass runs 8 waves (the [T x N] tiles on all 8 when NT >= 4, else on 4) and
        # the forward pass SPL blocks of 4 waves (SPL = 4 for NT = 8, else 2; NH = NT / SPL tiles
        # each); C B^T takes 4 waves per (batch, group, chunk).
        NT = 2 if p.nstate <= 32 else 4 if p.nstate <= 64 else 8
        nch = (p.length + 31) // 32
        blocks = p.batch * p.heads * (P // 64)
        NB, NR = max(NT // 4, 1), NT // 2
        bcw = 8 if NT >= 4 else 4
        SPL = 4 if NT >= 8 else 2
        if p.in_dtype == "bf16":
            # v_mfma_f32_16x16x32_bf16 (16384 flops): an f32 operand split in hi and lo costs a
            # product three instructions (two when the other operand is bf16 already: u, B, C)
            rev = 4 * 2 * 2 + bcw * (2 * NB * 3 + 2 * NB * 2 + 2 * NB * 2) + 8 * (NT // 2 * 2 + 3 + NR * 2)
            fwd = SPL * 4 * (NT // SPL) * 2
            cbt = 4 * (16 * NT // 32)
            # the reverse pass's sequence segments (about five blocks per CU, at least 8 chunks
            # each): a pre-pass over every segment but the first forms its part of the adjoint,
            # 4 waves x NT tiles x 2 (dy split, C exact) per chunk
            S = max(1, min(-(-5 * 256 // blocks), nch // 8))
            cps = -(-nch // S)
            pre_chunks = nch - cps if -(-nch // cps) > 1 else 0
            mf = (blocks * nch * (rev + fwd) + blocks * pre_chunks * 4 * NT * 2 +
                  p.batch * p.groups * nch * cbt) * 16384.0
            peak = BF16_MFMA_PEAK_TFLOPS
        else:
            # v_mfma_f32_16x16x4_f32 (2048 flops each)
            mf = (blocks * nch * 4 * (32 + 48 * NT) + p.batch * p.groups * nch * 4 * 4 * NT) * 2048.0
            peak = FP32_MATRIX_PEAK_TFLOPS
        rl = out["roofline"]
        out["roofline"] = {
            "bound": "mfma", "achieved": mf / per / 1e12, "peak": peak, "unit": "TFLOP/s",
            "frac": mf / per / 1e12 / peak, "traffic": traffic, "call_ms": rl["call_ms"],
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


PROBE_KINDS = {0: "v_mul_f32", 1: "v_fma_f32", 2: "v_exp_f32", 3: "v_mul_f32_dpp",
               4: "v_exp_f32 + v_fma_f32 alternating", 5: "one v_exp_f32 in four (three v_fma_f32)"}


def probe_bench(args, dev):
    """Ceiling probes (libssprobe.so, include/ss_probe.h): cycles per wave64 instruction per SIMD
    for the instruction kinds the diagonal scan is made of, at 1 to 8 waves per SIMD, and the HBM
    rates of a streaming copy and a streaming read of 1 GiB.  Prints one JSON line; with
    --probe-out DIR also writes the text summaries DIR/probe_valu.txt and DIR/probe_hbm_copy.txt."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "selective_state_space_88_amd", "libssprobe.so")
    if not os.path.exists(path):
        print("libssprobe.so is not built (run selective_state_space_88_amd/build.py)", file=sys.stderr)
        sys.exit(1)
    lib = ctypes.CDLL(path)
    lib.ssp_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p]
    lib.ssp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.ssp_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    iters = 4000
    valu = {}
    clocks = []
    for kind, name in PROBE_KINDS.items():
        for w in (1, 2, 3, 4, 8):
            blocks = cus * w   # 4 waves per block: w waves per SIMD
            out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
            clk = torch.zeros(2, dtype=torch.int64, device=dev)
            run = lambda: lib.ssp_valu(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(clk.data_ptr()), ctypes.c_void_p(sid))
            assert run() == 0
            sec = timed(run, 5)
            c = clk.cpu().tolist()
            hz = c[0] / c[1] * 1e8 if c[1] else 0.0
            clocks.append(hz)
            per_simd = w * iters * 32     # instructions issued by each SIMD
            valu.setdefault(name, {})[w] = {"ns_per_instr": sec * 1e9 / per_simd,
                                            "cycles_per_instr": sec * hz / per_simd, "clock_GHz": hz / 1e9}
            del out, clk
    # HBM: 1 GiB streams, 8 blocks of 256 threads per CU (grid-stride)
    n16 = (1 << 30) // 16
    src = torch.ones(n16 * 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    blocks = cus * 8
    red = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    t_copy = timed(lambda: lib.ssp_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                        n16, blocks, ctypes.c_void_p(sid)), 20)
    t_read = timed(lambda: lib.ssp_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(red.data_ptr()),
                                        n16, blocks, ctypes.c_void_p(sid)), 20)
    copy_gbps = 2 * n16 * 16 / t_copy / 1e9
    read_gbps = n16 * 16 / t_read / 1e9
    out = {"metric": "ceiling probes", "device": props.name, "compute_units": cus,
           "clock_GHz_median": float(np.median(clocks)) / 1e9, "valu": valu,
           "hbm": {"copy_GBps": copy_gbps, "read_GBps": read_gbps, "bytes_per_copy": 2 * n16 * 16,
                   "frac_of_8TBps_copy": copy_gbps / HBM_PEAK_GBPS, "frac_of_8TBps_read": read_gbps / HBM_PEAK_GBPS}}
    print(json.dumps(out), flush=True)
    if args.probe_out:
        cmd = "python3 bench.py --probe --probe-out profiles"
        with open(os.path.join(args.probe_out, "probe_valu.txt"), "w") as f:
            f.write("# VALU issue probes on %s (%d CUs), libssprobe.so (include/ss_probe.h)\n" % (props.name, cus))
            f.write("# command (from the repository root): %s\n" % cmd)
            f.write("# cycles per wave64 instruction per SIMD (independent instructions, no dependency "
                    "stalls), at 1-8 waves per SIMD;\n# clock from s_memtime / s_memrealtime in the run\n")
            f.write("%-40s %s\n" % ("instruction", "  ".join("w=%d" % w for w in (1, 2, 3, 4, 8))))
            for name, row in valu.items():
                f.write("%-40s %s\n" % (name, "  ".join("%5.2f" % row[w]["cycles_per_instr"] for w in (1, 2, 3, 4, 8))))
            f.write("clock_GHz_median: %.3f\n" % (float(np.median(clocks)) / 1e9))
        with open(os.path.join(args.probe_out, "probe_hbm_copy.txt"), "w") as f:
            f.write("# HBM streaming probes on %s, libssprobe.so: 1 GiB, 16-byte nontemporal accesses, "
                    "%d blocks of 256 threads\n" % (props.name, blocks))
            f.write("# command (from the repository root): %s\n" % cmd)
            f.write("copy_GBps: %.1f\n" % copy_gbps)
            f.write("read_GBps: %.1f\n" % read_gbps)
            f.write("copy_frac_of_8000: %.3f\n" % (copy_gbps / HBM_PEAK_GBPS))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clock ramps up over the first tens of milliseconds of sustained work (workload 1:
    # 0.142 ms per launch over 100 back-to-back launches, 0.129 over 1000), so the defaults warm
    # up for ~25 ms and time ~0.13 s of steady state.
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 30 on the 1M-step layer, 1000 on the others)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: 10 on the 1M-step layer, 200 on the others)")
    ap.add_argument("--workload", type=int, default=3, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--report", metavar="FILE", default=None,
                    help="also measure workloads 1-4 (forward) and write one JSON line per workload to FILE")
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
    ap.add_argument("--gate", action="store_true",
                    help="with --backward on the scalar-decay workload: add a silu gate on a seeded z "
                         "(the layout the workload itself leaves ungated)")
    ap.add_argument("--conv", action="store_true",
                    help="time the causal depthwise convolution in front of the scan (ss_conv1d, silu) "
                         "on the workload's scan input instead of the scan")
    ap.add_argument("--conv-width", type=int, default=4, help="taps of --conv (1..8)")
    ap.add_argument("--probe", action="store_true",
                    help="run the ceiling probes (VALU issue costs, HBM copy and read rates) instead of the scan")
    ap.add_argument("--probe-out", metavar="DIR", default=None,
                    help="with --probe: write the summaries probe_valu.txt and probe_hbm_copy.txt into DIR")
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
    if args.probe:
        probe_bench(args, dev)
        return
    big = args.workload == 3
    if args.steps is None:
        args.steps = 30 if big else 1000
    if args.warmup is None:
        args.warmup = 10 if big else 200
    p = inputs.make(args.workload, gate=True) if args.gate else inputs.make(args.workload)

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

    out = forward_line(args, p, args.workload, to_dev, dev, steps=args.steps, warmup=args.warmup,
                       cpu=not args.no_cpu_baseline)
    if args.report:
        # the per-workload report: every large workload measured the same way, one JSON line each
        with open(args.report, "w") as f:
            for k in (1, 2, 3, 4):
                if k == args.workload:
                    line = out
                else:
                    q = inputs.make(k)
                    line = forward_line(args, q, k, to_dev, dev, steps=REPORT_STEPS[k], warmup=REPORT_WARMUP[k],
                                        cpu=False)
                    del q
                f.write(json.dumps(line) + "\n")
                f.flush()
                print("report: workload %d %.3f ms per launch, HBM %.3f of peak" %
                      (k, line["roofline"]["launch_ms"], line["roofline"]["frac"]), file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


# steps and warm-up launches of the per-workload report (about 0.2 s of timed work each)
REPORT_STEPS = {1: 1000, 2: 400, 3: 20, 4: 600}
REPORT_WARMUP = {1: 200, 2: 100, 3: 5, 4: 100}


def forward_line(args, p, workload, to_dev, dev, *, steps, warmup, cpu):
    """Measure one workload's forward and return its JSON record.

    Timed region: `steps` back-to-back ss_scan_fwd calls (descriptors built once), bracketed by
    device synchronisation, with HIP events on the launch stream around them: their span / steps
    is the average launch duration used for the roofline.  Then the same number of launches each
    between its own event pair (median and min per launch) and, when the layer's bytes fit the
    256 MB Infinity Cache a few times over, launches each preceded by a 1 GiB write that evicts
    it (cold median and min)."""
    import torch

    from selective_state_space_88_amd.scan import fwd_launcher

    t = {k: to_dev(getattr(p, k)) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    y = torch.empty(p.u.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # one ss_scan_fwd call per step, its descriptors built once (the per-call marshalling of
    # scan_fwd takes host time comparable to a short kernel, which would leave the GPU idle
    # between launches)
    step = fwd_launcher(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], y,
                        softplus=p.softplus, stream=stream.cuda_stream, zoh=args.zoh, trapezoid=args.trapezoid)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    copy_calibration(args, dev)

    # timed region: K back-to-back steps
    K = steps
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(K):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = e_start.elapsed_time(e_end) * 1e-3 / K

    # per-launch events: median and min
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in ev])

    nbytes = algorithmic_bytes(p, 4)
    cold = None
    if nbytes <= 4 * MALL_BYTES:
        scratch = torch.empty(2 ** 28, dtype=torch.float32, device=dev)   # 1 GiB
        R = max(10, min(50, K))
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R)]
        for a, b in cev:
            scratch.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        cper = np.array([a.elapsed_time(b) for a, b in cev])
        cold = {"reps": R, "median_ms": float(np.median(cper)), "min_ms": float(np.min(cper)),
                "eviction": "1 GiB written before each launch"}
        del scratch

    E = p.batch * p.channels * p.length
    value = E * K / wall
    hbm_gbps = nbytes / avg_launch_s / 1e9
    slots = alu_slots_per_element(p)
    alu_floor_s = E * slots / VALU_LANE_OPS
    # the kernel that dominates the step (the diagonal path is that one kernel alone)
    kernel = scan_kernel(p, torch.cuda.get_device_properties(dev).multi_processor_count)
    traffic = stored_traffic(kernel, workload, kernel_source_digest(kernel))
    copy_peak = stored_copy_peak()

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
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
            "heads": p.heads, "inputs": p.in_dtype, "y": "f32", "arithmetic": "f32",
            "kernel": kernel,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": hbm_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": hbm_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "launch_ms": avg_launch_s * 1e3,
            "launch_ms_median": float(np.median(per)),
            "launch_ms_min": float(np.min(per)),
            "cold": cold if cold is not None else
            "not needed: %.2f GB per launch against a %d MB cache" % (nbytes / 1e9, MALL_BYTES >> 20),
            "hbm_algorithmic_bytes_per_launch": nbytes,
            "frac_of_copy_peak": (hbm_gbps / copy_peak) if copy_peak else None,
            "copy_peak_GBps": copy_peak,
            "alu": {"slots_per_element": slots, "lane_ops_per_s": VALU_LANE_OPS,
                    "floor_ms": alu_floor_s * 1e3, "frac": alu_floor_s / avg_launch_s},
        },
        "cpu_baseline": None,
    }

    if kernel == "ssd_scan_kernel":
        # the VALU model counts per-(t, p, n) FP32 operations that the matrix form does on the
        # matrix cores instead: it bounds nothing here
        del out["roofline"]["alu"]
        # The matrix form is a chain of dense contractions on v_mfma_f32_16x16x32_bf16
        # (16*16*32*2 flops each).  Per (batch, head, 64-channel slab, 32-step chunk) each of 4
        # waves issues 4 for the masked product, Np/8 for the readout from the carried state and
        # Np/8 for the state update (Np = N padded to a multiple of 32), counting the bf16 hi/lo
        # split passes; the state pass that hands state between sequence segments is not counted.
        # Its arithmetic intensity (flops per algorithmic byte) is below the ridge point of the
        # bf16 matrix peak over HBM (2500 / 8 = 312), so HBM stays its roofline; the matrix-core
        # rate is reported beside it.
        Np = (p.nstate + 31) // 32 * 32
        nch = (p.length + 31) // 32
        mf = p.batch * p.heads * (p.channels // p.heads // 64) * nch * 4 * (4 + Np // 4) * 16384.0
        out["roofline"]["mfma"] = {"flops_per_launch": mf, "achieved_TFLOPs": mf / avg_launch_s / 1e12,
                                   "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
                                   "frac": mf / avg_launch_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                                   "flops_per_byte": mf / nbytes}

    if cpu:
        import oracle

        cores = oracle.default_threads()
        # bounded sample: the whole workload when it is small, else a prefix of its rows
        total_rows = p.batch * p.channels
        budget = 6.0e9  # state-steps (t, n) per repeat: a few seconds on a few dozen cores
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
    return out


def stored_copy_peak():
    """The measured HBM copy rate (GB/s, bytes read + written) from the committed probe summary
    profiles/probe_hbm_copy.txt, if present."""
    path = os.path.join(ROOT, "profiles", "probe_hbm_copy.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("copy_GBps:"):
                try:
                    return float(line.split(":", 1)[1])
                except ValueError:
                    return None
    return None


if __name__ == "__main__":
    main()
