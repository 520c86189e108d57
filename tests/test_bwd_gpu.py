"""Backward (ss_scan_bwd) on the GPU against the CPU oracle's float64 gradients.

Metric: normwise max|g - g_ref| / max|g_ref| per gradient.  Bars: 2e-3 for bf16 inputs, as for
y; 2e-5 for f32 inputs (the gradients of A, B, C and D are sums of up to L * channels f32
products -- the forward's bar 1e-5 doubled for that summation).
"""
import numpy as np
import pytest

import oracle
from conftest import normwise
from gpu_helpers import dev_problem, say, to_dev, torch_dev
from selective_state_space_88_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 2e-3}
NAMES = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias")


def check_bwd(p, label, seed=11, dy_dtype=None):
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_bwd

    dy = inputs.seeded_normal(seed, (p.batch, p.channels, p.length))
    t = dev_problem(p)
    dyt = to_dev(dy)
    if dy_dtype is not None:
        dyt = dyt.to(dy_dtype)
        dy = dyt.float().cpu().numpy()
    say("[bwd] %s: batch=%d channels=%d L=%d N=%d groups=%d dtype=%s gate=%s softplus=%s" % (
        label, p.batch, p.channels, p.length, p.nstate, p.groups, p.in_dtype, p.gate, p.softplus))
    g = scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], dyt,
                 softplus=p.softplus)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd_problem(p, dy)
    errs = {}
    for k in NAMES:
        if ref[k] is None:
            assert g[k] is None, k
            continue
        got = g[k].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), k
        errs[k] = normwise(got, ref[k])
    say("[bwd] %s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())))
    bad = {k: v for k, v in errs.items() if v > TOL[p.in_dtype]}
    assert not bad, (label, bad)


@pytest.mark.parametrize("N,L,dtype,gate", [(16, 1500, "bf16", True), (7, 333, "f32", False),
                                            (16, 512, "f32", True), (64, 1100, "bf16", False),
                                            (1, 40, "f32", True), (128, 600, "bf16", True)])
def test_gradients(N, L, dtype, gate):
    check_bwd(inputs.random_problem(700 + N + L, 2, 8, L, N, in_dtype=dtype, gate=gate),
              "N=%d L=%d %s gate=%s" % (N, L, dtype, gate))


@pytest.mark.parametrize("opts", [dict(softplus=False), dict(with_D=False), dict(with_bias=False),
                                  dict(groups=2)])
def test_gradient_options(opts):
    check_bwd(inputs.random_problem(720, 1, 16, 700, 16, in_dtype="f32", **opts), "options %s" % opts)


def test_workload_1_layer_shapes_small_batch():
    """The Mamba-130M-like layer's shapes and distributions (S4D-real A, dt log-uniform) at batch 1
    and 256 channels: windows in reverse with carries across 4 windows."""
    p = inputs.make(1, batch=1, channels=256)
    check_bwd(p, "workload-1 shapes, 1x256x2048")


def test_bf16_upstream_gradient():
    torch = torch_dev()
    check_bwd(inputs.random_problem(730, 1, 8, 300, 16), "dy bf16", dy_dtype=torch.bfloat16)


@pytest.mark.parametrize("case", ["scalar N16 bf16", "scalar N128 f32", "scalar head of 4", "scalar head of 2",
                                  "diag heads of 4", "diag heads of 2", "scalar groups 2", "scalar no bias"])
def test_gradients_with_heads(case):
    """Step sizes shared by a head's channels (delta [batch, heads, L]) with a diagonal A, and the
    scalar decay A [heads] with D per head: per-head gradients summed over the head's channels
    (through LDS when the block's 4 channels share a head, by per-channel atomics otherwise)."""
    mk = {
        "scalar N16 bf16": lambda: inputs.random_problem(750, 2, 128, 700, 16, heads=2, scalar_decay=True),
        "scalar N128 f32": lambda: inputs.random_problem(751, 1, 64, 600, 128, heads=1, scalar_decay=True,
                                                         in_dtype="f32", gate=False),
        "scalar head of 4": lambda: inputs.random_problem(752, 2, 16, 530, 8, heads=4, scalar_decay=True,
                                                          in_dtype="f32"),
        "scalar head of 2": lambda: inputs.random_problem(753, 1, 8, 300, 5, heads=4, scalar_decay=True,
                                                          in_dtype="f32"),
        "diag heads of 4": lambda: inputs.random_problem(754, 2, 16, 777, 16, heads=4, in_dtype="f32"),
        "diag heads of 2": lambda: inputs.random_problem(755, 1, 8, 300, 4, heads=4, in_dtype="f32", gate=False),
        "scalar groups 2": lambda: inputs.random_problem(756, 1, 32, 520, 16, heads=4, groups=2, scalar_decay=True,
                                                         in_dtype="f32"),
        "scalar no bias": lambda: inputs.random_problem(757, 1, 16, 400, 16, heads=2, scalar_decay=True,
                                                        in_dtype="f32", softplus=False, with_D=False),
    }
    check_bwd(mk[case](), case)


def test_workload_4_layer_shapes_reduced():
    """The scalar-decay multi-head layer's distributions (A_h = -U(1, 16), N 128, heads of 64
    channels, no gate) at 4 heads and L 2048."""
    check_bwd(inputs.make(4, batch=1, heads=4, length=2048), "workload-4 shapes, 1x(4x64)x2048")


MATRIX_CASES = {
    # scalar decay, no gate, heads and groups in whole 64-channel slabs: the chunked matrix form
    "N16 bf16 L700": lambda: inputs.random_problem(760, 2, 128, 700, 16, heads=2, scalar_decay=True, gate=False),
    "N128 f32 L600": lambda: inputs.random_problem(761, 1, 64, 600, 128, heads=1, scalar_decay=True,
                                                   in_dtype="f32", gate=False),
    "N33 f32 ragged": lambda: inputs.random_problem(762, 2, 64, 97, 33, heads=1, scalar_decay=True, in_dtype="f32",
                                                    gate=False),
    "N1 one step": lambda: inputs.random_problem(763, 1, 64, 1, 1, heads=1, scalar_decay=True, in_dtype="f32",
                                                 gate=False),
    "N64 L31": lambda: inputs.random_problem(764, 1, 128, 31, 64, heads=2, scalar_decay=True, in_dtype="f32",
                                             gate=False),
    "two slabs per head": lambda: inputs.random_problem(765, 1, 256, 300, 16, heads=2, scalar_decay=True,
                                                        in_dtype="f32", gate=False),
    "two groups": lambda: inputs.random_problem(766, 1, 256, 200, 32, heads=4, groups=2, scalar_decay=True,
                                                in_dtype="f32", gate=False),
    "no softplus, no D": lambda: inputs.random_problem(767, 1, 128, 333, 16, heads=2, scalar_decay=True,
                                                       in_dtype="f32", gate=False, softplus=False, with_D=False),
    "no bias": lambda: inputs.random_problem(768, 1, 64, 257, 16, heads=1, scalar_decay=True, in_dtype="f32",
                                             gate=False, with_bias=False),
    "long decay-free": lambda: inputs.random_problem(769, 1, 64, 1500, 16, heads=1, scalar_decay=True,
                                                     in_dtype="f32", gate=False, dt=(1e-4, 1e-3)),
}


@pytest.mark.parametrize("case", sorted(MATRIX_CASES))
def test_matrix_backward(case):
    """The scalar-decay backward in the chunked matrix form (fp32 MFMA): ragged chunk tails, N from
    1 to 128 (padded to 32, 64, 128), heads of two slabs (ddelta summed by atomics), two B/C groups,
    D per head, softplus off, slow decays (states carried across many chunks)."""
    check_bwd(MATRIX_CASES[case](), "matrix " + case)


GATED_MATRIX_CASES = {
    # scalar decay with a gate, heads and groups in whole 64-channel slabs: the forward without
    # the gate recomputes y0, an elementwise pass gives dz and dy0 = dy s(z), then the matrix form
    "N16 bf16 L700": lambda: inputs.random_problem(780, 2, 128, 700, 16, heads=2, scalar_decay=True, gate=True),
    "N128 f32 L600": lambda: inputs.random_problem(781, 1, 64, 600, 128, heads=1, scalar_decay=True,
                                                   in_dtype="f32", gate=True),
    "N33 f32 ragged": lambda: inputs.random_problem(782, 2, 64, 97, 33, heads=1, scalar_decay=True, in_dtype="f32",
                                                    gate=True),
    "two groups": lambda: inputs.random_problem(783, 1, 256, 200, 32, heads=4, groups=2, scalar_decay=True,
                                                in_dtype="f32", gate=True),
    "no softplus, no D": lambda: inputs.random_problem(784, 1, 128, 333, 16, heads=2, scalar_decay=True,
                                                       in_dtype="f32", gate=True, softplus=False, with_D=False),
    "N64 bf16 L1": lambda: inputs.random_problem(785, 1, 64, 1, 64, heads=1, scalar_decay=True, gate=True),
}


MATRIX_SEGMENT_CASES = {
    # few (batch, head, slab) rows and long sequences: the matrix form's reverse pass is cut into
    # sequence segments (at least 8 chunks of 32 steps each), each started from the R that the
    # segments to its right hand over
    "N128 bf16 L5000, 19 segments": lambda: inputs.random_problem(790, 1, 64, 5000, 128, heads=1, scalar_decay=True,
                                                                 gate=False),
    "N33 f32 ragged L4001, 15 segments": lambda: inputs.random_problem(791, 1, 64, 4001, 33, heads=1,
                                                                      scalar_decay=True, in_dtype="f32", gate=False),
    "gated N64 bf16 two heads L3000": lambda: inputs.random_problem(792, 1, 128, 3000, 64, heads=2, scalar_decay=True,
                                                                   gate=True),
    "N16 f32 two batches L2600": lambda: inputs.random_problem(793, 2, 64, 2600, 16, heads=1, scalar_decay=True,
                                                               in_dtype="f32", gate=False),
}


@pytest.mark.parametrize("case", sorted(MATRIX_SEGMENT_CASES))
def test_matrix_backward_sequence_segments(case):
    check_bwd(MATRIX_SEGMENT_CASES[case](), "matrix segments: " + case)


FORWARD_SEGMENT_CASES = {
    # one batch row, L a multiple of two segments of 1024-step windows (at least three each): the
    # recompute before the gate runs as 2 sequence segments (pre-pass in 16 and 8 pieces) and
    # writes the checkpoints of both into the whole sequence's layout
    "gated bf16 N16 L16384": lambda: inputs.random_problem(7306, 1, 8, 16384, 16, gate=True),
    "gated bf16 N24 L12288": lambda: inputs.random_problem(7307, 1, 4, 12288, 24, gate=True),
}


@pytest.mark.parametrize("case", sorted(FORWARD_SEGMENT_CASES))
def test_gated_backward_recompute_in_segments(case):
    """A gated one-row layer: the backward's recompute of the output before the gate takes the
    forward's sequence segments (each started from the state the combine hands it), and its
    checkpoints feed the per-channel backward."""
    check_bwd(FORWARD_SEGMENT_CASES[case](), "forward segments: " + case)


UNGATED_SLOTS_CASES = {
    # one batch row without a gate on the window-slot path: the forward (into a scratch output)
    # stores the checkpoints instead of the checkpoint pass; on 2 sequence segments, and
    # unsegmented with a partial last window
    "bf16 N16 L16384, segments": lambda: inputs.random_problem(7308, 1, 8, 16384, 16, gate=False),
    "bf16 N12 L5000 ragged": lambda: inputs.random_problem(7309, 1, 8, 5000, 12, gate=False),
    "two batches bf16 N16 L4096": lambda: inputs.random_problem(7310, 2, 4, 4096, 16, gate=False),
}


@pytest.mark.parametrize("case", sorted(UNGATED_SLOTS_CASES))
def test_ungated_backward_checkpoints_from_the_forward(case):
    check_bwd(UNGATED_SLOTS_CASES[case](), "ungated, checkpoints from the forward: " + case)


def test_sequence_segments_bf16_upstream_gradient():
    """dy in bf16 through both segmented layouts (the pre-passes read dy in its own type)."""
    torch = torch_dev()
    check_bwd(inputs.random_problem(7305, 1, 8, 12000, 16, gate=True), "segments, bf16 dy", dy_dtype=torch.bfloat16)
    check_bwd(inputs.random_problem(794, 1, 64, 4096, 64, heads=1, scalar_decay=True, gate=False),
              "matrix segments, bf16 dy", dy_dtype=torch.bfloat16)


@pytest.mark.parametrize("case", sorted(GATED_MATRIX_CASES))
def test_gated_matrix_backward(case):
    check_bwd(GATED_MATRIX_CASES[case](), "gated matrix " + case)


@pytest.mark.parametrize("case", ["slots", "one channel per wave", "two channels per wave"])
def test_gated_backward_checkpoints_from_the_forward(case):
    """A gated diagonal layer's backward takes its checkpoints (the state every 512 steps) from
    the forward that recomputes the output before the gate: from the window-slot kernel (few
    rows, at least three 1024-step windows; a partial last window), from one channel per wave
    (1024-step windows: the window's start and 512 steps in) and from two channels per wave
    (512-step windows)."""
    p = {"slots": lambda: inputs.random_problem(790, 1, 8, 4 * 1024 + 264, 16, gate=True),
         "one channel per wave": lambda: inputs.random_problem(791, 2, 8, 2048 + 520, 12, gate=True, in_dtype="f32"),
         "two channels per wave": lambda: inputs.random_problem(792, 1, 4608, 1024 + 96, 6, gate=True)}[case]()
    check_bwd(p, "gated checkpoints from the forward: " + case)


def test_gated_backward_checkpoints_under_timing_stress():
    """The window-slot forward that stores the checkpoints, run with SS_PERTURB (every wave
    sleeps a pseudo-random time at each step): the gradients still match the oracle."""
    import os

    os.environ["SS_PERTURB"] = "7"
    try:
        check_bwd(inputs.random_problem(793, 1, 8, 5 * 1024 + 264, 16, gate=True),
                  "gated checkpoints from the window slots, timing stress")
    finally:
        del os.environ["SS_PERTURB"]


def test_gated_matrix_backward_bf16_dy():
    torch = torch_dev()
    check_bwd(inputs.random_problem(786, 1, 128, 400, 16, heads=2, scalar_decay=True, gate=True),
              "gated matrix dy bf16", dy_dtype=torch.bfloat16)


def test_matrix_backward_bf16_dy():
    torch = torch_dev()
    check_bwd(inputs.random_problem(770, 1, 128, 400, 16, heads=2, scalar_decay=True, gate=False), "matrix dy bf16",
              dy_dtype=torch.bfloat16)


SEGMENT_CASES = {
    # (rows of 8-channel blocks, windows of 512 steps): 1 block, 40 windows -> 8 segments of 5
    "gated bf16 N16": lambda: inputs.random_problem(7301, 1, 8, 20000, 16, gate=True),
    # 2 blocks, 20 windows (ragged last window) -> 5 segments of 4
    "f32 N7 ragged": lambda: inputs.random_problem(7302, 1, 16, 10001, 7, in_dtype="f32", gate=False),
    # scalar decay per head on the per-channel kernel (f32), 32 states: 12 windows -> 3 segments
    "scalar heads of 4 f32 N32": lambda: inputs.random_problem(7303, 1, 8, 6000, 32, heads=2, scalar_decay=True,
                                                               in_dtype="f32", gate=False),
    # two B/C groups (2 blocks), 18 windows -> 4 segments of 5 (the last of 3)
    "two groups bf16 N16": lambda: inputs.random_problem(7304, 1, 16, 9000, 16, groups=2, gate=True),
}


@pytest.mark.parametrize("case", sorted(SEGMENT_CASES))
def test_gradients_sequence_segments(case):
    """Few rows with long sequences: the per-channel backward cuts each row into sequence
    segments (enough for two 8-channel blocks per CU, each at least 4 windows of 512 steps), every
    segment started from the adjoint that the segments to its right hand over."""
    check_bwd(SEGMENT_CASES[case](), "segments: " + case)


@pytest.mark.parametrize("case", ["12 channels", "two groups of 4", "heads of 4 in groups of 12"])
def test_gradients_partial_channel_blocks(case):
    """The per-channel kernel takes 8 channels of a group per block: groups of 4 mod 8 channels leave
    the last block's last 4 waves without a channel (they must contribute nothing)."""
    mk = {
        "12 channels": lambda: inputs.random_problem(780, 2, 12, 530, 16, in_dtype="f32"),
        "two groups of 4": lambda: inputs.random_problem(781, 1, 8, 300, 8, groups=2, in_dtype="f32"),
        "heads of 4 in groups of 12": lambda: inputs.random_problem(782, 1, 12, 400, 16, heads=3, in_dtype="f32",
                                                                    gate=False),
    }
    check_bwd(mk[case](), case)


def _compare(g, ref, pairs, label, tol):
    errs = {}
    for name, got_ix, ref_key in pairs:
        if ref[ref_key] is None:
            continue
        got = g[name][got_ix].cpu().numpy().astype(np.float64)
        errs[name] = normwise(got, ref[ref_key])
    say("[bwd] %s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())))
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, (label, bad)


def test_workload_1_full_size_sampled_channels():
    """The 130M-class layer at full size (8x1536x2048, N 16, gate) in the launch the benchmark times;
    the per-channel gradients (du, ddelta, dz, dA, dD, ddelta_bias) of 6 sampled channels against
    the oracle run on those channels alone (they depend only on their own inputs and the shared B, C)."""
    import dataclasses

    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_bwd

    p = inputs.make(1)
    dy = inputs.seeded_normal(12, (p.batch, p.channels, p.length))
    t = dev_problem(p)
    g = scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], to_dev(dy),
                 softplus=p.softplus)
    torch.cuda.synchronize()
    ch = np.array(sorted({0, p.channels - 1, 700} | set(np.random.default_rng(5).choice(p.channels, 3, False))))
    sub = dataclasses.replace(p, channels=len(ch), heads=len(ch), u=p.u[:, ch], delta=p.delta[:, ch], z=p.z[:, ch],
                              A=p.A[ch], D=p.D[ch], delta_bias=p.delta_bias[ch])
    ref = oracle.scan_bwd_problem(sub, np.ascontiguousarray(dy[:, ch]))
    c = torch.as_tensor(ch, device="cuda")
    pairs = [("du", (slice(None), c), "du"), ("ddelta", (slice(None), c), "ddelta"), ("dz", (slice(None), c), "dz"),
             ("dA", c, "dA"), ("dD", c, "dD"), ("ddelta_bias", c, "ddelta_bias")]
    _compare(g, ref, pairs, "workload 1 full size, channels %s" % ch.tolist(), TOL["bf16"])


def test_workload_4_gated_full_size_sampled_heads():
    """The scalar-decay multi-head layer at full size with a silu gate on z: the composed
    gated path (forward recompute, gate pass, matrix-form backward); du, dz, ddelta, dA, dD and
    ddelta_bias of 2 sampled heads against the oracle run on those heads alone."""
    import dataclasses

    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_bwd

    p = inputs.make(4, gate=True)
    P = p.channels // p.heads
    dy = inputs.seeded_normal(14, (p.batch, p.channels, p.length))
    say("[bwd] workload 4 gated full size: batch=%d channels=%d L=%d N=%d" % (p.batch, p.channels, p.length,
                                                                           p.nstate))
    t = dev_problem(p)
    g = scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], to_dev(dy),
                 softplus=p.softplus)
    torch.cuda.synchronize()
    hs = np.array([3, 79])
    ch = np.concatenate([np.arange(h * P, (h + 1) * P) for h in hs])
    sub = dataclasses.replace(p, channels=len(ch), heads=len(hs), u=p.u[:, ch], delta=p.delta[:, hs],
                              A=p.A[hs], D=p.D[hs], delta_bias=p.delta_bias[hs], z=p.z[:, ch])
    ref = oracle.scan_bwd_problem(sub, np.ascontiguousarray(dy[:, ch]))
    c = torch.as_tensor(ch, device="cuda")
    h = torch.as_tensor(hs, device="cuda")
    pairs = [("du", (slice(None), c), "du"), ("dz", (slice(None), c), "dz"), ("ddelta", (slice(None), h), "ddelta"),
             ("dA", h, "dA"), ("dD", h, "dD"), ("ddelta_bias", h, "ddelta_bias")]
    _compare(g, ref, pairs, "workload 4 gated full size, heads %s" % hs.tolist(), TOL["bf16"])


def test_workload_4_full_size_sampled_heads():
    """The scalar-decay multi-head layer at full size (2x(80x64)x8192, N 128) through the matrix-form
    backward; the per-head gradients (du of the head's channels, ddelta, dA, dD, ddelta_bias) of 2
    sampled heads against the oracle run on those heads alone."""
    import dataclasses

    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_bwd

    p = inputs.make(4)
    P = p.channels // p.heads
    dy = inputs.seeded_normal(13, (p.batch, p.channels, p.length))
    t = dev_problem(p)
    g = scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], to_dev(dy),
                 softplus=p.softplus)
    torch.cuda.synchronize()
    hs = np.array([0, 57])
    ch = np.concatenate([np.arange(h * P, (h + 1) * P) for h in hs])
    sub = dataclasses.replace(p, channels=len(ch), heads=len(hs), u=p.u[:, ch], delta=p.delta[:, hs],
                              A=p.A[hs], D=p.D[hs], delta_bias=p.delta_bias[hs])
    ref = oracle.scan_bwd_problem(sub, np.ascontiguousarray(dy[:, ch]))
    c = torch.as_tensor(ch, device="cuda")
    h = torch.as_tensor(hs, device="cuda")
    pairs = [("du", (slice(None), c), "du"), ("ddelta", (slice(None), h), "ddelta"), ("dA", h, "dA"),
             ("dD", h, "dD"), ("ddelta_bias", h, "ddelta_bias")]
    _compare(g, ref, pairs, "workload 4 full size, heads %s" % hs.tolist(), TOL["bf16"])
