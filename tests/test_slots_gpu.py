"""Parity of the diagonal kernel's window-slot layout (GPU): few (batch, channel) rows, each with
three windows of 1024 steps in flight, two states a step, the carried state handed from slot to
slot through LDS.

The launch takes that layout for bf16 inputs with 16-byte aligned rows, L a multiple of 8 and at
least three windows, N >= 5, when the rows fit one wave per SIMD (4 x the compute units: 1024 on
MI355X).  These cases cover the skew (N from 5 to 128, odd and even), lengths around whole rounds of the
three slots and with a partial last window, a last block with fewer than four channels, heads and
groups, every mode, the state in and out, y in bf16, bitwise determinism and causality across
slot boundaries, and a wait between waves forced to run out (reported by ss_check, no hang).
Bars as in the other parity tests: normwise 2e-3 for bf16 inputs, the same for the final state,
plus the per-row and elementwise checks of test_parity_gpu.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from conftest import normwise
from gpu_helpers import dev_problem, run_hip, say, to_dev, torch_dev
from selective_state_space_88_amd import inputs
from test_parity_gpu import diagnostics

pytestmark = pytest.mark.gpu

TOL = 2e-3

CASES = {
    # exactly one round of the three slots
    "N16 3 windows": lambda: inputs.random_problem(1300, 1, 8, 3072, 16),
    # a partial last window (L a multiple of 8, not of 1024), several rounds
    "N16 ragged": lambda: inputs.random_problem(1301, 2, 6, 5 * 1024 + 264, 16),
    # the smallest N with a skew (three steps of two states, skew 1; the last step's second
    # state absent) and others around the skew's bounds
    "N5": lambda: inputs.random_problem(1304, 1, 9, 4 * 1024 + 512, 5),
    "N6": lambda: inputs.random_problem(1302, 1, 5, 4096 + 8, 6),
    "N7": lambda: inputs.random_problem(1303, 1, 4, 7 * 1024, 7, gate=False),
    "N17": lambda: inputs.random_problem(1305, 1, 7, 6 * 1024 + 8, 17),
    "N64": lambda: inputs.random_problem(1306, 1, 4, 3 * 1024 + 1000, 64),
    "N128": lambda: inputs.random_problem(1307, 1, 3, 4 * 1024, 128, gate=False),
    # heads of several channels sharing a step size, two B/C groups of 6 (blocks of 4 + 2)
    "heads and groups": lambda: inputs.random_problem(1308, 2, 12, 3 * 1024 + 16, 16, heads=3, groups=2),
    # many windows per slot
    "long": lambda: inputs.random_problem(1309, 1, 2, 40 * 1024 + 8, 16),
}


def check(p, label):
    y = run_hip(p)
    ref = oracle.scan_problem(p)
    err = normwise(y, ref)
    d = diagnostics(y, ref, p.length, TOL)
    say("[slots] %s: normwise %.3e, worst row %.3e, elementwise excess %.3e" % (label, err, d["worst_row"],
                                                                                 d["excess"]))
    assert np.all(np.isfinite(y))
    assert err <= TOL and d["worst_row"] <= TOL and d["excess"] <= 0, (label, err, d)


@pytest.mark.parametrize("case", sorted(CASES))
def test_slots_layout(case):
    torch_dev()
    p = CASES[case]()
    say("[slots] %s: batch=%d channels=%d L=%d N=%d heads=%d groups=%d gate=%s"
        % (case, p.batch, p.channels, p.length, p.nstate, p.heads, p.groups, p.gate))
    check(p, case)


@pytest.mark.parametrize("opts", [dict(softplus=False), dict(with_D=False), dict(with_bias=False)])
def test_slots_options(opts):
    torch_dev()
    p = inputs.random_problem(1310, 1, 4, 3 * 1024 + 8, 16, **opts)
    say("[slots] options %s" % opts)
    check(p, "options %s" % opts)


@pytest.mark.parametrize("case", ["N16 ragged", "N5", "N128"])
@pytest.mark.parametrize("mode", ["zoh", "trapezoid", "zoh+trapezoid"])
def test_slots_modes(case, mode):
    torch_dev()
    p = dataclasses.replace(CASES[case](), zoh="zoh" in mode, trapezoid="trapezoid" in mode)
    say("[slots] %s %s: channels=%d L=%d N=%d" % (case, mode, p.channels, p.length, p.nstate))
    check(p, "%s %s" % (case, mode))


@pytest.mark.parametrize("case", ["N16 ragged", "N5", "heads and groups"])
@pytest.mark.parametrize("mode", ["euler", "trapezoid"])
def test_slots_with_state(case, mode):
    """h_init in, h_final out: the first window of slot 0 starts from h_init, and the final state
    is the carried word after the last window (whichever slot ran it)."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = dataclasses.replace(CASES[case](), trapezoid=mode == "trapezoid")
    say("[slots] state %s %s: channels=%d L=%d N=%d" % (case, mode, p.channels, p.length, p.nstate))
    h0 = inputs.random_state(92, p.batch, p.channels, p.nstate)
    t = dev_problem(p)
    hf = torch.full((p.batch, p.channels, p.nstate), float("nan"), device="cuda")
    y = scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], softplus=p.softplus,
                 h_init=to_dev(h0), h_final=hf, trapezoid=p.trapezoid)
    torch.cuda.synchronize()
    ry, rh = oracle.scan_problem(p, h0=h0.reshape(-1, p.nstate).astype(np.float64), return_state=True)
    ey = normwise(y.cpu().numpy().astype(np.float64), ry)
    eh = normwise(hf.cpu().numpy().astype(np.float64).reshape(-1, p.nstate), rh)
    say("[slots] state %s %s: y %.3e, final state %.3e" % (case, mode, ey, eh))
    assert ey <= TOL and eh <= TOL, (case, mode, ey, eh)


def test_slots_bf16_output():
    torch = torch_dev()
    p = CASES["N16 ragged"]()
    say("[slots] bf16 y: channels=%d L=%d" % (p.channels, p.length))
    y = run_hip(p, out_dtype=torch.bfloat16)
    ref = oracle.scan_problem(p)
    excess = np.max(np.abs(y - ref) - (2.0 ** -8 * np.abs(ref) + 2e-3 * np.max(np.abs(ref))))
    say("[slots] bf16 y: max excess over bound %.3e" % excess)
    assert excess <= 0


def test_slots_deterministic_and_causal():
    """Bitwise identical on repeat; a change at step t0 leaves every earlier output bitwise
    unchanged, with t0 inside a window, on a window edge and on the edge between two rounds of
    the slots."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = inputs.make(3, batch=1, channels=8, length=8 * 1024)
    say("[slots] determinism/causality: channels=%d L=%d" % (p.channels, p.length))
    t = dev_problem(p)
    run = lambda u: scan_fwd(u, t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"]).cpu().numpy()
    y1, y2 = run(t["u"]), run(t["u"])
    assert np.array_equal(y1, y2)
    for t0 in (1000, 1024, 2047, 3072, 5000):
        u2 = t["u"].clone()
        u2[..., t0] = u2[..., t0] + 1.0
        y3 = run(u2)
        assert np.array_equal(y3[..., :t0], y1[..., :t0]), t0
        assert not np.array_equal(y3[..., t0], y1[..., t0]), t0


def test_slots_pieces_compose():
    """A long row scanned in two calls with the state carried equals one call (both calls take
    the slot layout)."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = inputs.make(3, batch=1, channels=4, length=9 * 1024)
    T = 4 * 1024 + 512
    say("[slots] pieces: channels=%d L=%d split at %d" % (p.channels, p.length, T))
    whole = dev_problem(p)
    y = scan_fwd(whole["u"], whole["delta"], whole["A"], whole["B"], whole["C"], whole["D"], whole["z"],
                 whole["delta_bias"]).cpu().numpy()
    a, b = dev_problem(inputs.time_slice(p, 0, T)), dev_problem(inputs.time_slice(p, T, p.length))
    h1 = torch.empty((1, 4, p.nstate), device="cuda")
    h2 = torch.empty((1, 4, p.nstate), device="cuda")
    ya = scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["delta_bias"], h_final=h1)
    yb = scan_fwd(b["u"], b["delta"], b["A"], b["B"], b["C"], b["D"], b["z"], b["delta_bias"], h_init=h1, h_final=h2)
    torch.cuda.synchronize()
    ycat = np.concatenate([ya.cpu().numpy(), yb.cpu().numpy()], axis=-1)
    err = normwise(ycat, y)
    say("[slots] pieces: normwise against one call %.3e" % err)
    assert err <= 1e-5


def test_slots_forced_wait_failure_is_reported():
    """SS_SPIN_LIMIT=0 makes every wait between waves give up at its first unsuccessful poll:
    the kernel still ends (its waves go on), ss_check reports SS_ERR_DEADLOCK once, and the next
    call with the normal bound is correct and reports nothing."""
    import os

    torch = torch_dev()
    from selective_state_space_88_amd import scan

    p = inputs.make(3, batch=1, channels=64, length=32 * 1024)
    say("[slots] forced wait failure: channels=%d L=%d" % (p.channels, p.length))
    t = dev_problem(p)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    stream = torch.cuda.current_stream().cuda_stream
    assert scan.check(stream) == 0
    os.environ["SS_SPIN_LIMIT"] = "0"
    try:
        for _ in range(3):
            scan.scan_fwd(*args, stream=stream)
        rc = scan.check(stream)
    finally:
        del os.environ["SS_SPIN_LIMIT"]
    say("[slots] forced wait failure: ss_check %d" % rc)
    assert rc == -9
    assert scan.check(stream) == 0          # the record was cleared
    y = scan.scan_fwd(*args, stream=stream)
    assert scan.check(stream) == 0
    ref = oracle.scan_problem(p, rows=np.array([0, 63]))
    err = normwise(y.cpu().numpy().reshape(-1, p.length)[[0, 63]], ref)
    say("[slots] after the forced failure: normwise %.3e" % err)
    assert err <= TOL


@pytest.mark.parametrize("case", ["N16 ragged", "N5", "N17", "N128", "heads and groups"])
def test_slots_timing_stress(case):
    """SS_PERTURB=<seed> makes every wave sleep a pseudo-random time at each step (now and then
    a whole step), so the waves reach their waits in orders the normal run rarely produces: the
    output stays bitwise that of the normal run, for three seeds, and no wait runs out."""
    import os

    torch = torch_dev()
    from selective_state_space_88_amd import scan

    p = CASES[case]()
    say("[slots] timing stress %s: channels=%d L=%d N=%d" % (case, p.channels, p.length, p.nstate))
    t = dev_problem(p)
    y0 = run_hip(p, dev=t)
    for seed in (1, 2, 3):
        os.environ["SS_PERTURB"] = str(seed)
        try:
            y = run_hip(p, dev=t)
        finally:
            del os.environ["SS_PERTURB"]
        same = np.array_equal(y, y0)
        say("[slots] timing stress %s seed %d: bitwise equal %s" % (case, seed, same))
        assert same, (case, seed)
    assert scan.check(torch.cuda.current_stream().cuda_stream) == 0


def test_slots_stable_over_100_runs():
    """100 launches on the same inputs give bitwise the same y (the hand-over between slots has
    no order-dependent arithmetic)."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = inputs.make(3, batch=1, channels=64, length=16 * 1024)
    say("[slots] 100 runs: channels=%d L=%d" % (p.channels, p.length))
    t = dev_problem(p)
    first = scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    y = torch.empty_like(first)
    bad = 0
    for _ in range(99):
        scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], y=y)
        bad += int(not torch.equal(y, first))
    torch.cuda.synchronize()
    say("[slots] 100 runs: %d differ from the first" % bad)
    assert bad == 0
