"""The exponential-trapezoidal rule (SS_TRAPEZOID) on the GPU against the oracle with the same
option, on every kernel path; with state in/out (a sequence scanned in two pieces through the
carried state h + e/2), decoding steps, and combined with zero-order hold.  Bars as for the
exponential-Euler scan."""
import dataclasses

import numpy as np
import pytest

import oracle
from conftest import normwise
from gpu_helpers import dev_problem, run_hip, say, to_dev, torch_dev
from selective_state_space_88_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


def trap(p, zoh=False):
    return dataclasses.replace(p, trapezoid=True, zoh=zoh)


CASES = {
    "diag f32 N16": lambda: inputs.random_problem(820, 2, 8, 700, 16, in_dtype="f32"),
    "diag bf16 N7": lambda: inputs.random_problem(821, 1, 12, 333, 7, gate=False),
    "diag f32 two channels per wave": lambda: inputs.random_problem(822, 1, 12288, 64, 4, in_dtype="f32", gate=False),
    "scalar f32 head-aligned": lambda: inputs.random_problem(824, 1, 128, 400, 32, heads=2, scalar_decay=True,
                                                             in_dtype="f32"),
    "scalar f32 generic": lambda: inputs.random_problem(825, 2, 32, 300, 20, heads=4, scalar_decay=True,
                                                        in_dtype="f32"),
    "matrix bf16": lambda: inputs.random_problem(826, 1, 128, 700, 64, heads=2, scalar_decay=True, gate=False),
    "matrix bf16 segments": lambda: inputs.random_problem(827, 1, 64, 4096, 128, heads=1, scalar_decay=True,
                                                          gate=False),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_trapezoid_scan(case):
    torch_dev()
    p = trap(CASES[case]())
    y = run_hip(p)
    ref = oracle.scan_problem(p)
    err = normwise(y, ref)
    euler = oracle.scan_problem(dataclasses.replace(p, trapezoid=False))
    say("[trap] %s: normwise %.3e (trapezoid vs euler %.3e)" % (case, err, normwise(euler, ref)))
    assert normwise(euler, ref) > 10 * TOL[p.in_dtype]
    assert err <= TOL[p.in_dtype], (case, err)


@pytest.mark.parametrize("case", ["diag f32 N16", "matrix bf16"])
def test_trapezoid_with_zoh(case):
    torch_dev()
    p = trap(CASES[case](), zoh=True)
    assert normwise(run_hip(p), oracle.scan_problem(p)) <= TOL[p.in_dtype]


@pytest.mark.parametrize("case", ["diag f32 N16", "scalar f32 generic", "matrix bf16 segments"])
def test_trapezoid_in_two_pieces(case):
    """[0, T) then [T, L) from the carried state reproduces one scan (the state convention)."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = trap(CASES[case]())
    T = (p.length * 3) // 7
    outs = []
    h = None
    for piece in (inputs.time_slice(p, 0, T), inputs.time_slice(p, T, p.length)):
        t = dev_problem(piece)
        hf = torch.empty((p.batch, p.channels, p.nstate), device="cuda")
        outs.append(scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                             softplus=p.softplus, h_init=h, h_final=hf, trapezoid=True))
        h = hf
    torch.cuda.synchronize()
    y = torch.cat(outs, dim=-1).cpu().numpy()
    ry, rh = oracle.scan_problem(p, return_state=True)
    assert normwise(y, ry) <= TOL[p.in_dtype]
    assert normwise(h.cpu().numpy().reshape(-1, p.nstate), rh) <= TOL[p.in_dtype]


@pytest.mark.parametrize("case", ["diag f32 N16", "diag bf16 N7", "scalar f32 generic", "matrix bf16"])
def test_trapezoid_decode_steps(case):
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_step

    p = trap(inputs.time_slice(CASES[case](), 0, 20))
    h0 = inputs.random_state(92, p.batch, p.channels, p.nstate)
    h = to_dev(h0)
    ys = []
    for step in range(p.length):
        s = dev_problem(inputs.step_slice(p, step))
        ys.append(scan_step(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"], h,
                            softplus=p.softplus, trapezoid=True))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=-1).cpu().numpy()
    ry, rh = oracle.scan_problem(p, h0=h0.reshape(-1, p.nstate).astype(np.float64), return_state=True)
    assert normwise(y, ry) <= TOL[p.in_dtype]
    assert normwise(h.cpu().numpy().reshape(-1, p.nstate), rh) <= TOL[p.in_dtype]
