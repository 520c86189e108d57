"""Zero-order hold (SS_ZOH) on the GPU against the oracle with the same option, on every kernel
path: diagonal (one and two channels per wave, with and without state in/out), the scalar-decay
kernels (f32 inputs), the scalar-decay matrix form (bf16, heads of 64) and the decoding step.
Bars as for the exponential-Euler scan (normwise 1e-5 for f32 inputs, 2e-3 for bf16)."""
import dataclasses

import numpy as np
import pytest

import oracle
from conftest import normwise
from gpu_helpers import dev_problem, run_hip, say, to_dev, torch_dev
from selective_state_space_88_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


def zoh(p):
    return dataclasses.replace(p, zoh=True)


CASES = {
    "diag f32 N16": lambda: inputs.random_problem(800, 2, 8, 700, 16, in_dtype="f32"),
    "diag bf16 N7": lambda: inputs.random_problem(801, 1, 12, 333, 7, gate=False),
    "diag f32 two channels per wave": lambda: inputs.random_problem(802, 1, 12288, 64, 4, in_dtype="f32", gate=False),
    "diag raw delta": lambda: inputs.random_problem(803, 1, 8, 500, 16, in_dtype="f32", softplus=False),
    "scalar f32 head-aligned": lambda: inputs.random_problem(804, 1, 128, 400, 32, heads=2, scalar_decay=True,
                                                             in_dtype="f32"),
    "scalar f32 generic": lambda: inputs.random_problem(805, 2, 32, 300, 20, heads=4, scalar_decay=True,
                                                        in_dtype="f32"),
    "matrix bf16": lambda: inputs.random_problem(806, 1, 128, 700, 64, heads=2, scalar_decay=True, gate=False),
    "matrix bf16 segments": lambda: inputs.random_problem(807, 1, 64, 4096, 128, heads=1, scalar_decay=True,
                                                          gate=False),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_zoh_scan(case):
    torch_dev()
    p = zoh(CASES[case]())
    y = run_hip(p)
    ref = oracle.scan_problem(p)
    err = normwise(y, ref)
    # the option changes the result (so the flag reached the kernel)
    euler = oracle.scan_problem(dataclasses.replace(p, zoh=False))
    say("[zoh] %s: normwise %.3e (zoh vs euler %.3e)" % (case, err, normwise(euler, ref)))
    assert normwise(euler, ref) > 10 * TOL[p.in_dtype]
    assert err <= TOL[p.in_dtype], (case, err)


@pytest.mark.parametrize("case", ["diag f32 N16", "matrix bf16 segments", "scalar f32 generic"])
def test_zoh_with_state(case):
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = zoh(CASES[case]())
    h0 = inputs.random_state(90, p.batch, p.channels, p.nstate)
    t = dev_problem(p)
    hf = torch.empty((p.batch, p.channels, p.nstate), device="cuda")
    y = scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], softplus=p.softplus,
                 h_init=to_dev(h0), h_final=hf, zoh=True)
    torch.cuda.synchronize()
    ry, rh = oracle.scan_problem(p, h0=h0.reshape(-1, p.nstate).astype(np.float64), return_state=True)
    assert normwise(y.cpu().numpy(), ry) <= TOL[p.in_dtype]
    assert normwise(hf.cpu().numpy().reshape(-1, p.nstate), rh) <= TOL[p.in_dtype]


@pytest.mark.parametrize("case", ["diag f32 N16", "diag bf16 N7", "scalar f32 generic", "matrix bf16"])
def test_zoh_decode_steps(case):
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_step

    p = zoh(inputs.time_slice(CASES[case](), 0, 20))
    h0 = inputs.random_state(91, p.batch, p.channels, p.nstate)
    h = to_dev(h0)
    ys = []
    for step in range(p.length):
        s = dev_problem(inputs.step_slice(p, step))
        ys.append(scan_step(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"], h,
                            softplus=p.softplus, zoh=True))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=-1).cpu().numpy()
    ry, rh = oracle.scan_problem(p, h0=h0.reshape(-1, p.nstate).astype(np.float64), return_state=True)
    assert normwise(y, ry) <= TOL[p.in_dtype]
    assert normwise(h.cpu().numpy().reshape(-1, p.nstate), rh) <= TOL[p.in_dtype]


def test_backward_rejects_zoh():
    torch = torch_dev()
    from selective_state_space_88_amd import scan

    p = inputs.random_problem(808, 1, 8, 64, 16)
    t = dev_problem(p)
    dy = torch.zeros((1, 8, 64), device="cuda")
    g = {k: torch.empty(v.shape, device="cuda") for k, v in
         dict(du=t["u"], ddelta=t["delta"], dA=t["A"], dB=t["B"], dC=t["C"], dD=t["D"], dz=t["z"]).items()}
    d = scan.describe
    rc = scan.call_bwd(d(t["u"]), d(t["delta"]), d(t["A"]), d(t["B"]), d(t["C"]), d(t["D"]), d(t["z"]),
                       d(t["delta_bias"]), scan.SS_DELTA_SOFTPLUS | scan.SS_Z_GATE_SILU | scan.SS_ZOH, d(dy),
                       d(g["du"]), d(g["ddelta"]), d(g["dA"]), d(g["dB"]), d(g["dC"]), d(g["dD"]), d(g["dz"]), None,
                       None)
    assert rc == -6
