"""Parity of the diagonal kernel's two-channels-per-wave layout with bf16 inputs, where the two
states of a pair run one after the other, in every mode (GPU).

The launch takes that layout once the rows outnumber one wave per SIMD (4 x the compute units:
1024 on MI355X); these cases have a little more than that (1100 or 1025 rows), or exactly 1024
(one channel per wave) for the boundary.  Bars as in the other parity tests: normwise 2e-3 for
bf16 inputs, the same for the final state.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from conftest import normwise
from gpu_helpers import dev_problem, run_hip, say, to_dev, torch_dev
from selective_state_space_88_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 2e-3

CASES = {
    # aligned rows, two whole 512-step windows and a partial one; gate on
    "N16 gate": lambda: inputs.random_problem(1200, 1, 1100, 1064, 16),
    # odd N (the last pair's second state absent), unaligned length (element-wise loads)
    "N7 ragged": lambda: inputs.random_problem(1201, 1, 1100, 333, 7, gate=False),
    # one row more than a single round of one channel per wave: the last block's last wave
    # holds one channel
    "1025 rows": lambda: inputs.random_problem(1202, 1, 1025, 600, 16),
    # the boundary itself (one channel per wave)
    "1024 rows": lambda: inputs.random_problem(1203, 2, 512, 600, 16),
    # heads of several channels sharing a step size, two B/C groups
    "heads and groups": lambda: inputs.random_problem(1204, 2, 640, 777, 16, heads=160, groups=2),
    # the largest state (64 pairs: 8 KB of per-pair parameters, two blocks per CU) and an odd one
    "N128": lambda: inputs.random_problem(1205, 1, 1100, 300, 128, gate=False),
    "N33": lambda: inputs.random_problem(1206, 1, 1100, 515, 33),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("mode", ["euler", "zoh", "trapezoid", "zoh+trapezoid"])
def test_split_layout(case, mode):
    torch_dev()
    p = CASES[case]()
    p = dataclasses.replace(p, zoh="zoh" in mode, trapezoid="trapezoid" in mode)
    say("[split] %s %s: batch=%d channels=%d L=%d N=%d heads=%d groups=%d"
        % (case, mode, p.batch, p.channels, p.length, p.nstate, p.heads, p.groups))
    y = run_hip(p)
    ref = oracle.scan_problem(p)
    err = normwise(y, ref)
    say("[split] %s %s: normwise %.3e" % (case, mode, err))
    assert np.all(np.isfinite(y))
    assert err <= TOL, (case, mode, err)


@pytest.mark.parametrize("case", ["N16 gate", "N7 ragged", "1025 rows"])
@pytest.mark.parametrize("mode", ["euler", "zoh", "trapezoid"])
def test_split_layout_with_state(case, mode):
    """h_init in, h_final out through the two-channels-per-wave layout."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = CASES[case]()
    p = dataclasses.replace(p, zoh=mode == "zoh", trapezoid=mode == "trapezoid")
    say("[split] state %s %s: channels=%d L=%d N=%d" % (case, mode, p.channels, p.length, p.nstate))
    h0 = inputs.random_state(91, p.batch, p.channels, p.nstate)
    t = dev_problem(p)
    hf = torch.full((p.batch, p.channels, p.nstate), float("nan"), device="cuda")
    y = scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], softplus=p.softplus,
                 h_init=to_dev(h0), h_final=hf, zoh=p.zoh, trapezoid=p.trapezoid)
    torch.cuda.synchronize()
    ry, rh = oracle.scan_problem(p, h0=h0.reshape(-1, p.nstate).astype(np.float64), return_state=True)
    ey = normwise(y.cpu().numpy().astype(np.float64), ry)
    eh = normwise(hf.cpu().numpy().astype(np.float64).reshape(-1, p.nstate), rh)
    say("[split] state %s %s: y %.3e, final state %.3e" % (case, mode, ey, eh))
    assert ey <= TOL and eh <= TOL, (case, mode, ey, eh)
