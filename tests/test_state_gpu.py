"""State in / out on the GPU: ss_scan_fwd_state (initial and final state) and ss_scan_step (one
decoding step), against the CPU oracle started from the same state.

Bars as in test_parity_gpu.py (normwise 1e-5 for f32 inputs, 2e-3 for bf16 inputs), for y and
for the final state alike.  Every kernel path is covered: the diagonal kernel, the scalar-decay
kernels (per-step, for f32 inputs: head-aligned and generic) and the scalar-decay matrix form
(bf16 inputs, with and without sequence segments).
"""
import numpy as np
import pytest

import oracle
from conftest import normwise
from gpu_helpers import dev_problem, say, to_dev, torch_dev
from selective_state_space_88_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}

CASES = {
    "diag bf16 N16": lambda: inputs.random_problem(900, 2, 24, 1500, 16),
    "diag f32 N7 ragged": lambda: inputs.random_problem(901, 1, 12, 333, 7, in_dtype="f32", gate=False),
    "scalar f32 head-aligned": lambda: inputs.random_problem(902, 1, 128, 700, 32, heads=2, scalar_decay=True,
                                                             in_dtype="f32"),
    "scalar f32 generic": lambda: inputs.random_problem(903, 2, 32, 300, 20, heads=4, scalar_decay=True,
                                                        in_dtype="f32"),
    "matrix bf16": lambda: inputs.random_problem(904, 1, 128, 500, 64, heads=2, scalar_decay=True, gate=False),
    "matrix bf16 segments": lambda: inputs.random_problem(905, 1, 64, 4096, 128, heads=1, scalar_decay=True,
                                                          gate=False),
}


def run_state(p, h0, want_final=True, dev=None):
    """y and the final state from ss_scan_fwd_state (float64 numpy)."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    t = dev if dev is not None else dev_problem(p)
    hi = None if h0 is None else to_dev(h0)
    hf = torch.full((p.batch, p.channels, p.nstate), float("nan"), dtype=torch.float32, device="cuda") \
        if want_final else None
    y = scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                 softplus=p.softplus, h_init=hi, h_final=hf)
    torch.cuda.synchronize()
    return (y.cpu().numpy().astype(np.float64),
            None if hf is None else hf.cpu().numpy().astype(np.float64))


def oracle_state(p, h0):
    h = None if h0 is None else h0.reshape(-1, p.nstate).astype(np.float64)
    y, hf = oracle.scan_problem(p, h0=h, return_state=True)
    return y, hf.reshape(p.batch, p.channels, p.nstate)


@pytest.mark.parametrize("case", sorted(CASES))
def test_initial_and_final_state(case):
    p = CASES[case]()
    h0 = inputs.random_state(77, p.batch, p.channels, p.nstate)
    say("[state] %s: batch=%d channels=%d L=%d N=%d heads=%d dtype=%s" % (case, p.batch, p.channels, p.length,
                                                                          p.nstate, p.heads, p.in_dtype))
    y, hf = run_state(p, h0)
    ry, rh = oracle_state(p, h0)
    ey, eh = normwise(y, ry), normwise(hf, rh)
    say("[state] %s: y %.3e, final state %.3e" % (case, ey, eh))
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
    assert ey <= TOL[p.in_dtype] and eh <= TOL[p.in_dtype], (case, ey, eh)


@pytest.mark.parametrize("case", ["diag bf16 N16", "scalar f32 generic", "matrix bf16 segments"])
def test_final_state_from_zero(case):
    """Without h_init the scan starts at zero (as ss_scan_fwd) and still reports its final state."""
    p = CASES[case]()
    y, hf = run_state(p, None)
    ry, rh = oracle_state(p, None)
    assert normwise(y, ry) <= TOL[p.in_dtype] and normwise(hf, rh) <= TOL[p.in_dtype]


@pytest.mark.parametrize("case", ["diag bf16 N16", "scalar f32 head-aligned", "matrix bf16 segments"])
def test_chunked_prefill_composes(case):
    """Scanning [0, T) and then [T, L) from the carried state reproduces one scan over [0, L)
    (the segment-composition property of the recurrence, on the GPU)."""
    p = CASES[case]()
    T = (p.length * 3) // 7
    first, second = inputs.time_slice(p, 0, T), inputs.time_slice(p, T, p.length)
    y1, h1 = run_state(first, None)
    y2, h2 = run_state(second, h1.astype(np.float32))
    ry, rh = oracle_state(p, None)
    e = normwise(np.concatenate([y1, y2], axis=-1), ry)
    say("[state] prefill %s split at %d: y %.3e, state %.3e" % (case, T, e, normwise(h2, rh)))
    assert e <= TOL[p.in_dtype] and normwise(h2, rh) <= TOL[p.in_dtype]


def test_zero_length_copies_the_state():
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_fwd

    p = inputs.time_slice(CASES["diag bf16 N16"](), 0, 0)
    t = dev_problem(p)
    h0 = inputs.random_state(5, p.batch, p.channels, p.nstate)
    for init in (h0, None):
        hf = torch.full((p.batch, p.channels, p.nstate), float("nan"), device="cuda")
        scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                 h_init=None if init is None else to_dev(init), h_final=hf)
        torch.cuda.synchronize()
        want = np.zeros_like(h0) if init is None else h0
        assert np.array_equal(hf.cpu().numpy(), want)


# ---------------------------------------------------------------- decoding steps


def run_steps(p, h0, steps, out_dtype=None):
    """y [batch, channels, steps] and the final state from ss_scan_step, one call per step."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_step

    h = to_dev(h0) if h0 is not None else torch.zeros((p.batch, p.channels, p.nstate), device="cuda")
    ys = []
    for t in range(steps):
        s = dev_problem(inputs.step_slice(p, t))
        y = scan_step(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"], h,
                      softplus=p.softplus, out_dtype=out_dtype or torch.float32)
        ys.append(y.float())
    torch.cuda.synchronize()
    return (torch.stack(ys, dim=-1).cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("case", sorted(CASES))
def test_one_step(case):
    p = inputs.time_slice(CASES[case](), 0, 1)
    h0 = inputs.random_state(78, p.batch, p.channels, p.nstate)
    y, h = run_steps(p, h0, 1)
    ry, rh = oracle_state(p, h0)
    ey, eh = normwise(y, ry), normwise(h, rh)
    say("[step] %s: y %.3e, state %.3e" % (case, ey, eh))
    assert ey <= TOL[p.in_dtype] and eh <= TOL[p.in_dtype], (case, ey, eh)


@pytest.mark.parametrize("case", ["diag bf16 N16", "scalar f32 generic", "matrix bf16"])
def test_steps_match_a_scan(case):
    """40 decoding steps from a state equal the scan over those 40 steps from that state."""
    p = inputs.time_slice(CASES[case](), 0, 40)
    h0 = inputs.random_state(79, p.batch, p.channels, p.nstate)
    y, h = run_steps(p, h0, 40)
    ry, rh = oracle_state(p, h0)
    ey, eh = normwise(y, ry), normwise(h, rh)
    say("[step] 40 steps %s: y %.3e, state %.3e" % (case, ey, eh))
    assert ey <= TOL[p.in_dtype] and eh <= TOL[p.in_dtype], (case, ey, eh)


def test_step_bf16_output_and_large_state():
    """N = 128 (32 lanes per row), y written in bf16 (one rounding on top of the f32 result)."""
    torch = torch_dev()
    p = inputs.time_slice(inputs.random_problem(906, 3, 40, 8, 128), 0, 1)
    h0 = inputs.random_state(80, p.batch, p.channels, p.nstate)
    y, h = run_steps(p, h0, 1, out_dtype=torch.bfloat16)
    ry, rh = oracle_state(p, h0)
    scale = np.max(np.abs(ry))
    assert np.all(np.abs(y - ry) <= 2.0 ** -8 * np.abs(ry) + 2e-3 * scale)
    assert normwise(h, rh) <= TOL[p.in_dtype]


def test_steps_in_a_graph_match_eager():
    """Decoding steps captured in a HIP graph (the way a serving loop runs them) and replayed
    several times, with eager work and synchronisation between replays: every replay equals the
    same steps run eagerly from the same state."""
    torch = torch_dev()
    from selective_state_space_88_amd.scan import scan_step

    p = inputs.time_slice(CASES["diag bf16 N16"](), 0, 4)
    steps = [dev_problem(inputs.step_slice(p, t)) for t in range(4)]
    h0 = to_dev(inputs.random_state(81, p.batch, p.channels, p.nstate))
    h = h0.clone()
    ys = [torch.empty((p.batch, p.channels), device="cuda") for _ in steps]

    def run(hh, outs):
        for s, y in zip(steps, outs):
            scan_step(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"], hh, y=y)

    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run(h, ys)
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(h0)
        g.replay()
        torch.cuda.synchronize()
        h_ref = h0.clone()
        y_ref = [torch.empty_like(y) for y in ys]
        run(h_ref, y_ref)
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), rep
        for a, b in zip(ys, y_ref):
            assert torch.equal(a, b), rep
