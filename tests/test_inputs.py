"""The seeded input generator: bf16 rounding, reproducibility, value ranges."""
import numpy as np
import pytest

from selective_state_space_88_amd import inputs


def test_bf16_rne_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0, 1e-30, -3.5e38],
                                 dtype=np.float32)])
    # ties: 1 + 2^-8 lies halfway between two bf16 values (rounds to even), 1 + 3*2^-9 rounds up
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_reproducible_and_seed_dependent():
    a = inputs.make(1, batch=1, channels=4, length=32)
    b = inputs.make(1, batch=1, channels=4, length=32)
    c = inputs.make(1, batch=1, channels=4, length=32, seed=5)
    assert np.array_equal(a.u, b.u) and np.array_equal(a.B, b.B) and np.array_equal(a.D, b.D)
    assert not np.array_equal(a.u, c.u)


@pytest.mark.parametrize("cfg,lo,hi", [(0, 1e-3, 1e-1), (1, 1e-3, 1e-1), (3, 1e-4, 1e-2), (4, 1e-3, 1e-1)])
def test_step_bias_inverts_softplus(cfg, lo, hi):
    kw = dict(batch=1, length=16)
    if cfg == 4:
        kw.update(heads=8, headdim=4)
    else:
        kw.update(channels=64)
    p = inputs.make(cfg, **kw)
    dt = np.logaddexp(0.0, p.delta_bias.astype(np.float64))
    assert np.all(dt > lo * (1 - 1e-5)) and np.all(dt < hi * (1 + 1e-5))


def test_shapes_and_dtypes():
    p = inputs.make(4, batch=1, heads=3, headdim=8, length=10)
    assert p.u.shape == (1, 24, 10) and p.delta.shape == (1, 3, 10)
    assert p.B.shape == (1, 1, 128, 10) and p.A.shape == (3,) and p.D.shape == (3,)
    assert p.u.dtype == np.uint16 and p.z is None and p.scalar_decay
    assert np.all(p.A <= -1.0) and np.all(p.A >= -16.0)
    q = inputs.make(0)
    assert q.u.dtype == np.float32 and q.A.shape == (16, 4) and np.array_equal(q.A[3], [-1, -2, -3, -4])
    r = inputs.make(3, channels=8, length=4096)
    scale = np.std(inputs.to_f32(r.B))
    assert 0.2 < scale < 0.3  # N(0,1)/sqrt(16)


def test_device_drawn_rows_are_the_same_bits():
    """device_problem / device_row (drawn here on the CPU device): the one-channel row problem
    holds exactly the bits of the drawn tensors at (b, d), its head's step row and its group's B
    and C, and the parameters of its channel (head with scalar decay)."""
    torch = pytest.importorskip("torch")
    t, p = inputs.device_problem(11, 2, 8, 40, 6, groups=2, device="cpu", rows_per_draw=3)
    bits = lambda x: x.view(torch.int16).numpy().view(np.uint16)
    assert t["u"].dtype == torch.bfloat16 and tuple(t["B"].shape) == (2, 2, 6, 40)
    assert np.array_equal(p.A[5], -np.arange(1, 7, dtype=np.float32))
    r = inputs.device_row(t, p, 1, 5)
    assert np.array_equal(r.u[0, 0], bits(t["u"][1, 5])) and np.array_equal(r.z[0, 0], bits(t["z"][1, 5]))
    assert np.array_equal(r.delta[0, 0], bits(t["delta"][1, 5]))
    assert np.array_equal(r.B[0, 0], bits(t["B"][1, 1])) and np.array_equal(r.C[0, 0], bits(t["C"][1, 1]))
    assert r.D[0] == p.D[5] and r.delta_bias[0] == p.delta_bias[5] and np.array_equal(r.A[0], p.A[5])
    # B, C ~ N(0, 1/N); the stream is reproducible
    t2, _ = inputs.device_problem(11, 2, 8, 40, 6, groups=2, device="cpu", rows_per_draw=3)
    assert torch.equal(t["C"], t2["C"])
    s, q = inputs.device_problem(12, 1, 8, 16, 4, heads=2, scalar_decay=True, gate=False, device="cpu")
    assert s["z"] is None and q.A.shape == (2,) and np.all(q.A <= -1.0) and np.all(q.A >= -16.0)
    rq = inputs.device_row(s, q, 0, 7)
    assert np.array_equal(rq.delta[0, 0], bits(s["delta"][0, 1])) and rq.A[0] == q.A[1] and rq.D[0] == q.D[1]
