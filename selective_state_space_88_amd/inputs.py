"""Seeded synthetic inputs for the selective-scan forward.

This module only draws random numbers and encodes them; it holds none of the
scan's arithmetic.  Both the HIP path (through the binding) and the CPU oracle
consume the arrays it returns, so both sides see the same bf16 bit patterns.

Workloads are the five Mamba-shaped layers of the scan's benchmark set:

  0  tiny fp32 layer: batch 1, 16 channels, L 64, N 4
  1  Mamba-130M-like: batch 8, 1536 channels, L 2048, N 16, bf16 inputs
  2  Mamba-2.8B-like: batch 4, 5120 channels, L 4096, N 16, bf16 inputs
  3  long-sequence layer: batch 1, 1024 channels, L 1,048,576, N 16, bf16 inputs
  4  scalar-decay multi-head layer: batch 2, 80 heads x 64 channels, L 8192, N 128

Recipe (per workload k): ``numpy.random.default_rng(1000 + k)`` (PCG64).
Tensors are drawn in the fixed order u, delta_raw, z, B, C, dt, D, A as float32
(dt as float64) and rounded to bf16 with round-to-nearest-even where the
workload is bf16.  Large tensors are drawn in fixed-size blocks, so the stream
is defined block by block.  A is the S4D-real diagonal A[d, n] = -(n + 1) for
workloads 0-3 (no draw) and -U(1, 16) per head for workload 4.  The step bias
is delta_bias = log(expm1(dt)) (the inverse of softplus) computed in float64
and stored as float32, with dt log-uniform, one per channel (per head in
workload 4).

Every size can be overridden to make smaller cases with the same value
distributions and flags.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_BLOCK = 1 << 24  # elements drawn per block for large tensors


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Problem:
    """One scan problem.  Arrays are contiguous; bf16 tensors are uint16 bit patterns.

    Layouts (L innermost):
      u, z      [batch, channels, L]
      delta     [batch, heads, L]            heads == channels unless scalar_decay
      A         [channels, N] or [heads]     (scalar decay per head)
      B, C      [batch, groups, N, L]
      D         [channels] or [heads]
      delta_bias[heads]
    """

    name: str
    batch: int
    channels: int
    length: int
    nstate: int
    groups: int
    heads: int
    in_dtype: str  # "f32" or "bf16"
    u: np.ndarray
    delta: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: Optional[np.ndarray]
    z: Optional[np.ndarray]
    delta_bias: Optional[np.ndarray]
    softplus: bool = True
    scalar_decay: bool = False
    meta: dict = field(default_factory=dict)
    zoh: bool = False  # zero-order-hold input coefficient instead of exponential-Euler
    trapezoid: bool = False  # exponential-trapezoidal rule

    @property
    def elements(self) -> int:
        return self.batch * self.channels * self.length

    @property
    def gate(self) -> bool:
        return self.z is not None


DEFAULTS = {
    0: dict(batch=1, channels=16, length=64, nstate=4, heads=None, in_dtype="f32", gate=False,
            bc_scale=1.0, dt=(1e-3, 1e-1)),
    1: dict(batch=8, channels=1536, length=2048, nstate=16, heads=None, in_dtype="bf16", gate=True,
            bc_scale=1.0, dt=(1e-3, 1e-1)),
    2: dict(batch=4, channels=5120, length=4096, nstate=16, heads=None, in_dtype="bf16", gate=True,
            bc_scale=1.0, dt=(1e-3, 1e-1)),
    3: dict(batch=1, channels=1024, length=1 << 20, nstate=16, heads=None, in_dtype="bf16", gate=True,
            bc_scale=0.25, dt=(1e-4, 1e-2)),
    4: dict(batch=2, channels=80 * 64, length=8192, nstate=128, heads=80, in_dtype="bf16", gate=False,
            bc_scale=None, dt=(1e-3, 1e-1)),
}

NAMES = {
    0: "tiny-fp32 (1x16x64, N=4)",
    1: "mamba-130m-layer (8x1536x2048, N=16)",
    2: "mamba-2.8b-layer (4x5120x4096, N=16)",
    3: "long-seq-layer (1x1024x1048576, N=16)",
    4: "scalar-decay-multihead (2x(80x64)x8192, N=128)",
}


def _normal(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    """Standard normal draws (float32), times ``scale`` in float32, encoded as ``dtype``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    s = np.float32(scale)
    for lo in range(0, n, _BLOCK):
        hi = min(n, lo + _BLOCK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x = x * s
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out.reshape(shape)


def make(cfg: int, *, batch: Optional[int] = None, channels: Optional[int] = None,
         length: Optional[int] = None, nstate: Optional[int] = None, heads: Optional[int] = None,
         headdim: Optional[int] = None, seed: Optional[int] = None, in_dtype: Optional[str] = None,
         gate: Optional[bool] = None, with_D: bool = True, with_bias: bool = True) -> Problem:
    """Build workload ``cfg`` (0-4), optionally resized.  Deterministic for a given seed.

    For the scalar-decay workload (4) the channel count is ``heads * headdim``
    (defaults 80 and 64); ``channels`` is ignored there.
    """
    d = dict(DEFAULTS[cfg])
    Bt = batch if batch is not None else d["batch"]
    N = nstate if nstate is not None else d["nstate"]
    L = length if length is not None else d["length"]
    dt_lo, dt_hi = d["dt"]
    dtype = in_dtype if in_dtype is not None else d["in_dtype"]
    use_gate = d["gate"] if gate is None else gate
    scalar = cfg == 4
    if scalar:
        H = heads if heads is not None else d["heads"]
        P = headdim if headdim is not None else 64
        Dc = H * P
    else:
        Dc = channels if channels is not None else d["channels"]
        H = Dc
    G = 1
    bc_scale = d["bc_scale"] if d["bc_scale"] is not None else 1.0 / np.sqrt(N)
    rng = np.random.default_rng(1000 + cfg if seed is None else seed)

    u = _normal(rng, (Bt, Dc, L), 1.0, dtype)
    delta = _normal(rng, (Bt, H, L), 1.0, dtype)
    z = _normal(rng, (Bt, Dc, L), 1.0, dtype) if use_gate else None
    B = _normal(rng, (Bt, G, N, L), bc_scale, dtype)
    C = _normal(rng, (Bt, G, N, L), bc_scale, dtype)
    dt = np.exp(rng.uniform(np.log(dt_lo), np.log(dt_hi), size=H))
    delta_bias = np.log(np.expm1(dt)).astype(np.float32) if with_bias else None
    Dvec = rng.standard_normal(H if scalar else Dc, dtype=np.float32)
    if scalar:
        A = (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    else:
        A = np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (Dc, N)).copy()
    return Problem(
        name=NAMES[cfg], batch=Bt, channels=Dc, length=L, nstate=N, groups=G, heads=H,
        in_dtype=dtype, u=u, delta=delta, A=A, B=B, C=C,
        D=Dvec if with_D else None, z=z, delta_bias=delta_bias, softplus=True,
        scalar_decay=scalar, meta=dict(cfg=cfg, seed=1000 + cfg if seed is None else seed),
    )


def to_f32(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Decode an input array (bf16 bits or float32) to float32."""
    if a is None:
        return None
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def random_problem(seed: int, batch: int, channels: int, length: int, nstate: int, *,
                   heads: Optional[int] = None, groups: int = 1, scalar_decay: bool = False,
                   in_dtype: str = "bf16", gate: bool = True, with_D: bool = True,
                   with_bias: bool = True, softplus: bool = True,
                   dt: tuple = (1e-3, 1e-1), bc_scale: float = 1.0) -> Problem:
    """A general problem for edge cases: per-channel random A (not S4D), any heads/groups.

    u, delta_raw, z, B, C ~ N(0,1) (B, C times bc_scale); A[d, n] ~ -U(0.5, 4) (or A[h] per
    head when scalar_decay); D ~ N(0,1); delta_bias = inv_softplus(dt), dt log-uniform in ``dt``.
    With softplus off the raw steps are U(0.001, 0.3) and no bias is drawn.
    """
    H = channels if heads is None else heads
    rng = np.random.default_rng(seed)
    Bt, Dc, L, N, G = batch, channels, length, nstate, groups
    u = _normal(rng, (Bt, Dc, L), 1.0, in_dtype)
    if softplus:
        delta = _normal(rng, (Bt, H, L), 1.0, in_dtype)
    else:
        raw = rng.uniform(0.001, 0.3, size=(Bt, H, L)).astype(np.float32)
        delta = f32_to_bf16_bits(raw).reshape(raw.shape) if in_dtype == "bf16" else raw
    z = _normal(rng, (Bt, Dc, L), 1.0, in_dtype) if gate else None
    B = _normal(rng, (Bt, G, N, L), bc_scale, in_dtype)
    C = _normal(rng, (Bt, G, N, L), bc_scale, in_dtype)
    dts = np.exp(rng.uniform(np.log(dt[0]), np.log(dt[1]), size=H))
    bias = np.log(np.expm1(dts)).astype(np.float32) if (with_bias and softplus) else None
    Dv = rng.standard_normal(H if scalar_decay else Dc, dtype=np.float32) if with_D else None
    if scalar_decay:
        A = (-rng.uniform(0.5, 4.0, size=H)).astype(np.float32)
    else:
        A = (-rng.uniform(0.5, 4.0, size=(Dc, N))).astype(np.float32)
    return Problem(name="random", batch=Bt, channels=Dc, length=L, nstate=N, groups=G, heads=H,
                   in_dtype=in_dtype, u=u, delta=delta, A=A, B=B, C=C, D=Dv, z=z,
                   delta_bias=bias, softplus=softplus, scalar_decay=scalar_decay,
                   meta=dict(seed=seed))


def device_problem(seed: int, batch: int, channels: int, length: int, nstate: int, *,
                   heads: Optional[int] = None, groups: int = 1, scalar_decay: bool = False,
                   gate: bool = True, dt: tuple = (1e-4, 1e-2), bc_scale: Optional[float] = None,
                   device="cuda", rows_per_draw: int = 32):
    """A bf16 problem too large to draw on the host (more than 2^31 elements), drawn on `device`.

    u, delta_raw, z ~ N(0, 1) and B, C ~ N(0, 1) bc_scale (default 1/sqrt(N)) come from torch's
    generator on the device seeded with `seed`, drawn in that order as float32, `rows_per_draw`
    time rows at a time, and rounded to bf16 (round to nearest even).  The small parameters come
    from ``numpy.random.default_rng(seed)`` as in the workloads: A[d, n] = -(n + 1) (or A[h] =
    -U(1, 16) per head with scalar decay), D ~ N(0, 1) per channel (per head with scalar
    decay), delta_bias = inv_softplus(dt) with dt log-uniform in ``dt``, one per head.

    Returns (tensors, p): the device tensors by argument name, and a Problem holding the small
    parameters (its per-step arrays are None; ``device_row`` copies rows back for the oracle).
    """
    import torch

    H = channels if heads is None else heads
    Bt, Dc, L, N, G = batch, channels, length, nstate, groups
    scale = (1.0 / np.sqrt(N)) if bc_scale is None else bc_scale
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def draw(shape, sc):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = out.view(-1, shape[-1])
        for r in range(0, flat.shape[0], rows_per_draw):
            x = torch.randn((min(rows_per_draw, flat.shape[0] - r), shape[-1]), generator=gen, device=device,
                            dtype=torch.float32)
            flat[r:r + x.shape[0]] = (x * sc if sc != 1.0 else x).to(torch.bfloat16)
        return out

    t = dict(u=draw((Bt, Dc, L), 1.0), delta=draw((Bt, H, L), 1.0), z=draw((Bt, Dc, L), 1.0) if gate else None)
    t["B"] = draw((Bt, G, N, L), scale)
    t["C"] = draw((Bt, G, N, L), scale)
    rng = np.random.default_rng(seed)
    dts = np.exp(rng.uniform(np.log(dt[0]), np.log(dt[1]), size=H))
    bias = np.log(np.expm1(dts)).astype(np.float32)
    Dv = rng.standard_normal(H if scalar_decay else Dc, dtype=np.float32)
    if scalar_decay:
        A = (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    else:
        A = np.tile(-np.arange(1, N + 1, dtype=np.float32), (Dc, 1))
    t.update(A=torch.from_numpy(A).to(device), D=torch.from_numpy(Dv).to(device),
             delta_bias=torch.from_numpy(bias).to(device))
    p = Problem(name="device", batch=Bt, channels=Dc, length=L, nstate=N, groups=G, heads=H, in_dtype="bf16",
                u=None, delta=None, A=A, B=None, C=None, D=Dv, z=None, delta_bias=bias, softplus=True,
                scalar_decay=scalar_decay, meta=dict(seed=seed, device_drawn=True))
    return t, p


def device_normal(seed: int, shape, device="cuda", rows_per_draw: int = 32):
    """float32 ~ N(0, 1) of the given shape drawn on `device` (torch's generator seeded with
    `seed`, `rows_per_draw` rows of the last dimension at a time): e.g. the upstream gradient of
    a backward over a device-drawn problem."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(-1, shape[-1])
    for r in range(0, flat.shape[0], rows_per_draw):
        n = min(rows_per_draw, flat.shape[0] - r)
        flat[r:r + n] = torch.randn((n, shape[-1]), generator=gen, device=device, dtype=torch.float32)
    return out


def device_row(t: dict, p: Problem, b: int, d: int) -> Problem:
    """Row (b, d) of a device-drawn problem as a one-channel host Problem (the same bf16 bits)."""
    import torch

    def bits(x):
        return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    h = d // (p.channels // p.heads)
    g = d // (p.channels // p.groups)
    one = lambda x: None if x is None else bits(x[b:b + 1, d:d + 1])
    A = p.A[h:h + 1] if p.scalar_decay else p.A[d:d + 1]
    Dv = p.D[h:h + 1] if p.scalar_decay else p.D[d:d + 1]
    return Problem(name="device row", batch=1, channels=1, length=p.length, nstate=p.nstate, groups=1, heads=1,
                   in_dtype="bf16", u=one(t["u"]), delta=bits(t["delta"][b:b + 1, h:h + 1]),
                   A=np.ascontiguousarray(A), B=bits(t["B"][b:b + 1, g:g + 1]), C=bits(t["C"][b:b + 1, g:g + 1]),
                   D=np.ascontiguousarray(Dv), z=one(t["z"]), delta_bias=np.ascontiguousarray(p.delta_bias[h:h + 1]),
                   softplus=True, scalar_decay=p.scalar_decay, meta=dict(p.meta, row=(b, d)))


def random_state(seed: int, batch: int, channels: int, nstate: int, scale: float = 1.0) -> np.ndarray:
    """A seeded state h [batch, channels, N] float32 ~ N(0, scale^2), for the state entry points."""
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((batch, channels, nstate))).astype(np.float32)


def time_slice(p: Problem, t0: int, t1: int) -> Problem:
    """The same problem restricted to steps [t0, t1) (the per-step tensors are sliced along
    time; A, D and delta_bias are shared)."""
    def cut(a):
        return None if a is None else np.ascontiguousarray(a[..., t0:t1])

    return dataclasses.replace(p, length=t1 - t0, u=cut(p.u), delta=cut(p.delta), B=cut(p.B), C=cut(p.C),
                               z=cut(p.z), meta=dict(p.meta, time_slice=(t0, t1)))


def step_slice(p: Problem, t: int) -> Problem:
    """Step t of the problem as one decoding step: u, z [batch, channels], delta [batch, heads],
    B, C [batch, groups, N]."""
    def at(a):
        return None if a is None else np.ascontiguousarray(a[..., t])

    return dataclasses.replace(p, length=1, u=at(p.u), delta=at(p.delta), B=at(p.B), C=at(p.C), z=at(p.z),
                               meta=dict(p.meta, step=t))


def seeded_normal(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """float32 ~ N(0, scale^2) of the given shape (e.g. the upstream gradient dy of a backward)."""
    return (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)


def random_conv(seed: int, batch: int, channels: int, length: int, width: int, *, in_dtype: str = "bf16",
                with_bias: bool = True, with_state: bool = True) -> dict:
    """Inputs of the causal depthwise convolution in front of the scan: x [batch, channels, L] ~ N(0, 1)
    (encoded as ``in_dtype``), weight [channels, W] and bias [channels] ~ U(-1/sqrt(W), 1/sqrt(W))
    (the usual fan-in initialisation of a depthwise convolution), and a state [batch, channels, W - 1]
    ~ N(0, 1) float32 (the inputs before the sequence).  Drawn in that order from
    ``numpy.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (batch, channels, length), 1.0, in_dtype)
    bound = 1.0 / np.sqrt(width)
    w = rng.uniform(-bound, bound, size=(channels, width)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=channels).astype(np.float32) if with_bias else None
    state = rng.standard_normal((batch, channels, width - 1), dtype=np.float32) if with_state else None
    return dict(x=x, w=w, bias=bias, state=state)
