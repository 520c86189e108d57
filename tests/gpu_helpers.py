"""Helpers for GPU tests: move generator arrays to the device and call the HIP path.

Holds none of the scan's arithmetic: only dtype plumbing and the call through the binding.
"""
import sys

import numpy as np


def torch_dev():
    import torch

    if not torch.cuda.is_available():
        import pytest

        pytest.skip("no GPU")
    return torch


def to_dev(a, device="cuda"):
    """numpy array (float32, or uint16 bf16 bit patterns) -> torch tensor on the GPU."""
    import torch

    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def dev_problem(p):
    return dict(u=to_dev(p.u), delta=to_dev(p.delta), A=to_dev(p.A), B=to_dev(p.B), C=to_dev(p.C),
                D=to_dev(p.D), z=to_dev(p.z), delta_bias=to_dev(p.delta_bias))


def run_hip(p, out_dtype=None, dev=None):
    """y from the HIP path (through the C ABI) for a generator Problem, as a float64 numpy array."""
    import torch

    from selective_state_space_88_amd.scan import scan_fwd

    t = dev if dev is not None else dev_problem(p)
    y = scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                 softplus=p.softplus, out_dtype=out_dtype or torch.float32, zoh=getattr(p, "zoh", False),
                 trapezoid=getattr(p, "trapezoid", False))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()
