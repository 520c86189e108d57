"""MI355X-native (gfx950) selective-scan forward (Mamba S6).

The scan runs in hand-written HIP kernels behind the C ABI of libssscan.so
(include/ss_scan.h); ``scan.scan_fwd`` is its Python binding.  ``inputs`` holds the seeded
synthetic workloads.  Submodules load lazily so that importing the package needs neither
torch nor the built library.
"""
import importlib

__all__ = ["scan_fwd", "ScanError", "scan", "inputs"]


def __getattr__(name):
    if name in ("scan", "inputs"):
        return importlib.import_module(__name__ + "." + name)
    if name in ("scan_fwd", "ScanError"):
        return getattr(importlib.import_module(__name__ + ".scan"), name)
    raise AttributeError(name)
