"""Build libssscan.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssscan.so")
SOURCES = ["ss_api.hip", "ss_diag.hip", "ss_scalar.hip", "ss_ssd.hip", "ss_step.hip", "ss_bwd.hip",
           "ss_ssd_bwd.hip", "ss_conv.hip"]
# the ceiling probes (include/ss_probe.h): a measurement library of its own
PROBE_LIB = os.path.join(HERE, "libssprobe.so")
PROBE_SOURCES = ["ss_probe.hip"]
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # packed FP32 (v_pk_*_f32) stays off: plain f32 VALU code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the scan updates them with VALU work every chunk
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 (one hipcc per file, in parallel) and link them into
    selective_state_space_88_amd/libssscan.so, and the probes into libssprobe.so."""
    _link(SOURCES + PROBE_SOURCES, {LIB: SOURCES, PROBE_LIB: PROBE_SOURCES}, verbose)
    return LIB


def _link(sources, libs, verbose):
    tag = "%d" % os.getpid()
    objs, procs = [], []
    for src in sources:
        obj = os.path.join(CSRC, src.replace(".hip", ".%s.o" % tag))
        cmd = [hipcc()] + [f for f in FLAGS if f != "-shared"] + ["-c", "-o", obj, os.path.join(CSRC, src)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errors = []
    for cmd, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            errors.append("%s\n%s" % (" ".join(cmd), err))
        elif verbose:
            print(" ".join(cmd))
            print(err)
    try:
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        obj_of = dict(zip(sources, objs))
        for lib, srcs in libs.items():
            tmp = lib + ".tmp" + tag
            cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [obj_of[x] for x in srcs]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
            os.replace(tmp, lib)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)


if __name__ == "__main__":
    print(build(verbose=True))
