"""Build liblattn.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblattn.so")
ARCH = os.environ.get("LATTN_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "general.hip", "fast.hip", "misc.hip", "hla.hip", "loglinear.hip", "backward.hip", "backward_chunk.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # Packed fp32 VALU ops are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA sources and results stay in ordinary VGPRs (no accumulation-register
    # forms): the solve feeds MFMA results straight back in as B operands.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


# Sources of the bf16 MFMA kernels: none of their kernels may use scratch
# memory (a register spill there costs time and HBM writes, and has crept in
# unnoticed before), so the build fails if one does.
SCRATCH_FREE = ("fast.hip", "loglinear.hip", "backward_chunk.hip")
_RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(remarks: str):
    """(function, bytes per lane) of every function the compiler's resource
    remarks report with scratch memory."""
    import re

    out = []
    for block in remarks.split("Function Name: ")[1:]:
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block)
        if m and int(m.group(1)) > 0:
            out.append((block.split()[0], int(m.group(1))))
    return out


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless.
    noise = "packed-fp32-ops"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    return res.returncode, errs


def build(verbose: bool = False, extra=None, jobs: int = 0) -> str:
    """Compile every source to an object in parallel (each carries its own gfx950
    code object), then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra or [])
    inc = ["-I", os.path.join(ROOT, "include")]
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[hipcc, *flags, *inc, "-c", "-o", o, s] + ([_RESOURCE_REMARK] if os.path.basename(s) in SCRATCH_FREE else [])
            for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, errs), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{errs}")
        if os.path.basename(s) in SCRATCH_FREE:
            bad = scratch_users(errs)
            if bad:
                raise RuntimeError(f"{os.path.basename(s)}: kernels using scratch memory (bytes per lane): {bad}")
            errs = "\n".join(l for l in errs.splitlines() if "kernel-resource-usage" not in l
                             and not l.lstrip().startswith(("|", "^")) and "remark" not in l)
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, errs = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
