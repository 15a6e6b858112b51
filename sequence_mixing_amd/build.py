"""Build liblinattn.so in-tree for gfx950 with hipcc.

Usage: ``python -m sequence_mixing_amd.build`` (or ``build()`` from Python).
The library links only the HIP runtime; no torch headers or symbols.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblinattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 ops are disabled for all device code: plain float code is left
# as scalar v_fma/v_add/v_mul.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
# (source, extra defines): the forward/decode kernels are built once per
# (feature map, element type), so the objects compile in parallel.
_PHIS = ["LINATTN_PHI_ELU1", "LINATTN_PHI_RELU", "LINATTN_PHI_SOFTPLUS"]
_ELEMS = ["LINATTN_F32", "LINATTN_BF16", "LINATTN_F16", "LINATTN_FP8_E4M3", "LINATTN_FP8_E5M2"]
SOURCES = [(os.path.join(CSRC, "linattn_fmt.hip"), [f"-DLINATTN_FMT_PHI={p}", f"-DLINATTN_FMT_ELEM={e}"])
           for p in _PHIS for e in _ELEMS] + [
    (os.path.join(CSRC, "linattn_bwd.hip"), []), (os.path.join(CSRC, "linattn.hip"), []),
    (os.path.join(CSRC, "linattn_plan.cpp"), [])]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return r.returncode, err


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB) -> str:
    """Compiles every source to an object in parallel, then links the library."""
    from concurrent.futures import ThreadPoolExecutor

    objs = [f"{out}.{i}.{os.path.basename(src)}.o" for i, (src, _) in enumerate(SOURCES)]
    cmds = [[HIPCC, *FLAGS, *(extra_flags or []), *defs, "-c", src, "-o", obj]
            for (src, defs), obj in zip(SOURCES, objs)]
    cmds = [[a for a in c if a != "-shared"] for c in cmds]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), (src, _) in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = out + ".tmp"
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    for obj in objs:
        if os.path.exists(obj):
            os.remove(obj)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
