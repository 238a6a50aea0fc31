"""Build liblinattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Every csrc/*.hip unit is compiled to an object in <repo>/_build, in
parallel, then linked into causal_linear_attention_linattn_amd/liblinattn.so.
The measurement probe (csrc/probe/*.hip) is linked separately into
liblinattn_probe.so, which only bench.py loads.
Run `python -m causal_linear_attention_linattn_amd._build` or call build().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
PROBE_LIB = os.path.join(PKG, "liblinattn_probe.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -amdgpu-mfma-vgpr-form: keep MFMA accumulators in ordinary VGPRs (gfx950
# allows it), which removes the v_accvgpr_read copies before every VALU use
# of an accumulator.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.relpath(src, CSRC).replace(os.sep, "_") + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr[-8000:]}")
    return obj


def build(jobs: int | None = None, extra: list[str] | None = None,
          verbose: bool = False) -> str:
    """Compile every HIP unit and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    extra = list(extra or [])
    allsrc = srcs + probe_srcs
    jobs = jobs or min(len(allsrc), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), allsrc))
    for out, lib_objs in ((LIB, objs[:len(srcs)]), (PROBE_LIB, objs[len(srcs):])):
        if not lib_objs:
            continue
        tmp = out + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *lib_objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr[-8000:]}")
        os.replace(tmp, out)
        if verbose:
            print(f"built {out}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
