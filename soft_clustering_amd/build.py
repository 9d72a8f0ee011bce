"""Build libgmm.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m soft_clustering_amd.build            # build
    python -m soft_clustering_amd.build --asm DIR  # also keep the gfx950 ISA

Every translation unit in csrc/ is compiled by hipcc for gfx950 only, with
packed-fp32 instructions disabled, and linked into soft_clustering_amd/libgmm.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libgmm.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Translation units whose kernels never test floats for NaN: IEEE mode off
# lets max/min fold into DPP forms (one v_max_f32_dpp per reduction step).
NO_IEEE = {f: ["-fno-honor-nans", "-mno-amdgpu-ieee"] for f in ("diag_split.hip", "largek.hip")}

# The full-covariance kernel's second-moment loops must unroll completely (its
# accumulator blocks live in registers); the default size cap for requested
# unrolling stops short of D = 64.
EXTRA = {"full_fused.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"]}


def _compile(src: str, asm_dir: str | None) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    base = os.path.basename(src)
    flags = [*FLAGS, *NO_IEEE.get(base, []), *EXTRA.get(base, [])]
    cmds = [[HIPCC, *flags, "-c", src, "-o", obj]]
    if asm_dir:   # the device code's ISA, compiled on its own
        asm = os.path.join(os.path.abspath(asm_dir), base.replace(".hip", f"-{ARCH}.s"))
        cmds.append([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", asm])
    for cmd in cmds:
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    return obj


def build(asm_dir: str | None = None, jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm_dir), srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources")
    return OUT


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory to keep the gfx950 assembly in")
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args(argv)
    build(a.asm, a.j)


if __name__ == "__main__":
    sys.exit(main())
