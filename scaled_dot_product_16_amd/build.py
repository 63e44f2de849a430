"""Build libattn.so in-tree for gfx950 with hipcc.

Usage: python -m scaled_dot_product_16_amd.build  (or call build()).
The host validation layer is plain C++; the kernels are HIP.  Both link into
one shared library next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # Min/max need no NaN-quieting canonicalisation (no signalling NaNs are
    # produced or tested for); MFMA accumulators stay in VGPRs so the softmax
    # reads them without accvgpr moves.
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    "-mllvm", "--amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed: {' '.join(cmd)}")
    # Drop the host pass's notice about the GPU-only feature flag.
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if err.strip():
        sys.stderr.write(err + "\n")


# (dtype enum value, head dim or fp32 register bucket) of every compiled instance.
INSTANCES = [(2, 32), (2, 40), (2, 64), (2, 80),   # bf16
             (1, 32), (1, 40), (1, 64), (1, 80),   # f16
             (0, 32), (0, 64), (0, 128)]           # f32


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link libattn.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    cmds, objs = [], []
    for name in ("attn_api", "attn_dispatch"):
        o = os.path.join(obj_dir, name + ".o")
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-c",
                     os.path.join(CSRC, name + ".cpp"), "-o", o])
        objs.append(o)
    # The backward entry point that allocates nothing (its fixed device array).
    o = os.path.join(obj_dir, "attn_noalloc.o")
    cmds.append([cc, *HIP_FLAGS, "-c", os.path.join(CSRC, "attn_noalloc.hip"), "-o", o])
    objs.append(o)
    for dt, d in INSTANCES:
        o = os.path.join(obj_dir, f"attn_inst_{dt}_{d}.o")
        cmds.append([cc, *HIP_FLAGS, f"-DINST_DT={dt}", f"-DINST_D={d}", "-c",
                     os.path.join(CSRC, "attn_inst.hip"), "-o", o])
        objs.append(o)
    jobs = jobs or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    # A plain C caller of the library (host code only), run by the GPU tests.
    c_src = os.path.join(os.path.dirname(HERE), "tests", "c_abi", "attn_fwd_c.c")
    if os.path.exists(c_src) and shutil.which("gcc"):
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(cc)))
        _run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(os.path.dirname(HERE), "include"), "-I", os.path.join(rocm, "include"),
              c_src, "-o", os.path.join(obj_dir, "attn_fwd_c"), "-L", HERE, "-lattn",
              "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
              "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(rocm, "lib")])
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
