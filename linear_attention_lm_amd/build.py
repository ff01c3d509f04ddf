"""Build libbased.so (HIP, gfx950 only) in-tree.

    python -m linear_attention_lm_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and links the shared
library next to this file.  Always recompiles (a few seconds per file, in
parallel).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbased.so")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in device code.
# -amdgpu-mfma-vgpr-form: matrix-core operands and results in VGPRs (AGPRs
# only as spill space): the occupancy-1 linear-attention kernels (d_v 96 and
# 128) run faster so (d_v 128: ~3 % for the fused layer, ~8 % for the linear
# attention alone); both forms give the same results, and the d_v <= 64
# kernels compile identically.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
CXXFLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
            "-Wno-unused-command-line-argument"] + DEVICE_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the Based HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = True) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([cc, *CXXFLAGS, "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SANITIZED_LIB = os.path.join(BUILD, "libbased_sanitized.so")


def build_sanitized(verbose: bool = False) -> str:
    """The C ABI's argument validation alone (api.cpp and the host-side
    planning, kernel launchers stubbed out) built for the host with
    AddressSanitizer and UndefinedBehaviorSanitizer: a shared library with
    every entry point that has no device code of its own, for the ABI tests
    to run against (loaded with the sanitizer runtimes preloaded)."""
    os.makedirs(BUILD, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(PKG, "sanitize", "launch_stubs.cpp"), "-Wl,--no-undefined", "-lasan", "-lubsan",
           "-o", SANITIZED_LIB]
    out = _run(cmd)
    if verbose:
        print(out or f"built {SANITIZED_LIB}")
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose="-q" not in sys.argv)
