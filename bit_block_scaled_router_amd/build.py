"""Build the w4moe HIP library for gfx950 in-tree (libw4moe.so next to this file).

    python -m bit_block_scaled_router_amd.build

hipcc cross-compiles the device code for gfx950, so this runs on a machine
without a GPU.  Each source is compiled to an object in its own hipcc process
(in parallel), then the objects are linked into the shared library.  Packed
fp32 VALU instructions are disabled for all device code.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4moe.so")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["w4moe_kernels.hip", "w4moe_grouped.hip", "w4moe_decode.hip", "w4moe_host.cpp"]
ARCH = "gfx950"
NOISE = "packed-fp32-ops' is not a recognized feature"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the w4moe library)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(os.path.dirname(HERE), "include"),
    ]


def _stderr(text):
    return "\n".join(ln for ln in text.splitlines() if NOISE not in ln)


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o")
        cmd = [cc] + compile_flags() + ["-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errors = []
    for s, p in procs:
        _, err = p.communicate()
        err = _stderr(err)
        if p.returncode != 0:
            errors.append(f"{s}: hipcc failed ({p.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if errors:
        raise RuntimeError("\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_stderr(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
