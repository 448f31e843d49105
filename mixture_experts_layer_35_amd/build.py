"""Build the gfx950 shared library in-tree with hipcc.

python -m mixture_experts_layer_35_amd.build

Each source is compiled to an object in its own hipcc process (in parallel),
then the objects are linked into libmoe_mi355x.so next to this file.
"""
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_NAME = "libmoe_mi355x.so"
SOURCES = ["csrc/moe_kernels.hip", "csrc/moe_grouped.hip", "csrc/moe_grouped_bf16.hip",
           "csrc/moe_grouped_fp8.hip", "csrc/moe_grouped_mxfp4.hip", "csrc/moe_grouped_nvfp4.hip",
           "csrc/moe_api.cpp"]
# packed FP32 instructions stay off: hipcc -O3 would otherwise form them
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="moe_build_") as td:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(td, os.path.basename(src) + ".o")
            cmd = [hipcc()] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-x", "hip",
                                           "-c", os.path.join(PKG, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = False
        for src, p in procs:
            log, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(log)
                failed = True
        if failed:
            raise RuntimeError("hipcc failed")
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc link failed ({r.returncode})")
    os.replace(tmp, out)
    build_driver(verbose)
    return out


DRIVER = "moe_profile_driver"


def build_driver(verbose: bool = False) -> str:
    """The stand-alone profiling driver (csrc/moe_profile_driver.cpp), linked
    against the library next to it."""
    out = os.path.join(PKG, DRIVER)
    cmd = [hipcc()] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-x", "hip",
                                   os.path.join(PKG, "csrc", DRIVER + ".cpp"), "-o", out + ".tmp",
                                   "-L", PKG, "-l:" + LIB_NAME, "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc (profiling driver) failed ({r.returncode})")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
