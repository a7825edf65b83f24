"""Build libmk.so (gfx950) in-tree with hipcc.

    python -m persistent_megakernel_decode_amd.build

Every HIP translation unit is compiled with the packed-fp32 target feature
disabled (the compiler otherwise forms v_pk_* fp32 instructions by itself).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmk.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
HIP_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        raise RuntimeError("build step failed: %s" % os.path.basename(cmd[-1]))
    if out.strip():
        sys.stderr.write(out + "\n")


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, lang in (("mk_kernels.hip", "hip"), ("mk_api.cpp", "hip")):
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, "-c", "-x", lang] + COMMON + HIP_FLAGS + [os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    obj = os.path.join(BUILD, "plan.cpp.o")
    _run(["g++", "-c"] + COMMON + [os.path.join(CSRC, "plan.cpp"), "-o", obj])
    objs.append(obj)
    tmp = OUT + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
