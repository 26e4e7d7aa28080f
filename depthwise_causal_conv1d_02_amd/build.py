"""Build libccv.so (the gfx950 HIP library behind include/ccv.h) in-tree.

    python -m depthwise_causal_conv1d_02_amd.build [-D NAME=VALUE ...] [-o OUT]

hipcc compiles the kernels for gfx950 only, with packed-FP32 instructions
disabled (-packed-fp32-ops) and hardware FP32 atomics (-munsafe-fp-atomics).
"""
import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libccv.so")
SOURCES = [os.path.join(CSRC, "ccv_api.cpp"), os.path.join(CSRC, "ccv_kernels.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(out=LIB, defines=(), verbose=False):
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + ["-D" + d for d in defines]
    cmd += SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("-o", dest="out", default=LIB)
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.out, args.defines, args.v))


if __name__ == "__main__":
    sys.exit(main())
