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
WIDTHS = (2, 3, 4)
# (source, extra defines, object stem): the per-width kernels compile from one
# source once per width, in parallel with the rest.
UNITS = [("ccv_api.cpp", [], "ccv_api"), ("ccv_misc.hip", [], "ccv_misc")] + [
    ("ccv_width.hip", ["CCV_WIDTH=%d" % w], "ccv_width%d" % w) for w in WIDTHS]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(out=LIB, defines=(), verbose=False, jobs=None):
    from concurrent.futures import ThreadPoolExecutor
    import tempfile

    os.makedirs(os.path.dirname(out), exist_ok=True)
    objdir = tempfile.mkdtemp(prefix="ccv_build_")
    common = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + ["-D" + d for d in defines]

    def compile_unit(unit):
        src, extra, stem = unit
        obj = os.path.join(objdir, stem + ".o")
        cmd = common + ["-D" + d for d in extra] + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(jobs or min(len(UNITS), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_unit, UNITS))
    tmp = out + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, out)
    for o in objs:
        os.remove(o)
    os.rmdir(objdir)
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
