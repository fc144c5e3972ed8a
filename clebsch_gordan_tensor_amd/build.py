"""Build libcgtp.so (HIP, gfx950 only) in-tree.

    python -m clebsch_gordan_tensor_amd.build [--jobs N]

Every source under csrc/ is compiled by hipcc for gfx950 into _build/, then
linked into clebsch_gordan_tensor_amd/libcgtp.so. Packed-FP32 instructions are
disabled (-packed-fp32-ops): the kernels are written for the plain VALU.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcgtp.so")
SOURCES = ["plan.cpp", "capi.cpp", "tp_kernels.hip", "conv_kernels.hip", "graph_kernels.hip",
           "sh_kernels.hip", "linear_kernels.hip", "double_backward.hip", "uvw_kernels.hip", "uvuv_kernels.hip", "radial_kernels.hip"]
# one translation unit per large kernel instantiation, compiled in parallel
SOURCES += sorted(os.path.join("inst", f) for f in os.listdir(os.path.join(CSRC, "inst")) if f.endswith(".hip"))
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags(defines=()):
    return (["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + ["-D" + d for d in defines])


def compile_one(src, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.splitext(src.replace(os.sep, "_"))[0] + ".o")
    cmd = [hipcc()] + common_flags(defines) + ["-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj, time.time() - t0, r.stderr


def build(jobs=None, verbose=True, lib=LIB, build_dir=BUILD, defines=()):
    """Compile and link; `lib`, `build_dir` and `defines` (-D tuning knobs) default
    to the in-tree library."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    objs = []
    # the big instantiation units first, so the pool stays busy
    order = sorted(SOURCES, key=lambda f: (not f.startswith("inst"), f))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, dt, err in ex.map(lambda f: compile_one(f, build_dir, defines), order):
            objs.append(obj)
            if verbose:
                print("  compiled %-24s %6.1fs" % (os.path.basename(obj), dt), flush=True)
                warn = "\n".join(l for l in err.splitlines() if "warning" in l and "packed-fp32" not in l)
                if warn:
                    print(warn, flush=True)
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("  linked", lib, flush=True)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--lib", default=LIB, help="output library path")
    ap.add_argument("--build-dir", default=BUILD)
    ap.add_argument("-D", dest="defines", action="append", default=[], help="preprocessor knob")
    a = ap.parse_args()
    try:
        build(a.jobs, lib=a.lib, build_dir=a.build_dir, defines=a.defines)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
