"""Builds the gfx950 HIP library libmoe_cache.so in-tree with hipcc."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_cache.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit a*b+c fusion: kernels that must agree bit for bit round
    # alike wherever they are inlined (explicit fmaf still fuses)
    "-ffp-contract=off",
    # gfx950 loads the leading kernel arguments into scalar registers at
    # wave launch (up to 14 dwords), so kernels that put their hot scalar
    # arguments first need no argument load before their first request
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


# Host-only C++ (the CPU half of the hybrid decode step), built by the
# host compiler for x86-64 with AVX2 and FMA.
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-pthread", "-mavx2", "-mfma"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def cpp_sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compiles every source to an object in parallel, then links the
    shared library.  Always recompiles."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    procs, objs = [], []
    srcs = sources()
    # the longest compile first
    srcs.sort(key=lambda f: os.path.getsize(f) * (4 if "k_expert_" in f else 1), reverse=True)
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc, *HIPCC_FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        while len([p for p in procs if p.poll() is None]) >= jobs:
            procs[[p.poll() is None for p in procs].index(True)].wait()
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
    cxx = os.environ.get("CXX", "g++")
    for src in cpp_sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [cxx, *CXX_FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
    errs = []
    for p in procs:
        _, err = p.communicate()
        if p.returncode != 0:
            errs.append(err)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-pthread", "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
