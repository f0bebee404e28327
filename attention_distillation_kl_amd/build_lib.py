"""Compile the HIP sources under ``csrc/`` into ``libstreamkl.so`` for gfx950.

Every translation unit is compiled with hipcc (in parallel), then linked into
one shared library next to this file.  ``build()`` always recompiles.
``build(debug=True)`` compiles the same sources with -DSTREAMKL_DEBUG into
``libstreamkl_debug.so``: every global-memory access of the kernels, and the
LDS accesses of their tile loops, checked against its buffer's extent (see
streamkl_debug_take in include/streamkl.h).  Without the macro the checks
compile to nothing.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libstreamkl.so")
DEBUG_LIB = os.path.join(HERE, "libstreamkl_debug.so")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU
# instructions (v_pk_fma_f32 and friends); all fp32 math stays scalar.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra, objdir=OBJDIR):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj


def build(verbose: bool = False, extra_flags=(), debug: bool = False) -> str:
    objdir = os.path.join(OBJDIR, "debug") if debug else OBJDIR
    lib = DEBUG_LIB if debug else LIB
    flags = list(extra_flags) + (["-DSTREAMKL_DEBUG"] if debug else [])
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, objdir), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_all(verbose: bool = False) -> tuple:
    """The release and the debug library, compiled in one pool of workers."""
    jobs = [(s, [], OBJDIR) for s in sources()] + \
           [(s, ["-DSTREAMKL_DEBUG"], os.path.join(OBJDIR, "debug")) for s in sources()]
    for _, _, d in jobs:
        os.makedirs(d, exist_ok=True)
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(objs) // 2
    out = []
    for lib, group in ((LIB, objs[:n]), (DEBUG_LIB, objs[n:])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *group, "-o", tmp]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
        out.append(lib)
    return tuple(out)


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv[1:]))
