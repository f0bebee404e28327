"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two pieces of host code are rebuilt with -fsanitize=address,undefined:
  * the fp64 oracle (plain C), with clang;
  * the host side of the C ABI layer (``csrc/streamkl_api.hip``: argument
    validation, workspace checks, the no-alloc scratch lookup and dispatch),
    with hipcc, each sanitizer flag given to the host compilation only
    (-Xarch_host), linked with the ordinary kernel objects.  GPU code is never
    built with a sanitizer.
The oracle's pins and the ABI's host tests then run against those builds in a
child process with clang's sanitizer runtime preloaded; any report stops the
child with a non-zero status.  A copy of the oracle with a planted
out-of-bounds read shows that the harness does report one.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/lib/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _asan_runtime():
    hits = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC) and _asan_runtime()),
                                reason="clang, hipcc or the sanitizer runtime is missing")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _oracle(src, out):
    _run([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", *SAN, "-shared-libsan", "-fPIC", "-shared", "-fopenmp",
          src, "-o", out, "-lm"])
    return out


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    oracle_lib = _oracle(os.path.join(ROOT, "oracle", "streamkl_oracle.c"), str(d / "liboracle_san.so"))
    from attention_distillation_kl_amd import build_lib
    kernel_objs = [os.path.join(build_lib.OBJDIR, os.path.basename(s) + ".o")
                   for s in build_lib.sources() if not s.endswith("streamkl_api.hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        build_lib.build()
    api_obj = str(d / "streamkl_api_san.o")
    host_san = [f for flag in SAN + ["-fno-omit-frame-pointer"] for f in ("-Xarch_host", flag)]
    _run([HIPCC, *build_lib.HIP_FLAGS, "-O1", "-g", *host_san, "-c",
          os.path.join(build_lib.CSRC, "streamkl_api.hip"), "-o", api_obj])
    lib = str(d / "libstreamkl_san.so")
    _run([HIPCC, f"--offload-arch={build_lib.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-shared-libsan",
          *[f for flag in SAN for f in ("-Xarch_host", flag)], api_obj, *kernel_objs, "-o", lib])
    return {"dir": d, "oracle": oracle_lib, "lib": lib}


CHILD = """
import os, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, os.path.join({root!r}, "tests"))
import attention_distillation_kl_amd._lib as L
L.LIB_PATH = {lib!r}
from oracle import build_oracle
build_oracle.LIB = {oracle!r}
import oracle, pytest
rc = pytest.main({args!r})
assert {lib!r} in open("/proc/self/maps").read() or {lib_optional}, "sanitized library not loaded"
assert {oracle!r} in open("/proc/self/maps").read(), "sanitized oracle not loaded"
sys.exit(rc)
"""


def _child(builds, args, oracle_lib=None, lib_optional=False):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.setdefault("OMP_NUM_THREADS", "4")
    code = CHILD.format(root=ROOT, lib=builds["lib"], oracle=oracle_lib or builds["oracle"],
                        # sys-level capture only: a sanitizer report is
                        # written to fd 2 by a process about to exit
                        args=args + ["-q", "-p", "no:cacheprovider", "-m", "not gpu", "--capture=sys"],
                        lib_optional=lib_optional)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                          timeout=600)


def test_oracle_pins_and_abi_checks_are_clean_under_sanitizers(builds):
    r = _child(builds, ["tests/test_oracle_pins.py", "tests/test_abi_host.py"])
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out


def test_the_harness_reports_a_planted_overflow(builds):
    """A copy of the oracle whose score loop reads one key row past the end
    (on the CPU, in a temporary build): the same child must stop with an
    AddressSanitizer report."""
    src = open(os.path.join(ROOT, "oracle", "streamkl_oracle.c")).read()
    needle = "for (int j = 0; j < nj; ++j) {\n    s1[j] = scale * dot(qi1, k1 + (size_t)j * d, d);"
    assert needle in src
    bad = src.replace(needle, "for (int j = 0; j <= nj; ++j) {\n    s1[j] = scale * dot(qi1, k1 + (size_t)j * d, d);")
    path = os.path.join(str(builds["dir"]), "oracle_overflow.c")
    with open(path, "w") as fh:
        fh.write(bad)
    lib = _oracle(path, os.path.join(str(builds["dir"]), "liboracle_overflow.so"))
    r = _child(builds, ["tests/test_oracle_pins.py", "-x"], oracle_lib=lib, lib_optional=True)
    out = r.stdout + r.stderr
    assert r.returncode != 0
    assert "AddressSanitizer" in out and "heap-buffer-overflow" in out, out[-3000:]
